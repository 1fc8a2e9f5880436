// Prefill-chunk attention on CDNA4 matrix cores (fp16/bf16 caches, chunks of
// many query rows): out = softmax(q K^T / sqrt(D)) V with the bottom-right
// causal mask of a chunk that sits at offset s ("KV cache, incremental decode,
// ...", section 2.3; "kv-cache-decoding", "Prefill and decode": one parallel
// pass with a score matrix per head). A chunk of T queries against s + T keys
// is a dense contraction, so both products run on v_mfma_f32_32x32x16.
//
// Shapes and layouts (32x32x16 MFMA: A 32x16, B 16x32, C 32x32 fp32):
//  * Columns. A work-group owns one (batch row b, KV head g) and a block of the
//    chunk's queries. Its columns are (query i, query head r) pairs, query-major
//    (c = i * G + r), so all G heads that share K/V sit in the same tiles and
//    every K/V tile staged in LDS serves all of them ("Heads, GQA and K/V
//    cache": a group of queries shares the same keys and values). Each of the
//    8 waves owns NT tiles of 32 columns; two waves share a SIMD, so one's
//    softmax runs while the other's MFMAs do.
//  * S^T = K Q^T. A = K tile rows from LDS (16 bytes per lane), B = Q^T held in
//    registers for the whole launch. The C layout gives each lane one column
//    (lane % 32) and 16 of the 32 keys; the other 16 are in lane ^ 32, so the
//    softmax reductions are in-lane plus one exchange.
//  * O^T = V^T P^T. The probabilities in S^T's C registers are already the B
//    operand of this product when the 32 keys of a tile are taken in the order
//    the C layout holds them; V^T's A operand uses the same order, read from a
//    transposed copy of the V tile in LDS. O^T's C layout again gives each lane
//    its own column, so rescaling needs no data movement.
//  * Online softmax in base 2 with a lazily moved reference max (moved only
//    when a score passes it by 2^8); P is rounded to the storage type for the
//    MFMA and the normaliser sums the rounded values.
//  * Masking. Key tiles entirely visible to the work-group's queries skip the
//    mask; tiles past the last query's diagonal are never loaded.
#include <type_traits>

#include "kvc_device.h"

namespace kvc {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#ifndef KVC_PF_NT
#define KVC_PF_NT 1           // 32-column tiles per wave
#endif
#ifndef KVC_PF_WAVES_PER_EU
#define KVC_PF_WAVES_PER_EU 2   // two waves per SIMD: one's softmax overlaps the other's MFMAs
#endif
#ifndef KVC_PF_STAGES
#define KVC_PF_STAGES 3       // key/value tiles in the LDS ring
#endif

#ifndef KVC_PF_WAVES
#define KVC_PF_WAVES 8        // waves per work-group: every staged K/V tile serves 8 x 32 columns
#endif
constexpr int kPWaves = KVC_PF_WAVES;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kNT = KVC_PF_NT;
constexpr int kNB = KVC_PF_STAGES;
constexpr int kBN = 32;                // keys per tile
constexpr float kPRescaleLog2 = 8.f;

template <int ST>
__device__ __forceinline__ f32x16_t mfma32(const u32x4& a, const u32x4& b, const f32x16_t& c) {
    if constexpr (ST == BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                      __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                     __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

template <int ST>
__device__ __forceinline__ uint32_t to_st(float x) {
    return ST == BF16 ? f32_to_bf16_rne(x) : f32_to_f16_rne(x);
}

// Two probabilities rounded to the storage type (round to nearest even) and
// packed low-then-high into one word: one v_cvt_pk_bf16_f32 for bf16. The
// values are finite and non-negative, so no NaN case is needed.
template <int ST>
__device__ __forceinline__ uint32_t pack_p(float lo, float hi) {
    if constexpr (ST == BF16) {
        const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
        return __builtin_bit_cast(uint32_t, v);
    } else {
        const f16x2_t v = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
        return __builtin_bit_cast(uint32_t, v);
    }
}

// acc + the two values of a packed pair, as stored: a dot product with (1, 1)
// (exact products, float32 sum) in one instruction.
template <int ST>
__device__ __forceinline__ float add_pair(uint32_t w, float acc) {
    if constexpr (ST == BF16) {
        const bf16x2_t one = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), one, acc, false);
    } else {
        const f16x2_t one = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w), one, acc, false);
    }
}

// Wait until at most N vector-memory operations of this wave are outstanding
// and all LDS operations are done (gfx9 s_waitcnt encoding; expcnt not waited).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | ((N >> 4) << 14));
}

template <int D>
struct PCfg {
    static constexpr int CPR = D / 8;           // 16-byte chunks per key row
    static constexpr int DS = D / 16;           // MFMA k-steps over the head dimension
    static constexpr int DT = D / 32;           // 32-wide tiles of the head dimension
    static constexpr int TILE = kBN * D;        // elements per K (or V) tile
    static constexpr int TILE_BYTES = TILE * 2;
    static constexpr int NLD = TILE * 2 / 1024; // 1 KB LDS-DMA instructions per tile and tensor
    static constexpr int LPW = 2 * ((NLD + kPWaves - 1) / kPWaves);   // DMA loads per wave per stage
    static constexpr int K_OFF = 0;                      // byte offset of the K stages
    static constexpr int V_OFF = kNB * TILE_BYTES;       // byte offset of the V stages
    static constexpr int LDS_BYTES = 2 * kNB * TILE_BYTES;
    // The stage and row offsets travel as the 16-bit immediate of the LDS reads.
    static_assert(V_OFF + (kNB - 1) * TILE_BYTES + 24 * D * 2 < 65536, "LDS read offsets fit 16 bits");

    // K tile: rows of D elements with the 16-byte chunks XOR-swizzled by the row,
    // so the 32 lanes that read one chunk of 32 different rows hit distinct banks.
    __device__ static constexpr int kslot(int r, int c) { return c ^ (r & (CPR - 1)); }

    // V tile: rows of D elements, 16-byte chunk c of row r at slot vslot(r, c).
    // The transposed reads take 8 bytes per lane from 4 rows r (r % 4 = 0..3)
    // at the same 32-byte pair of chunks, in two pairs per 16-lane group; the
    // permutation puts those 4 x 2 pieces on distinct 32-byte bank groups of a
    // 256-byte bank period, and the 4 pieces of one group on distinct ones of
    // a 128-byte period.
    __device__ static constexpr int vslot(int r, int c) {
        const int u = c >> 1, h = c & 1;
        int up = 0;
        if constexpr (D == 128) up = 4 * (u & 1) + (((u >> 1) + r) & 3);
        else if constexpr (D == 64) up = (u + r) & 3;
        else up = u ^ ((r >> 1) & 1);
        return 2 * up + h;
    }
    // inverse of vslot for a fixed row: which chunk lands in slot sl
    __device__ static constexpr int vchunk(int r, int sl) {
        const int up = sl >> 1, h = sl & 1;
        int u = 0;
        if constexpr (D == 128) u = 2 * ((up - r) & 3) + (up >> 2);
        else if constexpr (D == 64) u = (up - r) & 3;
        else u = up ^ ((r >> 1) & 1);
        return 2 * u + h;
    }
};

// ---- LDS reads (explicit, each group waits for its own data) -------------
// The transposed read ds_read_b64_tr_b16 works on groups of 16 lanes: lane
// 16g + 4a + b receives element b of the 8 bytes read by lanes 16g + 4i + a,
// i = 0..3, as its elements i. Each lane here reads 4 head elements of one key,
// so every lane gets 4 consecutive keys of one head element.
#define KVC_RD128(o, a) "ds_read_b128 %" #o ", %" #a " offset:%[off]\n\t"
#define KVC_RDTR(o, a, imm) "ds_read_b64_tr_b16 %" #o ", %" #a " offset:%[" #imm "]\n\t"

// K operands of one tile: DS reads of 16 bytes at addr[ds] + OFF.
template <int DS, int OFF>
__device__ __forceinline__ void read_k(u32x4 (&k)[DS], const uint32_t (&addr)[DS]) {
    if constexpr (DS == 8) {
        asm volatile(KVC_RD128(0, 8) KVC_RD128(1, 9) KVC_RD128(2, 10) KVC_RD128(3, 11)
                     KVC_RD128(4, 12) KVC_RD128(5, 13) KVC_RD128(6, 14) KVC_RD128(7, 15) "s_waitcnt lgkmcnt(0)"
                     : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]), "=&v"(k[6]), "=&v"(k[7])
                     : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]),
                       "v"(addr[6]), "v"(addr[7]), [off] "i"(OFF)
                     : "memory");
    } else if constexpr (DS == 4) {
        asm volatile(KVC_RD128(0, 4) KVC_RD128(1, 5) KVC_RD128(2, 6) KVC_RD128(3, 7) "s_waitcnt lgkmcnt(0)"
                     : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3])
                     : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), [off] "i"(OFF)
                     : "memory");
    } else {
        static_assert(DS == 2, "head dimension 32, 64 or 128");
        asm volatile(KVC_RD128(0, 2) KVC_RD128(1, 3) "s_waitcnt lgkmcnt(0)"
                     : "=&v"(k[0]), "=&v"(k[1])
                     : "v"(addr[0]), "v"(addr[1]), [off] "i"(OFF)
                     : "memory");
    }
}

// V^T operands of one tile: for head tile dt and key step kk, two transposed
// reads (keys +0..3 and +8..11 of the lane's 4-key group) at addr[dt] + OFF +
// (16 kk + 8 h) rows.
template <int DT, int OFF, int ROWB>
__device__ __forceinline__ void read_vt(u32x2 (&v)[DT][2][2], const uint32_t (&addr)[DT]) {
    constexpr int o00 = OFF, o01 = OFF + 8 * ROWB, o10 = OFF + 16 * ROWB, o11 = OFF + 24 * ROWB;
    if constexpr (DT == 4) {
        asm volatile(KVC_RDTR(0, 16, o00) KVC_RDTR(1, 16, o01) KVC_RDTR(2, 16, o10) KVC_RDTR(3, 16, o11)
                     KVC_RDTR(4, 17, o00) KVC_RDTR(5, 17, o01) KVC_RDTR(6, 17, o10) KVC_RDTR(7, 17, o11)
                     KVC_RDTR(8, 18, o00) KVC_RDTR(9, 18, o01) KVC_RDTR(10, 18, o10) KVC_RDTR(11, 18, o11)
                     KVC_RDTR(12, 19, o00) KVC_RDTR(13, 19, o01) KVC_RDTR(14, 19, o10) KVC_RDTR(15, 19, o11)
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(v[0][0][0]), "=&v"(v[0][0][1]), "=&v"(v[0][1][0]), "=&v"(v[0][1][1]),
                       "=&v"(v[1][0][0]), "=&v"(v[1][0][1]), "=&v"(v[1][1][0]), "=&v"(v[1][1][1]),
                       "=&v"(v[2][0][0]), "=&v"(v[2][0][1]), "=&v"(v[2][1][0]), "=&v"(v[2][1][1]),
                       "=&v"(v[3][0][0]), "=&v"(v[3][0][1]), "=&v"(v[3][1][0]), "=&v"(v[3][1][1])
                     : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]),
                       [o00] "i"(o00), [o01] "i"(o01), [o10] "i"(o10), [o11] "i"(o11)
                     : "memory");
    } else if constexpr (DT == 2) {
        asm volatile(KVC_RDTR(0, 8, o00) KVC_RDTR(1, 8, o01) KVC_RDTR(2, 8, o10) KVC_RDTR(3, 8, o11)
                     KVC_RDTR(4, 9, o00) KVC_RDTR(5, 9, o01) KVC_RDTR(6, 9, o10) KVC_RDTR(7, 9, o11)
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(v[0][0][0]), "=&v"(v[0][0][1]), "=&v"(v[0][1][0]), "=&v"(v[0][1][1]),
                       "=&v"(v[1][0][0]), "=&v"(v[1][0][1]), "=&v"(v[1][1][0]), "=&v"(v[1][1][1])
                     : "v"(addr[0]), "v"(addr[1]),
                       [o00] "i"(o00), [o01] "i"(o01), [o10] "i"(o10), [o11] "i"(o11)
                     : "memory");
    } else {
        static_assert(DT == 1, "head dimension 32, 64 or 128");
        asm volatile(KVC_RDTR(0, 4, o00) KVC_RDTR(1, 4, o01) KVC_RDTR(2, 4, o10) KVC_RDTR(3, 4, o11)
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(v[0][0][0]), "=&v"(v[0][0][1]), "=&v"(v[0][1][0]), "=&v"(v[0][1][1])
                     : "v"(addr[0]), [o00] "i"(o00), [o01] "i"(o01), [o10] "i"(o10), [o11] "i"(o11)
                     : "memory");
    }
}
#undef KVC_RD128
#undef KVC_RDTR

template <int D, int ST>
__global__ __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(KVC_PF_WAVES_PER_EU)))
void prefill_attn(PrefillArgs a) {
    using P = PCfg<D>;
    // K stages then V stages. The loop reads them only through the explicit
    // LDS reads above, after its own wait and barrier.
    __shared__ __attribute__((aligned(16))) uint16_t smem[P::LDS_BYTES / 2];
    static_assert(kNB >= 2 && kNB <= 4, "the ring has two to four stages");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches on it
    const int col32 = lane & 31;
    const int hl = lane >> 5;                   // which half of the k-dimension this lane feeds

    // -- which (row, KV head, query block) this work-group owns; consecutive query
    //    blocks of one unit stay on one XCD when the unit count is a multiple of 8
    const int n_units = a.rows * a.Hkv;
    const int unit = blockIdx.x % n_units;
    const int qblk = blockIdx.x / n_units;
    const int b = unit / a.Hkv;
    const int g = unit - b * a.Hkv;
    const int s = a.offset[b];                  // the chunk's query offset for this row
    const int qpt = a.qpt;                      // queries per 32-column tile
    const int q_lo = a.i0 + qblk * a.q_per_block;   // first query of this work-group
    if (q_lo >= a.i0 + a.Ti) return;
    int q_hi = q_lo + a.q_per_block - 1;
    if (q_hi > a.i0 + a.Ti - 1) q_hi = a.i0 + a.Ti - 1;

    const int64_t head_base = a.layer_off + b * a.row_stride + g * a.head_stride;
    const uint16_t* kg = static_cast<const uint16_t*>(a.k_cache) + head_base;
    const uint16_t* vg = static_cast<const uint16_t*>(a.v_cache) + head_base;

    // -- this lane's columns: query i and head r of each of its tiles
    int col_i[kNT], col_r[kNT];
    bool col_ok[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        const int tile = wave * kNT + nt;
        const int i = q_lo + tile * qpt + col32 / a.Gc;
        const int r = col32 % a.Gc;
        col_ok[nt] = col32 < qpt * a.Gc && i <= q_hi;
        col_i[nt] = col_ok[nt] ? i : q_lo;
        col_r[nt] = r;
    }

    // -- key range: the last query of the work-group sees keys [0, s + q_hi]
    const int n_keys = s + q_hi + 1;
    const int n_tiles = (n_keys + kBN - 1) / kBN;
    const int vis_all = s + q_lo;               // keys <= this are visible to every column

    // -- the LDS ring: stage = one K tile and one V tile, moved by LDS-DMA loads
    //    (16 bytes per lane, lane i at byte 16 * i of the instruction's 1 KB).
    //    Tiles past the range are issued too, clamped to the last key, so every
    //    wave issues the same number of loads per stage.
    auto issue = [&](auto slot_c, int t) {
        constexpr int S = decltype(slot_c)::value;
        uint16_t* kd = smem + (P::K_OFF + S * P::TILE_BYTES) / 2;
        uint16_t* vd = smem + (P::V_OFF + S * P::TILE_BYTES) / 2;
#pragma unroll
        for (int n = wave; n < P::NLD; n += kPWaves) {
            const int e = n * 512 + lane * 8;       // element offset inside the tile
            const int r = e / D;
            const int sl = (e % D) >> 3;
            int j = t * kBN + r;
            j = j < n_keys ? j : n_keys - 1;
            const int64_t row = static_cast<int64_t>(j) * D;
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1)))*)(kg + row + P::kslot(r, sl) * 8),
                (void __attribute__((address_space(3)))*)(kd + n * 512), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1)))*)(vg + row + P::vchunk(r, sl) * 8),
                (void __attribute__((address_space(3)))*)(vd + n * 512), 16, 0, 0);
        }
    };
    issue(std::integral_constant<int, 0>{}, 0);
    if constexpr (kNB > 2) issue(std::integral_constant<int, 1>{}, 1);
    if constexpr (kNB > 3) issue(std::integral_constant<int, 2>{}, 2);

    // -- LDS read addresses of this lane (stage and row steps are immediates)
    const uint32_t lds0 = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint16_t*)smem));
    uint32_t kaddr[P::DS];
#pragma unroll
    for (int ds = 0; ds < P::DS; ++ds)
        kaddr[ds] = lds0 + (col32 * D + P::kslot(col32, 2 * ds + hl) * 8) * 2;
    uint32_t vaddr[P::DT];
    {
        const int grp = lane >> 4, ii = (lane >> 2) & 3, aa = lane & 3;
        const int rv = (grp >> 1) * 4 + ii;     // key row read by this lane (+ 8 and + 16 steps)
#pragma unroll
        for (int dt = 0; dt < P::DT; ++dt) {
            const int cv = dt * 4 + 2 * (grp & 1) + (aa >> 1);
            vaddr[dt] = lds0 + (rv * D + P::vslot(rv, cv) * 8) * 2 + (aa & 1) * 8;
        }
    }

    // -- Q^T as the B operand, rounded as the storage type: 8 consecutive head
    //    elements of this lane's column per k-step
    u32x4 qb[kNT][P::DS];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        const int h = g * a.G + a.r0 + col_r[nt];
        const int64_t qrow = ((static_cast<int64_t>(a.row0 + b) * a.Hq + h) * a.T + col_i[nt]) * D;
#pragma unroll
        for (int ds = 0; ds < P::DS; ++ds) {
            const int64_t e0 = qrow + ds * 16 + hl * 8;
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float x0, x1;
                if (a.q_dtype == F32) {
                    x0 = static_cast<const float*>(a.q)[e0 + 2 * e];
                    x1 = static_cast<const float*>(a.q)[e0 + 2 * e + 1];
                } else if (a.q_dtype == BF16) {
                    x0 = bf16_to_f32(static_cast<const uint16_t*>(a.q)[e0 + 2 * e]);
                    x1 = bf16_to_f32(static_cast<const uint16_t*>(a.q)[e0 + 2 * e + 1]);
                } else {
                    x0 = f16_to_f32(static_cast<const uint16_t*>(a.q)[e0 + 2 * e]);
                    x1 = f16_to_f32(static_cast<const uint16_t*>(a.q)[e0 + 2 * e + 1]);
                }
                w[e] = to_st<ST>(x0) | (to_st<ST>(x1) << 16);
            }
            qb[nt][ds] = u32x4{w[0], w[1], w[2], w[3]};
        }
    }

    // -- per-column softmax state and the O^T accumulators
    float m[kNT], lsum[kNT];
    f32x16_t o[kNT][P::DT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        m[nt] = -INFINITY;
        lsum[nt] = 0.f;
#pragma unroll
        for (int dt = 0; dt < P::DT; ++dt) o[nt][dt] = f32x16_t{};
    }
    const float c = a.scale_log2;
    const float thresh = kPRescaleLog2 / c;

    auto step = [&](auto slot_c, int t) {
        constexpr int S = decltype(slot_c)::value;
        // this wave's loads of tile t are done (the kNB - 2 later stages may still
        // be in flight); then every wave's are, and every wave is done with tile t - 1
        wait_vm_lgkm0<(kNB - 2) * P::LPW>();
        __builtin_amdgcn_s_barrier();
        issue(std::integral_constant<int, (S + kNB - 1) % kNB>{}, t + kNB - 1);

        const int j0 = t * kBN;
        const bool plain = j0 + kBN - 1 <= vis_all && j0 + kBN <= n_keys;

        // S^T tile per column tile: 32 keys x 32 columns
        u32x4 ka[P::DS];
        read_k<P::DS, P::K_OFF + S * P::TILE_BYTES>(ka, kaddr);
        f32x16_t sacc[kNT];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) sacc[nt] = f32x16_t{};
#pragma unroll
        for (int ds = 0; ds < P::DS; ++ds)
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) sacc[nt] = mfma32<ST>(ka[ds], qb[nt][ds], sacc[nt]);

        // V^T operands, read while the score MFMAs run
        u32x2 vt[P::DT][2][2];
        read_vt<P::DT, P::V_OFF + S * P::TILE_BYTES, D * 2>(vt, vaddr);

        // scores -> probabilities, in the C layout: value jj is key
        // j0 + (jj / 4) * 8 + hl * 4 + jj % 4 of this lane's column
        u32x4 pb[kNT][2];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            float sv_[16];
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) sv_[jj] = sacc[nt][jj];
            if (!plain) {
                const int lim = s + col_i[nt];
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) {
                    const int j = j0 + (jj >> 2) * 8 + hl * 4 + (jj & 3);
                    if (j > lim || j >= n_keys) sv_[jj] = -INFINITY;
                }
            }
            // The reference max moves only when a score passes it by the
            // threshold; each half-column checks its own 16 keys, and only then
            // is the column's max formed across the two halves (lane ^ 32).
            float mt = sv_[0];
#pragma unroll
            for (int jj = 1; jj < 16; ++jj) mt = fmaxf(mt, sv_[jj]);
            if (__any(mt - m[nt] > thresh)) {
                mt = fmaxf(mt, __shfl_xor(mt, 32));
                if (mt - m[nt] > thresh) {
                    const float alpha = m[nt] == -INFINITY ? 0.f : fexp2((m[nt] - mt) * c);
                    m[nt] = mt;
                    lsum[nt] *= alpha;
#pragma unroll
                    for (int dt = 0; dt < P::DT; ++dt) o[nt][dt] *= alpha;
                }
            }
            const float nmc = m[nt] == -INFINITY ? 0.f : -m[nt] * c;
            uint32_t w[8];
            float ls[2] = {0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                w[e] = pack_p<ST>(fexp2(fmaf(sv_[2 * e], c, nmc)), fexp2(fmaf(sv_[2 * e + 1], c, nmc)));
                ls[e & 1] = add_pair<ST>(w[e], ls[e & 1]);
            }
            lsum[nt] += ls[0] + ls[1];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) pb[nt][kk] = u32x4{w[kk * 4 + 0], w[kk * 4 + 1], w[kk * 4 + 2], w[kk * 4 + 3]};
        }

        // O^T += V^T P^T: for key step kk, A element e of the lane is key
        // kk * 16 + (e / 4) * 8 + hl * 4 + e % 4 at head element dt * 32 + lane % 32
#pragma unroll
        for (int dt = 0; dt < P::DT; ++dt)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const u32x4 va = {vt[dt][kk][0][0], vt[dt][kk][0][1], vt[dt][kk][1][0], vt[dt][kk][1][1]};
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) o[nt][dt] = mfma32<ST>(va, pb[nt][kk], o[nt][dt]);
            }
    };
    for (int t0 = 0; t0 < n_tiles; t0 += kNB) {
        step(std::integral_constant<int, 0>{}, t0);
        if (t0 + 1 >= n_tiles) break;
        step(std::integral_constant<int, 1>{}, t0 + 1);
        if constexpr (kNB > 2) {
            if (t0 + 2 >= n_tiles) break;
            step(std::integral_constant<int, 2>{}, t0 + 2);
        }
        if constexpr (kNB > 3) {
            if (t0 + 3 >= n_tiles) break;
            step(std::integral_constant<int, 3>{}, t0 + 3);
        }
    }
    wait_vm_lgkm0<0>();   // drain the ring's clamped tail loads before the work-group ends

    // -- normalise and write: lane holds column col32, head elements
    //    dt * 32 + (jj / 4) * 8 + hl * 4 + jj % 4
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
        const float l_all = lsum[nt] + __shfl_xor(lsum[nt], 32);
        if (!col_ok[nt]) continue;
        const float inv = 1.f / l_all;
        const int h = g * a.G + a.r0 + col_r[nt];
        float* dst = a.out + ((static_cast<int64_t>(a.row0 + b) * a.Hq + h) * a.T + col_i[nt]) * D;
#pragma unroll
        for (int dt = 0; dt < P::DT; ++dt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d = dt * 32 + q4 * 8 + hl * 4;
                *reinterpret_cast<float4*>(dst + d) =
                    make_float4(o[nt][dt][q4 * 4 + 0] * inv, o[nt][dt][q4 * 4 + 1] * inv,
                                o[nt][dt][q4 * 4 + 2] * inv, o[nt][dt][q4 * 4 + 3] * inv);
            }
    }
}

template <int D>
hipError_t run_p(const PrefillArgs& a, hipStream_t s, unsigned grid) {
    if (a.st_dtype == BF16) prefill_attn<D, BF16><<<grid, kPThreads, 0, s>>>(a);
    else if (a.st_dtype == F16) prefill_attn<D, F16><<<grid, kPThreads, 0, s>>>(a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

int prefill_columns_per_block() { return kPWaves * kNT * 32; }

bool prefill_supported(int D, int st_dtype) {
    return (D == 32 || D == 64 || D == 128) && (st_dtype == F16 || st_dtype == BF16);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
    if (a.Gc < 1 || a.Gc > 32 || a.qpt < 1 || a.qpt * a.Gc > 32) return hipErrorInvalidValue;
    const int n_qblk = (a.Ti + a.q_per_block - 1) / a.q_per_block;
    const int64_t grid = static_cast<int64_t>(n_qblk) * a.rows * a.Hkv;
    if (grid < 1 || grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    switch (a.D) {
        case 32: return run_p<32>(a, s, static_cast<unsigned>(grid));
        case 64: return run_p<64>(a, s, static_cast<unsigned>(grid));
        case 128: return run_p<128>(a, s, static_cast<unsigned>(grid));
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvc
