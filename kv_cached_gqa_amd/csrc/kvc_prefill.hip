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

#include "kvc_mfma.h"


namespace kvc {
namespace {

#ifndef KVC_PF_NT
#define KVC_PF_NT 1           // 32-column tiles per wave
#endif
#ifndef KVC_PF_WAVES_PER_EU
#define KVC_PF_WAVES_PER_EU 2   // two waves per SIMD: one's softmax overlaps the other's MFMAs
#endif
#ifndef KVC_PF_KV_CPOL
#define KVC_PF_KV_CPOL 0      // cache-policy bits of the K/V tile loads (default: the query blocks
                              // of a unit share its tiles in L2; non-temporal measured ~1% slower)
#endif
#ifndef KVC_PF_QVEC
#define KVC_PF_QVEC 1         // q already in the storage type: one 16-byte load per k-step (~2% faster)
#endif
#ifndef KVC_PF_STAGES
#define KVC_PF_STAGES 4       // key/value tiles in the LDS ring (64 KB; 3 measured ~0.6% slower)
#endif

#ifndef KVC_PF_WAVES
#define KVC_PF_WAVES 8        // waves per work-group: every staged K/V tile serves 8 x 32 columns
#endif
constexpr int kPWaves = KVC_PF_WAVES;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kNT = KVC_PF_NT;
constexpr int kNB = KVC_PF_STAGES;
constexpr float kPRescaleLog2 = 8.f;

template <int D>
struct PCfg : TileLayout<D> {
    using L = TileLayout<D>;
    static constexpr int LPW = 2 * ((L::NLD + kPWaves - 1) / kPWaves);   // DMA loads per wave per stage
    static constexpr int K_OFF = 0;                         // byte offset of the K stages
    static constexpr int V_OFF = kNB * L::TILE_BYTES;       // byte offset of the V stages
    static constexpr int LDS_BYTES = 2 * kNB * L::TILE_BYTES;
    // The stage and row offsets travel as the 16-bit immediate of the LDS reads.
    static_assert(V_OFF + (kNB - 1) * L::TILE_BYTES + 24 * D * 2 < 65536, "LDS read offsets fit 16 bits");
};

// PS: P as a 16-bit hi + lo pair, the residual of the first rounding rounded
// again and multiplied with V by a second product (error ~1e-6 instead of
// ~1e-3 for a once-rounded P; half again as many products).
template <int D, int ST, bool PAGED, bool PS>
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

    // contiguous storage: this head's rows; paged storage: the layer's pool
    const int64_t head_base = PAGED ? a.layer_off : a.layer_off + b * a.row_stride + g * a.head_stride;
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
    //    Paged storage: a 32-key tile lies in one block (blocks hold a power of
    //    two >= 64 keys); a tile past the range is clamped to the last tile, and
    //    the block's pool offset comes from a scalar load of the table.
    auto issue = [&](auto slot_c, int t) {
        constexpr int S = decltype(slot_c)::value;
        uint16_t* kd = smem + (P::K_OFF + S * P::TILE_BYTES) / 2;
        uint16_t* vd = smem + (P::V_OFF + S * P::TILE_BYTES) / 2;
        int64_t blk_base = 0;
        if constexpr (PAGED) {
            t = t < n_tiles ? t : n_tiles - 1;
            const auto* tab = (const __attribute__((address_space(4))) int32_t*)(a.btab);
            int bi = (t * kBN) >> a.bshift;
            bi = bi < a.btab_stride ? bi : a.btab_stride - 1;
            int p = tab[static_cast<int64_t>(b) * a.btab_stride + bi];
            p = p < 0 ? 0 : (p >= a.pool_blocks ? a.pool_blocks - 1 : p);
            blk_base = ((static_cast<int64_t>(p) * a.Hkv + g) << a.bshift) * D;
        }
#pragma unroll
        for (int n = wave; n < P::NLD; n += kPWaves) {
            const int e = n * 512 + lane * 8;       // element offset inside the tile
            const int r = e / D;
            const int sl = (e % D) >> 3;
            int j = t * kBN + r;
            j = j < n_keys ? j : n_keys - 1;
            int64_t row;
            if constexpr (PAGED)
                row = blk_base + static_cast<int64_t>(j & ((1 << a.bshift) - 1)) * D;
            else
                row = static_cast<int64_t>(j) * D;
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1)))*)(kg + row + P::kslot(r, sl) * 8),
                (void __attribute__((address_space(3)))*)(kd + n * 512), 16, 0, KVC_PF_KV_CPOL);
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1)))*)(vg + row + P::vchunk(r, sl) * 8),
                (void __attribute__((address_space(3)))*)(vd + n * 512), 16, 0, KVC_PF_KV_CPOL);
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
            if (KVC_PF_QVEC && a.q_dtype == ST) {
                // the caller's 16-bit q as stored: 8 elements, 16 bytes (rounding a
                // 16-bit value to the same type leaves it as it is)
                qb[nt][ds] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.q) + e0);
                continue;
            }
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
        u32x4 pl[kNT][2];
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
                mt = xor_op<32, true>(mt);
                if (mt - m[nt] > thresh) {
                    const float alpha = m[nt] == -INFINITY ? 0.f : fexp2((m[nt] - mt) * c);
                    m[nt] = mt;
                    lsum[nt] *= alpha;
#pragma unroll
                    for (int dt = 0; dt < P::DT; ++dt) o[nt][dt] *= alpha;
                }
            }
            const float nmc = m[nt] == -INFINITY ? 0.f : -m[nt] * c;
            uint32_t w[8], wl[8];
            float ls[2] = {0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p0 = fexp2(fmaf(sv_[2 * e], c, nmc)), p1 = fexp2(fmaf(sv_[2 * e + 1], c, nmc));
                w[e] = pack_p<ST>(p0, p1);
                ls[e & 1] = add_pair<ST>(w[e], ls[e & 1]);
                if constexpr (PS) {
                    // the rounding residual of each probability, rounded again: P = hi + lo
                    wl[e] = pack_p<ST>(p0 - low_half<ST>(w[e]), p1 - high_half<ST>(w[e]));
                    ls[e & 1] = add_pair<ST>(wl[e], ls[e & 1]);
                }
            }
            lsum[nt] += ls[0] + ls[1];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) pb[nt][kk] = u32x4{w[kk * 4 + 0], w[kk * 4 + 1], w[kk * 4 + 2], w[kk * 4 + 3]};
            if constexpr (PS) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    pl[nt][kk] = u32x4{wl[kk * 4 + 0], wl[kk * 4 + 1], wl[kk * 4 + 2], wl[kk * 4 + 3]};
            }
        }

        // O^T += V^T P^T: for key step kk, A element e of the lane is key
        // kk * 16 + (e / 4) * 8 + hl * 4 + e % 4 at head element dt * 32 + lane % 32
#pragma unroll
        for (int dt = 0; dt < P::DT; ++dt)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const u32x4 va = {vt[dt][kk][0][0], vt[dt][kk][0][1], vt[dt][kk][1][0], vt[dt][kk][1][1]};
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt) {
                    o[nt][dt] = mfma32<ST>(va, pb[nt][kk], o[nt][dt]);
                    if constexpr (PS) o[nt][dt] = mfma32<ST>(va, pl[nt][kk], o[nt][dt]);
                }
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
        const float l_all = xor_op<32, false>(lsum[nt]);
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

template <int D, bool PAGED, bool PS>
hipError_t run_pps(const PrefillArgs& a, hipStream_t s, unsigned grid) {
    if (a.st_dtype == BF16) prefill_attn<D, BF16, PAGED, PS><<<grid, kPThreads, 0, s>>>(a);
    else if (a.st_dtype == F16) prefill_attn<D, F16, PAGED, PS><<<grid, kPThreads, 0, s>>>(a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

template <int D, bool PAGED>
hipError_t run_pp(const PrefillArgs& a, hipStream_t s, unsigned grid) {
    return a.p_split ? run_pps<D, PAGED, true>(a, s, grid) : run_pps<D, PAGED, false>(a, s, grid);
}

template <int D>
hipError_t run_p(const PrefillArgs& a, hipStream_t s, unsigned grid) {
    if (a.btab) {
        if ((1 << a.bshift) < kBN) return hipErrorInvalidValue;   // a tile within one block
        return run_pp<D, true>(a, s, grid);
    }
    return run_pp<D, false>(a, s, grid);
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
