// Decode attention: softmax(q K^T / sqrt(D)) V for a few query rows per KV
// head, over all keys the cache holds for each batch row
// ("KV cache, incremental decode, ...", section 2.3, the bottom-right mask;
// "kv-cache-decoding", "Prefill and decode": one row of t + 1 scores per head).
//
// Decode reads every cached key and value once and does ~4 flops per byte,
// so it is bound by HBM bandwidth. The design keeps many bytes in flight on
// every CU, for the whole launch, and keeps the vector ALU work per key small:
//
//  * Work split ("stream-K"). Unit u = (batch row b, KV head g) owns n_b keys.
//    The units are laid end to end along one axis of sum(n_b) * H_kv keys and
//    every work-group takes an equal slice of it, so ragged row lengths cost
//    no load imbalance. One work-group per CU: all of them start together, so
//    none is starved by older waves at the memory arbiters. A slice that
//    crosses unit boundaries is cut into segments; segment (work-group k,
//    unit u) is stored at index k + u, which is unique because each new
//    segment starts at a slice boundary, a unit boundary or both.
//  * Loads. Each wave streams its own keys through a private ring of NS LDS
//    stages filled by LDS-DMA (global_load_lds, 16 bytes per lane): NS - 1
//    stages are in flight while one is used, with no registers held for them.
//    The ring runs straight across segment boundaries, so the next unit's keys
//    are already on their way while a segment is merged. Each wave waits for
//    its own loads only (an explicit vmcnt), so the loop has no barrier.
//  * Lane layout. One key row of D elements is LPK lanes x 16 bytes; a load of
//    64 lanes covers KPW = 64 / LPK consecutive keys, one contiguous 1 KB. All
//    query rows of the slab (the G query heads that share the KV head, times
//    the chunk's query positions) are held in every lane group, so each key
//    and value is read from HBM exactly once for the whole group ("Heads, GQA
//    and K/V cache": heads sharing one K/V). A segment's query rows travel the
//    same way: wave 0 loads them by LDS-DMA into one of NS query slots just
//    before the segment's first stage, so its own wait for the stage before
//    covers them, and the barriers of the previous segment's merge publish them
//    to every wave; each wave converts them to the storage type itself.
//  * q.k: 16-bit dot2 instructions (exact products, fp32 accumulation) or fp32
//    FMA, then a DPP sum over the LPK lanes of the key. Scores stay in raw
//    q.k units; the softmax scale and log2(e) are folded into one FMA before
//    exp2. The running max only triggers a rescale when it grows somewhere in
//    the wave. p stays fp32 and p*v is an fp32 FMA.
//  * Merge. At the end of a segment the lane groups and the waves merge their
//    (max, sum, output). A unit held by one segment is normalised and written
//    at once; otherwise the segment's partial record goes to the workspace and
//    a second, small kernel merges each split unit's records.
#pragma once

#include <type_traits>

#include "kvc_mfma.h"

namespace kvc {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#ifndef KVC_DECODE_WAVES
#define KVC_DECODE_WAVES 4        // waves per work-group
#endif
#ifndef KVC_DECODE_STAGES
#define KVC_DECODE_STAGES 3       // LDS ring stages per wave
#endif
#ifndef KVC_DECODE_U
#define KVC_DECODE_U 2            // 1 KB loads per tensor per stage (4 query rows or fewer)
#endif
#ifndef KVC_DECODE_RESCALE_LOG2
#define KVC_DECODE_RESCALE_LOG2 8.0f
#endif
#ifndef KVC_DECODE_BLOCKS_PER_CU
#define KVC_DECODE_BLOCKS_PER_CU 2
#endif
#ifndef KVC_DECODE_KV_CPOL
// Cache-policy bits of the vector kernels' K/V loads: non-temporal (each key
// and value is read once per call; measured ~9% faster on the batched-decode
// workload than the default policy).
#define KVC_DECODE_KV_CPOL 2
#endif
#ifndef KVC_DECODE_MFMA_KV_CPOL
#define KVC_DECODE_MFMA_KV_CPOL 2 // the same for the matrix-core decode kernel (~11% faster)
#endif
#ifndef KVC_DECODE_LATE_PCT
#define KVC_DECODE_LATE_PCT 70       // slice of a later-dispatched work-group, % of a first-round one
#endif
#ifndef KVC_DECODE_ODD_XCD_PCT
#define KVC_DECODE_ODD_XCD_PCT 90    // slice of a work-group on an odd XCD, % of one on an even XCD (measured on
                                     // batched decode: 86 65.0, 88 64.6, 90 64.0, 93 64.3 us)
#endif
#ifndef KVC_DECODE_MFMA_ODD_XCD_PCT_WIDE
#define KVC_DECODE_MFMA_ODD_XCD_PCT_WIDE 86   // the same on the matrix-core kernel for slabs of more than 16 query
                                              // rows (32-row long context: 86 173.8, 88 175.2, 90 176.3 us)
#endif

// Rescale threshold (log2 units): the running reference max moves only when a
// score exceeds it by more than this, so p = exp2(s - m) stays below 2^8.
constexpr float kRescaleLog2 = KVC_DECODE_RESCALE_LOG2;
constexpr int kLdsLimit = 160 * 1024;

template <int ST>
__device__ __forceinline__ float dot16(const uint32_t (&q)[4], const u32x4& k, float acc) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        // copy the element out first: a bit cast applied to a vector element
        // directly has been seen to read element 0 for every e
        const uint32_t kw = k[e];
        if constexpr (ST == BF16)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[e]), __builtin_bit_cast(bf16x2_t, kw),
                                                  acc, false);
        else
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q[e]), __builtin_bit_cast(f16x2_t, kw), acc, false);
    }
    return acc;
}

template <int ST, int EPC>
__device__ __forceinline__ void unpack_v(const u32x4& v, float (&o)[EPC]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if constexpr (ST == F32) {
            o[e] = __uint_as_float(v[e]);
        } else if constexpr (ST == BF16) {
            o[2 * e] = __uint_as_float(v[e] << 16);
            o[2 * e + 1] = __uint_as_float(v[e] & 0xFFFF0000u);
        } else {
            o[2 * e] = f16_to_f32(v[e] & 0xFFFFu);
            o[2 * e + 1] = f16_to_f32(v[e] >> 16);
        }
    }
}

template <int D, int ST, int R>
struct Cfg {
    static constexpr int ESZ = ST == F32 ? 4 : 2;
    static constexpr int EPC = 16 / ESZ;               // elements per lane (16 bytes)
    static constexpr int LPK = D / EPC;                // lanes per key row
    static constexpr int KPW = 64 / LPK;               // keys per 1 KB load
    static constexpr int WAVES = KVC_DECODE_WAVES;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int U = (R <= 4 && ST != F32) ? KVC_DECODE_U : 1;   // loads per tensor per stage
    static constexpr int KPS = U * KPW;                // keys per wave per stage
    static constexpr int KPB = WAVES * KPS;            // keys per work-group batch
    static constexpr int STAGE_BYTES = U * 2048;       // K and V of one stage of one wave
    // one query slot: the slab's R rows as the caller passed them (up to 4 bytes
    // an element), in whole 1 KB DMA blocks
    static constexpr int QSLOT_BYTES = (R * D * 4 + 1023) / 1024 * 1024;
    static constexpr int MERGE_BYTES = WAVES * R * (D + 2) * 4;
    static constexpr int lds_for(int ns) {
        return WAVES * ns * STAGE_BYTES + ns * QSLOT_BYTES + MERGE_BYTES;
    }
    // ring stages: as many as asked for, fewer if the LDS budget (at the work-groups
    // per CU asked for) does not hold them
    static constexpr int fit_stages() {
        int ns = KVC_DECODE_STAGES;
        const int per_cu = KVC_DECODE_BLOCKS_PER_CU > 0 ? KVC_DECODE_BLOCKS_PER_CU : 1;
        while (ns > 2 && lds_for(ns) * per_cu > kLdsLimit) --ns;
        return ns;
    }
    static constexpr int NS = fit_stages();
    static constexpr int RING_BYTES = WAVES * NS * STAGE_BYTES;
    static constexpr int LDS_BYTES = lds_for(NS);
    static_assert(NS >= 2, "ring stages");
    static_assert(LDS_BYTES <= kLdsLimit, "decode LDS budget");
    static_assert((NS - 1) * 2 * U < 64, "vmcnt field");
    static_assert((NS - 1) * STAGE_BYTES + STAGE_BYTES < 65536, "ring offsets fit the LDS immediate");
};

// Wait until at most N vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding; LDS and export counters not waited).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Work-group barrier for LDS data only: this wave's LDS operations are done,
// then every wave has arrived. (__syncthreads would also wait for every load
// in flight, draining the DMA ring.) The clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// K and V words of this lane for one 1 KB load of a stage: ring bytes at
// addr + OFF and addr + OFF + 1024, read after their own wait.
template <int OFF>
__device__ __forceinline__ void read_kv(u32x4& k, u32x4& v, uint32_t addr) {
    asm volatile("ds_read_b128 %0, %2 offset:%3\n\tds_read_b128 %1, %2 offset:%4\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(k), "=&v"(v)
                 : "v"(addr), "i"(OFF), "i"(OFF + 1024)
                 : "memory");
}

// An LDS read the compiler does not see. Before an LDS access of its own that
// might alias a pending LDS-DMA write it waits for every load in flight; this
// read carries its own wait instead.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
}
__device__ __forceinline__ u32x4 lds_read_b128(uint32_t addr) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
    return v;
}
// f(integral_constant<0>), ..., f(integral_constant<N - 1>), unrolled.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (N > 0) {
        static_for<N - 1>(f);
        f(std::integral_constant<int, N - 1>{});
    }
}

template <int LPK, int M>
__device__ __forceinline__ void lane_group_sum(float (&x)[M]) {
    if constexpr (LPK <= 16) {
        group_sum_n<LPK, M>(x);
    } else {
#pragma unroll
        for (int i = 0; i < M; ++i) x[i] = group_sum<LPK>(x[i]);
    }
}

// One segment of a work-group's slice: keys [j0, j1) of unit (b, g), whose
// last slab query sits at position n_b - Tc.
// The row of key-axis position x on the padded axis (row b starts at
// prefix[b] + b * row_pad): the b whose rows start at or before x, and the
// padded starts of rows b and b + 1, found with one round
// of vector loads from the kernel arguments (load_prefix_lanes: lane l reads
// entries l, l + 64, ...; entries past the last row hold INT64_MAX) and
// ballots that count the entries at or below x (row_of). A binary search over
// the arguments waits for one dependent scalar load per step; at a
// work-group's start that held its first K/V load back by over a microsecond.
// The whole wave must be active.
struct RowOf {
    int b;
    int64_t p0, p1;
};
template <int S>
struct PrefixLanes {
    static constexpr int kSlots = S;
    int64_t e[S];              // entries lane, lane + 64, ...
};
// the table of argument block A (the kernel's own: A is its parameter type)
template <class A>
__device__ __forceinline__ PrefixLanes<(A::kPrefix + 63) / 64> load_prefix_lanes() {
    constexpr int last = A::kPrefix - 1;
    const auto* args = (const __attribute__((address_space(4))) char*)__builtin_amdgcn_kernarg_segment_ptr();
    const auto* pf = reinterpret_cast<const __attribute__((address_space(4))) int64_t*>(args + offsetof(A, prefix));
    const int lane = static_cast<int>(threadIdx.x) & 63;
    PrefixLanes<(A::kPrefix + 63) / 64> p;
#pragma unroll
    for (int j = 0; j < p.kSlots; ++j) {
        // every lane loads (a vector load: a lane-0-only load would become a
        // scalar one that the compiler waits for at once)
        const int i = lane + 64 * j;
        const int64_t v = pf[i <= last ? i : last];
        p.e[j] = i <= last ? v : INT64_MAX;
    }
    return p;
}
template <int S>
__device__ __forceinline__ RowOf row_of(const PrefixLanes<S>& p, int64_t x, int64_t row_pad) {
    // entry i on the padded axis: prefix[i] + i * row_pad
    const int lane = static_cast<int>(threadIdx.x) & 63;
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < S; ++j) {
        const int64_t ep = p.e[j] == INT64_MAX ? INT64_MAX : p.e[j] + static_cast<int64_t>(lane + 64 * j) * row_pad;
        cnt += __popcll(__ballot(ep <= x));
    }
    // entry i: read from lane i mod 64 of every slot, then the slot i / 64
    // picked among the (uniform) results
    auto entry = [&](int i) __attribute__((always_inline)) -> int64_t {
        const int j = i >> 6, l = i & 63;
        int64_t v = 0;
#pragma unroll
        for (int jj = 0; jj < S; ++jj) {
            const uint64_t u = static_cast<uint64_t>(p.e[jj]);
            const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(u), l);
            const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(u >> 32), l);
            if (j == jj) v = static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
        }
        return v;
    };
    RowOf r;
    r.b = cnt - 1;
    r.p0 = entry(r.b) + r.b * row_pad;
    r.p1 = entry(r.b + 1) + (r.b + 1) * row_pad;
    return r;
}

// row_of for launches of fewer than 64 rows: every entry, the one past the last
// row included, sits in the first slot.
__device__ __forceinline__ RowOf row_of_one(int64_t e0, int64_t x, int64_t row_pad) {
    const int lane = static_cast<int>(threadIdx.x) & 63;
    const int64_t ep = e0 == INT64_MAX ? INT64_MAX : e0 + static_cast<int64_t>(lane) * row_pad;
    RowOf r;
    r.b = static_cast<int>(__popcll(__ballot(ep <= x))) - 1;
    auto entry = [&](int i) __attribute__((always_inline)) -> int64_t {
        const uint64_t u = static_cast<uint64_t>(e0);
        const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(u), i);
        const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(u >> 32), i);
        return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
    };
    r.p0 = entry(r.b) + r.b * row_pad;
    r.p1 = entry(r.b + 1) + (r.b + 1) * row_pad;
    return r;
}

struct Seg {
    int b, g;
    int j0, j1, n_b;
    int nbat;                // work-group batches of KPB keys
    int64_t head;            // element offset of the unit's key 0
    int64_t x_end;           // key-axis position where the segment ends
    int64_t rec;             // workspace record, or -1: the whole unit, written directly
};

// Paged storage, issue side: pool offsets of head g's rows in the physical
// blocks of an issue cursor's logical blocks blk and blk + 1 (a batch, stage
// or tile spans at most these two), and the raw table entry of block blk + 2.
// That entry is read by a scalar load when the cursor enters blk and first used
// when it enters blk + 1: a value needed at once would make the wave wait for
// the load at every block, with the next loads not yet issued, while this one
// arrives under the waits for the loads in flight.
template <int D>
struct PagedCursor {
    int blk;
    int64_t base, next;
    int ahead;

    template <class A>
    __device__ __forceinline__ static int entry(const A& a, int b, int blk) {
        const auto* tab = (const __attribute__((address_space(4))) int32_t*)(a.btab);
        const int bi = blk < a.btab_stride ? blk : a.btab_stride - 1;
        return tab[static_cast<int64_t>(b) * a.btab_stride + bi];
    }
    template <class A>
    __device__ __forceinline__ static int64_t rows(const A& a, int p, int g) {
        p = p < 0 ? 0 : (p >= a.pool_blocks ? a.pool_blocks - 1 : p);
        return a.layer_off + ((static_cast<int64_t>(p) * a.Hkv + g) << a.bshift) * D;
    }
    // the cursor starts unit (b, g) at logical block b0
    template <class A>
    __device__ __forceinline__ void enter(const A& a, int b, int g, int b0) {
        const int e0 = entry(a, b, b0), e1 = entry(a, b, b0 + 1);    // the three loads, then one wait
        ahead = entry(a, b, b0 + 2);
        blk = b0;
        base = rows(a, e0, g);
        next = rows(a, e1, g);
    }
    // the cursor moves on to block nb = blk + 1
    template <class A>
    __device__ __forceinline__ void step(const A& a, int b, int g, int nb) {
        blk = nb;
        base = next;
        next = rows(a, ahead, g);
        ahead = entry(a, b, nb + 2);
    }
    // element offset of key j (in block blk or blk + 1) of the unit's head
    template <class A>
    __device__ __forceinline__ int64_t row(const A& a, int j) const {
        return ((j >> a.bshift) == blk ? base : next) + static_cast<int64_t>(j & ((1 << a.bshift) - 1)) * D;
    }
};

// The slab's query rows, lane's share (EPC elements from element sub * EPC of
// each row), converted to the storage format, from an LDS slot at byte address
// `slot` that holds the rows as the caller passed them (row r at r * D * qsize).
template <int D, int ST, int R>
__device__ __forceinline__ void load_q_rows(uint32_t (&qp)[R][4], uint32_t slot, int q_dtype, int sub) {
    constexpr int EPC = ST == F32 ? 4 : 8;
    if (q_dtype == ST) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const u32x4 w = lds_read_b128(slot + r * D * (ST == F32 ? 4 : 2) + sub * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) qp[r][e] = w[e];
        }
        return;
    }
    // a different query type: widen to float, then round to the storage type
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float f[EPC];
        if (q_dtype == F32) {
            // EPC floats: 16 or 32 bytes
#pragma unroll
            for (int h = 0; h < EPC / 4; ++h) {
                const u32x4 w = lds_read_b128(slot + r * D * 4 + sub * EPC * 4 + h * 16);
#pragma unroll
                for (int e = 0; e < 4; ++e) f[h * 4 + e] = __uint_as_float(w[e]);
            }
        } else {
            // EPC 16-bit values: 8 or 16 bytes (an aligned 16-byte read covers them)
            const uint32_t at = slot + r * D * 2 + sub * EPC * 2;
            const u32x4 w = lds_read_b128(at & ~15u);
            const int w0 = (at & 15u) >> 2;
#pragma unroll
            for (int e = 0; e < EPC / 2; ++e) {
                uint32_t x = w[0];
                if constexpr (EPC == 4) x = w0 + e == 1 ? w[1] : (w0 + e == 2 ? w[2] : (w0 + e == 3 ? w[3] : w[0]));
                else x = e == 1 ? w[1] : (e == 2 ? w[2] : (e == 3 ? w[3] : w[0]));
                const uint32_t lo = x & 0xFFFFu, hi = x >> 16;
                f[2 * e] = q_dtype == BF16 ? bf16_to_f32(lo) : f16_to_f32(lo);
                f[2 * e + 1] = q_dtype == BF16 ? bf16_to_f32(hi) : f16_to_f32(hi);
            }
        }
        if constexpr (ST == F32) {
#pragma unroll
            for (int e = 0; e < 4; ++e) qp[r][e] = __float_as_uint(f[e]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo = ST == BF16 ? f32_to_bf16_rne(f[2 * e]) : f32_to_f16_rne(f[2 * e]);
                const uint32_t hi = ST == BF16 ? f32_to_bf16_rne(f[2 * e + 1]) : f32_to_f16_rne(f[2 * e + 1]);
                qp[r][e] = (lo & 0xFFFFu) | (hi << 16);
            }
        }
    }
}

template <class A, int D, int ST, int R, bool PAGED>
__global__ __launch_bounds__((Cfg<D, ST, R>::THREADS)) __attribute__((amdgpu_waves_per_eu(1)))
void decode_attn(A a) {
    using C = Cfg<D, ST, R>;
    constexpr int kWaves = C::WAVES, kThreads = C::THREADS;
    constexpr int EPC = C::EPC, LPK = C::LPK, KPW = C::KPW, U = C::U, NS = C::NS;
    constexpr int KPS = C::KPS, KPB = C::KPB, ESZ = C::ESZ;

    // Separate LDS objects: the ring and the query slots (written by LDS-DMA
    // and read only through the explicit reads above) and the merge area.
    __shared__ __attribute__((aligned(16))) uint8_t ring[C::RING_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t qslot[NS][C::QSLOT_BYTES];
    __shared__ float sm_o[kWaves][R][D];
    __shared__ float sm_m[kWaves][R];
    __shared__ float sm_l[kWaves][R];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane / LPK;
    const int sub = lane % LPK;
    const int rows_act = a.Gc * a.Tc;
    const float c = a.scale_log2;
    const float thresh = kRescaleLog2 / c;     // the threshold in raw q.k units
    const int qrow_bytes = D * (a.q_dtype == F32 ? 4 : 2);

    const int64_t x_begin = decode_slice_begin(a, blockIdx.x);
    int64_t x_end = x_begin + decode_slice_size(a, blockIdx.x);
    if (x_end > a.total_keys) x_end = a.total_keys;
    if (x_begin >= x_end) return;

    const char* kc = static_cast<const char*>(a.k_cache);
    const char* vc = static_cast<const char*>(a.v_cache);
    const char* qg = static_cast<const char*>(a.q);

    // -- segments: the one of unit (b, g) that starts at key-axis position x --
    auto make_seg = [&](int b, int g, int64_t x) __attribute__((always_inline)) -> Seg {
        Seg sg;
        sg.b = b;
        sg.g = g;
        const int64_t n_b = decode_div_hkv(a, a.prefix[b + 1] - a.prefix[b]);
        const int64_t unit_start = a.prefix[b] + static_cast<int64_t>(g) * n_b;
        int64_t seg_end = unit_start + n_b;
        if (seg_end > x_end) seg_end = x_end;
        sg.j0 = static_cast<int>(x - unit_start);
        sg.j1 = static_cast<int>(seg_end - unit_start);
        sg.n_b = static_cast<int>(n_b);
        sg.nbat = (sg.j1 - sg.j0 + KPB - 1) / KPB;
        sg.head = a.layer_off + b * a.row_stride + g * a.head_stride;
        sg.x_end = seg_end;
        sg.rec = (sg.j0 == 0 && sg.j1 == sg.n_b) ? -1 : static_cast<int64_t>(blockIdx.x) + b * a.Hkv + g;
        return sg;
    };
    auto locate = [&](int64_t x) __attribute__((always_inline)) -> Seg {
        int lo = 0, hi = a.rows;   // prefix[lo] <= x < prefix[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.prefix[mid] <= x) lo = mid; else hi = mid;
        }
        const int64_t n_b = decode_div_hkv(a, a.prefix[lo + 1] - a.prefix[lo]);
        return make_seg(lo, static_cast<int>(decode_quot(x - a.prefix[lo], n_b)), x);
    };
    // the segment after sg (which ended at its unit's end): the next unit
    auto next_seg = [&](const Seg& sg) __attribute__((always_inline)) -> Seg {
        int b = sg.b, g = sg.g + 1;
        if (g == a.Hkv) {
            g = 0;
            ++b;
        }
        return make_seg(b, g, sg.x_end);
    };
    // -- the slab's query rows of a segment into a query slot (wave 0; one
    //    LDS-DMA load per 1 KB; rows past the slab repeat its last row) --
    auto issue_q = [&](const Seg& sg, int slot) __attribute__((always_inline)) {
        const int cpr = qrow_bytes / 16;                 // 16-byte chunks per row
        const int n16 = R * cpr;
        for (int n = 0; n * 64 < n16; ++n) {
            int ch = n * 64 + lane;
            if (ch >= n16) ch = n16 - 1;
            int r = ch / cpr;
            const int part = ch - r * cpr;
            if (r >= rows_act) r = rows_act - 1;
            const int h = sg.g * a.G + a.r0 + r / a.Tc;
            const int i = a.i0 + r % a.Tc;
            const int64_t off = ((static_cast<int64_t>(a.row0 + sg.b) * a.Hq + h) * a.T + i) * qrow_bytes + part * 16;
            __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(qg + off),
                                             (void __attribute__((address_space(3)))*)(&qslot[slot][n * 1024]), 16, 0,
                                             0);
        }
    };

    // -- issue side: the next stage of this wave's keys. A finished segment is
    //    left at the start of the next call, for the next unit (wave 0 first
    //    loads that unit's queries); past the slice's end it reloads the last
    //    key (never used) --
    Seg is = locate(x_begin);
    int is_t = 0, is_sn = 0;
    bool is_live = true;
    // paged storage: the issue cursor's blocks (a work-group batch of KPB
    // keys, at most one block, spans at most two)
    PagedCursor<D> pg{};
    auto pg_enter = [&]() __attribute__((always_inline)) { pg.enter(a, is.b, is.g, is.j0 >> a.bshift); };
    if constexpr (PAGED) pg_enter();
    uint8_t* const ring_w = ring + wave * (NS * C::STAGE_BYTES);
    auto issue = [&](auto slot_c) __attribute__((always_inline)) {
        constexpr int S = decltype(slot_c)::value;
        if (is_live && is_t == is.nbat) {
            if (is.x_end < x_end) {
                is = next_seg(is);
                is_t = 0;
                ++is_sn;
                if (wave == 0) issue_q(is, is_sn % NS);
                if constexpr (PAGED) pg_enter();
            } else {
                is_live = false;
            }
        }
        if constexpr (PAGED) {
            const int blk = (is.j0 + is_t * KPB) >> a.bshift;
            if (is_live && blk != pg.blk) pg.step(a, is.b, is.g, blk);    // the batch starts in the next block
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int j = is.j0 + is_t * KPB + wave * KPS + u * KPW + grp;
            j = j < is.j1 ? j : is.j1 - 1;
            int64_t off;
            if constexpr (PAGED) {
                off = (pg.row(a, j) + sub * EPC) * ESZ;
            } else {
                off = (is.head + static_cast<int64_t>(j) * D + sub * EPC) * ESZ;
            }
            const char* kp = kc;
            const char* vp = vc;
            if (a.k_new != nullptr) {
                // fused append: the chunk's new keys come from the caller's input
                const int jn = j - (is.n_b - a.T);
                if (jn >= 0) {
                    kp = static_cast<const char*>(a.k_new);
                    vp = static_cast<const char*>(a.v_new);
                    off = ((((static_cast<int64_t>(a.row0 + is.b) * a.Hkv + is.g) * a.T + jn) * D) + sub * EPC) * ESZ;
                }
            }
            uint8_t* dst = ring_w + S * C::STAGE_BYTES + u * 2048;
            __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(kp + off),
                                             (void __attribute__((address_space(3)))*)(dst), 16, 0,
                                             KVC_DECODE_KV_CPOL);
            __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(vp + off),
                                             (void __attribute__((address_space(3)))*)(dst + 1024), 16, 0,
                                             KVC_DECODE_KV_CPOL);
        }
        if (is_live) ++is_t;
    };
    // -- consume side --
    const uint32_t rd_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                                 (__attribute__((address_space(3))) uint8_t*)ring_w)) + lane * 16;
    Seg cs = locate(x_begin);
    int cs_t = 0, cs_sn = 0;
    uint32_t qp[R][4];                 // the lane's 16 bytes of each query row
    int qpos[R];
    float m[R], l[R], o[R][EPC];
    auto start_segment = [&]() __attribute__((always_inline)) {
        load_q_rows<D, ST, R>(qp, lds_addr(qslot[cs_sn % NS]), a.q_dtype, sub);
        const int qpos0 = cs.n_b - a.Tc;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            qpos[r] = r < rows_act ? qpos0 + r % a.Tc : -1;
            m[r] = -INFINITY;
            l[r] = 0.f;
#pragma unroll
            for (int e = 0; e < EPC; ++e) o[r][e] = 0.f;
        }
    };

    auto consume = [&](auto slot_c) __attribute__((always_inline)) {
        constexpr int S = decltype(slot_c)::value;
        const int kb = cs.j0 + cs_t * KPB + wave * KPS;          // this wave's first key of the stage
        const bool plain = kb + KPS - 1 < cs.j1 && kb + KPS - 1 <= cs.n_b - a.Tc;
        u32x4 kx[U], vx[U];
        static_for<U>([&](auto u_c) {
            constexpr int u = decltype(u_c)::value;
            read_kv<S * C::STAGE_BYTES + u * 2048>(kx[u], vx[u], rd_addr);
        });
        float s[U * R];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float acc = 0.f;
                if constexpr (ST == F32) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc = fmaf(__uint_as_float(qp[r][e]), __uint_as_float(kx[u][e]), acc);
                } else {
                    acc = dot16<ST>(qp[r], kx[u], acc);
                }
                s[u * R + r] = acc;
            }
        }
        lane_group_sum<LPK, U * R>(s);
        if (!plain) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = kb + u * KPW + grp;
#pragma unroll
                for (int r = 0; r < R; ++r)
                    if (!(j < cs.j1 && j <= qpos[r])) s[u * R + r] = -INFINITY;
            }
        }
        // the reference max moves only when a score passes it by the threshold
        float mt[R];
        bool need = false;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            mt[r] = s[r];
#pragma unroll
            for (int u = 1; u < U; ++u) mt[r] = fmaxf(mt[r], s[u * R + r]);
            need |= mt[r] - m[r] > thresh;
        }
        if (__any(need)) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if (mt[r] - m[r] > thresh) {
                    const float alpha = m[r] == -INFINITY ? 0.f : fexp2((m[r] - mt[r]) * c);
                    m[r] = mt[r];
                    l[r] *= alpha;
#pragma unroll
                    for (int e = 0; e < EPC; ++e) o[r][e] *= alpha;
                }
            }
        }
        float nmc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) nmc[r] = m[r] == -INFINITY ? 0.f : -m[r] * c;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vf[EPC];
            unpack_v<ST, EPC>(vx[u], vf);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float p = fexp2(fmaf(s[u * R + r], c, nmc[r]));
                l[r] += p;
#pragma unroll
                for (int e = 0; e < EPC; ++e) o[r][e] = fmaf(p, vf[e], o[r][e]);
            }
        }
    };
    // -- end of a segment: merge the lane groups, then the waves; write the
    //    output itself or the segment's partial record --
    auto finish_segment = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float mw = m[r];
            mw = across_groups<LPK, true>(mw);
            const float w = mw == -INFINITY ? 0.f : fexp2((m[r] - mw) * c);
            float lw = l[r] * w;
            lw = across_groups<LPK, false>(lw);
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                float ow = o[r][e] * w;
                ow = across_groups<LPK, false>(ow);
                o[r][e] = ow;
            }
            m[r] = mw;
            l[r] = lw;
        }
        if (grp == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int e = 0; e < EPC; ++e) sm_o[wave][r][sub * EPC + e] = o[r][e];
        }
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                sm_m[wave][r] = m[r];
                sm_l[wave][r] = l[r];
            }
        }
        lds_barrier();
        for (int idx = tid; idx < rows_act * D; idx += kThreads) {
            const int r = idx / D, d = idx - (idx / D) * D;
            float M = sm_m[0][r];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][r]);
            float ov = 0.f, lv = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float f = sm_m[w][r] == -INFINITY ? 0.f : fexp2((sm_m[w][r] - M) * c);
                ov = fmaf(sm_o[w][r][d], f, ov);
                lv = fmaf(sm_l[w][r], f, lv);
            }
            if (cs.rec < 0) {
                const int h = cs.g * a.G + a.r0 + r / a.Tc;
                const int i = a.i0 + r % a.Tc;
                a.out[((static_cast<int64_t>(a.row0 + cs.b) * a.Hq + h) * a.T + i) * D + d] = ov / lv;
            } else {
                const int64_t rr = cs.rec * a.rec_rows + r;
                a.ws_o[rr * D + d] = ov;
                if (d == 0) {
                    a.ws_ml[rr * 2] = M;
                    a.ws_ml[rr * 2 + 1] = lv;
                }
            }
        }
        lds_barrier();
    };

    // -- the loop: stage t sits in slot t % NS; NS - 1 stages are issued ahead.
    //    Wave 0 loads the first segment's queries before them; every wave
    //    reads them once they have landed --
    if (wave == 0) issue_q(is, 0);
    static_for<NS - 1>([&](auto k) { issue(k); });
    if (wave == 0) wait_vm<(NS - 1) * 2 * U>();    // the query loads precede every stage load
    lds_barrier();
    start_segment();
    bool done = false;
    auto step = [&](auto slot_c) __attribute__((always_inline)) {
        constexpr int S = decltype(slot_c)::value;
        issue(std::integral_constant<int, (S + NS - 1) % NS>{});
        wait_vm<(NS - 1) * 2 * U>();      // this stage's loads have landed
        consume(slot_c);
        if (++cs_t == cs.nbat) {
            // the next segment's queries were loaded before its first stage,
            // which the wait above covers for wave 0; the barriers in
            // finish_segment make them visible to every wave
            finish_segment();
            if (cs.x_end >= x_end) {
                done = true;
            } else {
                cs = next_seg(cs);
                cs_t = 0;
                ++cs_sn;
                start_segment();
            }
        }
    };
    while (!done) {
        static_for<NS>([&](auto k) {
            if (!done) step(k);
        });
    }
    wait_vm<0>();   // the ring's trailing reloads land before the work-group ends
}

// ---- slabs of 9 to 32 query rows: row-split work-groups --------------------
// A KV head with more query rows than one lane group holds (for example 8 heads
// x a 4-token draft block) is served by RS waves of 8 rows each over the same
// keys, so the cache is streamed once for all of them. The work-group shares
// one LDS ring: each wave loads its share of a stage (UB 1 KB blocks of K and
// of V), waits for its own loads, and one barrier per stage makes the stage
// visible to all waves and frees the one read before. Each wave merges only its
// lane groups and writes its own rows; there is no cross-wave merge.

#ifndef KVC_DECODE_ROWS_UB
#define KVC_DECODE_ROWS_UB 2          // 1 KB blocks per tensor each wave loads per stage
#endif
#ifndef KVC_DECODE_ROWS_STAGES
#define KVC_DECODE_ROWS_STAGES 3
#endif

template <int D, int ST, int RS>
struct RCfg {
    static constexpr int ESZ = ST == F32 ? 4 : 2;
    static constexpr int EPC = 16 / ESZ;
    static constexpr int LPK = D / EPC;
    static constexpr int KPW = 64 / LPK;               // keys per 1 KB block
    static constexpr int R = 8;                        // query rows per wave
    static constexpr int ROWS = RS * R;
    static constexpr int THREADS = 64 * RS;
    static constexpr int UB = KVC_DECODE_ROWS_UB;
    static constexpr int BLOCKS = RS * UB;             // blocks per tensor per stage
    static constexpr int KPS = BLOCKS * KPW;           // keys per stage
    static constexpr int STAGE_BYTES = BLOCKS * 2048;
    static constexpr int QSEGS = 2;                    // segments the query table holds
    static constexpr int QROW_WORDS = D * ESZ / 4;
    static constexpr int FIXED_BYTES = QSEGS * ROWS * D * ESZ;
    static constexpr int fit_stages() {
        int ns = KVC_DECODE_ROWS_STAGES;
        while (ns > 2 && (ns * STAGE_BYTES + FIXED_BYTES) * 2 > kLdsLimit) --ns;
        return ns;
    }
    static constexpr int NS = fit_stages();
    static constexpr int LDS_BYTES = NS * STAGE_BYTES + FIXED_BYTES;
    static_assert(LDS_BYTES <= kLdsLimit, "decode LDS budget");
    static_assert(NS * STAGE_BYTES < 65536, "ring offsets fit the LDS immediate");
};

template <class A, int D, int ST, int RS, bool PAGED>
__global__ __launch_bounds__((RCfg<D, ST, RS>::THREADS)) __attribute__((amdgpu_waves_per_eu(1)))
void decode_rows(A a) {
    using C = RCfg<D, ST, RS>;
    constexpr int EPC = C::EPC, LPK = C::LPK, KPW = C::KPW, UB = C::UB, NS = C::NS, R = C::R;
    constexpr int KPS = C::KPS, ESZ = C::ESZ, ROWS = C::ROWS;

    __shared__ __attribute__((aligned(16))) uint8_t ring[NS * C::STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) uint32_t qtab[C::QSEGS][ROWS][C::QROW_WORDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane / LPK;
    const int sub = lane % LPK;
    const int rows_act = a.Gc * a.Tc;
    const float c = a.scale_log2;
    const float thresh = kRescaleLog2 / c;

    const int64_t x_begin = decode_slice_begin(a, blockIdx.x);
    int64_t x_end = x_begin + decode_slice_size(a, blockIdx.x);
    if (x_end > a.total_keys) x_end = a.total_keys;
    if (x_begin >= x_end) return;

    const char* kc = static_cast<const char*>(a.k_cache);
    const char* vc = static_cast<const char*>(a.v_cache);

    auto locate = [&](int64_t x) __attribute__((always_inline)) -> Seg {
        int lo = 0, hi = a.rows;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.prefix[mid] <= x) lo = mid; else hi = mid;
        }
        Seg sg;
        sg.b = lo;
        const int64_t n_b = decode_div_hkv(a, a.prefix[lo + 1] - a.prefix[lo]);
        sg.g = static_cast<int>(decode_quot(x - a.prefix[lo], n_b));
        const int64_t unit_start = a.prefix[lo] + static_cast<int64_t>(sg.g) * n_b;
        int64_t seg_end = unit_start + n_b;
        if (seg_end > x_end) seg_end = x_end;
        sg.j0 = static_cast<int>(x - unit_start);
        sg.j1 = static_cast<int>(seg_end - unit_start);
        sg.n_b = static_cast<int>(n_b);
        sg.nbat = (sg.j1 - sg.j0 + KPS - 1) / KPS;
        sg.head = a.layer_off + sg.b * a.row_stride + sg.g * a.head_stride;
        sg.x_end = seg_end;
        sg.rec = (sg.j0 == 0 && sg.j1 == sg.n_b) ? -1 : static_cast<int64_t>(blockIdx.x) + sg.b * a.Hkv + sg.g;
        return sg;
    };

    auto load_qtab = [&](int64_t x) __attribute__((always_inline)) {
        for (int sgi = 0; sgi < C::QSEGS && x < x_end; ++sgi) {
            const Seg sg = locate(x);
            for (int idx = tid; idx < ROWS * D; idx += C::THREADS) {
                const int r = idx / D, e = idx - (idx / D) * D;
                float val = 0.f;
                if (r < rows_act) {
                    const int h = sg.g * a.G + a.r0 + r / a.Tc;
                    const int i = a.i0 + r % a.Tc;
                    const int64_t qe = ((static_cast<int64_t>(a.row0 + sg.b) * a.Hq + h) * a.T + i) * D + e;
                    if (a.q_dtype == F32) val = static_cast<const float*>(a.q)[qe];
                    else if (a.q_dtype == BF16) val = bf16_to_f32(static_cast<const uint16_t*>(a.q)[qe]);
                    else val = f16_to_f32(static_cast<const uint16_t*>(a.q)[qe]);
                }
                if constexpr (ST == F32) {
                    reinterpret_cast<float*>(qtab[sgi][r])[e] = val;
                } else {
                    const uint32_t h16 = ST == BF16 ? f32_to_bf16_rne(val) : f32_to_f16_rne(val);
                    reinterpret_cast<uint16_t*>(qtab[sgi][r])[e] = static_cast<uint16_t>(h16);
                }
            }
            x = sg.x_end;
        }
        __syncthreads();
    };

    // -- issue side: this wave's UB blocks of the next stage --
    Seg is = locate(x_begin);
    int is_t = 0;
    bool is_live = true;
    // paged storage: the issue cursor's blocks (a stage of KPS keys spans at
    // most two)
    PagedCursor<D> pg{};
    auto pg_enter = [&]() __attribute__((always_inline)) { pg.enter(a, is.b, is.g, is.j0 >> a.bshift); };
    if constexpr (PAGED) pg_enter();
    auto issue = [&](auto slot_c) __attribute__((always_inline)) {
        constexpr int S = decltype(slot_c)::value;
        if constexpr (PAGED) {
            const int blk = (is.j0 + is_t * KPS) >> a.bshift;
            if (is_live && blk != pg.blk) pg.step(a, is.b, is.g, blk);    // the stage starts in the next block
        }
#pragma unroll
        for (int ub = 0; ub < UB; ++ub) {
            const int bi = wave * UB + ub;
            int j = is.j0 + is_t * KPS + bi * KPW + grp;
            j = j < is.j1 ? j : is.j1 - 1;
            int64_t off;
            if constexpr (PAGED)
                off = (pg.row(a, j) + sub * EPC) * ESZ;
            else
                off = (is.head + static_cast<int64_t>(j) * D + sub * EPC) * ESZ;
            uint8_t* dst = ring + S * C::STAGE_BYTES + bi * 2048;
            __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(kc + off),
                                             (void __attribute__((address_space(3)))*)(dst), 16, 0,
                                             KVC_DECODE_KV_CPOL);
            __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(vc + off),
                                             (void __attribute__((address_space(3)))*)(dst + 1024), 16, 0,
                                             KVC_DECODE_KV_CPOL);
        }
        if (is_live && ++is_t == is.nbat) {
            if (is.x_end >= x_end) {
                is_live = false;
            } else {
                is = locate(is.x_end);
                is_t = 0;
                if constexpr (PAGED) pg_enter();
            }
        }
    };

    // -- consume side: this wave's rows wave * R .. wave * R + R - 1 of the slab --
    const uint32_t rd_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                                 (__attribute__((address_space(3))) uint8_t*)ring)) + lane * 16;
    Seg cs = locate(x_begin);
    int cs_t = 0, cs_q = 0;
    uint32_t qp[R][4];
    int qpos[R];
    float m[R], l[R], o[R][EPC];
    auto start_segment = [&]() __attribute__((always_inline)) {
        const int qpos0 = cs.n_b - a.Tc;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int rr = wave * R + r;
            const u32x4 w = *reinterpret_cast<const u32x4*>(&qtab[cs_q][rr][sub * 4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) qp[r][e] = w[e];
            qpos[r] = rr < rows_act ? qpos0 + rr % a.Tc : -1;
            m[r] = -INFINITY;
            l[r] = 0.f;
#pragma unroll
            for (int e = 0; e < EPC; ++e) o[r][e] = 0.f;
        }
    };

    auto consume = [&](auto slot_c) __attribute__((always_inline)) {
        constexpr int S = decltype(slot_c)::value;
        const int kb = cs.j0 + cs_t * KPS;               // first key of the stage
        const bool plain = kb + KPS - 1 < cs.j1 && kb + KPS - 1 <= cs.n_b - a.Tc;
        static_for<C::BLOCKS>([&](auto bi_c) {
            constexpr int bi = decltype(bi_c)::value;
            u32x4 kx, vx;
            read_kv<S * C::STAGE_BYTES + bi * 2048>(kx, vx, rd_addr);
            float s[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float acc = 0.f;
                if constexpr (ST == F32) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc = fmaf(__uint_as_float(qp[r][e]), __uint_as_float(kx[e]), acc);
                } else {
                    acc = dot16<ST>(qp[r], kx, acc);
                }
                s[r] = acc;
            }
            lane_group_sum<LPK, R>(s);
            if (!plain) {
                const int j = kb + bi * KPW + grp;
#pragma unroll
                for (int r = 0; r < R; ++r)
                    if (!(j < cs.j1 && j <= qpos[r])) s[r] = -INFINITY;
            }
            bool need = false;
#pragma unroll
            for (int r = 0; r < R; ++r) need |= s[r] - m[r] > thresh;
            if (__any(need)) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if (s[r] - m[r] > thresh) {
                        const float alpha = m[r] == -INFINITY ? 0.f : fexp2((m[r] - s[r]) * c);
                        m[r] = s[r];
                        l[r] *= alpha;
#pragma unroll
                        for (int e = 0; e < EPC; ++e) o[r][e] *= alpha;
                    }
                }
            }
            float vf[EPC];
            unpack_v<ST, EPC>(vx, vf);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float p = fexp2(fmaf(s[r], c, m[r] == -INFINITY ? 0.f : -m[r] * c));
                l[r] += p;
#pragma unroll
                for (int e = 0; e < EPC; ++e) o[r][e] = fmaf(p, vf[e], o[r][e]);
            }
        });
    };

    // -- end of a segment: merge this wave's lane groups, write its rows --
    auto finish_segment = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float mw = m[r];
            mw = across_groups<LPK, true>(mw);
            const float w = mw == -INFINITY ? 0.f : fexp2((m[r] - mw) * c);
            float lw = l[r] * w;
            lw = across_groups<LPK, false>(lw);
            float ow[EPC];
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                ow[e] = o[r][e] * w;
                ow[e] = across_groups<LPK, false>(ow[e]);
            }
            const int rr = wave * R + r;
            if (grp == 0 && rr < rows_act) {
                if (cs.rec < 0) {
                    const int h = cs.g * a.G + a.r0 + rr / a.Tc;
                    const int i = a.i0 + rr % a.Tc;
                    float* dst = a.out + ((static_cast<int64_t>(a.row0 + cs.b) * a.Hq + h) * a.T + i) * D + sub * EPC;
#pragma unroll
                    for (int e = 0; e < EPC; ++e) dst[e] = ow[e] / lw;
                } else {
                    const int64_t rec = cs.rec * a.rec_rows + rr;
#pragma unroll
                    for (int e = 0; e < EPC; ++e) a.ws_o[rec * D + sub * EPC + e] = ow[e];
                    if (sub == 0) {
                        a.ws_ml[rec * 2] = mw;
                        a.ws_ml[rec * 2 + 1] = lw;
                    }
                }
            }
        }
    };

    // -- the loop: stage t in slot t % NS, NS - 1 stages issued ahead --
    static_for<NS - 1>([&](auto k) { issue(k); });
    load_qtab(x_begin);
    start_segment();
    bool done = false;
    auto step = [&](auto slot_c) __attribute__((always_inline)) {
        constexpr int S = decltype(slot_c)::value;
        wait_vm<(NS - 2) * 2 * UB>();   // this wave's part of stage t has landed
        lds_barrier();                   // every wave's part has; every wave is done with stage t - 1
        issue(std::integral_constant<int, (S + NS - 1) % NS>{});
        consume(slot_c);
        if (++cs_t == cs.nbat) {
            finish_segment();
            if (cs.x_end >= x_end) {
                done = true;
            } else {
                cs = locate(cs.x_end);
                cs_t = 0;
                if (++cs_q == C::QSEGS) {    // more segments than the table holds: reload it
                    load_qtab(cs.x_end - (cs.j1 - cs.j0));
                    cs_q = 0;
                }
                start_segment();
            }
        }
    };
    while (!done) {
        static_for<NS>([&](auto k) {
            if (!done) step(k);
        });
    }
    wait_vm<0>();
}

// ---- slabs of 5 to 32 query rows, 16-bit caches: matrix cores --------------
// With 8 heads x a 4-token draft (or any G*T in 5..32) one KV head serves up to
// 32 query rows, up to 32 flops per byte: the vector ALUs do not keep up with
// HBM (at 8 rows they already trail the matrix-core kernel by a third), so
// the two products run as MFMA tiles, the same S^T = K Q^T and O^T = V^T P^T
// tiles as the prefill kernel, with the slab's rows as the 32 columns. One wave
// per work-group streams 32-key K and V tiles of its slice through a private
// LDS ring (LDS-DMA, explicit vmcnt waits, no barrier); the slab queries of its
// first segments sit in an LDS table; each segment ends in a partial record
// (or the output) per column, merged by decode_combine.

#ifndef KVC_DECODE_MFMA_STAGES
#define KVC_DECODE_MFMA_STAGES 2       // one tile in flight per wave ...
#endif
#ifndef KVC_DECODE_MFMA_BLOCKS_PER_CU
#define KVC_DECODE_MFMA_BLOCKS_PER_CU 3   // ... and three waves per CU (measured best at d_h 128)
#endif
// smaller heads: a wave's chain of waits, products and softmax per 32-key
// tile serves fewer bytes, so more single-wave work-groups share a CU (their
// registers allow it). Batched decode (B scaled to the same bytes), % of HBM
// peak by work-groups per CU: d_h 64: 3 69.7, 4 71.9, 5 68.4, 6 68.9; d_h 32:
// 3 48.6, 4 61.2, 5 59.8, 6 64.8, 7 67.4, 8 68.0, 10 64.2, 12 68.0
#ifndef KVC_DECODE_MFMA_BLOCKS_PER_CU_D64
#define KVC_DECODE_MFMA_BLOCKS_PER_CU_D64 4
#endif
#ifndef KVC_DECODE_MFMA_BLOCKS_PER_CU_D32
#define KVC_DECODE_MFMA_BLOCKS_PER_CU_D32 8
#endif
template <int D>
constexpr int mfma_blocks_per_cu() {
    return D == 128 ? KVC_DECODE_MFMA_BLOCKS_PER_CU : D == 64 ? KVC_DECODE_MFMA_BLOCKS_PER_CU_D64
                                                              : KVC_DECODE_MFMA_BLOCKS_PER_CU_D32;
}
#ifndef KVC_DECODE_MFMA_QSEGS
#define KVC_DECODE_MFMA_QSEGS 2
#endif
#ifndef KVC_DECODE_MFMA_PSPLIT
#define KVC_DECODE_MFMA_PSPLIT 1      // 1: P as a 16-bit hi + lo pair (two products with V); 0: P rounded once
#endif
#ifndef KVC_DECODE_MFMA_MIN_ROWS
#define KVC_DECODE_MFMA_MIN_ROWS 1    // 16-bit slabs with fewer rows run on the vector kernel
#endif
#ifndef KVC_DECODE_TIMESTAMPS
#define KVC_DECODE_TIMESTAMPS 0   // 1: per-work-group timestamps for kv_cached_gqa_amd.probe (never in the library)
#endif
#if KVC_DECODE_TIMESTAMPS
// Timestamp probe: per matrix-core decode work-group its start, first segment
// located, first tile issued and end (s_memrealtime, 100 MHz), its XCC and
// hardware ids and its slice's keys; per merge block its start, contributors
// known, records merged and end. Each launch overwrites what it records.
constexpr int kProbeMergeBlocks = 16384;
static __device__ unsigned long long kvc_probe_wg[kMaxDecodeBlocks * 6];
static __device__ unsigned long long kvc_probe_merge[kProbeMergeBlocks * 4];
__device__ __forceinline__ unsigned long long probe_now() { return __builtin_amdgcn_s_memrealtime(); }
__device__ __forceinline__ unsigned long long probe_ids() {
    unsigned x, h;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(h));
    return (static_cast<unsigned long long>(x) << 32) | h;
}
#endif

#ifndef KVC_DECODE_MFMA_UNIT_PAD
// virtual keys charged to every unit on the key axis: a work-group whose slice
// holds a unit boundary streams a part tile on each side of it, about one tile
// more for the same keys (the latest work-groups of the batched-decode call
// were all such)
#define KVC_DECODE_MFMA_UNIT_PAD 48   // measured: 0 65.3, 16 65.0, 32 64.8, 48 64.3-64.6, 64-112 64.6-65.1 us per batched-decode call
#endif
#ifndef KVC_DECODE_MFMA_LATE_PCT
// equal slices: with three single-wave work-groups per CU an uneven split
// measured slower on the long-context workload (e.g. 193 against 180 us at a
// 4-token draft with 70%)
#define KVC_DECODE_MFMA_LATE_PCT 100
#endif

template <int D>
struct MCfg : TileLayout<D> {
    using L = TileLayout<D>;
    static constexpr int QSEGS = KVC_DECODE_MFMA_QSEGS;      // segments the query table holds
    static constexpr int QT_BYTES = QSEGS * 32 * D * 2;      // 32 columns of D 16-bit elements each
    static constexpr int fit_stages() {
        int ns = KVC_DECODE_MFMA_STAGES;
        while (ns > 2 && ((ns * 2 * L::TILE_BYTES + QT_BYTES) * mfma_blocks_per_cu<D>() > kLdsLimit ||
                          ns * 2 * L::TILE_BYTES + 24 * D * 2 > 65535))
            --ns;
        return ns;
    }
    static constexpr int NS = fit_stages();
    static constexpr int STAGE_BYTES = 2 * L::TILE_BYTES;    // K tile, then V tile
    static constexpr int LDS_BYTES = NS * STAGE_BYTES;
    static_assert((NS - 1) * 2 * L::NLD < 64, "vmcnt field");
    static_assert((NS - 1) * STAGE_BYTES + L::TILE_BYTES + 24 * D * 2 < 65536, "LDS read offsets fit 16 bits");
};

template <class A, int D, int ST, bool PAGED>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1)))
void decode_mfma(A a) {
    using P = MCfg<D>;
    constexpr int NS = P::NS, DS = P::DS, DT = P::DT, NLD = P::NLD;
    __shared__ __attribute__((aligned(16))) uint16_t smem[P::LDS_BYTES / 2];
    __shared__ __attribute__((aligned(16))) uint16_t qtab[P::QSEGS][32][D];

    const int lane = threadIdx.x;
    const int col32 = lane & 31;                 // this lane's column: slab row col32
    const int hl = lane >> 5;
    const int rows_act = a.Gc * a.Tc;
    const float c = a.scale_log2;
    const float thresh = kRescaleLog2 / c;

#if KVC_DECODE_TIMESTAMPS
    const unsigned long long pt_start = probe_now();
#endif
    const auto pfx = load_prefix_lanes<A>();   // in flight while the slice is worked out
    // The scalars that locating the first segment needs, read from the
    // arguments in one round trip and held as opaque copies (the compiler would
    // otherwise read each again near its use, one dependent wait each), and the
    // argument lines the first tile's addresses need, fetched in the same trip.
    int64_t kpb = a.keys_per_block, kpbo = a.keys_per_block_odd, kpb2 = a.keys_per_block2,
            kpb2o = a.keys_per_block2_odd, total = a.total_keys;
    int32_t n1 = a.n_first, hkv = a.Hkv, upad = a.unit_pad, hshift = a.hkv_shift, nrows = a.rows;
    uint64_t hinv = a.hkv_inv;
    asm volatile("" : "+s"(kpb), "+s"(kpbo), "+s"(kpb2), "+s"(kpb2o), "+s"(total), "+s"(n1), "+s"(hkv), "+s"(upad),
                 "+s"(hshift), "+s"(hinv), "+s"(nrows)
                 : "s"(a.k_cache), "s"(a.v_cache), "s"(a.layer_off), "s"(a.row_stride), "s"(a.head_stride),
                   "s"(a.T), "s"(a.row0), "s"(a.k_new), "s"(a.v_new), "s"(a.prefix[A::kPrefix - 1]));
    const int64_t x_begin = decode_slice_begin(blockIdx.x, n1, kpb, kpbo, kpb2, kpb2o);
    int64_t x_end = x_begin + decode_slice_size(blockIdx.x, n1, kpb, kpbo, kpb2, kpb2o);
    if (x_end > total) x_end = total;
    if (x_begin >= x_end) return;

    const uint16_t* kg = static_cast<const uint16_t*>(a.k_cache);
    const uint16_t* vg = static_cast<const uint16_t*>(a.v_cache);

    // the segment at padded position x of row lo, whose units start at p0 and
    // end at p1 on the padded axis: each unit is unit_pad virtual keys, then
    // its n_b real ones; a segment that holds no real key has nbat = 0
    const int64_t row_pad = static_cast<int64_t>(hkv) * upad;
    // (unit (b, g) of a row starting at p0 whose units are n_e long, x inside it)
    auto seg_make = [&](int b, int g, int64_t n_e, int64_t p0, int64_t x) __attribute__((always_inline)) -> Seg {
        Seg sg;
        sg.b = b;
        sg.g = g;
        const int64_t unit_start = p0 + static_cast<int64_t>(g) * n_e + upad;   // its first real key
        int64_t seg_end = unit_start + (n_e - upad);
        if (seg_end > x_end) seg_end = x_end;
        sg.j0 = x > unit_start ? static_cast<int>(x - unit_start) : 0;
        sg.j1 = static_cast<int>(seg_end - unit_start);
        sg.n_b = static_cast<int>(n_e - upad);
        sg.nbat = sg.j1 > sg.j0 ? (sg.j1 - sg.j0 + kBN - 1) / kBN : 0;
        sg.head = a.layer_off + sg.b * a.row_stride + sg.g * a.head_stride;
        sg.x_end = seg_end;
        sg.rec = (sg.j0 == 0 && sg.j1 == sg.n_b) ? -1 : static_cast<int64_t>(blockIdx.x) + sg.b * a.Hkv + sg.g;
        return sg;
    };
    // the segment after sg, which ended at its unit's end inside the slice:
    // the next KV head of the row, or the first of the next row (whose end is
    // the one prefix entry read here)
    auto locate_next = [&](const Seg& sg) __attribute__((always_inline)) -> Seg {
        const int64_t n_e = static_cast<int64_t>(sg.n_b) + upad;
        if (sg.g + 1 < hkv) return seg_make(sg.b, sg.g + 1, n_e, sg.x_end - static_cast<int64_t>(sg.g + 1) * n_e, sg.x_end);
        const int64_t p1 = a.prefix[sg.b + 2] + (sg.b + 2) * row_pad;
        return seg_make(sg.b + 1, 0, decode_div_exact(p1 - sg.x_end, hshift, hinv), sg.x_end, sg.x_end);
    };
    // the first segment, found without a search's chain of scalar loads: its
    // row from the prefix entries' ballots, its KV head g from a ballot of
    // l * n_e <= x - p0 over lanes l = 1 .. Hkv - 1 (a division past 64 heads)
    const Seg first = [&]() __attribute__((always_inline)) {
        const RowOf r = nrows < 64 ? row_of_one(pfx.e[0], x_begin, row_pad) : row_of(pfx, x_begin, row_pad);
        const int64_t n_e = decode_div_exact(r.p1 - r.p0, hshift, hinv);
        const int64_t dx = x_begin - r.p0;
        int g;
        if (hkv <= 64) {
            const int l = static_cast<int>(threadIdx.x) & 63;
            g = static_cast<int>(__popcll(__ballot(l >= 1 && l < hkv && static_cast<int64_t>(l) * n_e <= dx)));
        } else {
            g = static_cast<int>(decode_quot(dx, n_e));
        }
        return seg_make(r.b, g, n_e, r.p0, x_begin);
    }();
    if (first.nbat == 0) return;   // a slice of virtual keys only
#if KVC_DECODE_TIMESTAMPS
    const unsigned long long pt_located = probe_now();
#endif

    // -- the query table: 32 columns (slab rows; past the slab zero) per segment,
    //    rounded to the storage type --
    auto load_qtab = [&](const Seg& s0) __attribute__((always_inline)) {
        Seg sg = s0;
        for (int sgi = 0; sgi < P::QSEGS; ++sgi) {
            if (sgi > 0) {
                if (sg.x_end >= x_end) break;
                sg = locate_next(sg);
                if (sg.nbat == 0) break;
            }
            if (a.q_dtype == ST) {
                // q already in the storage type: 8 elements (16 bytes) at a time
                for (int c8 = lane; c8 < 4 * D; c8 += 64) {
                    const int r = c8 / (D / 8), e = (c8 - r * (D / 8)) * 8;
                    u32x4 w = {0u, 0u, 0u, 0u};
                    if (r < rows_act) {
                        const int h = sg.g * a.G + a.r0 + r / a.Tc;
                        const int i = a.i0 + r % a.Tc;
                        const int64_t qe = ((static_cast<int64_t>(a.row0 + sg.b) * a.Hq + h) * a.T + i) * D + e;
                        w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.q) + qe);
                    }
                    *reinterpret_cast<u32x4*>(&qtab[sgi][r][e]) = w;
                }
                continue;
            }
            for (int idx = lane; idx < 32 * D; idx += 64) {
                const int r = idx / D, e = idx - (idx / D) * D;
                float val = 0.f;
                if (r < rows_act) {
                    const int h = sg.g * a.G + a.r0 + r / a.Tc;
                    const int i = a.i0 + r % a.Tc;
                    const int64_t qe = ((static_cast<int64_t>(a.row0 + sg.b) * a.Hq + h) * a.T + i) * D + e;
                    if (a.q_dtype == F32) val = static_cast<const float*>(a.q)[qe];
                    else if (a.q_dtype == BF16) val = bf16_to_f32(static_cast<const uint16_t*>(a.q)[qe]);
                    else val = f16_to_f32(static_cast<const uint16_t*>(a.q)[qe]);
                }
                qtab[sgi][r][e] = static_cast<uint16_t>(ST == BF16 ? f32_to_bf16_rne(val) : f32_to_f16_rne(val));
            }
        }
        __syncthreads();
    };

    // -- issue side: the next 32-key tile, K chunks XOR-swizzled, V chunks
    //    permuted for the transposed reads; nothing once the slice is done --
    Seg is = first;
    int is_t = 0;
    bool is_live = true;
    // paged storage: the issue cursor's blocks (a 32-key tile spans at most
    // two)
    PagedCursor<D> pg{};
    auto pg_enter = [&]() __attribute__((always_inline)) { pg.enter(a, is.b, is.g, is.j0 >> a.bshift); };
    if constexpr (PAGED) pg_enter();
    // byte offsets, inside a tile, of this lane's 16 bytes of each load (D =
    // 128: load n covers rows 4n .. 4n + 3; the K chunks' swizzle repeats
    // every 4 loads, so ko4[n % 4] + (n / 4) * 4096 is load n's; the V
    // permutation depends on the row mod 4 only, so vo0 + 1024 n is)
    uint32_t ko4[4], vo0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int e = m * 512 + lane * 8;
        const int r = e / D;
        const int sl = (e % D) >> 3;
        ko4[m] = static_cast<uint32_t>(r * D + P::kslot(r, sl) * 8) * 2u;
        if (m == 0) vo0 = static_cast<uint32_t>(r * D + P::vchunk(r, sl) * 8) * 2u;
    }
    auto issue = [&](auto slot_c) __attribute__((always_inline)) {
        constexpr int S = decltype(slot_c)::value;
        if (!is_live) return;
        uint16_t* kd = smem + S * P::STAGE_BYTES / 2;
        uint16_t* vd = kd + P::TILE;
        if constexpr (PAGED) {
            const int blk = (is.j0 + is_t * kBN) >> a.bshift;
            if (is_live && blk != pg.blk) pg.step(a, is.b, is.g, blk);    // the tile starts in the next block
        }
        // a fused append's new keys (the unit's last T) sit in its last tile at
        // most: only a tile that reaches them selects an address per lane
        const bool new_keys = a.k_new != nullptr && is.j0 + (is_t + 1) * kBN > is.n_b - a.T;
        const int j0t = is.j0 + is_t * kBN;
        bool whole = j0t + kBN <= is.j1 && !new_keys;    // 32 keys of the cache, no row clamped
        if constexpr (PAGED) whole = whole && ((j0t + kBN - 1) >> a.bshift) == (j0t >> a.bshift);
        if (whole) {
            // the tile's rows are consecutive: one uniform base per tensor, and
            // a 32-bit offset per lane and load (the same for every tile)
            int64_t tb;
            if constexpr (PAGED)
                tb = pg.row(a, j0t);
            else
                tb = is.head + static_cast<int64_t>(j0t) * D;
            const char* kb = reinterpret_cast<const char*>(kg + tb);
            const char* vb = reinterpret_cast<const char*>(vg + tb);
#pragma unroll
            for (int n = 0; n < NLD; ++n) {
                uint32_t ko, vo;
                if constexpr (D == 128) {
                    ko = ko4[n & 3];
                    vo = vo0;
                } else {
                    const int e = n * 512 + lane * 8;
                    const int r = e / D;
                    const int sl = (e % D) >> 3;
                    ko = static_cast<uint32_t>(r * D + P::kslot(r, sl) * 8) * 2u;
                    vo = static_cast<uint32_t>(r * D + P::vchunk(r, sl) * 8) * 2u;
                }
                // (D = 128: the uniform part of each load's address first)
                const char* kbn = D == 128 ? kb + (n >> 2) * 4096 : kb;
                const char* vbn = D == 128 ? vb + n * 1024 : vb;
                __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(kbn + ko),
                                                 (void __attribute__((address_space(3)))*)(kd + n * 512), 16, 0,
                                                 KVC_DECODE_MFMA_KV_CPOL);
                __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(vbn + vo),
                                                 (void __attribute__((address_space(3)))*)(vd + n * 512), 16, 0,
                                                 KVC_DECODE_MFMA_KV_CPOL);
            }
        }
#pragma unroll
        for (int n = 0; n < NLD && !whole; ++n) {
            const int e = n * 512 + lane * 8;    // element offset inside the tile
            const int r = e / D;
            const int sl = (e % D) >> 3;
            int j = j0t + r;
            j = j < is.j1 ? j : is.j1 - 1;
            int64_t row;
            if constexpr (PAGED)
                row = pg.row(a, j);
            else
                row = is.head + static_cast<int64_t>(j) * D;
            const uint16_t* kp = kg;
            const uint16_t* vp = vg;
            if (new_keys) {
                // fused append: the chunk's new keys come from the caller's input
                const int jn = j - (is.n_b - a.T);
                if (jn >= 0) {
                    kp = static_cast<const uint16_t*>(a.k_new);
                    vp = static_cast<const uint16_t*>(a.v_new);
                    row = ((static_cast<int64_t>(a.row0 + is.b) * a.Hkv + is.g) * a.T + jn) * D;
                }
            }
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1)))*)(kp + row + P::kslot(r, sl) * 8),
                (void __attribute__((address_space(3)))*)(kd + n * 512), 16, 0, KVC_DECODE_MFMA_KV_CPOL);
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1)))*)(vp + row + P::vchunk(r, sl) * 8),
                (void __attribute__((address_space(3)))*)(vd + n * 512), 16, 0, KVC_DECODE_MFMA_KV_CPOL);
        }
        if (is_live && ++is_t == is.nbat) {
            if (is.x_end >= x_end) {
                is_live = false;
            } else {
                is = locate_next(is);
                is_t = 0;
                if (is.nbat == 0) is_live = false;          // the slice ends in virtual keys
                else if constexpr (PAGED) pg_enter();
            }
        }
    };

    // -- LDS read addresses of this lane (stage offsets are immediates) --
    const uint32_t lds0 = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint16_t*)smem));
    uint32_t kaddr[DS];
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) kaddr[ds] = lds0 + (col32 * D + P::kslot(col32, 2 * ds + hl) * 8) * 2;
    uint32_t vaddr[DT];
    {
        const int grp = lane >> 4, ii = (lane >> 2) & 3, aa = lane & 3;
        const int rv = (grp >> 1) * 4 + ii;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int cv = dt * 4 + 2 * (grp & 1) + (aa >> 1);
            vaddr[dt] = lds0 + P::TILE_BYTES + (rv * D + P::vslot(rv, cv) * 8) * 2 + (aa & 1) * 8;
        }
    }

    // -- consume side --
    Seg cs = first;
    int cs_t = 0, cs_q = 0;
    u32x4 qb[DS];
    int qpos;
    float m, lsum;
    f32x16_t o[DT];
    auto start_segment = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
            qb[ds] = *reinterpret_cast<const u32x4*>(&qtab[cs_q][col32][ds * 16 + hl * 8]);
        qpos = col32 < rows_act ? cs.n_b - a.Tc + col32 % a.Tc : -1;
        m = -INFINITY;
        lsum = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16_t{};
    };

    auto consume = [&](auto slot_c) __attribute__((always_inline)) {
        constexpr int S = decltype(slot_c)::value;
        const int j0 = cs.j0 + cs_t * kBN;
        const bool plain = j0 + kBN <= cs.j1 && j0 + kBN - 1 <= cs.n_b - a.Tc;
        u32x4 ka[DS];
        read_k<DS, S * P::STAGE_BYTES>(ka, kaddr);
        f32x16_t sacc = f32x16_t{};
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) sacc = mfma32<ST>(ka[ds], qb[ds], sacc);
        u32x2 vt[DT][2][2];
        read_vt<DT, S * P::STAGE_BYTES, D * 2>(vt, vaddr);

        // scores -> probabilities; value jj is key j0 + (jj / 4) * 8 + hl * 4 + jj % 4
        float sv_[16];
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) sv_[jj] = sacc[jj];
        if (!plain) {
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const int j = j0 + (jj >> 2) * 8 + hl * 4 + (jj & 3);
                if (!(j < cs.j1 && j <= qpos)) sv_[jj] = -INFINITY;
            }
        }
        float mt = sv_[0];
#pragma unroll
        for (int jj = 1; jj < 16; ++jj) mt = fmaxf(mt, sv_[jj]);
        if (__any(mt - m > thresh)) {
            mt = xor_op<32, true>(mt);
            if (mt - m > thresh) {
                const float alpha = m == -INFINITY ? 0.f : fexp2((m - mt) * c);
                m = mt;
                lsum *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
            }
        }
        const float nmc = m == -INFINITY ? 0.f : -m * c;
        // each probability as a 16-bit pair hi + lo: hi = p rounded to the
        // storage type, lo = the (exact) residual p - hi rounded again, so
        // hi + lo carries p to ~2^-17 relative (bf16) and the product with V
        // runs twice; the normaliser sums the same hi and lo values
        uint32_t w[8], wl[8];
        float ls[2] = {0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p0 = fexp2(fmaf(sv_[2 * e], c, nmc));
            const float p1 = fexp2(fmaf(sv_[2 * e + 1], c, nmc));
            w[e] = pack_p<ST>(p0, p1);
            ls[e & 1] = add_pair<ST>(w[e], ls[e & 1]);
            if constexpr (KVC_DECODE_MFMA_PSPLIT) {
                wl[e] = pack_p<ST>(p0 - low_half<ST>(w[e]), p1 - high_half<ST>(w[e]));
                ls[e & 1] = add_pair<ST>(wl[e], ls[e & 1]);
            }
        }
        lsum += ls[0] + ls[1];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const u32x4 va = {vt[dt][kk][0][0], vt[dt][kk][0][1], vt[dt][kk][1][0], vt[dt][kk][1][1]};
                const u32x4 pb = {w[kk * 4 + 0], w[kk * 4 + 1], w[kk * 4 + 2], w[kk * 4 + 3]};
                o[dt] = mfma32<ST>(va, pb, o[dt]);
                if constexpr (KVC_DECODE_MFMA_PSPLIT) {
                    const u32x4 pl = {wl[kk * 4 + 0], wl[kk * 4 + 1], wl[kk * 4 + 2], wl[kk * 4 + 3]};
                    o[dt] = mfma32<ST>(va, pl, o[dt]);
                }
            }
    };

    // -- end of a segment: column col32's (max, sum, output); the lane holds
    //    head elements dt * 32 + (jj / 4) * 8 + hl * 4 + jj % 4 --
    auto finish_segment = [&]() __attribute__((always_inline)) {
        const float l_all = xor_op<32, false>(lsum);
        if (col32 < rows_act) {
            if (cs.rec < 0) {
                const float inv = 1.f / l_all;
                const int h = cs.g * a.G + a.r0 + col32 / a.Tc;
                const int i = a.i0 + col32 % a.Tc;
                float* dst = a.out + ((static_cast<int64_t>(a.row0 + cs.b) * a.Hq + h) * a.T + i) * D;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
                        *reinterpret_cast<float4*>(dst + dt * 32 + q4 * 8 + hl * 4) =
                            make_float4(o[dt][q4 * 4 + 0] * inv, o[dt][q4 * 4 + 1] * inv,
                                        o[dt][q4 * 4 + 2] * inv, o[dt][q4 * 4 + 3] * inv);
            } else {
                const int64_t rr = cs.rec * a.rec_rows + col32;
                float* dst = a.ws_o + rr * D;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
                        *reinterpret_cast<float4*>(dst + dt * 32 + q4 * 8 + hl * 4) =
                            make_float4(o[dt][q4 * 4 + 0], o[dt][q4 * 4 + 1], o[dt][q4 * 4 + 2], o[dt][q4 * 4 + 3]);
                if (hl == 0) {
                    a.ws_ml[rr * 2] = m;
                    a.ws_ml[rr * 2 + 1] = l_all;
                }
            }
        }
    };

    // -- the loop: tile t in slot t % NS, NS - 1 tiles issued ahead --
    static_for<NS - 1>([&](auto k) { issue(k); });
#if KVC_DECODE_TIMESTAMPS
    const unsigned long long pt_issued = probe_now();
#endif
    load_qtab(first);
    start_segment();
    bool done = false;
    auto step = [&](auto slot_c) __attribute__((always_inline)) {
        constexpr int S = decltype(slot_c)::value;
        // this tile's loads have landed: NS - 1 tiles stay in flight, or none
        // at the slice's end (no loads are issued past it)
        const bool more = is_live;
        issue(std::integral_constant<int, (S + NS - 1) % NS>{});
        if (more) wait_vm<(NS - 1) * 2 * NLD>();
        else wait_vm<0>();
        consume(slot_c);
        if (++cs_t == cs.nbat) {
            finish_segment();
            if (cs.x_end >= x_end) {
                done = true;
            } else {
                cs = locate_next(cs);
                if (cs.nbat == 0) {          // the slice ends in virtual keys
                    done = true;
                } else {
                    cs_t = 0;
                    if (++cs_q == P::QSEGS) {    // more segments than the table holds: reload it
                        load_qtab(cs);
                        cs_q = 0;
                    }
                    start_segment();
                }
            }
        }
    };
    while (!done) {
        static_for<NS>([&](auto k) {
            if (!done) step(k);
        });
    }
    wait_vm<0>();
#if KVC_DECODE_TIMESTAMPS
    if (lane == 0) {
        unsigned long long* w = kvc_probe_wg + static_cast<int64_t>(blockIdx.x) * 6;
        w[0] = pt_start;
        w[1] = pt_located;
        w[2] = pt_issued;
        w[3] = probe_now();
        w[4] = probe_ids();
        w[5] = static_cast<unsigned long long>(x_end - x_begin);
    }
#endif
}

// Merge the partial records of units whose keys span several work-groups
// (units held by one work-group were written by the attention kernel and are
// skipped). Work-group (u, y) covers outputs y*256 .. y*256+255 of unit u's
// slab, one (row, element) per thread.
template <class A, int D>
__global__ __launch_bounds__(256) void decode_combine(A a) {
    constexpr int kMaxSeg = 16;
    // grid (H_kv, rows of 256 outputs [+ the store row], batch rows): the row
    // b is known without the arguments, so its prefix entries and every
    // argument used below are fetched in one round trip, and held as opaque
    // copies (the compiler would otherwise read some again near their use,
    // one dependent wait each)
#if KVC_DECODE_TIMESTAMPS
    const unsigned long long pt_start = probe_now();
#endif
    const int g = blockIdx.x;
    const int b = blockIdx.z;
    int64_t p0 = a.prefix[b], p1 = a.prefix[b + 1];
    int64_t kpb = a.keys_per_block, kpbo = a.keys_per_block_odd, kpb2 = a.keys_per_block2,
            kpb2o = a.keys_per_block2_odd;
    float pinv = a.pair_inv, pinv2 = a.pair2_inv;
    int32_t n1 = a.n_first, hkv = a.Hkv, upad = a.unit_pad, hshift = a.hkv_shift, mrows = a.merge_rows;
    uint64_t hinv = a.hkv_inv;
    const void* knew = a.k_new;
    asm volatile("" : "+s"(p0), "+s"(p1), "+s"(kpb), "+s"(kpbo), "+s"(kpb2), "+s"(kpb2o), "+s"(pinv), "+s"(pinv2),
                 "+s"(n1), "+s"(hkv), "+s"(upad), "+s"(hshift), "+s"(mrows), "+s"(hinv), "+s"(knew)
                 : "s"(a.ws_o), "s"(a.ws_ml), "s"(a.rec_rows), "s"(a.out), "s"(a.Gc), "s"(a.Tc), "s"(a.scale_log2));
    const int u = b * hkv + g;
    const int64_t n_b = decode_div_exact(p1 - p0, hshift, hinv);
    // the unit's first real key on the (padded) key axis
    const int64_t ustart = p0 + static_cast<int64_t>(b) * hkv * upad + g * (n_b + upad) + upad;
    if (knew != nullptr && static_cast<int>(blockIdx.y) == mrows) {
        // fused append: store unit (b, g)'s T new keys and values at slots
        // n_b - T .. n_b - 1 (the input has the storage type: bit copies, with a
        // 16-bit NaN stored as the canonical quiet NaN of its sign, as the
        // append kernel's rounding stores it)
        const int esz = a.st_dtype == F32 ? 4 : 2;
        const int64_t src0 = ((static_cast<int64_t>(a.row0 + b) * hkv + g) * a.T) * D;
        for (int e = threadIdx.x; e < a.T * D; e += 256) {
            const int t = e / D, d = e - (e / D) * D;
            const int64_t p = n_b - a.T + t;
            int64_t dst;
            if (a.btab != nullptr) {
                int blk = a.btab[static_cast<int64_t>(b) * a.btab_stride + (p >> a.bshift)];
                blk = blk < 0 ? 0 : (blk >= a.pool_blocks ? a.pool_blocks - 1 : blk);
                dst = a.layer_off + (((static_cast<int64_t>(blk) * hkv + g) << a.bshift) + (p & ((1 << a.bshift) - 1))) * D + d;
            } else {
                dst = a.layer_off + b * a.row_stride + g * a.head_stride + p * D + d;
            }
            if (esz == 4) {
                static_cast<float*>(const_cast<void*>(a.k_cache))[dst] = static_cast<const float*>(knew)[src0 + e];
                static_cast<float*>(const_cast<void*>(a.v_cache))[dst] = static_cast<const float*>(a.v_new)[src0 + e];
            } else {
                const uint32_t inf = a.st_dtype == BF16 ? 0x7F80u : 0x7C00u;
                const uint32_t qnan = a.st_dtype == BF16 ? 0x7FC0u : 0x7E00u;
                auto canon = [&](uint32_t h) -> uint16_t {
                    return static_cast<uint16_t>((h & 0x7FFFu) > inf ? (h & 0x8000u) | qnan : h);
                };
                static_cast<uint16_t*>(const_cast<void*>(a.k_cache))[dst] =
                    canon(static_cast<const uint16_t*>(knew)[src0 + e]);
                static_cast<uint16_t*>(const_cast<void*>(a.v_cache))[dst] =
                    canon(static_cast<const uint16_t*>(a.v_new)[src0 + e]);
            }
        }
        return;
    }
    const int k_first = static_cast<int>(decode_slice_of(ustart, n1, kpb, kpbo, kpb2, kpb2o, pinv, pinv2));
    const int k_last = static_cast<int>(decode_slice_of(ustart + n_b - 1, n1, kpb, kpbo, kpb2, kpb2o, pinv, pinv2));
#if KVC_DECODE_TIMESTAMPS
    const unsigned long long pt_known = probe_now();
#endif
    if (k_first == k_last) return;
    const int idx = static_cast<int>(blockIdx.y) * 256 + static_cast<int>(threadIdx.x);
    if (idx >= a.Gc * a.Tc * D) return;
    const float c = a.scale_log2;
    const int r = idx / D, d = idx - (idx / D) * D;
    // the unit's records k_first + u .. k_last + u, one apart, each rec_rows
    // rows of D outputs and of a (max, sum) pair
    const int n = k_last - k_first + 1;
    const int64_t rec0 = static_cast<int64_t>(k_first + u) * a.rec_rows + r;
    const float* po = a.ws_o + rec0 * D + d;
    const float2* pml = reinterpret_cast<const float2*>(a.ws_ml) + rec0;
    const int64_t so = static_cast<int64_t>(a.rec_rows) * D;
    float M = -INFINITY, ov = 0.f, lv = 0.f;
    for (int t0 = 0; t0 < n; t0 += kMaxSeg) {
        float2 ml[kMaxSeg];
        float ok[kMaxSeg];
#pragma unroll
        for (int t = 0; t < kMaxSeg; ++t) {
            if (t0 + t < n) {
                ml[t] = pml[static_cast<int64_t>(t0 + t) * a.rec_rows];
                ok[t] = po[(t0 + t) * so];
            } else {
                ml[t] = make_float2(-INFINITY, 0.f);
                ok[t] = 0.f;
            }
        }
        float Mn = M;
#pragma unroll
        for (int t = 0; t < kMaxSeg; ++t) Mn = fmaxf(Mn, ml[t].x);
        const float sc = M == -INFINITY ? 0.f : fexp2((M - Mn) * c);
        ov *= sc;
        lv *= sc;
#pragma unroll
        for (int t = 0; t < kMaxSeg; ++t) {
            const float f = ml[t].x == -INFINITY ? 0.f : fexp2((ml[t].x - Mn) * c);
            ov = fmaf(ok[t], f, ov);
            lv = fmaf(ml[t].y, f, lv);
        }
        M = Mn;
    }
#if KVC_DECODE_TIMESTAMPS
    const unsigned long long pt_merged = probe_now();
#endif
    const int h = g * a.G + a.r0 + r / a.Tc;
    const int i = a.i0 + r % a.Tc;
    a.out[((static_cast<int64_t>(a.row0 + b) * a.Hq + h) * a.T + i) * D + d] = ov / lv;
#if KVC_DECODE_TIMESTAMPS
    const unsigned bid = (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
    if (threadIdx.x == 0 && bid < kProbeMergeBlocks) {
        unsigned long long* w = kvc_probe_merge + static_cast<int64_t>(bid) * 4;
        w[0] = pt_start;
        w[1] = pt_known;
        w[2] = pt_merged;
        w[3] = probe_now();
    }
#endif
}

// CUs of the current device (cached per device).
hipError_t device_cus(int& n_cu) {
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    if (cus[dev & 63] == 0) {
        int n = 0;
        const hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        cus[dev & 63] = n > 0 ? n : 1;
    }
    n_cu = cus[dev & 63];
    return hipSuccess;
}

// Launches `f` with the launch's arguments: a copy cut to the short prefix
// table when the launch has at most kSmallRows rows (less for the runtime to
// copy), else the full block.
template <class F>
hipError_t with_args(const DecodeArgs& a, F&& f) {
    if (a.rows <= kSmallRows) {
        DecodeArgsSmall sm;
        std::memcpy(&sm, &a, sizeof(sm));
        f(sm);
    } else {
        f(a);
    }
    return hipGetLastError();
}

// The merge pass, if some unit spans several work-groups.
template <int D>
hipError_t combine_if_split(DecodeArgs& a, hipStream_t s) {
    bool split = false;
    for (int b = 0; b < a.rows && !split; ++b) {
        const int64_t n_b = decode_div_hkv(a, a.prefix[b + 1] - a.prefix[b]);
        for (int g = 0; g < a.Hkv && !split; ++g) {
            const int64_t us = a.prefix[b] + static_cast<int64_t>(b) * a.Hkv * a.unit_pad + g * (n_b + a.unit_pad) + a.unit_pad;
            split = decode_slice_of(a, us) != decode_slice_of(a, us + n_b - 1);
        }
    }
    // a fused append adds one row of work-groups that store the new keys and values
    if (!split && a.k_new == nullptr) return hipSuccess;
    const unsigned merge_rows = split ? (a.Gc * a.Tc * D + 255) / 256 : 0;
    a.merge_rows = static_cast<int32_t>(merge_rows);
    const dim3 grid(a.Hkv, merge_rows + (a.k_new != nullptr ? 1 : 0), a.rows);
    return with_args(a, [&](const auto& args) {
        decode_combine<std::decay_t<decltype(args)>, D><<<grid, 256, 0, s>>>(args);
    });
}

template <int D, int ST, int R>
hipError_t run(DecodeArgs& a, hipStream_t s) {
    int n_cu = 0;
    hipError_t e = device_cus(n_cu);
    if (e != hipSuccess) return e;
    a.rec_rows = R;
    decode_split_slices(a, n_cu, KVC_DECODE_BLOCKS_PER_CU, 2 * Cfg<D, ST, R>::KPB, KVC_DECODE_LATE_PCT, KVC_DECODE_ODD_XCD_PCT);
    if (a.btab && (1 << a.bshift) < Cfg<D, ST, R>::KPB) return hipErrorInvalidValue;   // a batch within two blocks
    e = with_args(a, [&](const auto& args) {
        using A = std::decay_t<decltype(args)>;
        if (a.btab) decode_attn<A, D, ST, R, true><<<a.n_blocks, Cfg<D, ST, R>::THREADS, 0, s>>>(args);
        else decode_attn<A, D, ST, R, false><<<a.n_blocks, Cfg<D, ST, R>::THREADS, 0, s>>>(args);
    });
    if (e != hipSuccess) return e;
    return combine_if_split<D>(a, s);
}

template <int D, int ST, int RS>
hipError_t run_rows(DecodeArgs& a, hipStream_t s) {
    int n_cu = 0;
    hipError_t e = device_cus(n_cu);
    if (e != hipSuccess) return e;
    a.rec_rows = RCfg<D, ST, RS>::ROWS;
    decode_split_slices(a, n_cu, 2, 2 * RCfg<D, ST, RS>::KPS, KVC_DECODE_LATE_PCT, KVC_DECODE_ODD_XCD_PCT);
    if (a.btab && (1 << a.bshift) < RCfg<D, ST, RS>::KPS) return hipErrorInvalidValue;   // a stage within two blocks
    e = with_args(a, [&](const auto& args) {
        using A = std::decay_t<decltype(args)>;
        if (a.btab) decode_rows<A, D, ST, RS, true><<<a.n_blocks, RCfg<D, ST, RS>::THREADS, 0, s>>>(args);
        else decode_rows<A, D, ST, RS, false><<<a.n_blocks, RCfg<D, ST, RS>::THREADS, 0, s>>>(args);
    });
    if (e != hipSuccess) return e;
    return combine_if_split<D>(a, s);
}

template <int D, int ST>
hipError_t run_mfma(DecodeArgs& a, hipStream_t s) {
    int n_cu = 0;
    hipError_t e = device_cus(n_cu);
    if (e != hipSuccess) return e;
    a.rec_rows = (a.Gc * a.Tc + 3) & ~3;   // records as wide as the slab (rounded up to 4 rows)
    // every unit charged one tile more on the key axis (its part tiles)
    a.unit_pad = KVC_DECODE_MFMA_UNIT_PAD;
    a.total_keys += static_cast<int64_t>(a.rows) * a.Hkv * a.unit_pad;
    const int odd_pct = a.Gc * a.Tc > 16 ? KVC_DECODE_MFMA_ODD_XCD_PCT_WIDE : KVC_DECODE_ODD_XCD_PCT;
    decode_split_slices(a, n_cu, mfma_blocks_per_cu<D>(), 2 * kBN, KVC_DECODE_MFMA_LATE_PCT, odd_pct);
    if (a.btab && (1 << a.bshift) < kBN) return hipErrorInvalidValue;   // a tile within two blocks
    e = with_args(a, [&](const auto& args) {
        using A = std::decay_t<decltype(args)>;
        if (a.btab) decode_mfma<A, D, ST, true><<<a.n_blocks, 64, 0, s>>>(args);
        else decode_mfma<A, D, ST, false><<<a.n_blocks, 64, 0, s>>>(args);
    });
    if (e != hipSuccess) return e;
    return combine_if_split<D>(a, s);
}

template <int D, int ST>
hipError_t run_r(DecodeArgs& a, hipStream_t s) {
    const int rows = a.Gc * a.Tc;
    // a fused append is one slab covering the whole chunk
    if (a.k_new != nullptr && (a.Gc != a.G || a.Tc != a.T || a.r0 || a.i0)) return hipErrorInvalidValue;
    if constexpr (ST != F32) {
        // 16-bit caches: the matrix-core kernel for every slab (it streams the
        // cache faster than the vector kernel even at one query row)
        if constexpr (KVC_DECODE_MFMA_MIN_ROWS > 1) {
            if (rows < KVC_DECODE_MFMA_MIN_ROWS) {
                if (rows > 8) return hipErrorInvalidValue;
                return rows <= 4 ? run<D, ST, 4>(a, s) : run<D, ST, 8>(a, s);
            }
        }
        return run_mfma<D, ST>(a, s);
    } else {
        if (a.k_new != nullptr && rows > 8) return hipErrorInvalidValue;
        if (rows <= 4) return run<D, ST, 4>(a, s);
        if (rows <= 8) return run<D, ST, 8>(a, s);
        if (rows <= 16) return run_rows<D, ST, 2>(a, s);
        return run_rows<D, ST, 4>(a, s);
    }
}

}  // namespace

// Entry points of one (head dimension, storage type): each is instantiated in
// its own translation unit (kvc_decode_d<D>_<type>.hip) so that the kernels
// compile in parallel.
template <int D, int ST>
hipError_t decode_run(DecodeArgs& a, hipStream_t s) {
    return run_r<D, ST>(a, s);
}

template <int D, int ST>
int decode_batch_keys(int rows) {
    const int vec = rows <= 4 ? Cfg<D, ST, 4>::KPB : Cfg<D, ST, 8>::KPB;
    if constexpr (ST == F32) return vec;
    else return KVC_DECODE_MFMA_MIN_ROWS > 1 && vec > kBN ? vec : kBN;
}

}  // namespace kvc
