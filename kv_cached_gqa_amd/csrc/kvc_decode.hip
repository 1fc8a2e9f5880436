// Decode attention: softmax(q K^T / sqrt(D)) V for a few query rows per KV
// head, over all keys the cache holds for each batch row
// ("KV cache, incremental decode, ...", section 2.3, the bottom-right mask;
// "kv-cache-decoding", "Prefill and decode": one row of t + 1 scores per head).
//
// Decode reads every cached key and value once and does ~4 flops per byte,
// so it is bound by HBM bandwidth. The design keeps the loads wide and
// coalesced and does the arithmetic in vector registers:
//
//  * Work split ("stream-K"). Unit u = (batch row b, KV head g) owns n_b keys.
//    The units are laid end to end along one axis of sum(n_b) * H_kv keys and
//    every work-group takes an equal slice of it, so ragged row lengths cost
//    no load imbalance. A slice that crosses unit boundaries is cut into
//    segments; segment (work-group k, unit u) is stored at index k + u, which
//    is unique because each new segment starts at a slice boundary, a unit
//    boundary or both.
//  * Lane layout. One key row of D elements is LPK lanes x 16 bytes; a wave
//    covers KPW = 64 / LPK consecutive keys per load, i.e. one contiguous
//    stretch of memory. All query rows of the slab (the G query heads that
//    share the KV head, times the chunk's query positions) are held in every
//    lane group, so each key and value is read from HBM exactly once for the
//    whole group ("Heads, GQA and K/V cache": heads sharing one K/V).
//  * q.k: 16-bit dot2 instructions (exact products, fp32 accumulation) or fp32
//    FMA, then a DPP sum over the LPK lanes of the key.
//  * Online softmax per lane group in base 2 (log2(e) is folded into the
//    scale), rescaled once per batch of U keys; p stays fp32 and p*v is an fp32
//    FMA. At the end of a segment the lane groups and the four waves merge
//    their (max, sum, output) and the work-group writes one partial record.
//  * A second kernel merges a unit's partial records and normalises.
#include "kvc_device.h"

namespace kvc {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <int ST>
struct Layout {
    static constexpr int esz = ST == F32 ? 4 : 2;
    static constexpr int epl = 16 / esz;   // elements per lane per 16-byte load
};

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Load EPL elements of q (any dtype) and round them as the storage type ST.
template <int ST, int EPL>
__device__ __forceinline__ void load_q(const void* q, int q_dtype, int64_t elem, float (&o)[EPL]) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        float x;
        if (q_dtype == F32) x = static_cast<const float*>(q)[elem + e];
        else if (q_dtype == BF16) x = bf16_to_f32(static_cast<const uint16_t*>(q)[elem + e]);
        else x = f16_to_f32(static_cast<const uint16_t*>(q)[elem + e]);
        o[e] = round_as<ST>(x);
    }
}

template <int D, int ST, int R>
__global__ __launch_bounds__(kThreads) void decode_partial(DecodeArgs a) {
    using L = Layout<ST>;
    constexpr int EPL = L::epl;
    constexpr int LPK = D / EPL;           // lanes per key row
    constexpr int KPW = 64 / LPK;          // keys per wave per load
    constexpr int U = R <= 4 ? 4 : 2;      // loads in flight per lane per tensor
    constexpr int KEYS_PER_WAVE_TRIP = KPW * U;
    constexpr int KEYS_PER_TRIP = KEYS_PER_WAVE_TRIP * kWaves;
    constexpr int NQ = ST == F32 ? EPL : EPL / 2;   // q registers per row

    __shared__ float sm_o[kWaves][R][D];
    __shared__ float sm_m[kWaves][R];
    __shared__ float sm_l[kWaves][R];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int grp = lane / LPK;
    const int sub = lane % LPK;
    const int rows_act = a.Gc * a.Tc;

    const int64_t x_begin = static_cast<int64_t>(blockIdx.x) * a.keys_per_block;
    int64_t x_end = x_begin + a.keys_per_block;
    if (x_end > a.total_keys) x_end = a.total_keys;

    const uint16_t* kc16 = static_cast<const uint16_t*>(a.k_cache);
    const uint16_t* vc16 = static_cast<const uint16_t*>(a.v_cache);
    const float* kc32 = static_cast<const float*>(a.k_cache);
    const float* vc32 = static_cast<const float*>(a.v_cache);

    for (int64_t x = x_begin; x < x_end;) {
        // -- locate the unit holding key x (wave-uniform) --
        int lo = 0, hi = a.rows;   // prefix[lo] <= x < prefix[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.prefix[mid] <= x) lo = mid; else hi = mid;
        }
        const int b = lo;
        const int64_t n_b = (a.prefix[b + 1] - a.prefix[b]) / a.Hkv;
        const int64_t off = x - a.prefix[b];
        const int g = static_cast<int>(off / n_b);
        const int64_t unit_start = a.prefix[b] + static_cast<int64_t>(g) * n_b;
        int64_t seg_end = unit_start + n_b;
        if (seg_end > x_end) seg_end = x_end;
        const int j0 = static_cast<int>(x - unit_start);
        const int j1 = static_cast<int>(seg_end - unit_start);
        const int seg = blockIdx.x + b * a.Hkv + g;

        const int64_t head_base = a.layer_off + b * a.row_stride + g * a.head_stride;
        const int qpos_base = static_cast<int>(n_b) - a.Tc;   // absolute position of slab query 0

        // -- the slab's queries, rounded as the storage type --
        float qf[R][EPL];
        uint32_t qp[R][NQ];
        int qpos[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int hr = r / a.Tc, ir = r - (r / a.Tc) * a.Tc;
            qpos[r] = r < rows_act ? qpos_base + ir : -1;
            if (r < rows_act) {
                const int h = g * a.G + a.r0 + hr;
                const int i = a.i0 + ir;
                const int64_t qe = ((static_cast<int64_t>(a.row0 + b) * a.Hq + h) * a.T + i) * D + sub * EPL;
                load_q<ST, EPL>(a.q, a.q_dtype, qe, qf[r]);
            } else {
#pragma unroll
                for (int e = 0; e < EPL; ++e) qf[r][e] = 0.f;
            }
            if constexpr (ST != F32) {
#pragma unroll
                for (int e = 0; e < NQ; ++e) {
                    const uint32_t lo16 = ST == BF16 ? f32_to_bf16_rne(qf[r][2 * e]) : f32_to_f16_rne(qf[r][2 * e]);
                    const uint32_t hi16 = ST == BF16 ? f32_to_bf16_rne(qf[r][2 * e + 1]) : f32_to_f16_rne(qf[r][2 * e + 1]);
                    qp[r][e] = lo16 | (hi16 << 16);
                }
            }
        }

        float m[R], l[R], o[R][EPL];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            m[r] = -INFINITY;
            l[r] = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[r][e] = 0.f;
        }

        // -- stream the segment's keys --
        const int wave_key0 = j0 + wave * KEYS_PER_WAVE_TRIP + grp;
        for (int t0 = 0; j0 + t0 < j1; t0 += KEYS_PER_TRIP) {
            uint4 kr[U], vr[U];
            int jk[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                jk[u] = wave_key0 + t0 + u * KPW;
                const int jc = jk[u] < j1 ? jk[u] : j1 - 1;
                const int64_t e = head_base + static_cast<int64_t>(jc) * D + sub * EPL;
                if constexpr (ST == F32) {
                    kr[u] = *reinterpret_cast<const uint4*>(kc32 + e);
                    vr[u] = *reinterpret_cast<const uint4*>(vc32 + e);
                } else {
                    kr[u] = *reinterpret_cast<const uint4*>(kc16 + e);
                    vr[u] = *reinterpret_cast<const uint4*>(vc16 + e);
                }
            }
            float s[U][R];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t kw[4] = {kr[u].x, kr[u].y, kr[u].z, kr[u].w};
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float acc = 0.f;
                    if constexpr (ST == F32) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc = fmaf(qf[r][e], __uint_as_float(kw[e]), acc);
                    } else if constexpr (ST == BF16) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qp[r][e]),
                                                                  __builtin_bit_cast(bf16x2_t, kw[e]), acc, false);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, qp[r][e]),
                                                         __builtin_bit_cast(f16x2_t, kw[e]), acc, false);
                    }
                    acc = group_sum<LPK>(acc) * a.scale_log2;
                    s[u][r] = (jk[u] < j1 && jk[u] <= qpos[r]) ? acc : -INFINITY;
                }
            }
            float vf[U][EPL];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t vw[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (ST == F32) {
                        vf[u][e] = __uint_as_float(vw[e]);
                    } else if constexpr (ST == BF16) {
                        vf[u][2 * e] = bf16_to_f32(vw[e] & 0xFFFFu);
                        vf[u][2 * e + 1] = bf16_to_f32(vw[e] >> 16);
                    } else {
                        vf[u][2 * e] = f16_to_f32(vw[e] & 0xFFFFu);
                        vf[u][2 * e + 1] = f16_to_f32(vw[e] >> 16);
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float mt = s[0][r];
#pragma unroll
                for (int u = 1; u < U; ++u) mt = fmaxf(mt, s[u][r]);
                const float mn = fmaxf(m[r], mt);
                const float mu = mn == -INFINITY ? 0.f : mn;
                const float alpha = fexp2(m[r] - mu);
                m[r] = mn;
                l[r] *= alpha;
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[r][e] *= alpha;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const float p = fexp2(s[u][r] - mu);
                    l[r] += p;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) o[r][e] = fmaf(p, vf[u][e], o[r][e]);
                }
            }
        }

        // -- merge the lane groups of this wave --
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float mw = m[r];
#pragma unroll
            for (int d = LPK; d < 64; d <<= 1) mw = fmaxf(mw, __shfl_xor(mw, d));
            const float mu = mw == -INFINITY ? 0.f : mw;
            const float w = fexp2(m[r] - mu);
            float lw = l[r] * w;
#pragma unroll
            for (int d = LPK; d < 64; d <<= 1) lw += __shfl_xor(lw, d);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                float ow = o[r][e] * w;
#pragma unroll
                for (int d = LPK; d < 64; d <<= 1) ow += __shfl_xor(ow, d);
                o[r][e] = ow;
            }
            m[r] = mw;
            l[r] = lw;
        }
        if (grp == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int e = 0; e < EPL; ++e) sm_o[wave][r][sub * EPL + e] = o[r][e];
        }
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                sm_m[wave][r] = m[r];
                sm_l[wave][r] = l[r];
            }
        }
        __syncthreads();
        // -- merge the waves and write the segment's partial record --
        for (int idx = tid; idx < rows_act * D; idx += kThreads) {
            const int r = idx / D, d = idx - (idx / D) * D;
            float M = sm_m[0][r];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][r]);
            const float mu = M == -INFINITY ? 0.f : M;
            float ov = 0.f, lv = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float f = fexp2(sm_m[w][r] - mu);
                ov = fmaf(sm_o[w][r][d], f, ov);
                lv = fmaf(sm_l[w][r], f, lv);
            }
            const int64_t rec = static_cast<int64_t>(seg) * kMaxDecodeRows + r;
            a.ws_o[rec * D + d] = ov;
            if (d == 0) {
                a.ws_ml[rec * 2] = M;
                a.ws_ml[rec * 2 + 1] = lv;
            }
        }
        __syncthreads();
        x = seg_end;
    }
}

// One wave per (unit, slab row): merge the unit's partial records.
template <int D>
__global__ __launch_bounds__(256) void decode_combine(DecodeArgs a) {
    const int lane = threadIdx.x & 63;
    const int rows_act = a.Gc * a.Tc;
    const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int64_t n_items = static_cast<int64_t>(a.rows) * a.Hkv * rows_act;
    if (item >= n_items) return;
    const int r = static_cast<int>(item % rows_act);
    const int64_t u = item / rows_act;
    const int b = static_cast<int>(u / a.Hkv);
    const int g = static_cast<int>(u - static_cast<int64_t>(b) * a.Hkv);
    const int64_t n_b = (a.prefix[b + 1] - a.prefix[b]) / a.Hkv;
    const int64_t ustart = a.prefix[b] + g * n_b;
    const int k_first = static_cast<int>(ustart / a.keys_per_block);
    const int k_last = static_cast<int>((ustart + n_b - 1) / a.keys_per_block);

    float M = -INFINITY;
    for (int k = k_first; k <= k_last; ++k) {
        const int64_t rec = static_cast<int64_t>(k + u) * kMaxDecodeRows + r;
        M = fmaxf(M, a.ws_ml[rec * 2]);
    }
    const float mu = M == -INFINITY ? 0.f : M;
    constexpr int PER = (D + 63) / 64;
    float acc[PER] = {};
    float lsum = 0.f;
    for (int k = k_first; k <= k_last; ++k) {
        const int64_t rec = static_cast<int64_t>(k + u) * kMaxDecodeRows + r;
        const float f = fexp2(a.ws_ml[rec * 2] - mu);
        lsum = fmaf(a.ws_ml[rec * 2 + 1], f, lsum);
#pragma unroll
        for (int c = 0; c < PER; ++c) {
            const int d = lane + 64 * c;
            if (d < D) acc[c] = fmaf(a.ws_o[rec * D + d], f, acc[c]);
        }
    }
    const float inv = 1.f / lsum;
    const int h = g * a.G + a.r0 + r / a.Tc;
    const int i = a.i0 + r % a.Tc;
    float* dst = a.out + ((static_cast<int64_t>(a.row0 + b) * a.Hq + h) * a.T + i) * D;
#pragma unroll
    for (int c = 0; c < PER; ++c) {
        const int d = lane + 64 * c;
        if (d < D) dst[d] = acc[c] * inv;
    }
}

template <int D, int ST>
hipError_t run(const DecodeArgs& a, hipStream_t s) {
    const int rows_act = a.Gc * a.Tc;
    if (rows_act <= 4) decode_partial<D, ST, 4><<<a.n_blocks, kThreads, 0, s>>>(a);
    else decode_partial<D, ST, 8><<<a.n_blocks, kThreads, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t items = static_cast<int64_t>(a.rows) * a.Hkv * rows_act;
    decode_combine<D><<<static_cast<unsigned>((items + 3) / 4), 256, 0, s>>>(a);
    return hipGetLastError();
}

template <int D>
hipError_t run_d(const DecodeArgs& a, hipStream_t s) {
    switch (a.st_dtype) {
        case F32: return run<D, F32>(a, s);
        case F16: return run<D, F16>(a, s);
        case BF16: return run<D, BF16>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool decode_supported(int D, int st_dtype) {
    return (D == 32 || D == 64 || D == 128) && (st_dtype == F32 || st_dtype == F16 || st_dtype == BF16);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    if (a.Gc * a.Tc < 1 || a.Gc * a.Tc > kMaxDecodeRows) return hipErrorInvalidValue;
    if (a.n_blocks < 1 || a.n_blocks > kMaxDecodeBlocks) return hipErrorInvalidValue;
    switch (a.D) {
        case 32: return run_d<32>(a, s);
        case 64: return run_d<64>(a, s);
        case 128: return run_d<128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvc
