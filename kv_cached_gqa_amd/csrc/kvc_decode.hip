// Decode attention: softmax(q K^T / sqrt(D)) V for a few query rows per KV
// head, over all keys the cache holds for each batch row
// ("KV cache, incremental decode, ...", section 2.3, the bottom-right mask;
// "kv-cache-decoding", "Prefill and decode": one row of t + 1 scores per head).
//
// Decode reads every cached key and value once and does ~4 flops per byte,
// so it is bound by HBM bandwidth. The design keeps the loads wide, coalesced
// and always in flight, and keeps the vector ALU work per key small:
//
//  * Work split ("stream-K"). Unit u = (batch row b, KV head g) owns n_b keys.
//    The units are laid end to end along one axis of sum(n_b) * H_kv keys and
//    every work-group takes an equal slice of it, so ragged row lengths cost
//    no load imbalance. The grid is exactly the number of work-groups the GPU
//    keeps resident, so there is one round and no tail. A slice that crosses
//    unit boundaries is cut into segments; segment (work-group k, unit u) is
//    stored at index k + u, which is unique because each new segment starts at
//    a slice boundary, a unit boundary or both.
//  * Lane layout. One key row of D elements is LPK lanes x 16 bytes; a wave
//    covers KPW = 64 / LPK consecutive keys per load, i.e. one contiguous
//    stretch of memory. All query rows of the slab (the G query heads that
//    share the KV head, times the chunk's query positions) are held in every
//    lane group, so each key and value is read from HBM exactly once for the
//    whole group ("Heads, GQA and K/V cache": heads sharing one K/V).
//    Loads are double-buffered: the next batch is in flight while the current
//    one is being used.
//  * q.k: 16-bit dot2 instructions (exact products, fp32 accumulation) or fp32
//    FMA, then a DPP sum over the LPK lanes of the key. Scores stay in raw
//    q.k units; the softmax scale and log2(e) are folded into one FMA before
//    exp2. The running max only triggers a rescale when it grows somewhere in
//    the wave. p stays fp32 and p*v is an fp32 FMA.
//  * Merge. At the end of a segment the lane groups and the four waves merge
//    their (max, sum, output). A unit held by one segment is normalised and
//    written at once; otherwise the segment's partial record goes to the
//    workspace and a second, small kernel merges each split unit's records.
//    (Merging inside the first kernel would need agent-scope fences per
//    segment, which write back and invalidate an XCD's L2 and cost far more
//    than the second launch.)
#include "kvc_device.h"

namespace kvc {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

#ifndef KVC_DECODE_WAVES4
#define KVC_DECODE_WAVES4 4   // waves per work-group for 4 query rows or fewer
#endif
#ifndef KVC_DECODE_WAVES8
#define KVC_DECODE_WAVES8 4   // waves per work-group for 5 to 8 query rows
#endif

template <int ST>
struct Layout {
    static constexpr int esz = ST == F32 ? 4 : 2;
    static constexpr int epl = 16 / esz;   // elements per lane per 16-byte load
};

template <int ST>
__device__ __forceinline__ float dot16(const uint32_t (&q)[4], const uint4& k, float acc) {
    const uint32_t kw[4] = {k.x, k.y, k.z, k.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if constexpr (ST == BF16)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[e]),
                                                  __builtin_bit_cast(bf16x2_t, kw[e]), acc, false);
        else
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q[e]),
                                         __builtin_bit_cast(f16x2_t, kw[e]), acc, false);
    }
    return acc;
}

template <int ST, int EPL>
__device__ __forceinline__ void unpack_v(const uint4& v, float (&o)[EPL]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if constexpr (ST == F32) {
            o[e] = __uint_as_float(w[e]);
        } else if constexpr (ST == BF16) {
            o[2 * e] = __uint_as_float(w[e] << 16);
            o[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
        } else {
            o[2 * e] = f16_to_f32(w[e] & 0xFFFFu);
            o[2 * e + 1] = f16_to_f32(w[e] >> 16);
        }
    }
}

#ifndef KVC_DECODE_U
#define KVC_DECODE_U 1        // keys per lane group in one batch
#endif
#ifndef KVC_DECODE_NBUF
#define KVC_DECODE_NBUF 3     // batches held in registers: NBUF - 1 in flight while one is used
#endif

#ifndef KVC_DECODE_CH
#define KVC_DECODE_CH 1       // 16-byte chunks per lane per key row (4 query rows or fewer)
#endif
#ifndef KVC_DECODE_RESCALE_LOG2
#define KVC_DECODE_RESCALE_LOG2 8.0f
#endif
#ifndef KVC_DECODE_BLOCKS_PER_CU
#define KVC_DECODE_BLOCKS_PER_CU 0   // 0: as many as stay resident
#endif

// Rescale threshold (log2 units): the running reference max moves only when a
// score exceeds it by more than this, so p = exp2(s - m) stays below 2^8.
constexpr float kRescaleLog2 = KVC_DECODE_RESCALE_LOG2;

template <int D, int ST, int R>
struct Cfg {
    static constexpr int ESZ = Layout<ST>::esz;
    static constexpr int CH = R <= 4 ? KVC_DECODE_CH : 1;   // 16-byte chunks per lane per key row
    static constexpr int EPC = 16 / ESZ;           // elements per chunk
    static constexpr int EPL = CH * EPC;           // elements per lane
    static constexpr int LPK = D / EPL;            // lanes per key row
    static constexpr int KPW = 64 / LPK;           // keys per wave per load
    static constexpr int U = KVC_DECODE_U;
    static constexpr int WAVES = R <= 4 ? KVC_DECODE_WAVES4 : KVC_DECODE_WAVES8;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int NBUF = KVC_DECODE_NBUF;
    static constexpr int KEYS_PER_WAVE = KPW * U;  // keys per wave per batch
    static constexpr int KEYS_PER_BATCH = KEYS_PER_WAVE * WAVES;    // keys per work-group round
    static constexpr int NQ = ST == F32 ? EPL : EPL / 2;   // q registers per row
    // element index of chunk c, element e of lane `sub`
    __device__ static constexpr int elem(int sub, int c, int e) { return c * (D / CH) + sub * EPC + e; }
};

template <int D, int ST, int R>
struct Batch {
    uint4 k[Cfg<D, ST, R>::U][Cfg<D, ST, R>::CH];
    uint4 v[Cfg<D, ST, R>::U][Cfg<D, ST, R>::CH];
};

template <int LPK, int M>
__device__ __forceinline__ void lane_group_sum(float (&x)[M]) {
    if constexpr (LPK <= 16) {
        group_sum_n<LPK, M>(x);
    } else {
#pragma unroll
        for (int i = 0; i < M; ++i) x[i] = group_sum<LPK>(x[i]);
    }
}

#ifndef KVC_DECODE_WAVES_PER_EU
#define KVC_DECODE_WAVES_PER_EU 1
#endif

template <int D, int ST, int R>
__global__ __launch_bounds__((Cfg<D, ST, R>::THREADS)) __attribute__((amdgpu_waves_per_eu(KVC_DECODE_WAVES_PER_EU)))
void decode_attn(DecodeArgs a) {
    using C = Cfg<D, ST, R>;
    constexpr int kWaves = C::WAVES, kThreads = C::THREADS;
    constexpr int EPL = C::EPL, EPC = C::EPC, CH = C::CH, LPK = C::LPK, KPW = C::KPW, U = C::U, NQ = C::NQ;
    constexpr int ESZ = C::ESZ;

    __shared__ float sm_o[kWaves][R][D];
    __shared__ float sm_m[kWaves][R];
    __shared__ float sm_l[kWaves][R];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int grp = lane / LPK;
    const int sub = lane % LPK;
    const int rows_act = a.Gc * a.Tc;
    const float c = a.scale_log2;
    const float thresh = kRescaleLog2 / c;     // the threshold in raw q.k units (0: any growth)

    const int64_t x_begin = static_cast<int64_t>(blockIdx.x) * a.keys_per_block;
    int64_t x_end = x_begin + a.keys_per_block;
    if (x_end > a.total_keys) x_end = a.total_keys;

    const char* kc = static_cast<const char*>(a.k_cache);
    const char* vc = static_cast<const char*>(a.v_cache);

    for (int64_t x = x_begin; x < x_end;) {
        // -- locate the unit holding key x (wave-uniform) --
        int lo = 0, hi = a.rows;   // prefix[lo] <= x < prefix[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.prefix[mid] <= x) lo = mid; else hi = mid;
        }
        const int b = lo;
        const int64_t n_b = (a.prefix[b + 1] - a.prefix[b]) / a.Hkv;
        const int g = static_cast<int>((x - a.prefix[b]) / n_b);
        const int u_idx = b * a.Hkv + g;
        const int64_t unit_start = a.prefix[b] + static_cast<int64_t>(g) * n_b;
        int64_t seg_end = unit_start + n_b;
        if (seg_end > x_end) seg_end = x_end;
        const int j0 = static_cast<int>(x - unit_start);
        const int j1 = static_cast<int>(seg_end - unit_start);
        const bool whole_unit = j0 == 0 && j1 == n_b;

        const int64_t head_base = a.layer_off + b * a.row_stride + g * a.head_stride;
        const int qpos0 = static_cast<int>(n_b) - a.Tc;   // absolute position of slab query 0

        float qf[ST == F32 ? R : 1][ST == F32 ? EPL : 1];   // fp32 caches: q as float
        uint32_t qp[R][NQ];                                 // 16-bit caches: q as packed pairs
        int qpos[R];
        float m[R], l[R], o[R][EPL];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            m[r] = -INFINITY;
            l[r] = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[r][e] = 0.f;
        }

        // -- stream the segment's keys through a ring of register batches --
        // Batch t of wave w = keys [j0 + t * KEYS_PER_BATCH + w * KEYS_PER_WAVE, + KEYS_PER_WAVE).
        // The assignment is static, so the summation order (and the result) is the same
        // on every run.
        const int key_w0 = j0 + wave * C::KEYS_PER_WAVE + grp;   // this lane's first key
        const int n_batches = (j1 - j0 + C::KEYS_PER_BATCH - 1) / C::KEYS_PER_BATCH;

        auto issue = [&](Batch<D, ST, R>& bt, int t) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                int j = key_w0 + t * C::KEYS_PER_BATCH + u * KPW;
                j = j < j1 ? j : j1 - 1;
                const int64_t row = (head_base + static_cast<int64_t>(j) * D) * ESZ;
#pragma unroll
                for (int ch = 0; ch < CH; ++ch) {
                    const int64_t off = row + C::elem(sub, ch, 0) * ESZ;
                    bt.k[u][ch] = *reinterpret_cast<const uint4*>(kc + off);
                    bt.v[u][ch] = *reinterpret_cast<const uint4*>(vc + off);
                }
            }
        };

        auto consume = [&](const Batch<D, ST, R>& bt, int t) {
            const int jb = key_w0 + t * C::KEYS_PER_BATCH;           // key of u = 0 for this lane
            const int jw_last = j0 + wave * C::KEYS_PER_WAVE + t * C::KEYS_PER_BATCH + C::KEYS_PER_WAVE - 1;
            const bool plain = jw_last < j1 && jw_last <= qpos0;     // no key of this wave is masked
            float s[U * R];
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float acc = 0.f;
#pragma unroll
                    for (int ch = 0; ch < CH; ++ch) {
                        if constexpr (ST == F32) {
                            const uint32_t kw[4] = {bt.k[u][ch].x, bt.k[u][ch].y, bt.k[u][ch].z, bt.k[u][ch].w};
#pragma unroll
                            for (int e = 0; e < 4; ++e) acc = fmaf(qf[r][ch * 4 + e], __uint_as_float(kw[e]), acc);
                        } else {
                            acc = dot16<ST>(reinterpret_cast<const uint32_t(&)[4]>(qp[r][ch * 4]), bt.k[u][ch], acc);
                        }
                    }
                    s[u * R + r] = acc;
                }
            }
            lane_group_sum<LPK, U * R>(s);
            if (!plain) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int j = jb + u * KPW;
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        if (!(j < j1 && j <= qpos[r])) s[u * R + r] = -INFINITY;
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
                need |= (mt[r] - m[r] > thresh) || (mt[r] > m[r] && thresh == 0.f);
            }
            if (__any(need)) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if ((mt[r] - m[r] > thresh) || (mt[r] > m[r] && thresh == 0.f)) {
                        const float alpha = m[r] == -INFINITY ? 0.f : fexp2((m[r] - mt[r]) * c);
                        m[r] = mt[r];
                        l[r] *= alpha;
#pragma unroll
                        for (int e = 0; e < EPL; ++e) o[r][e] *= alpha;
                    }
                }
            }
            float nmc[R];
#pragma unroll
            for (int r = 0; r < R; ++r) nmc[r] = m[r] == -INFINITY ? 0.f : -m[r] * c;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float vf[EPL];
#pragma unroll
                for (int ch = 0; ch < CH; ++ch)
                    unpack_v<ST, EPC>(bt.v[u][ch], reinterpret_cast<float(&)[EPC]>(vf[ch * EPC]));
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float p = fexp2(fmaf(s[u * R + r], c, nmc[r]));
                    l[r] += p;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) o[r][e] = fmaf(p, vf[e], o[r][e]);
                }
            }
        };

        // -- the slab's queries, as raw 16-byte words. Every load below is issued
        //    unconditionally (rows past the slab reread row 0 and are zeroed, a
        //    16-bit q rereads its first word): a load under a branch would make
        //    the compiler wait for all outstanding loads where the paths meet,
        //    which serialises the key/value pipeline.
        // A lane needs EPC * qsz bytes per chunk: 32 (two words of 16), 16, or 8
        // (fp32 cache, 16-bit q), read from the enclosing aligned 16 bytes, which
        // lie inside the row because rows are multiples of 16 bytes.
        const int qsz = a.q_dtype == F32 ? 4 : 2;
        const int qnb = EPC * qsz;
        uint4 qraw[R][CH][2];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int rr = r < rows_act ? r : 0;
            const int hr = rr / a.Tc, ir = rr - (rr / a.Tc) * a.Tc;
            const int h = g * a.G + a.r0 + hr;
            const int i = a.i0 + ir;
            const int64_t qrow = ((static_cast<int64_t>(a.row0 + b) * a.Hq + h) * a.T + i) * D;
#pragma unroll
            for (int ch = 0; ch < CH; ++ch) {
                const char* qb = static_cast<const char*>(a.q) + (qrow + C::elem(sub, ch, 0)) * qsz;
                const char* p0 = qnb == 8 ? qb - (reinterpret_cast<uintptr_t>(qb) & 15) : qb;
                qraw[r][ch][0] = *reinterpret_cast<const uint4*>(p0);
                qraw[r][ch][1] = *reinterpret_cast<const uint4*>(qnb == 32 ? qb + 16 : p0);
            }
        }
        // word offset of the lane's first element inside the 16 bytes read (8-byte case)
        const int qwsh = qnb == 8 ? static_cast<int>((C::elem(sub, 0, 0) * qsz / 8) & 1) * 2 : 0;

        // ring of NBUF batches: batch t lives in slot t % NBUF, NBUF - 1 batches ahead.
        // Batches past the segment's end are issued too (clamped to its last key).
        Batch<D, ST, R> ring[C::NBUF];
#pragma unroll
        for (int k = 0; k < C::NBUF - 1; ++k) issue(ring[k], k);

        // -- convert the queries (waits only for the q words), rounded as the storage type --
#pragma unroll
        for (int r = 0; r < R; ++r) {
            qpos[r] = r < rows_act ? qpos0 + r % a.Tc : -1;
#pragma unroll
            for (int ch = 0; ch < CH; ++ch) {
                float tmp[EPC];
                const uint32_t w0[8] = {qraw[r][ch][0].x, qraw[r][ch][0].y, qraw[r][ch][0].z, qraw[r][ch][0].w,
                                        qraw[r][ch][1].x, qraw[r][ch][1].y, qraw[r][ch][1].z, qraw[r][ch][1].w};
                uint32_t w[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) w[e] = qwsh ? w0[(e + 2) & 7] : w0[e];
#pragma unroll
                for (int e = 0; e < EPC; ++e) {
                    float x;
                    if (a.q_dtype == F32) x = __uint_as_float(w[e]);
                    else if (a.q_dtype == BF16) x = bf16_to_f32((w[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
                    else x = f16_to_f32((w[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
                    tmp[e] = r < rows_act ? round_as<ST>(x) : 0.f;
                }
                if constexpr (ST == F32) {
#pragma unroll
                    for (int e = 0; e < EPC; ++e) qf[r][ch * EPC + e] = tmp[e];
                } else {
#pragma unroll
                    for (int e = 0; e < EPC / 2; ++e) {
                        const uint32_t lo16 = ST == BF16 ? f32_to_bf16_rne(tmp[2 * e]) : f32_to_f16_rne(tmp[2 * e]);
                        const uint32_t hi16 = ST == BF16 ? f32_to_bf16_rne(tmp[2 * e + 1]) : f32_to_f16_rne(tmp[2 * e + 1]);
                        qp[r][ch * (EPC / 2) + e] = lo16 | (hi16 << 16);
                    }
                }
            }
        }

        for (int t0 = 0; t0 < n_batches; t0 += C::NBUF) {
#pragma unroll
            for (int k = 0; k < C::NBUF; ++k) {
                const int t = t0 + k;
                if (t >= n_batches) break;
                issue(ring[(k + C::NBUF - 1) % C::NBUF], t + C::NBUF - 1);
                consume(ring[k], t);
            }
        }

        // -- merge the lane groups of this wave --
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float mw = m[r];
#pragma unroll
            for (int d = LPK; d < 64; d <<= 1) mw = fmaxf(mw, __shfl_xor(mw, d));
            const float w = mw == -INFINITY ? 0.f : fexp2((m[r] - mw) * c);
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
                for (int ch = 0; ch < CH; ++ch)
#pragma unroll
                    for (int e = 0; e < EPC; ++e) sm_o[wave][r][C::elem(sub, ch, e)] = o[r][ch * EPC + e];
        }
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                sm_m[wave][r] = m[r];
                sm_l[wave][r] = l[r];
            }
        }
        __syncthreads();

        // -- merge the waves: the output itself, or this segment's partial record --
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
            if (whole_unit) {
                const int h = g * a.G + a.r0 + r / a.Tc;
                const int i = a.i0 + r % a.Tc;
                a.out[((static_cast<int64_t>(a.row0 + b) * a.Hq + h) * a.T + i) * D + d] = ov / lv;
            } else {
                const int64_t rec = static_cast<int64_t>(blockIdx.x + u_idx) * kMaxDecodeRows + r;
                a.ws_o[rec * D + d] = ov;
                if (d == 0) {
                    a.ws_ml[rec * 2] = M;
                    a.ws_ml[rec * 2 + 1] = lv;
                }
            }
        }
        __syncthreads();
        x = seg_end;
    }
}

// One work-group per unit: merge the partial records of a unit whose keys
// span several work-groups (units held by one work-group were written by
// decode_attn and are skipped).
template <int D>
__global__ __launch_bounds__(256) void decode_combine(DecodeArgs a) {
    constexpr int kMaxSeg = 16;
    const int u = blockIdx.x;
    const int b = u / a.Hkv;
    const int g = u - b * a.Hkv;
    const int64_t n_b = (a.prefix[b + 1] - a.prefix[b]) / a.Hkv;
    const int64_t ustart = a.prefix[b] + g * n_b;
    const int k_first = static_cast<int>(ustart / a.keys_per_block);
    const int k_last = static_cast<int>((ustart + n_b - 1) / a.keys_per_block);
    if (k_first == k_last) return;
    const int rows_act = a.Gc * a.Tc;
    const float c = a.scale_log2;
    for (int idx = threadIdx.x; idx < rows_act * D; idx += 256) {
        const int r = idx / D, d = idx - (idx / D) * D;
        float M = -INFINITY, ov = 0.f, lv = 0.f;
        for (int k0 = k_first; k0 <= k_last; k0 += kMaxSeg) {
            float mk[kMaxSeg], lk[kMaxSeg], okv[kMaxSeg];
#pragma unroll
            for (int t = 0; t < kMaxSeg; ++t) {
                const int k = k0 + t;
                const int64_t rec = static_cast<int64_t>((k <= k_last ? k : k_last) + u) * kMaxDecodeRows + r;
                mk[t] = k <= k_last ? a.ws_ml[rec * 2] : -INFINITY;
                lk[t] = a.ws_ml[rec * 2 + 1];
                okv[t] = a.ws_o[rec * D + d];
            }
            float Mn = M;
#pragma unroll
            for (int t = 0; t < kMaxSeg; ++t) Mn = fmaxf(Mn, mk[t]);
            const float sc = M == -INFINITY ? 0.f : fexp2((M - Mn) * c);
            ov *= sc;
            lv *= sc;
#pragma unroll
            for (int t = 0; t < kMaxSeg; ++t) {
                const float f = mk[t] == -INFINITY ? 0.f : fexp2((mk[t] - Mn) * c);
                ov = fmaf(okv[t], f, ov);
                lv = fmaf(lk[t], f, lv);
            }
            M = Mn;
        }
        const int h = g * a.G + a.r0 + r / a.Tc;
        const int i = a.i0 + r % a.Tc;
        a.out[((static_cast<int64_t>(a.row0 + b) * a.Hq + h) * a.T + i) * D + d] = ov / lv;
    }
}

template <int D, int ST, int R>
hipError_t run(DecodeArgs& a, hipStream_t s) {
    auto kernel = decode_attn<D, ST, R>;
    // Resident work-groups per CU for this instantiation, per device (cached).
    static int resident[64] = {};
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    const int slot = dev & 63;
    if (resident[slot] == 0) {
        int per_cu = 0, n_cu = 0;
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, Cfg<D, ST, R>::THREADS, 0);
        if (e != hipSuccess) return e;
        e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        cus[slot] = n_cu > 0 ? n_cu : 1;
        resident[slot] = per_cu > 0 ? per_cu : 1;
    }
    int64_t nb = static_cast<int64_t>(cus[slot]) *
                 (KVC_DECODE_BLOCKS_PER_CU > 0 ? KVC_DECODE_BLOCKS_PER_CU : resident[slot]);
    if (nb > kMaxDecodeBlocks) nb = kMaxDecodeBlocks;
    // at least a couple of load batches per work-group
    constexpr int64_t kMinKeys = 2 * Cfg<D, ST, R>::KEYS_PER_BATCH;
    const int64_t by_size = (a.total_keys + kMinKeys - 1) / kMinKeys;
    if (nb > by_size) nb = by_size;
    if (nb < 1) nb = 1;
    a.keys_per_block = (a.total_keys + nb - 1) / nb;
    a.n_blocks = static_cast<int32_t>((a.total_keys + a.keys_per_block - 1) / a.keys_per_block);
    kernel<<<a.n_blocks, Cfg<D, ST, R>::THREADS, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the merge pass is needed only if some unit spans several work-groups
    bool split = false;
    for (int b = 0; b < a.rows && !split; ++b) {
        const int64_t n_b = (a.prefix[b + 1] - a.prefix[b]) / a.Hkv;
        for (int g = 0; g < a.Hkv && !split; ++g) {
            const int64_t us = a.prefix[b] + g * n_b;
            split = us / a.keys_per_block != (us + n_b - 1) / a.keys_per_block;
        }
    }
    if (!split) return hipSuccess;
    decode_combine<D><<<a.rows * a.Hkv, 256, 0, s>>>(a);
    return hipGetLastError();
}

template <int D, int ST>
hipError_t run_r(DecodeArgs& a, hipStream_t s) {
    if (a.Gc * a.Tc <= 4) return run<D, ST, 4>(a, s);
    return run<D, ST, 8>(a, s);
}

template <int D>
hipError_t run_d(DecodeArgs& a, hipStream_t s) {
    switch (a.st_dtype) {
        case F32: return run_r<D, F32>(a, s);
        case F16: return run_r<D, F16>(a, s);
        case BF16: return run_r<D, BF16>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool decode_supported(int D, int st_dtype) {
    return (D == 32 || D == 64 || D == 128) && (st_dtype == F32 || st_dtype == F16 || st_dtype == BF16);
}

hipError_t launch_decode(DecodeArgs& a, hipStream_t s) {
    if (a.Gc * a.Tc < 1 || a.Gc * a.Tc > kMaxDecodeRows) return hipErrorInvalidValue;
    if (a.total_keys < 1) return hipErrorInvalidValue;
    switch (a.D) {
        case 32: return run_d<32>(a, s);
        case 64: return run_d<64>(a, s);
        case 128: return run_d<128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvc
