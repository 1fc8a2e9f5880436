// Matrix-core building blocks shared by the prefill-chunk kernel and the
// matrix-core decode kernel: MFMA 32x32x16 on 16-bit data, probability
// packing, and the LDS layout and explicit LDS reads of 32-key K/V tiles.
#pragma once

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

constexpr int kBN = 32;                // keys per K/V tile

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

// The float values of the low and high element of a packed 16-bit pair.
template <int ST>
__device__ __forceinline__ float low_half(uint32_t w) {
    if constexpr (ST == BF16) return __uint_as_float(w << 16);
    else return f16_to_f32(w & 0xFFFFu);
}
template <int ST>
__device__ __forceinline__ float high_half(uint32_t w) {
    if constexpr (ST == BF16) return __uint_as_float(w & 0xFFFF0000u);
    else return f16_to_f32(w >> 16);
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
struct TileLayout {
    static constexpr int CPR = D / 8;           // 16-byte chunks per key row
    static constexpr int DS = D / 16;           // MFMA k-steps over the head dimension
    static constexpr int DT = D / 32;           // 32-wide tiles of the head dimension
    static constexpr int TILE = kBN * D;        // elements per K (or V) tile
    static constexpr int TILE_BYTES = TILE * 2;
    static constexpr int NLD = TILE * 2 / 1024; // 1 KB LDS-DMA instructions per tile and tensor

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


}  // namespace
}  // namespace kvc
