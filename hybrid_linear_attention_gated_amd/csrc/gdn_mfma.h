// gdn_mfma.h -- bf16 MFMA fragment helpers for gfx950 (v_mfma_f32_16x16x32_bf16).
//
// One 16x16x32 MFMA on a 64-lane wavefront: lane l = 16*gq + i (gq = l / 16,
// i = l % 16) supplies row i of A and column i of B, eight k-slots each, and
// receives D[4*gq + r][i] for r = 0..3 (the "accumulator layout").  The
// hardware pairs A's and B's k-slots by (gq, slot), so any bijection between
// (gq, slot) and the 32 logical k indices of a step gives the same product as
// long as A and B use the same one.  This library always uses
//
//     kmap(s, gq, slot) = 32*s + 16*(slot / 4) + 4*gq + (slot % 4)
//
// for step s.  With it, a matrix held in accumulator layout (lane keeps rows
// 4*gq + r of a 16-row tile) is already a B operand along k: slot e of step s
// is element r = e % 4 of tile 2*s + e / 4.  State tiles, Delta tiles and the
// W and K fragments produced for the scan therefore move between products
// without any cross-lane shuffle or LDS round trip.
#pragma once

#include "gdn_internal.h"

namespace gdn {

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t to_bf16(float x) { return f32_to_bf16_bits(x); }
__device__ __forceinline__ float from_bf16(uint16_t h) { return bf16_bits_to_f32(h); }

__device__ __forceinline__ bf16x8 as_bf16x8(u16x8 u) { return __builtin_bit_cast(bf16x8, u); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Two fp32 -> two bf16 (round to nearest even) in one 32-bit word, element 0
// in the low half: a single v_cvt_pk_bf16_f32.
__device__ __forceinline__ unsigned cvt2_bf16(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}
// The two bf16 halves of a packed word, widened back to fp32 (exact).
__device__ __forceinline__ float lo_half_f32(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_half_f32(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Eight fp32 values -> one bf16 fragment (round to nearest even).
__device__ __forceinline__ bf16x8 pack_bf16(const float (&x)[8]) {
    const u32x4 w = {cvt2_bf16(x[0], x[1]), cvt2_bf16(x[2], x[3]), cvt2_bf16(x[4], x[5]),
                     cvt2_bf16(x[6], x[7])};
    return __builtin_bit_cast(bf16x8, w);
}

// Eight fp32 values -> hi + lo bf16 fragments: hi = RNE(x), lo = RNE(x - hi),
// so hi + lo carries about 16 significant bits of x.
__device__ __forceinline__ void split_bf16(const float (&x)[8], bf16x8 &hi, bf16x8 &lo) {
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = cvt2_bf16(x[2 * i], x[2 * i + 1]);
        l[i] = cvt2_bf16(x[2 * i] - lo_half_f32(h[i]), x[2 * i + 1] - hi_half_f32(h[i]));
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// Two accumulator tiles (consecutive 16-row blocks along k) -> the 8 k-slots of one step.
__device__ __forceinline__ void acc_pair_to_slots(f32x4 t0, f32x4 t1, float (&x)[8]) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        x[r] = t0[r];
        x[4 + r] = t1[r];
    }
}

// A fragment from a row-major bf16 matrix in LDS: row `row`, step s, group gq.
// Reads elements [32s + 4gq, +4) and [32s + 16 + 4gq, +4) of the row.
__device__ __forceinline__ bf16x8 lds_frag_bf16(const uint16_t *rowp, int s, int gq) {
    const u16x4 a = *reinterpret_cast<const u16x4 *>(rowp + 32 * s + 4 * gq);
    const u16x4 b = *reinterpret_cast<const u16x4 *>(rowp + 32 * s + 16 + 4 * gq);
    u16x8 u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        u[e] = a[e];
        u[4 + e] = b[e];
    }
    return as_bf16x8(u);
}

// The same 8 k-slots from a row-major fp32 matrix in LDS, as floats.
__device__ __forceinline__ void lds_slots_f32(const float *rowp, int s, int gq, float (&x)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(rowp + 32 * s + 4 * gq);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(rowp + 32 * s + 16 + 4 * gq);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[e] = a[e];
        x[4 + e] = b[e];
    }
}

// k index of slot e (0..7) of step s for lane group gq.
__device__ __forceinline__ int kmap(int s, int gq, int e) { return 32 * s + 16 * (e >> 2) + 4 * gq + (e & 3); }

}  // namespace gdn
