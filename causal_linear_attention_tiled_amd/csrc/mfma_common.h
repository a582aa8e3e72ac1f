// Matrix-core building blocks for gfx950 (CDNA4), wave64.
//
// All products use v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] B[32x16]
// with float32 accumulation.  Lane l (g = l / 16, i = l % 16) holds
//   A operand : A[i][kappa(g, e)]           e = 0..7 (8 bf16)
//   B operand : B[kappa(g, e)][i]
//   C/D       : D[4 g + r][i]                r = 0..3 (4 floats)
// where kappa is any fixed bijection of (g, e) onto 0..31 used by both
// operands.  We use kappa(g, e) = 4 g + e for e < 4 and 16 + 4 g + (e - 4)
// for e >= 4: with it, the accumulators of the two 16x16 tiles covering rows
// 0..15 and 16..31 of a 32-row block are exactly an operand whose k index
// runs over those 32 rows, so a result can feed the next product from
// registers.  A row-major operand is read with two 8-byte loads per lane
// (columns 4g..4g+3 and 16+4g..16+4g+3 of its row).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Round two floats to bf16 (nearest even) and pack them, low half first
// (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Operand from two 8-byte halves (kappa order: first half e = 0..3, second e = 4..7).
__device__ __forceinline__ bf16x8 operand(const u32x2& lo, const u32x2& hi) {
    u32x4 v{lo.x, lo.y, hi.x, hi.y};
    return __builtin_bit_cast(bf16x8, v);
}

// Operand from the accumulators of two vertically adjacent 16x16 tiles.
__device__ __forceinline__ bf16x8 operand_from_acc(const f32x4& top, const f32x4& bottom) {
    u32x4 v{pack_bf16(top[0], top[1]), pack_bf16(top[2], top[3]), pack_bf16(bottom[0], bottom[1]),
            pack_bf16(bottom[2], bottom[3])};
    return __builtin_bit_cast(bf16x8, v);
}

// x - bf16(x) for two floats (bf16 as pack_bf16 rounds), rounded to bf16 and packed.
__device__ __forceinline__ uint32_t pack_bf16_residual(float lo, float hi) {
    const uint32_t h = pack_bf16(lo, hi);
    return pack_bf16(lo - __uint_as_float(h << 16), hi - __uint_as_float(h & 0xFFFF0000u));
}

// The rounding residual of operand_from_acc: the two operands together carry the
// accumulators to about 16 significant bits, for a product whose operand is large
// next to the result it feeds.
__device__ __forceinline__ bf16x8 operand_residual_from_acc(const f32x4& top, const f32x4& bottom) {
    u32x4 v{pack_bf16_residual(top[0], top[1]), pack_bf16_residual(top[2], top[3]),
            pack_bf16_residual(bottom[0], bottom[1]), pack_bf16_residual(bottom[2], bottom[3])};
    return __builtin_bit_cast(bf16x8, v);
}

// Read a kappa-ordered operand fragment from a row-major bf16 tile in LDS:
// row `row`, k columns [k0, k0 + 32).  `pitch` is the row pitch in elements.
__device__ __forceinline__ bf16x8 lds_operand(const uint16_t* base, int row, int pitch, int k0, int g) {
    const uint16_t* p = base + row * pitch + k0 + 4 * g;
    const u32x2 lo = *reinterpret_cast<const u32x2*>(p);
    const u32x2 hi = *reinterpret_cast<const u32x2*>(p + 16);
    return operand(lo, hi);
}

}  // namespace la
