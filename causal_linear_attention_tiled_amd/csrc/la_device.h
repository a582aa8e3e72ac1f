// Device helpers shared by the kernels: storage conversion and decay powers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest even; NaN stays NaN (quiet bit forced).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Element access for the two storage types.
template <bool BF16>
__device__ __forceinline__ float ld(const void* p, int64_t i) {
    if constexpr (BF16)
        return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
    else
        return static_cast<const float*>(p)[i];
}

template <bool BF16>
__device__ __forceinline__ void st(void* p, int64_t i, float x) {
    if constexpr (BF16)
        static_cast<uint16_t*>(p)[i] = f32_to_bf16(x);
    else
        static_cast<float*>(p)[i] = x;
}

// lam^e for e >= 0, by binary powering in double.  lam^0 = 1 exactly, also for lam = 0.
__device__ __forceinline__ double lam_pow64(float lam, int64_t e) {
    double base = static_cast<double>(lam), r = 1.0;
    while (e > 0) {
        if (e & 1) r *= base;
        base *= base;
        e >>= 1;
    }
    return r;
}

// The same rounded once to float.
__device__ __forceinline__ float lam_pow(float lam, int64_t e) { return static_cast<float>(lam_pow64(lam, e)); }

// keep ? pw[e] : 0 for a decay table pw in LDS.  The read is unconditional (the
// index is clamped to the table), so several of them issue back to back rather
// than as one masked branch and LDS round trip each.
__device__ __forceinline__ float masked_pw(const float* pw, int e, bool keep) {
    const float v = pw[e > 0 ? e : 0];
    return keep ? v : 0.f;
}

}  // namespace la
