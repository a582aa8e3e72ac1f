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

// d(lam^e)/dlam = e lam^(e-1) in double, 0 for e = 0 (lam^-1 is never formed, so lam = 0
// gives 1 for e = 1 and 0 beyond).
__device__ __forceinline__ double lam_dpow64(float lam, int64_t e) {
    return e > 0 ? static_cast<double>(e) * lam_pow64(lam, e - 1) : 0.0;
}
__device__ __forceinline__ float lam_dpow(float lam, int64_t e) { return static_cast<float>(lam_dpow64(lam, e)); }

// Elementwise kernel feature maps on queries and keys (identity, elu(x) + 1,
// relu); both non-identity maps have a derivative that is a function of phi(x)
// itself: min(1, phi) for elu + 1, [phi > 0] for relu.
enum { kPhiIdentity = 0, kPhiElu1 = 1, kPhiRelu = 2 };

__device__ __forceinline__ float phi_apply(float x, int kind) {
    if (kind == kPhiElu1) return x > 0.f ? x + 1.f : __expf(x);
    if (kind == kPhiRelu) return x > 0.f ? x : 0.f;
    return x;
}

__device__ __forceinline__ float dphi_of_phi(float y, int kind) {
    if (kind == kPhiElu1) return fminf(y, 1.f);
    if (kind == kPhiRelu) return y > 0.f ? 1.f : 0.f;
    return 1.f;
}

__device__ __forceinline__ float dphi_of_x(float x, int kind) { return dphi_of_phi(phi_apply(x, kind), kind); }

// keep ? pw[e] : 0 for a decay table pw in LDS.  The read is unconditional (the
// index is clamped to the table), so several of them issue back to back rather
// than as one masked branch and LDS round trip each.
__device__ __forceinline__ float masked_pw(const float* pw, int e, bool keep) {
    const float v = pw[e > 0 ? e : 0];
    return keep ? v : 0.f;
}

// Largest b in [0, nseq) with key(b) <= x, for a nondecreasing key (a binary search
// over kernel-argument values, uniform across the workgroup).
template <typename Key>
__device__ __forceinline__ int find_last_le(int nseq, int x, Key key) {
    int lo = 0, hi = nseq - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (key(mid) <= x)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// What one workgroup of a sweep works on: chunk c of one (sequence, head).
struct Work {
    int64_t base;    // element offset of the sequence's token 0
    int64_t ld;      // elements from one token's row to the next
    int64_t n;       // tokens in the sequence
    int64_t t_begin, t_end;
    int64_t state;   // index of the sequence's D x D initial / final state
    int64_t slot0;   // slot of the state entering chunk 1; chunk c's is slot0 + (c - 1) * step
    int c, chunks, slot_step, head;
};

// Dense [P][N][D] problems (pair = blockIdx / chunks) or a ragged batch (VarlenArgs).
template <bool VARLEN, typename SA, typename VA>
__device__ __forceinline__ Work work_item(const SA& a, const VA* v, int64_t blk) {
    Work w;
    if constexpr (!VARLEN) {
        const int64_t pair = blk / a.chunks;
        w.c = static_cast<int>(blk % a.chunks);
        w.chunks = a.chunks;
        w.head = static_cast<int>(pair % a.H);
        w.n = a.N;
        w.base = pair * a.N * a.D;
        w.ld = a.D;
        w.state = pair;
        // chunk c >= 1 starts from slot c * k - 1 of the sequence's (chunks - 1) k slots
        const int64_t k = a.slot_k > 1 ? a.slot_k : 1;
        w.slot0 = pair * (a.chunks - 1) * k + k - 1;
        w.slot_step = static_cast<int>(k);
    } else {
        // full chunks first (sequence-major), then every sequence's last chunk, longest first
        const int h = static_cast<int>(blk % a.H);
        const int wi = static_cast<int>(blk / a.H);
        const int full = v->wp[v->nseq] - v->nseq;
        int b;
        if (wi < full) {
            b = find_last_le(v->nseq, wi, [&](int i) { return v->wp[i] - i; });
            w.c = wi - (v->wp[b] - b);
        } else {
            b = v->last_order[wi - full];
            w.c = v->wp[b + 1] - v->wp[b] - 1;
        }
        w.chunks = v->wp[b + 1] - v->wp[b];
        w.head = h;
        w.n = v->cu[b + 1] - v->cu[b];
        w.base = (static_cast<int64_t>(v->cu[b]) * a.H + h) * a.D;
        w.ld = static_cast<int64_t>(a.H) * a.D;
        w.state = static_cast<int64_t>(b) * a.H + h;
        w.slot0 = static_cast<int64_t>(v->wp[b] - b) * a.H + h;
        w.slot_step = a.H;
    }
    w.t_begin = static_cast<int64_t>(w.c) * a.L;
    w.t_end = min(w.n, w.t_begin + a.L);
    return w;
}

}  // namespace la
