// Derivative of the loss with respect to the per-head decay.
//
// Lightning Attention-2 (Tiling paragraph; record mechanism field) carries a
// D x D key-value state from block to block; with a per-head decay lam the state
// before block b is S_b = sum_{j < b Bk} lam^(b Bk - 1 - j) k_j v_j^T (plus lam^(b Bk) S0).
// The decay enters the output only through powers of lam, so the derivative of
// L = <dO, O> + <F, S_N> follows the same tiling with the derivative of every
// power: d(lam^e)/dlam = e lam^(e-1).  Per block with local index s and m tokens:
//   intra:  sum_{s' < s} (s-s') lam^(s-s'-1) (q_s . k_s')(dO_s . v_s')
//   inter:  sum_s [ (s+1) lam^s q_s S_b dO_s + lam^(s+1) q_s T_b dO_s ]
// where T_b = dS_b/dlam is carried next to S_b:
//   T_{b+1} = lam^m T_b + m lam^(m-1) S_b + sum_s (m-1-s) lam^(m-2-s) k_s v_s^T,
//   S_{b+1} = lam^m S_b + sum_s lam^(m-1-s) k_s v_s^T,
// and the end of the sequence adds <F, T_N>.  The chunked prefix over blocks
// works as for the forward pass, with (S, T) as the carried pair: chunk
// aggregates of both, a scan (S, T) <- (lam^L S + dS, lam^L T + L lam^(L-1) S + dT),
// then one sweep per (sequence, chunk), each leaving one partial sum, and a last
// kernel adds the partials of every sequence and chunk of a head.
//
// Generic kernels (any supported D, Bk, float32 or bfloat16 storage) work in
// float32 on rows staged in LDS; the matrix-core kernels (bf16, D = 128, Bk = 64) keep
// both states in MFMA accumulators, with the same operand layouts as the
// register-staged forward kernel.  Partial sums are accumulated in double.
#include "la_device.h"
#include "la_internal.h"
#include "mfma_common.h"

namespace la {
namespace {

constexpr int kMaxD = 128;
constexpr int kMaxBk = 128;

__device__ __forceinline__ double block_sum(double x, double* red) {
    const int tid = threadIdx.x;
    red[tid] = x;
    __syncthreads();
    for (int h = kThreads / 2; h > 0; h >>= 1) {
        if (tid < h) red[tid] += red[tid + h];
        __syncthreads();
    }
    return red[0];
}

// ------------------------------------------------------------------ generic kernels
// Chunk aggregates of (S, T) over chunk c = blockIdx % (chunks - 1) of sequence
// blockIdx / (chunks - 1), both started from zero; x = k (through the feature map
// when phi_mask bit 0 is set), y = v.  Each block (at most 64 tokens: the aggregate is
// the same at any block size) has its rows read from global memory once, into LDS
// (rows padded to DG + 1 floats); thread i owns state elements i, i + 256, ... of both,
// in registers.  DG (= a.D) is a compile-time constant, so the loops over features unroll.
constexpr int kStateRows = 64;
template <bool BF16, int DG>
__global__ __launch_bounds__(kThreads) void k_dlam_state_generic(ChunkStateArgs a, LamArgs lam) {
    constexpr int rp = DG + 1, DD = DG * DG;
    constexpr int NE = (DD + kThreads - 1) / kThreads;
    __shared__ float xs[kStateRows * (kMaxD + 1)];
    __shared__ float ys[kStateRows * (kMaxD + 1)];
    __shared__ float pw[kStateRows + 1], dpw[kStateRows + 1];
    const int per = a.chunks - 1;
    const int64_t pair = blockIdx.x / per;
    const int c = blockIdx.x % per;
    const int Bs = min(a.Bk, kStateRows), tid = threadIdx.x;
    const float lv = lam.lam[pair % a.H];
    const int phi = (a.phi_mask & 1) ? a.phi : 0;
    for (int e = tid; e <= Bs; e += kThreads) {
        pw[e] = lam_pow(lv, e);
        dpw[e] = lam_dpow(lv, e);
    }
    float S[NE], T[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) S[e] = T[e] = 0.f;
    const int64_t t_begin = static_cast<int64_t>(c) * a.L;
    const int64_t t_end = min(a.N, t_begin + a.L);
    const int64_t base = pair * a.N * DG;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += Bs) {
        const int m = static_cast<int>(min(static_cast<int64_t>(Bs), t_end - t0));
        const int64_t r0 = base + t0 * DG;
        __syncthreads();  // the previous block's rows are done with (and the powers are in)
        for (int i = tid; i < m * DG; i += kThreads) {
            const int row = i / DG, col = i % DG;
            xs[row * rp + col] = phi_apply(ld<BF16>(a.x, r0 + row * DG + col), phi);
            ys[row * rp + col] = ld<BF16>(a.y, r0 + row * DG + col);
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const int i = tid + e * kThreads;
            if (i < DD) {
                const int f = i / DG, col = i % DG;
                float a1 = 0.f, a2 = 0.f;
#pragma unroll 8
                for (int s2 = 0; s2 < m; ++s2) {
                    const float xy = xs[s2 * rp + f] * ys[s2 * rp + col];
                    a1 += pw[m - 1 - s2] * xy;
                    a2 += dpw[m - 1 - s2] * xy;
                }
                const float s_old = S[e];
                T[e] = pw[m] * T[e] + dpw[m] * s_old + a2;
                S[e] = pw[m] * s_old + a1;
            }
        }
    }
    float* dst = a.slots + (pair * per + c) * 2 * static_cast<int64_t>(DD);
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        const int i = tid + e * kThreads;
        if (i < DD) {
            dst[i] = S[e];
            dst[DD + i] = T[e];
        }
    }
}

// In-place scan over the (S, T) slots of every sequence, one thread per state element.
__global__ __launch_bounds__(kThreads) void k_dlam_scan(ScanArgs a, LamArgs lam) {
    const int DD = a.D * a.D;
    const int per_pair = (DD + kThreads - 1) / kThreads;
    const int64_t pair = blockIdx.x / per_pair;
    const int e = (blockIdx.x % per_pair) * kThreads + threadIdx.x;
    if (e >= DD) return;
    const float lv = lam.lam[pair % a.H];
    const float lamL = lam_pow(lv, a.L), dlamL = lam_dpow(lv, a.L);
    float* sl = a.slots + pair * (a.chunks - 1) * 2 * static_cast<int64_t>(DD) + e;
    float S = a.kv_in ? a.kv_in[pair * DD + e] : 0.f, T = 0.f;
    const int n = a.chunks - 1;
    // each batch's loads go out before any of its stores (one memory latency per batch)
    constexpr int kBatch = 8;
    float xs[kBatch], xt[kBatch];
    for (int c0 = 0; c0 < n; c0 += kBatch) {
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const float* p = sl + static_cast<int64_t>(c0 + j) * 2 * DD;
            xs[j] = c0 + j < n ? p[0] : 0.f;
            xt[j] = c0 + j < n ? p[DD] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
            if (c0 + j < n) {
                float* p = sl + static_cast<int64_t>(c0 + j) * 2 * DD;
                T = lamL * T + dlamL * S + xt[j];
                S = lamL * S + xs[j];
                p[0] = S;
                p[DD] = T;
            }
    }
}

// The sweep's LDS: S and T ([DG][DG]; every access runs along a row, one column per
// thread, so they need no padding), the block's q, k, v and dO rows (feature map applied to
// q and k; rows padded to DG + 1 floats) and the decay powers and their derivatives, for
// blocks of Bs tokens, the largest block dividing the call's Bk that fits
// (dlam_generic_block: 8 tokens at D = 128, where the two states take 128 KiB).
constexpr int kDlamPoolFloats = 37 * 1024;  // 148 KiB
constexpr int kDlamMinBlock = 8;
__host__ __device__ constexpr int dlam_pool_floats(int D, int Bs) { return 2 * D * D + 4 * Bs * (D + 1) + 2 * (Bs + 2); }
static_assert(dlam_pool_floats(kMaxD, kDlamMinBlock) <= kDlamPoolFloats, "every D fits at the smallest block");

// The sweep over one (sequence, chunk): states in LDS, each block's rows read from global
// memory once, into LDS; DG (= a.D) a compile-time constant, so the loops over features unroll.
template <bool BF16, int DG>
__global__ __launch_bounds__(kThreads) void k_dlam_generic(DlamArgs a, LamArgs lam) {
    __shared__ float pool[kDlamPoolFloats];
    __shared__ double red[kThreads];
    constexpr int rp = DG + 1, DD = DG * DG;
    const int64_t pair = blockIdx.x / a.chunks;
    const int c = blockIdx.x % a.chunks;
    const int Bk = a.Bk, tid = threadIdx.x;
    float* S = pool;              // [DG][DG]
    float* T = S + DD;
    float* qs = T + DD;           // [Bk][DG + 1] each: phi(q), phi(k), v, dO
    float* ks = qs + Bk * rp;
    float* vs = ks + Bk * rp;
    float* gs = vs + Bk * rp;
    float* pw = gs + Bk * rp;     // lam^e, e = 0..Bk + 1
    float* dpw = pw + Bk + 2;     // d(lam^e)/dlam
    const float lv = lam.lam[pair % a.H];
    const int64_t base = pair * a.N * DG;
    const int64_t t_begin = static_cast<int64_t>(c) * a.L;
    const int64_t t_end = min(a.N, t_begin + a.L);
    for (int e = tid; e <= Bk + 1; e += kThreads) {
        pw[e] = lam_pow(lv, e);
        dpw[e] = lam_dpow(lv, e);
    }
    if (c == 0) {
        const float* s0 = a.kv_in ? a.kv_in + pair * DD : nullptr;
        for (int i = tid; i < DD; i += kThreads) {
            S[i] = s0 ? s0[i] : 0.f;
            T[i] = 0.f;
        }
    } else {
        const float* src = a.slots + dlam_slot_offset(a, pair, c);
        for (int i = tid; i < DD; i += kThreads) {
            S[i] = src[i];
            T[i] = src[DD + i];
        }
    }
    double acc = 0.0;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += Bk) {
        const int m = static_cast<int>(min(static_cast<int64_t>(Bk), t_end - t0));
        const int64_t r0 = base + t0 * DG;
        __syncthreads();  // the previous block's rows and state update are done with
        for (int i = tid; i < m * DG; i += kThreads) {
            const int row = i / DG, col = i % DG;
            const int64_t at = r0 + row * DG + col;
            qs[row * rp + col] = phi_apply(ld<BF16>(a.q, at), a.phi);
            ks[row * rp + col] = phi_apply(ld<BF16>(a.k, at), a.phi);
            vs[row * rp + col] = ld<BF16>(a.v, at);
            gs[row * rp + col] = ld<BF16>(a.g, at);
        }
        __syncthreads();
        for (int i = tid; i < m * m; i += kThreads) {
            const int s1 = i / m, s2 = i % m;
            if (s2 >= s1) continue;
            float qk = 0.f, gv = 0.f;
#pragma unroll
            for (int f = 0; f < DG; ++f) {
                qk += qs[s1 * rp + f] * ks[s2 * rp + f];
                gv += gs[s1 * rp + f] * vs[s2 * rp + f];
            }
            acc += static_cast<double>(dpw[s1 - s2] * qk * gv);
        }
        for (int i = tid; i < m * DG; i += kThreads) {
            const int s1 = i / DG, col = i % DG;
            float u = 0.f, w = 0.f;
#pragma unroll
            for (int f = 0; f < DG; ++f) {
                const float x = qs[s1 * rp + f];
                u += x * S[f * DG + col];
                w += x * T[f * DG + col];
            }
            acc += static_cast<double>(gs[s1 * rp + col] * (dpw[s1 + 1] * u + pw[s1 + 1] * w));
        }
        __syncthreads();  // S and T are read above and rewritten below
        for (int i = tid; i < DD; i += kThreads) {
            const int f = i / DG, col = i % DG;
            float a1 = 0.f, a2 = 0.f;
#pragma unroll 8
            for (int s2 = 0; s2 < m; ++s2) {
                const float xy = ks[s2 * rp + f] * vs[s2 * rp + col];
                a1 += pw[m - 1 - s2] * xy;
                a2 += dpw[m - 1 - s2] * xy;
            }
            const float s_old = S[i];
            T[i] = pw[m] * T[i] + dpw[m] * s_old + a2;
            S[i] = pw[m] * s_old + a1;
        }
    }
    __syncthreads();
    if (a.g_final && c == a.chunks - 1) {
        const float* F = a.g_final + pair * DD;
        for (int i = tid; i < DD; i += kThreads) acc += static_cast<double>(F[i] * T[i]);
    }
    const double tot = block_sum(acc, red);
    if (tid == 0) a.partial[pair * a.chunks + c] = tot;
}

// dlam[h] = sum over the batch and the chunks of the partials of head h; one workgroup per head.
__global__ __launch_bounds__(kThreads) void k_dlam_reduce(const double* partial, int64_t B, int H, int chunks,
                                                          float* out) {
    __shared__ double red[kThreads];
    const int h = blockIdx.x;
    const int64_t total = B * chunks;
    double acc = 0.0;
    for (int64_t i = threadIdx.x; i < total; i += kThreads) {
        const int64_t b = i / chunks, c = i % chunks;
        acc += partial[(b * H + h) * chunks + c];
    }
    const double tot = block_sum(acc, red);
    if (threadIdx.x == 0) out[h] = static_cast<float>(tot);
}

// ------------------------------------------------------------------ matrix-core kernels
constexpr int D = 128;

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float elemf(const u32x4& x, int e) {
    const uint32_t w = x[e >> 1];
    return (e & 1) ? hi_bf16(w) : lo_bf16(w);
}

__device__ __forceinline__ uint32_t elem16(const u32x4& x, int e) {
    const uint32_t w = x[e >> 1];
    return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// The feature map on 8 packed bf16 values, rounded back to bf16.
__device__ __forceinline__ u32x4 phi8(const u32x4& x, int kind) {
    if (kind == kPhiIdentity) return x;
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = pack_bf16(phi_apply(lo_bf16(x[j]), kind), phi_apply(hi_bf16(x[j]), kind));
    return r;
}

// Chunk aggregates of (S, T) on matrix cores: wave w owns value columns [32w, 32w+32)
// of both states (accumulators S[at][vt][r] = S[16 at + 4 g + r][32 w + 16 vt + li]).
// Per block the decayed key tile K~ = diag(lam^(m-1-s)) K and its derivative tile
// K' = diag((m-1-s) lam^(m-2-s)) K are written transposed to LDS next to V^T.
template <int BK>
__global__ __launch_bounds__(kThreads, 2) void k_dlam_state_mfma(ChunkStateArgs a, LamArgs lam) {
    constexpr int TP = BK + 8, NKS = BK / 32, RPT = BK / 16;
    __shared__ uint16_t xt[D * TP];
    __shared__ uint16_t xd[D * TP];
    __shared__ uint16_t yt[D * TP];
    __shared__ float pw[BK + 1], dpw[BK + 1];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, li = lane & 15;
    const int per = a.chunks - 1;
    const int64_t pair = blockIdx.x / per;
    const int c = blockIdx.x % per;
    const int phi = (a.phi_mask & 1) ? a.phi : 0;
    const int64_t t_begin = static_cast<int64_t>(c) * a.L;
    const int64_t t_end = min(a.N, t_begin + a.L);
    const int64_t base = pair * a.N * D;
    const uint16_t* __restrict__ Xg = static_cast<const uint16_t*>(a.x) + base;
    const uint16_t* __restrict__ Yg = static_cast<const uint16_t*>(a.y) + base;
    const float lv = lam.lam[pair % a.H];
    for (int e = tid; e <= BK; e += kThreads) {
        pw[e] = lam_pow(lv, e);
        dpw[e] = lam_dpow(lv, e);
    }

    f32x4 S[8][2], T[8][2];
#pragma unroll
    for (int at = 0; at < 8; ++at)
#pragma unroll
        for (int vt = 0; vt < 2; ++vt) S[at][vt] = T[at][vt] = zero4();

    const int fg = tid & 15, r0 = RPT * (tid >> 4);
    const int64_t nblk = (t_end - t_begin + BK - 1) / BK;
    u32x4 gx[RPT], gy[RPT];
    auto load_tile = [&](int64_t n) {
        const int64_t t0 = t_begin + n * BK;
        const int m = static_cast<int>(min(static_cast<int64_t>(BK), t_end - t0));
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            // rows past the end of a partial block read the last valid row and are zeroed
            const int row = r0 + i;
            const int64_t off = (t0 + min(row, m - 1)) * D + 8 * fg;
            const u32x4 z{0, 0, 0, 0};
            const u32x4 xx = *reinterpret_cast<const u32x4*>(Xg + off);
            const u32x4 xy = *reinterpret_cast<const u32x4*>(Yg + off);
            gx[i] = row < m ? xx : z;
            gy[i] = row < m ? xy : z;
        }
    };
    load_tile(0);
    __syncthreads();  // decay tables

    for (int64_t n = 0; n < nblk; ++n) {
        const int64_t t0 = t_begin + n * BK;
        const int m = static_cast<int>(min(static_cast<int64_t>(BK), t_end - t0));
        float wx[RPT], wd[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int s = r0 + i;
            wx[i] = masked_pw(pw, m - 1 - s, s < m);
            wd[i] = masked_pw(dpw, m - 1 - s, s < m);
        }
        u32x4 fx[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) fx[i] = phi8(gx[i], phi);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint32_t xw[RPT / 2], dw[RPT / 2], yw[RPT / 2];
#pragma unroll
            for (int i = 0; i < RPT; i += 2) {
                const float x0 = elemf(fx[i], e), x1 = elemf(fx[i + 1], e);
                xw[i / 2] = pack_bf16(x0 * wx[i], x1 * wx[i + 1]);
                dw[i / 2] = pack_bf16(x0 * wd[i], x1 * wd[i + 1]);
                yw[i / 2] = elem16(gy[i], e) | (elem16(gy[i + 1], e) << 16);
            }
            const int o = (8 * fg + e) * TP + r0;
            if constexpr (RPT == 4) {
                *reinterpret_cast<u32x2*>(&xt[o]) = u32x2{xw[0], xw[1]};
                *reinterpret_cast<u32x2*>(&xd[o]) = u32x2{dw[0], dw[1]};
                *reinterpret_cast<u32x2*>(&yt[o]) = u32x2{yw[0], yw[1]};
            } else {
                *reinterpret_cast<u32x4*>(&xt[o]) = u32x4{xw[0], xw[1], xw[2], xw[3]};
                *reinterpret_cast<u32x4*>(&xd[o]) = u32x4{dw[0], dw[1], dw[2], dw[3]};
                *reinterpret_cast<u32x4*>(&yt[o]) = u32x4{yw[0], yw[1], yw[2], yw[3]};
            }
        }
        __syncthreads();
        if (n + 1 < nblk) load_tile(n + 1);
        bf16x8 yf[2][NKS];
#pragma unroll
        for (int vt = 0; vt < 2; ++vt)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) yf[vt][ks] = lds_operand(yt, 32 * w + 16 * vt + li, TP, 32 * ks, g);
        const float lm = pw[m], dlm = dpw[m];
#pragma unroll
        for (int at = 0; at < 8; ++at) {
#pragma unroll
            for (int vt = 0; vt < 2; ++vt) {
                T[at][vt] = lm * T[at][vt] + dlm * S[at][vt];
                S[at][vt] *= lm;
            }
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8 kf = lds_operand(xt, 16 * at + li, TP, 32 * ks, g);
                const bf16x8 df = lds_operand(xd, 16 * at + li, TP, 32 * ks, g);
#pragma unroll
                for (int vt = 0; vt < 2; ++vt) {
                    S[at][vt] = mfma16(kf, yf[vt][ks], S[at][vt]);
                    T[at][vt] = mfma16(df, yf[vt][ks], T[at][vt]);
                }
            }
        }
        __syncthreads();
    }
    float* dst = a.slots + (pair * per + c) * 2 * static_cast<int64_t>(D * D);
#pragma unroll
    for (int at = 0; at < 8; ++at)
#pragma unroll
        for (int vt = 0; vt < 2; ++vt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int e = (16 * at + 4 * g + r) * D + 32 * w + 16 * vt + li;
                dst[e] = S[at][vt][r];
                dst[D * D + e] = T[at][vt][r];
            }
}

template <int BK>
struct DlamTiles {
    static constexpr int QP = D + 8;   // row pitch of the row-major tiles
    static constexpr int TP = BK + 8;  // row pitch of the transposed tiles
    uint16_t q[BK * QP];  // phi(Q)
    uint16_t k[BK * QP];  // phi(K)
    uint16_t v[BK * QP];
    uint16_t g[BK * QP];  // dO
    uint16_t kt[D * TP];  // kt[f][s] = bf16(lam^(m-1-s) phi(K)[s][f])
    uint16_t kd[D * TP];  // kd[f][s] = bf16((m-1-s) lam^(m-2-s) phi(K)[s][f])
    uint16_t vt[D * TP];  // vt[v][s] = V[s][v]
    float pw[BK + 2];
    float dpw[BK + 2];
    double red[kThreads / 64];
};

// The sweep on matrix cores: one workgroup (4 waves) per (sequence, chunk).  Wave w
// owns value columns [32w, 32w+32) of S and T.  Per block:
//   intra: the causal 16x16 tiles of P^T = K Q^T and G^T = V dO^T (shared out over the
//          waves), multiplied elementwise with the derivative mask and summed;
//   inter: X^T = S^T Q^T and Y^T = T^T Q^T for the wave's columns, dotted with dO^T
//          under the row weights (s+1) lam^s and lam^(s+1);
//   then T and S advance by one block.
template <int BK>
__global__ __launch_bounds__(kThreads, 1) void k_dlam_mfma(DlamArgs a, LamArgs lam) {
    using Tl = DlamTiles<BK>;
    constexpr int NT = BK / 16, QP = Tl::QP, TP = Tl::TP;
    constexpr int NKS = BK / 32, RPT = BK / 16;
    __shared__ Tl sm;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, li = lane & 15;
    const int64_t pair = blockIdx.x / a.chunks;
    const int c = blockIdx.x % a.chunks;
    const float lv = lam.lam[pair % a.H];
    const int64_t t_begin = static_cast<int64_t>(c) * a.L;
    const int64_t t_end = min(a.N, t_begin + a.L);
    const int64_t base = pair * a.N * D;
    const uint16_t* __restrict__ Qg = static_cast<const uint16_t*>(a.q) + base;
    const uint16_t* __restrict__ Kg = static_cast<const uint16_t*>(a.k) + base;
    const uint16_t* __restrict__ Vg = static_cast<const uint16_t*>(a.v) + base;
    const uint16_t* __restrict__ Gg = static_cast<const uint16_t*>(a.g) + base;

    for (int e = tid; e <= BK + 1; e += kThreads) {
        sm.pw[e] = lam_pow(lv, e);
        sm.dpw[e] = lam_dpow(lv, e);
    }

    f32x4 S[8][2], T[8][2];
    {
        const float* s_src = nullptr;
        const float* t_src = nullptr;
        if (c == 0) {
            s_src = a.kv_in ? a.kv_in + pair * D * D : nullptr;
        } else {
            s_src = a.slots + dlam_slot_offset(a, pair, c);
            t_src = s_src + D * D;
        }
#pragma unroll
        for (int at = 0; at < 8; ++at)
#pragma unroll
            for (int vt = 0; vt < 2; ++vt) {
                const int col = 32 * w + 16 * vt + li;
                f32x4 xs = zero4(), xt = zero4();
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int e = (16 * at + 4 * g + r) * D + col;
                    if (s_src) xs[r] = s_src[e];
                    if (t_src) xt[r] = t_src[e];
                }
                S[at][vt] = xs;
                T[at][vt] = xt;
            }
    }

    const int fg = tid & 15, r0 = RPT * (tid >> 4);
    u32x4 gq[RPT], gk[RPT], gv[RPT], gg[RPT];
    auto load_tile = [&](int64_t t0, int m) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            // rows past the end of a partial block read the last valid row and are zeroed
            const int row = r0 + i;
            const int64_t off = (t0 + min(row, m - 1)) * D + 8 * fg;
            const u32x4 z{0, 0, 0, 0};
            const u32x4 xq = *reinterpret_cast<const u32x4*>(Qg + off);
            const u32x4 xk = *reinterpret_cast<const u32x4*>(Kg + off);
            const u32x4 xv = *reinterpret_cast<const u32x4*>(Vg + off);
            const u32x4 xg = *reinterpret_cast<const u32x4*>(Gg + off);
            gq[i] = row < m ? xq : z;
            gk[i] = row < m ? xk : z;
            gv[i] = row < m ? xv : z;
            gg[i] = row < m ? xg : z;
        }
    };
    load_tile(t_begin, static_cast<int>(min(static_cast<int64_t>(BK), t_end - t_begin)));
    __syncthreads();  // decay tables

    double acc = 0.0;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += BK) {
        const int m = static_cast<int>(min(static_cast<int64_t>(BK), t_end - t0));

        // ---- 1. staged registers -> LDS (padded rows: v and dO are zero, the key
        //         weights are zero, so they contribute nothing whatever phi(0) is)
        {
            float wk[RPT], wd[RPT];
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int s = r0 + i;
                wk[i] = masked_pw(sm.pw, m - 1 - s, s < m);
                wd[i] = masked_pw(sm.dpw, m - 1 - s, s < m);
            }
            u32x4 fk[RPT];
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                fk[i] = phi8(gk[i], a.phi);
                const int o = (r0 + i) * QP + 8 * fg;
                *reinterpret_cast<u32x4*>(&sm.q[o]) = phi8(gq[i], a.phi);
                *reinterpret_cast<u32x4*>(&sm.k[o]) = fk[i];
                *reinterpret_cast<u32x4*>(&sm.v[o]) = gv[i];
                *reinterpret_cast<u32x4*>(&sm.g[o]) = gg[i];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint32_t kw[RPT / 2], dw[RPT / 2], vw[RPT / 2];
#pragma unroll
                for (int i = 0; i < RPT; i += 2) {
                    const float x0 = elemf(fk[i], e), x1 = elemf(fk[i + 1], e);
                    kw[i / 2] = pack_bf16(x0 * wk[i], x1 * wk[i + 1]);
                    dw[i / 2] = pack_bf16(x0 * wd[i], x1 * wd[i + 1]);
                    vw[i / 2] = elem16(gv[i], e) | (elem16(gv[i + 1], e) << 16);
                }
                const int o = (8 * fg + e) * TP + r0;
                if constexpr (RPT == 4) {
                    *reinterpret_cast<u32x2*>(&sm.kt[o]) = u32x2{kw[0], kw[1]};
                    *reinterpret_cast<u32x2*>(&sm.kd[o]) = u32x2{dw[0], dw[1]};
                    *reinterpret_cast<u32x2*>(&sm.vt[o]) = u32x2{vw[0], vw[1]};
                } else {
                    *reinterpret_cast<u32x4*>(&sm.kt[o]) = u32x4{kw[0], kw[1], kw[2], kw[3]};
                    *reinterpret_cast<u32x4*>(&sm.kd[o]) = u32x4{dw[0], dw[1], dw[2], dw[3]};
                    *reinterpret_cast<u32x4*>(&sm.vt[o]) = u32x4{vw[0], vw[1], vw[2], vw[3]};
                }
            }
        }
        __syncthreads();

        // ---- 2. prefetch the next block while this one computes
        if (t0 + BK < t_end) load_tile(t0 + BK, static_cast<int>(min(static_cast<int64_t>(BK), t_end - t0 - BK)));

        float part = 0.f;
        // ---- 3. intra: tile (at, st) of P^T and G^T holds entries [s' = 16 at + 4 g + r][s = 16 st + li];
        //         weight (s-s') lam^(s-s'-1) for s' < s (the table's entry 0 is 0)
#pragma unroll
        for (int st = 0; st < NT; ++st)
#pragma unroll
            for (int at = 0; at <= st; ++at) {
                const int idx = st * (st + 1) / 2 + at;
                if (idx % 4 != w) continue;
                f32x4 p = zero4(), q2 = zero4();
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    p = mfma16(lds_operand(sm.k, 16 * at + li, QP, 32 * ks, g),
                               lds_operand(sm.q, 16 * st + li, QP, 32 * ks, g), p);
                    q2 = mfma16(lds_operand(sm.v, 16 * at + li, QP, 32 * ks, g),
                                lds_operand(sm.g, 16 * st + li, QP, 32 * ks, g), q2);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int e = 16 * (st - at) + li - 4 * g - r;
                    part += masked_pw(sm.dpw, e, e > 0) * p[r] * q2[r];
                }
            }

        // ---- 4. inter: per 16-token column st, X^T = S^T Q^T and Y^T = T^T Q^T for this
        //         wave's columns col = 32 w + 16 vt + 4 g + r, against dO[s][col]; T enters as
        //         its bf16 operand plus the residual of that rounding
        {
            bf16x8 sb[2][4], tb[2][4];
#pragma unroll
            for (int vt = 0; vt < 2; ++vt)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    sb[vt][ks] = operand_from_acc(S[2 * ks][vt], S[2 * ks + 1][vt]);
                    tb[vt][ks] = operand_from_acc(T[2 * ks][vt], T[2 * ks + 1][vt]);
                }
#pragma unroll
            for (int st = 0; st < NT; ++st) {
                const int s = 16 * st + li;
                bf16x8 qf[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) qf[ks] = lds_operand(sm.q, s, QP, 32 * ks, g);
                const float w1 = sm.dpw[s + 1], w2 = sm.pw[s + 1];
#pragma unroll
                for (int vt = 0; vt < 2; ++vt) {
                    f32x4 x = zero4(), y = zero4();
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        x = mfma16(sb[vt][ks], qf[ks], x);
                        y = mfma16(tb[vt][ks], qf[ks], y);
                        // T is large next to the result near lam = 1: add its rounding residual
                        y = mfma16(operand_residual_from_acc(T[2 * ks][vt], T[2 * ks + 1][vt]), qf[ks], y);
                    }
                    const u32x2 d = *reinterpret_cast<const u32x2*>(&sm.g[s * QP + 32 * w + 16 * vt + 4 * g]);
                    const float d0 = lo_bf16(d.x), d1 = hi_bf16(d.x), d2 = lo_bf16(d.y), d3 = hi_bf16(d.y);
                    part += d0 * (w1 * x[0] + w2 * y[0]) + d1 * (w1 * x[1] + w2 * y[1]) +
                            d2 * (w1 * x[2] + w2 * y[2]) + d3 * (w1 * x[3] + w2 * y[3]);
                }
                // keep the scheduler from hoisting every column's LDS reads (register pressure)
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        acc += static_cast<double>(part);

        // ---- 5. T <- lam^m T + m lam^(m-1) S + K'^T V,  S <- lam^m S + K~^T V
        {
            bf16x8 vf[2][NKS];
#pragma unroll
            for (int vt = 0; vt < 2; ++vt)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) vf[vt][ks] = lds_operand(sm.vt, 32 * w + 16 * vt + li, TP, 32 * ks, g);
            const float lm = sm.pw[m], dlm = sm.dpw[m];
#pragma unroll
            for (int at = 0; at < 8; ++at) {
#pragma unroll
                for (int vt = 0; vt < 2; ++vt) {
                    T[at][vt] = lm * T[at][vt] + dlm * S[at][vt];
                    S[at][vt] *= lm;
                }
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const bf16x8 kf = lds_operand(sm.kt, 16 * at + li, TP, 32 * ks, g);
                    const bf16x8 df = lds_operand(sm.kd, 16 * at + li, TP, 32 * ks, g);
#pragma unroll
                    for (int vt = 0; vt < 2; ++vt) {
                        S[at][vt] = mfma16(kf, vf[vt][ks], S[at][vt]);
                        T[at][vt] = mfma16(df, vf[vt][ks], T[at][vt]);
                    }
                }
            }
        }
        __syncthreads();
    }

    if (a.g_final && c == a.chunks - 1) {
        const float* F = a.g_final + pair * D * D;
        float part = 0.f;
#pragma unroll
        for (int at = 0; at < 8; ++at)
#pragma unroll
            for (int vt = 0; vt < 2; ++vt)
#pragma unroll
                for (int r = 0; r < 4; ++r) part += F[(16 * at + 4 * g + r) * D + 32 * w + 16 * vt + li] * T[at][vt][r];
        acc += static_cast<double>(part);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (lane == 0) sm.red[w] = acc;
    __syncthreads();
    if (tid == 0) a.partial[pair * a.chunks + c] = sm.red[0] + sm.red[1] + sm.red[2] + sm.red[3];
}

}  // namespace

namespace {
template <bool BF16>
void (*dlam_state_generic_kernel(int d))(ChunkStateArgs, LamArgs) {
    switch (d) {
        case 16: return k_dlam_state_generic<BF16, 16>;
        case 32: return k_dlam_state_generic<BF16, 32>;
        case 64: return k_dlam_state_generic<BF16, 64>;
        default: return k_dlam_state_generic<BF16, 128>;
    }
}
template <bool BF16>
void (*dlam_generic_kernel(int d))(DlamArgs, LamArgs) {
    switch (d) {
        case 16: return k_dlam_generic<BF16, 16>;
        case 32: return k_dlam_generic<BF16, 32>;
        case 64: return k_dlam_generic<BF16, 64>;
        default: return k_dlam_generic<BF16, 128>;
    }
}
}  // namespace

void launch_dlam_state_generic(const ChunkStateArgs& a, const LamArgs& lam, int bf16, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(a.pairs * (a.chunks - 1)));
    auto kern = bf16 ? dlam_state_generic_kernel<true>(a.D) : dlam_state_generic_kernel<false>(a.D);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, s, a, lam);
}

void launch_dlam_state_mfma(const ChunkStateArgs& a, const LamArgs& lam, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(a.pairs * (a.chunks - 1)));
    hipLaunchKernelGGL(k_dlam_state_mfma<64>, grid, dim3(kThreads), 0, s, a, lam);
}

void launch_dlam_scan(const ScanArgs& a, const LamArgs& lam, hipStream_t s) {
    const int per_pair = (a.D * a.D + kThreads - 1) / kThreads;
    dim3 grid(static_cast<unsigned>(a.pairs * per_pair));
    hipLaunchKernelGGL(k_dlam_scan, grid, dim3(kThreads), 0, s, a, lam);
}

// The block the generic sweep steps: the largest of Bk, Bk/2, ... that fits (the block only
// decides which terms pass through the in-block sum and which through the carried states).
DlamArgs dlam_generic_block(const DlamArgs& a) {
    DlamArgs b = a;
    while (b.Bk > kDlamMinBlock && dlam_pool_floats(b.D, b.Bk) > kDlamPoolFloats) b.Bk /= 2;
    return b;
}

void launch_dlam_generic(const DlamArgs& a, const LamArgs& lam, int bf16, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(a.pairs * a.chunks));
    const DlamArgs b = dlam_generic_block(a);
    auto kern = bf16 ? dlam_generic_kernel<true>(b.D) : dlam_generic_kernel<false>(b.D);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, s, b, lam);
}

bool dlam_mfma_supported(int d, int bk) { return d == D && bk == 64; }

void launch_dlam_mfma(const DlamArgs& a, const LamArgs& lam, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(a.pairs * a.chunks));
    hipLaunchKernelGGL(k_dlam_mfma<64>, grid, dim3(kThreads), 0, s, a, lam);
}

void launch_dlam_reduce(const double* partial, int64_t B, int H, int chunks, float* out, hipStream_t s) {
    hipLaunchKernelGGL(k_dlam_reduce, dim3(static_cast<unsigned>(H)), dim3(kThreads), 0, s, partial, B, H, chunks,
                       out);
}

}  // namespace la
