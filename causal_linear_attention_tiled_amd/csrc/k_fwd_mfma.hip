// Fused forward sweep on matrix cores (bf16 storage, D = 128, Bk in {64, 128}).
//
// Lightning Attention-2 (Tiling paragraph; record mechanism field): each
// block of Bk tokens gets its intra-block part from a masked, decayed dense
// product like ordinary attention, and its inter-block part from the running
// D x D key-value state, which is then decayed and updated; the same carry
// gives the final state.  Per block b with local index s and m tokens:
//     O_b     = diag(lam^(s+1)) Q_b S_b + ((Q_b K_b^T) o M) V_b,
//     M[s][s'] = lam^(s-s') for s >= s', else 0,
//     S_{b+1} = lam^m S_b + (diag(lam^(m-1-s)) K_b)^T V_b.
//
// One workgroup (4 waves) runs one (sequence, chunk) block by block.  Wave w
// owns value columns [32w, 32w+32): its slice of the float32 state lives in
// MFMA accumulators (8 x 2 tiles of 16x16) for the whole sweep, and it
// computes the transposed output O^T[its columns][s] = S^T Q^T + V^T A^T,
// where A^T = (K Q^T) o M^T is shared through LDS.  Computing transposes lets
// accumulators feed the next product directly (see mfma_common.h):
//   - the state accumulators are the A operand of S^T Q^T,
//   - the score accumulators K Q^T are the B operand of V^T A^T,
//   - V^T fragments serve both V^T A^T and the state update K~^T V.
// The next block's Q, K, V are loaded into registers while the current block
// computes; the tiles are written to LDS row-major (Q, K) and transposed
// (K~ = decayed K, V) once per block.
#include "la_device.h"
#include "la_internal.h"
#include "mfma_common.h"

namespace la {
namespace {

constexpr int D = 128;

template <int BK>
struct FwdTiles {
    static constexpr int QP = D + 8;   // row pitch (elements) of the row-major Q and K tiles
    static constexpr int TP = BK + 8;  // row pitch of the transposed tiles
    static constexpr int NT = BK / 16;
    static constexpr int NCAUSAL = NT * (NT + 1) / 2;
    uint16_t q[BK * QP];
    uint16_t k[BK * QP];
    uint16_t kt[D * TP];  // kt[f][s] = bf16(lam^(m-1-s) K[s][f])
    uint16_t vt[D * TP];  // vt[v][s] = V[s][v]
    uint32_t at[NCAUSAL * 128];  // masked decayed scores K Q^T, one 16x16 tile = 64 lanes x 8 bytes
    float pw[BK + 1];
};

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t lo16(uint32_t w) { return w & 0xFFFFu; }
__device__ __forceinline__ uint32_t hi16(uint32_t w) { return w >> 16; }

// Element e (0..7) of 8 bf16 packed in a u32x4, as raw 16 bits.
__device__ __forceinline__ uint32_t elem16(const u32x4& x, int e) {
    const uint32_t w = x[e >> 1];
    return (e & 1) ? hi16(w) : lo16(w);
}

__device__ __forceinline__ float elemf(const u32x4& x, int e) {
    const uint32_t w = x[e >> 1];
    return (e & 1) ? hi_bf16(w) : lo_bf16(w);
}

template <int BK>
__global__ __launch_bounds__(kThreads, (BK == 64) ? 2 : 1) void k_fwd_mfma(SweepArgs a, LamArgs lam) {
    using T = FwdTiles<BK>;
    constexpr int NT = T::NT, QP = T::QP, TP = T::TP;
    constexpr int NKS = BK / 32;  // 32-wide k steps over the tokens of a block
    constexpr int RPT = BK / 16;  // rows staged per thread
    __shared__ T sm;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, li = lane & 15;
    const int64_t pair = blockIdx.x / a.chunks;
    const int c = blockIdx.x % a.chunks;
    const float lv = lam.lam[pair % a.H];
    const int64_t t_begin = static_cast<int64_t>(c) * a.L;
    const int64_t t_end = min(a.N, t_begin + a.L);
    const int64_t base = pair * a.N * D;
    const uint16_t* __restrict__ Qg = static_cast<const uint16_t*>(a.a) + base;
    const uint16_t* __restrict__ Kg = static_cast<const uint16_t*>(a.b) + base;
    const uint16_t* __restrict__ Vg = static_cast<const uint16_t*>(a.c) + base;
    uint16_t* __restrict__ Og = static_cast<uint16_t*>(a.out0) + base;

    for (int e = tid; e <= BK; e += kThreads) sm.pw[e] = lam_pow(lv, e);

    // Initial state of this chunk: the state accumulators hold
    // S[16 at + 4 g + r][32 w + 16 vt + li] in S[at][vt][r].
    f32x4 S[8][2];
    {
        const float* init = nullptr;
        bool tr = false, poison = false;
        if (c == 0) {
            if (a.kv_in) {
                init = a.kv_in + pair * D * D;
                tr = a.kv_in_transposed != 0;
            }
        } else {
            init = a.slots + fwd_slot_index(a, pair, c) * D * D;
            tr = a.slots_transposed != 0;
            poison = !given_states_match(a);
        }
#pragma unroll
        for (int at = 0; at < 8; ++at)
#pragma unroll
            for (int vt = 0; vt < 2; ++vt) {
                const int col = 32 * w + 16 * vt + li;
                f32x4 x = zero4();
                if (init) {
                    if (tr) {
                        const float4 t4 = *reinterpret_cast<const float4*>(init + col * D + 16 * at + 4 * g);
                        x = f32x4{t4.x, t4.y, t4.z, t4.w};
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) x[r] = init[(16 * at + 4 * g + r) * D + col];
                    }
                }
                if (poison) x = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
                S[at][vt] = x;
            }
    }

    // Staging: thread owns feature group fg (8 features) of rows r0 .. r0+RPT-1.
    const int fg = tid & 15, r0 = RPT * (tid >> 4);
    u32x4 gq[RPT], gk[RPT], gv[RPT];
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
            gq[i] = row < m ? xq : z;
            gk[i] = row < m ? xk : z;
            gv[i] = row < m ? xv : z;
        }
    };
    load_tile(t_begin, static_cast<int>(min(static_cast<int64_t>(BK), t_end - t_begin)));
    __syncthreads();  // decay table

    // Per-lane row scale lam^(s+1) of output column s = 16 st + li.
    float rs[NT];
#pragma unroll
    for (int st = 0; st < NT; ++st) rs[st] = sm.pw[16 * st + li + 1];

    for (int64_t t0 = t_begin; t0 < t_end; t0 += BK) {
        const int m = static_cast<int>(min(static_cast<int64_t>(BK), t_end - t0));

        // ---- 1. staged registers -> LDS
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            *reinterpret_cast<u32x4*>(&sm.q[(r0 + i) * QP + 8 * fg]) = gq[i];
            *reinterpret_cast<u32x4*>(&sm.k[(r0 + i) * QP + 8 * fg]) = gk[i];
        }
        {
            float wk[RPT];
#pragma unroll
            for (int i = 0; i < RPT; ++i) wk[i] = masked_pw(sm.pw, m - 1 - (r0 + i), r0 + i < m);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint32_t kw[RPT / 2], vw[RPT / 2];
#pragma unroll
                for (int i = 0; i < RPT; i += 2) {
                    kw[i / 2] = pack_bf16(elemf(gk[i], e) * wk[i], elemf(gk[i + 1], e) * wk[i + 1]);
                    vw[i / 2] = elem16(gv[i], e) | (elem16(gv[i + 1], e) << 16);
                }
                uint16_t* kd = &sm.kt[(8 * fg + e) * TP + r0];
                uint16_t* vd = &sm.vt[(8 * fg + e) * TP + r0];
                if constexpr (RPT == 4) {
                    *reinterpret_cast<u32x2*>(kd) = u32x2{kw[0], kw[1]};
                    *reinterpret_cast<u32x2*>(vd) = u32x2{vw[0], vw[1]};
                } else {
                    *reinterpret_cast<u32x4*>(kd) = u32x4{kw[0], kw[1], kw[2], kw[3]};
                    *reinterpret_cast<u32x4*>(vd) = u32x4{vw[0], vw[1], vw[2], vw[3]};
                }
            }
        }
        __syncthreads();

        // ---- 2. prefetch the next block while this one computes
        if (t0 + BK < t_end) load_tile(t0 + BK, static_cast<int>(min(static_cast<int64_t>(BK), t_end - t0 - BK)));

        // ---- 3. this wave's share of the masked, decayed score tiles A^T = (K Q^T) o M^T.
        // Tile (at, st) holds A^T[16 at + 4 g + r][16 st + li]; it is kept iff s' <= s and
        // scaled by lam^(s - s') = lam^(16 (st - at) + li - 4 g - r).
#pragma unroll
        for (int st = 0; st < NT; ++st)
#pragma unroll
            for (int at = 0; at <= st; ++at) {
                const int idx = st * (st + 1) / 2 + at;
                if (idx % 4 != w) continue;
                f32x4 p = zero4();
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    p = mfma16(lds_operand(sm.k, 16 * at + li, QP, 32 * ks, g),
                               lds_operand(sm.q, 16 * st + li, QP, 32 * ks, g), p);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int d = 16 * (st - at) + li - 4 * g - r;
                    p[r] *= masked_pw(sm.pw, d, d >= 0);
                }
                *reinterpret_cast<u32x2*>(&sm.at[idx * 128 + 2 * lane]) =
                    u32x2{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])};
            }
        __syncthreads();

        // ---- 4. per 16-token column st: O^T = diag(lam^(s+1)) S^T Q^T + V^T A^T, then store.
        bf16x8 vf[2][NKS];
#pragma unroll
        for (int vt = 0; vt < 2; ++vt)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) vf[vt][ks] = lds_operand(sm.vt, 32 * w + 16 * vt + li, TP, 32 * ks, g);
        bf16x8 sb[2][4];
#pragma unroll
        for (int vt = 0; vt < 2; ++vt)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) sb[vt][ks] = operand_from_acc(S[2 * ks][vt], S[2 * ks + 1][vt]);
#pragma unroll
        for (int st = 0; st < NT; ++st) {
            bf16x8 qf[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) qf[ks] = lds_operand(sm.q, 16 * st + li, QP, 32 * ks, g);
            f32x4 o[2];
#pragma unroll
            for (int vt = 0; vt < 2; ++vt) {
                f32x4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) acc = mfma16(sb[vt][ks], qf[ks], acc);
                o[vt] = acc * rs[st];
            }
#pragma unroll
            for (int ks = 0; ks <= st / 2; ++ks) {
                const int a0 = 2 * ks, a1 = 2 * ks + 1;
                const u32x2 lo = *reinterpret_cast<const u32x2*>(&sm.at[(st * (st + 1) / 2 + a0) * 128 + 2 * lane]);
                u32x2 hi = u32x2{0, 0};
                if (a1 <= st) hi = *reinterpret_cast<const u32x2*>(&sm.at[(st * (st + 1) / 2 + a1) * 128 + 2 * lane]);
                const bf16x8 b = operand(lo, hi);
#pragma unroll
                for (int vt = 0; vt < 2; ++vt) o[vt] = mfma16(vf[vt][ks], b, o[vt]);
            }
            // o[vt][r] = O[16 st + li][32 w + 16 vt + 4 g + r]
            const int s = 16 * st + li;
            if (s < m) {
#pragma unroll
                for (int vt = 0; vt < 2; ++vt) {
                    uint16_t* dst = Og + (t0 + s) * D + 32 * w + 16 * vt + 4 * g;
                    *reinterpret_cast<u32x2*>(dst) =
                        u32x2{pack_bf16(o[vt][0], o[vt][1]), pack_bf16(o[vt][2], o[vt][3])};
                }
            }
            // keep the scheduler from hoisting every column's LDS reads (register pressure)
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- 6. S <- lam^m S + K~^T V
        const float lm = sm.pw[m];
#pragma unroll
        for (int at = 0; at < 8; ++at) {
            S[at][0] *= lm;
            S[at][1] *= lm;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8 kf = lds_operand(sm.kt, 16 * at + li, TP, 32 * ks, g);
                S[at][0] = mfma16(kf, vf[0][ks], S[at][0]);
                S[at][1] = mfma16(kf, vf[1][ks], S[at][1]);
            }
        }
        __syncthreads();
    }

    if (a.kv_out && c == a.chunks - 1) {
        float* dst = a.kv_out + pair * D * D;
#pragma unroll
        for (int at = 0; at < 8; ++at)
#pragma unroll
            for (int vt = 0; vt < 2; ++vt)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[(16 * at + 4 * g + r) * D + 32 * w + 16 * vt + li] = S[at][vt][r];
    }
}

// Chunk aggregate (see ChunkStateArgs): the state update alone, started from zero.
//   forward: acc <- lam^m acc + (diag(lam^(m-1-s)) X_b)^T Y_b over blocks in order
//   reverse: acc <- lam^m acc + (diag(lam^s) X_b)^T Y_b over blocks from last to first
template <int BK>
__global__ __launch_bounds__(kThreads, 2) void k_chunk_state_mfma(ChunkStateArgs a, LamArgs lam) {
    constexpr int TP = BK + 8, NKS = BK / 32, RPT = BK / 16;
    __shared__ uint16_t xt[D * TP];
    __shared__ uint16_t yt[D * TP];
    __shared__ float pw[BK + 1];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, li = lane & 15;
    const int per = a.chunks - 1;
    const int64_t pair = blockIdx.x / per;
    const int slot = blockIdx.x % per;
    const int c = a.reverse ? slot + 1 + a.part0 : slot;
    const int64_t t_begin = static_cast<int64_t>(c) * a.L;
    const int64_t t_end = min(a.N, t_begin + a.L);
    const int64_t base = pair * a.N * D;
    const uint16_t* __restrict__ Xg = static_cast<const uint16_t*>(a.x) + base;
    const uint16_t* __restrict__ Yg = static_cast<const uint16_t*>(a.y) + base;
    for (int e = tid; e <= BK; e += kThreads) pw[e] = lam_pow(lam.lam[pair % a.H], e);

    f32x4 S[8][2];
#pragma unroll
    for (int at = 0; at < 8; ++at) S[at][0] = S[at][1] = zero4();

    const int fg = tid & 15, r0 = RPT * (tid >> 4);
    const int64_t nblk = (t_end - t_begin + BK - 1) / BK;
    u32x4 gx[RPT], gy[RPT];
    auto load_tile = [&](int64_t n) {
        const int64_t bi = a.reverse ? nblk - 1 - n : n;
        const int64_t t0 = t_begin + bi * BK;
        const int m = static_cast<int>(min(static_cast<int64_t>(BK), t_end - t0));
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
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
    __syncthreads();

    for (int64_t n = 0; n < nblk; ++n) {
        const int64_t bi = a.reverse ? nblk - 1 - n : n;
        const int64_t t0 = t_begin + bi * BK;
        const int m = static_cast<int>(min(static_cast<int64_t>(BK), t_end - t0));
        float wx[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int s = r0 + i;
            wx[i] = (s < m) ? (a.reverse ? pw[s] : pw[m - 1 - s]) : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint32_t xw[RPT / 2], yw[RPT / 2];
#pragma unroll
            for (int i = 0; i < RPT; i += 2) {
                xw[i / 2] = pack_bf16(elemf(gx[i], e) * wx[i], elemf(gx[i + 1], e) * wx[i + 1]);
                yw[i / 2] = elem16(gy[i], e) | (elem16(gy[i + 1], e) << 16);
            }
            uint16_t* xd = &xt[(8 * fg + e) * TP + r0];
            uint16_t* yd = &yt[(8 * fg + e) * TP + r0];
            if constexpr (RPT == 4) {
                *reinterpret_cast<u32x2*>(xd) = u32x2{xw[0], xw[1]};
                *reinterpret_cast<u32x2*>(yd) = u32x2{yw[0], yw[1]};
            } else {
                *reinterpret_cast<u32x4*>(xd) = u32x4{xw[0], xw[1], xw[2], xw[3]};
                *reinterpret_cast<u32x4*>(yd) = u32x4{yw[0], yw[1], yw[2], yw[3]};
            }
        }
        __syncthreads();
        if (n + 1 < nblk) load_tile(n + 1);
        bf16x8 yf[2][NKS];
#pragma unroll
        for (int vt = 0; vt < 2; ++vt)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) yf[vt][ks] = lds_operand(yt, 32 * w + 16 * vt + li, TP, 32 * ks, g);
        const float lm = pw[m];
#pragma unroll
        for (int at = 0; at < 8; ++at) {
            S[at][0] *= lm;
            S[at][1] *= lm;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8 xf = lds_operand(xt, 16 * at + li, TP, 32 * ks, g);
                S[at][0] = mfma16(xf, yf[0][ks], S[at][0]);
                S[at][1] = mfma16(xf, yf[1][ks], S[at][1]);
            }
        }
        __syncthreads();
    }
    float* dst = a.slots + (pair * per + slot) * D * D;
#pragma unroll
    for (int at = 0; at < 8; ++at)
#pragma unroll
        for (int vt = 0; vt < 2; ++vt)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(16 * at + 4 * g + r) * D + 32 * w + 16 * vt + li] = S[at][vt][r];
}

}  // namespace

bool mfma_supported(int d, int bk) { return d == 128 && (bk == 64 || bk == 128); }

void launch_fwd_mfma(const SweepArgs& a, const LamArgs& lam, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(a.pairs * a.chunks));
    if (a.Bk == 64)
        hipLaunchKernelGGL(k_fwd_mfma<64>, grid, dim3(kThreads), 0, s, a, lam);
    else
        hipLaunchKernelGGL(k_fwd_mfma<128>, grid, dim3(kThreads), 0, s, a, lam);
}

void launch_chunk_state_mfma(const ChunkStateArgs& a, const LamArgs& lam, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(a.pairs * (a.chunks - 1)));
    if (a.Bk == 64)
        hipLaunchKernelGGL(k_chunk_state_mfma<64>, grid, dim3(kThreads), 0, s, a, lam);
    else
        hipLaunchKernelGGL(k_chunk_state_mfma<128>, grid, dim3(kThreads), 0, s, a, lam);
}

}  // namespace la
