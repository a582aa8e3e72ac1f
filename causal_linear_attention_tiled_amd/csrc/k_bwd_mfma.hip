// Reverse (dK, dV) sweep on matrix cores (bf16 storage, D = 128, Bk = 64).
//
// The backward half of Lightning Attention-2's tiling (Tiling paragraph:
// the same intra/inter split in the backward pass): blocks are visited from
// last to first, carrying the gradient state
//     dS = sum_{i >= end of block} lam^(i - end) q_i dO_i^T     (D x D)
// and per block b with local index s and m tokens:
//     dK_b = ((dO_b V_b^T) o M)^T Q_b + diag(lam^(m-s)) V_b dS^T
//     dV_b = ((Q_b K_b^T) o M)^T dO_b + diag(lam^(m-s)) K_b dS
//     dS  <- lam^m dS + (diag(lam^s) Q_b)^T dO_b,
// with M[i][j] = lam^(i-j) for i >= j, else 0.
//
// One workgroup (4 waves) runs one (sequence, chunk).  Wave w keeps two
// float32 copies of dS in MFMA accumulators: dS[:, 32w..32w+32) (value
// columns, feeds dV) and dS^T[:, 32w..32w+32) (key rows, feeds dK); each
// copy is the A operand of its inter-block product straight from registers.
// The wave computes dV^T for its value columns and dK^T for its key rows.
// The masked score tiles P = Q K^T and G = dO V^T are computed once per block
// (shared across the waves through LDS) and enter as B operands.
#include "la_device.h"
#include "la_internal.h"
#include "mfma_common.h"

namespace la {
namespace {

constexpr int D = 128;
constexpr int BK = 64;
constexpr int QP = D + 8;
constexpr int TP = BK + 8;
constexpr int NT = BK / 16;
constexpr int NKS = BK / 32;
constexpr int NCAUSAL = NT * (NT + 1) / 2;
constexpr int RPT = BK / 16;

struct RevTiles {
    uint16_t q[BK * QP];
    uint16_t k[BK * QP];
    uint16_t v[BK * QP];
    uint16_t g[BK * QP];    // dO
    uint16_t qt[D * TP];    // qt[f][s] = Q[s][f]
    uint16_t gt[D * TP];    // gt[c][s] = dO[s][c]
    uint32_t p[NCAUSAL * 128];   // masked decayed P = Q K^T tiles (i >= j), B-operand fragments
    uint32_t gg[NCAUSAL * 128];  // masked decayed G = dO V^T tiles
    float pw[BK + 1];
};

__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t elem16(const u32x4& x, int e) {
    const uint32_t w = x[e >> 1];
    return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// Multiply the 8 bf16 of an operand by per-element weights, rounding back to bf16.
__device__ __forceinline__ bf16x8 scale_operand(const bf16x8& x, const float* wt) {
    const u32x4 u = __builtin_bit_cast(u32x4, x);
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = pack_bf16(lo_bf(u[i]) * wt[2 * i], hi_bf(u[i]) * wt[2 * i + 1]);
    return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ u32x2 ld_frag(const uint32_t* buf, int idx, int lane) {
    return *reinterpret_cast<const u32x2*>(&buf[idx * 128 + 2 * lane]);
}

__global__ __launch_bounds__(kThreads, 1) void k_rev_mfma(SweepArgs a, LamArgs lam) {
    __shared__ RevTiles sm;
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
    const uint16_t* __restrict__ Gg = static_cast<const uint16_t*>(a.g) + base;
    uint16_t* __restrict__ dKg = static_cast<uint16_t*>(a.out0) + base;
    uint16_t* __restrict__ dVg = static_cast<uint16_t*>(a.out1) + base;

    for (int e = tid; e <= BK; e += kThreads) sm.pw[e] = lam_pow(lv, e);

    // dS entering this chunk from the right (0 for the last chunk).
    //   Sv[at][vt][r] = dS[16 at + 4 g + r][32 w + 16 vt + li]
    //   Sk[vt][kt][r] = dS^T[16 vt + 4 g + r][32 w + 16 kt + li] = dS[32 w + 16 kt + li][16 vt + 4 g + r]
    f32x4 Sv[8][2], Sk[8][2];
    {
        const float* init = (c < a.chunks - 1) ? a.slots + rev_slot_index(a, pair, c) * D * D
                                               : (a.g_final ? a.g_final + pair * D * D : nullptr);
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f32x4 x = zero4(), y = zero4();
                if (init) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) x[r] = init[(16 * t8 + 4 * g + r) * D + 32 * w + 16 * h + li];
                    const float4 t4 = *reinterpret_cast<const float4*>(init + (32 * w + 16 * h + li) * D + 16 * t8 + 4 * g);
                    y = f32x4{t4.x, t4.y, t4.z, t4.w};
                }
                Sv[t8][h] = x;
                Sk[t8][h] = y;
            }
    }

    const int fg = tid & 15, r0 = RPT * (tid >> 4);
    const int64_t nblk = (t_end - t_begin + BK - 1) / BK;
    u32x4 gq[RPT], gk[RPT], gv[RPT], gd[RPT];
    auto load_tile = [&](int64_t n) {
        const int64_t t0 = t_begin + n * BK;
        const int m = static_cast<int>(min(static_cast<int64_t>(BK), t_end - t0));
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            // rows past the end of a partial block read the last valid row and are zeroed
            const int row = r0 + i;
            const int64_t off = (t0 + min(row, m - 1)) * D + 8 * fg;
            const u32x4 z{0, 0, 0, 0};
            const u32x4 xq = *reinterpret_cast<const u32x4*>(Qg + off);
            const u32x4 xk = *reinterpret_cast<const u32x4*>(Kg + off);
            const u32x4 xv = *reinterpret_cast<const u32x4*>(Vg + off);
            const u32x4 xd = *reinterpret_cast<const u32x4*>(Gg + off);
            gq[i] = row < m ? xq : z;
            gk[i] = row < m ? xk : z;
            gv[i] = row < m ? xv : z;
            gd[i] = row < m ? xd : z;
        }
    };
    load_tile(nblk - 1);
    __syncthreads();  // decay table

    // lam^s weights of the dS update for s = 32 ks + kappa(g, e) (independent of m: rows past m are 0)
    float wq[NKS][8];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) wq[ks][e] = sm.pw[32 * ks + (e < 4 ? 4 * g + e : 16 + 4 * g + e - 4)];

    for (int64_t n = nblk - 1; n >= 0; --n) {
        // the final-state gradient reaches the sequence's last block one power less decayed
        const int shift = (c == a.chunks - 1 && a.g_final && n == nblk - 1) ? 1 : 0;
        const int64_t t0 = t_begin + n * BK;
        const int m = static_cast<int>(min(static_cast<int64_t>(BK), t_end - t0));

        // ---- 1. staged registers -> LDS (row-major Q, K, V, dO; transposed Q, dO)
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int o = (r0 + i) * QP + 8 * fg;
            *reinterpret_cast<u32x4*>(&sm.q[o]) = gq[i];
            *reinterpret_cast<u32x4*>(&sm.k[o]) = gk[i];
            *reinterpret_cast<u32x4*>(&sm.v[o]) = gv[i];
            *reinterpret_cast<u32x4*>(&sm.g[o]) = gd[i];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const u32x2 qw{elem16(gq[0], e) | (elem16(gq[1], e) << 16), elem16(gq[2], e) | (elem16(gq[3], e) << 16)};
            const u32x2 dw{elem16(gd[0], e) | (elem16(gd[1], e) << 16), elem16(gd[2], e) | (elem16(gd[3], e) << 16)};
            *reinterpret_cast<u32x2*>(&sm.qt[(8 * fg + e) * TP + r0]) = qw;
            *reinterpret_cast<u32x2*>(&sm.gt[(8 * fg + e) * TP + r0]) = dw;
        }
        __syncthreads();
        if (n > 0) load_tile(n - 1);

        // ---- 2. shared masked score tiles: u < NCAUSAL -> P tile u, else G tile u - NCAUSAL.
        // Tile (it, jt), it >= jt, holds X[16 it + 4 g + r][16 jt + li], kept iff i >= j,
        // scaled by lam^(i - j).
#pragma unroll
        for (int it = 0; it < NT; ++it)
#pragma unroll
            for (int jt = 0; jt <= it; ++jt)
#pragma unroll
                for (int which = 0; which < 2; ++which) {
                    const int idx = it * (it + 1) / 2 + jt;
                    if ((idx + which * NCAUSAL) % 4 != w) continue;
                    const uint16_t* A = which ? sm.g : sm.q;
                    const uint16_t* B = which ? sm.v : sm.k;
                    f32x4 x = zero4();
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        x = mfma16(lds_operand(A, 16 * it + li, QP, 32 * ks, g), lds_operand(B, 16 * jt + li, QP, 32 * ks, g), x);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int d = 16 * (it - jt) + 4 * g + r - li;
                        x[r] *= masked_pw(sm.pw, d, d >= 0);
                    }
                    uint32_t* dst = which ? sm.gg : sm.p;
                    *reinterpret_cast<u32x2*>(&dst[idx * 128 + 2 * lane]) = u32x2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
                }
        __syncthreads();

        // ---- 3. per 16-token column jt: dV^T (this wave's value columns) and dK^T (its key rows)
        bf16x8 gtf[2][NKS], qtf[2][NKS];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                gtf[h][ks] = lds_operand(sm.gt, 32 * w + 16 * h + li, TP, 32 * ks, g);
                qtf[h][ks] = lds_operand(sm.qt, 32 * w + 16 * h + li, TP, 32 * ks, g);
            }
#pragma unroll
        for (int jt = 0; jt < NT; ++jt) {
            const int j = 16 * jt + li;
            const float lj = masked_pw(sm.pw, m - shift - j, j < m);
            bf16x8 kb[4], vb[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                kb[ks] = lds_operand(sm.k, j, QP, 32 * ks, g);
                vb[ks] = lds_operand(sm.v, j, QP, 32 * ks, g);
            }
            f32x4 dv[2], dk[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f32x4 x = zero4(), y = zero4();
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    x = mfma16(operand_from_acc(Sv[2 * ks][h], Sv[2 * ks + 1][h]), kb[ks], x);
                    y = mfma16(operand_from_acc(Sk[2 * ks][h], Sk[2 * ks + 1][h]), vb[ks], y);
                }
                dv[h] = x * lj;
                dk[h] = y * lj;
            }
#pragma unroll
            for (int ks = jt / 2; ks < NKS; ++ks) {
                const int i0 = 2 * ks, i1 = 2 * ks + 1;
                const u32x2 z{0, 0};
                const u32x2 plo = (i0 >= jt) ? ld_frag(sm.p, i0 * (i0 + 1) / 2 + jt, lane) : z;
                const u32x2 phi = (i1 >= jt) ? ld_frag(sm.p, i1 * (i1 + 1) / 2 + jt, lane) : z;
                const u32x2 glo = (i0 >= jt) ? ld_frag(sm.gg, i0 * (i0 + 1) / 2 + jt, lane) : z;
                const u32x2 ghi = (i1 >= jt) ? ld_frag(sm.gg, i1 * (i1 + 1) / 2 + jt, lane) : z;
                const bf16x8 pb = operand(plo, phi), gb = operand(glo, ghi);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    dv[h] = mfma16(gtf[h][ks], pb, dv[h]);
                    dk[h] = mfma16(qtf[h][ks], gb, dk[h]);
                }
            }
            // dv[h][r] = dV[j][32 w + 16 h + 4 g + r], dk[h][r] = dK[j][32 w + 16 h + 4 g + r]
            if (j < m) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int64_t off = (t0 + j) * D + 32 * w + 16 * h + 4 * g;
                    *reinterpret_cast<u32x2*>(dVg + off) = u32x2{pack_bf16(dv[h][0], dv[h][1]), pack_bf16(dv[h][2], dv[h][3])};
                    *reinterpret_cast<u32x2*>(dKg + off) = u32x2{pack_bf16(dk[h][0], dk[h][1]), pack_bf16(dk[h][2], dk[h][3])};
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- 4. dS <- lam^m dS + (diag(lam^s) Q)^T dO, both copies
        const float lm = sm.pw[m - shift];
        bf16x8 qs[2][NKS];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) qs[h][ks] = scale_operand(qtf[h][ks], wq[ks]);
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                Sv[t8][h] *= lm;
                Sk[t8][h] *= lm;
            }
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8 qa = scale_operand(lds_operand(sm.qt, 16 * t8 + li, TP, 32 * ks, g), wq[ks]);
                const bf16x8 ga = lds_operand(sm.gt, 16 * t8 + li, TP, 32 * ks, g);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    Sv[t8][h] = mfma16(qa, gtf[h][ks], Sv[t8][h]);
                    Sk[t8][h] = mfma16(ga, qs[h][ks], Sk[t8][h]);
                }
            }
        }
        __syncthreads();
    }
    if (c == 0 && a.ds_out) {
        // gradient of the initial state: lam dS, from the value-column copy
        float* dst = a.ds_out + pair * D * D;
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[(16 * t8 + 4 * g + r) * D + 32 * w + 16 * h + li] = lv * Sv[t8][h][r];
    }
}

}  // namespace

bool mfma_rev_supported(int d, int bk) { return d == 128 && bk == 64; }

void launch_rev_mfma(const SweepArgs& a, const LamArgs& lam, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(a.pairs * a.chunks));
    hipLaunchKernelGGL(k_rev_mfma, grid, dim3(kThreads), 0, s, a, lam);
}

}  // namespace la
