// Reverse (dK, dV) sweep, Bk = 64, D = 128, bf16, fed by direct
// global-to-LDS loads.
//
// Same arithmetic as the register-staged reverse kernel (the backward half
// of Lightning Attention-2's tiling, Tiling paragraph): blocks from last to
// first, carrying dS = sum_{i >= end of block} lam^(i - end) q_i dO_i^T,
//     dK_b = ((dO_b V_b^T) o M)^T Q_b + diag(lam^(m-s)) V_b dS^T
//     dV_b = ((Q_b K_b^T) o M)^T dO_b + diag(lam^(m-s)) K_b dS
//     dS  <- lam^m dS + (diag(lam^s) Q_b)^T dO_b.
// The four waves stream the raw row-major Q, K, V, dO tiles of the next block
// (in sweep order) into the second of two LDS stages while they compute the
// current one (each block starts with vmcnt(0), so loads and stores may share
// the counter in any order); every operand whose contraction runs over
// tokens (dO^T, Q^T, the decayed Q) is read from the row-major tiles with the
// transposing LDS read (lds_dma.h).  Wave w keeps dS[:, 32w..32w+32) and
// dS^T[:, 32w..32w+32) in MFMA accumulators, computes dV^T for its value
// columns and dK^T for its key rows, and the masked score tiles P = Q K^T and
// G = dO V^T are shared through LDS.
#include "la_device.h"
#include "la_internal.h"
#include "lds_dma.h"
#include "mfma_common.h"

namespace la {
namespace {

constexpr int D = 128;
constexpr int BK = 64;
constexpr int NT = BK / 16;
constexpr int NKS = BK / 32;
constexpr int NSTAGE = 2;
constexpr int TILE = BK * D;
constexpr int NCAUSAL = NT * (NT + 1) / 2;
constexpr int NW = 4;  // compute waves

struct RevDmaTiles {
    uint16_t t[NSTAGE][4][TILE];     // per stage: Q, K, V, dO (row-major, swizzled)
    uint32_t p[NCAUSAL * 128];       // masked decayed P = Q K^T tiles (i >= j), B-operand fragments
    uint32_t gg[NCAUSAL * 128];      // masked decayed G = dO V^T tiles
    float pw[BK + 1];
};

__device__ __forceinline__ u32x2 ld_frag(const uint32_t* buf, int idx, int lane) {
    return *reinterpret_cast<const u32x2*>(&buf[idx * 128 + 2 * lane]);
}

__global__ __launch_bounds__(64 * NW, 1) void k_rev_dma(SweepArgs a, LamArgs lam) {
    __shared__ RevDmaTiles sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, li = lane & 15;
    const int64_t pair = blockIdx.x / a.chunks;
    const int c = blockIdx.x % a.chunks;
    const float lv = lam.lam[pair % a.H];
    const int64_t t_begin = static_cast<int64_t>(c) * a.L;
    const int64_t t_end = min(a.N, t_begin + a.L);
    const int64_t nblk = (t_end - t_begin + BK - 1) / BK;
    const int64_t base = pair * a.N * D;

    for (int e = tid; e <= BK; e += 64 * NW) sm.pw[e] = lam_pow(lv, e);

    // DMA: wave w streams tensor w (Q, K, V, dO) of the i-th block of the sweep
    // (block nblk - 1 - i of the chunk) into stage i % 2, 16 loads of 1 KiB.
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const void* src = wu == 0 ? a.a : wu == 1 ? a.b : wu == 2 ? a.c : a.g;
    const u32x4 rsrc = buffer_rsrc(static_cast<const uint16_t*>(src) + base, static_cast<uint32_t>(a.N * D * 2));
    auto issue = [&](int64_t i) {
        const int stage = static_cast<int>(i % NSTAGE);
        const int64_t t0 = t_begin + (nblk - 1 - i) * BK;
        const int sub = lane >> 4, p = lane & 15;
#pragma unroll
        for (int rg = 0; rg < BK / 4; ++rg) {
            const int r = 4 * rg + sub;
            const int chunk = p ^ (r & 15);
            const int voff = static_cast<int>(((t0 + r) * D + 8 * chunk) * 2);
            dma16(rsrc, &sm.t[stage][wu][4 * rg * D], voff);
        }
    };
    issue(0);

    // ---------------------------------------------------------------- compute waves
    uint16_t* __restrict__ dKg = static_cast<uint16_t*>(a.out0) + base;
    uint16_t* __restrict__ dVg = static_cast<uint16_t*>(a.out1) + base;
    // dS entering this chunk from the right (0 for the last chunk).
    //   Sv[t8][h][r] = dS[16 t8 + 4 g + r][32 w + 16 h + li]
    //   Sk[t8][h][r] = dS^T[16 t8 + 4 g + r][32 w + 16 h + li]
    f32x4 Sv[8][2], Sk[8][2];
    {
        const float* init = (c < a.chunks - 1) ? a.slots + (pair * (a.chunks - 1) + c) * D * D : nullptr;
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
    // lam^s weights of the dS update, s = 32 ks + kappa(g, e) (rows past m are zero)
    float wq[NKS][8];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) wq[ks][e] = sm.pw[32 * ks + (e < 4 ? 4 * g + e : 16 + 4 * g + e - 4)];

    for (int64_t i = 0; i < nblk; ++i) {
        const int64_t n = nblk - 1 - i;
        const int64_t t0 = t_begin + n * BK;
        const int m = static_cast<int>(min(static_cast<int64_t>(BK), t_end - t0));
        const int stage = static_cast<int>(i % NSTAGE);
        const uint16_t* Qs = sm.t[stage][0];
        const uint16_t* Ks = sm.t[stage][1];
        const uint16_t* Vs = sm.t[stage][2];
        const uint16_t* Gs = sm.t[stage][3];
        // Only this block's loads (and earlier stores) are outstanding here.
        wait_vmcnt<0>();
        __syncthreads();  // A(i): stage i % 2 is ready; stage (i+1) % 2 is no longer read

        // ---- shared score tiles: P = Q K^T and G = dO V^T, (it, jt) with it >= jt,
        // element (16 it + 4 g + r, 16 jt + li) kept iff i >= j and scaled by lam^(i - j)
#pragma unroll
        for (int it = 0; it < NT; ++it)
#pragma unroll
            for (int jt = 0; jt <= it; ++jt)
#pragma unroll
                for (int which = 0; which < 2; ++which) {
                    const int idx = it * (it + 1) / 2 + jt;
                    if ((idx + which * NCAUSAL) % NW != w) continue;
                    const uint16_t* A = which ? Gs : Qs;
                    const uint16_t* B = which ? Vs : Ks;
                    f32x4 x = zero4();
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        x = mfma16(op_row(A, 16 * it + li, 32 * ks, g), op_row(B, 16 * jt + li, 32 * ks, g), x);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int d = 16 * (it - jt) + 4 * g + r - li;
                        x[r] *= d >= 0 ? sm.pw[d] : 0.f;
                    }
                    uint32_t* dst = which ? sm.gg : sm.p;
                    *reinterpret_cast<u32x2*>(&dst[idx * 128 + 2 * lane]) = u32x2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
                }
        __syncthreads();  // B(i)
        // Next block's loads go out after B(i), so that barrier never waits on them.
        if (i + 1 < nblk) issue(i + 1);

        // ---- per 16-token column jt: dV^T (value columns 32w..) and dK^T (key rows 32w..)
        bf16x8 gtf[2][NKS], qtf[2][NKS];  // dO^T[32w+16h+li][s], Q^T[32w+16h+li][s]
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                gtf[h][ks] = op_tr(Gs, 32 * ks, 32 * w + 16 * h, g, li);
                qtf[h][ks] = op_tr(Qs, 32 * ks, 32 * w + 16 * h, g, li);
            }
#pragma unroll
        for (int jt = 0; jt < NT; ++jt) {
            const int j = 16 * jt + li;
            const float lj = (j < m) ? sm.pw[m - j] : 0.f;
            bf16x8 kb[4], vb[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                kb[ks] = op_row(Ks, j, 32 * ks, g);
                vb[ks] = op_row(Vs, j, 32 * ks, g);
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

        // ---- dS <- lam^m dS + (diag(lam^s) Q)^T dO, both copies
        const float lm = sm.pw[m];
        bf16x8 qs[2][NKS];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) qs[h][ks] = scale8(qtf[h][ks], wq[ks]);
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                Sv[t8][h] *= lm;
                Sk[t8][h] *= lm;
            }
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8 qa = scale8(op_tr(Qs, 32 * ks, 16 * t8, g, li), wq[ks]);
                const bf16x8 ga = op_tr(Gs, 32 * ks, 16 * t8, g, li);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    Sv[t8][h] = mfma16(qa, gtf[h][ks], Sv[t8][h]);
                    Sk[t8][h] = mfma16(ga, qs[h][ks], Sk[t8][h]);
                }
            }
        }
    }
}

}  // namespace

bool rev_dma_supported(int d, int bk, int64_t n) { return d == 128 && bk == 64 && n * d * 2 < (int64_t(1) << 31); }

void launch_rev_dma(const SweepArgs& a, const LamArgs& lam, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(a.pairs * a.chunks));
    hipLaunchKernelGGL(k_rev_dma, grid, dim3(64 * NW), 0, s, a, lam);
}

}  // namespace la
