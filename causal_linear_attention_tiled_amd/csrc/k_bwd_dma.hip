// Reverse (dK, dV) sweep, Bk = 64, D = 128, bf16, fed by direct
// global-to-LDS loads.
//
// Same arithmetic as the register-staged reverse kernel (the backward half
// of Lightning Attention-2's tiling, Tiling paragraph): blocks from last to
// first, carrying dS = sum_{i >= end of block} lam^(i - end) q_i dO_i^T,
//     dK_b = ((dO_b V_b^T) o M)^T Q_b + diag(lam^(m-s)) V_b dS^T
//     dV_b = ((Q_b K_b^T) o M)^T dO_b + diag(lam^(m-s)) K_b dS
//     dS  <- lam^m dS + (diag(lam^s) Q_b)^T dO_b.
// A gradient F arriving at the final state is the last chunk's starting dS, with the
// exponents of the sequence's last block lowered by one (it reaches token j as
// lam^(N-1-j) F); chunk 0 ends with lam dS, the gradient of the initial state.
// The four waves stream the raw row-major Q, K, V, dO tiles of the next block
// (in sweep order) into the second of two LDS stages while they compute the
// current one (each block starts with vmcnt(0), so loads and stores may share
// the counter in any order); every operand whose contraction runs over
// tokens (dO^T, Q^T, the decayed Q) is read from the row-major tiles with the
// transposing LDS read in the kappa k order, and every operand contracted
// over features is a single 16-byte row read in the natural order (lds_dma.h).  Wave w keeps dS[:, 32w..32w+32) and
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
constexpr int NT = BK / 16;   // 16-token columns j per block
constexpr int NKB = BK / 32;  // 32-token k blocks per block
constexpr int NSTAGE = 2;
constexpr int TILE = BK * D;
constexpr int NW = 4;

constexpr int NCAUSAL = NT * (NT + 1) / 2;  // score tiles (it, jt) with it >= jt

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
            const int chunk = p ^ swz_key(r);
            const int voff = static_cast<int>(((t0 + r) * D + 8 * chunk) * 2);
            dma16(rsrc, &sm.t[stage][wu][4 * rg * D], voff);
        }
    };
    issue(0);

    uint16_t* __restrict__ dKg = static_cast<uint16_t*>(a.out0) + base;
    uint16_t* __restrict__ dVg = static_cast<uint16_t*>(a.out1) + base;
    // dS entering this chunk from the right (0 for the last chunk), in two tile sets
    // over the interleaved rows rho (lds_dma.h):
    //   Sv[at][h][r] = dS  [32 (at/2) + rho(at%2, 4g + r)][32 w + 16 h + li]   (value columns)
    //   Sk[at][h][r] = dS^T[32 (at/2) + rho(at%2, 4g + r)][32 w + 16 h + li]   (key rows)
    f32x4 Sv[8][2], Sk[8][2];
    {
        const float* init = (c < a.chunks - 1) ? a.slots + rev_slot_index(a, pair, c) * D * D
                                               : (a.g_final ? a.g_final + pair * D * D : nullptr);
#pragma unroll
        for (int at = 0; at < 8; ++at)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int row0 = 32 * (at >> 1) + rho(at & 1, 4 * g);
                const int col = 32 * w + 16 * h + li;
                f32x4 x = zero4(), y = zero4();
                if (init) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) x[r] = init[(row0 + r) * D + col];
                    const float4 t4 = *reinterpret_cast<const float4*>(init + col * D + row0);
                    y = f32x4{t4.x, t4.y, t4.z, t4.w};
                }
                Sv[at][h] = x;
                Sk[at][h] = y;
            }
    }
    // lam^s weights of the dS update for s = 32 kb + kappa(g, e) (rows past m are zero)
    float wq[NKB][8];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e) wq[kb][e] = 0.f;

    for (int64_t i = 0; i < nblk; ++i) {
        const int64_t n = nblk - 1 - i;
        const int64_t t0 = t_begin + n * BK;
        const int m = static_cast<int>(min(static_cast<int64_t>(BK), t_end - t0));
        const int stage = static_cast<int>(i % NSTAGE);
        // the final-state gradient reaches the sequence's last block one power less decayed
        const int shift = (c == a.chunks - 1 && a.g_final && i == 0) ? 1 : 0;
        const uint16_t* Qs = sm.t[stage][0];
        const uint16_t* Ks = sm.t[stage][1];
        const uint16_t* Vs = sm.t[stage][2];
        const uint16_t* Gs = sm.t[stage][3];
        // Only this block's loads (and earlier stores) are outstanding here.
        wait_vmcnt<0>();
        __syncthreads();  // A(i): stage i % 2 is ready; stage (i+1) % 2 is no longer read
        // Next block's loads: untracked by the compiler (inline asm), so no later
        // barrier or LDS read waits for them; the next A waits with vmcnt(0).
        if (i + 1 < nblk) issue(i + 1);
        if (i == 0) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int e = 0; e < 8; ++e) wq[kb][e] = sm.pw[32 * kb + kappa(g, e)];
        }

        // ---- shared score tiles: P = Q K^T and G = dO V^T; tile (it, jt), it >= jt, holds
        // X[i][j] for i = 16 it + 4 g + r, j = 16 jt + li, kept iff i >= j and scaled by lam^(i - j)
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
                        x[r] *= masked_pw(sm.pw, d, d >= 0);
                    }
                    uint32_t* dst = which ? sm.gg : sm.p;
                    *reinterpret_cast<u32x2*>(&dst[idx * 128 + 2 * lane]) = u32x2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
                }
        __syncthreads();  // B(i)

        // ---- per 16-token column jt: dV^T (value columns 32w..) and dK^T (key rows 32w..)
        bf16x8 gtf[2][NKB], qtf[2][NKB];  // dO[32 kb + kappa(g, e)][32w + 16h + li], Q[...][...]
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                gtf[h][kb] = op_tr_k(Gs, 32 * kb, 32 * w + 16 * h, 4, g, li);
                qtf[h][kb] = op_tr_k(Qs, 32 * kb, 32 * w + 16 * h, 4, g, li);
            }
#pragma unroll
        for (int jt = 0; jt < NT; ++jt) {
            const int j = 16 * jt + li;
            const float lj = masked_pw(sm.pw, m - shift - j, j < m);
            f32x4 dv[2], dk[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) dv[h] = dk[h] = zero4();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const bf16x8 kr = op_row(Ks, j, 32 * kb, g);
                const bf16x8 vr = op_row(Vs, j, 32 * kb, g);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    dv[h] = mfma16(operand_from_acc(Sv[2 * kb][h], Sv[2 * kb + 1][h]), kr, dv[h]);
                    dk[h] = mfma16(operand_from_acc(Sk[2 * kb][h], Sk[2 * kb + 1][h]), vr, dk[h]);
                }
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                dv[h] *= lj;
                dk[h] *= lj;
            }
#pragma unroll
            for (int kb = jt / 2; kb < NKB; ++kb) {
                const int i0 = 2 * kb, i1 = 2 * kb + 1;
                const u32x2 z{0, 0};
                const u32x2 plo = (i0 >= jt) ? ld_frag(sm.p, i0 * (i0 + 1) / 2 + jt, lane) : z;
                const u32x2 phi = (i1 >= jt) ? ld_frag(sm.p, i1 * (i1 + 1) / 2 + jt, lane) : z;
                const u32x2 glo = (i0 >= jt) ? ld_frag(sm.gg, i0 * (i0 + 1) / 2 + jt, lane) : z;
                const u32x2 ghi = (i1 >= jt) ? ld_frag(sm.gg, i1 * (i1 + 1) / 2 + jt, lane) : z;
                const bf16x8 pb = operand(plo, phi), gb = operand(glo, ghi);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    dv[h] = mfma16(gtf[h][kb], pb, dv[h]);
                    dk[h] = mfma16(qtf[h][kb], gb, dk[h]);
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

        // ---- dS <- lam^m dS + Q^T diag(lam^s) dO, both copies; the weights go on this wave's
        // own fragments (dO columns for the value copy, Q columns for the key copy)
        const float lm = sm.pw[m - shift];
        bf16x8 qs[2][NKB], gs[2][NKB];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                qs[h][kb] = scale8(qtf[h][kb], wq[kb]);
                gs[h][kb] = scale8(gtf[h][kb], wq[kb]);
            }
#pragma unroll
        for (int at = 0; at < 8; ++at) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                Sv[at][h] *= lm;
                Sk[at][h] *= lm;
            }
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                // Q^T / dO^T rows 32 (at/2) + rho(at%2, li), k index s = 32 kb + kappa(g, e)
                const bf16x8 qa = op_tr_k(Qs, 32 * kb, 32 * (at >> 1) + 4 * (at & 1), 8, g, li);
                const bf16x8 ga = op_tr_k(Gs, 32 * kb, 32 * (at >> 1) + 4 * (at & 1), 8, g, li);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    Sv[at][h] = mfma16(qa, gs[h][kb], Sv[at][h]);
                    Sk[at][h] = mfma16(ga, qs[h][kb], Sk[at][h]);
                }
            }
        }
    }
    if (c == 0 && a.ds_out) {
        // gradient of the initial state: lam dS, from the value-column copy
        float* dst = a.ds_out + pair * D * D;
#pragma unroll
        for (int at = 0; at < 8; ++at)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dst[(32 * (at >> 1) + rho(at & 1, 4 * g + r)) * D + 32 * w + 16 * h + li] = lv * Sv[at][h][r];
    }
}


// Eight-wave form: the value group (waves 0-3) keeps dS[:, 32 q .. 32 q + 32)
// and produces dV for those value columns, the key group (waves 4-7) keeps
// dS^T[:, 32 q .. 32 q + 32) and produces dK for those key rows (q = w mod 4).
// Each wave holds 64 accumulator registers instead of 128, so two waves share
// every SIMD and one hides the other's LDS and MFMA latency.  The value group
// builds the P tiles, the key group the G tiles.  dK and dV rows leave as
// 16-byte stores (a 16-lane swap pairs a lane's two 4-column pieces), which
// also drain sooner before the next block's vmcnt(0).
template <bool PHI>
__global__ __launch_bounds__(64 * 8, 1) void k_rev_dma_split(SweepArgs a, LamArgs lam) {
    __shared__ RevDmaTiles sm;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, li = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = w >> 2, q = w & 3;
    const int64_t pair = blockIdx.x / a.chunks;
    const int c = blockIdx.x % a.chunks;
    const float lv = lam.lam[pair % a.H];
    const int64_t t_begin = static_cast<int64_t>(c) * a.L;
    const int64_t t_end = min(a.N, t_begin + a.L);
    const int64_t nblk = (t_end - t_begin + BK - 1) / BK;
    const int64_t base = pair * a.N * D;

    for (int e = tid; e <= BK; e += 64 * 8) sm.pw[e] = lam_pow(lv, e);

    // DMA: wave w streams rows 32 (w & 1) .. + 32 of tensor w / 2 (Q, K, V, dO)
    // of the i-th block of the sweep into stage i % 2, 8 loads of 1 KiB.
    const int ten = w >> 1, half = w & 1;
    const void* src = ten == 0 ? a.a : ten == 1 ? a.b : ten == 2 ? a.c : a.g;
    const u32x4 rsrc = buffer_rsrc(static_cast<const uint16_t*>(src) + base, static_cast<uint32_t>(a.N * D * 2));
    auto issue = [&](int64_t i) {
        const int stage = static_cast<int>(i % NSTAGE);
        const int64_t t0 = t_begin + (nblk - 1 - i) * BK;
        const int sub = lane >> 4, p = lane & 15;
#pragma unroll
        for (int rg = 0; rg < BK / 8; ++rg) {
            const int r = 32 * half + 4 * rg + sub;
            const int chunk = p ^ swz_key(r);
            const int voff = static_cast<int>(((t0 + r) * D + 8 * chunk) * 2);
            dma16(rsrc, &sm.t[stage][ten][(32 * half + 4 * rg) * D], voff);
        }
    };
    issue(0);

    uint16_t* __restrict__ outg = static_cast<uint16_t*>(grp ? a.out0 : a.out1) + base;
    // The group's copy over the interleaved rows rho (lds_dma.h):
    //   S[at][h][r] = X[32 (at/2) + rho(at%2, 4g + r)][32 q + 16 h + li],  X = dS (value group)
    //   or dS^T (key group), entering this chunk from the right (0 for the last chunk).
    f32x4 S[8][2];
    {
        const float* init = (c < a.chunks - 1) ? a.slots + rev_slot_index(a, pair, c) * D * D
                                               : (a.g_final ? a.g_final + pair * D * D : nullptr);
#pragma unroll
        for (int at = 0; at < 8; ++at)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int row0 = 32 * (at >> 1) + rho(at & 1, 4 * g);
                const int col = 32 * q + 16 * h + li;
                f32x4 x = zero4();
                if (init) {
                    if (grp) {
                        const float4 t4 = *reinterpret_cast<const float4*>(init + col * D + row0);
                        x = f32x4{t4.x, t4.y, t4.z, t4.w};
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) x[r] = init[(row0 + r) * D + col];
                    }
                }
                S[at][h] = x;
            }
    }
    float wq[NKB][8];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e) wq[kb][e] = 0.f;

    for (int64_t i = 0; i < nblk; ++i) {
        const int64_t n = nblk - 1 - i;
        const int64_t t0 = t_begin + n * BK;
        const int m = static_cast<int>(min(static_cast<int64_t>(BK), t_end - t0));
        const int stage = static_cast<int>(i % NSTAGE);
        // the final-state gradient reaches the sequence's last block one power less decayed
        const int shift = (c == a.chunks - 1 && a.g_final && i == 0) ? 1 : 0;
        // value group: rows K, tiles P, token-contracted operand dO, update operand Q^T
        // key group:   rows V, tiles G, token-contracted operand Q,  update operand dO^T
        const uint16_t* Xs = sm.t[stage][grp ? 3 : 0];  // score tile A rows (Q or dO)
        const uint16_t* Rs = sm.t[stage][grp ? 2 : 1];  // score tile B rows and inter rows (K or V)
        const uint16_t* Ts = sm.t[stage][grp ? 0 : 3];  // intra A operand / update B (dO or Q)
        uint32_t* tiles = grp ? sm.gg : sm.p;
        wait_vmcnt<0>();
        __syncthreads();  // A(i)
        if (i + 1 < nblk) issue(i + 1);
        if constexpr (PHI) {
            // the feature map on this block's query and key tiles, once, in place
            phi_tile(sm.t[stage][0], a.phi, tid, 64 * 8);
            phi_tile(sm.t[stage][1], a.phi, tid, 64 * 8);
            __syncthreads();  // T(i)
        }
        if (i == 0) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int e = 0; e < 8; ++e) wq[kb][e] = sm.pw[32 * kb + kappa(g, e)];
        }

        // ---- this group's score tiles (it, jt), it >= jt: X[i][j] for i = 16 it + 4 g + r,
        // j = 16 jt + li, kept iff i >= j and scaled by lam^(i - j)
#pragma unroll
        for (int it = 0; it < NT; ++it)
#pragma unroll
            for (int jt = 0; jt <= it; ++jt) {
                const int idx = it * (it + 1) / 2 + jt;
                if (idx % 4 != q) continue;
                f32x4 x = zero4();
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    x = mfma16(op_row(Xs, 16 * it + li, 32 * ks, g), op_row(Rs, 16 * jt + li, 32 * ks, g), x);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int d = 16 * (it - jt) + 4 * g + r - li;
                    x[r] *= masked_pw(sm.pw, d, d >= 0);
                }
                *reinterpret_cast<u32x2*>(&tiles[idx * 128 + 2 * lane]) = u32x2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
            }

        // the group's state as operands, and the token-contracted operand of its columns
        bf16x8 sop[NKB * 2][2], tf[2][NKB];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int h = 0; h < 2; ++h) sop[kb][h] = operand_from_acc(S[2 * kb][h], S[2 * kb + 1][h]);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) tf[h][kb] = op_tr_k(Ts, 32 * kb, 32 * q + 16 * h, 4, g, li);
        __syncthreads();  // B(i)

#pragma unroll
        for (int jt = 0; jt < NT; ++jt) {
            const int j = 16 * jt + li;
            const float lj = masked_pw(sm.pw, m - shift - j, j < m);
            f32x4 acc[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) acc[h] = zero4();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const bf16x8 rr = op_row(Rs, j, 32 * kb, g);
#pragma unroll
                for (int h = 0; h < 2; ++h) acc[h] = mfma16(sop[kb][h], rr, acc[h]);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) acc[h] *= lj;
#pragma unroll
            for (int kb = jt / 2; kb < NKB; ++kb) {
                const int i0 = 2 * kb, i1 = 2 * kb + 1;
                const u32x2 z{0, 0};
                const u32x2 lo = (i0 >= jt) ? ld_frag(tiles, i0 * (i0 + 1) / 2 + jt, lane) : z;
                const u32x2 hi = (i1 >= jt) ? ld_frag(tiles, i1 * (i1 + 1) / 2 + jt, lane) : z;
                const bf16x8 tb = operand(lo, hi);
#pragma unroll
                for (int h = 0; h < 2; ++h) acc[h] = mfma16(tf[h][kb], tb, acc[h]);
            }
            // acc[h][r] = dV (value group) or dK (key group) [j][32 q + 16 h + 4 g + r]
            u32x2 pk[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (PHI && grp) {
                    // dK with respect to the raw keys: phi'(k) from the mapped key tile
                    const u32x2 kp = *reinterpret_cast<const u32x2*>(sm.t[stage][1] + swz(j, 32 * q + 16 * h + 4 * g));
                    acc[h][0] *= dphi_of_phi(__uint_as_float(kp.x << 16), a.phi);
                    acc[h][1] *= dphi_of_phi(__uint_as_float(kp.x & 0xFFFF0000u), a.phi);
                    acc[h][2] *= dphi_of_phi(__uint_as_float(kp.y << 16), a.phi);
                    acc[h][3] *= dphi_of_phi(__uint_as_float(kp.y & 0xFFFF0000u), a.phi);
                }
                pk[h] = u32x2{pack_bf16(acc[h][0], acc[h][1]), pack_bf16(acc[h][2], acc[h][3])};
            }
            {
                // 16-byte stores, as in the forward kernel: after swapping the odd 16-lane rows
                // of tile 0's words with the even rows of tile 1's, row group g holds the 8
                // consecutive columns 8 gs .. 8 gs + 7 of the wave's 32, gs = 0, 2, 1, 3
                const auto x = __builtin_amdgcn_permlane16_swap(pk[0].x, pk[1].x, false, false);
                const auto y = __builtin_amdgcn_permlane16_swap(pk[0].y, pk[1].y, false, false);
                const int gs = (g & 1) * 2 + (g >> 1);
                if (j < m)
                    *reinterpret_cast<u32x4*>(outg + (t0 + j) * D + 32 * q + 8 * gs) = u32x4{x[0], y[0], x[1], y[1]};
            }
        }

        // ---- X <- lam^m X + U^T diag(lam^s) T, U = Q (value group) or dO (key group)
        const float lm = sm.pw[m - shift];
        bf16x8 ts[2][NKB];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) ts[h][kb] = scale8(tf[h][kb], wq[kb]);
#pragma unroll
        for (int at = 0; at < 8; ++at) {
#pragma unroll
            for (int h = 0; h < 2; ++h) S[at][h] *= lm;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                // U^T rows 32 (at/2) + rho(at%2, li), k index s = 32 kb + kappa(g, e)
                const bf16x8 ua = op_tr_k(Xs, 32 * kb, 32 * (at >> 1) + 4 * (at & 1), 8, g, li);
#pragma unroll
                for (int h = 0; h < 2; ++h) S[at][h] = mfma16(ua, ts[h][kb], S[at][h]);
            }
        }
    }
    if (c == 0 && a.ds_out && grp == 0) {
        // gradient of the initial state: lam dS, from the value group's copy
        float* dst = a.ds_out + pair * D * D;
#pragma unroll
        for (int at = 0; at < 8; ++at)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dst[(32 * (at >> 1) + rho(at & 1, 4 * g + r)) * D + 32 * q + 16 * h + li] = lv * S[at][h][r];
    }
}

}  // namespace

// Bk = 128 runs its blocks as two 64-token halves (the dK, dV of a 128-token block need its
// four operand tiles twice over, more than LDS holds): the same function, with the
// second half's contribution to the first carried through dS instead of a score tile.
bool rev_dma_supported(int d, int bk, int64_t n) {
    return d == 128 && (bk == 64 || bk == 128) && n * d * 2 < (int64_t(1) << 31);
}

void launch_rev_dma(const SweepArgs& a, const LamArgs& lam, int waves, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(a.pairs * a.chunks));
    if (waves == 8 && a.phi)
        hipLaunchKernelGGL(k_rev_dma_split<true>, grid, dim3(64 * 8), 0, s, a, lam);
    else if (waves == 8)
        hipLaunchKernelGGL(k_rev_dma_split<false>, grid, dim3(64 * 8), 0, s, a, lam);
    else
        hipLaunchKernelGGL(k_rev_dma, grid, dim3(64 * NW), 0, s, a, lam);
}

}  // namespace la
