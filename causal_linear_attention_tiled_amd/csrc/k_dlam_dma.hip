// The decay-derivative sweep (bf16, D = 128, Bk = 64) on direct-to-LDS loads.
//
// Same computation as the sweep of k_dlam.hip (the tiling of Lightning
// Attention-2, Tiling paragraph, with every power of lam replaced by its
// derivative, carrying the state S and T = dS/dlam), laid out like the forward
// kernel (k_fwd_dma.hip):
//   - one loader wave streams the raw row-major Q, K, V, dO tiles of the next
//     block into a two-stage LDS ring with buffer_load_dwordx4 ... lds while the
//     current block computes (it never stores, so vmcnt(0) waits exactly for the
//     block it hands over);
//   - NW compute waves (4 or 8), wave w owning value columns [128w/NW, 128(w+1)/NW) of S and T
//     in MFMA accumulators (the forward kernel's interleaved-row layout);
//   - per block: the causal 16x16 tiles of P^T = K Q^T and G^T = V dO^T, shared
//     out over the waves, multiplied elementwise with the derivative mask
//     (s-s') lam^(s-s'-1) and summed; the inter-block terms as the elementwise
//     products of S and T with Q^T diag(w) dO under the row weights (s+1) lam^s
//     and lam^(s+1); then
//     T <- lam^m T + m lam^(m-1) S + K^T diag((m-1-s) lam^(m-2-s)) V and
//     S <- lam^m S + K^T diag(lam^(m-1-s)) V.
// The loader wave takes part in the final reduction, so every wave passes every
// barrier.
#include "la_device.h"
#include "la_internal.h"
#include "lds_dma.h"
#include "mfma_common.h"

namespace la {
namespace {

constexpr int D = 128;
constexpr int BK = 64;
constexpr int NT = BK / 16;
constexpr int NKB = BK / 32;
constexpr int NSTAGE = 2;
constexpr int TILE = BK * D;
constexpr int kMaxWaves = 8;

struct DlamTiles {
    uint16_t t[NSTAGE][4][TILE];  // per stage: Q, K, V, dO (row-major, swizzled)
    float pw[BK + 2];
    float dpw[BK + 2];
    // token weights by token s of an m-token block, zero for s >= m: (s+1) lam^s,
    // lam^(s+1), lam^(m-1-s), (m-1-s) lam^(m-2-s); set 0 for full blocks, set 1 for
    // the workgroup's last block.  A lane reads its 8 as two 16-byte runs.
    alignas(16) float wtab[2][4][BK];
    double red[kMaxWaves + 1];
};

// NW compute waves (4 or 8), each owning 128 / NW value columns.
template <int NW, bool PHI>
__global__ __launch_bounds__(64 * (NW + 1), 1) void k_dlam_dma(DlamArgs a, LamArgs lam) {
    constexpr int NVT = 8 / NW;  // 16-column value tiles per compute wave
    __shared__ DlamTiles sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, li = lane & 15;
    const int64_t pair = blockIdx.x / a.chunks;
    const int c = blockIdx.x % a.chunks;
    const float lv = lam.lam[pair % a.H];
    const int64_t t_begin = static_cast<int64_t>(c) * a.L;
    const int64_t t_end = min(a.N, t_begin + a.L);
    const int64_t nblk = (t_end - t_begin + BK - 1) / BK;
    const int64_t base = pair * a.N * D;

    for (int e = tid; e <= BK + 1; e += 64 * (NW + 1)) {
        sm.pw[e] = lam_pow(lv, e);
        sm.dpw[e] = lam_dpow(lv, e);
    }
    const int m_last = nblk > 0 ? static_cast<int>(t_end - t_begin - (nblk - 1) * BK) : BK;
    for (int i = tid; i < 2 * BK; i += 64 * (NW + 1)) {
        const int set = i / BK, e = i % BK, m = set ? m_last : BK;
        const bool in = e < m;
        sm.wtab[set][0][e] = in ? lam_dpow(lv, e + 1) : 0.f;
        sm.wtab[set][1][e] = in ? lam_pow(lv, e + 1) : 0.f;
        sm.wtab[set][2][e] = in ? lam_pow(lv, m - 1 - e) : 0.f;
        sm.wtab[set][3][e] = in ? lam_dpow(lv, m - 1 - e) : 0.f;
    }
    __syncthreads();  // tables; then every wave passes (2 + [phi]) barriers per block and one more

    double acc = 0.0;
    if (w == NW) {
        // ------------------------------------------------------------ loader wave
        const uint32_t bytes = static_cast<uint32_t>(a.N * D * 2);  // rows past the end read zero
        const u32x4 rs[4] = {buffer_rsrc(static_cast<const uint16_t*>(a.q) + base, bytes),
                             buffer_rsrc(static_cast<const uint16_t*>(a.k) + base, bytes),
                             buffer_rsrc(static_cast<const uint16_t*>(a.v) + base, bytes),
                             buffer_rsrc(static_cast<const uint16_t*>(a.g) + base, bytes)};
        const int sub = lane >> 4, p = lane & 15;
        auto issue = [&](int64_t n) {
            const int stage = static_cast<int>(n % NSTAGE);
            const int64_t t0 = t_begin + n * BK;
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int rg = 0; rg < BK / 4; ++rg) {
                    const int r = 4 * rg + sub;
                    const int voff = static_cast<int>(((t0 + r) * D + 8 * (p ^ swz_key(r))) * 2);
                    dma16(rs[x], &sm.t[stage][x][4 * rg * D], voff);
                }
        };
        if (nblk > 0) issue(0);
        for (int64_t n = 0; n < nblk; ++n) {
            wait_vmcnt<0>();                // block n has landed (the only loads in flight)
            __builtin_amdgcn_s_barrier();   // A(n); stage (n + 1) % 2 was last read in block n - 1
            if (n + 1 < nblk) issue(n + 1);
            if constexpr (PHI) __builtin_amdgcn_s_barrier();  // T(n)
            __builtin_amdgcn_s_barrier();   // B(n)
        }
    } else {
        // ------------------------------------------------------------ compute waves
        // S[at][vt][r] = S[32 (at/2) + rho(at%2, 4g + r)][16 (NVT w + vt) + li], T alike
        f32x4 S[8][NVT], T[8][NVT];
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
                for (int vt = 0; vt < NVT; ++vt) {
                    const int col = 16 * (NVT * w + vt) + li;
                    const int row0 = 32 * (at >> 1) + rho(at & 1, 4 * g);
                    f32x4 xs = zero4(), xt = zero4();
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (s_src) xs[r] = s_src[(row0 + r) * D + col];
                        if (t_src) xt[r] = t_src[(row0 + r) * D + col];
                    }
                    S[at][vt] = xs;
                    T[at][vt] = xt;
                }
        }

        for (int64_t n = 0; n < nblk; ++n) {
            const int64_t t0 = t_begin + n * BK;
            const int m = static_cast<int>(min(static_cast<int64_t>(BK), t_end - t0));
            const int stage = static_cast<int>(n % NSTAGE);
            __syncthreads();  // A(n)
            if constexpr (PHI) {
                phi_tile(sm.t[stage][0], a.phi, tid, 64 * NW);
                phi_tile(sm.t[stage][1], a.phi, tid, 64 * NW);
                __syncthreads();  // T(n)
            }
            const uint16_t* Qs = sm.t[stage][0];
            const uint16_t* Ks = sm.t[stage][1];
            const uint16_t* Vs = sm.t[stage][2];
            const uint16_t* Gs = sm.t[stage][3];
            const float (*wset)[BK] = sm.wtab[n == nblk - 1 ? 1 : 0];
            float part = 0.f;

            // ---- intra: tile (at, st) holds [s' = 16 at + 4 g + r][s = 16 st + li] of P^T and G^T
#pragma unroll
            for (int st = 0; st < NT; ++st)
#pragma unroll
                for (int at = 0; at <= st; ++at) {
                    const int idx = st * (st + 1) / 2 + at;
                    if (idx % NW != w) continue;
                    f32x4 pp = zero4(), gg = zero4();
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        pp = mfma16(op_row(Ks, 16 * at + li, 32 * ks, g), op_row(Qs, 16 * st + li, 32 * ks, g), pp);
                        gg = mfma16(op_row(Vs, 16 * at + li, 32 * ks, g), op_row(Gs, 16 * st + li, 32 * ks, g), gg);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int e = 16 * (st - at) + li - 4 * g - r;
                        part += masked_pw(sm.dpw, e, e > 0) * pp[r] * gg[r];
                    }
                }

            // ---- inter: the term sum_s w_s q_s X dO_s^T is the elementwise product of X with
            //      M = Q^T diag(w) dO, for X = S (w_s = (s+1) lam^s) and X = T (lam^(s+1)).  M is
            //      built on the matrix cores from the bf16 tiles, in the accumulators' own layout
            //      (Q read as the state update reads K), so the state itself never passes through
            //      bf16.  T grows like (t+1) S0 and the summed ages of the keys at lam near 1,
            //      large next to the result, so the weighted dO it meets also carries its
            //      rounding residual, as a second operand.
            {
                bf16x8 gs[NKB][NVT], gt[NKB][NVT], gr[NKB][NVT];
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const f32x4 ws0 = lane_weights(wset[0], kb, g, 0), ws1 = lane_weights(wset[0], kb, g, 1);
                    const f32x4 wt0 = lane_weights(wset[1], kb, g, 0), wt1 = lane_weights(wset[1], kb, g, 1);
                    const float ws[8] = {ws0[0], ws0[1], ws0[2], ws0[3], ws1[0], ws1[1], ws1[2], ws1[3]};
                    const float wt[8] = {wt0[0], wt0[1], wt0[2], wt0[3], wt1[0], wt1[1], wt1[2], wt1[3]};
#pragma unroll
                    for (int vt = 0; vt < NVT; ++vt) {
                        const bf16x8 gf = op_tr_k(Gs, 32 * kb, 16 * (NVT * w + vt), 4, g, li);
                        gs[kb][vt] = scale8(gf, ws);
                        scale8_split(gf, wt, gt[kb][vt], gr[kb][vt]);
                    }
                }
#pragma unroll
                for (int at = 0; at < 8; ++at) {
                    f32x4 ms[NVT], mt[NVT];
#pragma unroll
                    for (int vt = 0; vt < NVT; ++vt) ms[vt] = mt[vt] = zero4();
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) {
                        const bf16x8 qf = op_tr_k(Qs, 32 * kb, 32 * (at >> 1) + 4 * (at & 1), 8, g, li);
#pragma unroll
                        for (int vt = 0; vt < NVT; ++vt) {
                            ms[vt] = mfma16(qf, gs[kb][vt], ms[vt]);
                            mt[vt] = mfma16(qf, gt[kb][vt], mt[vt]);
                            mt[vt] = mfma16(qf, gr[kb][vt], mt[vt]);
                        }
                    }
#pragma unroll
                    for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
                        for (int r = 0; r < 4; ++r) part += S[at][vt][r] * ms[vt][r] + T[at][vt][r] * mt[vt][r];
                }
            }
            acc += static_cast<double>(part);

            // ---- T <- lam^m T + m lam^(m-1) S + K^T diag(dpw[m-1-s]) V,  S <- lam^m S + K^T diag(pw[m-1-s]) V
            {
                const float lm = sm.pw[m], dlm = sm.dpw[m];
#pragma unroll
                for (int at = 0; at < 8; ++at)
#pragma unroll
                    for (int vt = 0; vt < NVT; ++vt) {
                        T[at][vt] = lm * T[at][vt] + dlm * S[at][vt];
                        S[at][vt] *= lm;
                    }
                // one 32-token k block at a time; every accumulator adds k block 0 before 1
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const f32x4 wk0 = lane_weights(wset[2], kb, g, 0), wk1 = lane_weights(wset[2], kb, g, 1);
                    const f32x4 wd0 = lane_weights(wset[3], kb, g, 0), wd1 = lane_weights(wset[3], kb, g, 1);
                    const float wk[8] = {wk0[0], wk0[1], wk0[2], wk0[3], wk1[0], wk1[1], wk1[2], wk1[3]};
                    const float wd[8] = {wd0[0], wd0[1], wd0[2], wd0[3], wd1[0], wd1[1], wd1[2], wd1[3]};
                    // both weighted operands as bf16 pairs (hi + rounding residual): their single
                    // roundings, carried block after block in S and T, are what is left of the
                    // error where the result cancels by orders of magnitude
                    bf16x8 vw[NVT], vwr[NVT], vd[NVT], vdr[NVT];
#pragma unroll
                    for (int vt = 0; vt < NVT; ++vt) {
                        const bf16x8 vf = op_tr_k(Vs, 32 * kb, 16 * (NVT * w + vt), 4, g, li);
                        scale8_split(vf, wk, vw[vt], vwr[vt]);
                        scale8_split(vf, wd, vd[vt], vdr[vt]);
                    }
#pragma unroll
                    for (int at = 0; at < 8; ++at) {
                        const bf16x8 kf = op_tr_k(Ks, 32 * kb, 32 * (at >> 1) + 4 * (at & 1), 8, g, li);
#pragma unroll
                        for (int vt = 0; vt < NVT; ++vt) {
                            S[at][vt] = mfma16(kf, vw[vt], S[at][vt]);
                            T[at][vt] = mfma16(kf, vd[vt], T[at][vt]);
                            S[at][vt] = mfma16(kf, vwr[vt], S[at][vt]);
                            T[at][vt] = mfma16(kf, vdr[vt], T[at][vt]);
                        }
                    }
                }
            }
            __syncthreads();  // B(n)
        }

        if (a.g_final && c == a.chunks - 1) {
            const float* F = a.g_final + pair * D * D;
            float part = 0.f;
#pragma unroll
            for (int at = 0; at < 8; ++at)
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        part += F[(32 * (at >> 1) + rho(at & 1, 4 * g + r)) * D + 16 * (NVT * w + vt) + li] * T[at][vt][r];
            acc += static_cast<double>(part);
        }
    }

#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (lane == 0) sm.red[w] = acc;
    __syncthreads();
    if (tid == 0) {
        double tot = 0.0;
#pragma unroll
        for (int i = 0; i <= NW; ++i) tot += sm.red[i];
        a.partial[pair * a.chunks + c] = tot;
    }
}

}  // namespace

// Bk = 128 runs its blocks as two 64-token halves, as the dK, dV sweep does.
bool dlam_dma_supported(int d, int bk, int64_t n) {
    return d == D && (bk == BK || bk == 2 * BK) && n * d * 2 < (int64_t(1) << 31);
}

void launch_dlam_dma(const DlamArgs& a, const LamArgs& lam, int waves, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(a.pairs * a.chunks));
    if (waves == 8) {
        if (a.phi)
            hipLaunchKernelGGL((k_dlam_dma<8, true>), grid, dim3(64 * 9), 0, s, a, lam);
        else
            hipLaunchKernelGGL((k_dlam_dma<8, false>), grid, dim3(64 * 9), 0, s, a, lam);
    } else {
        if (a.phi)
            hipLaunchKernelGGL((k_dlam_dma<4, true>), grid, dim3(64 * 5), 0, s, a, lam);
        else
            hipLaunchKernelGGL((k_dlam_dma<4, false>), grid, dim3(64 * 5), 0, s, a, lam);
    }
}

}  // namespace la
