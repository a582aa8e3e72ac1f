// Forward sweep with 128-token blocks (bf16, D = 128, Bk = 128) on direct-to-LDS loads.
//
// Lightning Attention-2 (Tiling paragraph; record mechanism field), per block b of
// m <= 128 tokens with local index s:
//     O_b     = diag(lam^(s+1)) Q_b S_b + ((Q_b K_b^T) o M) V_b,   M[s][s'] = lam^(s-s') (s >= s')
//     S_{b+1} = lam^m S_b + K_b^T diag(lam^(m-1-s)) V_b.
// Three 128-token stages of Q, K, V would take 288 KiB of LDS, so the ring holds
// 64-token half blocks (three half stages of 48 KiB, the stage of the 64-token
// kernel in k_fwd_dma.hip) and a block is computed in two phases over its halves
// h0 = [0, 64) and h1 = [64, 128):
//   phase 1: O rows of h0 = diag(lam^(s+1)) Q_h0 S_b + A_00 V_h0 (10 causal score tiles);
//   phase 2: O rows of h1 = diag(lam^(64+s+1)) Q_h1 S_b + A_10 V_h0 + A_11 V_h1, where
//            A_10 (16 full tiles, decay lam^(64+s-s')) is the part of the block's score
//            matrix that pairs h1's queries with h0's keys, and A_11 is causal;
//   then the state update over all m tokens.
// The score tiles of one phase (at most 26, 13 KiB) are shared through LDS as in the
// 64-token kernel; everything else (loader wave with exact vmcnt waits, swizzled
// tiles, transposing reads, state in accumulators over interleaved rows, transposed
// outputs) is that kernel's.  Loads: half 2b+2 is issued when block b starts; the
// queries and values of half 2b+3 when phase 1 of block b ends (h0's values are held in
// registers from then on), its keys when block b ends (h0's keys feed the state
// update), so the first half of every block is a block ahead and most of the second
// half a phase ahead.
#include "la_device.h"
#include "la_internal.h"
#include "lds_dma.h"
#include "mfma_common.h"

namespace la {
namespace {

constexpr int D = 128;
constexpr int HB = 64;                     // tokens per half block (one ring stage)
constexpr int BK = 2 * HB;                 // tokens per block
constexpr int NT = HB / 16;                // 16-token output columns per half
constexpr int NKB = HB / 32;               // 32-token k blocks per half
constexpr int NSTAGE = 3;                  // half stages
constexpr int TILE = HB * D;
constexpr int DMA_PER_HALF = 3 * HB / 4;   // 1 KiB loads per half block
constexpr int NW = 4;                      // compute waves
constexpr int NVT = 8 / NW;                // 16-column value tiles per compute wave
constexpr int NDIAG = NT * (NT + 1) / 2;   // causal tiles of one half against itself
constexpr int NCROSS = NT * NT;            // tiles of h1's queries against h0's keys

struct Dma128Tiles {
    uint16_t t[NSTAGE][3][TILE];           // per half stage: Q, K, V (row-major, swizzled)
    uint32_t at[(NCROSS + NDIAG) * 128];   // one phase's score tiles (B-operand fragments)
    float pw[BK + 1];
};

template <bool PHI>
__global__ __launch_bounds__(64 * (NW + 1), 1) void k_fwd_dma128(SweepArgs a, LamArgs lam) {
    __shared__ Dma128Tiles sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, li = lane & 15;
    const Work wk = work_item<false>(a, static_cast<const VarlenArgs*>(nullptr), blockIdx.x);
    const int c = wk.c;
    const float lv = lam.lam[wk.head];
    const int64_t t_begin = wk.t_begin, t_end = wk.t_end;
    const int64_t nblk = (t_end - t_begin + BK - 1) / BK;
    const int64_t nhalf = 2 * nblk;  // both halves of every block are loaded (past the end: zero)
    const int64_t base = wk.base;
    constexpr int64_t ld = D;

    for (int e = tid; e <= BK; e += 64 * (NW + 1)) sm.pw[e] = lam_pow(lv, e);
    __syncthreads();  // decay table; every wave passes exactly (5 + 2 [phi]) barriers per block

    if (w == NW) {
        // ------------------------------------------------------------ loader wave
        const int bytes = wk.n > 0 ? static_cast<int>(((wk.n - 1) * ld + D) * 2) : 0;
        __amdgpu_buffer_rsrc_t rs[3];
        rs[0] = __builtin_amdgcn_make_buffer_rsrc((void*)(static_cast<const uint16_t*>(a.a) + base), 0, bytes, 0x00020000);
        rs[1] = __builtin_amdgcn_make_buffer_rsrc((void*)(static_cast<const uint16_t*>(a.b) + base), 0, bytes, 0x00020000);
        rs[2] = __builtin_amdgcn_make_buffer_rsrc((void*)(static_cast<const uint16_t*>(a.c) + base), 0, bytes, 0x00020000);
        const int sub = lane >> 4, p = lane & 15;
        // the tensors in `mask` (bit 0: Q, 1: K, 2: V) of half h, into ring stage h % 3
        auto issue = [&](int64_t h, int mask) {
            const int stage = static_cast<int>(h % NSTAGE);
            const int64_t t0 = t_begin + h * HB;
#pragma unroll
            for (int x = 0; x < 3; ++x)
                if (mask & (1 << x))
#pragma unroll
                for (int rg = 0; rg < HB / 4; ++rg) {
                    const int r = 4 * rg + sub;
                    const int chunk = p ^ swz_key(r);
                    const int voff = static_cast<int>(((t0 + r) * ld + 8 * chunk) * 2);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs[x], (lds_void*)&sm.t[stage][x][4 * rg * D], 16, voff, 0, 0, 0);
                }
        };
        // Issue points: at A1(b) all of half 2b+2 (its stage held h1 of block b-1); at A2(b)
        // the queries and values of half 2b+3 (they replace h0's: phase 2 reads no queries of
        // h0 and takes h0's values from registers); at B(b) the keys of half 2b+3 (h0's keys
        // are read until the state update).  In issue order the loads are 48, 32, 16 per
        // block, so at A1 and at A2 all but the last 48 loads in flight are the ones needed.
        if (nhalf > 0) {
            issue(0, 7);
            issue(1, 7);
        }
        for (int64_t b = 0; b < nblk; ++b) {
            wait_vmcnt<DMA_PER_HALF>();    // half 2b has landed
            __builtin_amdgcn_s_barrier();  // A1(b)
            const bool more = 2 * b + 2 < nhalf;
            if (more) issue(2 * b + 2, 7);
            if constexpr (PHI) __builtin_amdgcn_s_barrier();  // T1(b)
            __builtin_amdgcn_s_barrier();  // S1(b)
            if (more)
                wait_vmcnt<DMA_PER_HALF>();  // half 2b+1 has landed
            else
                wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();  // A2(b)
            if (more) issue(2 * b + 3, 5);
            if constexpr (PHI) __builtin_amdgcn_s_barrier();  // T2(b)
            __builtin_amdgcn_s_barrier();  // S2(b)
            __builtin_amdgcn_s_barrier();  // B(b)
            if (more) issue(2 * b + 3, 2);
        }
        return;
    }

    // ---------------------------------------------------------------- compute waves
    uint16_t* __restrict__ Og = static_cast<uint16_t*>(a.out0) + base;
    // S[at][vt][r] = S[32 (at/2) + rho(at%2, 4g + r)][16 (NVT w + vt) + li]
    f32x4 S[8][NVT];
    {
        const float* init = nullptr;
        bool tr = false, poison = false;
        if (c == 0) {
            if (a.kv_in) {
                init = a.kv_in + wk.state * D * D;
                tr = a.kv_in_transposed != 0;
            }
        } else {
            init = a.slots + (wk.slot0 + static_cast<int64_t>(c - 1) * wk.slot_step) * D * D;
            tr = a.slots_transposed != 0;
            poison = !given_states_match(a);
        }
#pragma unroll
        for (int at = 0; at < 8; ++at)
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) {
                const int col = 16 * (NVT * w + vt) + li;
                const int row0 = 32 * (at >> 1) + rho(at & 1, 4 * g);
                f32x4 x = zero4();
                if (init) {
                    if (tr) {
                        const float4 t4 = *reinterpret_cast<const float4*>(init + col * D + row0);
                        x = f32x4{t4.x, t4.y, t4.z, t4.w};
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) x[r] = init[(row0 + r) * D + col];
                    }
                }
                if (poison) x = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
                S[at][vt] = x;
            }
    }

    // score tile (at, st) of a half against itself, at <= st: A^T[s'][s], s' = 16 at + 4 g + r,
    // s = 16 st + li, kept iff s' <= s, scaled by lam^(s - s'); of h1's queries against h0's
    // keys: always kept, scaled by lam^(64 + s - s')
    auto score_tile = [&](const uint16_t* Ks, const uint16_t* Qs, int at, int st, int off, bool causal) {
        f32x4 p = zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            p = mfma16(op_row(Ks, 16 * at + li, 32 * ks, g), op_row(Qs, 16 * st + li, 32 * ks, g), p);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d = off + 16 * (st - at) + li - 4 * g - r;
            p[r] *= causal ? masked_pw(sm.pw, d, d >= 0) : sm.pw[d];
        }
        return u32x2{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])};
    };
    // V^T fragments of a half over its tokens (kappa order)
    auto v_frags = [&](const uint16_t* Vs, bf16x8 (&vf)[NVT][NKB]) {
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) vf[vt][kb] = op_tr_k(Vs, 32 * kb, 16 * (NVT * w + vt), 4, g, li);
    };
    // B operand over 32 key tokens from two stacked score tiles
    auto tile_pair = [&](int i0, int i1, bool have1) {
        const u32x2 lo = *reinterpret_cast<const u32x2*>(&sm.at[i0 * 128 + 2 * lane]);
        u32x2 hi = u32x2{0, 0};
        if (have1) hi = *reinterpret_cast<const u32x2*>(&sm.at[i1 * 128 + 2 * lane]);
        return operand(lo, hi);
    };
    // store one 16-token column of outputs (rows h * 64 + 16 st + li of the block)
    auto store = [&](int64_t t0, int m, int h, int st, const f32x4 (&o)[NVT]) {
        const int s = HB * h + 16 * st + li;
        u32x2 pk[NVT];
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) {
            f32x4 ov = o[vt];
            if (PHI && a.phi_grad) {
                // chain rule through the feature map: phi'(raw q) for the dQ sweep (rows past
                // the block's end read its last row and are not stored)
                const int64_t roff = (t0 + min(s, m - 1)) * ld + 16 * (NVT * w + vt) + 4 * g;
                const u32x2 raw = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(a.phi_grad) + base + roff);
                ov[0] *= dphi_of_x(__uint_as_float(raw.x << 16), a.phi);
                ov[1] *= dphi_of_x(__uint_as_float(raw.x & 0xFFFF0000u), a.phi);
                ov[2] *= dphi_of_x(__uint_as_float(raw.y << 16), a.phi);
                ov[3] *= dphi_of_x(__uint_as_float(raw.y & 0xFFFF0000u), a.phi);
            }
            pk[vt] = u32x2{pack_bf16(ov[0], ov[1]), pack_bf16(ov[2], ov[3])};
        }
        if constexpr (NVT == 2) {
            // 16-byte stores: the 16-lane swap of the forward kernel (row group g then holds
            // columns 8 gs .. 8 gs + 7 of the wave's 32, gs = 0, 2, 1, 3); every lane swaps
            const auto x = __builtin_amdgcn_permlane16_swap(pk[0].x, pk[1].x, false, false);
            const auto y = __builtin_amdgcn_permlane16_swap(pk[0].y, pk[1].y, false, false);
            const int gs = (g & 1) * 2 + (g >> 1);
            if (s < m) *reinterpret_cast<u32x4*>(Og + (t0 + s) * ld + 32 * w + 8 * gs) = u32x4{x[0], y[0], x[1], y[1]};
        } else if (s < m) {
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt)
                *reinterpret_cast<u32x2*>(Og + (t0 + s) * ld + 16 * (NVT * w + vt) + 4 * g) = pk[vt];
        }
    };
    // diag(lam^(off + s + 1)) S^T Q_h^T for the column st of a half
    auto inter = [&](const uint16_t* Qs, int st, int off, f32x4 (&o)[NVT]) {
#pragma unroll
        for (int at = 0; at < 8; ++at)
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) asm volatile("" : "+v"(S[at][vt]));
        bf16x8 qf[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) qf[kb] = op_row(Qs, 16 * st + li, 32 * kb, g);
        const float rs = sm.pw[off + 16 * st + li + 1];
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) acc = mfma16(operand_from_acc(S[2 * kb][vt], S[2 * kb + 1][vt]), qf[kb], acc);
            o[vt] = acc * rs;
        }
    };

    for (int64_t b = 0; b < nblk; ++b) {
        const int64_t t0 = t_begin + b * BK;
        const int m = static_cast<int>(min(static_cast<int64_t>(BK), t_end - t0));
        const int s0 = static_cast<int>((2 * b) % NSTAGE), s1 = static_cast<int>((2 * b + 1) % NSTAGE);
        const uint16_t* Q0 = sm.t[s0][0];
        const uint16_t* K0 = sm.t[s0][1];
        const uint16_t* V0 = sm.t[s0][2];
        const uint16_t* Q1 = sm.t[s1][0];
        const uint16_t* K1 = sm.t[s1][1];
        const uint16_t* V1 = sm.t[s1][2];

        // ================= phase 1: rows of h0
        __syncthreads();  // A1(b)
        if constexpr (PHI) {
#pragma unroll
            for (int x = 0; x < 3; ++x)
                if (a.phi_mask & (1 << x)) phi_tile(sm.t[s0][x], a.phi, tid, 64 * NW);
            __syncthreads();  // T1(b)
        }
#pragma unroll
        for (int st = 0; st < NT; ++st)
#pragma unroll
            for (int at = 0; at <= st; ++at) {
                const int idx = st * (st + 1) / 2 + at;
                if (idx % NW != w) continue;
                *reinterpret_cast<u32x2*>(&sm.at[idx * 128 + 2 * lane]) = score_tile(K0, Q0, at, st, 0, true);
            }
        __syncthreads();  // S1(b)
        bf16x8 vf0[NVT][NKB];
        v_frags(V0, vf0);
#pragma unroll
        for (int st = 0; st < NT; ++st) {
            f32x4 o[NVT];
            inter(Q0, st, 0, o);
#pragma unroll
            for (int kb = 0; kb <= st / 2; ++kb) {
                const bf16x8 bop = tile_pair(st * (st + 1) / 2 + 2 * kb, st * (st + 1) / 2 + 2 * kb + 1, 2 * kb + 1 <= st);
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt) o[vt] = mfma16(vf0[vt][kb], bop, o[vt]);
            }
            store(t0, m, 0, st, o);
            __builtin_amdgcn_sched_barrier(0);
        }

        // ================= phase 2: rows of h1
        __syncthreads();  // A2(b): half 2b+1 has landed; phase 1 no longer reads the score tiles
        if constexpr (PHI) {
#pragma unroll
            for (int x = 0; x < 3; ++x)
                if (a.phi_mask & (1 << x)) phi_tile(sm.t[s1][x], a.phi, tid, 64 * NW);
            __syncthreads();  // T2(b)
        }
        // tiles 0..15: h1's queries (st) against h0's keys (at), index 4 st + at;
        // tiles 16..25: h1 against itself, index 16 + st (st + 1) / 2 + at
#pragma unroll
        for (int idx = w; idx < NCROSS + NDIAG; idx += NW) {
            if (idx < NCROSS) {
                *reinterpret_cast<u32x2*>(&sm.at[idx * 128 + 2 * lane]) = score_tile(K0, Q1, idx % 4, idx / 4, HB, false);
            } else {
                const int j = idx - NCROSS;
                const int st = j < 1 ? 0 : j < 3 ? 1 : j < 6 ? 2 : 3;
                const int at = j - st * (st + 1) / 2;
                *reinterpret_cast<u32x2*>(&sm.at[idx * 128 + 2 * lane]) = score_tile(K1, Q1, at, st, 0, true);
            }
        }
        __syncthreads();  // S2(b)
        bf16x8 vf1[NVT][NKB];
        v_frags(V1, vf1);
#pragma unroll
        for (int st = 0; st < NT; ++st) {
            f32x4 o[NVT];
            inter(Q1, st, HB, o);
            // against h0's keys: all 64 of them
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const bf16x8 bop = tile_pair(4 * st + 2 * kb, 4 * st + 2 * kb + 1, true);
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt) o[vt] = mfma16(vf0[vt][kb], bop, o[vt]);
            }
            // against h1's own keys: causal
#pragma unroll
            for (int kb = 0; kb <= st / 2; ++kb) {
                const int i0 = NCROSS + st * (st + 1) / 2 + 2 * kb;
                const bf16x8 bop = tile_pair(i0, i0 + 1, 2 * kb + 1 <= st);
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt) o[vt] = mfma16(vf1[vt][kb], bop, o[vt]);
            }
            store(t0, m, 1, st, o);
            __builtin_amdgcn_sched_barrier(0);
        }

        // ================= S <- lam^m S + K^T diag(lam^(m-1-s)) V over both halves
        const float lm = sm.pw[m];
#pragma unroll
        for (int at = 0; at < 8; ++at)
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) S[at][vt] *= lm;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint16_t* Ks = h ? K1 : K0;
            bf16x8 vw[NVT][NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                float wgt[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int s = HB * h + 32 * kb + kappa(g, e);
                    wgt[e] = masked_pw(sm.pw, m - 1 - s, s < m);
                }
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt) vw[vt][kb] = scale8(h ? vf1[vt][kb] : vf0[vt][kb], wgt);
            }
#pragma unroll
            for (int at = 0; at < 8; ++at)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const bf16x8 kf = op_tr_k(Ks, 32 * kb, 32 * (at >> 1) + 4 * (at & 1), 8, g, li);
#pragma unroll
                    for (int vt = 0; vt < NVT; ++vt) S[at][vt] = mfma16(kf, vw[vt][kb], S[at][vt]);
                }
        }
        __syncthreads();  // B(b): both halves of block b are free
    }

    if (a.kv_out && c == wk.chunks - 1) {
        float* dst = a.kv_out + wk.state * D * D;
#pragma unroll
        for (int at = 0; at < 8; ++at)
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dst[(32 * (at >> 1) + rho(at & 1, 4 * g + r)) * D + 16 * (NVT * w + vt) + li] = S[at][vt][r];
    }
}

}  // namespace

bool fwd_dma128_supported(int d, int bk, int64_t n) {
    // the loader reads up to one half block past the end of the sequence
    return d == D && bk == BK && (n + HB) * d * 2 < (int64_t(1) << 31);
}

void launch_fwd_dma128(const SweepArgs& a, const LamArgs& lam, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(a.pairs * a.chunks));
    if (a.phi)
        hipLaunchKernelGGL(k_fwd_dma128<true>, grid, dim3(64 * (NW + 1)), 0, s, a, lam);
    else
        hipLaunchKernelGGL(k_fwd_dma128<false>, grid, dim3(64 * (NW + 1)), 0, s, a, lam);
}

}  // namespace la
