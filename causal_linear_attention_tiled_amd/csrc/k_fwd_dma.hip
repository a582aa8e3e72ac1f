// Forward sweep, Bk = 64, D = 128, bf16: a three-stage LDS pipeline fed by
// direct global-to-LDS loads.
//
// Lightning Attention-2 (Tiling paragraph; record mechanism field): per
// block b with local index s and m tokens,
//     O_b     = diag(lam^(s+1)) Q_b S_b + ((Q_b K_b^T) o M) V_b,
//     M[s][s'] = lam^(s-s') for s >= s', else 0,
//     S_{b+1} = lam^m S_b + K_b^T diag(lam^(m-1-s)) V_b.
//
// Data path:
//   - One extra "loader" wave issues buffer_load_dwordx4 ... lds for the raw
//     row-major Q, K, V tiles of the block two ahead of the one being
//     computed.  It never stores, so its vmcnt waits are exact, and it
//     hands each stage to the compute waves through the block's barriers.
//     Loads past the end of the sequence come back as zero (buffer bounds).
//   - Row-major operands are single 16-byte reads; operands contracted over
//     tokens (V^T, K^T) come from the same tiles through transposing reads
//     (lds_dma.h).
// Compute waves: NW; wave w owns 128/NW value columns of the float32 state
// and of the output, which is computed transposed: O^T = S^T Q^T + V^T A^T,
// with the masked, decayed scores A^T = (K Q^T) o M^T shared through LDS.
// Products contracted over features (K Q^T, S^T Q^T) take the natural k
// order, so their row-major operands are single 16-byte reads; the state
// accumulators are kept as tile pairs over the interleaved rows rho, which
// makes them directly the A operand of S^T Q^T.  Products contracted over
// tokens (V^T A^T and the state update) take the kappa order, whose
// transposing reads touch 16 consecutive rows; the score accumulators are
// then directly the B operand of V^T A^T.  Outputs leave as 16-byte stores:
// a lane's two 4-column pieces of a row (one per value tile) are regrouped by
// a 16-lane swap into 8 consecutive columns (8-byte stores write HBM slower).
#include "la_device.h"
#include "la_internal.h"
#include "lds_dma.h"
#include "mfma_common.h"

namespace la {
namespace {

constexpr int D = 128;
constexpr int BK = 64;
constexpr int NT = BK / 16;                // 16-token output columns per block
constexpr int NKB = BK / 32;               // 32-token k blocks per block
constexpr int NSTAGE = 3;
constexpr int TILE = BK * D;               // elements per tile
constexpr int DMA_PER_BLOCK = 3 * BK / 4;  // 1 KiB loads per block (4 rows of 256 B each)

constexpr int NCAUSAL = NT * (NT + 1) / 2;   // score tiles (at, st) with at <= st

struct DmaTiles {
    uint16_t t[NSTAGE][3][TILE];     // per stage: Q, K, V (row-major, swizzled)
    uint32_t at[NCAUSAL * 128];      // masked decayed score tiles, B-operand fragments
    float pw[BK + 1];
    // state-update weights by token s, lam^(m-1-s) (zero for s >= m): set 0 for full
    // blocks, set 1 for the workgroup's last block; read as 16-byte runs
    alignas(16) float wk[2][BK];
};

// FUSED: the chunked prefix in the same launch.  A workgroup whose chunk is not the last
// first walks its chunk's K and V (phase 1: the state update from zero, loads of K and V
// only) and publishes that chunk aggregate, per compute wave (each wave owns its value
// columns), followed by a flag holding the call's epoch; then (phase 2) each wave waits for
// the same wave of every earlier chunk of its sequence and sums their aggregates into its
// starting state, S = lam^(cL) S0 + sum_j lam^((c-1-j)L) dS_j, stores it where la_fwd
// keeps the states entering chunks, and sweeps its chunk (phase 3).  A workgroup waits only
// on lower workgroup indices, which the hardware dispatches first, so every awaited
// workgroup is running or done; the wait is bounded all the same (a.spin_limit polls),
// and a wave that gives up starts from NaN instead of hanging.
// The aggregates and flags travel as agent-scope atomic stores and loads, which the
// hardware keeps coherent across the XCDs' separate L2 caches line by line.  A wave raises
// its flag only after its aggregate stores have completed (vmcnt 0), and a waiting wave
// issues its aggregate loads only after it has read the flag, so the loads see the stores.
// Agent-scope release/acquire fences would give the same order through a write-back and an
// invalidate of the whole L2, which cost more than the two launches this form saves.

template <int NW, bool VARLEN, bool PHI, bool FUSED = false>
__device__ __forceinline__ void fwd_body(const SweepArgs& a, const LamArgs& lam, const VarlenArgs* var) {
    constexpr int NVT = 8 / NW;  // 16-column value tiles per compute wave
    static_assert(!FUSED || (!VARLEN && NW == 4), "the fused prefix is for dense sequences, 4 compute waves");
    __shared__ DmaTiles sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, li = lane & 15;
    const Work wk = work_item<VARLEN>(a, var, blockIdx.x);
    const int c = wk.c;
    const float lv = lam.lam[wk.head];
    const int64_t t_begin = wk.t_begin, t_end = wk.t_end;
    const int64_t nblk = (t_end - t_begin + BK - 1) / BK;
    const int64_t base = wk.base;
    const int64_t ld = VARLEN ? wk.ld : D;  // elements between token rows
    // FUSED: blocks 0 .. nblk1 - 1 walk the chunk for its aggregate (every chunk but the last
    // is whole), blocks nblk1 .. ntot - 1 sweep it
    const int64_t nblk1 = (FUSED && c < wk.chunks - 1) ? nblk : 0;
    const int64_t ntot = nblk1 + nblk;
    const int64_t pair = wk.state;

    for (int e = tid; e <= BK; e += 64 * (NW + 1)) sm.pw[e] = lam_pow(lv, e);
    const int m_last = nblk > 0 ? static_cast<int>(t_end - t_begin - (nblk - 1) * BK) : BK;
    for (int i = tid; i < 2 * BK; i += 64 * (NW + 1)) {
        const int e = i % BK, m = i < BK ? BK : m_last;
        sm.wk[i / BK][e] = e < m ? lam_pow(lv, m - 1 - e) : 0.f;
    }
    __syncthreads();  // decay table; every wave passes exactly 1 + (2 + [phi]) * nblk barriers

    if (w == NW) {
        // ------------------------------------------------------------ loader wave
        // loads at or past the sequence's last row come back as zero
        const int bytes = wk.n > 0 ? static_cast<int>(((wk.n - 1) * ld + D) * 2) : 0;
        __amdgpu_buffer_rsrc_t rs[3];
        rs[0] = __builtin_amdgcn_make_buffer_rsrc((void*)(static_cast<const uint16_t*>(a.a) + base), 0, bytes, 0x00020000);
        rs[1] = __builtin_amdgcn_make_buffer_rsrc((void*)(static_cast<const uint16_t*>(a.b) + base), 0, bytes, 0x00020000);
        rs[2] = __builtin_amdgcn_make_buffer_rsrc((void*)(static_cast<const uint16_t*>(a.c) + base), 0, bytes, 0x00020000);
        const int sub = lane >> 4, p = lane & 15;
        auto issue = [&](int64_t n) {
            const int stage = static_cast<int>(n % NSTAGE);
            const bool walk = FUSED && n < nblk1;  // phase 1: K and V only
            const int64_t t0 = t_begin + (walk ? n : n - nblk1) * BK;
#pragma unroll
            for (int x = 0; x < 3; ++x)
                if (!(walk && x == 0))
#pragma unroll
                for (int rg = 0; rg < BK / 4; ++rg) {
                    const int r = 4 * rg + sub;
                    const int chunk = p ^ swz_key(r);
                    const int voff = static_cast<int>(((t0 + r) * ld + 8 * chunk) * 2);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs[x], (lds_void*)&sm.t[stage][x][4 * rg * D], 16, voff, 0, 0, 0);
                }
        };
        if (ntot > 0) issue(0);
        if (ntot > 1) issue(1);
        // The loader's own vmcnt wait makes its LDS writes complete before it
        // reaches A(n); a fenced __syncthreads() here would also wait for the
        // loads still in flight, so the loader uses the bare barrier.
        for (int64_t n = 0; n < ntot; ++n) {
            // block n + 1 may still be in flight: 2/3 of a block's loads in phase 1
            if (n + 1 < ntot) {
                if (FUSED && n + 1 < nblk1)
                    wait_vmcnt<2 * BK / 4>();
                else
                    wait_vmcnt<DMA_PER_BLOCK>();
            } else {
                wait_vmcnt<0>();
            }
            __builtin_amdgcn_s_barrier();  // A(n): stage n is ready; stage (n+2) % 3 is free
            if (n + 2 < ntot) issue(n + 2);
            if constexpr (PHI) __builtin_amdgcn_s_barrier();  // T(n): feature map applied
            __builtin_amdgcn_s_barrier();  // B(n)
        }
        return;
    }

    // ---------------------------------------------------------------- compute waves
    uint16_t* __restrict__ Og = static_cast<uint16_t*>(a.out0) + base;
    // S[at][vt][r] = S[32 (at/2) + rho(at%2, 4g + r)][16 (NVT w + vt) + li]
    f32x4 S[8][NVT];
    if constexpr (FUSED) {
#pragma unroll
        for (int at = 0; at < 8; ++at)
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) S[at][vt] = zero4();
    } else {
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

    float rs[NT];
#pragma unroll
    for (int st = 0; st < NT; ++st) rs[st] = sm.pw[16 * st + li + 1];

    if constexpr (FUSED) {
        // ---- phase 1: S <- lam^64 S + K^T diag(lam^(63-s)) V over the (whole) chunk, from zero
        for (int64_t nn = 0; nn < nblk1; ++nn) {
            const int stage = static_cast<int>(nn % NSTAGE);
            const uint16_t* Ks = sm.t[stage][1];
            const uint16_t* Vs = sm.t[stage][2];
            __syncthreads();  // A(nn)
            if constexpr (PHI) {
#pragma unroll
                for (int x = 1; x < 3; ++x)
                    if (a.phi_mask & (1 << x)) phi_tile(sm.t[stage][x], a.phi, tid, 64 * NW);
                __syncthreads();  // T(nn)
            }
            __syncthreads();  // B(nn)
            const float lm = sm.pw[BK];
            const f32x4 w00 = lane_weights(sm.wk[0], 0, g, 0), w01 = lane_weights(sm.wk[0], 0, g, 1);
            const f32x4 w10 = lane_weights(sm.wk[0], 1, g, 0), w11 = lane_weights(sm.wk[0], 1, g, 1);
            const float wkb[NKB][8] = {{w00[0], w00[1], w00[2], w00[3], w01[0], w01[1], w01[2], w01[3]},
                                       {w10[0], w10[1], w10[2], w10[3], w11[0], w11[1], w11[2], w11[3]}};
            bf16x8 vw[NVT][NKB];
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
                    vw[vt][kb] = scale8(op_tr_k(Vs, 32 * kb, 16 * (NVT * w + vt), 4, g, li), wkb[kb]);
#pragma unroll
            for (int at = 0; at < 8; ++at) {
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt) S[at][vt] *= lm;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const bf16x8 kf = op_tr_k(Ks, 32 * kb, 32 * (at >> 1) + 4 * (at & 1), 8, g, li);
#pragma unroll
                    for (int vt = 0; vt < NVT; ++vt) S[at][vt] = mfma16(kf, vw[vt][kb], S[at][vt]);
                }
            }
        }
        if (nblk1 > 0) {
            // publish this wave's columns of the chunk aggregate, then its flag
            float* agg = a.fused_aggs + (pair * (wk.chunks - 1) + c) * D * D;
#pragma unroll
            for (int at = 0; at < 8; ++at)
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        __hip_atomic_store(agg + (32 * (at >> 1) + rho(at & 1, 4 * g + r)) * D + 16 * (NVT * w + vt) + li,
                                           S[at][vt][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            // the flag goes out only once every one of those stores has completed
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            wait_vmcnt<0>();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if (lane == 0)
                __hip_atomic_store(a.fused_flags + (pair * (wk.chunks - 1) + c) * NW + w, a.epoch,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }

        // ---- phase 2: the state entering this chunk, this wave's columns, Horner over the
        //      earlier chunks: S = lam^L (... (lam^L S0 + dS_0) ...) + dS_(c-1)
        const float* s0 = a.kv_in ? a.kv_in + pair * D * D : nullptr;
        const float lamL = lam_pow(lv, a.L);
#pragma unroll
        for (int at = 0; at < 8; ++at)
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) {
                const int col = 16 * (NVT * w + vt) + li;
                const int row0 = 32 * (at >> 1) + rho(at & 1, 4 * g);
                f32x4 x = zero4();
                if (s0) {
                    if (a.kv_in_transposed) {
                        const float4 t4 = *reinterpret_cast<const float4*>(s0 + col * D + row0);
                        x = f32x4{t4.x, t4.y, t4.z, t4.w};
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) x[r] = s0[(row0 + r) * D + col];
                    }
                }
                S[at][vt] = x;
            }
        bool ok = true;
        for (int j = 0; j < c; ++j) {
            // wait (bounded) for wave w of chunk j, which was dispatched before this workgroup
            const uint64_t* flag = a.fused_flags + (pair * (wk.chunks - 1) + j) * NW + w;
            int spins = 0;
            while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != a.wait_epoch) {
                if (++spins >= a.spin_limit) {
                    ok = false;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
            if (!ok) break;  // no further waits: this wave's columns become NaN
            __atomic_signal_fence(__ATOMIC_SEQ_CST);  // the loads below stay after the flag's
            const float* agg = a.fused_aggs + (pair * (wk.chunks - 1) + j) * D * D;
#pragma unroll
            for (int at = 0; at < 8; ++at)
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt) {
                    const int col = 16 * (NVT * w + vt) + li;
                    const int row0 = 32 * (at >> 1) + rho(at & 1, 4 * g);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        S[at][vt][r] = lamL * S[at][vt][r] +
                                       __hip_atomic_load(agg + (row0 + r) * D + col, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
        }
        if (!ok) {
#pragma unroll
            for (int at = 0; at < 8; ++at)
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt)
                    S[at][vt] = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
        }
        if (c > 0 && a.slots) {
            // where the three-launch form keeps the states entering chunks (la_bwd's fwd_ws)
            float* dst = const_cast<float*>(a.slots) + (wk.slot0 + static_cast<int64_t>(c - 1) * wk.slot_step) * D * D;
#pragma unroll
            for (int at = 0; at < 8; ++at)
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        dst[(32 * (at >> 1) + rho(at & 1, 4 * g + r)) * D + 16 * (NVT * w + vt) + li] = S[at][vt][r];
        }
        if (a.stamp_store && pair == 0 && c == 0 && w == 0 && lane == 0)
            for (int i = 0; i < kStampWords; ++i) a.stamp_store[i] = a.expect.w[i];
    }

    for (int64_t n = 0; n < nblk; ++n) {
        const int64_t nn = n + nblk1;  // the ring counts phase 1's blocks too
        const int stage = static_cast<int>(nn % NSTAGE);
        const uint16_t* Qs = sm.t[stage][0];
        const uint16_t* Ks = sm.t[stage][1];
        const uint16_t* Vs = sm.t[stage][2];
        const int64_t t0 = t_begin + n * BK;
        const int m = static_cast<int>(min(static_cast<int64_t>(BK), t_end - t0));
        __syncthreads();  // A(nn)
        if constexpr (PHI) {
            // the feature map on this block's query and key tiles (in the dQ sweep: the keys,
            // which sit in the value slot), once, in place
#pragma unroll
            for (int x = 0; x < 3; ++x)
                if (a.phi_mask & (1 << x)) phi_tile(sm.t[stage][x], a.phi, tid, 64 * NW);
            __syncthreads();  // T(n)
        }

        // ---- score tiles A^T = (K Q^T) o M^T: tile (at, st), at <= st, holds A^T[s'][s] for
        // s' = 16 at + 4 g + r, s = 16 st + li; kept iff s' <= s, scaled by lam^(s - s').
#pragma unroll
        for (int st = 0; st < NT; ++st)
#pragma unroll
            for (int at = 0; at <= st; ++at) {
                const int idx = st * (st + 1) / 2 + at;
                if (idx % NW != w) continue;
                f32x4 p = zero4();
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    p = mfma16(op_row(Ks, 16 * at + li, 32 * ks, g), op_row(Qs, 16 * st + li, 32 * ks, g), p);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int d = 16 * (st - at) + li - 4 * g - r;
                    p[r] *= masked_pw(sm.pw, d, d >= 0);
                }
                *reinterpret_cast<u32x2*>(&sm.at[idx * 128 + 2 * lane]) = u32x2{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])};
            }
        __syncthreads();  // B(n)

        // ---- V^T fragments over tokens (kappa order): A operand of V^T A^T; weighted by
        // lam^(m-1-s), the B operand of the state update
        bf16x8 vf[NVT][NKB];
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) vf[vt][kb] = op_tr_k(Vs, 32 * kb, 16 * (NVT * w + vt), 4, g, li);

        // raw queries of this block's output rows, for phi'(q) in the dQ sweep: loaded now, used
        // at the stores (rows past the block's end read its last row and are not stored)
        u32x2 qraw[PHI ? NT : 1][NVT];
        if constexpr (PHI) {
            if (a.phi_grad) {
#pragma unroll
                for (int st = 0; st < NT; ++st)
#pragma unroll
                    for (int vt = 0; vt < NVT; ++vt) {
                        const int64_t off = (t0 + min(16 * st + li, m - 1)) * ld + 16 * (NVT * w + vt) + 4 * g;
                        qraw[st][vt] = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(a.phi_grad) + base + off);
                    }
            }
        }

        // ---- per 16-token column: O^T = diag(lam^(s+1)) S^T Q^T + V^T A^T, store
        // the bf16 state operands, converted once per block
        bf16x8 sb[NVT][4];
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) sb[vt][kb] = operand_from_acc(S[2 * kb][vt], S[2 * kb + 1][vt]);
#pragma unroll
        for (int st = 0; st < NT; ++st) {
            bf16x8 qf[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) qf[kb] = op_row(Qs, 16 * st + li, 32 * kb, g);
            f32x4 o[NVT];
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) {
                f32x4 acc = zero4();
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) acc = mfma16(sb[vt][kb], qf[kb], acc);
                o[vt] = acc * rs[st];
            }
#pragma unroll
            for (int kb = 0; kb <= st / 2; ++kb) {
                const int a0 = 2 * kb, a1 = 2 * kb + 1;
                const u32x2 lo = *reinterpret_cast<const u32x2*>(&sm.at[(st * (st + 1) / 2 + a0) * 128 + 2 * lane]);
                u32x2 hi = u32x2{0, 0};
                if (a1 <= st) hi = *reinterpret_cast<const u32x2*>(&sm.at[(st * (st + 1) / 2 + a1) * 128 + 2 * lane]);
                const bf16x8 b = operand(lo, hi);
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt) o[vt] = mfma16(vf[vt][kb], b, o[vt]);
            }
            // o[vt][r] = O[16 st + li][16 (NVT w + vt) + 4 g + r]
            const int s = 16 * st + li;
            u32x2 pk[NVT];
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) {
                f32x4 ov = o[vt];
                if (PHI && a.phi_grad) {
                    // chain rule through the feature map: phi'(raw q) for the dQ sweep
                    const u32x2 raw = qraw[PHI ? st : 0][vt];
                    ov[0] *= dphi_of_x(__uint_as_float(raw.x << 16), a.phi);
                    ov[1] *= dphi_of_x(__uint_as_float(raw.x & 0xFFFF0000u), a.phi);
                    ov[2] *= dphi_of_x(__uint_as_float(raw.y << 16), a.phi);
                    ov[3] *= dphi_of_x(__uint_as_float(raw.y & 0xFFFF0000u), a.phi);
                }
                pk[vt] = u32x2{pack_bf16(ov[0], ov[1]), pack_bf16(ov[2], ov[3])};
            }
            if constexpr (NVT == 2) {
                // 16-byte stores (8-byte ones write HBM ~20% slower): swap the odd 16-lane rows
                // of the first tile's words with the even rows of the second's, which leaves
                // row group g holding 8 consecutive columns 8 gs .. 8 gs + 7 of the wave's 32,
                // gs = 0, 2, 1, 3 for g = 0..3 (all lanes take part; the store is masked)
                const auto x = __builtin_amdgcn_permlane16_swap(pk[0].x, pk[1].x, false, false);
                const auto y = __builtin_amdgcn_permlane16_swap(pk[0].y, pk[1].y, false, false);
                const int gs = (g & 1) * 2 + (g >> 1);
                if (s < m)
                    *reinterpret_cast<u32x4*>(Og + (t0 + s) * ld + 32 * w + 8 * gs) = u32x4{x[0], y[0], x[1], y[1]};
            } else if (s < m) {
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt)
                    *reinterpret_cast<u32x2*>(Og + (t0 + s) * ld + 16 * (NVT * w + vt) + 4 * g) = pk[vt];
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- S <- lam^m S + K^T diag(lam^(m-1-s)) V
        const float lm = sm.pw[m];
        bf16x8 vw[NVT][NKB];
        const float* wtab = sm.wk[n == nblk - 1 ? 1 : 0];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const f32x4 w0 = lane_weights(wtab, kb, g, 0), w1 = lane_weights(wtab, kb, g, 1);
            const float wk[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) vw[vt][kb] = scale8(vf[vt][kb], wk);
        }
#pragma unroll
        for (int at = 0; at < 8; ++at) {
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) S[at][vt] *= lm;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                // K^T[32 (at/2) + rho(at%2, li)][32 kb + kappa(g, e)]
                const bf16x8 kf = op_tr_k(Ks, 32 * kb, 32 * (at >> 1) + 4 * (at & 1), 8, g, li);
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt) S[at][vt] = mfma16(kf, vw[vt][kb], S[at][vt]);
            }
        }
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

template <int NW, bool PHI>
__global__ __launch_bounds__(64 * (NW + 1), 1) void k_fwd_dma(SweepArgs a, LamArgs lam) {
    fwd_body<NW, false, PHI>(a, lam, nullptr);
}

template <bool PHI>
__global__ __launch_bounds__(64 * 5, 1) void k_fwd_dma_fused(SweepArgs a, LamArgs lam) {
    fwd_body<4, false, PHI, true>(a, lam, nullptr);
}

template <bool PHI>
__global__ __launch_bounds__(64 * 5, 1) void k_fwd_dma_varlen(SweepArgs a, LamArgs lam, VarlenArgs v) {
    fwd_body<4, true, PHI>(a, lam, &v);
}

}  // namespace

bool fwd_dma_supported(int d, int bk, int64_t n) {
    return d == 128 && bk == 64 && n * d * 2 < (int64_t(1) << 31);
}

void launch_fwd_dma_varlen(const SweepArgs& a, const LamArgs& lam, const VarlenArgs& v, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(static_cast<int64_t>(v.wp[v.nseq]) * a.H));
    if (a.phi)
        hipLaunchKernelGGL(k_fwd_dma_varlen<true>, grid, dim3(64 * 5), 0, s, a, lam, v);
    else
        hipLaunchKernelGGL(k_fwd_dma_varlen<false>, grid, dim3(64 * 5), 0, s, a, lam, v);
}

void launch_fwd_dma(const SweepArgs& a, const LamArgs& lam, int waves, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(a.pairs * a.chunks));
    if (a.fused_flags) {
        if (a.phi)
            hipLaunchKernelGGL(k_fwd_dma_fused<true>, grid, dim3(64 * 5), 0, s, a, lam);
        else
            hipLaunchKernelGGL(k_fwd_dma_fused<false>, grid, dim3(64 * 5), 0, s, a, lam);
        return;
    }
    if (waves == 8) {
        if (a.phi)
            hipLaunchKernelGGL((k_fwd_dma<8, true>), grid, dim3(64 * 9), 0, s, a, lam);
        else
            hipLaunchKernelGGL((k_fwd_dma<8, false>), grid, dim3(64 * 9), 0, s, a, lam);
    } else {
        if (a.phi)
            hipLaunchKernelGGL((k_fwd_dma<4, true>), grid, dim3(64 * 5), 0, s, a, lam);
        else
            hipLaunchKernelGGL((k_fwd_dma<4, false>), grid, dim3(64 * 5), 0, s, a, lam);
    }
}

}  // namespace la
