// Chunk aggregates for the chunked prefix over blocks (bf16, D = 128,
// Bk = 64), fed by direct global-to-LDS loads.
//
// For every chunk c that another chunk depends on, the state update of the
// sweep (Lightning Attention-2, Tiling paragraph: the inter-block part is
// carried by the key-value state) summed over the chunk from zero:
//   forward: acc = sum_t lam^(E - 1 - t) x_t y_t^T   (E = end of the chunk)
//   reverse: acc = sum_t lam^(t - B) x_t y_t^T       (B = start of the chunk)
// with (x, y) = (k, v) for the forward and (q, dO) for the gradient state.
// The blocks are walked away from the reference token (last to first for the
// forward, first to last for the reverse), so every token's weight is
// c * lam^(offset in its block) with c = lam^(tokens already walked), a running
// product in double: the accumulators are never rescaled.  A weight that
// underflows stands for a term below float range next to the unit-size ones.
// The eight waves share the loads (4 of the 32 loads of a block each) over a
// two-stage ring: the next block's loads are issued as a block starts and
// waited for (vmcnt 0; the loop stores nothing) at the next.  The ring takes
// 64 KiB of LDS, so two workgroups share a compute unit and a launch of a few
// hundred chunks runs in one round.  Both operands come from the row-major
// tiles through transposing LDS reads; wave w accumulates columns
// [16w, 16w + 16) of the aggregate.
//
// The decay-derivative form (forward only) also sums dT = d(acc)/dlam =
// sum_t (E - 1 - t) lam^(E - 2 - t) x_t y_t^T.  It walks the blocks first to
// last and rescales instead: per m-token block, (acc, dT) <- (lam^m acc,
// lam^m dT + m lam^(m-1) acc) plus the block's own terms, token s weighing
// lam^(m-1-s) in acc and (m-1-s) lam^(m-2-s) in dT.  Folding a token's whole
// age into one rounded operand weight would give dT a rounding error of its
// own, unrelated to acc's; carried this way, dT stays the derivative of the
// acc that was actually summed, up to the rounding of the small in-block
// weights, which matters where the loss's decay derivative is a sum that
// cancels (lam near 1).  The two slots of a chunk are stored back to back
// (acc, then dT).
#include "la_device.h"
#include "la_internal.h"
#include "lds_dma.h"
#include "mfma_common.h"

namespace la {
namespace {

constexpr int D = 128;
constexpr int BK = 64;
constexpr int NKB = BK / 32;
constexpr int NSTAGE = 2;
constexpr int TILE = BK * D;
constexpr int NW = 8;
constexpr int LOADS_PER_WAVE = 2 * (BK / 4) / NW;  // 1 KiB loads per wave per block

struct StateTiles {
    uint16_t t[NSTAGE][2][TILE];  // per stage: X, Y (row-major, swizzled)
    float pw[BK + 1];
    float dpw[BK + 1];            // d(lam^e)/dlam (decay-derivative form)
};

template <bool VARLEN, bool PHI, bool DL>
__device__ __forceinline__ void state_body(const ChunkStateArgs& a, const LamArgs& lam, const VarlenArgs* var) {
    __shared__ StateTiles sm;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, li = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // this workgroup's chunk: c of (sequence, head), its token range and its slot
    int64_t base, ld, n_seq, dst_slot;
    int c, head;
    if constexpr (!VARLEN) {
        const int per = a.chunks - 1;
        const int64_t pair = blockIdx.x / per;
        const int slot = blockIdx.x % per;
        c = a.reverse ? slot + 1 + a.part0 : slot;
        base = pair * a.N * D;
        ld = D;
        n_seq = a.N;
        head = static_cast<int>(pair % a.H);
        dst_slot = pair * per + slot;
    } else {
        // forward only: slot s (per head) of sequence b with wp[b] - b <= s < wp[b+1] - b - 1
        head = static_cast<int>(blockIdx.x % a.H);
        const int s = static_cast<int>(blockIdx.x / a.H);
        const int b = find_last_le(var->nseq, s, [&](int i) { return var->wp[i] - i; });
        c = s - (var->wp[b] - b);
        base = (static_cast<int64_t>(var->cu[b]) * a.H + head) * D;
        ld = static_cast<int64_t>(a.H) * D;
        n_seq = var->cu[b + 1] - var->cu[b];
        dst_slot = static_cast<int64_t>(s) * a.H + head;
    }
    const int64_t t_begin = static_cast<int64_t>(c) * a.L;
    const int64_t t_end = min(n_seq, t_begin + a.L);
    const int64_t nblk = (t_end - t_begin + BK - 1) / BK;
    const float lv = lam.lam[head];
    for (int e = tid; e <= BK; e += 64 * NW) {
        sm.pw[e] = lam_pow(lv, e);
        if constexpr (DL) sm.dpw[e] = lam_dpow(lv, e);
    }
    const double lam_bk = lam_pow64(lv, BK);

    // loads at or past the sequence's last row come back as zero
    const uint32_t bytes = static_cast<uint32_t>(((n_seq - 1) * ld + D) * 2);
    const u32x4 rx = buffer_rsrc(static_cast<const uint16_t*>(a.x) + base, bytes);
    const u32x4 ry = buffer_rsrc(static_cast<const uint16_t*>(a.y) + base, bytes);
    // The n-th block of the walk goes to stage n % 2; wave w issues, for each
    // tensor, the loads of row groups w and w + 8 (4 rows each).
    auto block_of = [&](int64_t n) { return (a.reverse || DL) ? n : nblk - 1 - n; };
    auto issue = [&](int64_t n) {
        const int64_t t0 = t_begin + block_of(n) * BK;
        const int stage = static_cast<int>(n % NSTAGE);
        const int sub = lane >> 4, p = lane & 15;
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int i = 0; i < LOADS_PER_WAVE / 2; ++i) {
                const int rg = w + NW * i;
                const int r = 4 * rg + sub;
                const int voff = static_cast<int>(((t0 + r) * ld + 8 * (p ^ swz_key(r))) * 2);
                dma16(x == 0 ? rx : ry, &sm.t[stage][x][4 * rg * D], voff);
            }
    };
    if (nblk > 0) issue(0);

    // S[at][r] = acc[16 at + 4 g + r][16 w + li]
    f32x4 S[8], T[DL ? 8 : 1];
#pragma unroll
    for (int at = 0; at < 8; ++at) S[at] = zero4();
    if constexpr (DL) {
#pragma unroll
        for (int at = 0; at < 8; ++at) T[at] = zero4();
    }
    double cw = 1.0;  // lam^(tokens walked so far), for the form without rescaling

    for (int64_t n = 0; n < nblk; ++n) {
        const int64_t t0 = t_begin + block_of(n) * BK;
        const int m = static_cast<int>(min(static_cast<int64_t>(BK), t_end - t0));
        const int stage = static_cast<int>(n % NSTAGE);
        wait_vmcnt<0>();  // this block's loads (the only ones in flight)
        __syncthreads();  // stage n % 2 is complete; stage (n + 1) % 2 is no longer read
        if (n + 1 < nblk) issue(n + 1);
        if constexpr (PHI) {
            // the feature map on this block's keys or queries, once, in place
            if (a.phi_mask & 1) phi_tile(sm.t[stage][0], a.phi, tid, 64 * NW);
            if (a.phi_mask & 2) phi_tile(sm.t[stage][1], a.phi, tid, 64 * NW);
            __syncthreads();
        }
        const uint16_t* Xs = sm.t[stage][0];
        const uint16_t* Ys = sm.t[stage][1];
        // weights of token s = 32 kb + kappa(g, e), on the Y operand
        if constexpr (!DL) {
            const float cf = static_cast<float>(cw);
            float wx[NKB][8];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int s = 32 * kb + kappa(g, e);
                    wx[kb][e] = cf * masked_pw(sm.pw, a.reverse ? s : m - 1 - s, s < m);
                }
            bf16x8 yf[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) yf[kb] = scale8(op_tr_k(Ys, 32 * kb, 16 * w, 4, g, li), wx[kb]);
#pragma unroll
            for (int at = 0; at < 8; ++at)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) S[at] = mfma16(op_tr_k(Xs, 32 * kb, 16 * at, 4, g, li), yf[kb], S[at]);
        } else {
            // the blocks before this one age by m tokens: T first, from the S it had
            const float lmf = sm.pw[m], dlmf = sm.dpw[m];
#pragma unroll
            for (int at = 0; at < 8; ++at)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    T[at][r] = lmf * T[at][r] + dlmf * S[at][r];
                    S[at][r] = lmf * S[at][r];
                }
            // one 32-token k block at a time (fewer live registers); every accumulator still
            // adds k block 0 before k block 1
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                float wx[8], wd[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int s = 32 * kb + kappa(g, e);
                    wx[e] = masked_pw(sm.pw, m - 1 - s, s < m);
                    wd[e] = masked_pw(sm.dpw, m - 1 - s, s < m);
                }
                // the weighted operands as bf16 pairs (hi + rounding residual), as in the sweep
                const bf16x8 y = op_tr_k(Ys, 32 * kb, 16 * w, 4, g, li);
                bf16x8 yf, yfr, yd, ydr;
                scale8_split(y, wx, yf, yfr);
                scale8_split(y, wd, yd, ydr);
#pragma unroll
                for (int at = 0; at < 8; ++at) {
                    const bf16x8 xf = op_tr_k(Xs, 32 * kb, 16 * at, 4, g, li);
                    S[at] = mfma16(xf, yf, S[at]);
                    T[at] = mfma16(xf, yd, T[at]);
                    S[at] = mfma16(xf, yfr, S[at]);
                    T[at] = mfma16(xf, ydr, T[at]);
                }
            }
        }
        if constexpr (!DL) cw *= (m == BK) ? lam_bk : lam_pow64(lv, m);
    }
    float* dst = a.slots + dst_slot * (DL ? 2 : 1) * D * D;
#pragma unroll
    for (int at = 0; at < 8; ++at)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            dst[(16 * at + 4 * g + r) * D + 16 * w + li] = S[at][r];
            if constexpr (DL) dst[D * D + (16 * at + 4 * g + r) * D + 16 * w + li] = T[at][r];
        }
}

template <bool PHI>
__global__ __launch_bounds__(64 * NW, 2) void k_chunk_state_dma(ChunkStateArgs a, LamArgs lam) {
    state_body<false, PHI, false>(a, lam, nullptr);
}

// The same aggregates (forward and reverse, dense [P][N][D] sequences) fed by two loader
// waves, one per tensor, through a ring of LD_NST 64-token stages at one workgroup per
// compute unit: LD_NST - 1 blocks are in flight while one computes, against one in the
// form above, whose ring shares the compute unit between two workgroups.  Each loader
// issues its tensor's 16 loads of 1 KiB per block, so its vmcnt counts at most 16
// (LD_NST - 2) loads past the block it waits for.  Compute waves do what state_body
// does (the same operands, weights and order, so the results are identical).
constexpr int LD_NST = 3;
static_assert(LD_NST == 3, "the loaders' vmcnt waits assume one block in flight past the one awaited");

template <bool PHI>
__global__ __launch_bounds__(64 * (NW + 2), 1) void k_chunk_state_ld(ChunkStateArgs a, LamArgs lam) {
    __shared__ uint16_t ring[LD_NST][2][TILE];
    __shared__ float pw[BK + 1];
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, li = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int per = a.chunks - 1;
    const int64_t pair = blockIdx.x / per;
    const int slot = blockIdx.x % per;
    const int c = a.reverse ? slot + 1 + a.part0 : slot;
    const int64_t base = pair * a.N * D;
    const int64_t t_begin = static_cast<int64_t>(c) * a.L;
    const int64_t t_end = min(a.N, t_begin + a.L);
    const int64_t nblk = t_end > t_begin ? (t_end - t_begin + BK - 1) / BK : 0;
    const float lv = lam.lam[pair % a.H];
    for (int e = tid; e <= BK; e += 64 * (NW + 2)) pw[e] = lam_pow(lv, e);
    __syncthreads();
    // the n-th block of the walk: away from the reference token
    auto block_of = [&](int64_t n) { return a.reverse ? n : nblk - 1 - n; };

    if (w >= NW) {
        // loader wave x streams tensor x (0: X, 1: Y); rows at or past the sequence's end read zero
        const int x = w - NW;
        const uint32_t bytes = static_cast<uint32_t>(a.N * D * 2);
        const u32x4 rs = buffer_rsrc(static_cast<const uint16_t*>(x == 0 ? a.x : a.y) + base, bytes);
        const int sub = lane >> 4, p = lane & 15;
        auto issue = [&](int64_t n) {
            const int64_t t0 = t_begin + block_of(n) * BK;
            uint16_t* dst = ring[n % LD_NST][x];
#pragma unroll
            for (int rg = 0; rg < BK / 4; ++rg) {
                const int r = 4 * rg + sub;
                const int voff = static_cast<int>(((t0 + r) * D + 8 * (p ^ swz_key(r))) * 2);
                dma16(rs, dst + 4 * rg * D, voff);
            }
        };
        for (int64_t n = 0; n < min<int64_t>(LD_NST - 1, nblk); ++n) issue(n);
        for (int64_t n = 0; n < nblk; ++n) {
            // blocks issued after n that may still be in flight: min(LD_NST - 2, nblk - 1 - n)
            if (n + 1 < nblk)
                wait_vmcnt<16 * (LD_NST - 2)>();
            else
                wait_vmcnt<0>();
            __syncthreads();  // A(n): block n landed (both tensors); block n - 1's stage is free
            if (n + LD_NST - 1 < nblk) issue(n + LD_NST - 1);
            if constexpr (PHI) __syncthreads();  // T(n)
        }
        return;
    }

    f32x4 S[8];
#pragma unroll
    for (int at = 0; at < 8; ++at) S[at] = zero4();
    double cw = 1.0;  // lam^(tokens walked so far)
    const double lam_bk = lam_pow64(lv, BK);
    for (int64_t n = 0; n < nblk; ++n) {
        const int64_t t0 = t_begin + block_of(n) * BK;
        const int m = static_cast<int>(min(static_cast<int64_t>(BK), t_end - t0));
        uint16_t* Xs = ring[n % LD_NST][0];
        uint16_t* Ys = ring[n % LD_NST][1];
        __syncthreads();  // A(n)
        if constexpr (PHI) {
            if (a.phi_mask & 1) phi_tile(Xs, a.phi, tid, 64 * NW);
            if (a.phi_mask & 2) phi_tile(Ys, a.phi, tid, 64 * NW);
            __syncthreads();  // T(n)
        }
        const float cf = static_cast<float>(cw);
        float wx[NKB][8];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int s = 32 * kb + kappa(g, e);
                wx[kb][e] = cf * masked_pw(pw, a.reverse ? s : m - 1 - s, s < m);
            }
        bf16x8 yf[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) yf[kb] = scale8(op_tr_k(Ys, 32 * kb, 16 * w, 4, g, li), wx[kb]);
#pragma unroll
        for (int at = 0; at < 8; ++at)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) S[at] = mfma16(op_tr_k(Xs, 32 * kb, 16 * at, 4, g, li), yf[kb], S[at]);
        cw *= (m == BK) ? lam_bk : lam_pow64(lv, m);
    }
    float* dst = a.slots + (pair * per + slot) * D * D;
#pragma unroll
    for (int at = 0; at < 8; ++at)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(16 * at + 4 * g + r) * D + 16 * w + li] = S[at][r];
}

template <bool PHI>
__global__ __launch_bounds__(64 * NW, 2) void k_chunk_state_dma_varlen(ChunkStateArgs a, LamArgs lam, VarlenArgs v) {
    state_body<true, PHI, false>(a, lam, &v);
}

// The decay-derivative form carries S and T with both weighted operands as bf16 pairs:
// 184 registers, so one workgroup per compute unit (no spills).
template <bool PHI>
__global__ __launch_bounds__(64 * NW, 1) void k_dlam_state_dma(ChunkStateArgs a, LamArgs lam) {
    state_body<false, PHI, true>(a, lam, nullptr);
}

}  // namespace

// The aggregate of a chunk does not depend on the block size of the sweep (the chunk
// length is a multiple of it), so any block size that divides into 64-token blocks is served.
bool state_dma_supported(int d, int bk, int64_t n) {
    return d == 128 && (bk == 64 || bk == 128) && n * d * 2 < (int64_t(1) << 31);
}

void launch_chunk_state_dma(const ChunkStateArgs& a, const LamArgs& lam, bool loader_waves, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(a.pairs * (a.chunks - 1)));
    if (loader_waves) {
        if (a.phi)
            hipLaunchKernelGGL(k_chunk_state_ld<true>, grid, dim3(64 * (NW + 2)), 0, s, a, lam);
        else
            hipLaunchKernelGGL(k_chunk_state_ld<false>, grid, dim3(64 * (NW + 2)), 0, s, a, lam);
        return;
    }
    if (a.phi)
        hipLaunchKernelGGL(k_chunk_state_dma<true>, grid, dim3(64 * NW), 0, s, a, lam);
    else
        hipLaunchKernelGGL(k_chunk_state_dma<false>, grid, dim3(64 * NW), 0, s, a, lam);
}

void launch_dlam_state_dma(const ChunkStateArgs& a, const LamArgs& lam, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(a.pairs * (a.chunks - 1)));
    if (a.phi)
        hipLaunchKernelGGL(k_dlam_state_dma<true>, grid, dim3(64 * NW), 0, s, a, lam);
    else
        hipLaunchKernelGGL(k_dlam_state_dma<false>, grid, dim3(64 * NW), 0, s, a, lam);
}

void launch_chunk_state_dma_varlen(const ChunkStateArgs& a, const LamArgs& lam, const VarlenArgs& v,
                                   hipStream_t s) {
    dim3 grid(static_cast<unsigned>(static_cast<int64_t>(v.wp[v.nseq] - v.nseq) * a.H));
    if (a.phi)
        hipLaunchKernelGGL(k_chunk_state_dma_varlen<true>, grid, dim3(64 * NW), 0, s, a, lam, v);
    else
        hipLaunchKernelGGL(k_chunk_state_dma_varlen<false>, grid, dim3(64 * NW), 0, s, a, lam, v);
}

}  // namespace la
