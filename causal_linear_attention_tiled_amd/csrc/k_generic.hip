// Generic kernels: every shape the library accepts (D <= 128, Bk <= 128,
// float32 or bfloat16 storage), plain float32 arithmetic, no matrix cores.
// They follow the block decomposition of Lightning Attention-2 (Tiling
// paragraph: intra-block part as ordinary masked attention, inter-block part
// through the carried key-value state) and serve as the path for shapes the
// MFMA kernels do not cover, and for float32 storage.
//
// One workgroup handles one (sequence, chunk).  The D x D float32 state and
// one Bk x Bk score tile live in LDS; operands are read from global memory
// (through the caches) as they are needed.
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int kMaxD = 128;
constexpr int kMaxBk = 128;

struct Tile {
    float state[kMaxD * kMaxD];  // running state, [D][D]
    float score[kMaxBk * kMaxBk];  // masked, decayed scores of one block, [Bk][Bk]
    float pw[kMaxBk + 1];        // lam^e, e = 0..Bk
};

__device__ __forceinline__ void fill_powers(float* pw, float lam, int Bk) {
    for (int e = threadIdx.x; e <= Bk; e += kThreads) pw[e] = lam_pow(lam, e);
}

// Forward sweep over one chunk:
//   O_b = diag(lam^(s+1)) Q_b S + (Q_b K_b^T o M) V_b,  S <- lam^m S + (diag(lam^(m-1-s)) K_b)^T V_b
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_fwd_generic(SweepArgs a, LamArgs lam) {
    __shared__ Tile sh;
    const int64_t pair = blockIdx.x / a.chunks;
    const int c = blockIdx.x % a.chunks;
    const int D = a.D, Bk = a.Bk, tid = threadIdx.x;
    const float lv = lam.lam[pair % a.H];
    const int64_t t_begin = static_cast<int64_t>(c) * a.L;
    const int64_t t_end = min(a.N, t_begin + a.L);
    const int64_t base = pair * a.N * D;
    // operand x of slot bit (0: a, 1: b, 2: c), through the feature map when that slot takes it
    auto opd = [&](const void* p, int bit, int64_t i) {
        const float x = ld<BF16>(p, i);
        return (a.phi && ((a.phi_mask >> bit) & 1)) ? phi_apply(x, a.phi) : x;
    };
    fill_powers(sh.pw, lv, Bk);

    const float* init = nullptr;
    bool transposed = false;
    if (c == 0) {
        if (a.kv_in) {
            init = a.kv_in + pair * D * D;
            transposed = a.kv_in_transposed != 0;
        }
    } else {
        init = a.slots + fwd_slot_index(a, pair, c) * D * D;
        transposed = a.slots_transposed != 0;
    }
    for (int i = tid; i < D * D; i += kThreads) {
        float x = 0.f;
        if (init) x = transposed ? init[(i % D) * D + i / D] : init[i];
        sh.state[i] = x;
    }
    __syncthreads();

    for (int64_t t0 = t_begin; t0 < t_end; t0 += Bk) {
        const int m = static_cast<int>(min(static_cast<int64_t>(Bk), t_end - t0));
        const int64_t r0 = base + t0 * D;
        for (int i = tid; i < m * m; i += kThreads) {
            const int s = i / m, s2 = i % m;
            float x = 0.f;
            if (s2 <= s) {
                for (int f = 0; f < D; ++f) x += opd(a.a, 0, r0 + s * D + f) * opd(a.b, 1, r0 + s2 * D + f);
                x *= sh.pw[s - s2];
            }
            sh.score[s * kMaxBk + s2] = x;
        }
        __syncthreads();
        for (int i = tid; i < m * D; i += kThreads) {
            const int s = i / D, col = i % D;
            float inter = 0.f, intra = 0.f;
            for (int f = 0; f < D; ++f) inter += opd(a.a, 0, r0 + s * D + f) * sh.state[f * D + col];
            for (int s2 = 0; s2 <= s; ++s2) intra += sh.score[s * kMaxBk + s2] * opd(a.c, 2, r0 + s2 * D + col);
            const float gr = a.phi_grad ? dphi_of_x(ld<BF16>(a.phi_grad, r0 + s * D + col), a.phi) : 1.f;
            st<BF16>(a.out0, r0 + s * D + col, gr * (sh.pw[s + 1] * inter + intra));
        }
        __syncthreads();
        for (int i = tid; i < D * D; i += kThreads) {
            const int f = i / D, col = i % D;
            float acc = 0.f;
            for (int s = 0; s < m; ++s)
                acc += sh.pw[m - 1 - s] * opd(a.b, 1, r0 + s * D + f) * opd(a.c, 2, r0 + s * D + col);
            sh.state[i] = sh.pw[m] * sh.state[i] + acc;
        }
        __syncthreads();
    }
    if (a.kv_out && c == a.chunks - 1) {
        float* dst = a.kv_out + pair * D * D;
        for (int i = tid; i < D * D; i += kThreads) dst[i] = sh.state[i];
    }
}

// Reverse sweep over one chunk (blocks from last to first), carrying
// dS = sum_{i >= end of block} lam^(i - end) q_i dO_i^T:
//   dK_b = (G o M)^T Q_b + diag(lam^(m-s)) V_b dS^T,   G = dO_b V_b^T
//   dV_b = (P o M)^T dO_b + diag(lam^(m-s)) K_b dS,    P = Q_b K_b^T
//   dS  <- lam^m dS + (diag(lam^s) Q_b)^T dO_b
// A gradient F arriving at the final state enters as the last chunk's dS with the
// exponents of the sequence's last block lowered by one (F reaches token j as
// lam^(N-1-j) F, not lam^(N-j)); chunk 0 ends with lam dS = the gradient of S0.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_rev_generic(SweepArgs a, LamArgs lam) {
    __shared__ Tile sh;
    const int64_t pair = blockIdx.x / a.chunks;
    const int c = blockIdx.x % a.chunks;
    const int D = a.D, Bk = a.Bk, tid = threadIdx.x;
    const float lv = lam.lam[pair % a.H];
    const int64_t t_begin = static_cast<int64_t>(c) * a.L;
    const int64_t t_end = min(a.N, t_begin + a.L);
    const int64_t base = pair * a.N * D;
    // queries and keys through the feature map
    auto opd = [&](const void* p, int bit, int64_t i) {
        const float x = ld<BF16>(p, i);
        return (a.phi && ((a.phi_mask >> bit) & 1)) ? phi_apply(x, a.phi) : x;
    };
    fill_powers(sh.pw, lv, Bk);
    const bool last = c == a.chunks - 1;
    const float* init = !last ? a.slots + rev_slot_index(a, pair, c) * D * D
                              : (a.g_final ? a.g_final + pair * D * D : nullptr);
    for (int i = tid; i < D * D; i += kThreads) sh.state[i] = init ? init[i] : 0.f;
    __syncthreads();

    const int64_t nblk = (t_end - t_begin + Bk - 1) / Bk;
    for (int64_t bi = nblk - 1; bi >= 0; --bi) {
        const int64_t t0 = t_begin + bi * Bk;
        const int m = static_cast<int>(min(static_cast<int64_t>(Bk), t_end - t0));
        const int shift = (last && a.g_final && bi == nblk - 1) ? 1 : 0;
        const int64_t r0 = base + t0 * D;
        // G[i][j] = lam^(i-j) dO_i . v_j for i >= j
        for (int idx = tid; idx < m * m; idx += kThreads) {
            const int i = idx / m, j = idx % m;
            float x = 0.f;
            if (j <= i) {
                for (int f = 0; f < D; ++f) x += ld<BF16>(a.g, r0 + i * D + f) * ld<BF16>(a.c, r0 + j * D + f);
                x *= sh.pw[i - j];
            }
            sh.score[i * kMaxBk + j] = x;
        }
        __syncthreads();
        for (int idx = tid; idx < m * D; idx += kThreads) {
            const int j = idx / D, f = idx % D;
            float intra = 0.f, inter = 0.f;
            for (int i = j; i < m; ++i) intra += sh.score[i * kMaxBk + j] * opd(a.a, 0, r0 + i * D + f);
            for (int col = 0; col < D; ++col) inter += sh.state[f * D + col] * ld<BF16>(a.c, r0 + j * D + col);
            const float gr = a.phi ? dphi_of_x(ld<BF16>(a.b, r0 + j * D + f), a.phi) : 1.f;
            st<BF16>(a.out0, r0 + j * D + f, gr * (intra + sh.pw[m - shift - j] * inter));
        }
        __syncthreads();
        // P[i][j] = lam^(i-j) q_i . k_j for i >= j
        for (int idx = tid; idx < m * m; idx += kThreads) {
            const int i = idx / m, j = idx % m;
            float x = 0.f;
            if (j <= i) {
                for (int f = 0; f < D; ++f) x += opd(a.a, 0, r0 + i * D + f) * opd(a.b, 1, r0 + j * D + f);
                x *= sh.pw[i - j];
            }
            sh.score[i * kMaxBk + j] = x;
        }
        __syncthreads();
        for (int idx = tid; idx < m * D; idx += kThreads) {
            const int j = idx / D, col = idx % D;
            float intra = 0.f, inter = 0.f;
            for (int i = j; i < m; ++i) intra += sh.score[i * kMaxBk + j] * ld<BF16>(a.g, r0 + i * D + col);
            for (int f = 0; f < D; ++f) inter += opd(a.b, 1, r0 + j * D + f) * sh.state[f * D + col];
            st<BF16>(a.out1, r0 + j * D + col, intra + sh.pw[m - shift - j] * inter);
        }
        __syncthreads();
        for (int idx = tid; idx < D * D; idx += kThreads) {
            const int f = idx / D, col = idx % D;
            float acc = 0.f;
            for (int s = 0; s < m; ++s)
                acc += sh.pw[s] * opd(a.a, 0, r0 + s * D + f) * ld<BF16>(a.g, r0 + s * D + col);
            sh.state[idx] = sh.pw[m - shift] * sh.state[idx] + acc;
        }
        __syncthreads();
    }
    if (c == 0 && a.ds_out)
        for (int i = tid; i < D * D; i += kThreads) a.ds_out[pair * D * D + i] = lv * sh.state[i];
}

// Aggregate state of one chunk, started from zero (see ChunkStateArgs).
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_chunk_state_generic(ChunkStateArgs a, LamArgs lam) {
    __shared__ float state[kMaxD * kMaxD];
    __shared__ float pw[kMaxBk + 1];
    const int per = a.chunks - 1;
    const int64_t pair = blockIdx.x / per;
    const int slot = blockIdx.x % per;
    const int c = a.reverse ? slot + 1 + a.part0 : slot;
    const int D = a.D, Bk = a.Bk, tid = threadIdx.x;
    fill_powers(pw, lam.lam[pair % a.H], Bk);
    for (int i = tid; i < D * D; i += kThreads) state[i] = 0.f;
    __syncthreads();
    const int64_t t_begin = static_cast<int64_t>(c) * a.L;
    const int64_t t_end = min(a.N, t_begin + a.L);
    const int64_t base = pair * a.N * D;
    const int64_t nblk = (t_end - t_begin + Bk - 1) / Bk;
    for (int64_t n = 0; n < nblk; ++n) {
        const int64_t bi = a.reverse ? nblk - 1 - n : n;
        const int64_t t0 = t_begin + bi * Bk;
        const int m = static_cast<int>(min(static_cast<int64_t>(Bk), t_end - t0));
        const int64_t r0 = base + t0 * D;
        for (int i = tid; i < D * D; i += kThreads) {
            const int f = i / D, col = i % D;
            float acc = 0.f;
            for (int s = 0; s < m; ++s) {
                const float w = a.reverse ? pw[s] : pw[m - 1 - s];
                const float x = ld<BF16>(a.x, r0 + s * D + f), y = ld<BF16>(a.y, r0 + s * D + col);
                acc += w * ((a.phi_mask & 1) ? phi_apply(x, a.phi) : x) * ((a.phi_mask & 2) ? phi_apply(y, a.phi) : y);
            }
            state[i] = pw[m] * state[i] + acc;
        }
        __syncthreads();
    }
    float* dst = a.slots + (pair * per + slot) * D * D;
    for (int i = tid; i < D * D; i += kThreads) dst[i] = state[i];
}

constexpr int kScanBatch = 8;  // chunk slots whose loads a scan thread keeps in flight

__global__ __launch_bounds__(kThreads) void k_scan(ScanArgs a, LamArgs lam) {
    const int DD = a.D * a.D;
    const int per_pair = (DD + kThreads - 1) / kThreads;
    const int64_t pair = blockIdx.x / per_pair;
    const int e = (blockIdx.x % per_pair) * kThreads + threadIdx.x;
    if (e >= DD) return;
    const float lv = lam.lam[pair % a.H];
    const float lamL = lam_pow(lv, a.L);
    const int n = a.chunks - 1;
    float* sl = a.slots + pair * n * DD + e;
    // Each batch's loads are issued before any of its stores: the slots are distinct,
    // which the compiler cannot see, and a memory latency per slot would dominate.
    float x[kScanBatch];
    if (!a.reverse) {
        float S = 0.f;
        if (a.kv_in) {
            const float* src = a.kv_in + pair * DD;
            S = a.kv_in_transposed ? src[(e % a.D) * a.D + e / a.D] : src[e];
        }
        for (int c0 = 0; c0 < n; c0 += kScanBatch) {
#pragma unroll
            for (int j = 0; j < kScanBatch; ++j) x[j] = c0 + j < n ? sl[static_cast<int64_t>(c0 + j) * DD] : 0.f;
#pragma unroll
            for (int j = 0; j < kScanBatch; ++j)
                if (c0 + j < n) {
                    S = lamL * S + x[j];
                    sl[static_cast<int64_t>(c0 + j) * DD] = S;
                }
        }
    } else {
        // the final-state gradient enters at the last token undecayed, so it reaches the
        // start of chunk j decayed over N - 1 - j L tokens
        const float G = a.g_final ? a.g_final[pair * DD + e] : 0.f;
        auto start_of = [&](int c) { return (static_cast<int64_t>(c) + 1 + a.part0) * a.L; };
        float R = 0.f;
        bool started = false;
        for (int c1 = n - 1; c1 >= 0; c1 -= kScanBatch) {
#pragma unroll
            for (int j = 0; j < kScanBatch; ++j) {
                const int c = c1 - j;
                x[j] = (c >= 0 && start_of(c) < a.N) ? sl[static_cast<int64_t>(c) * DD] : 0.f;
            }
#pragma unroll
            for (int j = 0; j < kScanBatch; ++j) {
                const int c = c1 - j;
                if (c < 0) break;
                float* p = sl + static_cast<int64_t>(c) * DD;
                const int64_t start = start_of(c);
                if (start >= a.N) {
                    *p = 0.f;  // a part past the end of the sequence
                    continue;
                }
                R = started ? x[j] + lamL * R : x[j] + lam_pow(lv, a.N - 1 - start) * G;
                started = true;
                *p = R;
            }
        }
    }
}

// Forward scan over the chunk states of a ragged batch: per listed (sequence b,
// head h), S = kv_in[b][h] (or 0); for c = 0 .. n_slots - 1: S = lam^L S + slot;
// slot = S, with slot (sbase + c) * H + h.  Sequences without chunk states are
// not listed (nothing to scan).
__global__ __launch_bounds__(kThreads) void k_scan_varlen(ScanArgs a, LamArgs lam, ScanList list) {
    const int DD = a.D * a.D;
    const int per_pair = (DD + kThreads - 1) / kThreads;
    const int64_t pair = blockIdx.x / per_pair;  // i * H + h over the list
    const int e = (blockIdx.x % per_pair) * kThreads + threadIdx.x;
    if (e >= DD) return;
    const int i = static_cast<int>(pair / a.H), h = static_cast<int>(pair % a.H);
    const int b = list.seq[i] & 0xFF, n_slots = list.seq[i] >> 8;
    const float lamL = lam_pow(lam.lam[h], a.L);
    float S = a.kv_in ? a.kv_in[(static_cast<int64_t>(b) * a.H + h) * DD + e] : 0.f;
    float* sl = a.slots + (static_cast<int64_t>(list.sbase[i]) * a.H + h) * DD + e;
    const int64_t step = static_cast<int64_t>(a.H) * DD;
    float x[kScanBatch];
    for (int c0 = 0; c0 < n_slots; c0 += kScanBatch) {
#pragma unroll
        for (int j = 0; j < kScanBatch; ++j) x[j] = c0 + j < n_slots ? sl[(c0 + j) * step] : 0.f;
#pragma unroll
        for (int j = 0; j < kScanBatch; ++j)
            if (c0 + j < n_slots) {
                S = lamL * S + x[j];
                sl[(c0 + j) * step] = S;
            }
    }
}

// One recurrent step per (sequence, head): S <- lam S + k v^T, o = q S.
// Thread t owns the 4 columns 4 * (t % (D/4)) .. +3 of rows t / (D/4) + r * (1024/D).
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_decode(DecodeArgs a, LamArgs lam) {
    __shared__ float qs[kMaxD], ks[kMaxD], vs[kMaxD];
    __shared__ float red[kThreads * 4];
    const int64_t pair = blockIdx.x;
    const int D = a.D, tid = threadIdx.x;
    const float lv = lam.lam[pair % a.H];
    int64_t sp = pair;  // the state this (sequence, head) steps
    if (a.slot_of) {
        const int32_t slot = a.slot_of[pair / a.H];
        if (slot < 0 || slot >= a.pool_slots) {
            // an index outside the pool: no state is touched and the output row is NaN
            for (int i = tid; i < D; i += kThreads) st<BF16>(a.o, pair * D + i, __builtin_nanf(""));
            return;
        }
        sp = static_cast<int64_t>(slot) * a.H + pair % a.H;
    }
    for (int i = tid; i < D; i += kThreads) {
        qs[i] = phi_apply(ld<BF16>(a.q, pair * D + i), a.phi);
        ks[i] = phi_apply(ld<BF16>(a.k, pair * D + i), a.phi);
        vs[i] = ld<BF16>(a.v, pair * D + i);
    }
    __syncthreads();
    const int cols4 = D / 4;
    const int cg = tid % cols4;
    const int rstep = kThreads / cols4;
    float4* S = reinterpret_cast<float4*>(a.state + sp * D * D);
    const float4 vv = make_float4(vs[4 * cg], vs[4 * cg + 1], vs[4 * cg + 2], vs[4 * cg + 3]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int r = tid / cols4; r < D; r += rstep) {
        float4 x = S[r * cols4 + cg];
        const float kr = ks[r], qr = qs[r];
        x.x = lv * x.x + kr * vv.x;
        x.y = lv * x.y + kr * vv.y;
        x.z = lv * x.z + kr * vv.z;
        x.w = lv * x.w + kr * vv.w;
        S[r * cols4 + cg] = x;
        acc.x += qr * x.x;
        acc.y += qr * x.y;
        acc.z += qr * x.z;
        acc.w += qr * x.w;
    }
    red[tid * 4 + 0] = acc.x;
    red[tid * 4 + 1] = acc.y;
    red[tid * 4 + 2] = acc.z;
    red[tid * 4 + 3] = acc.w;
    __syncthreads();
    if (tid < D) {
        const int g = (tid / 4), comp = tid % 4;
        float o = 0.f;
        for (int rg = 0; rg < rstep; ++rg) o += red[(rg * cols4 + g) * 4 + comp];
        st<BF16>(a.o, pair * D + tid, o);
    }
}

}  // namespace

void launch_fwd_generic(const SweepArgs& a, const LamArgs& lam, int bf16, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(a.pairs * a.chunks));
    if (bf16)
        hipLaunchKernelGGL(k_fwd_generic<true>, grid, dim3(kThreads), 0, s, a, lam);
    else
        hipLaunchKernelGGL(k_fwd_generic<false>, grid, dim3(kThreads), 0, s, a, lam);
}

void launch_rev_generic(const SweepArgs& a, const LamArgs& lam, int bf16, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(a.pairs * a.chunks));
    if (bf16)
        hipLaunchKernelGGL(k_rev_generic<true>, grid, dim3(kThreads), 0, s, a, lam);
    else
        hipLaunchKernelGGL(k_rev_generic<false>, grid, dim3(kThreads), 0, s, a, lam);
}

void launch_chunk_state_generic(const ChunkStateArgs& a, const LamArgs& lam, int bf16, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(a.pairs * (a.chunks - 1)));
    if (bf16)
        hipLaunchKernelGGL(k_chunk_state_generic<true>, grid, dim3(kThreads), 0, s, a, lam);
    else
        hipLaunchKernelGGL(k_chunk_state_generic<false>, grid, dim3(kThreads), 0, s, a, lam);
}

void launch_scan_varlen(const ScanArgs& a, const LamArgs& lam, const ScanList& list, hipStream_t s) {
    const int per_pair = (a.D * a.D + kThreads - 1) / kThreads;
    dim3 grid(static_cast<unsigned>(static_cast<int64_t>(list.count) * a.H * per_pair));
    hipLaunchKernelGGL(k_scan_varlen, grid, dim3(kThreads), 0, s, a, lam, list);
}

void launch_scan(const ScanArgs& a, const LamArgs& lam, hipStream_t s) {
    const int per_pair = (a.D * a.D + kThreads - 1) / kThreads;
    dim3 grid(static_cast<unsigned>(a.pairs * per_pair));
    hipLaunchKernelGGL(k_scan, grid, dim3(kThreads), 0, s, a, lam);
}

void launch_decode(const DecodeArgs& a, const LamArgs& lam, int bf16, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(a.pairs));
    if (bf16)
        hipLaunchKernelGGL(k_decode<true>, grid, dim3(kThreads), 0, s, a, lam);
    else
        hipLaunchKernelGGL(k_decode<false>, grid, dim3(kThreads), 0, s, a, lam);
}

}  // namespace la
