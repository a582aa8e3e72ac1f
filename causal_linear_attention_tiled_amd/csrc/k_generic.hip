// Generic kernels: every shape the library accepts (D <= 128, Bk <= 128,
// float32 or bfloat16 storage), plain float32 arithmetic, no matrix cores.
// They follow the block decomposition of Lightning Attention-2 (Tiling
// paragraph: intra-block part as ordinary masked attention, inter-block part
// through the carried key-value state) and serve as the path for shapes the
// MFMA kernels do not cover, and for float32 storage.
//
// One workgroup handles one (sequence, chunk).  The sweeps keep the D x D float32
// state and one block's score tile in LDS and stage each block's rows there (read
// from global memory once); the chunk aggregates stage their rows and keep the state
// in registers.  D is a compile-time constant of every kernel that loops over features.
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int kMaxD = 128;

__device__ __forceinline__ void fill_powers(float* pw, float lam, int Bk) {
    for (int e = threadIdx.x; e <= Bk; e += kThreads) pw[e] = lam_pow(lam, e);
}

// The forward's LDS: the D x D state, one block's score tile, the block's Q, K and V rows
// (feature map applied) and its decay powers, for blocks of Bs tokens, the largest block
// that divides the call's Bk and fits (fwd_generic_block; the block only decides which
// terms pass through a score tile and which through the state, never the function).
constexpr int kFwdPoolFloats = 30 * 1024;  // 120 KiB
// (the staged rows are D + 1 floats apart, so that threads reading one column of
// consecutive rows hit distinct LDS banks)
__host__ __device__ constexpr int fwd_pool_floats(int D, int Bs) { return D * D + Bs * Bs + 3 * Bs * (D + 1) + Bs + 1; }
static_assert(fwd_pool_floats(kMaxD, 16) <= kFwdPoolFloats, "every D fits at the smallest block");

// Forward sweep over tokens [t_begin, t_end) of one (sequence, head), whose token rows
// start at element base and lie pitch elements apart, in blocks of a.Bk tokens:
//   O_b = diag(lam^(s+1)) Q_b S + (Q_b K_b^T o M) V_b,  S <- lam^m S + (diag(lam^(m-1-s)) K_b)^T V_b
// starting from init (or zero; read transposed when `transposed`; NaN when `poison`) and
// leaving the final state in kv_dst (unless null).  Each block's rows are read from
// global memory once, into LDS.  D (= a.D) is a compile-time constant, so the loops over
// features unroll and their LDS reads issue back to back instead of one dependent read
// per step (the float32 correctness shape B1 H2 N256 d16 runs on two workgroups, where
// that latency is the whole run time).
template <bool BF16, int D>
__device__ void generic_sweep(const SweepArgs& a, float* pool, float lv, int64_t t_begin, int64_t t_end,
                              int64_t base, int64_t pitch, const float* init, bool transposed, bool poison,
                              float* kv_dst) {
    const int Bk = a.Bk, tid = threadIdx.x;
    float* state = pool;             // [D][D]
    float* score = state + D * D;    // [Bk][Bk]
    const int rp = D + 1;            // staged row pitch
    float* qs = score + Bk * Bk;     // [Bk][D + 1] each
    float* ks = qs + Bk * rp;
    float* vs = ks + Bk * rp;
    float* pw = vs + Bk * rp;        // lam^e, e = 0..Bk
    // operand x of slot bit (0: a, 1: b, 2: c), through the feature map when that slot takes it
    auto opd = [&](const void* p, int bit, int64_t i) {
        const float x = ld<BF16>(p, i);
        return (a.phi && ((a.phi_mask >> bit) & 1)) ? phi_apply(x, a.phi) : x;
    };
    fill_powers(pw, lv, Bk);
    for (int i = tid; i < D * D; i += kThreads) {
        float x = 0.f;
        if (init) x = transposed ? init[(i % D) * D + i / D] : init[i];
        state[i] = poison ? __builtin_nanf("") : x;
    }

    for (int64_t t0 = t_begin; t0 < t_end; t0 += Bk) {
        const int m = static_cast<int>(min(static_cast<int64_t>(Bk), t_end - t0));
        const int64_t r0 = base + t0 * pitch;
        __syncthreads();  // the previous block's rows and the state update are done with
        for (int i = tid; i < m * D; i += kThreads) {
            const int row = i / D, col = i % D;
            const int64_t at = r0 + row * pitch + col;
            qs[row * rp + col] = opd(a.a, 0, at);
            ks[row * rp + col] = opd(a.b, 1, at);
            vs[row * rp + col] = opd(a.c, 2, at);
        }
        __syncthreads();
        for (int i = tid; i < m * m; i += kThreads) {
            const int s = i / m, s2 = i % m;
            float x = 0.f;
            if (s2 <= s) {
#pragma unroll
                for (int f = 0; f < D; ++f) x += qs[s * rp + f] * ks[s2 * rp + f];
                x *= pw[s - s2];
            }
            score[s * Bk + s2] = x;
        }
        __syncthreads();
        for (int i = tid; i < m * D; i += kThreads) {
            const int s = i / D, col = i % D;
            float inter = 0.f, intra = 0.f;
#pragma unroll
            for (int f = 0; f < D; ++f) inter += qs[s * rp + f] * state[f * D + col];
#pragma unroll 8
            for (int s2 = 0; s2 <= s; ++s2) intra += score[s * Bk + s2] * vs[s2 * rp + col];
            const float gr = a.phi_grad ? dphi_of_x(ld<BF16>(a.phi_grad, r0 + s * pitch + col), a.phi) : 1.f;
            st<BF16>(a.out0, r0 + s * pitch + col, gr * (pw[s + 1] * inter + intra));
        }
        __syncthreads();
        for (int i = tid; i < D * D; i += kThreads) {
            const int f = i / D, col = i % D;
            float acc = 0.f;
#pragma unroll 8
            for (int s = 0; s < m; ++s) acc += pw[m - 1 - s] * ks[s * rp + f] * vs[s * rp + col];
            state[i] = pw[m] * state[i] + acc;
        }
    }
    __syncthreads();
    if (kv_dst)
        for (int i = tid; i < D * D; i += kThreads) kv_dst[i] = state[i];
}

// One workgroup per (sequence, chunk) of a dense [P][N][D] problem (D = a.D).
template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void k_fwd_generic(SweepArgs a, LamArgs lam) {
    __shared__ float pool[kFwdPoolFloats];
    const int64_t pair = blockIdx.x / a.chunks;
    const int c = blockIdx.x % a.chunks;
    const int64_t t_begin = static_cast<int64_t>(c) * a.L;
    const int64_t t_end = min(a.N, t_begin + a.L);
    const float* init = nullptr;
    bool transposed = false, poison = false;
    if (c == 0) {
        if (a.kv_in) {
            init = a.kv_in + pair * D * D;
            transposed = a.kv_in_transposed != 0;
        }
    } else {
        init = a.slots + fwd_slot_index(a, pair, c) * D * D;
        transposed = a.slots_transposed != 0;
        poison = !given_states_match(a);
    }
    float* kv_dst = (a.kv_out && c == a.chunks - 1) ? a.kv_out + pair * D * D : nullptr;
    generic_sweep<BF16, D>(a, pool, lam.lam[pair % a.H], t_begin, t_end, pair * a.N * D, D, init, transposed,
                           poison, kv_dst);
}

// One workgroup per (sequence, head) of a ragged batch packed token-major [T][H][D]:
// sequence b holds tokens [v.cu[b], v.cu[b + 1]) and is swept whole from its own initial
// state (kv_in[b][h]) to its own final state (kv_out[b][h]) (D = a.D).
template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void k_fwd_generic_varlen(SweepArgs a, LamArgs lam, VarlenArgs v) {
    __shared__ float pool[kFwdPoolFloats];
    const int b = static_cast<int>(blockIdx.x / a.H), h = static_cast<int>(blockIdx.x % a.H);
    const int64_t DD = static_cast<int64_t>(D) * D;
    const int64_t st_off = (static_cast<int64_t>(b) * a.H + h) * DD;
    generic_sweep<BF16, D>(a, pool, lam.lam[h], v.cu[b], v.cu[b + 1], static_cast<int64_t>(h) * D,
                           static_cast<int64_t>(a.H) * D, a.kv_in ? a.kv_in + st_off : nullptr, false, false,
                           a.kv_out ? a.kv_out + st_off : nullptr);
}

// The reverse sweep's LDS: the D x D gradient state (rows padded to D + 1 floats, so that
// threads reading one column of consecutive rows hit distinct banks), one block's score
// tile, the block's Q, K, V and dO rows (feature map applied to Q and K; padded rows) and
// its decay powers, for blocks of Bs tokens, the largest block dividing the call's Bk that
// fits (rev_generic_block).
constexpr int kRevPoolFloats = 34 * 1024;  // 136 KiB
__host__ __device__ constexpr int rev_pool_floats(int D, int Bs) {
    return D * (D + 1) + Bs * Bs + 4 * Bs * (D + 1) + Bs + 2;
}
static_assert(rev_pool_floats(kMaxD, 16) <= kRevPoolFloats, "every D fits at the smallest block");

// Reverse sweep over one chunk (blocks from last to first), carrying
// dS = sum_{i >= end of block} lam^(i - end) q_i dO_i^T:
//   dK_b = (G o M)^T Q_b + diag(lam^(m-s)) V_b dS^T,   G = dO_b V_b^T
//   dV_b = (P o M)^T dO_b + diag(lam^(m-s)) K_b dS,    P = Q_b K_b^T
//   dS  <- lam^m dS + (diag(lam^s) Q_b)^T dO_b
// A gradient F arriving at the final state enters as the last chunk's dS with the
// exponents of the sequence's last block lowered by one (F reaches token j as
// lam^(N-1-j) F, not lam^(N-j)); chunk 0 ends with lam dS = the gradient of S0.
// Each block's rows are read from global memory once, into LDS; D (= a.D) is a
// compile-time constant, so the loops over features unroll.
template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void k_rev_generic(SweepArgs a, LamArgs lam) {
    __shared__ float pool[kRevPoolFloats];
    constexpr int rp = D + 1;  // row pitch of the state and the staged rows
    const int64_t pair = blockIdx.x / a.chunks;
    const int c = blockIdx.x % a.chunks;
    const int Bk = a.Bk, tid = threadIdx.x;
    float* state = pool;             // [D][D + 1]
    float* score = state + D * rp;   // [Bk][Bk]
    float* qs = score + Bk * Bk;     // [Bk][D + 1] each: phi(Q), phi(K), V, dO
    float* ks = qs + Bk * rp;
    float* vs = ks + Bk * rp;
    float* gs = vs + Bk * rp;
    float* pw = gs + Bk * rp;        // lam^e, e = 0..Bk
    const float lv = lam.lam[pair % a.H];
    const int64_t t_begin = static_cast<int64_t>(c) * a.L;
    const int64_t t_end = min(a.N, t_begin + a.L);
    const int64_t base = pair * a.N * D;
    // queries and keys through the feature map
    auto opd = [&](const void* p, int bit, int64_t i) {
        const float x = ld<BF16>(p, i);
        return (a.phi && ((a.phi_mask >> bit) & 1)) ? phi_apply(x, a.phi) : x;
    };
    fill_powers(pw, lv, Bk);
    const bool last = c == a.chunks - 1;
    const float* init = !last ? a.slots + rev_slot_index(a, pair, c) * D * D
                              : (a.g_final ? a.g_final + pair * D * D : nullptr);
    for (int i = tid; i < D * D; i += kThreads) state[(i / D) * rp + i % D] = init ? init[i] : 0.f;

    const int64_t nblk = (t_end - t_begin + Bk - 1) / Bk;
    for (int64_t bi = nblk - 1; bi >= 0; --bi) {
        const int64_t t0 = t_begin + bi * Bk;
        const int m = static_cast<int>(min(static_cast<int64_t>(Bk), t_end - t0));
        const int shift = (last && a.g_final && bi == nblk - 1) ? 1 : 0;
        const int64_t r0 = base + t0 * D;
        __syncthreads();  // the previous block's rows, scores and state update are done with
        for (int i = tid; i < m * D; i += kThreads) {
            const int row = i / D, col = i % D;
            const int64_t at = r0 + row * D + col;
            qs[row * rp + col] = opd(a.a, 0, at);
            ks[row * rp + col] = opd(a.b, 1, at);
            vs[row * rp + col] = ld<BF16>(a.c, at);
            gs[row * rp + col] = ld<BF16>(a.g, at);
        }
        __syncthreads();
        // G[i][j] = lam^(i-j) dO_i . v_j for i >= j
        for (int idx = tid; idx < m * m; idx += kThreads) {
            const int i = idx / m, j = idx % m;
            float x = 0.f;
            if (j <= i) {
#pragma unroll
                for (int f = 0; f < D; ++f) x += gs[i * rp + f] * vs[j * rp + f];
                x *= pw[i - j];
            }
            score[i * Bk + j] = x;
        }
        __syncthreads();
        for (int idx = tid; idx < m * D; idx += kThreads) {
            const int j = idx / D, f = idx % D;
            float intra = 0.f, inter = 0.f;
#pragma unroll 8
            for (int i = j; i < m; ++i) intra += score[i * Bk + j] * qs[i * rp + f];
#pragma unroll
            for (int col = 0; col < D; ++col) inter += state[f * rp + col] * vs[j * rp + col];
            const float gr = a.phi ? dphi_of_x(ld<BF16>(a.b, r0 + j * D + f), a.phi) : 1.f;
            st<BF16>(a.out0, r0 + j * D + f, gr * (intra + pw[m - shift - j] * inter));
        }
        __syncthreads();
        // P[i][j] = lam^(i-j) q_i . k_j for i >= j
        for (int idx = tid; idx < m * m; idx += kThreads) {
            const int i = idx / m, j = idx % m;
            float x = 0.f;
            if (j <= i) {
#pragma unroll
                for (int f = 0; f < D; ++f) x += qs[i * rp + f] * ks[j * rp + f];
                x *= pw[i - j];
            }
            score[i * Bk + j] = x;
        }
        __syncthreads();
        for (int idx = tid; idx < m * D; idx += kThreads) {
            const int j = idx / D, col = idx % D;
            float intra = 0.f, inter = 0.f;
#pragma unroll 8
            for (int i = j; i < m; ++i) intra += score[i * Bk + j] * gs[i * rp + col];
#pragma unroll
            for (int f = 0; f < D; ++f) inter += ks[j * rp + f] * state[f * rp + col];
            st<BF16>(a.out1, r0 + j * D + col, intra + pw[m - shift - j] * inter);
        }
        __syncthreads();
        for (int idx = tid; idx < D * D; idx += kThreads) {
            const int f = idx / D, col = idx % D;
            float acc = 0.f;
#pragma unroll 8
            for (int s2 = 0; s2 < m; ++s2) acc += pw[s2] * qs[s2 * rp + f] * gs[s2 * rp + col];
            state[f * rp + col] = pw[m - shift] * state[f * rp + col] + acc;
        }
    }
    __syncthreads();
    if (c == 0 && a.ds_out)
        for (int i = tid; i < D * D; i += kThreads) a.ds_out[pair * D * D + i] = lv * state[(i / D) * rp + i % D];
}

// Aggregate state of one chunk, started from zero (see ChunkStateArgs), in blocks of at
// most 64 tokens (the aggregate is the same at any block size): each block's x and y rows
// are read from global memory once, into LDS (feature map applied, rows padded to D + 1
// floats); each thread keeps its D * D / kThreads entries of the state in registers.
constexpr int kStateRows = 64;
template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void k_chunk_state_generic(ChunkStateArgs a, LamArgs lam) {
    constexpr int rp = D + 1;
    constexpr int NE = (D * D + kThreads - 1) / kThreads;  // state entries per thread
    __shared__ float xs[kStateRows * (kMaxD + 1)];
    __shared__ float ys[kStateRows * (kMaxD + 1)];
    __shared__ float pw[kStateRows + 1];
    const int per = a.chunks - 1;
    const int64_t pair = blockIdx.x / per;
    const int slot = blockIdx.x % per;
    const int c = a.reverse ? slot + 1 + a.part0 : slot;
    const int Bs = min(a.Bk, kStateRows), tid = threadIdx.x;
    fill_powers(pw, lam.lam[pair % a.H], Bs);
    float acc[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] = 0.f;
    const int64_t t_begin = static_cast<int64_t>(c) * a.L;
    const int64_t t_end = min(a.N, t_begin + a.L);
    const int64_t base = pair * a.N * D;
    const int64_t nblk = t_end > t_begin ? (t_end - t_begin + Bs - 1) / Bs : 0;
    for (int64_t n = 0; n < nblk; ++n) {
        const int64_t bi = a.reverse ? nblk - 1 - n : n;
        const int64_t t0 = t_begin + bi * Bs;
        const int m = static_cast<int>(min(static_cast<int64_t>(Bs), t_end - t0));
        const int64_t r0 = base + t0 * D;
        __syncthreads();  // the previous block's rows are done with (and the powers are in)
        for (int i = tid; i < m * D; i += kThreads) {
            const int row = i / D, col = i % D;
            const float x = ld<BF16>(a.x, r0 + row * D + col), y = ld<BF16>(a.y, r0 + row * D + col);
            xs[row * rp + col] = (a.phi_mask & 1) ? phi_apply(x, a.phi) : x;
            ys[row * rp + col] = (a.phi_mask & 2) ? phi_apply(y, a.phi) : y;
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const int i = tid + e * kThreads;
            if (i < D * D) {
                const int f = i / D, col = i % D;
                float sum = 0.f;
#pragma unroll 8
                for (int s2 = 0; s2 < m; ++s2) {
                    const float w = a.reverse ? pw[s2] : pw[m - 1 - s2];
                    sum += w * xs[s2 * rp + f] * ys[s2 * rp + col];
                }
                acc[e] = pw[m] * acc[e] + sum;
            }
        }
    }
    float* dst = a.slots + (pair * per + slot) * D * D;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        const int i = tid + e * kThreads;
        if (i < D * D) dst[i] = acc[e];
    }
}

constexpr int kScanBatch = 8;  // chunk slots whose loads a scan thread keeps in flight

__global__ __launch_bounds__(kThreads) void k_scan(ScanArgs a, LamArgs lam) {
    // one thread per 4 consecutive elements of the D x D state (D * D is a multiple of 4)
    const int DD = a.D * a.D, DD4 = DD / 4;
    const int per_pair = (DD4 + kThreads - 1) / kThreads;
    const int64_t pair = blockIdx.x / per_pair;
    const int e4 = (blockIdx.x % per_pair) * kThreads + threadIdx.x;
    if (e4 >= DD4) return;
    const int e = 4 * e4;
    const float lv = lam.lam[pair % a.H];
    const float lamL = lam_pow(lv, a.L);
    const int n = a.chunks - 1;
    const int keep = a.keep > 1 ? a.keep : 1;
    float4* sl = reinterpret_cast<float4*>(a.slots + pair * n * DD + e);
    auto slot = [&](int c) -> float4& { return sl[static_cast<int64_t>(c) * DD4]; };
    // Each batch's loads are issued before any of its stores: the slots are distinct,
    // which the compiler cannot see, and a memory latency per slot would dominate.
    float4 x[kScanBatch];
    if (!a.reverse) {
        if (a.stamp_out && blockIdx.x == 0 && threadIdx.x == 0)
            for (int i = 0; i < kStampWords; ++i) a.stamp_out[i] = a.stamp.w[i];
        float4 S = make_float4(0.f, 0.f, 0.f, 0.f);
        if (a.kv_in) {
            const float* src = a.kv_in + pair * DD;
            if (a.kv_in_transposed) {
                const int r = e / a.D, col = e % a.D;
                S = make_float4(src[col * a.D + r], src[(col + 1) * a.D + r], src[(col + 2) * a.D + r],
                                src[(col + 3) * a.D + r]);
            } else {
                S = *reinterpret_cast<const float4*>(src + e);
            }
        }
        for (int c0 = 0; c0 < n; c0 += kScanBatch) {
#pragma unroll
            for (int j = 0; j < kScanBatch; ++j)
                if (c0 + j < n) x[j] = slot(c0 + j);
#pragma unroll
            for (int j = 0; j < kScanBatch; ++j) {
                const int c = c0 + j;
                if (c < n) {
                    S.x = lamL * S.x + x[j].x;
                    S.y = lamL * S.y + x[j].y;
                    S.z = lamL * S.z + x[j].z;
                    S.w = lamL * S.w + x[j].w;
                    // only the slots a sweep reads: the state entering chunk (c + 1) / keep
                    if ((c + 1) % keep == 0) slot(c) = S;
                }
            }
        }
    } else {
        // the final-state gradient enters at the last token undecayed, so it reaches the
        // start of chunk j decayed over N - 1 - j L tokens
        const float4 G = a.g_final ? *reinterpret_cast<const float4*>(a.g_final + pair * DD + e)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
        auto start_of = [&](int c) { return (static_cast<int64_t>(c) + 1 + a.part0) * a.L; };
        float4 R = make_float4(0.f, 0.f, 0.f, 0.f);
        bool started = false;
        for (int c1 = n - 1; c1 >= 0; c1 -= kScanBatch) {
#pragma unroll
            for (int j = 0; j < kScanBatch; ++j) {
                const int c = c1 - j;
                x[j] = (c >= 0 && start_of(c) < a.N) ? slot(c) : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int j = 0; j < kScanBatch; ++j) {
                const int c = c1 - j;
                if (c < 0) break;
                const bool store = c % keep == 0;  // the slots a sweep reads: chunk c / keep ends here
                const int64_t start = start_of(c);
                if (start >= a.N) {
                    if (store) slot(c) = make_float4(0.f, 0.f, 0.f, 0.f);  // a part past the end
                    continue;
                }
                const float f = started ? lamL : lam_pow(lv, a.N - 1 - start);
                const float4 prev = started ? R : G;
                R.x = x[j].x + f * prev.x;
                R.y = x[j].y + f * prev.y;
                R.z = x[j].z + f * prev.z;
                R.w = x[j].w + f * prev.w;
                started = true;
                if (store) slot(c) = R;
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

// The block the generic forward steps: the largest of Bk, Bk/2, ... whose LDS pool fits.
SweepArgs fwd_generic_block(const SweepArgs& a) {
    SweepArgs b = a;
    while (b.Bk > 16 && fwd_pool_floats(b.D, b.Bk) > kFwdPoolFloats) b.Bk /= 2;
    return b;
}

namespace {
// the dense kernel for the storage type and D (16, 32, 64 or 128: what the library accepts)
template <bool BF16>
void (*fwd_generic_kernel(int D))(SweepArgs, LamArgs) {
    switch (D) {
        case 16: return k_fwd_generic<BF16, 16>;
        case 32: return k_fwd_generic<BF16, 32>;
        case 64: return k_fwd_generic<BF16, 64>;
        default: return k_fwd_generic<BF16, 128>;
    }
}
template <bool BF16>
void (*fwd_generic_varlen_kernel(int D))(SweepArgs, LamArgs, VarlenArgs) {
    switch (D) {
        case 16: return k_fwd_generic_varlen<BF16, 16>;
        case 32: return k_fwd_generic_varlen<BF16, 32>;
        case 64: return k_fwd_generic_varlen<BF16, 64>;
        default: return k_fwd_generic_varlen<BF16, 128>;
    }
}
}  // namespace

void launch_fwd_generic(const SweepArgs& a, const LamArgs& lam, int bf16, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(a.pairs * a.chunks));
    const SweepArgs b = fwd_generic_block(a);
    auto kern = bf16 ? fwd_generic_kernel<true>(b.D) : fwd_generic_kernel<false>(b.D);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, s, b, lam);
}

void launch_fwd_generic_varlen(const SweepArgs& a, const LamArgs& lam, const VarlenArgs& v, int bf16,
                               hipStream_t s) {
    dim3 grid(static_cast<unsigned>(static_cast<int64_t>(v.nseq) * a.H));
    const SweepArgs b = fwd_generic_block(a);
    auto kern = bf16 ? fwd_generic_varlen_kernel<true>(b.D) : fwd_generic_varlen_kernel<false>(b.D);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, s, b, lam, v);
}

namespace {
template <bool BF16>
void (*rev_generic_kernel(int D))(SweepArgs, LamArgs) {
    switch (D) {
        case 16: return k_rev_generic<BF16, 16>;
        case 32: return k_rev_generic<BF16, 32>;
        case 64: return k_rev_generic<BF16, 64>;
        default: return k_rev_generic<BF16, 128>;
    }
}
template <bool BF16>
void (*chunk_state_generic_kernel(int D))(ChunkStateArgs, LamArgs) {
    switch (D) {
        case 16: return k_chunk_state_generic<BF16, 16>;
        case 32: return k_chunk_state_generic<BF16, 32>;
        case 64: return k_chunk_state_generic<BF16, 64>;
        default: return k_chunk_state_generic<BF16, 128>;
    }
}
}  // namespace

// The block the generic reverse sweep steps: the largest of Bk, Bk/2, ... whose LDS pool fits.
SweepArgs rev_generic_block(const SweepArgs& a) {
    SweepArgs b = a;
    while (b.Bk > 16 && rev_pool_floats(b.D, b.Bk) > kRevPoolFloats) b.Bk /= 2;
    return b;
}

void launch_rev_generic(const SweepArgs& a, const LamArgs& lam, int bf16, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(a.pairs * a.chunks));
    const SweepArgs b = rev_generic_block(a);
    auto kern = bf16 ? rev_generic_kernel<true>(b.D) : rev_generic_kernel<false>(b.D);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, s, b, lam);
}

void launch_chunk_state_generic(const ChunkStateArgs& a, const LamArgs& lam, int bf16, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(a.pairs * (a.chunks - 1)));
    auto kern = bf16 ? chunk_state_generic_kernel<true>(a.D) : chunk_state_generic_kernel<false>(a.D);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, s, a, lam);
}

void launch_scan_varlen(const ScanArgs& a, const LamArgs& lam, const ScanList& list, hipStream_t s) {
    const int per_pair = (a.D * a.D + kThreads - 1) / kThreads;
    dim3 grid(static_cast<unsigned>(static_cast<int64_t>(list.count) * a.H * per_pair));
    hipLaunchKernelGGL(k_scan_varlen, grid, dim3(kThreads), 0, s, a, lam, list);
}

void launch_scan(const ScanArgs& a, const LamArgs& lam, hipStream_t s) {
    const int per_pair = (a.D * a.D / 4 + kThreads - 1) / kThreads;
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
