// Internal declarations shared by the host API (api.cpp) and the HIP kernels.
// Not part of the public ABI (include/liblinattn.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

constexpr int kMaxHeads = 256;  // per-head decay values travel in the kernel arguments
constexpr int kThreads = 256;   // threads per workgroup of every kernel here

// Per-head decay, passed by value as a kernel argument (1 KiB).
struct LamArgs {
    float lam[kMaxHeads];
};

// A ragged batch (passed by value as a kernel argument, 2.3 KiB): sequence b covers
// tokens [cu[b], cu[b+1]) of token-major [T][H][D] tensors, so the rows of one
// (sequence, head) are H * D elements apart, and is split into wp[b+1] - wp[b]
// chunks of L tokens (at least one, also for an empty sequence).  Sequence b's
// chunk states are slots (wp[b] - b + c) * H + h, c = 0 .. chunks - 2.
// The sweep runs the full chunks (every chunk but a sequence's last) first, then
// the last chunks in the order last_order (longest first), so that the longest
// pieces of work start earliest.
constexpr int kMaxVarlenSeqs = 256;
struct VarlenArgs {
    int nseq;
    int cu[kMaxVarlenSeqs + 1];
    int wp[kMaxVarlenSeqs + 1];
    uint8_t last_order[kMaxVarlenSeqs];
};

// One sweep over every (sequence, chunk) of a [P][N][D] problem.
// Sequence p = b * H + h uses decay lam[h].  Chunk c covers tokens
// [c * L, min(N, (c + 1) * L)); L is a multiple of Bk.
// Stamp that la_fwd leaves after the chunk states in its workspace: shape, chunk plan,
// decay values and the identity of the inputs (their addresses).  A dQ sweep fed those
// states (la_bwd's fwd_ws) compares it with the stamp its own arguments imply.
constexpr int kStampWords = 8;
struct Stamp {
    uint32_t w[kStampWords];
};

struct SweepArgs {
    const void* a;  // forward: Q      reverse: Q
    const void* b;  // forward: K      reverse: K
    const void* c;  // forward: V      reverse: V
    const void* g;  // reverse only: dO
    void* out0;     // forward: O (or dQ)   reverse: dK
    void* out1;     // reverse: dV
    const float* slots;   // [P][chunks-1][D][D] carried state entering chunk c (c >= 1 fwd,
                          // c <= chunks-2 reverse), or nullptr when chunks == 1
    const float* kv_in;   // [P][D][D] initial state of chunk 0 (forward only) or nullptr
    int kv_in_transposed; // read kv_in as its transpose (dQ sweep)
    int slots_transposed; // read the slots as their transposes (dQ sweep fed by the
                          // forward pass's chunk states)
    const uint32_t* stamp;// with slots_transposed: the stamp stored after those states;
                          // chunks whose words differ from `expect` start from a NaN state
    Stamp expect;
    // the fused chunked prefix (k_fwd_dma_fused): per-chunk aggregates [P][chunks-1][D][D],
    // their flags [P][chunks-1][4] (one per compute wave, set to `epoch`), and where the
    // first workgroup stores `expect` as the workspace stamp (or nullptr)
    float* fused_aggs;
    uint64_t* fused_flags;
    uint64_t epoch;
    uint64_t wait_epoch;  // the flag value a waiting wave takes as published (normally epoch)
    int spin_limit;       // polls before a waiting wave gives up and starts from NaN
    uint32_t* stamp_store;
    float* kv_out;        // [P][D][D] final state (forward only) or nullptr
    const float* g_final; // reverse only: [P][D][D] gradient arriving at the final state, the
                          // dS the last chunk starts from, or nullptr for zero
    float* ds_out;        // reverse only: [P][D][D] gradient of the initial state, lam times
                          // the dS chunk 0 ends with, or nullptr
    int64_t N;
    int64_t L;            // chunk length in tokens
    int D, Bk, H, chunks;
    int64_t pairs;
    int phi;              // feature map (kPhi*) applied to the operands in phi_mask
    int phi_mask;         // bit 0: a, bit 1: b, bit 2: c (forward: Q, K; dQ sweep: K in c)
    const void* phi_grad; // forward-direction sweeps: raw tensor whose phi' multiplies out0
                          // (the dQ sweep's raw Q), or nullptr
    int slot_k;           // the chunk aggregates were taken over chunks of L / slot_k tokens
                          // (0 or 1: over the sweep's chunks); see fwd_slot_index and
                          // rev_slot_index
};

// Slot holding the gradient state that enters chunk c <= chunks - 2 of sequence `pair`
// from the right in a reverse sweep (the reverse aggregates are taken over slot_k parts
// of every chunk but the first, so it is slot c * slot_k of (chunks - 1) * slot_k).
__host__ __device__ inline int64_t rev_slot_index(const SweepArgs& a, int64_t pair, int c) {
    const int64_t k = a.slot_k > 1 ? a.slot_k : 1;
    return (pair * (a.chunks - 1) + c) * k;
}

// Slot holding the state that enters chunk c >= 1 of sequence `pair` in a
// forward-direction sweep.
__host__ __device__ inline int64_t fwd_slot_index(const SweepArgs& a, int64_t pair, int c) {
    const int64_t k = a.slot_k > 1 ? a.slot_k : 1;
    return pair * (a.chunks - 1) * k + c * k - 1;
}

// Chunk aggregate states: for the forward direction chunk c (0..chunks-2)
//   slot[c] = sum_{t in c} lam^(end_c - 1 - t) x_t y_t^T
// and for the reverse direction chunk c (1..chunks-1)
//   slot[c-1] = sum_{t in c} lam^(t - start_c) x_t y_t^T.
struct ChunkStateArgs {
    const void* x;  // [P][N][D]
    const void* y;  // [P][N][D]
    float* slots;   // [P][chunks-1][D][D]
    int64_t N, L;
    int D, Bk, H, chunks;
    int64_t pairs;
    int reverse;
    int phi;        // feature map (kPhi*) ...
    int phi_mask;   // ... applied to x (bit 0) and / or y (bit 1)
    int part0;      // reverse: slot s aggregates chunk s + 1 + part0 (chunks of L tokens here
                    // being the parts of the sweep's chunks)
};

// In-place scan of the slots of every sequence.
//   forward: S = kv_in (or 0); for c = 0..chunks-2: S = lam^L S + slot[c]; slot[c] = S
//   reverse: slot c holds the aggregate of chunk j = c + 1 + part0 (chunks of L tokens,
//            starting at j L); from the last chunk that starts before N down to c = 0:
//            R = slot[c] + lam^(N - 1 - j L) G for the first one, R = slot[c] + lam^L R after;
//            slot[c] = R (0 for chunks past the end; G = g_final or 0)
struct ScanArgs {
    float* slots;
    const float* kv_in;   // forward: initial state, or nullptr
    int kv_in_transposed;
    const float* g_final; // reverse: gradient arriving at the final state, or nullptr
    int64_t N;
    int64_t L;
    int D, H, chunks;
    int64_t pairs;
    int reverse;
    int part0;
    int keep;             // k_scan: slots a sweep reads are every keep-th (chunk boundaries of
                          // aggregates over keep parts per chunk); only those are written
                          // (0 or 1: every slot)
    uint32_t* stamp_out;  // forward k_scan: where to store `stamp` (nullptr: nowhere)
    Stamp stamp;
};

// False when a sweep is fed a forward pass's chunk states whose stamp is not the one its
// own arguments imply (a workspace from another call): its state is then NaN.
__device__ __forceinline__ bool given_states_match(const SweepArgs& a) {
    if (!a.stamp) return true;
    bool ok = true;
#pragma unroll
    for (int i = 0; i < kStampWords; ++i) ok &= a.stamp[i] == a.expect.w[i];
    return ok;
}

struct DecodeArgs {
    float* state;  // [P][D][D], or the slot pool [pool_slots][H][D][D] when slot_of is set
    const void* q;
    const void* k;
    const void* v;
    void* o;
    int D, H;
    int64_t pairs;           // Bs * H
    const int32_t* slot_of;  // [Bs] pool slot of each sequence, or nullptr (state[p] for pair p)
    int64_t pool_slots;
    int phi;                 // feature map applied to q and k
};

// Derivative of L = <dO, O> + <F, S_N> with respect to lam, forward direction,
// carrying the state S and its derivative T = dS/dlam:
//   per block (m tokens, local index s):  the block adds
//     sum_{s' < s} (s-s') lam^(s-s'-1) (q_s . k_s')(dO_s . v_s')
//     + sum_s [ (s+1) lam^s q_s S dO_s + lam^(s+1) q_s T dO_s ],
//   then T <- lam^m T + m lam^(m-1) S + sum_s (m-1-s) lam^(m-2-s) k_s v_s^T,
//        S <- lam^m S + sum_s lam^(m-1-s) k_s v_s^T;
//   the sequence's last chunk adds <F, T> at its end.
// Chunk c starts from (S, T) = (kv_in or 0, 0) for c = 0, else from slot c-1 of
// a scan over the chunk aggregates (slots [P][chunks-1][2][D][D]: S then T).
struct DlamArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* g;          // dO
    const float* slots;     // scanned (S, T) entering chunks 1 .. chunks-1, or nullptr
    const float* kv_in;     // [P][D][D] or nullptr
    const float* g_final;   // [P][D][D] F, or nullptr
    double* partial;        // [P][chunks] contribution of each (sequence, chunk)
    int64_t N, L;
    int D, Bk, H, chunks;
    int64_t pairs;
    int phi;                // feature map on q and k
    int slot_k;             // the (S, T) aggregates were taken over chunks of L / slot_k
                            // tokens (0 or 1: over these chunks): chunk c >= 1 starts from
                            // slot c * slot_k - 1 of the sequence's (chunks - 1) * slot_k
};

// First float of the (S, T) slot pair that chunk c >= 1 of sequence `pair` starts from.
__host__ __device__ inline int64_t dlam_slot_offset(const DlamArgs& a, int64_t pair, int c) {
    const int64_t k = a.slot_k > 1 ? a.slot_k : 1;
    return (pair * (a.chunks - 1) * k + c * k - 1) * 2 * static_cast<int64_t>(a.D) * a.D;
}

// Launchers (each enqueues exactly one kernel on `s`; errors are read by the caller).
void launch_fwd_generic(const SweepArgs& a, const LamArgs& lam, int bf16, hipStream_t s);
// The ragged forward on the generic kernels: one workgroup per (sequence, head) of the
// v.nseq sequences (token offsets v.cu), each swept whole.
void launch_fwd_generic_varlen(const SweepArgs& a, const LamArgs& lam, const VarlenArgs& v, int bf16,
                               hipStream_t s);
void launch_rev_generic(const SweepArgs& a, const LamArgs& lam, int bf16, hipStream_t s);
void launch_chunk_state_generic(const ChunkStateArgs& a, const LamArgs& lam, int bf16, hipStream_t s);
void launch_scan(const ScanArgs& a, const LamArgs& lam, hipStream_t s);
void launch_decode(const DecodeArgs& a, const LamArgs& lam, int bf16, hipStream_t s);

// MFMA kernels (bf16 storage, D = 128, Bk in {64, 128}).
bool mfma_supported(int D, int Bk);
bool mfma_rev_supported(int D, int Bk);
void launch_fwd_mfma(const SweepArgs& a, const LamArgs& lam, hipStream_t s);
void launch_rev_mfma(const SweepArgs& a, const LamArgs& lam, hipStream_t s);
void launch_chunk_state_mfma(const ChunkStateArgs& a, const LamArgs& lam, hipStream_t s);

// Forward sweep with direct-to-LDS loads (bf16, D = 128, Bk = 64); `waves` compute waves (4 or 8).
bool fwd_dma_supported(int D, int Bk, int64_t N);
// With a.fused_flags set: the fused chunked prefix (4 compute waves), no aggregate or scan
// launch before it.
void launch_fwd_dma(const SweepArgs& a, const LamArgs& lam, int waves, hipStream_t s);
// The same over a ragged batch: one workgroup per (chunk of a sequence, head), wp[nseq] * H in all.
void launch_fwd_dma_varlen(const SweepArgs& a, const LamArgs& lam, const VarlenArgs& v, hipStream_t s);

// The same with 128-token blocks (k_fwd_dma128.hip; bf16, D = 128, Bk = 128; selected with
// LA_FWD128=1, otherwise a 128-token block is stepped by the 64-token kernel): a ring of
// 64-token half blocks, each block computed in two phases.
bool fwd_dma128_supported(int D, int Bk, int64_t N);
void launch_fwd_dma128(const SweepArgs& a, const LamArgs& lam, hipStream_t s);

// Reverse (dK, dV) sweep with direct-to-LDS loads (bf16, D = 128; 64-token blocks, Bk = 128
// as two halves).
bool rev_dma_supported(int D, int Bk, int64_t N);
void launch_rev_dma(const SweepArgs& a, const LamArgs& lam, int waves, hipStream_t s);

// Chunk aggregates with direct-to-LDS loads (bf16, D = 128; Bk = 64 or 128, walked in 64-token blocks).
bool state_dma_supported(int D, int Bk, int64_t N);
// loader_waves: the form with two loader waves and a three-stage ring at one workgroup per
// CU (dense sequences); otherwise every wave loads, two workgroups per CU.
void launch_chunk_state_dma(const ChunkStateArgs& a, const LamArgs& lam, bool loader_waves, hipStream_t s);
// Forward chunk aggregates of a ragged batch: one workgroup per (slot, head).
void launch_chunk_state_dma_varlen(const ChunkStateArgs& a, const LamArgs& lam, const VarlenArgs& v,
                                   hipStream_t s);
// The sequences of a ragged batch that have chunk states: entry i names sequence
// seq[i] & 0xFF with (seq[i] >> 8) slots starting at per-head slot sbase[i].
struct ScanList {
    int count;
    int seq[kMaxVarlenSeqs];
    int sbase[kMaxVarlenSeqs];
};
// Forward scan of a ragged batch's chunk states (ScanArgs.L is the chunk length):
// one workgroup per (listed sequence, head, 256 state elements).
void launch_scan_varlen(const ScanArgs& a, const LamArgs& lam, const ScanList& list, hipStream_t s);

// Decay derivative (k_dlam.hip).  Chunk aggregates of (S, T) over (x, y) = (k, v),
// forward direction, into slots [P][chunks-1][2][D][D] (ChunkStateArgs.slots; phi on x
// when phi_mask bit 0 is set); the scan (S, T) <- (lam^L S + dS, lam^L T + L lam^(L-1) S + dT)
// from (kv_in or 0, 0); the sweep; and the sum over batch and chunks per head.
void launch_dlam_state_generic(const ChunkStateArgs& a, const LamArgs& lam, int bf16, hipStream_t s);
void launch_dlam_state_mfma(const ChunkStateArgs& a, const LamArgs& lam, hipStream_t s);
void launch_dlam_state_dma(const ChunkStateArgs& a, const LamArgs& lam, hipStream_t s);  // k_state_dma.hip
void launch_dlam_scan(const ScanArgs& a, const LamArgs& lam, hipStream_t s);
void launch_dlam_generic(const DlamArgs& a, const LamArgs& lam, int bf16, hipStream_t s);
bool dlam_mfma_supported(int D, int Bk);
void launch_dlam_mfma(const DlamArgs& a, const LamArgs& lam, hipStream_t s);
void launch_dlam_reduce(const double* partial, int64_t B, int H, int chunks, float* out, hipStream_t s);
// The sweep on direct-to-LDS loads (k_dlam_dma.hip; bf16, D = 128; 64-token blocks, Bk = 128
// as two halves).
bool dlam_dma_supported(int D, int Bk, int64_t N);
void launch_dlam_dma(const DlamArgs& a, const LamArgs& lam, int waves, hipStream_t s);  // waves: 4 or 8

}  // namespace la
