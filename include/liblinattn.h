/*
 * liblinattn -- tiled causal linear attention with per-head decay on AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (Lightning Attention-2, "Tiling" paragraph and the record's
 * mechanism field: causal linear attention split into an intra-block part done
 * like ordinary attention and an inter-block part carried by a fixed-size
 * key-value state, in the forward and the backward pass; the glossary page
 * "Lightning Attention", features list: parallel form for training, recurrent
 * form with a constant-size state for inference).  For every sequence
 * (batch b, head h) of N tokens with head dim D and decay lam = lambda[h]:
 *
 *     O_t = sum_{j <= t} lam^(t-j) (q_t . k_j) v_j  +  lam^(t+1) q_t S0
 *
 * where S0 is an optional initial D x D state (kv_in).  The final state is
 *     S_N = lam^N S0 + sum_j lam^(N-1-j) k_j v_j^T     (kv_out).
 * The default feature map is the identity (LA_PHI_* below); there is no
 * normaliser; lam^0 = 1, so lam = 0 keeps only the j = t term.
 *
 * Conventions shared by every call
 *  - Layouts are contiguous row-major: Q, K, V, O, dO, dQ, dK, dV are
 *    [B][H][N][D]; states are [B][H][D][D] float32 with the key index as the
 *    row and the value index as the column.  Decode tensors are [Bs][H][D].
 *  - dtype LA_F32: tensors hold float32; LA_BF16: tensors hold bfloat16.
 *    Arithmetic accumulates in float32 either way; outputs are rounded to
 *    the tensor dtype (round to nearest even); states are always float32.
 *  - lambda is a HOST array of H float32 values in [0, 1], read during the
 *    call only.  Every other pointer is DEVICE memory owned by the caller;
 *    the library keeps no pointer after a call returns and never allocates
 *    device memory.  Device pointers must be 16-byte aligned.
 *  - Every call validates all arguments before it enqueues anything.  On an
 *    error nothing is enqueued and the code says why (la_strerror).  No call
 *    aborts or throws.  NaN and Inf inside tensors are not checked; they
 *    propagate.
 *  - Work is enqueued on `hip_stream` (a hipStream_t; NULL is the null
 *    stream) and the call returns without waiting.  Results are valid once
 *    the stream has reached that point.  Calls are thread-safe and keep no
 *    state between calls, except the optional profiling below.
 *  - Supported: D in {16, 32, 64, 128}, block size Bk in {16, 32, 64, 128,
 *    256}, 1 <= H <= 256, any N >= 1 (the last block may be partial).  The
 *    block size never changes the result beyond float rounding.  For bf16
 *    with D = 128 every sweep steps 64-token blocks: a 128-token block is
 *    stepped as two 64-token halves (the same function, with the second
 *    half's share of the first half's terms carried through the state
 *    instead of a score tile), and Bk only places the chunk boundaries of the
 *    chunked prefix on multiples of Bk.  LA_FWD128=1 runs the forward-
 *    direction sweeps (la_fwd, the dQ sweep of la_bwd) on whole 128-token
 *    blocks instead.  Bk = 256 is stepped as Bk = 128.
 *  - The environment variable LA_CHUNKS (a positive integer) overrides the
 *    number of chunks a sequence is split into for the chunked prefix over
 *    blocks, LA_AGG_K the number of parts of a chunk the chunk aggregates are
 *    taken over (la_plan; the chunks grow to a whole number of parts where
 *    the chunk count stays the same, else it is ignored); LA_KERNEL=generic
 *    forces the generic (non-MFMA) kernels; LA_FWD128=1 the 128-token-block
 *    forward-direction sweep;
 *    LA_STATE=dma2 the chunk aggregates with every wave loading at two
 *    workgroups per CU (instead of two loader waves at one);
 *    LA_FWD_WAVES=8, LA_REV_WAVES=4 and LA_DLAM_WAVES=4 select the
 *    other wave counts of the bf16 D = 128 direct-to-LDS sweeps (forward and
 *    dQ, dK and dV, decay derivative); LA_FUSED=0 / 1 keeps the chunked
 *    prefix out of / in the sweep's launch (la_fwd); LA_FUSED_SPIN (polls)
 *    lowers the bound on the fused prefix's waits and LA_FUSED_LOSE_FLAGS=1
 *    makes every such wait look for a flag value nobody publishes (both for
 *    failure-path tests: the waves that give up start from NaN, and the
 *    kernel ends normally).  They exist for tests and tuning; a
 *    query of the workspace size must be made under the same setting as the
 *    call it sizes.
 */
#ifndef LIBLINATTN_H
#define LIBLINATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LA_F32 = 0, LA_BF16 = 1 } la_dtype;

/* Elementwise kernel feature map phi applied to queries and keys (the glossary
 * page "Lightning Attention", features list and FAQ Q1: a kernel feature map
 * replaces the softmax; the pages do not name one), so that
 *     O_t = sum_{j <= t} lam^(t-j) (phi(q_t) . phi(k_j)) v_j (+ lam^(t+1) phi(q_t) S0).
 *   LA_PHI_IDENTITY : phi(x) = x
 *   LA_PHI_ELU1     : phi(x) = elu(x) + 1 (x + 1 for x > 0, e^x otherwise)
 *   LA_PHI_RELU     : phi(x) = max(x, 0), phi'(0) = 0
 * The map is applied in float32 and rounded to the tensor dtype before use.
 * Gradients are with respect to the raw Q and K.  The register-staged kernels
 * (selected with LA_FWD / LA_REV / LA_STATE / LA_DLAM = v1) have no feature
 * map: with one, those paths run the generic kernels. */
enum { LA_PHI_IDENTITY = 0, LA_PHI_ELU1 = 1, LA_PHI_RELU = 2 };

enum {
    LA_OK = 0,
    LA_EINVAL = 1,       /* null required pointer, non-positive size, lambda outside [0,1] or NaN,
                            unknown dtype, outputs overlapping inputs or each other */
    LA_EUNSUPPORTED = 2, /* D, Bk or H outside the supported set */
    LA_EALIGN = 3,       /* a device pointer not 16-byte aligned */
    LA_EWORKSPACE = 4,   /* workspace missing or smaller than the size query returns */
    LA_EHIP = 5,         /* the HIP runtime reported an error (launch, device query) */
    LA_ENODEV = 6,       /* no HIP device is available */
    LA_ESCRATCH = 7      /* la_fwd_noalloc: the call's chunk states exceed la_scratch_bytes() */
};

/* Forward pass (the tiled forward of Lightning Attention-2: per block an
 * intra-block masked, decayed Q K^T product with V, plus the inter-block
 * product of Q with the running state, which is then decayed and updated
 * with K^T V; the state is carried across blocks by a chunked prefix).
 *   Q, K, V : [B][H][N][D] dtype, device, read only.
 *   lambda  : host float32[H].
 *   phi     : LA_PHI_* feature map on Q and K (LA_EINVAL otherwise).
 *   kv_in   : [B][H][D][D] float32 device initial state S0, or NULL for zero.
 *   O       : [B][H][N][D] dtype, device, written.
 *   kv_out  : [B][H][D][D] float32 device, receives S_N; NULL skips it.
 *             Must not overlap kv_in.
 *   ws      : device workspace of at least la_fwd_workspace_bytes(...) bytes
 *             (may be NULL when that size is 0).  Its contents on entry do
 *             not matter; calls sharing a workspace must be stream-ordered.
 *             On return it holds the key-value state at the end of every
 *             chunk but the last (float32) and a stamp identifying this call,
 *             which la_bwd can take as fwd_ws instead of computing the states
 *             again.
 * When the sequence is split into at most 4 chunks of at most 2048 tokens
 * without aggregate parts (la_plan), on the 64-token sweep, the chunked
 * prefix runs inside the sweep's own launch: each chunk's workgroup first
 * aggregates its chunk, publishes it with a flag carrying a number unique to
 * the call, and sums the aggregates of the earlier chunks of its sequence
 * before sweeping (a workgroup waits only on workgroups dispatched before
 * it; the wait is bounded, in proportion to the awaited chunk's length
 * (about 200 us per 64-token block on top of several ms), and a wave that
 * gives up makes its columns NaN).
 * Under HIP graph capture, and with LA_FUSED=0, the aggregates and their
 * prefix run as two launches before the sweep instead (LA_FUSED=1 fuses any
 * plan, which is slower with more chunks, longer chunks or parts).  The two
 * forms round differently (within float rounding of the same sums). */
int la_fwd(const void* Q, const void* K, const void* V, const float* lambda, int64_t B, int64_t H,
           int64_t N, int64_t D, int32_t Bk, int32_t dtype, int32_t phi, const float* kv_in, void* O,
           float* kv_out, void* ws, size_t ws_bytes, void* hip_stream);

/* la_fwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation, kernels and arguments as la_fwd without a workspace.  The chunk
 * states that la_fwd keeps in `ws` go to a static device array of the library
 * instead, la_scratch_bytes() = 64 MiB per device (held until the process ends).
 * The call allocates nothing and creates no HIP object (no profiling events).
 *   Returns LA_ESCRATCH, with nothing enqueued, when the call needs more than
 *   la_scratch_bytes() (that is, when la_fwd_workspace_bytes(...) would exceed
 *   it); otherwise the statuses of la_fwd.
 *   Every call on a device shares that device's array, which keeps the last
 *   call's contents: calls that overlap in time on one device (different
 *   streams, or threads without ordering) race and give wrong results.
 *   Stream-ordered calls are safe.  The array's contents are not an output
 *   (pass la_fwd's workspace, not this one, to la_bwd as fwd_ws). */
int la_fwd_noalloc(const void* Q, const void* K, const void* V, const float* lambda, int64_t B, int64_t H,
                   int64_t N, int64_t D, int32_t Bk, int32_t dtype, int32_t phi, const float* kv_in, void* O,
                   float* kv_out, void* hip_stream);

/* Size of la_fwd_noalloc's static scratch array in bytes (per device). */
size_t la_scratch_bytes(void);

/* Workspace bytes la_fwd needs for this shape (0 when the sequence is not
 * split into chunks).  Returns 0 as well for invalid shapes. */
size_t la_fwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int32_t Bk, int32_t dtype);

/* The chunk plan la_fwd and la_bwd use for this shape (host only, no device
 * work): *chunks sequence chunks of *chunk_len tokens (the last may be
 * shorter; 1 chunk when the sequences alone fill the chip), and
 * *agg_parts, the parts of a chunk over which the forward direction takes
 * its chunk aggregates (the chunked prefix over blocks, Lightning
 * Attention-2, Tiling paragraph).  Any output pointer may be NULL.
 * Returns LA_OK, or the status la_fwd would return for the shape. */
int la_plan(int64_t B, int64_t H, int64_t N, int64_t D, int32_t Bk, int32_t dtype, int32_t* chunks,
            int64_t* chunk_len, int32_t* agg_parts);

/* Backward pass of L = <dO, O> + <F, S_N> for the forward above, where F is
 * an optional gradient arriving at the final state (the same tiling run in
 * the backward direction: a forward-order sweep for dQ that carries the key-
 * value state, and a reverse-order sweep for dK and dV that carries the
 * state's gradient A_t = sum_{i >= t} lam^(i-t) q_i dO_i^T + lam^(N-1-t) F):
 *   dQ_t = sum_{j<=t} lam^(t-j) (dO_t . v_j) k_j + lam^(t+1) S0 dO_t
 *   dK_j = A_j v_j  = sum_{i>=j} lam^(i-j) (dO_i . v_j) q_i + lam^(N-1-j) F v_j
 *   dV_j = A_j^T k_j = sum_{i>=j} lam^(i-j) (q_i . k_j) dO_i + lam^(N-1-j) F^T k_j
 *   dS0  = lam A_0  = sum_t lam^(t+1) q_t dO_t^T + lam^N F
 * The gradient of lambda is la_dlam's.  The call is stateless: Q, K, V and
 * kv_in are passed again.
 *   dO      : [B][H][N][D] dtype, device.
 *   dkv_out : [B][H][D][D] float32 device gradient F arriving at kv_out, or
 *             NULL for zero.
 *   dQ,dK,dV: [B][H][N][D] dtype, device, written; none may overlap an input
 *             or each other.
 *   dkv_in  : [B][H][D][D] float32 device, receives dS0 (the gradient of
 *             kv_in, also when kv_in is NULL); NULL skips it.  Must not
 *             overlap an input or another output.
 *   fwd_ws  : NULL, or the workspace of an la_fwd call with the same Q, K, V,
 *             lambda, shape, Bk, dtype, phi and kv_in, unchanged since that
 *             call (device, read only; same LA_CHUNKS setting).  The dQ sweep
 *             then reads the chunk states from it rather than making one more
 *             pass over K and V.  la_fwd stores a stamp after those states
 *             (shape, chunk plan, decay values, feature map and the addresses
 *             of Q, K, V and kv_in); the dQ sweep compares it, on the device,
 *             with the stamp these arguments imply, and where they differ
 *             every chunk that would start from those states starts from NaN,
 *             so its dQ rows come out NaN instead of wrong (chunk 0, dK, dV
 *             and dkv_in are unaffected).  The stamp cannot see tensors
 *             rewritten in place at the same addresses since la_fwd: with
 *             fwd_ws the call is not stateless.
 *   ws      : la_bwd_workspace_bytes(...) bytes, as for la_fwd; must not
 *             overlap fwd_ws.
 *   phi     : the feature map of the forward; dQ and dK are with respect to
 *             the raw Q and K (phi'(q), phi'(k) applied elementwise).
 *   other arguments as for la_fwd. */
int la_bwd(const void* Q, const void* K, const void* V, const void* dO, const float* lambda,
           int64_t B, int64_t H, int64_t N, int64_t D, int32_t Bk, int32_t dtype, int32_t phi,
           const float* kv_in, const float* dkv_out, void* dQ, void* dK, void* dV, float* dkv_in,
           const void* fwd_ws, void* ws, size_t ws_bytes, void* hip_stream);

size_t la_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int32_t Bk, int32_t dtype);

/* Derivative of the same loss L = <dO, O> + <F, S_N> with respect to the
 * per-head decay, summed over the batch:
 *     dlam[h] = sum_b dL/dlam_h
 *             = sum_b [ sum_t sum_{j<t} (t-j) lam^(t-j-1) (q_t . k_j)(dO_t . v_j)
 *                       + sum_t (t+1) lam^t q_t S0 dO_t
 *                       + <F, N lam^(N-1) S0 + sum_j (N-1-j) lam^(N-2-j) k_j v_j^T> ].
 * The decay enters the tiled computation (Lightning Attention-2, Tiling
 * paragraph) only through powers of lam, so the same block decomposition with
 * every power replaced by its derivative gives this sum: one forward-order
 * sweep that carries the state S and its derivative T = dS/dlam, with the
 * chunked prefix over blocks applied to the pair (S, T).  lam = 0 is allowed
 * (the derivative there keeps the first-order terms).  Same shapes, inputs
 * and feature map as la_bwd (phi applied to Q and K; it does not depend on
 * lam).
 *   dlam : [H] float32 device, written (4-byte aligned; must not overlap an
 *          input or the workspace).
 *   ws   : la_dlam_workspace_bytes(...) bytes of device memory (never 0: it
 *          holds one partial sum per (sequence, chunk)).
 * Accuracy: the block products run on bf16 operands with float32
 * accumulation (float32 storage: float32 throughout); partial sums are
 * added in double. */
int la_dlam(const void* Q, const void* K, const void* V, const void* dO, const float* lambda,
            int64_t B, int64_t H, int64_t N, int64_t D, int32_t Bk, int32_t dtype, int32_t phi,
            const float* kv_in, const float* dkv_out, float* dlam, void* ws, size_t ws_bytes,
            void* hip_stream);

size_t la_dlam_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int32_t Bk, int32_t dtype);

/* One recurrent decode step for Bs sequences and H heads (the recurrent
 * inference form with a fixed-size state, glossary page "Lightning
 * Attention", features list; constant decode memory, Lightning Attention-2
 * record, mechanism field).  Per (sequence, head), update then read, so the
 * new token sees itself:
 *     S <- lam S + k v^T,   o = q S
 *   state : [Bs][H][D][D] float32 device, updated in place.
 *   q,k,v : [Bs][H][D] dtype device.   o : [Bs][H][D] dtype device, written.
 *   phi   : LA_PHI_* feature map on q and k.
 * The state after n steps from S = 0 equals the kv_out of la_fwd over those
 * n tokens, and o equals that forward's output row. */
int la_decode_step(float* state, const void* q, const void* k, const void* v, const float* lambda,
                   int64_t Bs, int64_t H, int64_t D, int32_t dtype, int32_t phi, void* o,
                   void* hip_stream);

/* Forward pass over a ragged batch: B sequences of different lengths packed
 * token-major in one launch (the serving-side prefill that the constant-size
 * state makes cheap to continue, Lightning Attention-2 record, mechanism
 * field; the same tiling and chunked prefix as la_fwd).  Sequence b holds
 * tokens [seq_offsets[b], seq_offsets[b+1]) of the packed tensors.
 *   Q, K, V, O  : [T][H][D] dtype device (token-major, T = seq_offsets[B]);
 *                 row t of head h is (t * H + h) * D.
 *   seq_offsets : HOST int64[B + 1], seq_offsets[0] = 0, nondecreasing; read
 *                 during the call only.  Empty sequences are allowed (their
 *                 final state is kv_in, or 0).  B >= 1: batches of more than
 *                 256 sequences are launched as consecutive groups of 256 (one
 *                 launch per group and stage, all on hip_stream).
 *   kv_in       : [B][H][D][D] float32 device, or NULL for zero.
 *   kv_out      : [B][H][D][D] float32 device, or NULL to skip.
 *   ws          : la_fwd_varlen_workspace_bytes(...) bytes of device memory.
 * bf16 with D = 128 and Bk in {64, 128, 256} runs on the direct-to-LDS
 * kernels (chunk boundaries on multiples of Bk; blocks stepped as 64 tokens,
 * as in la_fwd; within every group of 256 sequences T_group * H * D * 2 <
 * 2^31, otherwise LA_EUNSUPPORTED).  Every other shape la_fwd accepts
 * (float32 storage, D in {16, 32, 64, 128}, Bk in {16, 32, 64, 128, 256})
 * runs on the generic kernels: one workgroup per (sequence, head) sweeping
 * the whole sequence in blocks of at most Bk and 128 tokens, no workspace, T <
 * 2^31.  Each sequence's results equal la_fwd over that sequence alone, up to
 * float rounding.  LA_VARLEN_L (a positive multiple of Bk) overrides the
 * chunk length of the direct-to-LDS path; a size query must see the same
 * setting. */
int la_fwd_varlen(const void* Q, const void* K, const void* V, const float* lambda,
                  const int64_t* seq_offsets, int64_t B, int64_t H, int64_t D, int32_t Bk,
                  int32_t dtype, int32_t phi, const float* kv_in, void* O, float* kv_out, void* ws,
                  size_t ws_bytes, void* hip_stream);

/* Workspace bytes for la_fwd_varlen (0 when no sequence is split into chunks,
 * or for unsupported or invalid arguments). */
size_t la_fwd_varlen_workspace_bytes(const int64_t* seq_offsets, int64_t B, int64_t H, int64_t D,
                                     int32_t Bk, int32_t dtype);

/* One recurrent decode step for Bs sequences whose states live in a pool of
 * slots (paged decode slots for serving; glossary page "Lightning Attention",
 * features list: recurrent inference with a constant-size state).
 *   pool    : [pool_slots][H][D][D] float32 device; sequence i steps the
 *             states of slot slot_of[i], in place.
 *   slot_of : [Bs] int32 device.  Entries must be distinct and in
 *             [0, pool_slots); an entry outside that range leaves the pool
 *             untouched and writes NaN to the sequence's output row (device
 *             values cannot be checked before the launch).
 *   q, k, v, o, lambda, dtype, D, phi: as for la_decode_step ([Bs][H][D]). */
int la_decode_step_paged(float* pool, int64_t pool_slots, const int32_t* slot_of, const void* q,
                         const void* k, const void* v, const float* lambda, int64_t Bs, int64_t H,
                         int64_t D, int32_t dtype, int32_t phi, void* o, void* hip_stream);

/* Static text for a status code.  For LA_EHIP the text of the last HIP error
 * seen by the calling thread is appended (thread-local buffer). */
const char* la_strerror(int code);

/* Library version, as major * 10000 + minor * 100 + patch. */
int la_version(void);

/* Optional profiling, used by the benchmark.  While enabled, every kernel the
 * library launches is bracketed by two HIP events recorded on the launch's
 * stream.  la_prof_collect waits for the recorded events, sums the elapsed
 * time per kernel name into `out` (at most `max_entries` entries), clears the
 * record and returns the number of entries written (or -LA_EHIP). */
typedef struct {
    char name[48];
    int64_t launches;
    double total_ms;
} la_prof_entry;

int la_prof_enable(int on);
int la_prof_collect(la_prof_entry* out, int max_entries);

#ifdef __cplusplus
}
#endif

#endif /* LIBLINATTN_H */
