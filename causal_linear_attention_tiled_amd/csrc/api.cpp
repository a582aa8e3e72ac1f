// Host side of liblinattn: argument validation, the chunk plan, kernel
// dispatch and optional per-kernel profiling.  See include/liblinattn.h for
// the contract of every exported call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/liblinattn.h"
#include "la_internal.h"

namespace {

using la::LamArgs;

// Target workgroup count for the chunk plan: one per compute unit of an MI355X
// (256 CUs).  The sweep kernels hold one workgroup per CU (their LDS rings), so
// 256 workgroups run in one round; measured, two rounds of half-length chunks
// are slower (B4 H16 N2048 forward 72 us against 55 us; B2 H32 N8192 forward and
// backward 559 us against 497 us) and the long-sequence points are unchanged.
constexpr int64_t kTargetWorkgroups = 256;
// A chunk should span at least this many blocks, so the per-chunk state
// traffic (a few D x D float32 matrices) stays small next to its tokens.
constexpr int64_t kMinBlocksPerChunk = 4;

thread_local char g_err[256];

int hip_fail(hipError_t e, const char* where) {
    std::snprintf(g_err, sizeof(g_err), "%s: %s", where, hipGetErrorString(e));
    return LA_EHIP;
}

// ------------------------------------------------------------------ profiling
struct ProfRec {
    const char* name;
    hipEvent_t start, stop;
};
std::atomic<int> g_prof_on{0};
std::mutex g_prof_mu;
std::vector<ProfRec> g_prof;

// Enqueue one kernel through `fn`, bracketed by events when profiling.
template <typename Fn>
int launch(const char* name, hipStream_t s, Fn&& fn) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    // events created for this launch are destroyed on every failure path
    auto fail = [&](hipError_t e, const char* where) {
        if (e0) (void)hipEventDestroy(e0);
        if (e1) (void)hipEventDestroy(e1);
        return hip_fail(e, where);
    };
    const bool prof = g_prof_on.load(std::memory_order_relaxed) != 0;
    if (prof) {
        hipError_t er = hipEventCreate(&e0);
        if (er == hipSuccess) er = hipEventCreate(&e1);
        if (er != hipSuccess) return fail(er, "hipEventCreate");
        er = hipEventRecord(e0, s);
        if (er != hipSuccess) return fail(er, "hipEventRecord");
    }
    fn();
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(e, name);
    if (prof) {
        hipError_t er = hipEventRecord(e1, s);
        if (er != hipSuccess) return fail(er, "hipEventRecord");
        std::lock_guard<std::mutex> lk(g_prof_mu);
        g_prof.push_back({name, e0, e1});
    }
    return LA_OK;
}

// ------------------------------------------------------------------ validation
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
    const void* p;
    size_t bytes;
};

bool overlap(const Range& a, const Range& b) {
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    auto a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    if (a <= 0 || b <= 0) return false;
    if (a > INT64_MAX / b) return false;
    *out = a * b;
    return true;
}

bool valid_phi(int32_t phi) { return phi == LA_PHI_IDENTITY || phi == LA_PHI_ELU1 || phi == LA_PHI_RELU; }

bool supported_D(int64_t D) { return D == 16 || D == 32 || D == 64 || D == 128; }
bool supported_Bk(int64_t Bk) { return Bk == 16 || Bk == 32 || Bk == 64 || Bk == 128 || Bk == 256; }

// The largest block the kernels step: a 256-token block changes where the chunk
// boundaries may fall (multiples of 256) and is swept as two 128-token blocks (the
// same function; 128-token blocks already fill the LDS of the forward kernel).
constexpr int32_t kMaxKernelBk = 128;

// Shape checks common to la_fwd / la_bwd and their size queries.
int check_shape(int64_t B, int64_t H, int64_t N, int64_t D, int32_t Bk, int32_t dtype, int64_t* elems) {
    if (dtype != LA_F32 && dtype != LA_BF16) return LA_EINVAL;
    if (B <= 0 || H <= 0 || N <= 0 || D <= 0 || Bk <= 0) return LA_EINVAL;
    if (!supported_D(D) || !supported_Bk(Bk) || H > la::kMaxHeads) return LA_EUNSUPPORTED;
    int64_t t;
    if (!mul_ok(B, H, &t) || !mul_ok(t, N, &t) || !mul_ok(t, D, &t) || t > (INT64_MAX / 8)) return LA_EINVAL;
    *elems = t;
    return LA_OK;
}

int load_lambda(const float* lambda, int64_t H, LamArgs* out) {
    if (!lambda) return LA_EINVAL;
    std::memset(out, 0, sizeof(*out));
    for (int64_t h = 0; h < H; ++h) {
        const float x = lambda[h];
        if (!(x >= 0.f && x <= 1.f)) return LA_EINVAL;  // also rejects NaN
        out->lam[h] = x;
    }
    return LA_OK;
}

// ------------------------------------------------------------------ plan
struct Plan {
    int chunks;
    int64_t L;     // chunk length in tokens (multiple of Bk)
    int32_t bk;    // block size the kernels step (Bk, or 128 for Bk = 256)
    bool mfma;
    int agg_k;     // forward direction: aggregates over chunks of L / agg_k tokens
};

bool env_is(const char* name, const char* value) {
    const char* e = std::getenv(name);
    return e && std::strcmp(e, value) == 0;
}

bool force_generic() {
    const char* e = std::getenv("LA_KERNEL");
    return e && std::strcmp(e, "generic") == 0;
}

Plan make_plan(int64_t B, int64_t H, int64_t N, int64_t D, int32_t Bk, int32_t dtype) {
    Plan p;
    const int64_t pairs = B * H;
    const int64_t nb = (N + Bk - 1) / Bk;
    int64_t C = 1;
    const char* env = std::getenv("LA_CHUNKS");
    if (env && std::atoll(env) > 0) {
        C = std::atoll(env);
    } else if (pairs < kTargetWorkgroups) {
        C = (kTargetWorkgroups + pairs - 1) / pairs;
        C = std::min<int64_t>(C, std::max<int64_t>(1, nb / kMinBlocksPerChunk));
    }
    C = std::max<int64_t>(1, std::min<int64_t>(C, nb));
    const int64_t bpc = (nb + C - 1) / C;
    p.L = bpc * Bk;
    p.chunks = static_cast<int>((nb + bpc - 1) / bpc);
    p.bk = std::min(Bk, kMaxKernelBk);
    p.mfma = dtype == LA_BF16 && la::mfma_supported(static_cast<int>(D), p.bk) && !force_generic();
    // The chunk aggregates (one workgroup each, two per CU) are taken over agg_k equal
    // parts of every chunk when the chunks alone would leave the pass below 3/4 of a
    // round of 512 workgroups; the scans then run over the parts, chunk c of a forward
    // sweep starts from part c * agg_k - 1 and chunk c of a reverse sweep from the
    // gradient entering part (c + 1) agg_k.  Each part keeps at least kMinBlocksPerChunk
    // blocks.  LA_AGG_K forces it (dividing the blocks per chunk).
    p.agg_k = 1;
    if (p.chunks > 1) {
        const char* ek = std::getenv("LA_AGG_K");
        if (ek && std::atoll(ek) > 0) {
            const int64_t k = std::atoll(ek);
            if (bpc % k == 0) p.agg_k = static_cast<int>(k);
        } else {
            while ((p.chunks - 1) * p.agg_k * pairs < 384 && bpc % (2 * p.agg_k) == 0 &&
                   bpc / (2 * p.agg_k) >= kMinBlocksPerChunk)
                p.agg_k *= 2;
        }
    }
    return p;
}

size_t slot_bytes(int64_t pairs, const Plan& p, int64_t D) {
    if (p.chunks <= 1) return 0;
    return static_cast<size_t>(pairs) * static_cast<size_t>(p.chunks - 1) * static_cast<size_t>(D * D) *
           sizeof(float);
}

// The forward direction's slots: agg_k per chunk boundary.
size_t fwd_slot_bytes(int64_t pairs, const Plan& p, int64_t D) {
    return slot_bytes(pairs, p, D) * static_cast<size_t>(p.agg_k);
}

size_t round_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// la_dlam: the (S, T) chunk slots, then one double per (sequence, chunk).
size_t dlam_ws_bytes(int64_t pairs, const Plan& p, int64_t D) {
    return round_up(2 * fwd_slot_bytes(pairs, p, D)) + round_up(static_cast<size_t>(pairs * p.chunks) * sizeof(double));
}

// ------------------------------------------------------------------ sweeps
// Forward-direction sweep (O of la_fwd, or dQ of la_bwd with operands
// (dO, V, K) and the transposed initial state).
// With `given` non-null the chunk states are not computed: the sweep reads
// them, transposed, from `given` (the chunk states a forward pass left in its
// workspace, which are the transposes of the dQ sweep's states).
// Where the feature map enters a forward-direction sweep over (q, k, v).
struct PhiUse {
    int kind;          // kPhi* (0: identity, the rest unused)
    int sweep_mask;    // operands of the sweep it maps (bit 0: q, 1: k, 2: v)
    int state_mask;    // operands of the chunk aggregates over (k, v) it maps (bit 0: k, 1: v)
    const void* grad;  // raw tensor whose phi' multiplies the sweep's output, or nullptr
};

int run_forward_sweep(const void* q, const void* k, const void* v, void* out, const float* kv_in,
                      int kv_in_t, float* kv_out, float* slots, const float* given, int64_t pairs,
                      int64_t N, int64_t D, int32_t Bk, int32_t H, int bf16, const Plan& p,
                      const LamArgs& lam, const PhiUse& phi, hipStream_t s, const char* tag) {
    int rc;
    // the register-staged kernels have no feature map: with one, the generic kernels run
    const bool v1_ok = phi.kind == 0;
    if (p.chunks > 1 && !given) {
        // aggregates and scan over the agg_k parts of every chunk but the last
        const int64_t Lf = p.L / p.agg_k;
        const int chunks_f = (p.chunks - 1) * p.agg_k + 1;
        la::ChunkStateArgs cs{k, v, slots, N, Lf, static_cast<int>(D), Bk, H, chunks_f, pairs, 0,
                              phi.kind, phi.state_mask};
        if (p.mfma && la::state_dma_supported(static_cast<int>(D), Bk, N) && !env_is("LA_STATE", "v1"))
            rc = launch("chunk_state_dma", s, [&] { la::launch_chunk_state_dma(cs, lam, s); });
        else if (p.mfma && v1_ok)
            rc = launch("chunk_state_mfma", s, [&] { la::launch_chunk_state_mfma(cs, lam, s); });
        else
            rc = launch("chunk_state_generic", s, [&] { la::launch_chunk_state_generic(cs, lam, bf16, s); });
        if (rc) return rc;
        la::ScanArgs sc{slots, kv_in, kv_in_t, nullptr, N, Lf, static_cast<int>(D), H, chunks_f, pairs, 0};
        rc = launch("state_scan", s, [&] { la::launch_scan(sc, lam, s); });
        if (rc) return rc;
    }
    la::SweepArgs a{};
    a.a = q;
    a.b = k;
    a.c = v;
    a.out0 = out;
    a.slots = given ? given : slots;
    a.slots_transposed = given ? 1 : 0;
    a.kv_in = kv_in;
    a.kv_in_transposed = kv_in_t;
    a.kv_out = kv_out;
    a.N = N;
    a.L = p.L;
    a.D = static_cast<int>(D);
    a.Bk = Bk;
    a.H = H;
    a.chunks = p.chunks;
    a.pairs = pairs;
    a.phi = phi.kind;
    a.phi_mask = phi.sweep_mask;
    a.phi_grad = phi.grad;
    a.slot_k = p.agg_k;
    if (p.mfma && la::fwd_dma_supported(static_cast<int>(D), Bk, N) && !env_is("LA_FWD", "v1")) {
        const int waves = env_is("LA_FWD_WAVES", "8") ? 8 : 4;
        return launch(tag[0] == 'd' ? "dq_dma" : "fwd_dma", s, [&] { la::launch_fwd_dma(a, lam, waves, s); });
    }
    if (p.mfma && la::fwd_dma128_supported(static_cast<int>(D), Bk, N) && !env_is("LA_FWD", "v1"))
        return launch(tag[0] == 'd' ? "dq_dma128" : "fwd_dma128", s, [&] { la::launch_fwd_dma128(a, lam, s); });
    if (p.mfma && v1_ok)
        return launch(tag[0] == 'd' ? "dq_mfma" : "fwd_mfma", s, [&] { la::launch_fwd_mfma(a, lam, s); });
    return launch(tag[0] == 'd' ? "dq_generic" : "fwd_generic", s, [&] { la::launch_fwd_generic(a, lam, bf16, s); });
}

// ------------------------------------------------------------------ ragged batches
struct VarPlan {
    la::VarlenArgs v;
    int64_t T;               // tokens in the batch
    int64_t L;               // chunk length (multiple of Bk), the same for every sequence
    int64_t slots_per_head;  // sum over sequences of (chunks - 1)
};

// Validates the host offsets and builds the plan.  One chunk length for the
// whole batch.  With the longest pieces of work dispatched first, a sequence up
// to twice a compute unit's average share (T H / 256 tokens) is best left whole:
// splitting it would add a chunk-aggregate pass whose few long workgroups cost
// more than the imbalance.  Longer sequences are cut into chunks of that share.
// LA_VARLEN_L (a positive multiple of Bk) forces the length.
int make_varplan(const int64_t* offs, int64_t B, int64_t H, int64_t D, int32_t Bk, VarPlan* p) {
    if (!offs || B <= 0 || H <= 0 || D <= 0) return LA_EINVAL;
    if (B > la::kMaxVarlenSeqs || H > la::kMaxHeads) return LA_EUNSUPPORTED;
    if (offs[0] != 0) return LA_EINVAL;
    for (int64_t b = 0; b < B; ++b)
        if (offs[b + 1] < offs[b]) return LA_EINVAL;
    const int64_t T = offs[B];
    // 32-bit buffer offsets: every element offset of one (sequence, head) stays below 2^31 bytes
    if (T >= (int64_t(1) << 31) / (H * D * 2)) return LA_EUNSUPPORTED;
    constexpr int64_t kComputeUnits = 256;
    const int64_t share = std::max<int64_t>(kMinBlocksPerChunk * Bk, (T * H + kComputeUnits - 1) / kComputeUnits);
    int64_t n_max = 0;
    for (int64_t b = 0; b < B; ++b) n_max = std::max<int64_t>(n_max, offs[b + 1] - offs[b]);
    int64_t L = n_max <= 2 * share ? std::max<int64_t>(n_max, Bk) : share;
    const char* env = std::getenv("LA_VARLEN_L");
    if (env && std::atoll(env) > 0) L = std::atoll(env);
    L = (L + Bk - 1) / Bk * Bk;
    p->T = T;
    p->L = L;
    p->v.nseq = static_cast<int>(B);
    p->v.wp[0] = 0;
    for (int64_t b = 0; b < B; ++b) {
        const int64_t n = offs[b + 1] - offs[b];
        const int64_t C = std::max<int64_t>(1, (n + L - 1) / L);
        p->v.cu[b] = static_cast<int>(offs[b]);
        p->v.wp[b + 1] = p->v.wp[b] + static_cast<int>(C);
    }
    p->v.cu[B] = static_cast<int>(T);
    p->slots_per_head = p->v.wp[B] - B;
    // last chunks, longest first
    std::vector<int> ord(static_cast<size_t>(B));
    for (int b = 0; b < B; ++b) ord[b] = b;
    auto last_len = [&](int b) {
        return (offs[b + 1] - offs[b]) - static_cast<int64_t>(p->v.wp[b + 1] - p->v.wp[b] - 1) * L;
    };
    std::stable_sort(ord.begin(), ord.end(), [&](int x, int y) { return last_len(x) > last_len(y); });
    for (int j = 0; j < B; ++j) p->v.last_order[j] = static_cast<uint8_t>(ord[j]);
    return LA_OK;
}

size_t varlen_slot_bytes(const VarPlan& p, int64_t H, int64_t D) {
    return static_cast<size_t>(p.slots_per_head * H) * static_cast<size_t>(D * D) * sizeof(float);
}

}  // namespace

// ====================================================================== ABI
extern "C" {

int la_version(void) { return 10000; }

const char* la_strerror(int code) {
    switch (code) {
        case LA_OK: return "ok";
        case LA_EINVAL: return "invalid argument";
        case LA_EUNSUPPORTED: return "unsupported shape (D in {16,32,64,128}, Bk in {16,32,64,128,256}, H <= 256)";
        case LA_EALIGN: return "device pointer not 16-byte aligned";
        case LA_EWORKSPACE: return "workspace missing or too small";
        case LA_EHIP: {
            static thread_local char buf[320];
            std::snprintf(buf, sizeof(buf), "HIP error: %s", g_err);
            return buf;
        }
        case LA_ENODEV: return "no HIP device";
        default: return "unknown status";
    }
}

int la_plan(int64_t B, int64_t H, int64_t N, int64_t D, int32_t Bk, int32_t dtype, int32_t* chunks,
            int64_t* chunk_len, int32_t* agg_parts) {
    int64_t elems;
    const int rc = check_shape(B, H, N, D, Bk, dtype, &elems);
    if (rc) return rc;
    const Plan p = make_plan(B, H, N, D, Bk, dtype);
    if (chunks) *chunks = p.chunks;
    if (chunk_len) *chunk_len = p.L;
    if (agg_parts) *agg_parts = p.agg_k;
    return LA_OK;
}

size_t la_fwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int32_t Bk, int32_t dtype) {
    int64_t elems;
    if (check_shape(B, H, N, D, Bk, dtype, &elems) != LA_OK) return 0;
    const Plan p = make_plan(B, H, N, D, Bk, dtype);
    return fwd_slot_bytes(B * H, p, D);
}

size_t la_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int32_t Bk, int32_t dtype) {
    int64_t elems;
    if (check_shape(B, H, N, D, Bk, dtype, &elems) != LA_OK) return 0;
    const Plan p = make_plan(B, H, N, D, Bk, dtype);
    return 2 * round_up(fwd_slot_bytes(B * H, p, D));
}

int la_fwd(const void* Q, const void* K, const void* V, const float* lambda, int64_t B, int64_t H,
           int64_t N, int64_t D, int32_t Bk, int32_t dtype, int32_t phi, const float* kv_in, void* O,
           float* kv_out, void* ws, size_t ws_bytes, void* hip_stream) {
    int64_t elems;
    int rc = check_shape(B, H, N, D, Bk, dtype, &elems);
    if (rc) return rc;
    if (!valid_phi(phi)) return LA_EINVAL;
    if (!Q || !K || !V || !O) return LA_EINVAL;
    LamArgs lam;
    if ((rc = load_lambda(lambda, H, &lam))) return rc;
    for (const void* p : {Q, K, V, static_cast<const void*>(O), static_cast<const void*>(kv_in),
                          static_cast<const void*>(kv_out), static_cast<const void*>(ws)})
        if (p && !aligned16(p)) return LA_EALIGN;
    const size_t tb = static_cast<size_t>(elems) * (dtype == LA_BF16 ? 2 : 4);
    const size_t sb = static_cast<size_t>(B * H * D * D) * sizeof(float);
    const Plan p = make_plan(B, H, N, D, Bk, dtype);
    Bk = p.bk;  // the block the kernels step
    const size_t need = fwd_slot_bytes(B * H, p, D);
    if (need && (!ws || ws_bytes < need)) return LA_EWORKSPACE;
    const Range rq{Q, tb}, rk{K, tb}, rv{V, tb}, ro{O, tb}, rin{kv_in, kv_in ? sb : 0},
        rout{kv_out, kv_out ? sb : 0}, rws{ws, need};
    for (const Range& r : {rq, rk, rv, rin})
        if (overlap(ro, r) || overlap(rout, r) || overlap(rws, r)) return LA_EINVAL;
    if (overlap(ro, rout) || overlap(ro, rws) || overlap(rout, rws)) return LA_EINVAL;

    int dev_count = 0;
    if (hipGetDeviceCount(&dev_count) != hipSuccess || dev_count == 0) return LA_ENODEV;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const PhiUse pu{phi, 3, 1, nullptr};  // phi(q), phi(k); the aggregates map k
    return run_forward_sweep(Q, K, V, O, kv_in, 0, kv_out, static_cast<float*>(ws), nullptr, B * H, N, D,
                             Bk, static_cast<int32_t>(H), dtype == LA_BF16, p, lam, pu, s, "fwd");
}

int la_bwd(const void* Q, const void* K, const void* V, const void* dO, const float* lambda, int64_t B,
           int64_t H, int64_t N, int64_t D, int32_t Bk, int32_t dtype, int32_t phi, const float* kv_in,
           const float* dkv_out, void* dQ, void* dK, void* dV, float* dkv_in, const void* fwd_ws, void* ws,
           size_t ws_bytes, void* hip_stream) {
    int64_t elems;
    int rc = check_shape(B, H, N, D, Bk, dtype, &elems);
    if (rc) return rc;
    if (!valid_phi(phi)) return LA_EINVAL;
    if (!Q || !K || !V || !dO || !dQ || !dK || !dV) return LA_EINVAL;
    LamArgs lam;
    if ((rc = load_lambda(lambda, H, &lam))) return rc;
    for (const void* p : {Q, K, V, dO, static_cast<const void*>(kv_in), static_cast<const void*>(dkv_out),
                          static_cast<const void*>(dQ), static_cast<const void*>(dK), static_cast<const void*>(dV),
                          static_cast<const void*>(dkv_in), fwd_ws, static_cast<const void*>(ws)})
        if (p && !aligned16(p)) return LA_EALIGN;
    const size_t tb = static_cast<size_t>(elems) * (dtype == LA_BF16 ? 2 : 4);
    const size_t sb = static_cast<size_t>(B * H * D * D) * sizeof(float);
    const Plan p = make_plan(B, H, N, D, Bk, dtype);
    Bk = p.bk;  // the block the kernels step
    // chunk states of the dQ sweep (forward direction) and of the dK, dV sweep (reverse
    // direction), both over agg_k parts per chunk boundary
    const size_t fq = fwd_slot_bytes(B * H, p, D), rv = fq;
    const size_t need = round_up(fq) + round_up(rv);
    if (need && (!ws || ws_bytes < need)) return LA_EWORKSPACE;
    const Range ins[] = {{Q, tb}, {K, tb}, {V, tb}, {dO, tb}, {kv_in, kv_in ? sb : 0},
                         {dkv_out, dkv_out ? sb : 0}, {fwd_ws, fwd_ws ? fq : 0}};
    const Range outs[] = {{dQ, tb}, {dK, tb}, {dV, tb}, {dkv_in, dkv_in ? sb : 0}, {ws, need}};
    constexpr int kOuts = sizeof(outs) / sizeof(outs[0]);
    for (const Range& o : outs)
        for (const Range& i : ins)
            if (overlap(o, i)) return LA_EINVAL;
    for (int a = 0; a < kOuts; ++a)
        for (int b = a + 1; b < kOuts; ++b)
            if (overlap(outs[a], outs[b])) return LA_EINVAL;

    int dev_count = 0;
    if (hipGetDeviceCount(&dev_count) != hipSuccess || dev_count == 0) return LA_ENODEV;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    float* slots_q = fq ? static_cast<float*>(ws) : nullptr;
    float* slots_kv = rv ? reinterpret_cast<float*>(static_cast<char*>(ws) + round_up(fq)) : nullptr;
    const int bf16 = dtype == LA_BF16;
    const int64_t pairs = B * H;
    const int32_t Hi = static_cast<int32_t>(H);

    // dQ: the forward sweep with (q, k, v) = (dO, V, K) and the transposed initial state.
    // the dQ sweep: phi(k) in the value slot, its own aggregates over (v, phi(k)), and
    // phi'(q) on the output
    const PhiUse pu{phi, 4, 2, phi ? Q : nullptr};
    rc = run_forward_sweep(dO, V, K, dQ, kv_in, 1, nullptr, slots_q, static_cast<const float*>(fwd_ws), pairs,
                           N, D, Bk, Hi, bf16, p, lam, pu, s, "dq");
    if (rc) return rc;

    // dK, dV: reverse sweep carrying dS, with a chunked suffix over blocks; the aggregates
    // are taken over the agg_k parts of every chunk but the first (a part past the end of
    // the sequence aggregates nothing)
    if (p.chunks > 1) {
        const int64_t Lf = p.L / p.agg_k;
        const int chunks_f = (p.chunks - 1) * p.agg_k + 1;
        la::ChunkStateArgs cs{Q, dO, slots_kv, N, Lf, static_cast<int>(D), Bk, Hi, chunks_f, pairs, 1,
                              phi, 1, p.agg_k - 1};
        if (p.mfma && la::state_dma_supported(static_cast<int>(D), Bk, N) && !env_is("LA_STATE", "v1"))
            rc = launch("chunk_state_rev_dma", s, [&] { la::launch_chunk_state_dma(cs, lam, s); });
        else if (p.mfma && phi == 0)
            rc = launch("chunk_state_rev_mfma", s, [&] { la::launch_chunk_state_mfma(cs, lam, s); });
        else
            rc = launch("chunk_state_rev_generic", s, [&] { la::launch_chunk_state_generic(cs, lam, bf16, s); });
        if (rc) return rc;
        la::ScanArgs sc{slots_kv, nullptr, 0, dkv_out, N, Lf, static_cast<int>(D), Hi, chunks_f, pairs, 1,
                        p.agg_k - 1};
        rc = launch("state_scan_rev", s, [&] { la::launch_scan(sc, lam, s); });
        if (rc) return rc;
    }
    la::SweepArgs a{};
    a.a = Q;
    a.b = K;
    a.c = V;
    a.g = dO;
    a.out0 = dK;
    a.out1 = dV;
    a.slots = slots_kv;
    a.g_final = dkv_out;
    a.ds_out = dkv_in;
    a.phi = phi;
    a.phi_mask = 3;
    a.slot_k = p.agg_k;
    a.N = N;
    a.L = p.L;
    a.D = static_cast<int>(D);
    a.Bk = Bk;
    a.H = Hi;
    a.chunks = p.chunks;
    a.pairs = pairs;
    if (p.mfma && la::rev_dma_supported(static_cast<int>(D), Bk, N) && !env_is("LA_REV", "v1"))
    {
        // the feature map is in the eight-wave form only
        const int waves = (env_is("LA_REV_WAVES", "4") && phi == 0) ? 4 : 8;
        return launch("dkdv_dma", s, [&] { la::launch_rev_dma(a, lam, waves, s); });
    }
    if (p.mfma && phi == 0 && la::mfma_rev_supported(static_cast<int>(D), Bk))
        return launch("dkdv_mfma", s, [&] { la::launch_rev_mfma(a, lam, s); });
    return launch("dkdv_generic", s, [&] { la::launch_rev_generic(a, lam, bf16, s); });
}

size_t la_dlam_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int32_t Bk, int32_t dtype) {
    int64_t elems;
    if (check_shape(B, H, N, D, Bk, dtype, &elems) != LA_OK) return 0;
    return dlam_ws_bytes(B * H, make_plan(B, H, N, D, Bk, dtype), D);
}

int la_dlam(const void* Q, const void* K, const void* V, const void* dO, const float* lambda, int64_t B,
            int64_t H, int64_t N, int64_t D, int32_t Bk, int32_t dtype, int32_t phi, const float* kv_in,
            const float* dkv_out, float* dlam, void* ws, size_t ws_bytes, void* hip_stream) {
    int64_t elems;
    int rc = check_shape(B, H, N, D, Bk, dtype, &elems);
    if (rc) return rc;
    if (!valid_phi(phi)) return LA_EINVAL;
    if (!Q || !K || !V || !dO || !dlam) return LA_EINVAL;
    LamArgs lam;
    if ((rc = load_lambda(lambda, H, &lam))) return rc;
    for (const void* p : {Q, K, V, dO, static_cast<const void*>(kv_in), static_cast<const void*>(dkv_out),
                          static_cast<const void*>(ws)})
        if (p && !aligned16(p)) return LA_EALIGN;
    if ((reinterpret_cast<uintptr_t>(dlam) & 3u) != 0) return LA_EALIGN;
    const size_t tb = static_cast<size_t>(elems) * (dtype == LA_BF16 ? 2 : 4);
    const size_t sb = static_cast<size_t>(B * H * D * D) * sizeof(float);
    const Plan p = make_plan(B, H, N, D, Bk, dtype);
    Bk = p.bk;  // the block the kernels step
    const size_t need = dlam_ws_bytes(B * H, p, D);
    if (!ws || ws_bytes < need) return LA_EWORKSPACE;
    const Range ins[] = {{Q, tb}, {K, tb}, {V, tb}, {dO, tb}, {kv_in, kv_in ? sb : 0}, {dkv_out, dkv_out ? sb : 0}};
    const Range rout{dlam, static_cast<size_t>(H) * sizeof(float)}, rws{ws, need};
    for (const Range& i : ins)
        if (overlap(rout, i) || overlap(rws, i)) return LA_EINVAL;
    if (overlap(rout, rws)) return LA_EINVAL;

    int dev_count = 0;
    if (hipGetDeviceCount(&dev_count) != hipSuccess || dev_count == 0) return LA_ENODEV;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const int64_t pairs = B * H;
    const int32_t Hi = static_cast<int32_t>(H);
    const int bf16 = dtype == LA_BF16;
    const bool dma = p.mfma && la::dlam_dma_supported(static_cast<int>(D), Bk, N) && !env_is("LA_DLAM", "v1");
    const bool mfma = p.mfma && la::dlam_mfma_supported(static_cast<int>(D), Bk);
    float* slots = static_cast<float*>(ws);
    double* partial = reinterpret_cast<double*>(static_cast<char*>(ws) + round_up(2 * fwd_slot_bytes(pairs, p, D)));
    // the (S, T) aggregates and their scan run over the agg_k parts of every chunk but the last
    const int64_t Lf = p.L / p.agg_k;
    const int chunks_f = (p.chunks - 1) * p.agg_k + 1;
    if (p.chunks > 1) {
        la::ChunkStateArgs cs{K, V, slots, N, Lf, static_cast<int>(D), Bk, Hi, chunks_f, pairs, 0, phi, 1};
        if (dma)
            rc = launch("dlam_state_dma", s, [&] { la::launch_dlam_state_dma(cs, lam, s); });
        else if (mfma)
            rc = launch("dlam_state_mfma", s, [&] { la::launch_dlam_state_mfma(cs, lam, s); });
        else
            rc = launch("dlam_state_generic", s, [&] { la::launch_dlam_state_generic(cs, lam, bf16, s); });
        if (rc) return rc;
        la::ScanArgs sc{slots, kv_in, 0, nullptr, N, Lf, static_cast<int>(D), Hi, chunks_f, pairs, 0};
        rc = launch("dlam_scan", s, [&] { la::launch_dlam_scan(sc, lam, s); });
        if (rc) return rc;
    }
    la::DlamArgs da{Q, K, V, dO, p.chunks > 1 ? slots : nullptr, kv_in, dkv_out, partial, N, p.L,
                    static_cast<int>(D), Bk, Hi, p.chunks, pairs, phi, p.agg_k};
    if (dma)
        rc = launch("dlam_dma", s, [&] { la::launch_dlam_dma(da, lam, env_is("LA_DLAM_WAVES", "4") ? 4 : 8, s); });
    else if (mfma)
        rc = launch("dlam_mfma", s, [&] { la::launch_dlam_mfma(da, lam, s); });
    else
        rc = launch("dlam_generic", s, [&] { la::launch_dlam_generic(da, lam, bf16, s); });
    if (rc) return rc;
    return launch("dlam_reduce", s, [&] { la::launch_dlam_reduce(partial, B, Hi, p.chunks, dlam, s); });
}

size_t la_fwd_varlen_workspace_bytes(const int64_t* seq_offsets, int64_t B, int64_t H, int64_t D, int32_t Bk,
                                     int32_t dtype) {
    if (dtype != LA_BF16 || D != 128 || Bk != 64) return 0;
    VarPlan p;
    if (make_varplan(seq_offsets, B, H, D, Bk, &p) != LA_OK) return 0;
    return varlen_slot_bytes(p, H, D);
}

int la_fwd_varlen(const void* Q, const void* K, const void* V, const float* lambda, const int64_t* seq_offsets,
                  int64_t B, int64_t H, int64_t D, int32_t Bk, int32_t dtype, int32_t phi, const float* kv_in,
                  void* O, float* kv_out, void* ws, size_t ws_bytes, void* hip_stream) {
    if (dtype != LA_F32 && dtype != LA_BF16) return LA_EINVAL;
    if (!valid_phi(phi)) return LA_EINVAL;
    VarPlan p;
    int rc = make_varplan(seq_offsets, B, H, D, Bk, &p);
    if (rc) return rc;
    if (dtype != LA_BF16 || D != 128 || Bk != 64) return LA_EUNSUPPORTED;
    if (p.T > 0 && (!Q || !K || !V || !O)) return LA_EINVAL;
    LamArgs lam;
    if ((rc = load_lambda(lambda, H, &lam))) return rc;
    for (const void* ptr : {Q, K, V, static_cast<const void*>(O), static_cast<const void*>(kv_in),
                            static_cast<const void*>(kv_out), static_cast<const void*>(ws)})
        if (ptr && !aligned16(ptr)) return LA_EALIGN;
    const size_t tb = static_cast<size_t>(p.T * H * D) * 2;
    const size_t sb = static_cast<size_t>(B * H * D * D) * sizeof(float);
    const size_t need = varlen_slot_bytes(p, H, D);
    if (need && (!ws || ws_bytes < need)) return LA_EWORKSPACE;
    const Range rq{Q, tb}, rk{K, tb}, rv{V, tb}, ro{O, tb}, rin{kv_in, kv_in ? sb : 0},
        rout{kv_out, kv_out ? sb : 0}, rws{ws, need};
    for (const Range& r : {rq, rk, rv, rin})
        if (overlap(ro, r) || overlap(rout, r) || overlap(rws, r)) return LA_EINVAL;
    if (overlap(ro, rout) || overlap(ro, rws) || overlap(rout, rws)) return LA_EINVAL;

    int dev_count = 0;
    if (hipGetDeviceCount(&dev_count) != hipSuccess || dev_count == 0) return LA_ENODEV;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const int32_t Hi = static_cast<int32_t>(H);
    float* slots = static_cast<float*>(ws);
    if (p.slots_per_head > 0) {
        la::ChunkStateArgs cs{K, V, slots, 0, p.L, static_cast<int>(D), Bk, Hi, 0, 0, 0, phi, 1};
        rc = launch("chunk_state_varlen_dma", s, [&] { la::launch_chunk_state_dma_varlen(cs, lam, p.v, s); });
        if (rc) return rc;
        la::ScanArgs sc{slots, kv_in, 0, nullptr, 0, p.L, static_cast<int>(D), Hi, 0, 0, 0};
        la::ScanList list;
        list.count = 0;
        for (int b = 0; b < p.v.nseq; ++b) {
            const int n_slots = p.v.wp[b + 1] - p.v.wp[b] - 1;
            if (n_slots > 0) {
                list.seq[list.count] = b | (n_slots << 8);
                list.sbase[list.count] = p.v.wp[b] - b;
                ++list.count;
            }
        }
        rc = launch("state_scan_varlen", s, [&] { la::launch_scan_varlen(sc, lam, list, s); });
        if (rc) return rc;
    }
    la::SweepArgs a{};
    a.a = Q;
    a.b = K;
    a.c = V;
    a.out0 = O;
    a.slots = slots;
    a.kv_in = kv_in;
    a.kv_out = kv_out;
    a.L = p.L;
    a.D = static_cast<int>(D);
    a.Bk = Bk;
    a.H = Hi;
    a.phi = phi;
    a.phi_mask = 3;
    return launch("fwd_varlen_dma", s, [&] { la::launch_fwd_dma_varlen(a, lam, p.v, s); });
}

int la_decode_step_paged(float* pool, int64_t pool_slots, const int32_t* slot_of, const void* q, const void* k,
                         const void* v, const float* lambda, int64_t Bs, int64_t H, int64_t D, int32_t dtype,
                         int32_t phi, void* o, void* hip_stream) {
    if (dtype != LA_F32 && dtype != LA_BF16) return LA_EINVAL;
    if (!valid_phi(phi)) return LA_EINVAL;
    if (Bs <= 0 || H <= 0 || D <= 0 || pool_slots <= 0) return LA_EINVAL;
    if (!supported_D(D) || H > la::kMaxHeads) return LA_EUNSUPPORTED;
    if (!pool || !slot_of || !q || !k || !v || !o) return LA_EINVAL;
    LamArgs lam;
    int rc = load_lambda(lambda, H, &lam);
    if (rc) return rc;
    for (const void* ptr : {static_cast<const void*>(pool), static_cast<const void*>(slot_of), q, k, v,
                            static_cast<const void*>(o)})
        if (!aligned16(ptr)) return LA_EALIGN;
    int64_t pairs, pool_pairs;
    if (!mul_ok(Bs, H, &pairs) || pairs > (int64_t(1) << 31)) return LA_EINVAL;
    if (!mul_ok(pool_slots, H, &pool_pairs) || pool_pairs > (int64_t(1) << 31)) return LA_EINVAL;
    const size_t vb = static_cast<size_t>(pairs * D) * (dtype == LA_BF16 ? 2 : 4);
    const size_t pb = static_cast<size_t>(pool_pairs * D * D) * sizeof(float);
    const Range rp{pool, pb}, ro{o, vb}, ridx{slot_of, static_cast<size_t>(Bs) * sizeof(int32_t)};
    for (const Range& r : {Range{q, vb}, Range{k, vb}, Range{v, vb}, ridx})
        if (overlap(rp, r) || overlap(ro, r)) return LA_EINVAL;
    if (overlap(rp, ro)) return LA_EINVAL;

    int dev_count = 0;
    if (hipGetDeviceCount(&dev_count) != hipSuccess || dev_count == 0) return LA_ENODEV;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    la::DecodeArgs a{pool, q, k, v, o, static_cast<int>(D), static_cast<int>(H), pairs, slot_of, pool_slots, phi};
    return launch("decode_paged", s, [&] { la::launch_decode(a, lam, dtype == LA_BF16, s); });
}

int la_decode_step(float* state, const void* q, const void* k, const void* v, const float* lambda,
                   int64_t Bs, int64_t H, int64_t D, int32_t dtype, int32_t phi, void* o, void* hip_stream) {
    if (dtype != LA_F32 && dtype != LA_BF16) return LA_EINVAL;
    if (!valid_phi(phi)) return LA_EINVAL;
    if (Bs <= 0 || H <= 0 || D <= 0) return LA_EINVAL;
    if (!supported_D(D) || H > la::kMaxHeads) return LA_EUNSUPPORTED;
    if (!state || !q || !k || !v || !o) return LA_EINVAL;
    LamArgs lam;
    int rc = load_lambda(lambda, H, &lam);
    if (rc) return rc;
    for (const void* p : {static_cast<const void*>(state), q, k, v, static_cast<const void*>(o)})
        if (!aligned16(p)) return LA_EALIGN;
    int64_t pairs;
    if (!mul_ok(Bs, H, &pairs) || pairs > (int64_t(1) << 31)) return LA_EINVAL;
    const size_t vb = static_cast<size_t>(pairs * D) * (dtype == LA_BF16 ? 2 : 4);
    const size_t sb = static_cast<size_t>(pairs * D * D) * sizeof(float);
    const Range rs{state, sb}, ro{o, vb};
    for (const Range& r : {Range{q, vb}, Range{k, vb}, Range{v, vb}})
        if (overlap(rs, r) || overlap(ro, r)) return LA_EINVAL;
    if (overlap(rs, ro)) return LA_EINVAL;

    int dev_count = 0;
    if (hipGetDeviceCount(&dev_count) != hipSuccess || dev_count == 0) return LA_ENODEV;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    la::DecodeArgs a{state, q, k, v, o, static_cast<int>(D), static_cast<int>(H), pairs, nullptr, 0, phi};
    return launch("decode", s, [&] { la::launch_decode(a, lam, dtype == LA_BF16, s); });
}

int la_prof_enable(int on) {
    g_prof_on.store(on ? 1 : 0);
    return LA_OK;
}

int la_prof_collect(la_prof_entry* out, int max_entries) {
    std::vector<ProfRec> recs;
    {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        recs.swap(g_prof);
    }
    std::vector<la_prof_entry> acc;
    int rc = LA_OK;
    for (const ProfRec& r : recs) {
        float ms = 0.f;
        hipError_t e = hipEventSynchronize(r.stop);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
        if (e != hipSuccess) rc = hip_fail(e, "la_prof_collect");
        (void)hipEventDestroy(r.start);
        (void)hipEventDestroy(r.stop);
        auto it = std::find_if(acc.begin(), acc.end(),
                               [&](const la_prof_entry& x) { return std::strcmp(x.name, r.name) == 0; });
        if (it == acc.end()) {
            la_prof_entry x{};
            std::snprintf(x.name, sizeof(x.name), "%s", r.name);
            acc.push_back(x);
            it = acc.end() - 1;
        }
        it->launches += 1;
        it->total_ms += ms;
    }
    if (rc) return -rc;
    const int n = std::min<int>(max_entries, static_cast<int>(acc.size()));
    for (int i = 0; i < n; ++i) out[i] = acc[i];
    return n;
}

}  // extern "C"
