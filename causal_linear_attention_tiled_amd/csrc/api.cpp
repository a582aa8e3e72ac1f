// Host side of liblinattn: argument validation, the chunk plan, kernel
// dispatch and optional per-kernel profiling.  See include/liblinattn.h for
// the contract of every exported call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <limits>
#include <atomic>
#include <chrono>
#include <random>
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

// Target workgroup count for the chunk plan: one per compute unit (256 on an
// MI355X; queried from the current device, 256 when none answers).  The sweep
// kernels hold one workgroup per CU (their LDS rings), so that many workgroups run
// in one round; measured, two rounds of half-length chunks are slower (B4 H16
// N2048 forward 72 us against 55 us; B2 H32 N8192 forward and backward 559 us
// against 497 us) and the long-sequence points are unchanged.
constexpr int64_t kDefaultComputeUnits = 256;
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

int64_t compute_units() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return kDefaultComputeUnits;
    }
    int n = g_cus[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
            (void)hipGetLastError();
            return kDefaultComputeUnits;
        }
        g_cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// A launch of W workgroups of up to 1024 threads keeps W * 1024 below 2^32, the
// limit on the threads of one grid dimension; larger calls are rejected before
// anything is enqueued.
constexpr int64_t kMaxWorkgroups = ((int64_t(1) << 32) - 1) / 1024;
// A chunk should span at least this many blocks, so the per-chunk state
// traffic (a few D x D float32 matrices) stays small next to its tokens.
constexpr int64_t kMinBlocksPerChunk = 4;
// The fixed cost of a round of aggregate workgroups, in tokens of one workgroup's stream
// (the chunk plan's cost model).
constexpr int64_t kRoundFill = 896;

thread_local char g_err[256];

int hip_fail(hipError_t e, const char* where) {
    std::snprintf(g_err, sizeof(g_err), "%s: %s", where, hipGetErrorString(e));
    return LA_EHIP;
}

// ------------------------------------------------------------------ profiling
// While alive on a thread, launches on that thread record no profiling events
// (la_fwd_noalloc creates no HIP objects).
thread_local bool g_no_events = false;
struct NoEventsGuard {
    bool prev;
    explicit NoEventsGuard(bool on) : prev(g_no_events) { g_no_events = g_no_events || on; }
    ~NoEventsGuard() { g_no_events = prev; }
};

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
    const bool prof = g_prof_on.load(std::memory_order_relaxed) != 0 && !g_no_events;
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

// ------------------------------------------------------------------ static scratch
// Device memory for la_fwd_noalloc, the entry point for callers that cannot
// allocate (HIP graph capture, serving loops, harnesses that forbid hipMalloc):
// its chunk states go here instead of a caller workspace.  Every device holds its
// own copy of the array, at its own address, until the process ends; the host
// name `scratch` is only a stand-in, so host code uses the address
// hipGetSymbolAddress returns for the current device, fetched once per device.
// Every call on a device shares the array: calls that overlap in time on one
// device race.  Nothing in it needs to start at zero (the aggregates and the
// scan write every chunk state before the sweep reads it).
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return LA_EUNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress");
        if (!p) return hip_fail(hipErrorInvalidSymbol, "hipGetSymbolAddress");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
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
    } else if (pairs < compute_units()) {
        const int64_t target = compute_units();
        C = (target + pairs - 1) / pairs;
        C = std::min<int64_t>(C, std::max<int64_t>(1, nb / kMinBlocksPerChunk));
    }
    C = std::max<int64_t>(1, std::min<int64_t>(C, nb));
    const int64_t bpc = (nb + C - 1) / C;
    p.L = bpc * Bk;
    p.chunks = static_cast<int>((nb + bpc - 1) / bpc);
    p.bk = std::min(Bk, kMaxKernelBk);
    p.mfma = dtype == LA_BF16 && la::mfma_supported(static_cast<int>(D), p.bk) && !force_generic();
    // The chunk aggregates are taken over agg_k equal parts of every chunk; the scans then
    // run over the parts, chunk c of a forward sweep starts from part c * agg_k - 1 and
    // chunk c of a reverse sweep from the gradient entering part (c + 1) agg_k.  The
    // aggregate kernels hold one workgroup per CU, so the W = (chunks - 1) agg_k pairs
    // workgroups run in rounds of CUs.  A round costs its part length plus kRoundFill tokens
    // (its launch, pipeline fill and drain, and the spread of its workgroups' finishing
    // times), scaled by max(1, its workgroups / (7/8 CUs)): about 7/8 of the CUs streaming
    // already saturate HBM, fewer leave the round bound by one workgroup's rate.  agg_k
    // minimises the summed cost (the smallest on a tie, for the fewest scan steps), each part
    // keeping at least kMinBlocksPerChunk blocks.  Measured, every choice of this rule the
    // fastest measured: ms of the forward aggregates, B8 H16 N16384 0.104 at 2 parts (0.111
    // at 4), B2 H16 N65536 0.163 at 1 (0.177 at 2), B1 H64 N262144 1.108 at 4 (1.179 at 1,
    // 1.278 at 2), B4 H16 N2048 0.0147 at 1 (0.0184 at 2), B2 H32 N8192 0.039 at 1; and ms
    // of la_fwd + la_bwd at B2 H32 (4 chunks), 1 part against 4: N40960 2.30 against 2.33,
    // N81920 4.56 against 4.54, N163840 9.44 against 9.31 (the fill of 256 tokens assumed
    // before switched to 4 parts at chunks of 7K tokens, 900 at 15K, between these two
    // measured crossings).  Parts need a chunk of a whole number of parts: where the blocks per chunk
    // do not divide by k, the chunks grow to the next multiple of k blocks if the chunk count
    // stays the same (the last chunk takes what is left), and the cost adds the sweep's
    // longer chunks at twice an aggregate token (a sweep streams four tensors, an aggregate
    // two).  LA_AGG_K forces k (when such a chunk length exists).
    p.agg_k = 1;
    if (p.chunks > 1) {
        // blocks per chunk with k parts, or 0 where rounding up would change the chunk count
        auto blocks_for = [&](int64_t k) -> int64_t {
            const int64_t b = (bpc + k - 1) / k * k;
            return (nb + b - 1) / b == p.chunks ? b : 0;
        };
        int64_t best_b = bpc;
        const char* ek = std::getenv("LA_AGG_K");
        if (ek && std::atoll(ek) > 0) {
            const int64_t k = std::atoll(ek);
            if (const int64_t b = blocks_for(k)) {
                p.agg_k = static_cast<int>(k);
                best_b = b;
            }
        } else {
            const int64_t cus = compute_units();
            const double sat = 0.875 * static_cast<double>(cus);
            auto cost = [&](int64_t k, int64_t b) {
                const int64_t w = (p.chunks - 1) * k * pairs;
                const double part = static_cast<double>(b / k * Bk + kRoundFill);
                const double full = static_cast<double>(w / cus), rem = static_cast<double>(w % cus);
                return part * (full * std::max(1.0, static_cast<double>(cus) / sat) +
                               (rem > 0 ? std::max(1.0, rem / sat) : 0.0)) +
                       2.0 * static_cast<double>((b - bpc) * Bk);
            };
            double best = cost(1, bpc);
            for (int64_t k = 2; k <= 16; k *= 2) {
                const int64_t b = blocks_for(k);
                if (!b) continue;
                if (b / k < kMinBlocksPerChunk) break;
                const double c = cost(k, b);
                if (c < best - 1e-12) {
                    best = c;
                    best_b = b;
                    p.agg_k = static_cast<int>(k);
                }
            }
        }
        p.L = best_b * Bk;
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

// la_fwd's workspace, each region from a 256-byte boundary: the chunk states; the
// per-chunk aggregates and their flags of the fused prefix; the stamp.
constexpr size_t kStampBytes = 256;
struct FwdWs {
    size_t slots, aggs, flags, stamp, total;  // offsets, and the size
};
FwdWs fwd_ws_layout(int64_t pairs, const Plan& p, int64_t D) {
    FwdWs l{};
    const size_t slots = fwd_slot_bytes(pairs, p, D);
    if (!slots) return l;
    const size_t chunk_states = static_cast<size_t>(pairs) * static_cast<size_t>(p.chunks - 1);
    l.aggs = round_up(slots);
    l.flags = l.aggs + round_up(chunk_states * static_cast<size_t>(D * D) * sizeof(float));
    l.stamp = l.flags + round_up(chunk_states * 4 * sizeof(uint64_t));
    l.total = l.stamp + kStampBytes;
    return l;
}
size_t fwd_ws_bytes(int64_t pairs, const Plan& p, int64_t D) { return fwd_ws_layout(pairs, p, D).total; }

// Epochs of fused launches: distinct for every launch of the process (its flags hold the
// epoch of the launch that set them), starting from a value no earlier process is likely
// to have left in reused memory.
std::atomic<uint64_t> g_epoch{0};
uint64_t next_epoch() {
    uint64_t e = g_epoch.load(std::memory_order_relaxed);
    if (e == 0) {
        std::random_device rd;
        const uint64_t seed = (static_cast<uint64_t>(rd()) << 32) ^ rd() ^
                              static_cast<uint64_t>(std::chrono::steady_clock::now().time_since_epoch().count());
        uint64_t expected = 0;
        g_epoch.compare_exchange_strong(expected, seed | 1);
    }
    uint64_t v;
    do {
        v = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
    } while (v == 0);
    return v;
}

// True when work enqueued on `s` now is being captured into a graph (a graph replays its
// kernels with the arguments of the capture, so a fused launch's epoch would repeat).
bool capturing(hipStream_t s) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &st) != hipSuccess) {
        (void)hipGetLastError();
        return true;
    }
    return st != hipStreamCaptureStatusNone;
}

uint32_t fnv1a(uint32_t h, const void* data, size_t n) {
    const unsigned char* b = static_cast<const unsigned char*>(data);
    for (size_t i = 0; i < n; ++i) h = (h ^ b[i]) * 16777619u;
    return h;
}

// What identifies the chunk states of one forward pass: shape, block size, dtype, feature
// map, chunk plan, decay values and the addresses of Q, K, V and kv_in.
la::Stamp make_stamp(int64_t B, int64_t H, int64_t N, int64_t D, int32_t Bk, int32_t dtype, int32_t phi,
                     const Plan& p, const LamArgs& lam, const void* Q, const void* K, const void* V,
                     const float* kv_in) {
    la::Stamp st{};
    st.w[0] = 0x4c414653u;  // "LAFS"
    st.w[1] = static_cast<uint32_t>(N) ^ static_cast<uint32_t>(N >> 32);
    st.w[2] = static_cast<uint32_t>(B * H) ^ static_cast<uint32_t>((B * H) >> 32) ^ (static_cast<uint32_t>(H) << 20);
    st.w[3] = static_cast<uint32_t>(D) | (static_cast<uint32_t>(Bk) << 8) | (static_cast<uint32_t>(dtype) << 20) |
              (static_cast<uint32_t>(phi) << 24);
    st.w[4] = static_cast<uint32_t>(p.chunks) | (static_cast<uint32_t>(p.agg_k) << 24);
    st.w[5] = static_cast<uint32_t>(p.L) ^ static_cast<uint32_t>(p.L >> 32);
    st.w[6] = fnv1a(2166136261u, lam.lam, sizeof(float) * static_cast<size_t>(H));
    const void* ptrs[4] = {Q, K, V, kv_in};
    st.w[7] = fnv1a(2166136261u, ptrs, sizeof(ptrs));
    return st;
}

// The fused chunked prefix (k_fwd_dma_fused: aggregates, their sum and the sweep in one
// launch) pays off while a chunk has few earlier chunks to sum and is short enough that the
// launches it saves count; LA_FUSED=0 / 1 switches it off / on for every plan.  Measured
// (us of la_fwd, one aggregate part, fused against three launches): B4 H16 N2048 (512-token
// chunks) 48 against 53, B4 H16 N4096 (1024) 80 against 81, B2 H32 N8192 (2048) 152
// against 154; B2 H32 N12288 (3072) 240-257 against 238, N20480 (5120) 385 against 374,
// N40960 (10240) 744-752 against 737.
constexpr int kMaxFusedChunks = 4;
constexpr int64_t kMaxFusedChunkLen = 2048;
// The fused sweep's bound on each wait, in polls of at least 128 cycles (a sleep and a load):
// a base of 2^17 polls (several ms) plus 4096 polls (over 200 us) per 64-token block of the
// awaited chunk's walk, so a wait gives up only when that walk runs about a hundred times
// slower than a block's measured 1.5 us, whatever the chunk length.  Plans without aggregate
// parts can have long chunks (an odd number of blocks per chunk admits no parts), whose walk
// takes tens of ms.  LA_FUSED_SPIN lowers the bound for failure-path tests.
constexpr int64_t kFusedSpinBase = int64_t(1) << 17;
constexpr int64_t kFusedSpinPerBlock = 4096;

int fused_spin_limit(const Plan& p) {
    const int64_t blocks = (p.L + 63) / 64;
    return static_cast<int>(std::min<int64_t>(std::numeric_limits<int>::max(),
                                              kFusedSpinBase + kFusedSpinPerBlock * blocks));
}

bool fused_wanted(const Plan& p) {
    if (env_is("LA_FUSED", "0")) return false;
    if (env_is("LA_FUSED", "1")) return true;
    // measured faster only with few, short chunks and no aggregate parts (the fused form
    // walks each chunk whole, and every chunk sums all earlier aggregates)
    return p.chunks <= kMaxFusedChunks && p.L <= kMaxFusedChunkLen && p.agg_k == 1;
}

// LA_TRACE=1: every call prints its plan to stderr (one line).
void trace_plan(const char* call, int64_t B, int64_t H, int64_t N, int64_t D, int32_t Bk, int32_t dtype,
                const Plan& p, size_t ws_bytes) {
    const char* e = std::getenv("LA_TRACE");
    if (!e || std::strcmp(e, "1") != 0) return;
    const int64_t pairs = B * H;
    const int64_t agg_wgs = p.chunks > 1 ? pairs * (p.chunks - 1) * p.agg_k : 0;
    std::fprintf(stderr,
                 "[liblinattn] %s B=%lld H=%lld N=%lld D=%lld %s Bk=%d (stepped %d) kernels=%s chunks=%d "
                 "chunk_len=%lld agg_parts=%d sweep_wgs=%lld aggregate_wgs=%lld cus=%lld workspace=%zu "
                 "fused=%d fused_spin=%d\n",
                 call, static_cast<long long>(B), static_cast<long long>(H), static_cast<long long>(N),
                 static_cast<long long>(D), dtype == LA_BF16 ? "bf16" : "f32", Bk,
                 p.mfma ? ((p.bk == 128 && env_is("LA_FWD128", "1")) ? 128 : 64) : p.bk,
                 p.mfma ? "mfma" : "generic", p.chunks, static_cast<long long>(p.L), p.agg_k,
                 static_cast<long long>(pairs * p.chunks), static_cast<long long>(agg_wgs),
                 static_cast<long long>(compute_units()), ws_bytes, p.chunks > 1 && fused_wanted(p) ? 1 : 0,
                 fused_spin_limit(p));
}

// Largest workgroup count any launch of a chunked call makes: the sweeps (one per
// sequence and chunk), the aggregates (agg_k per chunk boundary) and the scans
// (D * D / 256 per sequence).
bool plan_grid_ok(int64_t pairs, const Plan& p, int64_t D) {
    const int64_t per = std::max<int64_t>({static_cast<int64_t>(p.chunks),
                                           static_cast<int64_t>(p.chunks - 1) * p.agg_k,
                                           p.chunks > 1 ? (D * D + 255) / 256 : 1});
    return pairs <= kMaxWorkgroups / per;
}

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

// `stamp_out` (forward pass): where the scan (or the fused sweep) stores `stamp` after the
// chunk states; `stamp_in` (dQ sweep fed `given`): the stamp stored after those states,
// checked against `stamp`.  `fused_aggs` / `fused_flags`: workspace for the fused chunked
// prefix, or nullptr for the three-launch form.
int run_forward_sweep(const void* q, const void* k, const void* v, void* out, const float* kv_in,
                      int kv_in_t, float* kv_out, float* slots, const float* given, int64_t pairs,
                      int64_t N, int64_t D, int32_t Bk, int32_t H, int bf16, const Plan& p,
                      const LamArgs& lam, const PhiUse& phi, hipStream_t s, const char* tag,
                      uint32_t* stamp_out, const uint32_t* stamp_in, const la::Stamp& stamp,
                      float* fused_aggs = nullptr, uint64_t* fused_flags = nullptr) {
    int rc;
    // the register-staged kernels have no feature map: with one, the generic kernels run
    const bool v1_ok = phi.kind == 0;
    // A 128-token block is stepped as two 64-token blocks by the 64-token kernel: the same
    // function (the block size only decides which terms pass through a score tile and which
    // through the carried state), the same bytes, and on this GPU the faster sweep (its LDS
    // ring holds two 64-token blocks of look-ahead, where the 128-token kernel holds half a
    // block).  The chunk boundaries stay on multiples of 128.  LA_FWD128=1 selects the
    // 128-token kernel.
    const bool step128 = Bk == 128 && env_is("LA_FWD128", "1");
    const int32_t sweep_bk = (Bk == 128 && !step128) ? 64 : Bk;
    const bool dma = p.mfma && la::fwd_dma_supported(static_cast<int>(D), sweep_bk, N) && !env_is("LA_FWD", "v1");
    const int waves = env_is("LA_FWD_WAVES", "8") ? 8 : 4;
    const bool fused = fused_flags && p.chunks > 1 && !given && dma && waves == 4 && fused_wanted(p) && !capturing(s);
    if (p.chunks > 1 && !given && !fused) {
        // aggregates and scan over the agg_k parts of every chunk but the last
        const int64_t Lf = p.L / p.agg_k;
        const int chunks_f = (p.chunks - 1) * p.agg_k + 1;
        la::ChunkStateArgs cs{k, v, slots, N, Lf, static_cast<int>(D), Bk, H, chunks_f, pairs, 0,
                              phi.kind, phi.state_mask};
        if (p.mfma && la::state_dma_supported(static_cast<int>(D), Bk, N) && !env_is("LA_STATE", "v1"))
            rc = launch("chunk_state_dma", s,
                        [&] { la::launch_chunk_state_dma(cs, lam, !env_is("LA_STATE", "dma2"), s); });
        else if (p.mfma && v1_ok)
            rc = launch("chunk_state_mfma", s, [&] { la::launch_chunk_state_mfma(cs, lam, s); });
        else
            rc = launch("chunk_state_generic", s, [&] { la::launch_chunk_state_generic(cs, lam, bf16, s); });
        if (rc) return rc;
        la::ScanArgs sc{slots, kv_in, kv_in_t, nullptr, N, Lf, static_cast<int>(D), H, chunks_f, pairs, 0, 0,
                        p.agg_k};
        sc.stamp_out = stamp_out;
        sc.stamp = stamp;
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
    a.stamp = given ? stamp_in : nullptr;
    a.expect = stamp;
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
    if (fused) {
        a.fused_aggs = fused_aggs;
        a.fused_flags = fused_flags;
        a.epoch = next_epoch();
        // LA_FUSED_LOSE_FLAGS=1 (failure-path tests): waiting waves look for a value no wave
        // publishes, so every wait runs out (LA_FUSED_SPIN polls) and its columns become NaN
        a.wait_epoch = env_is("LA_FUSED_LOSE_FLAGS", "1") ? ~a.epoch : a.epoch;
        a.spin_limit = fused_spin_limit(p);
        if (const char* e = std::getenv("LA_FUSED_SPIN"); e && std::atoi(e) > 0)
            a.spin_limit = std::min(std::atoi(e), a.spin_limit);
        a.stamp_store = stamp_out;
    }
    if (dma) {
        a.Bk = sweep_bk;
        return launch(fused ? (tag[0] == 'd' ? "dq_dma_fused" : "fwd_dma_fused") : (tag[0] == 'd' ? "dq_dma" : "fwd_dma"),
                      s, [&] { la::launch_fwd_dma(a, lam, waves, s); });
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
    const int64_t cus = compute_units();
    const int64_t share = std::max<int64_t>(kMinBlocksPerChunk * Bk, (T * H + cus - 1) / cus);
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
    if (static_cast<int64_t>(p->v.wp[B]) * H > kMaxWorkgroups) return LA_EUNSUPPORTED;
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

// la_fwd and la_fwd_noalloc: the same validation and kernels; with use_scratch
// the chunk states go to the library's static scratch array instead of `ws`.
int fwd_entry(const void* Q, const void* K, const void* V, const float* lambda, int64_t B, int64_t H,
              int64_t N, int64_t D, int32_t Bk, int32_t dtype, int32_t phi, const float* kv_in, void* O,
              float* kv_out, void* ws, size_t ws_bytes, bool use_scratch, void* hip_stream) {
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
    if (!plan_grid_ok(B * H, p, D)) return LA_EUNSUPPORTED;
    const int32_t Bk_call = Bk;  // as asked (the stamp records it)
    Bk = p.bk;  // the block the kernels step
    // the static scratch holds the chunk states (and the fused prefix's aggregates and
    // flags when they fit); a caller workspace also the stamp
    const FwdWs lay = fwd_ws_layout(B * H, p, D);
    const size_t need = use_scratch ? fwd_slot_bytes(B * H, p, D) : lay.total;
    if (use_scratch) {
        if (need > kScratchBytes) return LA_ESCRATCH;
    } else if (need && (!ws || ws_bytes < need)) {
        return LA_EWORKSPACE;
    }
    trace_plan(use_scratch ? "la_fwd_noalloc" : "la_fwd", B, H, N, D, Bk_call, dtype, p, need);
    const Range rq{Q, tb}, rk{K, tb}, rv{V, tb}, ro{O, tb}, rin{kv_in, kv_in ? sb : 0},
        rout{kv_out, kv_out ? sb : 0}, rws{ws, need};
    for (const Range& r : {rq, rk, rv, rin})
        if (overlap(ro, r) || overlap(rout, r) || overlap(rws, r)) return LA_EINVAL;
    if (overlap(ro, rout) || overlap(ro, rws) || overlap(rout, rws)) return LA_EINVAL;

    int dev_count = 0;
    if (hipGetDeviceCount(&dev_count) != hipSuccess || dev_count == 0) return LA_ENODEV;
    if (use_scratch && need && (rc = scratch_address(&ws))) return rc;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const PhiUse pu{phi, 3, 1, nullptr};  // phi(q), phi(k); the aggregates map k
    const NoEventsGuard quiet(use_scratch);
    char* wsb = static_cast<char*>(ws);
    uint32_t* stamp_out = (!use_scratch && need) ? reinterpret_cast<uint32_t*>(wsb + lay.stamp) : nullptr;
    const bool fused_room = need && (!use_scratch || lay.stamp <= kScratchBytes);
    float* fused_aggs = fused_room ? reinterpret_cast<float*>(wsb + lay.aggs) : nullptr;
    uint64_t* fused_flags = fused_room ? reinterpret_cast<uint64_t*>(wsb + lay.flags) : nullptr;
    const la::Stamp stamp = make_stamp(B, H, N, D, Bk_call, dtype, phi, p, lam, Q, K, V, kv_in);
    return run_forward_sweep(Q, K, V, O, kv_in, 0, kv_out, static_cast<float*>(ws), nullptr, B * H, N, D,
                             Bk, static_cast<int32_t>(H), dtype == LA_BF16, p, lam, pu, s, "fwd", stamp_out,
                             nullptr, stamp, fused_aggs, fused_flags);
}

// A ragged batch is launched in groups of at most kMaxVarlenSeqs sequences (the batch table
// travels in the kernel arguments); each group has its own plan, with offsets rebased to its
// first token, and its own slice of the workspace.
struct VarGroup {
    int64_t b0, nb;    // first sequence, sequences
    int64_t t0;        // first token
    VarPlan plan;
    size_t ws_off, ws_bytes;
};

int varlen_groups(const int64_t* offs, int64_t B, int64_t H, int64_t D, int32_t Bk, std::vector<VarGroup>* out) {
    if (!offs || B <= 0 || H <= 0 || D <= 0) return LA_EINVAL;
    if (H > la::kMaxHeads) return LA_EUNSUPPORTED;
    if (offs[0] != 0) return LA_EINVAL;
    for (int64_t b = 0; b < B; ++b)
        if (offs[b + 1] < offs[b]) return LA_EINVAL;
    size_t off = 0;
    for (int64_t b0 = 0; b0 < B; b0 += la::kMaxVarlenSeqs) {
        VarGroup g;
        g.b0 = b0;
        g.nb = std::min<int64_t>(la::kMaxVarlenSeqs, B - b0);
        g.t0 = offs[b0];
        std::vector<int64_t> rel(static_cast<size_t>(g.nb + 1));
        for (int64_t i = 0; i <= g.nb; ++i) rel[static_cast<size_t>(i)] = offs[b0 + i] - g.t0;
        const int rc = make_varplan(rel.data(), g.nb, H, D, Bk, &g.plan);
        if (rc) return rc;
        g.ws_off = off;
        g.ws_bytes = round_up(varlen_slot_bytes(g.plan, H, D));
        off += g.ws_bytes;
        out->push_back(g);
    }
    return LA_OK;
}

bool varlen_supported(int32_t dtype, int64_t D, int32_t Bk) {
    return dtype == LA_BF16 && D == 128 && (Bk == 64 || Bk == 128 || Bk == 256);
}

// The ragged forward for every shape the direct-to-LDS kernels do not take (float32
// storage, D != 128, Bk of 16 or 32): the generic kernels, one workgroup per (sequence,
// head) over the whole sequence, in groups of kMaxVarlenSeqs sequences.  No chunks, so no
// workspace.
int fwd_varlen_generic(const void* Q, const void* K, const void* V, const float* lambda, const int64_t* offs,
                       int64_t B, int64_t H, int64_t D, int32_t Bk, int32_t dtype, int32_t phi,
                       const float* kv_in, void* O, float* kv_out, void* hip_stream) {
    if (!offs || B <= 0 || H <= 0 || D <= 0) return LA_EINVAL;
    if (offs[0] != 0) return LA_EINVAL;
    for (int64_t b = 0; b < B; ++b)
        if (offs[b + 1] < offs[b]) return LA_EINVAL;
    if (!supported_D(D) || !supported_Bk(Bk) || H > la::kMaxHeads) return LA_EUNSUPPORTED;
    const int64_t T = offs[B];
    if (T >= (int64_t(1) << 31)) return LA_EUNSUPPORTED;  // token offsets travel as int32
    if (T > 0 && (!Q || !K || !V || !O)) return LA_EINVAL;
    LamArgs lam;
    int rc = load_lambda(lambda, H, &lam);
    if (rc) return rc;
    for (const void* ptr : {Q, K, V, static_cast<const void*>(O), static_cast<const void*>(kv_in),
                            static_cast<const void*>(kv_out)})
        if (ptr && !aligned16(ptr)) return LA_EALIGN;
    const size_t esize = dtype == LA_BF16 ? 2 : 4;
    int64_t elems = 0, spairs = 0;
    if (!mul_ok(T, H * D, &elems) || !mul_ok(B, H, &spairs)) return LA_EINVAL;
    const size_t tb = static_cast<size_t>(elems) * esize;
    const size_t sb = static_cast<size_t>(spairs) * static_cast<size_t>(D * D) * sizeof(float);
    const Range rq{Q, tb}, rk{K, tb}, rv{V, tb}, ro{O, tb}, rin{kv_in, kv_in ? sb : 0},
        rout{kv_out, kv_out ? sb : 0};
    for (const Range& r : {rq, rk, rv, rin})
        if (overlap(ro, r) || overlap(rout, r)) return LA_EINVAL;
    if (overlap(ro, rout)) return LA_EINVAL;

    int dev_count = 0;
    if (hipGetDeviceCount(&dev_count) != hipSuccess || dev_count == 0) return LA_ENODEV;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    for (int64_t b0 = 0; b0 < B; b0 += la::kMaxVarlenSeqs) {
        const int64_t nb = std::min<int64_t>(la::kMaxVarlenSeqs, B - b0);
        const int64_t t0 = offs[b0];
        if (offs[b0 + nb] == t0 && !kv_out) continue;  // nothing to read or write
        la::VarlenArgs v{};
        v.nseq = static_cast<int>(nb);
        for (int64_t i = 0; i <= nb; ++i) v.cu[i] = static_cast<int>(offs[b0 + i] - t0);
        const size_t tok = static_cast<size_t>(t0 * H * D) * esize;
        la::SweepArgs a{};
        a.a = static_cast<const char*>(Q) + tok;
        a.b = static_cast<const char*>(K) + tok;
        a.c = static_cast<const char*>(V) + tok;
        a.out0 = static_cast<char*>(O) + tok;
        a.kv_in = kv_in ? kv_in + b0 * H * D * D : nullptr;
        a.kv_out = kv_out ? kv_out + b0 * H * D * D : nullptr;
        a.D = static_cast<int>(D);
        a.Bk = std::min(Bk, kMaxKernelBk);  // the same function at any block size; no chunks here
        a.H = static_cast<int32_t>(H);
        a.phi = phi;
        a.phi_mask = 3;
        if ((rc = launch("fwd_varlen_generic", s,
                         [&] { la::launch_fwd_generic_varlen(a, lam, v, dtype == LA_BF16, s); })))
            return rc;
    }
    return LA_OK;
}

// LA_TRACE=1: the plan of one group of a ragged batch.
void trace_varlen(int64_t nb, int64_t H, const VarPlan& p) {
    const char* e = std::getenv("LA_TRACE");
    if (!e || std::strcmp(e, "1") != 0) return;
    std::fprintf(stderr,
                 "[liblinattn] la_fwd_varlen group of %lld sequences T=%lld H=%lld chunk_len=%lld sweep_wgs=%lld "
                 "chunk_states=%lld\n",
                 static_cast<long long>(nb), static_cast<long long>(p.T), static_cast<long long>(H),
                 static_cast<long long>(p.L), static_cast<long long>(p.v.wp[nb]) * H,
                 static_cast<long long>(p.slots_per_head * H));
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
        case LA_ESCRATCH: return "chunk states exceed the static scratch of la_fwd_noalloc (la_scratch_bytes)";
        default: return "unknown status";
    }
}

int la_plan(int64_t B, int64_t H, int64_t N, int64_t D, int32_t Bk, int32_t dtype, int32_t* chunks,
            int64_t* chunk_len, int32_t* agg_parts) {
    int64_t elems;
    const int rc = check_shape(B, H, N, D, Bk, dtype, &elems);
    if (rc) return rc;
    const Plan p = make_plan(B, H, N, D, Bk, dtype);
    trace_plan("la_plan", B, H, N, D, Bk, dtype, p, fwd_ws_bytes(B * H, p, D));
    if (chunks) *chunks = p.chunks;
    if (chunk_len) *chunk_len = p.L;
    if (agg_parts) *agg_parts = p.agg_k;
    return LA_OK;
}

size_t la_fwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int32_t Bk, int32_t dtype) {
    int64_t elems;
    if (check_shape(B, H, N, D, Bk, dtype, &elems) != LA_OK) return 0;
    const Plan p = make_plan(B, H, N, D, Bk, dtype);
    return fwd_ws_bytes(B * H, p, D);
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
    return fwd_entry(Q, K, V, lambda, B, H, N, D, Bk, dtype, phi, kv_in, O, kv_out, ws, ws_bytes, false,
                     hip_stream);
}

int la_fwd_noalloc(const void* Q, const void* K, const void* V, const float* lambda, int64_t B, int64_t H,
                   int64_t N, int64_t D, int32_t Bk, int32_t dtype, int32_t phi, const float* kv_in, void* O,
                   float* kv_out, void* hip_stream) {
    return fwd_entry(Q, K, V, lambda, B, H, N, D, Bk, dtype, phi, kv_in, O, kv_out, nullptr, 0, true,
                     hip_stream);
}

size_t la_scratch_bytes(void) { return kScratchBytes; }

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
    if (!plan_grid_ok(B * H, p, D)) return LA_EUNSUPPORTED;
    const la::Stamp stamp = make_stamp(B, H, N, D, Bk, dtype, phi, p, lam, Q, K, V, kv_in);
    const int32_t Bk_call = Bk;
    Bk = p.bk;  // the block the kernels step
    // chunk states of the dQ sweep (forward direction) and of the dK, dV sweep (reverse
    // direction), both over agg_k parts per chunk boundary
    const size_t fq = fwd_slot_bytes(B * H, p, D), rv = fq;
    const size_t need = round_up(fq) + round_up(rv);
    if (need && (!ws || ws_bytes < need)) return LA_EWORKSPACE;
    trace_plan("la_bwd", B, H, N, D, Bk_call, dtype, p, need);
    const Range ins[] = {{Q, tb}, {K, tb}, {V, tb}, {dO, tb}, {kv_in, kv_in ? sb : 0},
                         {dkv_out, dkv_out ? sb : 0}, {fwd_ws, fwd_ws ? fwd_ws_bytes(B * H, p, D) : 0}};
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

    // dK, dV: reverse sweep carrying dS, with a chunked suffix over blocks; the aggregates
    // are taken over the agg_k parts of every chunk but the first (a part past the end of
    // the sequence aggregates nothing).  They run first: they read Q and dO, so the dQ sweep
    // after them finds part of dO still in the infinity cache (measured, fwd + bwd with the
    // forward's chunk states: B2 H32 N8192 470 against 477 us with the dQ sweep first,
    // B8 H16 N16384 1.676 against 1.686 ms).
    if (p.chunks > 1) {
        const int64_t Lf = p.L / p.agg_k;
        const int chunks_f = (p.chunks - 1) * p.agg_k + 1;
        la::ChunkStateArgs cs{Q, dO, slots_kv, N, Lf, static_cast<int>(D), Bk, Hi, chunks_f, pairs, 1,
                              phi, 1, p.agg_k - 1};
        if (p.mfma && la::state_dma_supported(static_cast<int>(D), Bk, N) && !env_is("LA_STATE", "v1"))
            rc = launch("chunk_state_rev_dma", s,
                        [&] { la::launch_chunk_state_dma(cs, lam, !env_is("LA_STATE", "dma2"), s); });
        else if (p.mfma && phi == 0)
            rc = launch("chunk_state_rev_mfma", s, [&] { la::launch_chunk_state_mfma(cs, lam, s); });
        else
            rc = launch("chunk_state_rev_generic", s, [&] { la::launch_chunk_state_generic(cs, lam, bf16, s); });
        if (rc) return rc;
        la::ScanArgs sc{slots_kv, nullptr, 0, dkv_out, N, Lf, static_cast<int>(D), Hi, chunks_f, pairs, 1,
                        p.agg_k - 1, p.agg_k};
        rc = launch("state_scan_rev", s, [&] { la::launch_scan(sc, lam, s); });
        if (rc) return rc;
    }
    // dQ: the forward sweep with (q, k, v) = (dO, V, K) and the transposed initial state.
    // the dQ sweep: phi(k) in the value slot, its own aggregates over (v, phi(k)), and
    // phi'(q) on the output
    const PhiUse pu{phi, 4, 2, phi ? Q : nullptr};
    const uint32_t* stamp_in =
        (fwd_ws && fq) ? reinterpret_cast<const uint32_t*>(static_cast<const char*>(fwd_ws) + fwd_ws_layout(pairs, p, D).stamp)
                       : nullptr;
    rc = run_forward_sweep(dO, V, K, dQ, kv_in, 1, nullptr, slots_q, static_cast<const float*>(fwd_ws), pairs,
                           N, D, Bk, Hi, bf16, p, lam, pu, s, "dq", nullptr, stamp_in, stamp);
    if (rc) return rc;

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
    if (!plan_grid_ok(B * H, p, D)) return LA_EUNSUPPORTED;
    const int32_t Bk_call = Bk;
    Bk = p.bk;  // the block the kernels step
    const size_t need = dlam_ws_bytes(B * H, p, D);
    if (!ws || ws_bytes < need) return LA_EWORKSPACE;
    trace_plan("la_dlam", B, H, N, D, Bk_call, dtype, p, need);
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
    if (!varlen_supported(dtype, D, Bk)) return 0;
    std::vector<VarGroup> groups;
    if (varlen_groups(seq_offsets, B, H, D, Bk, &groups) != LA_OK) return 0;
    size_t total = 0;
    for (const VarGroup& g : groups) total += g.ws_bytes;
    // a batch whose only group needs no chunk states needs no workspace
    return total;
}

int la_fwd_varlen(const void* Q, const void* K, const void* V, const float* lambda, const int64_t* seq_offsets,
                  int64_t B, int64_t H, int64_t D, int32_t Bk, int32_t dtype, int32_t phi, const float* kv_in,
                  void* O, float* kv_out, void* ws, size_t ws_bytes, void* hip_stream) {
    if (dtype != LA_F32 && dtype != LA_BF16) return LA_EINVAL;
    if (!valid_phi(phi)) return LA_EINVAL;
    if (!varlen_supported(dtype, D, Bk))
        return fwd_varlen_generic(Q, K, V, lambda, seq_offsets, B, H, D, Bk, dtype, phi, kv_in, O, kv_out,
                                  hip_stream);
    std::vector<VarGroup> groups;
    int rc = varlen_groups(seq_offsets, B, H, D, Bk, &groups);
    if (rc) return rc;
    const int64_t T = seq_offsets[B];
    if (T > 0 && (!Q || !K || !V || !O)) return LA_EINVAL;
    LamArgs lam;
    if ((rc = load_lambda(lambda, H, &lam))) return rc;
    for (const void* ptr : {Q, K, V, static_cast<const void*>(O), static_cast<const void*>(kv_in),
                            static_cast<const void*>(kv_out), static_cast<const void*>(ws)})
        if (ptr && !aligned16(ptr)) return LA_EALIGN;
    int64_t wgs = 0;
    size_t need = 0;
    for (const VarGroup& g : groups) {
        wgs = std::max<int64_t>(wgs, static_cast<int64_t>(g.plan.v.wp[g.nb]) * H);
        need += g.ws_bytes;
    }
    if (wgs > kMaxWorkgroups) return LA_EUNSUPPORTED;
    if (need && (!ws || ws_bytes < need)) return LA_EWORKSPACE;
    const size_t tb = static_cast<size_t>(T * H * D) * 2;
    const size_t sb = static_cast<size_t>(B * H * D * D) * sizeof(float);
    const Range rq{Q, tb}, rk{K, tb}, rv{V, tb}, ro{O, tb}, rin{kv_in, kv_in ? sb : 0},
        rout{kv_out, kv_out ? sb : 0}, rws{ws, need};
    for (const Range& r : {rq, rk, rv, rin})
        if (overlap(ro, r) || overlap(rout, r) || overlap(rws, r)) return LA_EINVAL;
    if (overlap(ro, rout) || overlap(ro, rws) || overlap(rout, rws)) return LA_EINVAL;

    int dev_count = 0;
    if (hipGetDeviceCount(&dev_count) != hipSuccess || dev_count == 0) return LA_ENODEV;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const int32_t Hi = static_cast<int32_t>(H);
    for (const VarGroup& g : groups) {
        const VarPlan& p = g.plan;
        if (p.T == 0 && !kv_out) continue;  // nothing to read or write
        const int64_t tok = g.t0 * H * D;   // element offset of the group's first token
        const int64_t st = g.b0 * H * D * D;
        const void* Qg = static_cast<const uint16_t*>(Q) + tok;
        const void* Kg = static_cast<const uint16_t*>(K) + tok;
        const void* Vg = static_cast<const uint16_t*>(V) + tok;
        void* Og = static_cast<uint16_t*>(O) + tok;
        const float* kin = kv_in ? kv_in + st : nullptr;
        float* kout = kv_out ? kv_out + st : nullptr;
        float* slots = reinterpret_cast<float*>(static_cast<char*>(ws) + g.ws_off);
        trace_varlen(g.nb, H, p);
        if (p.slots_per_head > 0) {
            la::ChunkStateArgs cs{Kg, Vg, slots, 0, p.L, static_cast<int>(D), 64, Hi, 0, 0, 0, phi, 1};
            rc = launch("chunk_state_varlen_dma", s, [&] { la::launch_chunk_state_dma_varlen(cs, lam, p.v, s); });
            if (rc) return rc;
            la::ScanArgs sc{slots, kin, 0, nullptr, 0, p.L, static_cast<int>(D), Hi, 0, 0, 0};
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
        a.a = Qg;
        a.b = Kg;
        a.c = Vg;
        a.out0 = Og;
        a.slots = slots;
        a.kv_in = kin;
        a.kv_out = kout;
        a.L = p.L;
        a.D = static_cast<int>(D);
        a.Bk = 64;  // the kernels step 64-token blocks; the chunk length is a multiple of Bk
        a.H = Hi;
        a.phi = phi;
        a.phi_mask = 3;
        rc = launch("fwd_varlen_dma", s, [&] { la::launch_fwd_dma_varlen(a, lam, p.v, s); });
        if (rc) return rc;
    }
    return LA_OK;
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
    if (pairs > kMaxWorkgroups) return LA_EUNSUPPORTED;
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
    if (pairs > kMaxWorkgroups) return LA_EUNSUPPORTED;
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
