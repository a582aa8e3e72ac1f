// Forward sweep, Bk = 64, D = 128, bf16: a three-stage LDS pipeline fed by
// direct global-to-LDS loads.
//
// Same arithmetic as the register-staged forward kernel (Lightning
// Attention-2, Tiling paragraph: per block the masked, decayed intra-block
// product plus the inter-block product with the carried state, then the
// state's decay and update), with a different data path:
//   - One extra "loader" wave issues buffer_load_dwordx4 ... lds for the raw
//     row-major Q, K, V tiles of the block two ahead of the one being
//     computed.  It never stores, so its vmcnt waits are exact, and it
//     hands each stage to the compute waves through the block's barriers.
//     Loads past the end of the sequence come back as zero (buffer bounds).
//   - Tiles stay row-major, with the 16-byte chunks of row r XOR-swizzled by
//     (r mod 16) so that both read patterns below are free of bank conflicts.
//   - Operands whose contraction runs over tokens (V^T for V^T A^T and for
//     the state update, decayed K^T for the state update) come straight from
//     the row-major tiles through ds_read_b64_tr_b16: within each 16-lane
//     group, output lane j element e is input lane j/4 + 4e element j%4, so
//     lanes reading rows kb+4g+i/4 at columns n0+4(i%4) deliver
//     B[kb + kappa(g, e)][n0 + lane%16].
// Compute waves: NW; wave w owns 128/NW value columns of the float32 state
// (MFMA accumulators) and of the output.
#include "la_device.h"
#include "la_internal.h"
#include "mfma_common.h"
#include "lds_dma.h"

namespace la {
namespace {

constexpr int D = 128;
constexpr int BK = 64;
constexpr int NT = BK / 16;
constexpr int NKS = BK / 32;
constexpr int NSTAGE = 3;
constexpr int TILE = BK * D;                // elements per tile
constexpr int NCAUSAL = NT * (NT + 1) / 2;
constexpr int DMA_PER_BLOCK = 3 * BK / 4;   // 1 KiB loads per block (4 rows of 256 B each)

struct DmaTiles {
    uint16_t t[NSTAGE][3][TILE];     // per stage: Q, K, V (row-major, swizzled)
    uint32_t at[NCAUSAL * 128];      // masked decayed score tiles, B-operand fragments
    float pw[BK + 1];
};

template <int NW>
__global__ __launch_bounds__(64 * (NW + 1), 1) void k_fwd_dma(SweepArgs a, LamArgs lam) {
    constexpr int NVT = 8 / NW;  // 16-column value tiles per compute wave
    __shared__ DmaTiles sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, li = lane & 15;
    const int64_t pair = blockIdx.x / a.chunks;
    const int c = blockIdx.x % a.chunks;
    const float lv = lam.lam[pair % a.H];
    const int64_t t_begin = static_cast<int64_t>(c) * a.L;
    const int64_t t_end = min(a.N, t_begin + a.L);
    const int64_t nblk = (t_end - t_begin + BK - 1) / BK;
    const int64_t base = pair * a.N * D;

    for (int e = tid; e <= BK; e += 64 * (NW + 1)) sm.pw[e] = lam_pow(lv, e);
    __syncthreads();  // decay table; every wave passes exactly 1 + 2 * nblk barriers

    if (w == NW) {
        // ------------------------------------------------------------ loader wave
        const int bytes = static_cast<int>(a.N * D * 2);
        __amdgpu_buffer_rsrc_t rs[3];
        rs[0] = __builtin_amdgcn_make_buffer_rsrc((void*)(static_cast<const uint16_t*>(a.a) + base), 0, bytes, 0x00020000);
        rs[1] = __builtin_amdgcn_make_buffer_rsrc((void*)(static_cast<const uint16_t*>(a.b) + base), 0, bytes, 0x00020000);
        rs[2] = __builtin_amdgcn_make_buffer_rsrc((void*)(static_cast<const uint16_t*>(a.c) + base), 0, bytes, 0x00020000);
        const int sub = lane >> 4, p = lane & 15;
        auto issue = [&](int64_t n) {
            const int stage = static_cast<int>(n % NSTAGE);
            const int64_t t0 = t_begin + n * BK;
#pragma unroll
            for (int x = 0; x < 3; ++x)
#pragma unroll
                for (int rg = 0; rg < BK / 4; ++rg) {
                    const int r = 4 * rg + sub;
                    const int chunk = p ^ (r & 15);
                    const int voff = static_cast<int>(((t0 + r) * D + 8 * chunk) * 2);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs[x], (lds_void*)&sm.t[stage][x][4 * rg * D], 16, voff, 0, 0, 0);
                }
        };
        issue(0);
        if (nblk > 1) issue(1);
        // The loader's own vmcnt wait makes its LDS writes complete before it
        // reaches A(n); a fenced __syncthreads() here would also wait for the
        // loads still in flight, so the loader uses the bare barrier.
        for (int64_t n = 0; n < nblk; ++n) {
            if (n + 1 < nblk)
                wait_vmcnt<DMA_PER_BLOCK>();
            else
                wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();  // A(n): stage n is ready; stage (n+2) % 3 is free
            if (n + 2 < nblk) issue(n + 2);
            __builtin_amdgcn_s_barrier();  // B(n)
        }
        return;
    }

    // ---------------------------------------------------------------- compute waves
    uint16_t* __restrict__ Og = static_cast<uint16_t*>(a.out0) + base;
    f32x4 S[8][NVT];
    {
        const float* init = nullptr;
        bool tr = false;
        if (c == 0) {
            if (a.kv_in) {
                init = a.kv_in + pair * D * D;
                tr = a.kv_in_transposed != 0;
            }
        } else {
            init = a.slots + (pair * (a.chunks - 1) + (c - 1)) * D * D;
        }
#pragma unroll
        for (int at = 0; at < 8; ++at)
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) {
                const int col = 16 * (NVT * w + vt) + li;
                f32x4 x = zero4();
                if (init) {
                    if (tr) {
                        const float4 t4 = *reinterpret_cast<const float4*>(init + col * D + 16 * at + 4 * g);
                        x = f32x4{t4.x, t4.y, t4.z, t4.w};
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) x[r] = init[(16 * at + 4 * g + r) * D + col];
                    }
                }
                S[at][vt] = x;
            }
    }

    float rs[NT];
#pragma unroll
    for (int st = 0; st < NT; ++st) rs[st] = sm.pw[16 * st + li + 1];
    // decay lam^(m-1-s) of the K operand rows s = 32 ks + kappa(g, e) of the state update
    float wk[NKS][8];
    auto set_wk = [&](int m) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int s = 32 * ks + (e < 4 ? 4 * g + e : 16 + 4 * g + e - 4);
                wk[ks][e] = s < m ? sm.pw[m - 1 - s] : 0.f;
            }
    };
    set_wk(BK);

    for (int64_t n = 0; n < nblk; ++n) {
        const int64_t t0 = t_begin + n * BK;
        const int m = static_cast<int>(min(static_cast<int64_t>(BK), t_end - t0));
        const int stage = static_cast<int>(n % NSTAGE);
        const uint16_t* Qs = sm.t[stage][0];
        const uint16_t* Ks = sm.t[stage][1];
        const uint16_t* Vs = sm.t[stage][2];
        if (m < BK) set_wk(m);
        __syncthreads();  // A(n)

        // ---- score tiles A^T = (K Q^T) o M^T, shared through LDS
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
                    p[r] *= d >= 0 ? sm.pw[d] : 0.f;
                }
                *reinterpret_cast<u32x2*>(&sm.at[idx * 128 + 2 * lane]) = u32x2{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])};
            }
        __syncthreads();  // B(n)

        // ---- V^T fragments (A operand of V^T A^T, B operand of the state update)
        bf16x8 vf[NVT][NKS];
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) vf[vt][ks] = op_tr(Vs, 32 * ks, 16 * (NVT * w + vt), g, li);
        bf16x8 sb[NVT][4];
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) sb[vt][ks] = operand_from_acc(S[2 * ks][vt], S[2 * ks + 1][vt]);

        // ---- per 16-token column: O^T = diag(lam^(s+1)) S^T Q^T + V^T A^T, store
#pragma unroll
        for (int st = 0; st < NT; ++st) {
            bf16x8 qf[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) qf[ks] = op_row(Qs, 16 * st + li, 32 * ks, g);
            f32x4 o[NVT];
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) {
                f32x4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) acc = mfma16(sb[vt][ks], qf[ks], acc);
                o[vt] = acc * rs[st];
            }
#pragma unroll
            for (int ks = 0; ks <= st / 2; ++ks) {
                const int a0 = 2 * ks, a1 = 2 * ks + 1;
                const u32x2 lo = *reinterpret_cast<const u32x2*>(&sm.at[(st * (st + 1) / 2 + a0) * 128 + 2 * lane]);
                u32x2 hi = u32x2{0, 0};
                if (a1 <= st) hi = *reinterpret_cast<const u32x2*>(&sm.at[(st * (st + 1) / 2 + a1) * 128 + 2 * lane]);
                const bf16x8 b = operand(lo, hi);
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt) o[vt] = mfma16(vf[vt][ks], b, o[vt]);
            }
            const int s = 16 * st + li;
            if (s < m) {
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt) {
                    uint16_t* dst = Og + (t0 + s) * D + 16 * (NVT * w + vt) + 4 * g;
                    *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16(o[vt][0], o[vt][1]), pack_bf16(o[vt][2], o[vt][3])};
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- S <- lam^m S + (diag(lam^(m-1-s)) K)^T V
        const float lm = sm.pw[m];
#pragma unroll
        for (int at = 0; at < 8; ++at) {
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) S[at][vt] *= lm;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8 kf = scale8(op_tr(Ks, 32 * ks, 16 * at, g, li), wk[ks]);
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt) S[at][vt] = mfma16(kf, vf[vt][ks], S[at][vt]);
            }
        }
    }

    if (a.kv_out && c == a.chunks - 1) {
        float* dst = a.kv_out + pair * D * D;
#pragma unroll
        for (int at = 0; at < 8; ++at)
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[(16 * at + 4 * g + r) * D + 16 * (NVT * w + vt) + li] = S[at][vt][r];
    }
}

}  // namespace

bool fwd_dma_supported(int d, int bk, int64_t n) {
    return d == 128 && bk == 64 && n * d * 2 < (int64_t(1) << 31);
}

void launch_fwd_dma(const SweepArgs& a, const LamArgs& lam, int waves, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(a.pairs * a.chunks));
    if (waves == 8)
        hipLaunchKernelGGL(k_fwd_dma<8>, grid, dim3(64 * 9), 0, s, a, lam);
    else
        hipLaunchKernelGGL(k_fwd_dma<4>, grid, dim3(64 * 5), 0, s, a, lam);
}

}  // namespace la
