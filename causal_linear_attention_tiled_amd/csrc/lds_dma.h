// LDS helpers for the direct-to-LDS kernels (gfx950): swizzled row-major
// [rows][128] bf16 tiles, operand reads from them (plain and transposing),
// and exact vmcnt waits.
//
// Tiles are row-major with the 16-byte chunks of row r XOR-swizzled by
// (r mod 16): a row read by 16 lanes on consecutive rows and the transposing
// read below both spread over all banks.
//
// ds_read_b64_tr_b16: within each 16-lane group, output lane j element e is
// input lane j/4 + 4e element j%4.  Lanes i of group g reading rows
// kb + 4g + i/4 at columns n0 + 4(i%4) therefore deliver the B operand
// B[kb + kappa(g, e)][n0 + lane%16] of a row-major tile whose rows are the
// contraction index (see mfma_common.h for kappa).
#pragma once

#include "mfma_common.h"

namespace la {

constexpr int kTileCols = 128;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

// Element offset of (row, col) in a swizzled [rows][128] tile.
__device__ __forceinline__ int swz(int row, int col) {
    return row * kTileCols + ((((col >> 3) ^ (row & 15))) << 3) + (col & 7);
}

// kappa-ordered operand from row `row`, k columns [k0, k0 + 32) (row-major read).
__device__ __forceinline__ bf16x8 op_row(const uint16_t* t, int row, int k0, int g) {
    const u32x2 lo = *reinterpret_cast<const u32x2*>(t + swz(row, k0 + 4 * g));
    const u32x2 hi = *reinterpret_cast<const u32x2*>(t + swz(row, k0 + 16 + 4 * g));
    return operand(lo, hi);
}

// Operand B[kb + kappa(g, e)][n0 + li] of a row-major tile (rows = k), by two transposing reads.
__device__ __forceinline__ bf16x8 op_tr(const uint16_t* t, int kb, int n0, int g, int li) {
    const int r = kb + 4 * g + (li >> 2), col = n0 + 4 * (li & 3);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(t + swz(r, col)));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(t + swz(r + 16, col)));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const v8i16 v{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// Multiply the 8 bf16 of an operand by per-element weights, rounding back to bf16.
__device__ __forceinline__ bf16x8 scale8(const bf16x8& x, const float* wt) {
    const u32x4 u = __builtin_bit_cast(u32x4, x);
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r[i] = pack_bf16(__uint_as_float(u[i] << 16) * wt[2 * i], __uint_as_float(u[i] & 0xFFFF0000u) * wt[2 * i + 1]);
    return __builtin_bit_cast(bf16x8, r);
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Raw-buffer resource (gfx9 V#) for `bytes` bytes at `base`, built in SGPRs.
// Loads at offsets >= bytes return zero.
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return u32x4{static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a & 0xFFFFFFFFu))),
                 static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>((a >> 32) & 0xFFFFu))),
                 static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(bytes))), 0x00020000u};
}

// 16 bytes per lane from buffer offset `voff` straight into LDS at
// lds_dst + 16 * lane (buffer_load_dwordx4 ... lds).  Written as inline asm so
// the compiler does not track it (it would otherwise wait for it before every
// later LDS read): the caller must wait_vmcnt before the data is read.  The
// instruction writes no register.
__device__ __forceinline__ void dma16(const u32x4& rsrc, const void* lds_dst, int voff) {
    const uint32_t m0 = static_cast<uint32_t>(
        __builtin_amdgcn_readfirstlane(static_cast<int>(reinterpret_cast<uintptr_t>((lds_void*)lds_dst))));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

}  // namespace la
