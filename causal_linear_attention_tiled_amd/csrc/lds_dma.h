// LDS helpers for the direct-to-LDS kernels (gfx950): swizzled row-major
// [rows][128] bf16 tiles, operand reads from them (plain and transposing),
// and exact vmcnt waits.
//
// Operands here use the natural k order (lane group g holds k = 8g .. 8g + 7)
// for both MFMA operands, so that every row-major operand is one 16-byte
// read.  Tiles are row-major with 16-byte chunks XOR-swizzled per row.
//
// ds_read_b64_tr_b16: within each 16-lane group, output lane j element e is
// input lane j/4 + 4e element j%4.  If input lane i reads 4 elements at row
// R + i/4 and column C + s * (i%4), output lane j holds rows R .. R+3 at
// column C + s * (j/4) + j%4, i.e. one half of an operand whose contraction
// index runs over the tile's rows.
#pragma once

#include "la_device.h"
#include "mfma_common.h"

namespace la {

constexpr int kTileCols = 128;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

// Swizzle of row r: chunk c of the row is stored at position c ^ key(r mod 16),
// key = 0 2 4 6 8 10 12 14 9 11 13 15 1 3 5 7.  The gfx950 LDS has 64 banks of
// 4 bytes; a 16-byte read serves, per half-wave, the lanes whose bits 2..4 have
// even parity in one cycle and the odd ones in the next, an 8-byte read serves
// 32 consecutive lanes per cycle.  With this key
//   - a row read (16 rows, 16 bytes each, lane group g at chunk c + g) hits
//     distinct banks in each cycle, since the keys of rows {0-3, 12-15} are
//     closed under xor 1;
//   - a transposing read of stride 4 (8 consecutive rows, two adjacent chunks
//     each) is conflict-free, since key / 2 is distinct over rows 0-7 and over
//     rows 8-15;
//   - a transposing read of stride 8 (8 rows, one half of four chunks each) is
//     2-way, the least possible when 32 lanes read the same half of a chunk.
// The key repeats every 16 rows, so reads 16 or 32 rows apart share an address
// register and differ by an immediate offset.
__device__ __forceinline__ int swz_key(int row) { return ((row << 1) & 14) ^ (((row >> 3) & 1) * 9); }

// Element offset of (row, col) in a swizzled [rows][128] tile.
__device__ __forceinline__ int swz(int row, int col) {
    return row * kTileCols + (((col >> 3) ^ swz_key(row)) << 3) + (col & 7);
}

// Natural-order operand: the 8 bf16 at row `row`, columns k0 + 8g .. k0 + 8g + 7
// (one 16-byte read).
__device__ __forceinline__ bf16x8 op_row(const uint16_t* t, int row, int k0, int g) {
    return *reinterpret_cast<const bf16x8*>(t + swz(row, k0 + 8 * g));
}

// Operand from a row-major tile X whose rows are the contraction index, by two
// transposing reads, with the k index in the kappa order of mfma_common.h: lane
// (g, li) gets X[kb + kappa(g, e)][col(li)], e = 0..7, with
// col(li) = n0 + cstride * (li / 4) + li % 4.  cstride = 4 gives col = n0 + li;
// cstride = 8 gives the interleaved rows rho_t(li) (n0 = 32b + 4t) of a tile pair.
// kb is a multiple of 32.
__device__ __forceinline__ bf16x8 op_tr_k(const uint16_t* t, int kb, int n0, int cstride, int g, int li) {
    const int r = kb + 4 * g + (li >> 2), col = n0 + cstride * (li & 3);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(t + swz(r, col)));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(t + swz(r + 16, col)));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const v8i16 v{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// kappa(g, e): the token offset inside a 32-token k block held by lane group g, element e.
__device__ __forceinline__ constexpr int kappa(int g, int e) { return e < 4 ? 4 * g + e : 16 + 4 * g + e - 4; }

// Weights of tokens 32 kb + kappa(g, e) from a 16-byte aligned table by token:
// e = 0..3 (half 0) or e = 4..7 (half 1), each a run of four tokens.
__device__ __forceinline__ f32x4 lane_weights(const float* tab, int kb, int g, int half) {
    return *reinterpret_cast<const f32x4*>(tab + 32 * kb + 16 * half + 4 * g);
}

// Row of a 32-row block covered by row i of its tile t (0 or 1): the two tiles
// of a block interleave in runs of four, so that their accumulators stacked
// (tile 0 for e < 4, tile 1 for e >= 4) are a natural-order operand whose k
// index runs over the block's 32 rows.
__device__ __forceinline__ constexpr int rho(int t, int i) { return 8 * (i >> 2) + 4 * t + (i & 3); }

// Multiply the 8 bf16 of an operand by per-element weights, rounding back to bf16.
__device__ __forceinline__ bf16x8 scale8(const bf16x8& x, const float* wt) {
    const u32x4 u = __builtin_bit_cast(u32x4, x);
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r[i] = pack_bf16(__uint_as_float(u[i] << 16) * wt[2 * i], __uint_as_float(u[i] & 0xFFFF0000u) * wt[2 * i + 1]);
    return __builtin_bit_cast(bf16x8, r);
}

// The same products as a pair of operands, hi = bf16(x * wt) and lo = bf16(x * wt - hi):
// together they carry the weighted operand to about 16 significant bits.
__device__ __forceinline__ void scale8_split(const bf16x8& x, const float* wt, bf16x8& hi, bf16x8& lo) {
    const u32x4 u = __builtin_bit_cast(u32x4, x);
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a = __uint_as_float(u[i] << 16) * wt[2 * i];
        const float b = __uint_as_float(u[i] & 0xFFFF0000u) * wt[2 * i + 1];
        h[i] = pack_bf16(a, b);
        l[i] = pack_bf16(a - __uint_as_float(h[i] << 16), b - __uint_as_float(h[i] & 0xFFFF0000u));
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// Apply the feature map to every element of a [64][128] bf16 tile in LDS, in
// place, rounding to bf16; thread t of nthr takes 16-byte pieces t, t + nthr, ...
// (the swizzle does not matter to an elementwise map).
__device__ __forceinline__ void phi_tile(uint16_t* tile, int kind, int t, int nthr) {
    for (int c = t; c < 64 * kTileCols / 8; c += nthr) {
        u32x4* p = reinterpret_cast<u32x4*>(tile + 8 * c);
        const u32x4 u = *p;
        u32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r[i] = pack_bf16(phi_apply(__uint_as_float(u[i] << 16), kind),
                             phi_apply(__uint_as_float(u[i] & 0xFFFF0000u), kind));
        *p = r;
    }
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
