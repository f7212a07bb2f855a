// LDS tiles of 64 rows x 128 16-bit elements (bf16 or fp16, 256-byte rows):
// swizzled copies from global memory by buffer_load ... lds, and the
// transposed MFMA operand reads (ds_read_b64_tr_b16) that take a column of
// 8 rows per lane.  Shared by the forward pass (K and V tiles) and the
// pooling pass (the first-order moments).
#pragma once

#include "common.h"

namespace sa {

constexpr int ROWB = 256;                  // bytes per 128-element 16-bit row
constexpr int TILEB = BLK * ROWB;          // bytes per 64-row tile (16 KiB)
constexpr int HALFB = TILEB / 2;           // 32 rows (8 KiB)

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;

// Physical 16-byte chunk of logical chunk c (0..15) in LDS row `row`.  The
// XOR key is a bijection of row & 15, so 16 consecutive rows reading the same
// logical chunk (K reads) hit 16 different chunks, and rows 0-3 (or 8-11)
// reading 4 consecutive chunks (V^T transposed reads) hit 16 different chunks.
__device__ __forceinline__ int swz(int row, int c) { return c ^ (((row & 3) << 2) | ((row >> 2) & 3)); }

// s_waitcnt with vmcnt <= n (expcnt and lgkmcnt left open), gfx9 encoding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14));
}

// ---- swizzled copies of half tiles ----

// 8 x buffer_load_dwordx4 ... lds: rows 32hk .. 32hk+31 of one 64-row tile
// into a half buffer.  Instruction m fills half-buffer rows 4m .. 4m+3; lane l
// lands at row 4m + l/16, physical chunk l%16, so it fetches the logical
// chunk that the swizzle maps there.  row & 15 = 4(m & 3) + l/16, so four lane
// offsets cover the eight instructions; the tile offset is a scalar.
__device__ __forceinline__ void dma_offsets(uint32_t off[4]) {
    const int l = lane_id();
    const int rsub = l >> 4, p = l & 15;
#pragma unroll
    for (int par = 0; par < 4; ++par)
        off[par] = rsub * ROWB + 16 * swz(4 * par + rsub, p);   // swz is an involution per row
}

// Instruction M: the immediate offset (M % 4) KiB applies to both the global
// and the LDS address, so M0 (the LDS base) and the scalar source offset
// change once per 4 KiB instead of once per instruction.
template <int M>
__device__ __forceinline__ void dma_one(__amdgpu_buffer_rsrc_t rs, uint32_t lds, uint32_t src, const uint32_t off[4]) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, reinterpret_cast<lds_void*>(static_cast<uintptr_t>(lds + (M >> 2) * 4096)),
                                             16, off[M & 3], src + (M >> 2) * 4096, (M & 3) * 1024, 0);
}

__device__ __forceinline__ void dma_half(__amdgpu_buffer_rsrc_t rs, uint8_t* buf, uint32_t src,
                                         const uint32_t off[4]) {
    // the low 32 bits of a generic pointer into LDS are the LDS address (no
    // null-pointer select per instruction, as a generic -> LDS cast would emit)
    const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(buf));
    dma_one<0>(rs, lds, src, off);
    dma_one<1>(rs, lds, src, off);
    dma_one<2>(rs, lds, src, off);
    dma_one<3>(rs, lds, src, off);
    dma_one<4>(rs, lds, src, off);
    dma_one<5>(rs, lds, src, off);
    dma_one<6>(rs, lds, src, off);
    dma_one<7>(rs, lds, src, off);
}

// ---- transposed operand reads ----

// Column operands through ds_read_b64_tr_b16: within each 16-lane group,
// output lane i receives element i%4 of the 8-byte pieces addressed by lanes
// i/4 + 4e (e = 0..3).  Supplying lane r addresses row key0 + r/4 at
// d0 + 4(r%4), so output lane i gets rows key0 .. key0+3 of column d0 + i.
// One operand = rows 4h + r/4 (offset oa) and rows 8 + 4h + r/4 (offset ob)
// of a 16-row step, column 32 db + l % 32; the next step adds 16 rows, which
// keeps row & 15.
__device__ __forceinline__ void pv_offsets(uint32_t oa[4], uint32_t ob[4]) {
    const int l = lane_id();
    const int h = l >> 5, g2 = (l >> 4) & 1, r = l & 15;
    const int rsub = r >> 2, csub = r & 3;
    const int row0 = 4 * h + rsub, row1 = row0 + 8;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const int chunk = 4 * db + 2 * g2 + (csub >> 1);
        oa[db] = row0 * ROWB + 16 * swz(row0, chunk) + (csub & 1) * 8;
        ob[db] = row1 * ROWB + 16 * swz(row1, chunk) + (csub & 1) * 8;
    }
}

__device__ __forceinline__ f16x8 tr_read_pair(const uint8_t* pa, const uint8_t* pb) {
    // rows 16kk + 4h + e (slots 0..3) and 16kk + 8 + 4h + e (slots 4..7)
    const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pa));
    const i16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pb));
    const i16x8 v8 = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
    return __builtin_bit_cast(f16x8, v8);
}

}  // namespace sa
