// bf16 compensated block-sparse attention forward for gfx950 (d = 128).
//
// What it computes (per query t of query block a, one softmax):
//   exact key blocks E          e^{s q.k_n} (v_n)                    bf16 MFMA
//   every other key block j     n_j e^{s q.k_bar_j} (v_bar_j)         order 0
//                               + e^{s q.k_bar_j} s q^T H_j (N only)  order 1
//   all skipped blocks together  s (sum_j e^{s q.k_bar_j}) q^T H_bar     global order 1
// PISA ("PISA: Piecewise Sparse Attention Is Wiser for Efficient Diffusion
// Transformers", section 2, "Algorithme Central" and "Implementation
// Materielle": exact phase on selected blocks, then a scan of the block
// aggregates, then the first-order correction, all inside one
// FlashAttention-style online softmax); SVG-EAR's centroid compensation
// ("SVG-EAR ...", section 2A).
//
// Work split.  One wave owns a whole 64-row query block, so every K/V byte
// brought into LDS feeds 64 query rows.
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16; A = K rows from LDS
//                 (ds_read_b128), B = Q^T held in AGPRs through the exact
//                 and centroid phases (the skim tiles, last, reuse them).
//                 A lane owns one query row per 32-row block; its 16
//                 accumulator entries are 16 of the 32 keys of a half tile,
//                 the other 16 sit in lane l ^ 32.
//   O^T += V^T P^T  B = P^T straight from S's accumulators (rounded to bf16),
//                 A = V^T read from the row-major LDS copy of V with
//                 ds_read_b64_tr_b16 (4 consecutive keys of one d per read).
// The P^T operand's key order follows S's accumulator layout: within each
// 16-key MFMA step, slot s holds key s with bits 2 and 3 swapped; the V^T
// reads use the same order.
//
// Exact tiles run as a software pipeline over half tiles (32 keys).  Each
// tile is four MFMA regions of 16 MFMAs,
//   A: S(keys 0-31, tile i)      C: S(keys 32-63, tile i)
//   B: PV(keys 32-63, tile i-1)  D: PV(keys 0-31, tile i),
// run in the order A B C D, and the exponentials of one row block of a half
// (48-56 VALU instructions) are interleaved between the MFMAs of each region, so
// the VALU work of the softmax runs under the matrix core.  K and V halves
// have LDS buffers of their own, filled by buffer_load ... lds (no VGPRs, no
// VALU address arithmetic) as soon as the region that reads them is done;
// each copy has the rest of its region and the next two to land.
//
// Softmax reference.  P = 2^(c2 s - m) with a per-row reference m that only
// moves when a half tile's weights overflow a bound (sum of one lane's 16
// weights > 2^40; the first tile always does, from m = -1e30).  Then m
// becomes the ceiling of the row max over that half and the accumulators are
// rescaled; otherwise no row max is computed at all.  Any m keeps the bf16
// weights and the fp32 sums exact to rounding as long as nothing overflows,
// which the bound guarantees.  The denominator is the fp32 sum of the
// unrounded weights and lse is m + log2 of it (exact to fp32 rounding); the
// MFMA consumes P rounded to bf16, so o = N / D scales the exact convex
// combination by sum(bf16(p)) / sum(p), within 2^-8 (the bf16 unit roundoff)
// of 1.  The first-order Taylor forms (per-block H_j, global H_bar) instead
// sum the bf16-rounded pairs with v_dot2_f32_bf16, which cancels that rounding
// in o (lse then within 2^-8 relative of the unrounded sum): their H terms
// leave less of the bf16 error budget.  Only there, because on gfx950 each
// v_dot2 holds up the next MFMA issue (8 per 16 MFMAs cost ~60 cycles), while
// FMA, v_exp_f32 and v_cvt_pk_bf16_f32 run under the MFMAs almost for free.
//
// Centroid pseudo-keys go through the same MFMA path as 64-wide tiles (means
// split into bf16 high + low parts so the fp32 means keep ~16 bits), with
// bias log2(n_j) and -inf at the exact blocks, and a lazily updated max.
//
// Workgroup = one wave; consecutive query blocks of one head are mapped to
// the same XCD so their overlapping K/V blocks are shared through its L2.
#include "common.h"
#include "launch.h"

namespace sa {

namespace {

constexpr int D = 128;
constexpr int ROWB = D * 2;                // bytes per bf16 row
constexpr int TILEB = BLK * ROWB;          // bytes per 64-key bf16 tile (16 KiB)
constexpr int HALFB = TILEB / 2;           // 32 rows (8 KiB)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float M_INIT = -1.0e30f;         // "no reference yet" (finite: 2^(-inf - M_INIT) = 0)
constexpr float OVF = 1099511627776.0f;    // 2^40: per-lane half-tile weight sum that moves m
constexpr uint32_t RSRC_WORD3 = 0x00020000u;  // raw buffer descriptor, 32-bit data format (gfx9)

// Physical 16-byte chunk of logical chunk c (0..15) in LDS row `row`.  The
// XOR key is a bijection of row & 15, so 16 consecutive rows reading the same
// logical chunk (K reads) hit 16 different chunks, and rows 0-3 (or 8-11)
// reading 4 consecutive chunks (V^T transposed reads) hit 16 different chunks.
__device__ __forceinline__ int swz(int row, int c) { return c ^ (((row & 3) << 2) | ((row >> 2) & 3)); }

__device__ __forceinline__ int xcd_remap(int bid, int grid) {
    const int xcd = bid & 7, slot = bid >> 3;
    const int per = grid >> 3, extra = grid & 7;
    return xcd * per + min(xcd, extra) + slot;
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// s_waitcnt with vmcnt <= n (expcnt and lgkmcnt left open), gfx9 encoding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14));
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((address_space(4))) const int32_t const_i32;   // read through the scalar cache

// ---- LDS copies of K and V half tiles ----

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

// Zero half-buffer rows r0 .. 31 (pad keys of the ragged tail block).
__device__ __forceinline__ void zero_rows(uint8_t* buf, int r0) {
    const int l = lane_id();
    for (int x = r0 * 16 + l; x < 32 * 16; x += 64) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(buf + x * 16) = z;
    }
}

// ---- online softmax state ----

struct State {
    f32x16 o[4][2];        // O^T[d-block][row-block]
    float m[2];            // reference (log2 units, an integer) per row block
    float l[2];            // this lane's partial row sums of the bf16-rounded P
    float a1[2];           // global first order: partial sums of e^{s q.k_bar_j} 2^{-m} over skipped j
};

__device__ __forceinline__ void rescale_row(State& st, int rb, float mnew) {
    const float alpha = __builtin_amdgcn_exp2f(st.m[rb] - mnew);
    st.l[rb] *= alpha;
    st.a1[rb] *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.o[db][rb][r] *= alpha;
    st.m[rb] = mnew;
}

// Lazy max for the centroid and skim tiles: the reference moves up to
// ceil(tile max) only when a tile max exceeds it by more than 8 (log2 units).
__device__ __forceinline__ void rescale_lazy(State& st, int rb, float mx) {
    const bool need = st.m[rb] == M_INIT ? mx > -INFINITY : mx > st.m[rb] + 8.0f;
    if (__ballot(need)) {
        if (need) rescale_row(st, rb, ceilf(mx));
    }
}

// Sum of a bf16 pair in fp32 (v_dot2 with ones).
__device__ __forceinline__ float sum_bf16_pair(uint32_t pair, float acc) {
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), ones, acc, false);
}

// P = 2^(c2 s - m) for the 16 logits a lane holds in one row block of a
// 32-key half, as the two bf16 B operands of that half's PV k-steps
// (p0: accumulator entries 0-7, p1: 8-15), and the sum of the weights: of
// the bf16-rounded ones (RS) or of the fp32 ones.
// 16 FMA + 16 v_exp_f32 + 8 v_cvt_pk_bf16_f32 + 8 v_dot2 (RS) or 16 v_add.
template <bool RS>
__device__ __forceinline__ void exp_rb(const f32x16& s, float m, float c2, bf16x8& p0, bf16x8& p1, float& ls) {
    const float negm = -m;
    float acc = 0.f;
    u32x4 w0, w1;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const float x0 = __builtin_amdgcn_exp2f(fmaf(s[e], c2, negm));
        const float x1 = __builtin_amdgcn_exp2f(fmaf(s[e + 1], c2, negm));
        w0[e >> 1] = pack_bf16x2(x0, x1);
        if constexpr (RS) acc = sum_bf16_pair(w0[e >> 1], acc);
        else acc += x0 + x1;
    }
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const float x0 = __builtin_amdgcn_exp2f(fmaf(s[8 + e], c2, negm));
        const float x1 = __builtin_amdgcn_exp2f(fmaf(s[8 + e + 1], c2, negm));
        w1[e >> 1] = pack_bf16x2(x0, x1);
        if constexpr (RS) acc = sum_bf16_pair(w1[e >> 1], acc);
        else acc += x0 + x1;
    }
    p0 = __builtin_bit_cast(bf16x8, w0);
    p1 = __builtin_bit_cast(bf16x8, w1);
    ls = acc;
}

// After both row blocks of a half have their weights: if any lane's sum
// overflowed the bound (first tile, or a large logit), move the reference of
// the affected rows to the ceiling of their max over this half, rescale, and
// redo the weights.  Then fold the half's sums into the row sums.
template <bool RS>
__device__ __forceinline__ void settle_half(State& st, const f32x16 s[2], float c2, bf16x8 pb[2][2], float ls[2]) {
    if (__builtin_expect(__ballot(ls[0] > OVF || ls[1] > OVF) != 0, 0)) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            float mx = s[rb][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[rb][r]);
            mx = pair_max(mx) * c2;
            const bool need = pair_max(ls[rb]) > OVF;
            if (need) rescale_row(st, rb, ceilf(mx));
            exp_rb<RS>(s[rb], st.m[rb], c2, pb[0][rb], pb[1][rb], ls[rb]);
        }
    }
    st.l[0] += ls[0];
    st.l[1] += ls[1];
}

// Keys at or beyond nvalid (ragged tail block) drop out: logit -inf.
__device__ __forceinline__ void mask_half(f32x16 s[2], int key0, int nvalid) {
    const int h = lane_id() >> 5;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (key0 + 8 * (r >> 2) + 4 * h + (r & 3) >= nvalid) s[rb][r] = -INFINITY;
}

// ---- LDS operand offsets ----

// K A operands: ka(ks) = K[half row l32][16ks + 8h .. +7] of a half buffer.
__device__ __forceinline__ void k_offsets(uint32_t off[8]) {
    const int l = lane_id(), h = l >> 5, l32 = l & 31;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) off[ks] = l32 * ROWB + 16 * swz(l32, 2 * ks + h);
}

// V^T A operands through ds_read_b64_tr_b16: within each 16-lane group,
// output lane i receives element i%4 of the 8-byte pieces addressed by lanes
// i/4 + 4e (e = 0..3).  Supplying lane r addresses row key0 + r/4 at
// d0 + 4(r%4), so output lane i gets keys key0 .. key0+3 of column d0 + i.
// One operand = rows 4h + r/4 (offset oa) and rows 8 + 4h + r/4 (offset ob)
// of a 16-key step; the next k-step adds 16 rows, which keeps row & 15.
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

__device__ __forceinline__ bf16x8 tr_read_pair(const uint8_t* pa, const uint8_t* pb) {
    // keys 16kk + 4h + e (slots 0..3) and 16kk + 8 + 4h + e (slots 4..7)
    const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pa));
    const i16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pb));
    const i16x8 v8 = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
    return __builtin_bit_cast(bf16x8, v8);
}

// ---- the four MFMA regions of the exact-tile pipeline ----
//
// Each region issues 16 MFMAs; after each MFMA come up to four VALU instructions
// of the weights of one row block of the other pending half (48-56 in all), the
// LDS reads run two steps ahead, and the eight buffer_load ... lds of one
// half-tile copy (into the buffer the previous region finished reading) get
// one slot per MFMA pair (the M0 chain still lets the scheduler bunch most of
// them near the end of the region).  IGroupLP sched_group_barriers lay out
// that pattern; sched_barrier(0) on both sides keeps each region a
// scheduling unit of its own.

// group masks; transcendental VALU (v_exp_f32) has its own bit (0x400) and is
// not covered by the VALU bit
constexpr int SG_VALU = 0x002, SG_TRANS = 0x400, SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100;

// With the fp32 weight sum (RS false) the exponentials join the VALU groups,
// four instructions after each MFMA.  With the v_dot2 sum the groups take
// three plain VALU instructions and the scheduler places the exponentials,
// which measured faster with the dot2 stalls.
template <int READS_PER_STEP, bool EXP, bool COPY, bool RS>
__device__ __forceinline__ void region_schedule() {
    constexpr int VM = RS ? SG_VALU : (SG_VALU | SG_TRANS);
    constexpr int VN = RS ? 3 : 4;
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2 * READS_PER_STEP, 0);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        if (t < 6) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, READS_PER_STEP, 0);
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        if (EXP) __builtin_amdgcn_sched_group_barrier(VM, VN, 0);
        if (COPY) __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 1, 0);
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        if (EXP) __builtin_amdgcn_sched_group_barrier(VM, VN, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
}

// One half-tile copy issued inside a region.
struct Copy {
    __amdgpu_buffer_rsrc_t rs;
    uint8_t* dst;
    uint32_t src;
};

// S^T of one half tile (K rows of half buffer kb_, both row blocks) while
// the weights of one row block (logits xs) of the other pending half are
// computed and the copy cp is issued.
template <bool RS>
__device__ __forceinline__ void region_s(const uint8_t* kb_, const uint32_t koff[8], const bf16x8 qb[2][8],
                                         f32x16 s[2], const f32x16& xs, float m, float c2, bf16x8& p0,
                                         bf16x8& p1, float& ls, const Copy& cp, const uint32_t dmaoff[4]) {
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 ka[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) ka[ks] = *reinterpret_cast<const bf16x8*>(kb_ + koff[ks]);
    const f32x16 zero = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
            s[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qb[rb][ks], ks ? s[rb] : zero, 0, 0, 0);
    exp_rb<RS>(xs, m, c2, p0, p1, ls);
    dma_half(cp.rs, cp.dst, cp.src, dmaoff);
    region_schedule<1, true, true, RS>();
}

// O^T += V^T P^T over one half tile (V rows in half buffer vb_, P^T operands
// pb[q2][rb]), with (EXP) the weights of one row block of the next half and
// (COPY) one half-tile copy.
template <bool EXP, bool COPY, bool RS>
__device__ __forceinline__ void region_pv(State& st, const uint8_t* vb_, const uint32_t oa[4], const uint32_t ob[4],
                                          const bf16x8 pb[2][2], const f32x16& xs, float m, float c2, bf16x8& p0,
                                          bf16x8& p1, float& ls, const Copy& cp, const uint32_t dmaoff[4]) {
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 va[2][4];
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int db = 0; db < 4; ++db)
            va[q2][db] = tr_read_pair(vb_ + oa[db] + q2 * 16 * ROWB, vb_ + ob[db] + q2 * 16 * ROWB);
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
                st.o[db][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[q2][db], pb[q2][rb], st.o[db][rb], 0, 0, 0);
    if (EXP) exp_rb<RS>(xs, m, c2, p0, p1, ls);
    if (COPY) dma_half(cp.rs, cp.dst, cp.src, dmaoff);
    if (EXP || COPY) region_schedule<2, EXP, COPY, RS>();
}

// ---- centroid units: the two row blocks staggered ----
//
// A unit of 32 centroids is four regions of 16 MFMAs: S of row block 0, S of
// row block 1 with the bias and weights of row block 0 between its MFMAs, PV
// of row block 0 (over the V high and low planes) with the bias and weights
// of row block 1, and PV of row block 1.  Each region reads its own operands
// from LDS (no operand registers live across regions).

// The weights computed inside a region must stay there: an empty volatile
// asm that takes them as inputs at the region's end keeps LLVM from sinking
// their computation into the code after it, out of reach of the schedule.
__device__ __forceinline__ void pin_weights(const bf16x8& p0, const bf16x8& p1, float ls) {
    asm volatile("" ::"v"(__builtin_bit_cast(u32x4, p0)), "v"(__builtin_bit_cast(u32x4, p1)), "v"(ls));
}

// One row block's overflow check (as settle_half, for row block RB only).
template <bool RS, int RB>
__device__ __forceinline__ void settle_row(State& st, const f32x16& s, float c2, bf16x8& p0, bf16x8& p1, float& ls) {
    if (__builtin_expect(__ballot(ls > OVF) != 0, 0)) {
        float mx = s[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = pair_max(mx);
        if (pair_max(ls) > OVF) rescale_row(st, RB, ceilf(mx));
        exp_rb<RS>(s, st.m[RB], 1.0f, p0, p1, ls);
    }
    st.l[RB] += ls;
}

// S^T of one row block over the unit's K high and low planes; with EXP, the
// other row block's logits xs get their bias and weights; without, the bias
// of the unit is set from cmh (this lane's compensated-centroid bits shifted
// down by 4h: accumulator entry r, centroid 8(r/4) + 4h + r%4, is bit
// 8(r/4) + r%4): log2 64 = 6 where set, -inf elsewhere.
template <bool RS, bool EXP>
__device__ __forceinline__ void region_cs_rb(const uint8_t* khb, const uint8_t* klb, const uint32_t koff[8],
                                             const bf16x8 qbr[8], f32x16& s, f32x16& xs, float bias[16],
                                             uint32_t cmh, float m, float c2, bf16x8& p0, bf16x8& p1, float& ls) {
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 khi[8], klo[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        khi[ks] = *reinterpret_cast<const bf16x8*>(khb + koff[ks]);
        klo[ks] = *reinterpret_cast<const bf16x8*>(klb + koff[ks]);
    }
    const f32x16 zero = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(khi[ks], qbr[ks], ks ? s : zero, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(klo[ks], qbr[ks], s, 0, 0, 0);
    }
    if (EXP) {
#pragma unroll
        for (int r = 0; r < 16; ++r) xs[r] = fmaf(xs[r], c2, bias[r]);
        exp_rb<RS>(xs, m, 1.0f, p0, p1, ls);
    } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) bias[r] = ((cmh >> (8 * (r >> 2) + (r & 3))) & 1u) ? 6.0f : -INFINITY;
    }
    region_schedule<2, true, false, RS>();    // 16 K reads, two per MFMA pair
    if (EXP) {
        pin_weights(p0, p1, ls);
    } else {
        asm volatile("" ::"v"(bias[0]), "v"(bias[1]), "v"(bias[2]), "v"(bias[3]), "v"(bias[4]), "v"(bias[5]),
                     "v"(bias[6]), "v"(bias[7]));
        asm volatile("" ::"v"(bias[8]), "v"(bias[9]), "v"(bias[10]), "v"(bias[11]), "v"(bias[12]),
                     "v"(bias[13]), "v"(bias[14]), "v"(bias[15]));
    }
}

// O^T += V^T P^T of row block RB over the unit's V high and low planes (P^T
// in pw[q2]); with EXP, the other row block's logits xs get bias and weights.
template <bool RS, bool EXP, int RB>
__device__ __forceinline__ void region_cpv_rb(State& st, const uint8_t* vhb, const uint8_t* vlb, const uint32_t oa[4],
                                              const uint32_t ob[4], const bf16x8& pw0, const bf16x8& pw1,
                                              f32x16& xs, const float bias[16], float m, float c2, bf16x8& p0,
                                              bf16x8& p1, float& ls) {
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 va[2][2][4];
#pragma unroll
    for (int pl = 0; pl < 2; ++pl)
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const uint8_t* vb_ = pl ? vlb : vhb;
                va[pl][q2][db] = tr_read_pair(vb_ + oa[db] + q2 * 16 * ROWB, vb_ + ob[db] + q2 * 16 * ROWB);
            }
#pragma unroll
    for (int pl = 0; pl < 2; ++pl)
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
            for (int db = 0; db < 4; ++db)
                st.o[db][RB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[pl][q2][db], q2 ? pw1 : pw0, st.o[db][RB], 0, 0, 0);
    if (EXP) {
#pragma unroll
        for (int r = 0; r < 16; ++r) xs[r] = fmaf(xs[r], c2, bias[r]);
        exp_rb<RS>(xs, m, 1.0f, p0, p1, ls);
    }
    region_schedule<4, EXP, false, RS>();     // 32 V^T reads, four per MFMA pair
    if (EXP) pin_weights(p0, p1, ls);
}

// fp8 e4m3 skim tiles with per-block power-of-two scales (E8M0 operand
// scales of v_mfma_scale_f32_32x32x64_f8f6f4):
//   S^T = (K~ 2^{e_k}) (Q~ 2^{e_q})^T; L = scale log2(e) S (pad keys -inf)
//   per row: c = ceil(max_tile L); codes p~ = e4m3(2^{8 + L - c})
//   O^T += (V~^T 2^{e_v}) (p~^T 2^{c - 8 - m}) with the per-row B scale;
//   the denominators take the unquantised 2^{L - m}.
// Q~ and K~ are row-major; V~ is stored block-transposed [d][64] in the key
// order of P's accumulator layout, so both fp8 PV operands are contiguous
// 32-byte loads and no LDS is needed.  The next tile's list entry and block
// exponents come through the scalar cache, and its K~ / V~ operands load
// while this tile computes.
// FMT 1: e4m3 copies with one power-of-two scale per block and tensor.
// FMT 2: MXFP4 copies; each lane's 32 reduction values of an operand carry
// their own E8M0 scale (Q, K: per token and 32 dimensions; V: per block and
// dimension), passed to the block-scaled MFMA per lane.  P stays e4m3.  Q and
// K are packed alike, so the order in which the matrix core reads a lane's
// fp4 values does not matter for Q K^T; for V (fp4) against P (e4m3) it does.
template <int FMT>
__device__ __forceinline__ void skim_tiles(const FwdArgs& a, State& st, size_t bh, int qa,
                                        const int32_t* listM, int cntM, float c2) {
    constexpr bool F4 = FMT == 2;
    constexpr int QB = F4 ? D / 2 : D;             // bytes per token row of the Q / K copies
    const int nb = a.N_pad / BLK;
    const int l = lane_id(), h = l >> 5, l32 = l & 31;
    const size_t head = bh * a.N_pad * D;
    const size_t headb = bh * a.N_pad * QB;
    const uint8_t* Q8 = (F4 ? a.q4 : a.q8) + headb;
    const uint8_t* K8 = (F4 ? a.k4 : a.k8) + headb;
    const uint8_t* V8 = (F4 ? a.v4 : a.v8) + headb;
    typedef __attribute__((address_space(4))) const uint8_t const_u8;
    const uint8_t* QS = F4 ? a.qs4 + bh * a.N_pad * (D / 32) : nullptr;
    const uint8_t* KS = F4 ? a.ks4 + bh * a.N_pad * (D / 32) : nullptr;
    const uint8_t* VS = F4 ? a.vs4 + bh * static_cast<size_t>(nb) * D : nullptr;
    typedef __attribute__((address_space(4))) const int8_t const_i8;
    const const_i8* EX = (const const_i8*)(a.exp8 + bh * nb * 3);
    const const_i32* LM = (const const_i32*)listM;
    i32x8 qb8[2][2];
    int qsc[2][2];                                  // MXFP4: E8M0 scale of each B operand
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int row = qa * BLK + 32 * rb + l32;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            i32x8 z = {};
            if constexpr (F4) {
                // 32 four-bit codes in the low four dwords
                const u32x4 w = *reinterpret_cast<const u32x4*>(Q8 + static_cast<size_t>(row) * QB + 32 * ks + 16 * h);
                z[0] = w[0]; z[1] = w[1]; z[2] = w[2]; z[3] = w[3];
                qsc[rb][ks] = QS[static_cast<size_t>(row) * (D / 32) + 2 * ks + h];
            } else {
                if (row < a.N) z = *reinterpret_cast<const i32x8*>(Q8 + static_cast<size_t>(row) * D + 64 * ks + 32 * h);
                qsc[rb][ks] = 0;
            }
            qb8[rb][ks] = z;
        }
    }
    const int sq = static_cast<int>(EX[qa * 3 + 0]) + 127;
    auto load_tile = [&](int j, i32x8 ka[2][2], i32x8 va[4], int ksc[2][2], int vsc[4]) __attribute__((always_inline)) {
        const uint8_t* Kj = K8 + static_cast<size_t>(j) * BLK * QB;
        const uint8_t* Vj = V8 + static_cast<size_t>(j) * BLK * QB;
        if constexpr (F4) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const u32x4 w = *reinterpret_cast<const u32x4*>(Kj + (32 * kb + l32) * QB + 32 * ks + 16 * h);
                    ka[kb][ks] = i32x8{static_cast<int>(w[0]), static_cast<int>(w[1]), static_cast<int>(w[2]),
                                       static_cast<int>(w[3]), 0, 0, 0, 0};
                    ksc[kb][ks] = KS[(static_cast<size_t>(j) * BLK + 32 * kb + l32) * (D / 32) + 2 * ks + h];
                }
            // An fp4 operand lane of half h holds reduction indices
            // 32 (p / 16) + 16 h + p % 16 for its nibbles p (the fp8 P operand:
            // 32 h + p), so V^T takes positions 16h .. 16h+15 and 32+16h .. 32+16h+15.
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const uint8_t* vr = Vj + (32 * db + l32) * (BLK / 2);
                const uint2 w0 = *reinterpret_cast<const uint2*>(vr + 8 * h);
                const uint2 w1 = *reinterpret_cast<const uint2*>(vr + 16 + 8 * h);
                va[db] = i32x8{static_cast<int>(w0.x), static_cast<int>(w0.y), static_cast<int>(w1.x),
                               static_cast<int>(w1.y), 0, 0, 0, 0};
                vsc[db] = VS[static_cast<size_t>(j) * D + 32 * db + l32];
            }
        } else {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    ka[kb][ks] = *reinterpret_cast<const i32x8*>(Kj + (32 * kb + l32) * D + 64 * ks + 32 * h);
                    ksc[kb][ks] = 0;
                }
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                va[db] = *reinterpret_cast<const i32x8*>(Vj + (32 * db + l32) * BLK + 32 * h);
                vsc[db] = 0;
            }
        }
    };
    if (cntM <= 0) return;
    // One skim tile: S^T = K Q^T on the scaled MFMA, quantised weights, O^T += V^T P^T.
    auto tile = [&](int j, int sk, int sv, const i32x8 ka[2][2], const i32x8 va[4], const int ksc[2][2],
                    const int vsc[4]) __attribute__((always_inline)) {
        const int nj = min(BLK, a.N - BLK * j);
        f32x16 s[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) s[kb][rb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    if constexpr (F4)
                        s[kb][rb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            ka[kb][ks], qb8[rb][ks], s[kb][rb], 4, 4, 0, ksc[kb][ks], 0, qsc[rb][ks]);
                    else
                        s[kb][rb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            ka[kb][ks], qb8[rb][ks], s[kb][rb], 0, 0, 0, sk, 0, sq);
                }
        // raw logits; pad keys of the ragged tail block -inf (c2 > 0 commutes with max)
        if (nj < BLK) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) mask_half(s[kb], 32 * kb, nj);
        }
        i32x8 pb[2];
        int sb[2];
        float mx[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            float m0 = s[0][rb][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) m0 = fmaxf(m0, s[kb][rb][r]);
            mx[rb] = pair_max(m0) * c2;
            rescale_lazy(st, rb, mx[rb]);
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            // y = 2^{8 + L - c} is the pre-quantisation code value; the
            // unquantised weight 2^{L - m} = y 2^{c - 8 - m}, so the denominator
            // takes 2^{c - 8 - m} times the sum of the y.
            const float mref = st.m[rb];
            const float ct = (mx[rb] == -INFINITY) ? mref : ceilf(mx[rb]);
            const float off = 8.0f - ct;
            float ysum = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    float y[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        y[u] = __builtin_amdgcn_exp2f(fmaf(s[kb][rb][4 * w + u], c2, off));
                        ysum += y[u];
                    }
                    const uint32_t lo = pack_fp8x2<false>(y[0], y[1], 0u);
                    pb[rb][4 * kb + w] = static_cast<int>(pack_fp8x2<true>(y[2], y[3], lo));
                }
            st.l[rb] = fmaf(ysum, ldexpf(1.0f, static_cast<int>(ct - mref) - 8), st.l[rb]);
            sb[rb] = min(max(static_cast<int>(ct - mref) - 8 + 127, 0), 254);
        }
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                if constexpr (F4)
                    st.o[db][rb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        va[db], pb[rb], st.o[db][rb], 4, 0, 0, vsc[db], 0, sb[rb]);
                else
                    st.o[db][rb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        va[db], pb[rb], st.o[db][rb], 0, 0, 0, sv, 0, sb[rb]);
            }
    };
    // Three register slots: each tile's loads are issued two tiles ahead of
    // its use (one ahead left the loads' latency exposed).  Loads past the end
    // of the list repeat the last tile (never used), so the load sequence is
    // straight-line and its waits stay counted.
    struct Slot {
        i32x8 ka[2][2], va[4];
        int ksc[2][2], vsc[4];
        int j, sk, sv;
    };
    // (the exponent bytes are vector loads: issued before the tile's own loads,
    // so that waiting for them leaves the tile loads in flight)
    auto fill = [&](Slot& sl, int e) __attribute__((always_inline)) {
        sl.j = LM[min(e, cntM - 1)];
        sl.sk = static_cast<int>(EX[sl.j * 3 + 1]) + 127;
        sl.sv = static_cast<int>(EX[sl.j * 3 + 2]) + 127;
        load_tile(sl.j, sl.ka, sl.va, sl.ksc, sl.vsc);
    };
    auto run = [&](const Slot& sl) __attribute__((always_inline)) {
        tile(sl.j, sl.sk, sl.sv, sl.ka, sl.va, sl.ksc, sl.vsc);
    };
    Slot s0, s1, s2;
    fill(s0, 0);
    fill(s1, 1);
    for (int e = 0; e < cntM; e += 3) {
        fill(s2, e + 2);
        run(s0);
        fill(s0, e + 3);
        if (e + 1 < cntM) run(s1);
        fill(s1, e + 4);
        if (e + 2 < cntM) run(s2);
    }
}

template <int COMP, int SKIM>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) void fwd_bf16_kernel(FwdArgs a) {
    // the first-order Taylor forms normalise with the sum of the bf16-rounded
    // weights (their H terms already spend most of the bf16 error budget);
    // order 0 and drop with the fp32 sum
    constexpr bool RS = COMP >= 1;
    // separate LDS objects per half tile, so that each copy is known not to
    // alias the reads of the other three
    __shared__ __attribute__((aligned(16))) uint8_t kbuf0[HALFB];    // K rows 0-31 (row-major, swizzled)
    __shared__ __attribute__((aligned(16))) uint8_t kbuf1[HALFB];    // K rows 32-63
    __shared__ __attribute__((aligned(16))) uint8_t vbuf0[HALFB];    // V rows 0-31
    __shared__ __attribute__((aligned(16))) uint8_t vbuf1[HALFB];    // V rows 32-63
    __shared__ uint32_t kept_mask[128];                              // blocks not compensated (nb <= 4096)
    // order-1 weights of 16 centroids, fp32 [centroid][row] (4 KiB: the LDS
    // footprint stays within four workgroups per CU)
    __shared__ float wbuf[COMP == 1 ? 16 * BLK : 1];

    const int nq = a.Nq_pad / BLK, nb = a.N_pad / BLK;
    const int lin0 = xcd_remap(blockIdx.x, gridDim.x);
    const int per_chunk = nq * a.H * a.B;
    const int chunk = a.dense ? lin0 / per_chunk : 0;   // dense mode: key chunk of this wave
    const int lin = lin0 - chunk * per_chunk;
    const int qa = lin % nq;
    const size_t bh = lin / nq;
    const int jlo = a.dense ? static_cast<int>(static_cast<long long>(chunk) * nb / a.dense) : 0;
    const int jhi = a.dense ? static_cast<int>(static_cast<long long>(chunk + 1) * nb / a.dense) : nb;
    const int l = lane_id(), h = l >> 5, l32 = l & 31;
    const size_t head = bh * a.N_pad * D;
    const size_t headq = bh * a.Nq_pad * D;
    const uint16_t* Q = static_cast<const uint16_t*>(a.q) + headq;
    const uint16_t* K = static_cast<const uint16_t*>(a.k) + head;
    const uint16_t* V = static_cast<const uint16_t*>(a.v) + head;
    const float c2 = a.scale * LOG2E;

    const size_t rowid = bh * nq + qa;
    const int cntE = a.dense ? jhi - jlo : (a.cap > 0 ? min(a.cnt[rowid], a.cap) : 0);
    const int32_t* listE = a.idx + rowid * a.cap;
    const const_i32* lstE = (const const_i32*)listE;
    const int cntM = SKIM ? min(a.cnt2[rowid], a.cap2) : 0;
    const int32_t* listM = SKIM ? a.idx2 + rowid * a.cap2 : nullptr;

    uint32_t dmaoff[4], oa[4], ob[4], koff[8];
    dma_offsets(dmaoff);
    pv_offsets(oa, ob);
    k_offsets(koff);

    // Q^T as B operands: qb[rb][ks] = Q[row 32rb + l32][16ks + 8h .. +7]
    bf16x8 qb[2][8];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int row = qa * BLK + 32 * rb + l32;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            bf16x8 z = {};
            if (row < a.Nq) z = *reinterpret_cast<const bf16x8*>(Q + static_cast<size_t>(row) * D + 16 * ks + 8 * h);
            // Q^T only ever feeds MFMA B operands, which read AGPRs directly:
            // keep it there and leave the VGPRs to the accumulators and weights.
            u32x4 zu = __builtin_bit_cast(u32x4, z);
            asm volatile("" : "+a"(zu));
            qb[rb][ks] = __builtin_bit_cast(bf16x8, zu);
        }
    }

    // K and V of this head as raw buffers (tile offsets are scalars)
    const int slab = a.N_pad * ROWB;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(K), 0, slab, RSRC_WORD3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(V), 0, slab, RSRC_WORD3);

    // First copies, in the order the steady state expects them: K(0, lo),
    // V(0, hi) (in place of the previous tile's V, read with P = 0), K(0, hi);
    // region A of the first tile issues V(0, lo).
    int j = 0;
    if (cntE > 0) {
        j = a.dense ? jlo : lstE[0];
        const uint32_t t0 = static_cast<uint32_t>(j) * TILEB;
        dma_half(rk, kbuf0, t0, dmaoff);
        dma_half(rv, vbuf1, t0 + HALFB, dmaoff);
        dma_half(rk, kbuf1, t0 + HALFB, dmaoff);
    }

    // blocks that are not compensated (exact and skim lists)
    for (int x = l; x < 128; x += 64) kept_mask[x] = 0u;
    wave_lds_sync();
    if (COMP >= 0) {
        for (int e = l; e < cntE; e += 64) {
            const int jj = listE[e];
            atomicOr(&kept_mask[jj >> 5], 1u << (jj & 31));
        }
        for (int e = l; e < cntM; e += 64) {
            const int jj = listM[e];
            atomicOr(&kept_mask[jj >> 5], 1u << (jj & 31));
        }
        wave_lds_sync();
    }

    State st;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) st.o[db][rb] = f32x16{};
    st.m[0] = st.m[1] = M_INIT;
    st.l[0] = st.l[1] = 0.f;
    st.a1[0] = st.a1[1] = 0.f;

    // ---- phase 1: exact key blocks, pipelined over half tiles ----
    // Each region refills the buffer the previous region read:
    //   A(i): V(i, lo) -> vbuf0      B(i): K(i+1, lo) -> kbuf0
    //   C(i): V(i, hi) -> vbuf1      D(i): K(i+1, hi) -> kbuf1
    // so every copy has two regions to land, and when a region starts two
    // half-tile copies (16 dwordx4 loads) were issued after the one it reads.
    if (cntE > 0) {
        f32x16 s0[2], s1[2];                 // logits of the low / high key half
        bf16x8 pb0[2][2], pb1[2][2];         // their bf16 weights [q2][rb]
        float ls0[2], ls1[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s1[rb][r] = -INFINITY;
            pb1[0][rb] = bf16x8{};
            pb1[1][rb] = bf16x8{};
            ls1[rb] = 0.f;
        }
        int nj = min(BLK, a.N - BLK * j);
        int nj_prev = nj;
        for (int i = 0; i < cntE; ++i) {
            const int jn = i + 1 < cntE ? (a.dense ? jlo + i + 1 : lstE[i + 1]) : j;   // the last tile copies itself again (never read)
            const uint32_t tj = static_cast<uint32_t>(j) * TILEB, tn = static_cast<uint32_t>(jn) * TILEB;

            // A: S(lo, i) | weights of (hi, i-1), row block 1 | copy V(i, lo)
            wait_vmcnt<16>();
            wave_lds_sync();
            region_s<RS>(kbuf0, koff, qb, s0, s1[1], st.m[1], c2, pb1[0][1], pb1[1][1], ls1[1],
                     Copy{rv, vbuf0, tj}, dmaoff);
            settle_half<RS>(st, s1, c2, pb1, ls1);
            if (nj < 32) mask_half(s0, 0, nj);

            // B: PV(hi, i-1) | weights of (lo, i), row block 0 | copy K(i+1, lo)
            wait_vmcnt<16>();
            if (nj_prev < BLK) zero_rows(vbuf1, max(nj_prev, 32) - 32);
            wave_lds_sync();
            region_pv<true, true, RS>(st, vbuf1, oa, ob, pb1, s0[0], st.m[0], c2, pb0[0][0], pb0[1][0], ls0[0],
                                  Copy{rk, kbuf0, tn}, dmaoff);

            // C: S(hi, i) | weights of (lo, i), row block 1 | copy V(i, hi)
            wait_vmcnt<16>();
            wave_lds_sync();
            region_s<RS>(kbuf1, koff, qb, s1, s0[1], st.m[1], c2, pb0[0][1], pb0[1][1], ls0[1],
                     Copy{rv, vbuf1, tj + HALFB}, dmaoff);
            settle_half<RS>(st, s0, c2, pb0, ls0);
            if (nj < BLK) mask_half(s1, 32, nj);

            // D: PV(lo, i) | weights of (hi, i), row block 0 | copy K(i+1, hi)
            wait_vmcnt<16>();
            if (nj < 32) zero_rows(vbuf0, nj);
            wave_lds_sync();
            region_pv<true, true, RS>(st, vbuf0, oa, ob, pb0, s1[0], st.m[0], c2, pb1[0][0], pb1[1][0], ls1[0],
                                  Copy{rk, kbuf1, tn + HALFB}, dmaoff);

            nj_prev = nj;
            j = jn;
            nj = min(BLK, a.N - BLK * j);
        }
        // drain: weights of (hi, last), row block 1, then PV(hi, last)
        exp_rb<RS>(s1[1], st.m[1], c2, pb1[0][1], pb1[1][1], ls1[1]);
        settle_half<RS>(st, s1, c2, pb1, ls1);
        wait_vmcnt<0>();
        if (nj_prev < BLK) zero_rows(vbuf1, max(nj_prev, 32) - 32);
        wave_lds_sync();
        {
            float unused_l;
            bf16x8 unused0, unused1;
            region_pv<false, false, RS>(st, vbuf1, oa, ob, pb1, s1[0], 0.f, c2, unused0, unused1, unused_l,
                                    Copy{rv, vbuf1, 0}, dmaoff);
        }
        wave_lds_sync();
    }


    // ---- phase 2 (and 3): centroid pseudo-keys of every compensated block ----
    // Units of 32 centroids.  The centroid planes (bf16 high and low parts of
    // the fp32 means, from the pooling pass) are copied into the four half
    // buffers: K hi -> kbuf0, K lo -> kbuf1, V hi -> vbuf0, V lo -> vbuf1; the
    // next unit's K planes load during this unit's softmax and PV, its V
    // planes during the next S.
    if (COMP >= 0) {
        const int nbc = BLK * ((nb + BLK - 1) / BLK);
        const int nu = (nb + 31) / 32;
        const uint16_t* C = static_cast<const uint16_t*>(a.cent) + bh * 4 * static_cast<size_t>(nbc) * D;
        const __amdgpu_buffer_rsrc_t rc =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(C), 0, 4 * nbc * ROWB, RSRC_WORD3);
        const uint32_t plane = static_cast<uint32_t>(nbc) * ROWB;
        const int nlast = a.N - BLK * (nb - 1);
        const float blast = __log2f(static_cast<float>(nlast));   // log2 n_j of the last block
        dma_half(rc, kbuf0, 0, dmaoff);
        dma_half(rc, kbuf1, plane, dmaoff);
        dma_half(rc, vbuf0, 2 * plane, dmaoff);
        dma_half(rc, vbuf1, 3 * plane, dmaoff);
        for (int u = 0; u < nu; ++u) {
            const bool more = u + 1 < nu;
            const uint32_t un = static_cast<uint32_t>(more ? u + 1 : u) * HALFB;
            // logits in log2 units with the count bias; -inf at exact / skim / pad
            // centroids: bit c of cm marks centroid 32 u + c as compensated
            const uint32_t valid = 32 * u + 32 <= nb ? 0xFFFFFFFFu : ((1u << (nb - 32 * u)) - 1u);
            const uint32_t keptw = kept_mask[u];
            const uint32_t cmh = (~keptw & valid) >> (4 * h);
            float bias[16];
            // K planes of unit u: only its V planes were issued after them
            wait_vmcnt<16>();
            wave_lds_sync();
            f32x16 s[2];
            bf16x8 pb[2][2];
            float ls[2];
            {
                float unused_l;
                bf16x8 unused0, unused1;
                region_cs_rb<RS, false>(kbuf0, kbuf1, koff, qb[0], s[0], s[1], bias, cmh, 0.f, c2, unused0,
                                        unused1, unused_l);
            }
            if (u == nu - 1 && nlast < BLK) {
                // the last block's centroid takes log2 of its own count
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (8 * (r >> 2) + 4 * h + (r & 3) == ((nb - 1) & 31) && bias[r] != -INFINITY) bias[r] = blast;
            }
            region_cs_rb<RS, true>(kbuf0, kbuf1, koff, qb[1], s[1], s[0], bias, 0u, st.m[0], c2, pb[0][0],
                                   pb[1][0], ls[0]);
            wave_lds_sync();
            if (more) {
                dma_half(rc, kbuf0, un, dmaoff);
                dma_half(rc, kbuf1, plane + un, dmaoff);
            }
            settle_row<RS, 0>(st, s[0], 1.0f, pb[0][0], pb[1][0], ls[0]);
            // V planes of unit u: only the next unit's K planes may still be in flight
            if (more) wait_vmcnt<16>(); else wait_vmcnt<0>();
            wave_lds_sync();
            region_cpv_rb<RS, true, 0>(st, vbuf0, vbuf1, oa, ob, pb[0][0], pb[1][0], s[1], bias, st.m[1], c2,
                                       pb[0][1], pb[1][1], ls[1]);
            settle_row<RS, 1>(st, s[1], 1.0f, pb[0][1], pb[1][1], ls[1]);
            {
                float unused_l;
                bf16x8 unused0, unused1;
                region_cpv_rb<RS, false, 1>(st, vbuf0, vbuf1, oa, ob, pb[0][1], pb[1][1], s[0], bias, 0.f, c2,
                                            unused0, unused1, unused_l);
            }
            wave_lds_sync();
            if (more) {
                dma_half(rc, vbuf0, 2 * plane + un, dmaoff);
                dma_half(rc, vbuf1, 3 * plane + un, dmaoff);
            }
            if (COMP == 2) {
                // PISA's global first-order weight: sum over skipped blocks of
                // alpha_{t,j} = e^{s q.k_bar_j}, relative to the reference m
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    float acc = 0.f;
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (bias[r] != -INFINITY) acc += __builtin_amdgcn_exp2f(s[rb][r] - bias[r] - st.m[rb]);
                    st.a1[rb] += acc;
                }
            }
            if (COMP == 1) {
                // O^T[., row] += w_j[row] T, T = H_j^T Q^T (fp32, 16 MFMAs per
                // 32-wide d block), for every compensated block j of this unit,
                // with w_j = scale 2^{L - m} / n_j (L without the count bias).
                // Two batches of 16 centroids (their weights staged in LDS); the A
                // operands (H_j^T in MFMA operand order) load two d blocks ahead.
                const uint16_t* MOM = static_cast<const uint16_t*>(a.kmom) + bh * nb * static_cast<size_t>(D) * D;
                // H_j^T in MFMA operand order: (d block, i step) operands are 1 KiB runs
                auto load_step = [&](int jj, int db, bf16x8 op[8]) __attribute__((always_inline)) {
                    const uint16_t* Hop = MOM + static_cast<size_t>(jj) * D * D + (db * 8 * 64 + l) * 8;
#pragma unroll
                    for (int ks = 0; ks < 8; ++ks) op[ks] = *reinterpret_cast<const bf16x8*>(Hop + ks * 64 * 8);
                };
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    // accumulator entries r = 8 hb .. 8 hb + 7 hold centroids 16 hb .. 16 hb + 15
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                        for (int r = 8 * hb; r < 8 * hb + 8; ++r) {
                            const int cc = 8 * (r >> 2) + 4 * h + (r & 3) - 16 * hb;
                            const float x = (bias[r] == -INFINITY) ? 0.f
                                : __builtin_amdgcn_exp2f(s[rb][r] - bias[r] - st.m[rb]) * a.scale;
                            wbuf[cc * BLK + 32 * rb + l32] = x;
                        }
                    wave_lds_sync();
                    uint32_t pend = 0;                    // compensated blocks of this batch
#pragma unroll
                    for (int c = 0; c < 16; ++c) {
                        const int cc = 16 * hb + c;
                        if (32 * u + cc < nb && !((keptw >> cc) & 1u)) pend |= 1u << c;
                    }
                    if (pend) {
                        // steps (block, d block) in order; each step's eight A
                        // operands load two steps (32 MFMAs) ahead into one of two
                        // operand sets
                        int c = __builtin_ctz(pend);
                        pend &= pend - 1;
                        bf16x8 buf[2][8];
                        load_step(32 * u + 16 * hb + c, 0, buf[0]);
                        load_step(32 * u + 16 * hb + c, 1, buf[1]);
                        for (;;) {
                            const float w0 = wbuf[c * BLK + l32], w1 = wbuf[c * BLK + 32 + l32];
                            const int nc = pend ? __builtin_ctz(pend) : -1;
#pragma unroll
                            for (int db = 0; db < 4; ++db) {
                                f32x16 t[2] = {f32x16{}, f32x16{}};
#pragma unroll
                                for (int ks = 0; ks < 8; ++ks)
#pragma unroll
                                    for (int rb = 0; rb < 2; ++rb)
                                        t[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(buf[db & 1][ks], qb[rb][ks], t[rb], 0, 0, 0);
                                if (db < 2) load_step(32 * u + 16 * hb + c, db + 2, buf[db & 1]);
                                else if (nc >= 0) load_step(32 * u + 16 * hb + nc, db - 2, buf[db & 1]);
#pragma unroll
                                for (int r = 0; r < 16; ++r) {
                                    st.o[db][0][r] = fmaf(t[0][r], w0, st.o[db][0][r]);
                                    st.o[db][1][r] = fmaf(t[1][r], w1, st.o[db][1][r]);
                                }
                            }
                            if (nc < 0) break;
                            c = nc;
                            pend &= pend - 1;
                        }
                    }
                    wave_lds_sync();
                }
            }
        }
        wait_vmcnt<0>();
        if (COMP == 2) {
            // O^T[., row] += s A_row (H_bar^T Q^T)[., row], A_row = sum_j alpha_{t,j}:
            // one d x d product per query block (H_bar split into bf16 high +
            // low parts, fp32 accumulation)
            const float* HB = a.hbar + bh * static_cast<size_t>(D) * D;    // value-major G[o][i]
            const float w0 = a.scale * pair_sum(st.a1[0]), w1 = a.scale * pair_sum(st.a1[1]);
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                f32x16 t[2] = {f32x16{}, f32x16{}};
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) {
                    const float* g = HB + (32 * db + l32) * D + 16 * ks + 8 * h;
                    const float4 x0 = *reinterpret_cast<const float4*>(g);
                    const float4 x1 = *reinterpret_cast<const float4*>(g + 4);
                    const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                    u32x4 whi, wlo;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        whi[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
                        wlo[e] = pack_bf16x2(x[2 * e] - bf16_to_f32(static_cast<uint16_t>(whi[e] & 0xFFFFu)),
                                             x[2 * e + 1] - bf16_to_f32(static_cast<uint16_t>(whi[e] >> 16)));
                    }
                    const bf16x8 ghi = __builtin_bit_cast(bf16x8, whi), glo = __builtin_bit_cast(bf16x8, wlo);
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb) {
                        t[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ghi, qb[rb][ks], t[rb], 0, 0, 0);
                        t[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(glo, qb[rb][ks], t[rb], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    st.o[db][0][r] = fmaf(t[0][r], w0, st.o[db][0][r]);
                    st.o[db][1][r] = fmaf(t[1][r], w1, st.o[db][1][r]);
                }
            }
        }
    }

    // ---- phase 3: skim blocks (Triage's low-precision tier) ----
    // after the centroids, so that the bf16 Q^T operands are dead and their
    // registers hold the skim tiles in flight
    if constexpr (SKIM > 0) skim_tiles<SKIM>(a, st, bh, qa, listM, cntM, c2);

    // ---- normalise and write O (bf16) and lse ----
    const size_t cofs = static_cast<size_t>(chunk) * per_chunk * BLK;   // B H Nq_pad rows per chunk
    uint16_t* O = static_cast<uint16_t*>(a.out) + headq + cofs * D;
    float* OF = static_cast<float*>(a.out) + headq + cofs * D;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const float lt = pair_sum(st.l[rb]);
        const int row = qa * BLK + 32 * rb + l32;
        const bool valid = row < a.Nq;
        const float inv = valid ? 1.0f / lt : 0.f;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int dd = 32 * db + 8 * q4 + 4 * h;
                if (a.out_f32) {
                    const f32x4 w = {st.o[db][rb][4 * q4 + 0] * inv, st.o[db][rb][4 * q4 + 1] * inv,
                                     st.o[db][rb][4 * q4 + 2] * inv, st.o[db][rb][4 * q4 + 3] * inv};
                    *reinterpret_cast<f32x4*>(OF + static_cast<size_t>(row) * D + dd) = w;
                    continue;
                }
                uint2 w;
                w.x = pack_bf16x2(st.o[db][rb][4 * q4 + 0] * inv, st.o[db][rb][4 * q4 + 1] * inv);
                w.y = pack_bf16x2(st.o[db][rb][4 * q4 + 2] * inv, st.o[db][rb][4 * q4 + 3] * inv);
                *reinterpret_cast<uint2*>(O + static_cast<size_t>(row) * D + dd) = w;
            }
        }
        if (a.lse && h == 0) a.lse[cofs + bh * a.Nq_pad + row] = valid ? (st.m[rb] + __log2f(lt)) * LN2 : 0.f;
    }
}

template <int COMP, int SKIM>
hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
    const int nq = a.Nq_pad / BLK;
    dim3 grid(nq * a.H * a.B * (a.dense > 0 ? a.dense : 1));
    hipLaunchKernelGGL((fwd_bf16_kernel<COMP, SKIM>), grid, dim3(64), 0, s, a);
    return hipGetLastError();
}

template <int SKIM>
hipError_t launch_c(const FwdArgs& a, hipStream_t s) {
    switch (a.comp) {
        case -1: return launch_t<-1, SKIM>(a, s);
        case 0: return launch_t<0, SKIM>(a, s);
        case 1: return launch_t<1, SKIM>(a, s);
        default: return launch_t<2, SKIM>(a, s);
    }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) {
    const bool skim = a.idx2 != nullptr && a.cap2 > 0;
    if (!skim) return launch_c<0>(a, s);
    return a.skim_fmt == 1 ? launch_c<2>(a, s) : launch_c<1>(a, s);
}

}  // namespace sa
