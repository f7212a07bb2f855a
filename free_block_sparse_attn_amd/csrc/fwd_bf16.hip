// bf16 compensated block-sparse attention forward for gfx950 (d = 128).
//
// What it computes (per query t of query block a, one softmax):
//   exact key blocks E          e^{s q.k_n} (v_n)                    bf16 MFMA
//   every other key block j     n_j e^{s q.k_bar_j} (v_bar_j)         order 0
//                               + e^{s q.k_bar_j} s q^T H_j (N only)  order 1
// PISA ("PISA: Piecewise Sparse Attention Is Wiser for Efficient Diffusion
// Transformers", section 2, "Algorithme Central" and "Implementation
// Materielle": exact phase on selected blocks, then a scan of the block
// aggregates, then the first-order correction, all inside one
// FlashAttention-style online softmax); SVG-EAR's centroid compensation
// ("SVG-EAR ...", section 2A).
//
// Work split.  One wave owns a whole 64-row query block, so a 64-key tile is
// 2 x 2 blocks of 32x32 and every K/V byte loaded feeds 64 query rows.
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, A = K rows loaded straight from
//                 global memory into VGPRs one tile ahead, B = Q^T held in
//                 VGPRs for the whole kernel.  Each lane ends up owning one
//                 query row per 32-row block, so the row max / row sum need a
//                 single exchange with the other half of the wave.
//   O^T += V^T P^T  B = P^T straight from S's accumulators (rounded to bf16),
//                 A = V^T read from a row-major LDS copy of V with
//                 ds_read_b64_tr_b16 (4 consecutive keys of one d per read).
//                 V tiles reach LDS by global_load_lds_dwordx4 (no VGPRs),
//                 double buffered one tile ahead, with a 16-byte XOR swizzle.
// The P^T operand's key order follows S's accumulator layout: within each
// 16-key MFMA step, slot s holds key s with bits 2 and 3 swapped; the V^T
// reads use the same order.  Centroid pseudo-keys go through the same MFMA
// path as 64-wide tiles (means split into bf16 high + low parts so the fp32
// means keep ~16 bits), with bias log2(n_j) and -inf at the exact blocks.
// The running max is updated lazily (only when a row's tile max exceeds it
// by more than 8 in log2 units), which keeps the accumulator rescale off the
// common path.  The softmax denominator sums the same bf16-rounded P that
// the MFMA consumes, so rounding of P cancels in o = N / D.
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
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float M_INIT = -1.0e30f;         // "no reference yet" (finite: 2^(-inf - M_INIT) = 0)

// physical 16-byte chunk of logical chunk c (0..15) in LDS row `row`
__device__ __forceinline__ int swz(int row, int c) { return c ^ ((row & 7) << 1); }

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

// 16 x global_load_lds_dwordx4: the whole 64x128 bf16 V tile into one LDS
// buffer.  Instruction m fills LDS rows 4m .. 4m+3; lane l lands at row
// 4m + l/16, physical chunk l%16, so it fetches the logical chunk that the
// swizzle maps there.  The swizzle depends on row & 7, i.e. on m & 1, so two
// lane offsets cover all 16 instructions.
__device__ __forceinline__ void dma_offsets(uint32_t off[2]) {
    const int l = lane_id();
    const int rsub = l >> 4, p = l & 15;
#pragma unroll
    for (int par = 0; par < 2; ++par)
        off[par] = rsub * ROWB + 16 * swz(4 * par + rsub, p);   // swz is an involution
}

__device__ __forceinline__ void dma_v_tile(const uint16_t* vrow0, uint8_t* buf, const uint32_t off[2]) {
    const uint8_t* src = reinterpret_cast<const uint8_t*>(vrow0);
#pragma unroll
    for (int m = 0; m < 16; ++m)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src + m * 4 * ROWB + off[m & 1]),
                                         (lds_void*)(buf + m * 1024), 16, 0, 0);
}

// Zero rows nvalid..63 of an LDS tile (pad keys of the ragged tail block).
__device__ __forceinline__ void zero_tail_rows(uint8_t* buf, int nvalid) {
    const int l = lane_id();
    for (int x = nvalid * 16 + l; x < BLK * 16; x += 64) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(buf + x * 16) = z;
    }
}

// Write 64 fp32 mean rows (centroid values) as bf16 rows into an LDS tile:
// the high parts (LO = false) or the residuals x - bf16(x) (LO = true).
template <bool LO>
__device__ __forceinline__ void stage_means(const float* vrow0, int nvalid, uint8_t* buf) {
    const int l = lane_id();
    const int rsub = l >> 4, c = l & 15;
#pragma unroll 4
    for (int m = 0; m < 16; ++m) {
        const int row = 4 * m + rsub;
        float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (row < nvalid) {
            const float4 x0 = *reinterpret_cast<const float4*>(vrow0 + row * D + 8 * c);
            const float4 x1 = *reinterpret_cast<const float4*>(vrow0 + row * D + 8 * c + 4);
            x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
            x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
        }
        if (LO) {
#pragma unroll
            for (int t = 0; t < 8; ++t) x[t] -= bf16_to_f32(f32_to_bf16(x[t]));
        }
        u32x4 w;
#pragma unroll
        for (int t = 0; t < 4; ++t) w[t] = pack_bf16x2(x[2 * t], x[2 * t + 1]);
        *reinterpret_cast<u32x4*>(buf + row * ROWB + 16 * swz(row, c)) = w;
    }
}

struct State {
    f32x16 o[4][2];        // O^T[d-block][row-block]
    float m[2];            // running reference max (log2 units, an integer) per row block
    float l[2];            // partial row sums of the bf16-rounded P (normalises O)
    float le[2];           // partial row sums of the unrounded weights (for lse)
};

// Lazy max: the reference of a row (log2 units, an integer so that powers of
// two relative to it are exact) moves up to ceil(tile max) only when a tile
// max exceeds it by more than 8; then the row's accumulators are rescaled.
__device__ __forceinline__ void rescale_lazy(State& st, int rb, float mx) {
    const bool need = st.m[rb] == M_INIT ? mx > -INFINITY : mx > st.m[rb] + 8.0f;
    if (__ballot(need)) {
        const float mnew = need ? ceilf(mx) : st.m[rb];
        const float alpha = __builtin_amdgcn_exp2f(st.m[rb] - mnew);
        st.l[rb] *= alpha;
        st.le[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) st.o[db][rb][r] *= alpha;
        st.m[rb] = mnew;
    }
}

__device__ __forceinline__ float sum_bf16_pair(uint32_t pair, float acc) {
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), ones, acc, false);
}

// Online-softmax update of one 64-key tile of raw logits s[kb][rb] (before
// the log2(e) * scale factor c2; scale > 0).  bias (optional) adds a per-key
// log2 term; -inf marks keys that do not take part.  Returns P^T as the bf16
// B operands of the O^T update, pb[2 kb + q2][rb].  P = 2^(c2 s + bias - m)
// comes from one FMA and one v_exp_f32; the row sum for O's normalisation
// adds the bf16-rounded P pairs with v_dot2_f32_bf16, the lse sum the
// unrounded values.
template <bool BIAS>
__device__ __forceinline__ void softmax_tile(State& st, f32x16 s[2][2], bf16x8 pb[4][2], float c2,
                                             const float bias[2][16]) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float v = BIAS ? fmaf(s[kb][rb][r], c2, bias[kb][r]) : s[kb][rb][r];
                if (BIAS) s[kb][rb][r] = v;
                mx = fmaxf(mx, v);
            }
        mx = fmaxf(mx, swap_halves(mx));
        rescale_lazy(st, rb, BIAS ? mx : mx * c2);
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const float negm = -st.m[rb];
        float ls = 0.f, le = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
                u32x4 w;
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const float a0 = s[kb][rb][8 * q2 + e], a1 = s[kb][rb][8 * q2 + e + 1];
                    const float x0 = __builtin_amdgcn_exp2f(BIAS ? a0 + negm : fmaf(a0, c2, negm));
                    const float x1 = __builtin_amdgcn_exp2f(BIAS ? a1 + negm : fmaf(a1, c2, negm));
                    const uint32_t pr = pack_bf16x2(x0, x1);
                    w[e >> 1] = pr;
                    ls = sum_bf16_pair(pr, ls);
                    le += x0;
                    le += x1;
                }
                pb[2 * kb + q2][rb] = __builtin_bit_cast(bf16x8, w);
            }
        }
        st.l[rb] += ls;
        st.le[rb] += le;
    }
}

// Lane offsets (bytes within a V tile buffer) of the transposed reads, one per
// 32-wide d block.  ds_read_b64_tr_b16: within each 16-lane group, output
// lane i receives element i%4 of the 8-byte pieces addressed by lanes i/4 + 4e
// (e = 0..3).  Supplying lane r addresses row key0 + r/4 at d0 + 4(r%4), so
// output lane i gets keys key0 .. key0+3 of column d0 + i.  The row swizzle
// depends only on row & 7 = (4h + r/4) & 7, the same for every k-step.
__device__ __forceinline__ void pv_offsets(uint32_t off[4]) {
    const int l = lane_id();
    const int h = l >> 5, g2 = (l >> 4) & 1, r = l & 15;
    const int rsub = r >> 2, csub = r & 3;
    const int row0 = 4 * h + rsub;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const int chunk = 4 * db + 2 * g2 + (csub >> 1);
        off[db] = row0 * ROWB + 16 * swz(row0, chunk) + (csub & 1) * 8;
    }
}

__device__ __forceinline__ bf16x8 tr_read_pair(const uint8_t* base) {
    // keys 16kk + 4h + e (slots 0..3) and 16kk + 8 + 4h + e (slots 4..7)
    const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base));
    const i16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 8 * ROWB));
    const i16x8 v8 = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
    return __builtin_bit_cast(bf16x8, v8);
}

// O^T += V^T P^T for one tile whose V rows sit in LDS buffer `buf`; the
// transposed reads of the next (d block, k-step) are issued before the
// MFMAs of the current one.
__device__ __forceinline__ void pv_tile(State& st, const uint8_t* buf, const uint32_t off[4],
                                        const bf16x8 pb[4][2]) {
    bf16x8 cur = tr_read_pair(buf + off[0]), nxt;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const int db = t >> 2, kk = t & 3;
        if (t < 15) {
            const int db1 = (t + 1) >> 2, kk1 = (t + 1) & 3;
            nxt = tr_read_pair(buf + off[db1] + kk1 * 16 * ROWB);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
            st.o[db][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, pb[kk][rb], st.o[db][rb], 0, 0, 0);
        cur = nxt;
    }
}

// fp8 e4m3 skim tiles with per-block power-of-two scales (E8M0 operand
// scales of v_mfma_scale_f32_32x32x64_f8f6f4):
//   S^T = (K~ 2^{e_k}) (Q~ 2^{e_q})^T; L = scale log2(e) S (pad keys -inf)
//   per row: c = ceil(max_tile L); codes p~ = e4m3(2^{8 + L - c})
//   O^T += (V~^T 2^{e_v}) (p~^T 2^{c - 8 - m}) with the per-row B scale;
//   the denominators take the unquantised 2^{L - m}.
// Q~ and K~ are row-major; V~ is stored block-transposed [d][64] in the key
// order of P's accumulator layout, so both fp8 PV operands are contiguous
// 32-byte loads and no LDS is needed.
__device__ __forceinline__ void skim_tiles(const FwdArgs& a, State& st, size_t bh, int qa,
                                        const int32_t* listM, int cntM, float c2) {
    const int nb = a.N_pad / BLK;
    const int l = lane_id(), h = l >> 5, l32 = l & 31;
    const size_t head = bh * a.N_pad * D;
    const uint8_t* Q8 = a.q8 + head;
    const uint8_t* K8 = a.k8 + head;
    const uint8_t* V8 = a.v8 + head;
    const int8_t* EX = a.exp8 + bh * nb * 3;
    i32x8 qb8[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int row = qa * BLK + 32 * rb + l32;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            i32x8 z = {};
            if (row < a.N) z = *reinterpret_cast<const i32x8*>(Q8 + static_cast<size_t>(row) * D + 64 * ks + 32 * h);
            qb8[rb][ks] = z;
        }
    }
    const int sq = static_cast<int>(EX[qa * 3 + 0]) + 127;
    for (int e = 0; e < cntM; ++e) {
        const int j = listM[e];
        const int nj = min(BLK, a.N - BLK * j);
        const int sk = static_cast<int>(EX[j * 3 + 1]) + 127;
        const int sv = static_cast<int>(EX[j * 3 + 2]) + 127;
        const uint8_t* Kj = K8 + static_cast<size_t>(j) * BLK * D;
        i32x8 ka[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                ka[kb][ks] = *reinterpret_cast<const i32x8*>(Kj + (32 * kb + l32) * D + 64 * ks + 32 * h);
        const uint8_t* Vj = V8 + static_cast<size_t>(j) * BLK * D;
        i32x8 va[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) va[db] = *reinterpret_cast<const i32x8*>(Vj + (32 * db + l32) * BLK + 32 * h);
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
                for (int rb = 0; rb < 2; ++rb)
                    s[kb][rb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        ka[kb][ks], qb8[rb][ks], s[kb][rb], 0, 0, 0, sk, 0, sq);
        i32x8 pb[2];
        int sb[2];
        float mx[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            float m0 = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
                    const float x = (key < nj) ? s[kb][rb][r] * c2 : -INFINITY;
                    s[kb][rb][r] = x;
                    m0 = fmaxf(m0, x);
                }
            mx[rb] = fmaxf(m0, swap_halves(m0));
            rescale_lazy(st, rb, mx[rb]);
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const float mref = st.m[rb];
            const float ct = (mx[rb] == -INFINITY) ? mref : ceilf(mx[rb]);
            const float mult = ldexpf(1.0f, 8 + static_cast<int>(mref - ct));
            float le = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    float y[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const float x = __builtin_amdgcn_exp2f(s[kb][rb][4 * w + u] - mref);
                        le += x;
                        y[u] = x * mult;
                    }
                    const uint32_t lo = pack_fp8x2<false>(y[0], y[1], 0u);
                    pb[rb][4 * kb + w] = static_cast<int>(pack_fp8x2<true>(y[2], y[3], lo));
                }
            st.l[rb] += le;
            st.le[rb] += le;
            sb[rb] = min(max(static_cast<int>(ct - mref) - 8 + 127, 0), 254);
        }
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
                st.o[db][rb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    va[db], pb[rb], st.o[db][rb], 0, 0, 0, sv, 0, sb[rb]);
    }
}

// K tile A operands come from the row-major, swizzled LDS copy of K:
// ka(kb, ks) = K[32kb + l32][16ks + 8h .. +7].  Lane offsets for ks = 0..7
// (kb = 1 adds 32 rows); the swizzle depends on row & 7 = l32 & 7.
__device__ __forceinline__ void k_offsets(uint32_t off[8]) {
    const int l = lane_id(), h = l >> 5, l32 = l & 31;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) off[ks] = l32 * ROWB + 16 * swz(l32, 2 * ks + h);
}

__device__ __forceinline__ void s_tile_lds(const uint8_t* kbuf, const uint32_t koff[8], const bf16x8 qb[2][8],
                                           f32x16 s[2][2]) {
    const f32x16 zero = {};
    // two k-steps of LDS reads in flight ahead of the MFMAs that use them
    bf16x8 cur[2], nxt[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) cur[kb] = *reinterpret_cast<const bf16x8*>(kbuf + koff[0] + kb * 32 * ROWB);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        if (ks < 7) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                nxt[kb] = *reinterpret_cast<const bf16x8*>(kbuf + koff[ks + 1] + kb * 32 * ROWB);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
                s[kb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur[kb], qb[rb][ks], ks ? s[kb][rb] : zero, 0, 0, 0);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) cur[kb] = nxt[kb];
    }
}

template <int COMP, bool SKIM>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) void fwd_bf16_kernel(FwdArgs a) {
    // separate LDS objects so that the K and V copies are known not to alias
    __shared__ __attribute__((aligned(16))) uint8_t kbuf[TILEB];     // K tile (row-major, swizzled)
    __shared__ __attribute__((aligned(16))) uint8_t vbuf[TILEB];     // V tile (row-major, swizzled)
    __shared__ uint32_t kept_mask[128];                              // blocks not compensated (nb <= 4096)
    __shared__ float wbuf_s[COMP == 1 ? BLK * (BLK + 1) : 1];        // order-1 weights [centroid][row]
    float* wbuf = wbuf_s;
    struct { uint32_t* kept; } lds = {kept_mask};

    const int nq = a.N_pad / BLK, nb = nq;
    const int lin = xcd_remap(blockIdx.x, gridDim.x);
    const int qa = lin % nq;
    const size_t bh = lin / nq;
    const int l = lane_id(), h = l >> 5, l32 = l & 31;
    const size_t head = bh * a.N_pad * D;
    const uint16_t* Q = static_cast<const uint16_t*>(a.q) + head;
    const uint16_t* K = static_cast<const uint16_t*>(a.k) + head;
    const uint16_t* V = static_cast<const uint16_t*>(a.v) + head;
    const float c2 = a.scale * LOG2E;

    const size_t rowid = bh * nq + qa;
    const int cntE = a.cap > 0 ? min(a.cnt[rowid], a.cap) : 0;
    const int32_t* listE = a.idx + rowid * a.cap;
    const int cntM = SKIM ? min(a.cnt2[rowid], a.cap2) : 0;
    const int32_t* listM = SKIM ? a.idx2 + rowid * a.cap2 : nullptr;

    uint32_t dmaoff[2], troff[4], koff[8];
    dma_offsets(dmaoff);
    pv_offsets(troff);
    k_offsets(koff);

    // first exact tile in flight before anything else
    if (cntE > 0) {
        const int j0 = listE[0];
        dma_v_tile(K + static_cast<size_t>(j0) * BLK * D, kbuf, dmaoff);
        dma_v_tile(V + static_cast<size_t>(j0) * BLK * D, vbuf, dmaoff);
    }

    // Q^T as B operands: qb[rb][ks] = Q[row 32rb + l32][16ks + 8h .. +7]
    bf16x8 qb[2][8];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int row = qa * BLK + 32 * rb + l32;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            bf16x8 z = {};
            if (row < a.N) z = *reinterpret_cast<const bf16x8*>(Q + static_cast<size_t>(row) * D + 16 * ks + 8 * h);
            qb[rb][ks] = z;
        }
    }

    // blocks that are not compensated (exact and skim lists)
    for (int x = l; x < 128; x += 64) lds.kept[x] = 0u;
    wave_lds_sync();
    if (COMP >= 0) {
        for (int e = l; e < cntE; e += 64) {
            const int j = listE[e];
            atomicOr(&lds.kept[j >> 5], 1u << (j & 31));
        }
        for (int e = l; e < cntM; e += 64) {
            const int j = listM[e];
            atomicOr(&lds.kept[j >> 5], 1u << (j & 31));
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
    st.le[0] = st.le[1] = 0.f;

    // ---- phase 1: exact key blocks ----
    // K and V each have one LDS buffer; each is refilled for the next tile as
    // soon as this tile is done reading it, so the K copy overlaps softmax and
    // PV, and the V copy overlaps the next S and softmax.
    for (int e = 0; e < cntE; ++e) {
        const int j = listE[e];
        const int nj = min(BLK, a.N - BLK * j);
        const bool more = e + 1 < cntE;
        const int jn = more ? listE[e + 1] : j;
        // K of this tile: only this tile's V copy may still be in flight
        wait_vmcnt<16>();
        wave_lds_sync();
        f32x16 s[2][2];
        s_tile_lds(kbuf, koff, qb, s);
        wave_lds_sync();                                   // every lane's K reads have returned
        if (more) dma_v_tile(K + static_cast<size_t>(jn) * BLK * D, kbuf, dmaoff);
        if (nj < BLK) {                                    // ragged tail block only
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
                        if (key >= nj) s[kb][rb][r] = -INFINITY;
                    }
        }
        bf16x8 pb[4][2];
        softmax_tile<false>(st, s, pb, c2, nullptr);
        // V of this tile: only the next tile's K copy may still be in flight
        if (more) wait_vmcnt<16>(); else wait_vmcnt<0>();
        if (nj < BLK) zero_tail_rows(vbuf, nj);
        wave_lds_sync();
        pv_tile(st, vbuf, troff, pb);
        wave_lds_sync();                                   // every lane's V reads have returned
        if (more) dma_v_tile(V + static_cast<size_t>(jn) * BLK * D, vbuf, dmaoff);
    }
    wait_vmcnt<0>();

    // ---- phase 1b: fp8 skim blocks (Triage's low-precision tier) ----
    if constexpr (SKIM) skim_tiles(a, st, bh, qa, listM, cntM, c2);

    // ---- phase 2 (and 3): centroid pseudo-keys of every compensated block ----
    if (COMP >= 0) {
        const float* KB = a.kbar + bh * nb * D;
        const float* VB = a.vbar + bh * nb * D;
        for (int c0 = 0; c0 < nb; c0 += BLK) {
            const int nc = min(BLK, nb - c0);
            f32x16 s[2][2];
            const f32x16 zero = {};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int cj = min(c0 + 32 * kb + l32, nb - 1);
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) {
                    const float4 x0 = *reinterpret_cast<const float4*>(KB + static_cast<size_t>(cj) * D + 16 * ks + 8 * h);
                    const float4 x1 = *reinterpret_cast<const float4*>(KB + static_cast<size_t>(cj) * D + 16 * ks + 8 * h + 4);
                    const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                    u32x4 whi, wlo;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        whi[t] = pack_bf16x2(x[2 * t], x[2 * t + 1]);
                        const float r0 = x[2 * t] - bf16_to_f32(static_cast<uint16_t>(whi[t] & 0xFFFFu));
                        const float r1 = x[2 * t + 1] - bf16_to_f32(static_cast<uint16_t>(whi[t] >> 16));
                        wlo[t] = pack_bf16x2(r0, r1);
                    }
                    const bf16x8 khi = __builtin_bit_cast(bf16x8, whi), klo = __builtin_bit_cast(bf16x8, wlo);
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb) {
                        s[kb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(khi, qb[rb][ks], ks ? s[kb][rb] : zero, 0, 0, 0);
                        s[kb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(klo, qb[rb][ks], s[kb][rb], 0, 0, 0);
                    }
                }
            }
            float bias[2][16];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int jj = c0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
                    float bv = -INFINITY;
                    if (jj < nb && !((lds.kept[jj >> 5] >> (jj & 31)) & 1u))
                        bv = __log2f(static_cast<float>(min(BLK, a.N - BLK * jj)));
                    bias[kb][r] = bv;
                }
            bf16x8 pb[4][2];
            softmax_tile<true>(st, s, pb, c2, bias);
            if (COMP == 1) {
                // order-1 weights w = scale * 2^{L - m} / n_j (L without the count bias)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int cc = 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
                            const float x = (bias[kb][r] == -INFINITY) ? 0.f
                                : __builtin_amdgcn_exp2f(s[kb][rb][r] - bias[kb][r] - st.m[rb]) * a.scale;
                            wbuf[cc * (BLK + 1) + 32 * rb + l32] = x;
                        }
            }
            stage_means<false>(VB + static_cast<size_t>(c0) * D, nc, vbuf);
            wave_lds_sync();
            pv_tile(st, vbuf, troff, pb);
            wave_lds_sync();
            stage_means<true>(VB + static_cast<size_t>(c0) * D, nc, vbuf);
            wave_lds_sync();
            pv_tile(st, vbuf, troff, pb);
            wave_lds_sync();
            if (COMP == 1) {
                // O^T += H_j^T (Q^T diag(w_j)) for every compensated block of this tile:
                // the per-row weight scales the B operand, so the MFMA accumulates
                // straight into O.
                const uint16_t* MOM = static_cast<const uint16_t*>(a.kmom);
                for (int cc = 0; cc < nc; ++cc) {
                    const int jj = c0 + cc;
                    if ((lds.kept[jj >> 5] >> (jj & 31)) & 1u) continue;
                    const uint16_t* Hj = MOM + (bh * nb + jj) * static_cast<size_t>(D) * D;
                    const float w[2] = {wbuf[cc * (BLK + 1) + l32], wbuf[cc * (BLK + 1) + 32 + l32]};
                    bf16x8 qs[2][8];
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                        for (int ks = 0; ks < 8; ++ks) {
                            const u32x4 qw = __builtin_bit_cast(u32x4, qb[rb][ks]);
                            u32x4 o;
#pragma unroll
                            for (int t = 0; t < 4; ++t)
                                o[t] = pack_bf16x2(__uint_as_float(qw[t] << 16) * w[rb],
                                                   __uint_as_float(qw[t] & 0xFFFF0000u) * w[rb]);
                            qs[rb][ks] = __builtin_bit_cast(bf16x8, o);
                        }
#pragma unroll
                    for (int db = 0; db < 4; ++db) {
                        bf16x8 ha[8];
#pragma unroll
                        for (int ks = 0; ks < 8; ++ks)
                            ha[ks] = *reinterpret_cast<const bf16x8*>(Hj + (32 * db + l32) * D + 16 * ks + 8 * h);
#pragma unroll
                        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
                            for (int rb = 0; rb < 2; ++rb)
                                st.o[db][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ha[ks], qs[rb][ks], st.o[db][rb], 0, 0, 0);
                    }
                }
                wave_lds_sync();
            }
        }
    }

    // ---- normalise and write O (bf16) and lse ----
    uint16_t* O = static_cast<uint16_t*>(a.out) + head;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const float lt = st.l[rb] + swap_halves(st.l[rb]);
        const float le = st.le[rb] + swap_halves(st.le[rb]);
        const int row = qa * BLK + 32 * rb + l32;
        const bool valid = row < a.N;
        const float inv = valid ? 1.0f / lt : 0.f;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int dd = 32 * db + 8 * q4 + 4 * h;
                uint2 w;
                w.x = pack_bf16x2(st.o[db][rb][4 * q4 + 0] * inv, st.o[db][rb][4 * q4 + 1] * inv);
                w.y = pack_bf16x2(st.o[db][rb][4 * q4 + 2] * inv, st.o[db][rb][4 * q4 + 3] * inv);
                *reinterpret_cast<uint2*>(O + static_cast<size_t>(row) * D + dd) = w;
            }
        }
        if (a.lse && h == 0) a.lse[bh * a.N_pad + row] = valid ? (st.m[rb] + __log2f(le)) * LN2 : 0.f;
    }
}

template <int COMP, bool SKIM>
hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
    const int nq = a.N_pad / BLK;
    dim3 grid(nq * a.H * a.B);
    hipLaunchKernelGGL((fwd_bf16_kernel<COMP, SKIM>), grid, dim3(64), 0, s, a);
    return hipGetLastError();
}

template <bool SKIM>
hipError_t launch_c(const FwdArgs& a, hipStream_t s) {
    switch (a.comp) {
        case -1: return launch_t<-1, SKIM>(a, s);
        case 0: return launch_t<0, SKIM>(a, s);
        default: return launch_t<1, SKIM>(a, s);
    }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) {
    const bool skim = a.idx2 != nullptr && a.cap2 > 0;
    return skim ? launch_c<true>(a, s) : launch_c<false>(a, s);
}

}  // namespace sa
