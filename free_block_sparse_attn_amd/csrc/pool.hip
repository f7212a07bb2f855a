// Block pooling: means (routing features), key counts and the optional
// per-block statistics the forward pass and the routers read.
//
// Page basis: PISA ("PISA: Piecewise Sparse Attention Is Wiser for Efficient
// Diffusion Transformers", section 2, "Implementation Materielle") precomputes
// block centroids, value sums and per-block first-order matrices before the
// attention pass; SVG-EAR (section 2A) approximates skipped blocks by their
// means; Triage's router works from block statistics.
//
// One workgroup (4 waves) per (b, h, block).  The kernel is HBM-bound: every
// token row is read once with 16-byte coalesced loads and parked in LDS in a
// column-major (transposed) layout, so that per-column sums, the moment MFMAs
// and the spreads all read contiguous LDS runs.
#include "common.h"
#include "launch.h"
#include "lds_tile.h"

#include <mutex>

// the device library's wavefront sum (DPP, a fixed order)
extern "C" __device__ float __ockl_wfred_add_f32(float);

namespace sa {

namespace {

template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int PER16 = 4;
    static __device__ __forceinline__ float get(const u32x4& r, int e) { return __uint_as_float(r[e]); }
    static __device__ __forceinline__ float raw(const u32x4& r, int e) { return __uint_as_float(r[e]); }
    static __device__ __forceinline__ float val(float x) { return x; }
};
template <> struct Elem<uint16_t> {
    static constexpr int PER16 = 8;
    static __device__ __forceinline__ float get(const u32x4& r, int e) {
        uint32_t w = r[e >> 1];
        return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
    }
    static __device__ __forceinline__ uint16_t raw(const u32x4& r, int e) {
        return static_cast<uint16_t>((e & 1) ? (r[e >> 1] >> 16) : (r[e >> 1] & 0xFFFFu));
    }
    static __device__ __forceinline__ float val(uint16_t x) { return bf16_to_f32(x); }
};

constexpr int THREADS = 256;
constexpr int HBAR_PARTS = 64;    // partial sums of PISA's H_bar per head (blocks j = c mod 64)

// Centroid planes of one (b, h): plane p row j at cent + ((bh * 4 + p) * nbc + j) * D.
__device__ __forceinline__ uint16_t* cent_row(void* cent, size_t bh, int plane, int nbc, int j, int D) {
    return static_cast<uint16_t*>(cent) + ((bh * 4 + plane) * nbc + static_cast<size_t>(j)) * D;
}

// fp16 high part and rounded residual of an fp32 mean (m - hi is exact in
// fp32), so hi + lo carries m to about 22 bits.
__device__ __forceinline__ void split_hi_lo(float m, uint16_t& hi, uint16_t& lo) {
    hi = f32_to_f16(m);
    lo = f32_to_f16(m - f16_to_f32(hi));
}

// fp16 copy of one 16-byte chunk of bf16 values (8 elements), RNE.
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(const u32x4& r) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_f16x2(__uint_as_float(r[e] << 16), __uint_as_float(r[e] & 0xFFFF0000u));
    return w;
}

// Exponent e of the fp16 moment copy H_j 2^-e: amax 2^-e in [2^14, 2^15)
// (0 for an all-zero block), so the largest entry keeps 11 bits and the
// copy never overflows.
__device__ __forceinline__ int f16_block_exponent(float amax) {
    if (!(amax > 0.0f)) return 0;
    int k;
    frexpf(amax, &k);                  // amax in [2^(k-1), 2^k)
    return min(max(k - 15, -100), 100);
}
constexpr int TPITCH = BLK + 8;     // transposed row pitch in elements (16-byte multiple)

template <typename T, int D>
constexpr size_t pool_lds() { return 3 * D * TPITCH * sizeof(T) + (3 * D + 64) * sizeof(float); }

// MXFP4 block exponent: smallest e with amax * 2^-e <= 6 (amax = f 2^k,
// f in [0.5, 1): 6 = 0.75 * 2^3), kept within the E8M0 range.
__device__ __forceinline__ int fp4_block_exponent(float amax) {
    if (!(amax > 0.0f)) return 0;
    int k;
    const float f = frexpf(amax, &k);
    return max((f <= 0.75f) ? k - 3 : k - 2, -127);
}

// E2M1 code of y (|y| <= 6 by the scale rule), nearest with ties to the even
// code: the decision points 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 alternate
// between rounding down and up at the tie.  Magnitude 0 is +0.
__device__ __forceinline__ uint32_t e2m1_code(float y) {
    const float a = fabsf(y);
    const uint32_t m = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) +
                       (a > 5.0f);
    return m | ((y < 0.0f && m != 0u) ? 8u : 0u);
}

// E2M1 codes of two values (|x| <= 6) in the low byte, x0 in the low nibble,
// by the hardware conversion (round to nearest, ties to the even code: the
// same decisions as e2m1_code); a magnitude-0 code is made +0 (the conversion
// keeps the sign of a negative value that rounds to zero).
__device__ __forceinline__ uint32_t e2m1_pair(float x0, float x1) {
    uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x0, x1, 1.0f, 0) & 0xFFu;
    const uint32_t z0 = (c & 0x07u) == 0u ? 0x08u : 0u;
    const uint32_t z1 = (c & 0x70u) == 0u ? 0x80u : 0u;
    return c & ~(z0 | z1);
}

// Maximum over each 16-lane row of the wave (DPP row rotations; every lane
// of the row gets it).
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false)));  // row_ror:8
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false)));  // row_ror:4
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false)));  // row_ror:2
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false)));  // row_ror:1
    return x;
}

// Block exponent of the e4m3 copies: smallest e with amax * 2^-e <= 448.
// amax = f * 2^k, f in [0.5, 1): 448 * 2^(k-9) = 0.875 * 2^k.
__device__ __forceinline__ int e4m3_block_exponent(float amax) {
    if (!(amax > 0.0f)) return 0;
    int k;
    float f = frexpf(amax, &k);
    return (f <= 0.875f) ? k - 9 : k - 8;
}

// The fp16 copy H_j 2^-e of one block's moment (d = 128) from the four
// waves' accumulators (wave w: key columns 32 w .. 32 w + 31, value rows in
// four 32-row blocks; accumulator entry r of lane l: row 8 (r/4) + 4 (l/32)
// + r % 4, column l % 32): the block exponent e (largest entry in
// [2^14, 2^15)) from the maxima the waves leave in red4[0..3], then every
// element in the forward pass's MFMA A-operand order.
__device__ __forceinline__ void store_moment(const PoolArgs& a, const f32x16 acc[4], float* red4, int w,
                                             size_t blk) {
    constexpr int D = 128;
    const int l = threadIdx.x & 63, hl = l >> 5;
    float am = 0.0f;
#pragma unroll
    for (int ob = 0; ob < 4; ++ob)
#pragma unroll
        for (int r = 0; r < 16; ++r) am = fmaxf(am, fabsf(acc[ob][r]));
    for (int off = 32; off > 0; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
    if (l == 0) red4[w] = am;
    __syncthreads();
    am = fmaxf(fmaxf(red4[0], red4[1]), fmaxf(red4[2], red4[3]));
    const int ex = f16_block_exponent(am);
    if (threadIdx.x == 0) a.kmom_exp[blk] = static_cast<int8_t>(ex);
    // element (o, i) of H_j^T at ((o/32 * 8 + i/16) * 64 + o%32 + 32 (i/8 % 2))
    // * 8 + i%8, so each (32-row d block, 16-wide i step) operand is 1 KiB
    // contiguous
    const int icol = 32 * w + (l & 31);
    uint16_t* mom = static_cast<uint16_t*>(a.kmom) + blk * static_cast<size_t>(D) * D;
    const int ks = icol >> 4, hi8 = (icol >> 3) & 1, e8 = icol & 7;
#pragma unroll
    for (int ob = 0; ob < 4; ++ob) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int o32 = 8 * (r >> 2) + 4 * hl + (r & 3);
            mom[((ob * 8 + ks) * 64 + o32 + 32 * hi8) * 8 + e8] = f32_to_f16(ldexpf(acc[ob][r], -ex));
        }
    }
}

template <typename T, int D>
__global__ __launch_bounds__(THREADS) void pool_kernel(PoolArgs a) {
    using E = Elem<T>;
    constexpr int PER16 = E::PER16;
    constexpr int CPR = D / PER16;                 // 16-byte chunks per row
    constexpr int CHUNKS = BLK * CPR;              // chunks per tensor tile
    constexpr int PT = CHUNKS / THREADS;           // chunks per thread per tensor
    static_assert(CHUNKS % THREADS == 0, "tile must split evenly");

    // Transposed staging in the input dtype: xt[tensor][col][token]
    extern __shared__ __attribute__((aligned(16))) char smem[];
    T* xt = reinterpret_cast<T*>(smem);                                          // 3 * D * TPITCH
    float* means = reinterpret_cast<float*>(smem + 3 * D * TPITCH * sizeof(T));  // 3 * D
    float* red = means + 3 * D;                    // 64 scratch floats for reductions

    const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int nb = a.N_pad / BLK;
    const int nbc = BLK * ((nb + BLK - 1) / BLK);
    const size_t bh = static_cast<size_t>(b) * a.H + h;
    if (j >= nb) {
        // centroid pad rows (only launched when cent is requested)
        for (int x = tid; x < 4 * D; x += THREADS) cent_row(a.cent, bh, x / D, nbc, j, D)[x % D] = 0;
        return;
    }
    const int n = min(BLK, a.N - BLK * j);
    const size_t tok0 = (bh * a.N_pad + static_cast<size_t>(j) * BLK) * D;

    const T* src[3] = {static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v)};

    // Phase 1: coalesced 16-byte row loads (pad rows read as zero).
    u32x4 reg[3][PT];
#pragma unroll
    for (int t = 0; t < 3; ++t) {
#pragma unroll
        for (int c = 0; c < PT; ++c) {
            const int chunk = tid + THREADS * c;
            const int row = chunk / CPR;
            const int col0 = (chunk % CPR) * PER16;
            u32x4 z = {0u, 0u, 0u, 0u};
            if (row < n)
                z = *reinterpret_cast<const u32x4*>(src[t] + tok0 + static_cast<size_t>(row) * D + col0);
            reg[t][c] = z;
        }
    }
    // fp16 copy of V (bf16, d = 128); pad rows were loaded as zero
    if constexpr (sizeof(T) == 2 && D == 128) {
        if (a.v16) {
#pragma unroll
            for (int c = 0; c < PT; ++c) {
                const int chunk = tid + THREADS * c;
                const int row = chunk / CPR;
                const int col0 = (chunk % CPR) * PER16;
                *reinterpret_cast<u32x4*>(a.v16 + tok0 + static_cast<size_t>(row) * D + col0) = bf16x8_to_f16x8(reg[2][c]);
            }
        }
    }
    // transposed staging
#pragma unroll
    for (int t = 0; t < 3; ++t) {
#pragma unroll
        for (int c = 0; c < PT; ++c) {
            const int chunk = tid + THREADS * c;
            const int row = chunk / CPR;
            const int col0 = (chunk % CPR) * PER16;
#pragma unroll
            for (int e = 0; e < PER16; ++e)
                xt[(t * D + col0 + e) * TPITCH + row] = E::raw(reg[t][c], e);
        }
    }
    __syncthreads();

    // Phase 2: per-column fp64 sums in token order, mean = RN32(sum / n).
    for (int task = tid; task < 3 * D; task += THREADS) {
        const T* col = xt + task * TPITCH;
        double acc = 0.0;
        for (int r = 0; r < n; ++r) acc = acc + static_cast<double>(E::val(col[r]));
        const float m = static_cast<float>(acc / static_cast<double>(n));
        means[task] = m;
        const int t = task / D, i = task % D;
        float* dst = (t == 0) ? a.qbar : (t == 1) ? a.kbar : a.vbar;
        dst[(bh * nb + j) * D + i] = m;
        if (a.cent && t > 0) {
            uint16_t hi, lo;
            split_hi_lo(m, hi, lo);
            cent_row(a.cent, bh, 2 * (t - 1), nbc, j, D)[i] = hi;
            cent_row(a.cent, bh, 2 * (t - 1) + 1, nbc, j, D)[i] = lo;
        }
    }
    if (b == 0 && h == 0 && tid == 0) a.kcount[j] = n;
    __syncthreads();

    // Phase 3 (optional): spreads lambda = ln(r_k r_v), fp64.
    if (a.klam) {
        double part[2] = {0.0, 0.0};
        for (int task = tid; task < 2 * D; task += THREADS) {
            const int t = 1 + task / D;            // K then V
            const T* col = xt + (t * D + task % D) * TPITCH;
            const double mu = static_cast<double>(means[t * D + task % D]);
            double s = 0.0;
            for (int r = 0; r < n; ++r) {
                const double dv = static_cast<double>(E::val(col[r])) - mu;
                s = fma(dv, dv, s);
            }
            part[task / D] += s;
        }
        // wave reduction then across the 4 waves
        for (int p = 0; p < 2; ++p) {
            double v = part[p];
            for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
            part[p] = v;
        }
        double* dred = reinterpret_cast<double*>(red);
        if ((tid & 63) == 0) {
            dred[(tid >> 6) * 2 + 0] = part[0];
            dred[(tid >> 6) * 2 + 1] = part[1];
        }
        __syncthreads();
        if (tid == 0) {
            double rk = 0.0, rv = 0.0;
            for (int w = 0; w < THREADS / 64; ++w) { rk += dred[2 * w]; rv += dred[2 * w + 1]; }
            a.klam[bh * nb + j] = static_cast<float>(0.5 * log(rk) + 0.5 * log(rv));
        }
        __syncthreads();
    }

    if constexpr (sizeof(T) == 2 && D == 128) {
        // Phase 4 (optional): value-major moment kmom[o][i] = sum_n v_n[o] (k_n[i] - kbar[i])
        // via bf16 MFMA 32x32x16; centred keys are split hi + lo so the
        // product keeps ~16 mantissa bits; stored in fp16 with a per-block
        // power-of-two exponent.
        if (a.kmom) {
            const int w = tid >> 6, l = tid & 63, hl = l >> 5, l32 = l & 31;
            const int icol = 32 * w + l32;                 // this wave's i block
            const float kb = means[D + icol];
            f32x16 acc[4];
#pragma unroll
            for (int ob = 0; ob < 4; ++ob) acc[ob] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int t0 = 16 * ks + 8 * hl;
                bf16x8 bhi, blo;
                const T* kc = xt + (D + icol) * TPITCH + t0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = (t0 + e < n) ? E::val(kc[e]) - kb : 0.0f;
                    const __bf16 hi = static_cast<__bf16>(x);
                    bhi[e] = hi;
                    blo[e] = static_cast<__bf16>(x - static_cast<float>(hi));
                }
#pragma unroll
                for (int ob = 0; ob < 4; ++ob) {
                    const bf16x8 av = *reinterpret_cast<const bf16x8*>(xt + (2 * D + 32 * ob + l32) * TPITCH + t0);
                    acc[ob] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bhi, acc[ob], 0, 0, 0);
                    acc[ob] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, blo, acc[ob], 0, 0, 0);
                }
            }
            store_moment(a, acc, red + 48, w, bh * nb + j);   // slots no other phase uses
        }

        // Phase 5 (optional): per-block power-of-two scaled e4m3 copies.
        if (a.q8) {
            uint8_t* dst8[3] = {a.q8, a.k8, a.v8};
            float amax[3] = {0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 3; ++t)
#pragma unroll
                for (int c = 0; c < PT; ++c)
#pragma unroll
                    for (int e = 0; e < PER16; ++e) amax[t] = fmaxf(amax[t], fabsf(E::get(reg[t][c], e)));
#pragma unroll
            for (int t = 0; t < 3; ++t)
                for (int off = 32; off > 0; off >>= 1) amax[t] = fmaxf(amax[t], __shfl_xor(amax[t], off));
            if ((tid & 63) == 0)
                for (int t = 0; t < 3; ++t) red[(tid >> 6) * 3 + t] = amax[t];
            __syncthreads();
            int ex[3];
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                float m = 0.f;
                for (int w = 0; w < THREADS / 64; ++w) m = fmaxf(m, red[w * 3 + t]);
                ex[t] = e4m3_block_exponent(m);
            }
            if (tid < 3) a.exp8[(bh * nb + j) * 3 + tid] = static_cast<int8_t>(ex[tid]);
            // Q and K copies stay row-major
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int c = 0; c < PT; ++c) {
                    const int chunk = tid + THREADS * c;
                    const int row = chunk / CPR;
                    const int col0 = (chunk % CPR) * PER16;
                    uint32_t w0 = 0, w1 = 0;
                    w0 = pack_fp8x2<false>(ldexpf(E::get(reg[t][c], 0), -ex[t]), ldexpf(E::get(reg[t][c], 1), -ex[t]), w0);
                    w0 = pack_fp8x2<true>(ldexpf(E::get(reg[t][c], 2), -ex[t]), ldexpf(E::get(reg[t][c], 3), -ex[t]), w0);
                    w1 = pack_fp8x2<false>(ldexpf(E::get(reg[t][c], 4), -ex[t]), ldexpf(E::get(reg[t][c], 5), -ex[t]), w1);
                    w1 = pack_fp8x2<true>(ldexpf(E::get(reg[t][c], 6), -ex[t]), ldexpf(E::get(reg[t][c], 7), -ex[t]), w1);
                    if (row >= n) { w0 = 0; w1 = 0; }
                    uint2 out = {w0, w1};
                    *reinterpret_cast<uint2*>(dst8[t] + tok0 + static_cast<size_t>(row) * D + col0) = out;
                }
            }
            // V copy block-transposed, [d][64 positions]; position p holds key
            // 32((p%32)/16) + 8((p%16)/4) + 4(p/32) + p%4, the key order of the
            // fp8 P operand in the forward pass.  Pad keys get code 0.
            {
                const int dcol = tid >> 1, p0 = 32 * (tid & 1);
                const T* col = xt + (2 * D + dcol) * TPITCH;
                uint32_t w[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    float x[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int p = p0 + 4 * q + u;
                        const int key = 32 * ((p & 31) >> 4) + 8 * ((p & 15) >> 2) + 4 * (p >> 5) + (p & 3);
                        x[u] = (key < n) ? ldexpf(E::val(col[key]), -ex[2]) : 0.0f;
                    }
                    uint32_t v = pack_fp8x2<false>(x[0], x[1], 0u);
                    w[q] = pack_fp8x2<true>(x[2], x[3], v);
                }
                uint8_t* dstv = a.v8 + ((bh * nb + j) * static_cast<size_t>(D) + dcol) * BLK + p0;
                *reinterpret_cast<u32x4*>(dstv) = u32x4{w[0], w[1], w[2], w[3]};
                *reinterpret_cast<u32x4*>(dstv + 16) = u32x4{w[4], w[5], w[6], w[7]};
            }
        }

        // Phase 6 (optional): MXFP4 copies for the 4-bit skim tier.  Q and K:
        // one E8M0 scale per token and 32 dimensions (the four threads of a
        // 32-wide group combine their maxima); codes packed two per byte,
        // element 2i in the low nibble.  V: block-transposed like v8 (two
        // positions per byte) with one scale per block and dimension.
        if (a.q4) {
            uint8_t* dst4[2] = {a.q4, a.k4};
            uint8_t* sc4[2] = {a.qs4, a.ks4};
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int c = 0; c < PT; ++c) {
                    const int chunk = tid + THREADS * c;
                    const int row = chunk / CPR;
                    const int col0 = (chunk % CPR) * PER16;
                    float x[8];
                    float am = 0.0f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        x[e] = row < n ? E::get(reg[t][c], e) : 0.0f;
                        am = fmaxf(am, fabsf(x[e]));
                    }
                    am = fmaxf(am, __shfl_xor(am, 1));
                    am = fmaxf(am, __shfl_xor(am, 2));
                    const int ex = fp4_block_exponent(am);
                    uint32_t w = 0u;
#pragma unroll
                    for (int e = 0; e < 8; ++e) w |= e2m1_code(ldexpf(x[e], -ex)) << (4 * e);
                    const size_t tok = bh * a.N_pad + static_cast<size_t>(j) * BLK + row;
                    *reinterpret_cast<uint32_t*>(dst4[t] + tok * (D / 2) + col0 / 2) = w;
                    if ((tid & 3) == 0) sc4[t][tok * (D / 32) + col0 / 32] = static_cast<uint8_t>(ex + 127);
                }
            }
            {
                const int dcol = tid >> 1, p0 = 32 * (tid & 1);
                const T* col = xt + (2 * D + dcol) * TPITCH;
                float x[32];
                float am = 0.0f;
#pragma unroll
                for (int q = 0; q < 32; ++q) {
                    const int p = p0 + q;
                    const int key = 32 * ((p & 31) >> 4) + 8 * ((p & 15) >> 2) + 4 * (p >> 5) + (p & 3);
                    x[q] = (key < n) ? E::val(col[key]) : 0.0f;
                    am = fmaxf(am, fabsf(x[q]));
                }
                am = fmaxf(am, __shfl_xor(am, 1));            // the other 32 positions of the column
                const int ex = fp4_block_exponent(am);
                uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int q = 0; q < 32; ++q) w[q >> 3] |= e2m1_code(ldexpf(x[q], -ex)) << (4 * (q & 7));
                const size_t cj = (bh * nb + j) * static_cast<size_t>(D) + dcol;
                *reinterpret_cast<u32x4*>(a.v4 + cj * (BLK / 2) + p0 / 2) = u32x4{w[0], w[1], w[2], w[3]};
                if ((tid & 1) == 0) a.vs4[cj] = static_cast<uint8_t>(ex + 127);
            }
        }
    }
}

// Streaming pooling with the per-block statistics that need no matrix core
// (bf16 inputs, d = 128): one wave per block, lane l owning dimensions 2l
// and 2l + 1.  Each tensor's 64 x 256-byte block is copied into the wave's
// own 16 KiB of LDS by sixteen buffer_load ... lds instructions (no registers
// held while in flight), then read twice, row by row (lane l reads dword l of
// a row: no bank conflicts): pass 1 takes the fp64 column sums of the means
// contract in token order, the block maxima and the fp16 copy of V; pass 2,
// once the block statistics are known, the spreads about the means, the e4m3
// copies (block exponents) and the MXFP4 copies.
constexpr int SW_WAVES = 2;                     // waves (blocks) per workgroup

// Key position p of a block-transposed V copy holding key k (the inverse of
// kappa(p) = 32 ((p % 32) / 16) + 8 ((p % 16) / 4) + 4 (p / 32) + p % 4).
__device__ __forceinline__ constexpr int v8_position(int k) {
    return 32 * ((k >> 2) & 1) + 16 * (k >> 5) + 4 * ((k >> 3) & 3) + (k & 3);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

// Raw buffer descriptor over `bytes` bytes at p (32-bit data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), 0x00020000);
}

// Copy the 16 KiB block at `src` into LDS at `lds`: instruction m moves rows
// 4m .. 4m + 3 (lane l: row 4m + l/16, bytes 16 (l % 16) .. +15).  The
// immediate offset (m % 4) KiB applies to both addresses, so the LDS base and
// the scalar source offset change once per 4 KiB.
template <int M>
__device__ __forceinline__ void block_dma_one(__amdgpu_buffer_rsrc_t rs, uint32_t lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, reinterpret_cast<lds_void*>(static_cast<uintptr_t>(lds + (M >> 2) * 4096)),
                                             16, voff, (M >> 2) * 4096, (M & 3) * 1024, 0);
}

__device__ __forceinline__ void block_dma(__amdgpu_buffer_rsrc_t rs, uint32_t lds, uint32_t voff) {
    block_dma_one<0>(rs, lds, voff);
    block_dma_one<1>(rs, lds, voff);
    block_dma_one<2>(rs, lds, voff);
    block_dma_one<3>(rs, lds, voff);
    block_dma_one<4>(rs, lds, voff);
    block_dma_one<5>(rs, lds, voff);
    block_dma_one<6>(rs, lds, voff);
    block_dma_one<7>(rs, lds, voff);
    block_dma_one<8>(rs, lds, voff);
    block_dma_one<9>(rs, lds, voff);
    block_dma_one<10>(rs, lds, voff);
    block_dma_one<11>(rs, lds, voff);
    block_dma_one<12>(rs, lds, voff);
    block_dma_one<13>(rs, lds, voff);
    block_dma_one<14>(rs, lds, voff);
    block_dma_one<15>(rs, lds, voff);
}

__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <bool Q8, bool Q4>
__global__ __launch_bounds__(64 * SW_WAVES) void pool_stream_kernel(PoolArgs a) {
    constexpr int D = 128;
    __shared__ uint32_t stage[SW_WAVES][BLK * D / 2];
    const int lane = threadIdx.x & 63;
    // block index, wave-uniform (kept in scalar registers, so the buffer
    // descriptors built from it are scalar)
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = blockIdx.x * SW_WAVES + w;
    const int h = blockIdx.y, b = blockIdx.z;
    const int nb = a.N_pad / BLK;
    const int nbc = BLK * ((nb + BLK - 1) / BLK);
    const size_t bh = static_cast<size_t>(b) * a.H + h;
    const int d0 = 2 * lane;
    if (j >= nb) {
        // centroid pad rows
        if (a.cent && j < nbc)
            for (int p = 0; p < 4; ++p) *reinterpret_cast<uint32_t*>(cent_row(a.cent, bh, p, nbc, j, D) + d0) = 0u;
        return;
    }
    const int n = min(BLK, a.N - BLK * j);
    const size_t row0 = bh * a.N_pad + static_cast<size_t>(j) * BLK;      // first token row of the block
    const bool pass2 = Q8 || Q4 || a.klam;
    constexpr uint32_t rowb = 2 * D;
    const uint32_t* buf = stage[w];
    const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(stage[w]));
    const uint32_t dma_off = (lane >> 4) * rowb + 16 * (lane & 15);
    const __amdgpu_buffer_rsrc_t v16r = span_rsrc(a.v16 + row0 * D, BLK * rowb);
    double spread[2] = {0.0, 0.0};

#pragma unroll 1
    for (int t = 0; t < 3; ++t) {
        const uint16_t* src = static_cast<const uint16_t*>(t == 0 ? a.q : t == 1 ? a.k : a.v) + row0 * D;
        wave_lds_fence();                             // the previous tensor's LDS reads are done
        block_dma(span_rsrc(src, n * rowb), lds, dma_off);
        __builtin_amdgcn_s_waitcnt(0x0F70);           // vmcnt(0): the block is in LDS
        if (n < BLK)                                  // ragged tail block: rows n .. 63 read as zero
            for (int r = n; r < BLK; ++r) stage[w][r * (D / 2) + lane] = 0u;
        wave_lds_fence();

        // ---- pass 1: sums in token order, maxima, fp16 copy of V ----
        double s0 = 0.0, s1 = 0.0;
        float am0 = 0.0f, am1 = 0.0f;
#pragma unroll 16
        for (int r = 0; r < BLK; ++r) {
            const uint32_t xr = buf[r * (D / 2) + lane];
            const float lo = __uint_as_float(xr << 16), hi = __uint_as_float(xr & 0xFFFF0000u);
            s0 = s0 + static_cast<double>(lo);          // pad rows add +0.0: exact
            s1 = s1 + static_cast<double>(hi);
            am0 = fmaxf(am0, fabsf(lo));
            am1 = fmaxf(am1, fabsf(hi));
            if (t == 2 && a.v16) __builtin_amdgcn_raw_buffer_store_b32(pack_f16x2(lo, hi), v16r, 4 * lane + r * rowb, 0, 0);
        }
        const float am = wave_max(fmaxf(am0, am1));
        const float m0 = static_cast<float>(s0 / static_cast<double>(n));
        const float m1 = static_cast<float>(s1 / static_cast<double>(n));
        float* dst = (t == 0) ? a.qbar : (t == 1) ? a.kbar : a.vbar;
        *reinterpret_cast<float2*>(dst + (bh * nb + j) * D + d0) = make_float2(m0, m1);
        if (a.cent && t > 0) {
            uint16_t h0, l0, h1, l1;
            split_hi_lo(m0, h0, l0);
            split_hi_lo(m1, h1, l1);
            *reinterpret_cast<uint32_t*>(cent_row(a.cent, bh, 2 * (t - 1), nbc, j, D) + d0) =
                static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
            *reinterpret_cast<uint32_t*>(cent_row(a.cent, bh, 2 * (t - 1) + 1, nbc, j, D) + d0) =
                static_cast<uint32_t>(l0) | (static_cast<uint32_t>(l1) << 16);
        }
        if (!pass2) continue;

        // ---- pass 2 ----
        if (a.klam && t > 0) {
            // spread about the mean, over the block's n tokens in order
            double acc = 0.0;
            const double mm0 = m0, mm1 = m1;
#pragma unroll 8
            for (int r = 0; r < n; ++r) {
                const uint32_t xr = buf[r * (D / 2) + lane];
                const double e0 = static_cast<double>(__uint_as_float(xr << 16)) - mm0;
                const double e1 = static_cast<double>(__uint_as_float(xr & 0xFFFF0000u)) - mm1;
                acc = fma(e1, e1, fma(e0, e0, acc));
            }
            spread[t - 1] = acc;
        }
        const int ex8 = e4m3_block_exponent(am);
        if (Q8 && lane == 0) a.exp8[(bh * nb + j) * 3 + t] = static_cast<int8_t>(ex8);
        if (t == 0 || t == 1) {
            if (!(Q8 || Q4)) continue;
            const __amdgpu_buffer_rsrc_t o8 = span_rsrc((t == 0 ? a.q8 : a.k8) + row0 * D, Q8 ? BLK * D : 0);
            const __amdgpu_buffer_rsrc_t o4 = span_rsrc((t == 0 ? a.q4 : a.k4) + row0 * (D / 2), Q4 ? BLK * D / 2 : 0);
            const __amdgpu_buffer_rsrc_t s4 = span_rsrc((t == 0 ? a.qs4 : a.ks4) + row0 * (D / 32), Q4 ? BLK * D / 32 : 0);
#pragma unroll 16
            for (int r = 0; r < BLK; ++r) {
                const uint32_t xr = buf[r * (D / 2) + lane];
                const float lo = __uint_as_float(xr << 16), hi = __uint_as_float(xr & 0xFFFF0000u);
                if (Q8) {
                    const uint32_t pair = pack_fp8x2<false>(ldexpf(lo, -ex8), ldexpf(hi, -ex8), 0u);
                    __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(pair), o8, 2 * lane + r * D, 0, 0);
                }
                if (Q4) {
                    // one scale per token and 32 dimensions: lanes 16g .. 16g + 15
                    const float gm = row16_max(fmaxf(fabsf(lo), fabsf(hi)));
                    const int e4 = fp4_block_exponent(gm);
                    const uint32_t code = e2m1_pair(ldexpf(lo, -e4), ldexpf(hi, -e4));
                    __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(code), o4, lane + r * (D / 2), 0, 0);
                    if ((lane & 15) == 0)
                        __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(e4 + 127), s4, (lane >> 4) + r * (D / 32), 0, 0);
                }
            }
        } else if (Q8 || Q4) {
            // V copies, block-transposed in key-position order: this lane's two
            // dimensions (64 fp8 codes, or 32 bytes of fp4 codes, each)
            const int ev0 = fp4_block_exponent(am0), ev1 = fp4_block_exponent(am1);   // pad rows are zero
            uint32_t v8w[2][16], v4w[2][8];
#pragma unroll
            for (int q = 0; q < 16; ++q) { v8w[0][q] = 0u; v8w[1][q] = 0u; }
#pragma unroll
            for (int q = 0; q < 8; ++q) { v4w[0][q] = 0u; v4w[1][q] = 0u; }
#pragma unroll
            for (int r = 0; r < BLK; ++r) {
                const uint32_t xr = buf[r * (D / 2) + lane];
                const float lo = __uint_as_float(xr << 16), hi = __uint_as_float(xr & 0xFFFF0000u);
                const int p = v8_position(r);
                if (Q8) {
                    const uint32_t pair = pack_fp8x2<false>(ldexpf(lo, -ex8), ldexpf(hi, -ex8), 0u);
                    v8w[0][p >> 2] |= (pair & 0xFFu) << (8 * (p & 3));
                    v8w[1][p >> 2] |= ((pair >> 8) & 0xFFu) << (8 * (p & 3));
                }
                if (Q4) {
                    const uint32_t c = e2m1_pair(ldexpf(lo, -ev0), ldexpf(hi, -ev1));
                    v4w[0][p >> 3] |= (c & 0xFu) << (4 * (p & 7));
                    v4w[1][p >> 3] |= (c >> 4) << (4 * (p & 7));
                }
            }
            if (Q8) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    uint8_t* dstv = a.v8 + ((bh * nb + j) * static_cast<size_t>(D) + d0 + c) * BLK;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *reinterpret_cast<u32x4*>(dstv + 16 * q) =
                            u32x4{v8w[c][4 * q], v8w[c][4 * q + 1], v8w[c][4 * q + 2], v8w[c][4 * q + 3]};
                }
            }
            if (Q4) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const size_t cj = (bh * nb + j) * static_cast<size_t>(D) + d0 + c;
                    *reinterpret_cast<u32x4*>(a.v4 + cj * (BLK / 2)) = u32x4{v4w[c][0], v4w[c][1], v4w[c][2], v4w[c][3]};
                    *reinterpret_cast<u32x4*>(a.v4 + cj * (BLK / 2) + 16) = u32x4{v4w[c][4], v4w[c][5], v4w[c][6], v4w[c][7]};
                    a.vs4[cj] = static_cast<uint8_t>((c ? ev1 : ev0) + 127);
                }
            }
        }
    }
    if (b == 0 && h == 0 && lane == 0) a.kcount[j] = n;
    if (a.klam) {
        const double rk = wave_sum(spread[0]), rv = wave_sum(spread[1]);
        if (lane == 0) a.klam[bh * nb + j] = static_cast<float>(0.5 * log(rk) + 0.5 * log(rv));
    }
}

// Pooling with the first-order moments (bf16, d = 128): four waves per
// 64-token block.  Q, K and V are copied into LDS in the forward pass's
// swizzled 64-row tile layout (each wave copies 16 rows of each; no
// registers held while in flight).  Waves 0-2 then take the fp64 column sums
// of Q, K and V in token order (lane l: dimensions 2l, 2l + 1, as the
// streaming form) and wave 3 writes the fp16 copy of V.  The moment
// H_j = sum_n v_n (k_n - k_bar_j)^T comes from bf16 MFMAs whose operands are
// both column slices read with the transposed LDS reads: V^T for the value
// rows and the centred keys (split into bf16 high + low parts) for the key
// columns, wave w taking key columns 32 w .. 32 w + 31.
// HBAR false: one block per workgroup, H_j stored in fp16 (kmom).
// HBAR true: workgroup c of a head takes blocks c, c + HBAR_PARTS, ... and
// writes the sum of their H_j to its slot of hbar_ws (PISA's global H_bar,
// reduced by hbar_reduce_kernel), so K and V are read once for the means and
// the moments together.
template <bool HBAR>
__global__ __launch_bounds__(THREADS) void pool_moment_kernel(PoolArgs a) {
    constexpr int D = 128;
    __shared__ __attribute__((aligned(16))) uint8_t tile[3][TILEB];
    __shared__ float kmean[D];
    __shared__ float red[4];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = blockIdx.y, b = blockIdx.z;
    const int nb = a.N_pad / BLK;
    const int nbc = BLK * ((nb + BLK - 1) / BLK);
    const size_t bh = static_cast<size_t>(b) * a.H + h;
    uint32_t off[4], oa[4], ob[4];
    dma_offsets(off);
    pv_offsets(oa, ob);
    f32x16 acc[4];
#pragma unroll
    for (int o = 0; o < 4; ++o) acc[o] = f32x16{};

    // means, fp16 V copy and moment (added to acc) of block j
    auto block = [&](int j) __attribute__((always_inline)) {
        const int n = min(BLK, a.N - BLK * j);
        const size_t row0 = bh * a.N_pad + static_cast<size_t>(j) * BLK;   // first token row of the block
        // wave w copies rows 16 w .. 16 w + 15 of each tensor (rows past n read as 0)
        const uint32_t part = (w >> 1) * HALFB + (w & 1) * 4096;
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            const uint16_t* src = static_cast<const uint16_t*>(t == 0 ? a.q : t == 1 ? a.k : a.v) + row0 * D;
            const __amdgpu_buffer_rsrc_t rs = span_rsrc(src, n * ROWB);
            const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(tile[t])) + part;
            dma_one<0>(rs, lds, part, off);
            dma_one<1>(rs, lds, part, off);
            dma_one<2>(rs, lds, part, off);
            dma_one<3>(rs, lds, part, off);
        }
        wait_vmcnt<0>();
        __syncthreads();
        if (n < BLK) {                               // ragged tail block: rows n .. 63 are zero
#pragma unroll
            for (int t = 0; t < 3; ++t)
                for (int x = tid; x < (BLK - n) * (ROWB / 4); x += THREADS)
                    reinterpret_cast<uint32_t*>(tile[t] + n * ROWB)[x] = 0u;
            __syncthreads();
        }

        if (w < 3) {
            // means of tensor w: sums in token order (pad rows add +0.0: exact)
            const uint8_t* tb = tile[w];
            double s0 = 0.0, s1 = 0.0;
#pragma unroll 16
            for (int r = 0; r < BLK; ++r) {
                const uint32_t xr =
                    *reinterpret_cast<const uint32_t*>(tb + r * ROWB + 16 * swz(r, lane >> 2) + 4 * (lane & 3));
                s0 = s0 + static_cast<double>(__uint_as_float(xr << 16));
                s1 = s1 + static_cast<double>(__uint_as_float(xr & 0xFFFF0000u));
            }
            const int d0 = 2 * lane;
            const float m0 = static_cast<float>(s0 / static_cast<double>(n));
            const float m1 = static_cast<float>(s1 / static_cast<double>(n));
            float* dst = (w == 0) ? a.qbar : (w == 1) ? a.kbar : a.vbar;
            *reinterpret_cast<float2*>(dst + (bh * nb + j) * D + d0) = make_float2(m0, m1);
            if (a.cent && w > 0) {
                uint16_t h0, l0, h1, l1;
                split_hi_lo(m0, h0, l0);
                split_hi_lo(m1, h1, l1);
                *reinterpret_cast<uint32_t*>(cent_row(a.cent, bh, 2 * (w - 1), nbc, j, D) + d0) =
                    static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
                *reinterpret_cast<uint32_t*>(cent_row(a.cent, bh, 2 * (w - 1) + 1, nbc, j, D) + d0) =
                    static_cast<uint32_t>(l0) | (static_cast<uint32_t>(l1) << 16);
            }
            if (w == 1) {
                kmean[d0] = m0;
                kmean[d0 + 1] = m1;
            }
        } else if (a.v16) {
            // fp16 copy of V, 16-byte chunks (pad rows zero)
#pragma unroll 4
            for (int i = 0; i < 16; ++i) {
                const int r = 4 * i + (lane >> 4), c = lane & 15;
                const u32x4 x = *reinterpret_cast<const u32x4*>(tile[2] + r * ROWB + 16 * swz(r, c));
                *reinterpret_cast<u32x4*>(a.v16 + (row0 + r) * D + 8 * c) = bf16x8_to_f16x8(x);
            }
        }
        if (b == 0 && h == 0 && tid == 0) a.kcount[j] = n;
        __syncthreads();                             // kmean

        // H_j[o][i] for key columns i = 32 w + l % 32 and the four 32-row
        // value blocks; both operands walk a 16-row step in the transposed
        // reads' row order, so their reduction indices pair up
        const float kb = kmean[32 * w + (lane & 31)];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int step = (ks >> 1) * HALFB + (ks & 1) * 16 * ROWB;
            const u32x4 kr = __builtin_bit_cast(u32x4, tr_read_pair(tile[1] + step + oa[w], tile[1] + step + ob[w]));
            bf16x8 bhi, blo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t bits = (e & 1) ? (kr[e >> 1] & 0xFFFF0000u) : (kr[e >> 1] << 16);
                const float x = __uint_as_float(bits) - kb;
                const __bf16 hi = static_cast<__bf16>(x);
                bhi[e] = hi;
                blo[e] = static_cast<__bf16>(x - static_cast<float>(hi));
            }
#pragma unroll
            for (int o = 0; o < 4; ++o) {
                const bf16x8 av =
                    __builtin_bit_cast(bf16x8, tr_read_pair(tile[2] + step + oa[o], tile[2] + step + ob[o]));
                acc[o] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bhi, acc[o], 0, 0, 0);
                acc[o] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, blo, acc[o], 0, 0, 0);
            }
        }
    };

    if constexpr (!HBAR) {
        const int j = blockIdx.x;
        if (j >= nb) {
            // centroid pad rows (launched only when cent is requested)
            for (int x = tid; x < 4 * D; x += THREADS) cent_row(a.cent, bh, x / D, nbc, j, D)[x % D] = 0;
            return;
        }
        block(j);
        store_moment(a, acc, red, w, bh * nb + j);
    } else {
        const int c = blockIdx.x;
        if (a.cent && nb + c < nbc)                  // centroid pad row nb + c
            for (int x = tid; x < 4 * D; x += THREADS) cent_row(a.cent, bh, x / D, nbc, nb + c, D)[x % D] = 0;
        for (int j = c; j < nb; j += HBAR_PARTS) {
            block(j);
            __syncthreads();                         // every wave is done with the tiles
        }
        float* dst = a.hbar_ws + (bh * HBAR_PARTS + c) * static_cast<size_t>(D) * D;
        const int icol = 32 * w + (lane & 31), hl = lane >> 5;
#pragma unroll
        for (int o = 0; o < 4; ++o)
#pragma unroll
            for (int r = 0; r < 16; ++r) dst[(32 * o + 8 * (r >> 2) + 4 * hl + (r & 3)) * D + icol] = acc[o][r];
    }
}

// Means-only pooling (no optional statistics): each lane owns one 16-byte
// column chunk of one block of one tensor and folds the block's rows into fp64
// accumulators in token order (the same contract as above).  No LDS, small
// register footprint, many waves in flight: this is the HBM-streaming form.
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_means_kernel(PoolArgs a) {
    using E = Elem<T>;
    constexpr int PER16 = E::PER16;
    constexpr int CPR = D / PER16;                 // chunks per row
    constexpr int BPW = 64 / CPR;                  // blocks per wave
    constexpr int UNROLL = 8;
    const int tensor = blockIdx.y;
    const size_t bh = blockIdx.z;
    const int nb = a.N_pad / BLK;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = (blockIdx.x * 4 + wave) * BPW + lane / CPR;
    const int col0 = (lane % CPR) * PER16;
    const int nbc = BLK * ((nb + BLK - 1) / BLK);
    if (j >= nb) {
        // centroid pad rows (the grid covers nbc blocks when cent is requested)
        if constexpr (sizeof(T) == 2 && D == 128) {
            if (a.cent && tensor > 0 && j < nbc) {
                const u32x4 z = {0u, 0u, 0u, 0u};
                *reinterpret_cast<u32x4*>(cent_row(a.cent, bh, 2 * (tensor - 1), nbc, j, D) + col0) = z;
                *reinterpret_cast<u32x4*>(cent_row(a.cent, bh, 2 * (tensor - 1) + 1, nbc, j, D) + col0) = z;
            }
        }
        return;
    }
    const int n = min(BLK, a.N - BLK * j);
    const T* src = static_cast<const T*>(tensor == 0 ? a.q : tensor == 1 ? a.k : a.v) +
                   (bh * a.N_pad + static_cast<size_t>(j) * BLK) * D + col0;
    double acc[PER16];
#pragma unroll
    for (int e = 0; e < PER16; ++e) acc[e] = 0.0;
    // fp16 copy of V (bf16, d = 128): each lane rewrites its chunk of every row
    uint16_t* v16 = nullptr;
    if constexpr (sizeof(T) == 2 && D == 128) {
        if (a.v16 && tensor == 2) v16 = a.v16 + (bh * a.N_pad + static_cast<size_t>(j) * BLK) * D + col0;
    }
    for (int r0 = 0; r0 < n; r0 += UNROLL) {
        u32x4 x[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            u32x4 z = {0u, 0u, 0u, 0u};
            if (r0 + u < n) z = *reinterpret_cast<const u32x4*>(src + static_cast<size_t>(r0 + u) * D);
            x[u] = z;
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            if (r0 + u < n) {
#pragma unroll
                for (int e = 0; e < PER16; ++e) acc[e] = acc[e] + static_cast<double>(E::get(x[u], e));
            }
        }
        if constexpr (sizeof(T) == 2 && D == 128) {
            if (v16) {
#pragma unroll
                for (int u = 0; u < UNROLL; ++u)
                    if (r0 + u < BLK)
                        *reinterpret_cast<u32x4*>(v16 + static_cast<size_t>(r0 + u) * D) = bf16x8_to_f16x8(x[u]);
            }
        }
    }
    if constexpr (sizeof(T) == 2 && D == 128) {
        // pad rows of the copy (rows the loop above did not reach) are zero
        if (v16) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            for (int r = ((n + UNROLL - 1) / UNROLL) * UNROLL; r < BLK; ++r)
                *reinterpret_cast<u32x4*>(v16 + static_cast<size_t>(r) * D) = z;
        }
    }
    float* dst = (tensor == 0 ? a.qbar : tensor == 1 ? a.kbar : a.vbar) + (bh * nb + j) * D + col0;
    float mv[PER16];
#pragma unroll
    for (int e = 0; e < PER16; ++e) mv[e] = static_cast<float>(acc[e] / static_cast<double>(n));
#pragma unroll
    for (int e = 0; e < PER16; e += 4) {
        const float4 m = {mv[e], mv[e + 1], mv[e + 2], mv[e + 3]};
        *reinterpret_cast<float4*>(dst + e) = m;
    }
    if constexpr (sizeof(T) == 2 && D == 128) {
        if (a.cent && tensor > 0) {
            u32x4 whi, wlo;
#pragma unroll
            for (int e = 0; e < PER16; e += 2) {
                uint16_t h0, l0, h1, l1;
                split_hi_lo(mv[e], h0, l0);
                split_hi_lo(mv[e + 1], h1, l1);
                whi[e >> 1] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
                wlo[e >> 1] = static_cast<uint32_t>(l0) | (static_cast<uint32_t>(l1) << 16);
            }
            *reinterpret_cast<u32x4*>(cent_row(a.cent, bh, 2 * (tensor - 1), nbc, j, D) + col0) = whi;
            *reinterpret_cast<u32x4*>(cent_row(a.cent, bh, 2 * (tensor - 1) + 1, nbc, j, D) + col0) = wlo;
        }
    }
    if (tensor == 0 && bh == 0 && (lane % CPR) == 0) a.kcount[j] = n;
}

// PISA's global first-order statistic H_bar = (1/nb) sum_j H_j (section 2,
// "Algorithme Central").  Pass 1: workgroup (c, bh) accumulates the centred
// moments of blocks j = c, c + 64, ... in fp32 MFMA (the same staging and
// hi + lo split of the centred keys as the per-block moments above) and
// writes its partial G[o][i] = sum_j sum_n v_n[o] (k_n[i] - kbar_j[i]).
// Pass 2 adds the 64 partials of a head in a fixed order (fp64) and divides
// by nb, so H_bar is bit-reproducible.

// Adds block j's centred moment G[o][i] = sum_n v_n[o] (k_n[i] - kbar_j[i])
// to the workgroup's fp32 MFMA accumulators: wave w, lane l holds column
// i = 32 w + l % 32 and rows o = 32 ob + 8 (r / 4) + 4 ((l / 32) % 2) + r % 4 of
// acc[ob][r].  The centred keys are split into bf16 hi + lo parts, so the
// products carry about 16 bits of each key deviation (fp32 accumulation).
// xt: 2 * D * TPITCH bf16 of LDS, kb_s: D floats of LDS.
// This thread's share of block j's K and V rows (zero past the block's valid
// tokens) and of its key mean, in registers.
struct BlockRegs {
    static constexpr int PT = BLK * (128 / 8) / THREADS;
    u32x4 reg[2][PT];
    float kbj;
    int n;                                    // valid tokens of the block
};

__device__ __forceinline__ void load_block(const PoolArgs& a, size_t bh, int j, BlockRegs& br) {
    constexpr int D = 128;
    constexpr int CPR = D / 8;
    const int tid = threadIdx.x;
    const int nb = a.N_pad / BLK;
    const uint16_t* src[2] = {static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v)};
    const int n = min(BLK, a.N - BLK * j);
    const size_t tok0 = (bh * a.N_pad + static_cast<size_t>(j) * BLK) * D;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q = 0; q < BlockRegs::PT; ++q) {
            const int chunk = tid + THREADS * q;
            const int row = chunk / CPR, col0 = (chunk % CPR) * 8;
            u32x4 z = {0u, 0u, 0u, 0u};
            if (row < n) z = *reinterpret_cast<const u32x4*>(src[t] + tok0 + static_cast<size_t>(row) * D + col0);
            br.reg[t][q] = z;
        }
    br.kbj = tid < D ? a.kbar[(bh * nb + j) * D + tid] : 0.0f;
    br.n = n;
}

__device__ __forceinline__ void add_loaded_moment(const BlockRegs& br, uint16_t* xt, float* kb_s, f32x16 (&acc)[4]);

__device__ __forceinline__ void add_block_moment(const PoolArgs& a, size_t bh, int j, uint16_t* xt, float* kb_s,
                                                 f32x16 (&acc)[4]) {
    BlockRegs br;
    load_block(a, bh, j, br);
    add_loaded_moment(br, xt, kb_s, acc);
}

__device__ __forceinline__ void add_loaded_moment(const BlockRegs& br, uint16_t* xt, float* kb_s, f32x16 (&acc)[4]) {
    constexpr int D = 128;
    using E = Elem<uint16_t>;
    constexpr int CPR = D / 8;
    constexpr int PT = BlockRegs::PT;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, hl = l >> 5, l32 = l & 31;
    const int icol = 32 * w + l32;
    const int n = br.n;
    const float kbj = br.kbj;
    const auto& reg = br.reg;
    __syncthreads();                          // every wave is done with the previous staging
    if (tid < D) kb_s[tid] = kbj;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q = 0; q < PT; ++q) {
            const int chunk = tid + THREADS * q;
            const int row = chunk / CPR, col0 = (chunk % CPR) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) xt[(t * D + col0 + e) * TPITCH + row] = E::raw(reg[t][q], e);
        }
    __syncthreads();
    const float kb = kb_s[icol];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int t0 = 16 * ks + 8 * hl;
        bf16x8 bhi, blo;
        const uint16_t* kc = xt + icol * TPITCH + t0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = (t0 + e < n) ? E::val(kc[e]) - kb : 0.0f;
            const __bf16 hi = static_cast<__bf16>(x);
            bhi[e] = hi;
            blo[e] = static_cast<__bf16>(x - static_cast<float>(hi));
        }
#pragma unroll
        for (int ob = 0; ob < 4; ++ob) {
            const bf16x8 av = *reinterpret_cast<const bf16x8*>(xt + (D + 32 * ob + l32) * TPITCH + t0);
            acc[ob] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bhi, acc[ob], 0, 0, 0);
            acc[ob] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, blo, acc[ob], 0, 0, 0);
        }
    }
}

__global__ __launch_bounds__(THREADS) void hbar_partial_kernel(PoolArgs a) {
    constexpr int D = 128;
    __shared__ __attribute__((aligned(16))) uint16_t xt[2 * D * TPITCH];   // K^T, V^T of one block
    __shared__ float kb_s[D];
    const int c = blockIdx.x;
    const size_t bh = blockIdx.y;
    const int l = threadIdx.x & 63, hl = l >> 5;
    const int icol = 32 * (threadIdx.x >> 6) + (l & 31);
    const int nb = a.N_pad / BLK;
    f32x16 acc[4];
#pragma unroll
    for (int ob = 0; ob < 4; ++ob) acc[ob] = f32x16{};
    for (int j = c; j < nb; j += HBAR_PARTS) add_block_moment(a, bh, j, xt, kb_s, acc);
    float* part = a.hbar_ws + (bh * HBAR_PARTS + c) * static_cast<size_t>(D) * D;
#pragma unroll
    for (int ob = 0; ob < 4; ++ob)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int o = 32 * ob + 8 * (r >> 2) + 4 * hl + (r & 3);
            part[o * D + icol] = acc[ob][r];
        }
}

// One workgroup per (head, D*D / HBAR_SLICES elements): each element's 64
// partials added in a fixed order (c = 0 .. 63) whatever the split.
constexpr int HBAR_SLICES = 16;

__global__ __launch_bounds__(THREADS) void hbar_reduce_kernel(PoolArgs a) {
    constexpr int D = 128, PER = D * D / HBAR_SLICES;
    const size_t bh = blockIdx.x;
    const int nb = a.N_pad / BLK;
    const float* part = a.hbar_ws + bh * HBAR_PARTS * static_cast<size_t>(D) * D;
    for (int e = blockIdx.y * PER + threadIdx.x; e < (blockIdx.y + 1) * PER; e += THREADS) {
        double sum = 0.0;
#pragma unroll 16
        for (int c = 0; c < HBAR_PARTS; ++c) sum += static_cast<double>(part[static_cast<size_t>(c) * D * D + e]);
        a.hbar[bh * D * D + e] = static_cast<float>(sum / static_cast<double>(nb));
    }
}

// PISA's covariance-aware routing statistic ("PISA ...", section 2, "Routage
// Sensible a la Covariance"): M_j = ||H_j - H_bar||_2, written as ln M_j.
// One workgroup per (block, head): the block's moment is rebuilt in MFMA
// accumulators (never stored) and H_bar subtracted, so each wave holds 32
// columns of the deviation Dm[o][i] in that layout, plus a copy of them by
// rows (moved through LDS).  M_j^2 is the largest eigenvalue of Dm Dm^T (that
// of Dm^T Dm), found by at most COV_STEPS steps of the Lanczos recurrence
// (per step Dm^T q inside each wave, then Dm y from the four waves' partial
// sums added in a fixed order, so the result is deterministic) and then the
// largest eigenvalue of the Lanczos tridiagonal by 64-point multisection with
// Sturm counts.  Lanczos converges
// with the square root of the relative gap, so blocks whose two top singular
// values are within a few percent (where plain power iteration stalls) still
// come out to fp32 accuracy.  The Ritz value never exceeds M_j^2 beyond
// rounding.
constexpr int COV_STEPS = 32;

// Eigenvalues of the symmetric tridiagonal (diagonal al, off-diagonal be) below x.
__device__ __forceinline__ int sturm_below(const float* al, const float* be, int n, float x) {
    int c = 0;
    float d = 1.0f;
    for (int k = 0; k < n; ++k) {
        d = al[k] - x - (k > 0 ? __fdividef(be[k - 1] * be[k - 1], d) : 0.0f);
        if (fabsf(d) < 1e-30f) d = -1e-30f;
        c += d < 0.0f;
    }
    return c;
}

// Largest eigenvalue of the Lanczos tridiagonal T_steps (wave 0; every lane
// returns it): Gershgorin bracket, then five rounds of 64-point multisection
// (lane p tests lo + (p + 1) (hi - lo) / 64); the upper end of the bracket.
__device__ __forceinline__ float top_ritz(const float* al, const float* be, int steps, int l) {
    float lo = 0.0f, hi = 0.0f;
    for (int k = 0; k < steps; ++k) {
        const float off = (k > 0 ? fabsf(be[k - 1]) : 0.0f) + (k + 1 < steps ? fabsf(be[k]) : 0.0f);
        lo = fmaxf(lo, al[k]);
        hi = fmaxf(hi, al[k] + off);
    }
    hi = hi * (1.0f + 0x1p-20f) + 1e-30f;
    for (int rnd = 0; rnd < 5; ++rnd) {
        const float pt = lo + (hi - lo) * (static_cast<float>(l + 1) * (1.0f / 64.0f));
        const uint64_t all = __ballot(sturm_below(al, be, steps, pt) == steps);
        const int m = all ? __builtin_ctzll(all) : 63;
        const float nhi = __shfl(pt, m);
        const float nlo = m > 0 ? __shfl(pt, m - 1) : lo;
        lo = nlo;
        hi = nhi;
    }
    return hi;
}

// The recurrence stops early once the top Ritz value, taken every
// COV_CHECK steps, moved by at most 2^-15 of itself since the previous check
// (Ritz values rise monotonically towards M_j^2, faster than geometrically
// once they converge, so ln M_j is then within about 2^-16 of its limit).
constexpr int COV_CHECK = 8;

__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(3, 3))) void cov_norm_kernel(PoolArgs a) {
    constexpr int D = 128;
    constexpr int RP = 36;                    // row pitch (floats) of a wave's transposing area
    __shared__ __attribute__((aligned(16))) uint16_t stage[2 * D * TPITCH];
    __shared__ float kb_s[D];
    __shared__ __attribute__((aligned(16))) float qv_s[4][D];      // each wave's copy of q
    __shared__ __attribute__((aligned(16))) float yv_s[4][32];     // each wave's entries of Dm^T q
    __shared__ float part_s[2][4][D + 1];     // per step: Dm y over each wave's columns, then |y|^2 of them
    __shared__ float al_s[COV_STEPS], be_s[COV_STEPS];
    __shared__ float ritz_s;
    __shared__ int stop_s;
    static_assert(4 * 64 * RP * sizeof(float) <= sizeof(stage), "a 64-row half of Dm fits the staging buffer");
    const int j = blockIdx.x;
    const size_t bh = blockIdx.y;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, hl = l >> 5, l32 = l & 31;
    const int icol = 32 * w + l32;
    const int nb = a.N_pad / BLK;
    f32x16 acc[4];
#pragma unroll
    for (int ob = 0; ob < 4; ++ob) acc[ob] = f32x16{};
    add_block_moment(a, bh, j, stage, kb_s, acc);
    // acc[ob][r] = Dm[o][icol], o = 32 ob + 8 (r / 4) + 4 hl + r % 4: wave w holds columns 32 w .. 32 w + 31
    const float* hb = a.hbar + bh * D * D;
#pragma unroll
    for (int ob = 0; ob < 4; ++ob)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[ob][r] -= hb[(32 * ob + 8 * (r >> 2) + 4 * hl + (r & 3)) * D + icol];
    // second copy of the wave's columns by rows: tr[hf][c] = Dm[l + 64 hf][32 w + c],
    // moved through the wave's own part of the staging buffer
    float tr[2][32];
    float* mine = reinterpret_cast<float*>(stage) + w * 64 * RP;
    __syncthreads();                          // every wave is done with the block staging
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int ob = 2 * hf; ob < 2 * hf + 2; ++ob)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                mine[(32 * (ob - 2 * hf) + 8 * (r >> 2) + 4 * hl + (r & 3)) * RP + l32] = acc[ob][r];
        wave_lds_fence();
#pragma unroll
        for (int c4 = 0; c4 < 8; ++c4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(mine + l * RP + 4 * c4);
#pragma unroll
            for (int e = 0; e < 4; ++e) tr[hf][4 * c4 + e] = v[e];
        }
        wave_lds_fence();
    }
    // Lanczos on A = Dm Dm^T (the same nonzero eigenvalues as Dm^T Dm), q over
    // the 128 rows o; start q_o = x_o / |x|, x_o = 1 + frac(0.618034 o).  Lane
    // l keeps q_o and q_prev_o for o = l and l + 64.
    float n0 = 0.0f;
    for (int i = 0; i < D; ++i) {
        const float fi = static_cast<float>(i) * 0.618034f;
        const float xi = 1.0f + (fi - floorf(fi));
        n0 += xi * xi;
    }
    const float inv0 = rsqrtf(n0);
    float q0, q1, qp0 = 0.0f, qp1 = 0.0f;
    {
        const float f0 = static_cast<float>(l) * 0.618034f, f1 = static_cast<float>(l + 64) * 0.618034f;
        q0 = (1.0f + (f0 - floorf(f0))) * inv0;
        q1 = (1.0f + (f1 - floorf(f1))) * inv0;
    }
    float* qs = qv_s[w];
    qs[l] = q0;
    qs[l + 64] = q1;
    wave_lds_fence();
    int steps = 0;
    float beta = 0.0f;
    // One barrier per step: y = Dm^T q stays inside each wave (its own
    // columns); the wave partials of Dm y and |y|^2 are exchanged through LDS
    // and every wave adds them in the same order, so all waves hold the same
    // alpha, beta and q and take the same exits.  Every COV_CHECK steps wave 0
    // alone finds the top Ritz value and shares the stop decision.
    for (int k = 0; k < COV_STEPS; ++k) {
        float pp[4];                          // one chain per 32-row group
#pragma unroll
        for (int ob = 0; ob < 4; ++ob) {
            pp[ob] = 0.0f;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 qv = *reinterpret_cast<const f32x4*>(qs + 32 * ob + 8 * r4 + 4 * hl);
#pragma unroll
                for (int e = 0; e < 4; ++e) pp[ob] = fmaf(acc[ob][4 * r4 + e], qv[e], pp[ob]);
            }
        }
        const float p = (pp[0] + pp[1]) + (pp[2] + pp[3]);
        float po;                                    // the column's other 64 rows (lane l ^ 32)
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p), __float_as_uint(p), false, false);
            po = __uint_as_float(hl ? static_cast<uint32_t>(sw[0]) : static_cast<uint32_t>(sw[1]));
        }
        const float y = hl ? po + p : p + po;
        if (hl == 0) yv_s[w][l32] = y;
        const float y2 = __ockl_wfred_add_f32(hl == 0 ? y * y : 0.0f);
        wave_lds_fence();
        float wa[2][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}};   // two chains per row
#pragma unroll
        for (int c4 = 0; c4 < 8; ++c4) {
            const f32x4 yy = *reinterpret_cast<const f32x4*>(yv_s[w] + 4 * c4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                wa[0][c4 & 1] = fmaf(tr[0][4 * c4 + e], yy[e], wa[0][c4 & 1]);
                wa[1][c4 & 1] = fmaf(tr[1][4 * c4 + e], yy[e], wa[1][c4 & 1]);
            }
        }
        float* pt = part_s[k & 1][w];
        pt[l] = wa[0][0] + wa[0][1];
        pt[l + 64] = wa[1][0] + wa[1][1];
        if (l == 0) pt[D] = y2;
        __syncthreads();
        const float (*ps)[D + 1] = part_s[k & 1];
        const float alpha = ((ps[0][D] + ps[1][D]) + ps[2][D]) + ps[3][D];   // q^T A q = |Dm^T q|^2
        float s0 = ((ps[0][l] + ps[1][l]) + ps[2][l]) + ps[3][l];
        float s1 = ((ps[0][l + 64] + ps[1][l + 64]) + ps[2][l + 64]) + ps[3][l + 64];
        s0 = s0 - alpha * q0 - beta * qp0;
        s1 = s1 - alpha * q1 - beta * qp1;
        beta = sqrtf(__ockl_wfred_add_f32(s0 * s0 + s1 * s1));
        if (tid == 0) {
            al_s[k] = alpha;
            be_s[k] = beta;
        }
        steps = k + 1;
        if (!(beta > alpha * 0x1p-20f)) break;    // invariant subspace (or A = 0): T is exact
        if (steps % COV_CHECK == 0 && steps < COV_STEPS) {
            if (w == 0) {
                wave_lds_fence();                 // al / be of this step
                const float r = top_ritz(al_s, be_s, steps, l);
                if (l == 0) {
                    stop_s = steps > COV_CHECK && r - ritz_s <= r * 0x1p-15f;
                    ritz_s = r;
                }
            }
            __syncthreads();
            if (stop_s) break;
        }
        const float ib = 1.0f / beta;
        qp0 = q0;
        qp1 = q1;
        q0 = s0 * ib;
        q1 = s1 * ib;
        qs[l] = q0;
        qs[l + 64] = q1;
        wave_lds_fence();
    }
    if (w == 0) {
        wave_lds_fence();
        const float hi = top_ritz(al_s, be_s, steps, l);
        if (l == 0) {
            const bool zero = al_s[0] == 0.0f && steps == 1;
            a.kcov[bh * nb + j] = zero ? -INFINITY : 0.5f * logf(hi);
        }
    }
}

template <typename T, int D>
hipError_t launch_pool_t(const PoolArgs& a, hipStream_t s) {
    if constexpr (sizeof(T) == 2 && D == 128) {
        if (!a.kmom && (a.klam || a.q8 || a.q4)) {
            // streaming form for the statistics that need no matrix core
            const int nb = a.N_pad / BLK;
            const int rows = a.cent ? BLK * ((nb + BLK - 1) / BLK) : nb;
            dim3 grid((rows + SW_WAVES - 1) / SW_WAVES, a.H, a.B);
            const dim3 blk(64 * SW_WAVES);
            if (a.q8 && a.q4) hipLaunchKernelGGL((pool_stream_kernel<true, true>), grid, blk, 0, s, a);
            else if (a.q8) hipLaunchKernelGGL((pool_stream_kernel<true, false>), grid, blk, 0, s, a);
            else if (a.q4) hipLaunchKernelGGL((pool_stream_kernel<false, true>), grid, blk, 0, s, a);
            else hipLaunchKernelGGL((pool_stream_kernel<false, false>), grid, blk, 0, s, a);
            return hipGetLastError();
        }
    }
    if (!a.kmom && !a.klam && !a.q8 && !a.q4) {
        constexpr int BPW = 64 / (D / Elem<T>::PER16);
        const int nb = a.N_pad / BLK;
        const int rows = a.cent ? BLK * ((nb + BLK - 1) / BLK) : nb;   // centroid pad rows too
        dim3 grid((rows + 4 * BPW - 1) / (4 * BPW), 3, a.B * a.H);
        hipLaunchKernelGGL((pool_means_kernel<T, D>), grid, dim3(256), 0, s, a);
        return hipGetLastError();
    }
    const int nb = a.N_pad / BLK;
    dim3 grid(a.cent ? BLK * ((nb + BLK - 1) / BLK) : nb, a.H, a.B);
    if constexpr (sizeof(T) == 2 && D == 128) {
        if (a.kmom && !a.klam && !a.q8 && !a.q4) {
            hipLaunchKernelGGL(pool_moment_kernel<false>, grid, dim3(THREADS), 0, s, a);
            return hipGetLastError();
        }
    }
    const size_t lds = pool_lds<T, D>();
    hipLaunchKernelGGL((pool_kernel<T, D>), grid, dim3(THREADS), lds, s, a);
    return hipGetLastError();
}

}  // namespace

// Library-owned scratch of the allocation-free pooling entry point: the H_bar
// partial sums of up to POOL_STATIC_HEADS (b, h) pairs (HBAR_PARTS d x d fp32
// partials each, 128 MiB).  Every GPU the library runs on holds its own copy
// until the process ends; the host only ever uses the address that
// hipGetSymbolAddress returns for the current device.
constexpr size_t POOL_STATIC_FLOATS = static_cast<size_t>(POOL_STATIC_HEADS) * HBAR_PARTS * 128 * 128;
static __device__ __align__(256) float scratch[POOL_STATIC_FLOATS];

float* pool_static_scratch() {
    constexpr int MAX_DEVICES = 64;
    static std::mutex mu;
    static float* addr[MAX_DEVICES] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        addr[dev] = static_cast<float*>(p);
    }
    return addr[dev];
}

hipError_t launch_pool(const PoolArgs& a, bool bf16, hipStream_t s) {
    hipError_t e;
    if (bf16 && a.d == 128 && a.hbar && !a.kmom && !a.klam && !a.q8 && !a.q4) {
        // the means, the fp16 V copy and the H_bar partial sums in one pass over Q, K, V
        hipLaunchKernelGGL(pool_moment_kernel<true>, dim3(HBAR_PARTS, a.H, a.B), dim3(THREADS), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else {
        if (bf16) e = a.d == 128 ? launch_pool_t<uint16_t, 128>(a, s) : launch_pool_t<uint16_t, 64>(a, s);
        else e = a.d == 128 ? launch_pool_t<float, 128>(a, s) : launch_pool_t<float, 64>(a, s);
        if (e != hipSuccess || !a.hbar) return e;
        // after the means (the centring uses kbar)
        hipLaunchKernelGGL(hbar_partial_kernel, dim3(HBAR_PARTS, a.B * a.H), dim3(THREADS), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(hbar_reduce_kernel, dim3(a.B * a.H, HBAR_SLICES), dim3(THREADS), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess || !a.kcov) return e;
    hipLaunchKernelGGL(cov_norm_kernel, dim3(a.N_pad / BLK, a.B * a.H), dim3(THREADS), 0, s, a);
    return hipGetLastError();
}

}  // namespace sa
