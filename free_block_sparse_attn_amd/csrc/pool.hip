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

// Centroid planes of one (b, h): plane p row j at cent + ((bh * 4 + p) * nbc + j) * D.
__device__ __forceinline__ uint16_t* cent_row(void* cent, size_t bh, int plane, int nbc, int j, int D) {
    return static_cast<uint16_t*>(cent) + ((bh * 4 + plane) * nbc + static_cast<size_t>(j)) * D;
}

// bf16 high part and residual of an fp32 mean (m - hi is exact in fp32).
__device__ __forceinline__ void split_hi_lo(float m, uint16_t& hi, uint16_t& lo) {
    hi = f32_to_bf16(m);
    lo = f32_to_bf16(m - bf16_to_f32(hi));
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

// Block exponent of the e4m3 copies: smallest e with amax * 2^-e <= 448.
// amax = f * 2^k, f in [0.5, 1): 448 * 2^(k-9) = 0.875 * 2^k.
__device__ __forceinline__ int e4m3_block_exponent(float amax) {
    if (!(amax > 0.0f)) return 0;
    int k;
    float f = frexpf(amax, &k);
    return (f <= 0.875f) ? k - 9 : k - 8;
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
        // product keeps ~16 mantissa bits.
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
            // MFMA A-operand order of the forward pass: element (o, i) of H_j^T
            // at ((o/32 * 8 + i/16) * 64 + o%32 + 32 (i/8 % 2)) * 8 + i%8, so each
            // (32-row d block, 16-wide i step) operand is 1 KiB contiguous
            uint16_t* mom = static_cast<uint16_t*>(a.kmom) + (bh * nb + j) * static_cast<size_t>(D) * D;
            const int ks = icol >> 4, hi8 = (icol >> 3) & 1, e8 = icol & 7;
#pragma unroll
            for (int ob = 0; ob < 4; ++ob) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int o32 = 8 * (r >> 2) + 4 * hl + (r & 3);
                    mom[((ob * 8 + ks) * 64 + o32 + 32 * hi8) * 8 + e8] = f32_to_bf16(acc[ob][r]);
                }
            }
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
constexpr int HBAR_PARTS = 64;

// Adds block j's centred moment G[o][i] = sum_n v_n[o] (k_n[i] - kbar_j[i])
// to the workgroup's fp32 MFMA accumulators: wave w, lane l holds column
// i = 32 w + l % 32 and rows o = 32 ob + 8 (r / 4) + 4 ((l / 32) % 2) + r % 4 of
// acc[ob][r].  The centred keys are split into bf16 hi + lo parts, so the
// products carry about 16 bits of each key deviation (fp32 accumulation).
// xt: 2 * D * TPITCH bf16 of LDS, kb_s: D floats of LDS.
__device__ __forceinline__ void add_block_moment(const PoolArgs& a, size_t bh, int j, uint16_t* xt, float* kb_s,
                                                 f32x16 (&acc)[4]) {
    constexpr int D = 128;
    using E = Elem<uint16_t>;
    constexpr int CPR = D / 8;
    constexpr int PT = BLK * CPR / THREADS;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, hl = l >> 5, l32 = l & 31;
    const int nb = a.N_pad / BLK;
    const int icol = 32 * w + l32;
    const uint16_t* src[2] = {static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v)};
    const int n = min(BLK, a.N - BLK * j);
    const size_t tok0 = (bh * a.N_pad + static_cast<size_t>(j) * BLK) * D;
    u32x4 reg[2][PT];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q = 0; q < PT; ++q) {
            const int chunk = tid + THREADS * q;
            const int row = chunk / CPR, col0 = (chunk % CPR) * 8;
            u32x4 z = {0u, 0u, 0u, 0u};
            if (row < n) z = *reinterpret_cast<const u32x4*>(src[t] + tok0 + static_cast<size_t>(row) * D + col0);
            reg[t][q] = z;
        }
    const float kbj = tid < D ? a.kbar[(bh * nb + j) * D + tid] : 0.0f;
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

__global__ __launch_bounds__(THREADS) void hbar_reduce_kernel(PoolArgs a) {
    constexpr int D = 128;
    const size_t bh = blockIdx.x;
    const int nb = a.N_pad / BLK;
    const float* part = a.hbar_ws + bh * HBAR_PARTS * static_cast<size_t>(D) * D;
    for (int e = threadIdx.x; e < D * D; e += THREADS) {
        double sum = 0.0;
        for (int c = 0; c < HBAR_PARTS; ++c) sum += static_cast<double>(part[static_cast<size_t>(c) * D * D + e]);
        a.hbar[bh * D * D + e] = static_cast<float>(sum / static_cast<double>(nb));
    }
}

// PISA's covariance-aware routing statistic ("PISA ...", section 2, "Routage
// Sensible a la Covariance"): M_j = ||H_j - H_bar||_2, written as ln M_j.
// One workgroup per (block, head): the block's moment is rebuilt in MFMA
// accumulators (never stored), H_bar subtracted, and the deviation parked in
// LDS as fp32 value-major Dm[o][i], from which each thread keeps an 8 x 8 tile
// in registers.  M_j^2 is the largest eigenvalue of A = Dm^T Dm, found by
// COV_STEPS steps of the Lanczos recurrence on A (two tile products per step,
// partial sums combined across tiles in a fixed order through LDS, so the
// result is deterministic) and then the largest eigenvalue of the Lanczos
// tridiagonal by 64-point multisection with Sturm counts.  Lanczos converges
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
        d = al[k] - x - (k > 0 ? be[k - 1] * be[k - 1] / d : 0.0f);
        if (fabsf(d) < 1e-30f) d = -1e-30f;
        c += d < 0.0f;
    }
    return c;
}

__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(3, 3))) void cov_norm_kernel(PoolArgs a) {
    constexpr int D = 128;
    // the block staging, then half of Dm at a time (rows 64 hf .. 64 hf + 63)
    __shared__ __attribute__((aligned(16))) uint16_t stage[2 * D * TPITCH];
    constexpr int PP = D + 4;                 // padded partial-sum rows: the 16 column tiles' writes hit distinct banks
    __shared__ float part[16 * PP];
    __shared__ float yv_s[D], wv_s[D];
    __shared__ float red2[2][2];              // per-step wave partials of |y|^2 and |w|^2
    __shared__ float kb_s[D];
    __shared__ float al[COV_STEPS], be[COV_STEPS];
    float* dmh = reinterpret_cast<float*>(stage);
    static_assert(64 * D * sizeof(float) <= sizeof(stage), "half of Dm fits the staging buffer");
    const int j = blockIdx.x;
    const size_t bh = blockIdx.y;
    const int tid = threadIdx.x, l = tid & 63, hl = l >> 5;
    const int icol = 32 * (tid >> 6) + (l & 31);
    const int nb = a.N_pad / BLK;
    f32x16 acc[4];
#pragma unroll
    for (int ob = 0; ob < 4; ++ob) acc[ob] = f32x16{};
    add_block_moment(a, bh, j, stage, kb_s, acc);
    const float* hb = a.hbar + bh * D * D;
#pragma unroll
    for (int ob = 0; ob < 4; ++ob)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[ob][r] -= hb[(32 * ob + 8 * (r >> 2) + 4 * hl + (r & 3)) * D + icol];
    // thread tile: rows o = 8 tr + u, columns i = 8 tc + v, moved over in two row halves
    const int tr = tid >> 4, tc = tid & 15;
    float t[8][8];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        __syncthreads();                      // the staging / previous half is consumed
#pragma unroll
        for (int ob = 2 * hf; ob < 2 * hf + 2; ++ob)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                dmh[(32 * (ob - 2 * hf) + 8 * (r >> 2) + 4 * hl + (r & 3)) * D + icol] = acc[ob][r];
        __syncthreads();
        if ((tr >> 3) == hf) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float* row = dmh + (8 * (tr & 7) + u) * D + 8 * tc;
                const f32x4 lo = *reinterpret_cast<const f32x4*>(row);
                const f32x4 hi = *reinterpret_cast<const f32x4*>(row + 4);
#pragma unroll
                for (int v = 0; v < 4; ++v) { t[u][v] = lo[v]; t[u][v + 4] = hi[v]; }
            }
        }
    }
    // Lanczos start q_1 = x / |x|, x_i = 1 + frac(0.618034 i); q_0 = 0.  Thread
    // i < 128 keeps q_i and q_prev_i; the new q reaches every tile through wv_s.
    float n0 = 0.0f;
    for (int i = 0; i < D; ++i) {
        const float fi = static_cast<float>(i) * 0.618034f;
        const float xi = 1.0f + (fi - floorf(fi));
        n0 += xi * xi;
    }
    const float inv0 = rsqrtf(n0);
    float qi = 0.0f, qpi = 0.0f;
    if (tid < D) {
        const float fi = static_cast<float>(tid) * 0.618034f;
        qi = (1.0f + (fi - floorf(fi))) * inv0;
    }
    float x[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const float fi = static_cast<float>(8 * tc + v) * 0.618034f;
        x[v] = (1.0f + (fi - floorf(fi))) * inv0;
    }
    int steps = 0;
    float beta = 0.0f;
    // Four barriers per step (column sums, y to every tile, row sums, w to
    // every tile); the squared norms ride on the second and fourth as wave
    // partials.
    for (int k = 0; k < COV_STEPS; ++k) {
        // y = Dm q: partial sums over this tile's columns, summed over the 16 column tiles
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            float p = 0.0f;
#pragma unroll
            for (int v = 0; v < 8; ++v) p = fmaf(t[u][v], x[v], p);
            part[tc * PP + 8 * tr + u] = p;
        }
        __syncthreads();
        float y = 0.0f;
        if (tid < D) {
#pragma unroll
            for (int c = 0; c < 16; ++c) y += part[c * PP + tid];
            yv_s[tid] = y;
            float y2 = y * y;                 // alpha = q^T A q = |Dm q|^2: wave partials
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) y2 += __shfl_xor(y2, off);
            if ((tid & 63) == 0) red2[0][tid >> 6] = y2;
        }
        __syncthreads();
        const float alpha = red2[0][0] + red2[0][1];
        // w = Dm^T y - alpha q - beta q_prev: partial sums over this tile's rows
        float yy[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) yy[u] = yv_s[8 * tr + u];
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            float p = 0.0f;
#pragma unroll
            for (int u = 0; u < 8; ++u) p = fmaf(t[u][v], yy[u], p);
            part[tr * PP + 8 * tc + v] = p;
        }
        __syncthreads();
        float w = 0.0f;
        if (tid < D) {
#pragma unroll
            for (int r = 0; r < 16; ++r) w += part[r * PP + tid];
            w = w - alpha * qi - beta * qpi;
            wv_s[tid] = w;
            float w2 = w * w;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) w2 += __shfl_xor(w2, off);
            if ((tid & 63) == 0) red2[1][tid >> 6] = w2;
        }
        __syncthreads();
        beta = sqrtf(red2[1][0] + red2[1][1]);
        if (tid == 0) { al[k] = alpha; be[k] = beta; }
        steps = k + 1;
        if (!(beta > alpha * 0x1p-20f)) break;    // invariant subspace (or A = 0): T is exact
        const float ib = 1.0f / beta;
        qpi = qi;
        qi = w * ib;
#pragma unroll
        for (int v = 0; v < 8; ++v) x[v] = wv_s[8 * tc + v] * ib;
    }
    __syncthreads();
    if (tid < 64) {
        // largest eigenvalue of T: Gershgorin bracket, then five rounds of
        // 64-point multisection (lane p tests lo + (p + 1) (hi - lo) / 64)
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
        if (tid == 0) {
            const bool zero = al[0] == 0.0f && steps == 1;
            a.kcov[bh * nb + j] = zero ? -INFINITY : 0.5f * logf(hi);
        }
    }
}

template <typename T, int D>
hipError_t launch_pool_t(const PoolArgs& a, hipStream_t s) {
    if (!a.kmom && !a.klam && !a.q8 && !a.q4) {
        constexpr int BPW = 64 / (D / Elem<T>::PER16);
        const int nb = a.N_pad / BLK;
        const int rows = a.cent ? BLK * ((nb + BLK - 1) / BLK) : nb;   // centroid pad rows too
        dim3 grid((rows + 4 * BPW - 1) / (4 * BPW), 3, a.B * a.H);
        hipLaunchKernelGGL((pool_means_kernel<T, D>), grid, dim3(256), 0, s, a);
        return hipGetLastError();
    }
    const size_t lds = pool_lds<T, D>();
    const int nb = a.N_pad / BLK;
    dim3 grid(a.cent ? BLK * ((nb + BLK - 1) / BLK) : nb, a.H, a.B);
    hipLaunchKernelGGL((pool_kernel<T, D>), grid, dim3(THREADS), lds, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const PoolArgs& a, bool bf16, hipStream_t s) {
    hipError_t e;
    if (bf16) e = a.d == 128 ? launch_pool_t<uint16_t, 128>(a, s) : launch_pool_t<uint16_t, 64>(a, s);
    else e = a.d == 128 ? launch_pool_t<float, 128>(a, s) : launch_pool_t<float, 64>(a, s);
    if (e != hipSuccess || !a.hbar) return e;
    // after the means (the centring uses kbar)
    hipLaunchKernelGGL(hbar_partial_kernel, dim3(HBAR_PARTS, a.B * a.H), dim3(THREADS), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(hbar_reduce_kernel, dim3(a.B * a.H), dim3(THREADS), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess || !a.kcov) return e;
    hipLaunchKernelGGL(cov_norm_kernel, dim3(a.N_pad / BLK, a.B * a.H), dim3(THREADS), 0, s, a);
    return hipGetLastError();
}

}  // namespace sa
