// SparsePR's probe-fitted residual reconstruction ("Partition the Support,
// Reconstruct the Residual: ...", section 2B) as a post-pass on the sparse
// output: a few query rows are computed densely, their residual
// R = O_dense - O_sparse is fitted as an affine map of the sparse output,
// R ~ b + x B (ridge regression), the fit is restricted to the leading right
// singular vectors of R, and every other row gets o + (b + o B) P.
//
// Per head, in order on the caller's stream:
//   1. probe_gather_kernel   one probe per query block, row 64 a + ((phase +
//                            37 a) mod n_a): its query into a compact bf16
//                            tile set, its sparse output as fp32
//   2. the fused forward kernel in its dense mode (every key block exact,
//                            fp32 output) on the gathered probe queries, the
//                            key blocks split into chunks over more waves;
//                            combine_kernel merges the chunks by their lse
//   3. gram_kernel           fp64 partial sums of X^T X, X^T R, R^T R and the
//                            column sums over slices of the probes
//   4. fit_kernel            one workgroup per head: fixed-order reduction,
//                            centring, ridge, the top-r subspace V_r of R^T R
//                            (simultaneous iteration with Cholesky QR), then
//                            W = B P = G^{-1} (C V_r) V_r^T by a
//                            Cholesky solve with r right-hand sides (fp64,
//                            packed in LDS) and c = b P = rm P - xm W (fp32 out)
//   5. apply_kernel          o_t <- o_t + c + o_t W on every valid row, the
//                            dense output on probe rows (bf16, in place)
#include "common.h"
#include "launch.h"

namespace sa {

namespace {

constexpr int D = 128;
constexpr int THREADS = 256;
constexpr int NSPLIT = 8;                  // probe slices of the Gram partial sums
constexpr int KSUB = 8;                    // block width of the subspace iteration (rank <= KSUB)
constexpr int SUB_ITERS = 16;

__device__ __forceinline__ int probe_row(int a, int N, int phase) {
    const int n = min(BLK, N - BLK * a);
    return BLK * a + (phase + 37 * a) % n;
}

// ---- 1. gather ----
__global__ __launch_bounds__(THREADS) void probe_gather_kernel(ResidualArgs r) {
    const int nb = r.N_pad / BLK, mp = r.Mp;
    const size_t bh = blockIdx.y;
    const int x = blockIdx.x * THREADS + threadIdx.x;      // (probe, 8-wide chunk)
    if (x >= mp * (D / 8)) return;
    const int a = x / (D / 8), c = (x % (D / 8)) * 8;
    u32x4 qv = {0u, 0u, 0u, 0u}, ov = {0u, 0u, 0u, 0u};
    if (a < nb) {
        const size_t row = bh * r.N_pad + probe_row(a, r.N, r.phase);
        qv = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(r.q) + row * D + c);
        ov = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(r.out) + row * D + c);
    }
    *reinterpret_cast<u32x4*>(r.qp + (bh * mp + a) * D + c) = qv;
    float* xo = r.xp + (bh * mp + a) * D + c;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        xo[2 * e] = bf16_to_f32(static_cast<uint16_t>(ov[e] & 0xFFFFu));
        xo[2 * e + 1] = bf16_to_f32(static_cast<uint16_t>(ov[e] >> 16));
    }
}

// ---- 2b. merge the key chunks: O = sum_c e^{lse_c - lse_max} O_c / sum_c e^{lse_c - lse_max} ----
__global__ __launch_bounds__(THREADS) void combine_kernel(ResidualArgs r) {
    const size_t bh = blockIdx.y;
    const int x = blockIdx.x * THREADS + threadIdx.x;       // (probe row, dimension)
    if (x >= r.Mp * D) return;
    const int row = x / D, col = x % D;
    const size_t rows_per_chunk = static_cast<size_t>(r.B) * r.H * r.Mp;
    const size_t ridx = bh * r.Mp + row;
    float mx = -INFINITY;
    for (int c = 0; c < r.kchunks; ++c) mx = fmaxf(mx, r.lsep[c * rows_per_chunk + ridx]);
    float num = 0.0f, den = 0.0f;
    if (mx > -INFINITY) {
        for (int c = 0; c < r.kchunks; ++c) {
            const float w = __expf(r.lsep[c * rows_per_chunk + ridx] - mx);
            num = fmaf(w, r.odp[(c * rows_per_chunk + ridx) * D + col], num);
            den += w;
        }
    }
    r.od[ridx * D + col] = den > 0.0f ? num / den : 0.0f;
}

// ---- 3. Gram partial sums ----
// Workgroup (slice s, matrix m, head): probes p = s, s + NSPLIT, ...; thread t
// owns entries (i = t / 2, j = 64 (t % 2) .. + 63) of matrix m:
// m = 0: sum x_i x_j, 1: sum x_i r_j, 2: sum r_i r_j (r = o_dense - x).
// Matrix 1's workgroup (u = x, w = r) also sums the columns of x and r.
__global__ __launch_bounds__(THREADS) void gram_kernel(ResidualArgs r) {
    constexpr int STAGE = 8;
    __shared__ double u_s[STAGE][D], w_s[STAGE][D];
    const int s = blockIdx.x, m = blockIdx.y;
    const size_t bh = blockIdx.z;
    const int nb = r.N_pad / BLK, mp = r.Mp;
    const int tid = threadIdx.x, i = tid >> 1, j0 = 64 * (tid & 1);
    double acc[64];
#pragma unroll
    for (int jj = 0; jj < 64; ++jj) acc[jj] = 0.0;
    double colsum = 0.0;                          // m == 1: thread t < 128 sums x_t, t >= 128 sums r_{t-128}
    const float* X = r.xp + bh * mp * D;
    const float* O = r.od + bh * mp * D;
    for (int p0 = s; p0 < nb; p0 += NSPLIT * STAGE) {
        __syncthreads();
        for (int e = tid; e < STAGE * D; e += THREADS) {
            const int q = e / D, col = e % D;
            const int p = p0 + NSPLIT * q;
            double xv = 0.0, rv = 0.0;
            if (p < nb) {
                xv = static_cast<double>(X[static_cast<size_t>(p) * D + col]);
                rv = static_cast<double>(O[static_cast<size_t>(p) * D + col]) - xv;
            }
            u_s[q][col] = (m == 2) ? rv : xv;
            w_s[q][col] = (m == 0) ? xv : rv;
        }
        __syncthreads();
        if (m == 1) {
#pragma unroll
            for (int q = 0; q < STAGE; ++q) colsum += tid < D ? u_s[q][tid] : w_s[q][tid - D];
        }
#pragma unroll 1
        for (int q = 0; q < STAGE; ++q) {
            const double ui = u_s[q][i];
#pragma unroll
            for (int jj = 0; jj < 64; ++jj) acc[jj] = fma(ui, w_s[q][j0 + jj], acc[jj]);
        }
    }
    double* P = r.part + ((bh * NSPLIT + s) * (3 * D * D + 2 * D));
#pragma unroll
    for (int jj = 0; jj < 64; ++jj) P[m * D * D + i * D + j0 + jj] = acc[jj];
    if (m == 1) P[3 * D * D + tid] = colsum;      // x sums then r sums
}

// One thread: Cholesky of the KSUB x KSUB SPD matrix A (row-major) into its
// lower triangle, in registers.
__device__ void chol_small(double* A) {
    double a[KSUB][KSUB];
#pragma unroll
    for (int i = 0; i < KSUB; ++i)
#pragma unroll
        for (int j = 0; j < KSUB; ++j) a[i][j] = A[i * KSUB + j];
#pragma unroll
    for (int k = 0; k < KSUB; ++k) {
        double d = a[k][k];
#pragma unroll
        for (int t = 0; t < k; ++t) d -= a[k][t] * a[k][t];
        d = sqrt(fmax(d, 1e-300));
        a[k][k] = d;
#pragma unroll
        for (int i = k + 1; i < KSUB; ++i) {
            double v = a[i][k];
#pragma unroll
            for (int t = 0; t < k; ++t) v -= a[i][t] * a[k][t];
            a[i][k] = v / d;
        }
    }
#pragma unroll
    for (int i = 0; i < KSUB; ++i)
#pragma unroll
        for (int j = 0; j <= i; ++j) A[i * KSUB + j] = a[i][j];
}

// ---- 4. fit: one workgroup per head ----
// With V_r the top right singular vectors of R, W = B P = G^{-1} (C V_r) V_r^T
// and c = b P = rm P - xm W, so only `rank` right-hand sides are solved.
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

__global__ __launch_bounds__(THREADS) void fit_kernel(ResidualArgs r) {
    constexpr int LP = D * (D + 1) / 2;            // packed lower triangle, row i at i (i + 1) / 2
    __shared__ double Lp[LP];
    __shared__ double Qs[D * KSUB], Ys[D * KSUB];  // subspace blocks; later V_r, C V_r / solutions
    __shared__ double xm[D], rm[D];
    __shared__ double small[KSUB * KSUB];
    __shared__ double red[THREADS / 64];
    const size_t bh = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int nb = r.N_pad / BLK;
    const double M = static_cast<double>(nb);
    double* G = r.mat + bh * 3 * D * D;           // X^T X, then centred
    double* C = G + D * D;                        // X^T R, then centred
    double* S = C + D * D;                        // R^T R
    // reduce the partial sums in a fixed order
    const double* P = r.part + bh * NSPLIT * (3 * D * D + 2 * D);
    for (int e = tid; e < 3 * D * D + 2 * D; e += THREADS) {
        double v = 0.0;
        for (int s = 0; s < NSPLIT; ++s) v += P[static_cast<size_t>(s) * (3 * D * D + 2 * D) + e];
        if (e < 3 * D * D) G[e] = v;
        else if (e < 3 * D * D + D) xm[e - 3 * D * D] = v / M;
        else rm[e - 3 * D * D - D] = v / M;
    }
    __syncthreads();
    double tr = 0.0;
    for (int e = tid; e < D * D; e += THREADS) {
        const int i = e / D, j = e % D;
        G[e] -= M * xm[i] * xm[j];
        C[e] -= M * xm[i] * rm[j];
        if (i == j) tr += G[e];
    }
    tr = wave_sum(tr);
    if (lane == 0) red[wv] = tr;
    __syncthreads();
    const double lam = static_cast<double>(r.ridge) * (red[0] + red[1] + red[2] + red[3]) / D;

    // ---- top-rank subspace of S = R^T R: simultaneous iteration on KSUB
    // columns; after Cholesky QR the first j columns span the leading
    // j-dimensional invariant subspace in the limit, so the first `rank`
    // columns are taken as V_r.  S sits in LDS as fp32 (the space the
    // Cholesky factor takes afterwards). ----
    float* Sf = reinterpret_cast<float*>(Lp);
    static_assert(sizeof(Lp) >= D * D * sizeof(float), "S fits the factor's space");
    for (int e = tid; e < D * D; e += THREADS) Sf[e] = static_cast<float>(S[e]);
    double* Q = Qs;
    double* Y = Ys;
    double* Gs = small;
    for (int e = tid; e < D * KSUB; e += THREADS) {
        const int i = e / KSUB, c = e % KSUB;
        Q[e] = static_cast<double>(((i * 7 + c * 13 + 3) % 17) - 8) + (i == c ? 16.0 : 0.0);
    }
    __syncthreads();
    auto cholqr = [&](int reps) __attribute__((always_inline)) {     // Q <- Q L^{-T}
        for (int rep = 0; rep < reps; ++rep) {
            {
                // Gram entry tid / 4 over rows 32 (tid % 4) .. + 31, four lanes combined
                const int g = tid >> 2, a = g / KSUB, b = g % KSUB, i0 = 32 * (tid & 3);
                double v = 0.0;
                for (int i = i0; i < i0 + 32; ++i) v += Q[i * KSUB + a] * Q[i * KSUB + b];
                v += __shfl_xor(v, 1);
                v += __shfl_xor(v, 2);
                if ((tid & 3) == 0) Gs[g] = v;
            }
            __syncthreads();
            if (tid == 0) chol_small(Gs);
            __syncthreads();
            if (tid < D) {
                double row[KSUB];
#pragma unroll
                for (int c = 0; c < KSUB; ++c) {
                    double v = Q[tid * KSUB + c];
#pragma unroll
                    for (int t = 0; t < c; ++t) v -= row[t] * Gs[c * KSUB + t];
                    row[c] = v / Gs[c * KSUB + c];
                }
#pragma unroll
                for (int c = 0; c < KSUB; ++c) Q[tid * KSUB + c] = row[c];
            }
            __syncthreads();
        }
    };
    static_assert(KSUB * KSUB * 4 == THREADS, "one Gram entry per four threads");
    cholqr(2);
    for (int it = 0; it < SUB_ITERS; ++it) {
        for (int e = tid; e < D * KSUB; e += THREADS) {      // Y = S Q
            const int i = e / KSUB, c = e % KSUB;
            const float* srow = Sf + i * D;
            double v = 0.0;
            for (int l = 0; l < D; ++l) v += static_cast<double>(srow[l]) * Q[l * KSUB + c];
            Y[e] = v;
        }
        __syncthreads();
        for (int e = tid; e < D * KSUB; e += THREADS) Q[e] = Y[e];
        __syncthreads();
        cholqr(it + 1 < SUB_ITERS ? 1 : 2);
    }
    const int rk = r.rank;
    // V_r = the first rank columns of Q, into Y (stride KSUB)
    for (int e = tid; e < D * KSUB; e += THREADS) Y[e] = (e % KSUB) < rk ? Q[e] : 0.0;
    __syncthreads();
    // T = C V_r into Q (the right-hand sides)
    for (int e = tid; e < D * KSUB; e += THREADS) {
        const int i = e / KSUB, c = e % KSUB;
        double v = 0.0;
        if (c < rk)
            for (int l = 0; l < D; ++l) v += C[i * D + l] * Y[l * KSUB + c];
        Q[e] = v;
    }
    __syncthreads();

    // ---- Cholesky of G + lambda I, packed lower triangle in LDS ----
    for (int e = tid; e < D * D; e += THREADS) {
        const int i = e / D, j = e % D;
        if (j <= i) Lp[i * (i + 1) / 2 + j] = G[e] + (i == j ? lam : 0.0);
    }
    __syncthreads();
    for (int k = 0; k < D; ++k) {
        const int kk = k * (k + 1) / 2 + k;
        if (tid == 0) Lp[kk] = sqrt(fmax(Lp[kk], 1e-300));
        __syncthreads();
        const double inv = 1.0 / Lp[kk];
        for (int i = k + 1 + tid; i < D; i += THREADS) Lp[i * (i + 1) / 2 + k] *= inv;
        __syncthreads();
        // trailing update: a thread pair per row i > k, alternate columns j <= i
        const int i = k + 1 + (tid >> 1);
        if (i < D) {
            const int ri = i * (i + 1) / 2;
            const double lik = Lp[ri + k];
            for (int j = k + 1 + (tid & 1); j <= i; j += 2) Lp[ri + j] -= lik * Lp[j * (j + 1) / 2 + k];
        }
        __syncthreads();
    }
    // ---- solve (G + lambda I) Z = T for the rank columns: wave w takes columns
    // w, w + 4, ...; each row's dot product is spread over the 64 lanes ----
    for (int c = wv; c < rk; c += THREADS / 64) {
        for (int i = 0; i < D; ++i) {                        // forward: L y = t (in place in Q)
            const double* li = Lp + i * (i + 1) / 2;
            double part = 0.0;
            for (int t = lane; t < i; t += 64) part += li[t] * Q[t * KSUB + c];
            part = wave_sum(part);
            if (lane == 0) Q[i * KSUB + c] = (Q[i * KSUB + c] - part) / li[i];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        for (int i = D - 1; i >= 0; --i) {                   // backward: L^T z = y
            double part = 0.0;
            for (int t = i + 1 + lane; t < D; t += 64) part += Lp[t * (t + 1) / 2 + i] * Q[t * KSUB + c];
            part = wave_sum(part);
            if (lane == 0) Q[i * KSUB + c] = (Q[i * KSUB + c] - part) / Lp[i * (i + 1) / 2 + i];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }
    __syncthreads();
    // W = Z V_r^T (fp32 out); c = rm P - xm W
    float* Wo = r.wc + bh * (D * D + D);
    for (int e = tid; e < D * D; e += THREADS) {
        const int i = e / D, j = e % D;
        double v = 0.0;
        for (int c = 0; c < rk; ++c) v += Q[i * KSUB + c] * Y[j * KSUB + c];
        Wo[e] = static_cast<float>(v);
        G[e] = v;                                          // W kept in fp64 for c
    }
    __syncthreads();
    if (tid < D) {
        double rp = 0.0;
        for (int c = 0; c < rk; ++c) {
            double t = 0.0;
            for (int l = 0; l < D; ++l) t += rm[l] * Y[l * KSUB + c];
            rp += t * Y[tid * KSUB + c];
        }
        double xw = 0.0;
        for (int i = 0; i < D; ++i) xw += xm[i] * G[i * D + tid];
        Wo[D * D + tid] = static_cast<float>(rp - xw);
    }
}

// ---- 5. apply: 64 rows per workgroup, W in LDS; thread = 4 rows x 8 columns ----
constexpr int APPLY_ROWS = 64;
__global__ __launch_bounds__(THREADS) void apply_kernel(ResidualArgs r) {
    __shared__ __attribute__((aligned(16))) float w_s[D * D];
    __shared__ __attribute__((aligned(16))) float xt_s[D * APPLY_ROWS];    // transposed: [i][row]
    __shared__ float c_s[D];
    const size_t bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int row0 = blockIdx.x * APPLY_ROWS;
    const float* Wg = r.wc + bh * (D * D + D);
    for (int e = 4 * tid; e < D * D; e += 4 * THREADS)
        *reinterpret_cast<f32x4*>(w_s + e) = *reinterpret_cast<const f32x4*>(Wg + e);
    if (tid < D) c_s[tid] = Wg[D * D + tid];
    uint16_t* O = static_cast<uint16_t*>(r.out) + bh * r.N_pad * D;
    for (int e = tid; e < APPLY_ROWS * D / 8; e += THREADS) {
        const int rr = e / (D / 8), c0 = (e % (D / 8)) * 8;
        const u32x4 v = *reinterpret_cast<const u32x4*>(O + static_cast<size_t>(row0 + rr) * D + c0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            xt_s[(c0 + 2 * u) * APPLY_ROWS + rr] = bf16_to_f32(static_cast<uint16_t>(v[u] & 0xFFFFu));
            xt_s[(c0 + 2 * u + 1) * APPLY_ROWS + rr] = bf16_to_f32(static_cast<uint16_t>(v[u] >> 16));
        }
    }
    __syncthreads();
    const int rg = tid >> 4, c0 = 8 * (tid & 15);              // rows 4 rg .. 4 rg + 3
    float acc[4][8];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[q][u] = xt_s[(c0 + u) * APPLY_ROWS + 4 * rg + q] + c_s[c0 + u];
#pragma unroll 4
    for (int i = 0; i < D; ++i) {
        const f32x4 x4 = *reinterpret_cast<const f32x4*>(xt_s + i * APPLY_ROWS + 4 * rg);
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(w_s + i * D + c0);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(w_s + i * D + c0 + 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                acc[q][u] = fmaf(x4[q], w0[u], acc[q][u]);
                acc[q][u + 4] = fmaf(x4[q], w1[u], acc[q][u + 4]);
            }
        }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int row = row0 + 4 * rg + q;
        const int a = row / BLK;
        if (row < r.N && row == probe_row(a, r.N, r.phase)) {
            const float* od = r.od + (bh * r.Mp + a) * D + c0;
#pragma unroll
            for (int u = 0; u < 8; ++u) acc[q][u] = od[u];
        }
        u32x4 w;
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = row < r.N ? pack_bf16x2(acc[q][2 * u], acc[q][2 * u + 1]) : 0u;
        *reinterpret_cast<u32x4*>(O + static_cast<size_t>(row) * D + c0) = w;
    }
}

}  // namespace

int residual_key_chunks(int N_pad) { return min(8, N_pad / BLK); }

size_t residual_workspace_bytes(int B, int H, int N_pad) {
    const size_t bh = static_cast<size_t>(B) * H;
    const size_t mp = BLK * ((N_pad / BLK + BLK - 1) / BLK);
    const size_t kc = residual_key_chunks(N_pad);
    const size_t f64 = bh * (NSPLIT * (3 * D * D + 2 * D) + 3 * D * D);
    const size_t f32 = bh * (2 * mp * D + D * D + D) + kc * bh * mp * (D + 1);
    const size_t b16 = bh * mp * D;
    return f64 * 8 + f32 * 4 + b16 * 2;
}

void residual_carve(ResidualArgs& r, void* ws) {
    const size_t bh = static_cast<size_t>(r.B) * r.H;
    const size_t mp = r.Mp;
    char* p = static_cast<char*>(ws);
    r.part = reinterpret_cast<double*>(p); p += bh * NSPLIT * (3 * D * D + 2 * D) * 8;
    r.mat = reinterpret_cast<double*>(p);  p += bh * 3 * D * D * 8;
    r.xp = reinterpret_cast<float*>(p);    p += bh * mp * D * 4;
    r.od = reinterpret_cast<float*>(p);    p += bh * mp * D * 4;
    r.wc = reinterpret_cast<float*>(p);    p += bh * (D * D + D) * 4;
    r.kchunks = residual_key_chunks(r.N_pad);
    r.odp = reinterpret_cast<float*>(p);   p += r.kchunks * bh * mp * D * 4;
    r.lsep = reinterpret_cast<float*>(p);  p += r.kchunks * bh * mp * 4;
    r.qp = reinterpret_cast<uint16_t*>(p);
}

hipError_t launch_residual(const ResidualArgs& r, hipStream_t s) {
    const int bh = r.B * r.H;
    hipError_t e;
    hipLaunchKernelGGL(probe_gather_kernel, dim3((r.Mp * (D / 8) + THREADS - 1) / THREADS, bh), dim3(THREADS), 0, s, r);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // dense attention of the gathered probe queries (every key block exact, fp32 out)
    FwdArgs f{};
    f.B = r.B; f.H = r.H; f.N = r.N; f.N_pad = r.N_pad; f.d = D;
    f.comp = -1; f.scale = r.scale;
    f.q = r.qp; f.k = r.k; f.v = r.v;
    f.out = r.odp; f.lse = r.lsep;
    f.Nq = r.N_pad / BLK; f.Nq_pad = r.Mp;
    f.dense = r.kchunks; f.out_f32 = 1;
    if ((e = launch_fwd_bf16(f, s)) != hipSuccess) return e;
    hipLaunchKernelGGL(combine_kernel, dim3((r.Mp * D + THREADS - 1) / THREADS, bh), dim3(THREADS), 0, s, r);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(gram_kernel, dim3(NSPLIT, 3, bh), dim3(THREADS), 0, s, r);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(fit_kernel, dim3(bh), dim3(THREADS), 0, s, r);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(apply_kernel, dim3(r.N_pad / APPLY_ROWS, bh), dim3(THREADS), 0, s, r);
    return hipGetLastError();
}

}  // namespace sa
