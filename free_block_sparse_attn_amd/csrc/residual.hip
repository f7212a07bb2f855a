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
//   4. reduce_kernel         the partial sums in a fixed order, centred
//      fit_factor_kernel     two workgroups per head side by side: the top-r
//                            subspace V_r of R^T R (simultaneous iteration
//                            with Cholesky QR, then Rayleigh-Ritz), and the
//                            LDL^T factor of G + lambda I
//      fit_solve_kernel      one workgroup per head: Z = (G + lambda I)^{-1}
//                            C V_r by forward and back substitution, then
//                            W = Z V_r^T, c = (rm V_r - xm Z) V_r^T and the
//                            fp32 factors
//   5. apply_kernel          o_t <- o_t + c + (o_t Z) V_r^T on every valid
//                            row, the dense output on probe rows (bf16, in
//                            place)
#include "common.h"
#include "launch.h"

namespace sa {

namespace {

constexpr int D = 128;
constexpr int THREADS = 256;
constexpr int NSPLIT = 8;                  // probe slices of the Gram partial sums
constexpr int KSUB = 8;                    // block width of the subspace iteration (rank <= KSUB)
constexpr int SUB_MIN = 16;                // simultaneous-iteration steps: at least,
constexpr int SUB_MAX = 32;                // at most,
constexpr int SUB_CHECK = 4;               // and every this many a convergence check:
constexpr double SUB_TOL = 1e-10;          // sum of squared sines between the spans

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

// fp16 copy of V for the dense probe pass (the forward kernel's value side
// runs in fp16): one 16-byte chunk (8 values) per thread, RNE.
__global__ __launch_bounds__(THREADS) void value_f16_kernel(ResidualArgs r) {
    const size_t x = static_cast<size_t>(blockIdx.x) * THREADS + threadIdx.x;
    const size_t total = static_cast<size_t>(r.B) * r.H * r.N_pad * (D / 8);
    if (x >= total) return;
    const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(r.v) + x * 8);
    u32x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = pack_f16x2(__uint_as_float(w[e] << 16), __uint_as_float(w[e] & 0xFFFF0000u));
    *reinterpret_cast<u32x4*>(r.v16 + x * 8) = y;
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
// Workgroup (slice s, matrix m, head): probes p = s, s + NSPLIT, ... in
// order; thread (ti, tj) of a 16 x 16 grid owns the 8 x 8 entries
// (ti + 16 a, tj + 16 b) of matrix m: m = 0: sum x_i x_j, 1: sum x_i r_j,
// 2: sum r_i r_j (r = o_dense - x).  Per probe a thread reads 8 + 8 values
// for 64 products.  Matrix 1's workgroup also sums the columns of x and r.
__global__ __launch_bounds__(THREADS) void gram_kernel(ResidualArgs r) {
    constexpr int STAGE = 16;
    constexpr int PER = STAGE * D / THREADS;      // staged values per thread
    __shared__ double u_s[STAGE][D], w_s[STAGE][D];
    const int s = blockIdx.x, m = blockIdx.y;
    const size_t bh = blockIdx.z;
    const int nb = r.N_pad / BLK, mp = r.Mp;
    const int tid = threadIdx.x, ti = tid >> 4, tj = tid & 15;
    double acc[8][8];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = 0.0;
    double colsum = 0.0;                          // m == 1: thread t < 128 sums x_t, t >= 128 sums r_{t-128}
    const float* X = r.xp + bh * mp * D;
    const float* O = r.od + bh * mp * D;
    float xv[PER], ov[PER];
    auto fetch = [&](int p0) __attribute__((always_inline)) {
#pragma unroll
        for (int v = 0; v < PER; ++v) {
            const int e = tid + v * THREADS, q = e / D, col = e % D;
            const int p = p0 + NSPLIT * q;
            xv[v] = p < nb ? X[static_cast<size_t>(p) * D + col] : 0.0f;
            ov[v] = p < nb ? O[static_cast<size_t>(p) * D + col] : 0.0f;
        }
    };
    fetch(s);
    for (int p0 = s; p0 < nb; p0 += NSPLIT * STAGE) {
        __syncthreads();
#pragma unroll
        for (int v = 0; v < PER; ++v) {
            const int e = tid + v * THREADS, q = e / D, col = e % D;
            const double x = static_cast<double>(xv[v]);
            const double rr = static_cast<double>(ov[v]) - x;
            u_s[q][col] = (m == 2) ? rr : x;
            w_s[q][col] = (m == 0) ? x : rr;
        }
        __syncthreads();
        if (p0 + NSPLIT * STAGE < nb) fetch(p0 + NSPLIT * STAGE);
        if (m == 1) {
#pragma unroll
            for (int q = 0; q < STAGE; ++q) colsum += tid < D ? u_s[q][tid] : w_s[q][tid - D];
        }
#pragma unroll 2
        for (int q = 0; q < STAGE; ++q) {
            double uu[8], ww[8];
#pragma unroll
            for (int a = 0; a < 8; ++a) uu[a] = u_s[q][ti + 16 * a];
#pragma unroll
            for (int b = 0; b < 8; ++b) ww[b] = w_s[q][tj + 16 * b];
#pragma unroll
            for (int a = 0; a < 8; ++a)
#pragma unroll
                for (int b = 0; b < 8; ++b) acc[a][b] = fma(uu[a], ww[b], acc[a][b]);
        }
    }
    double* P = r.part + ((bh * NSPLIT + s) * (3 * D * D + 2 * D));
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) P[m * D * D + (ti + 16 * a) * D + tj + 16 * b] = acc[a][b];
    if (m == 1) P[3 * D * D + tid] = colsum;      // x sums then r sums
}

// ---- 4a. reduce the Gram partial sums in a fixed order and centre ----
// Workgroup (chunk, head): 4 entries per thread of the three d x d matrices;
// the column sums give the probe means xm, rm.
constexpr int RED_PER_WG = 4 * THREADS;
constexpr size_t PSTRIDE = 3 * D * D + 2 * D;   // doubles per slice of the partial sums
constexpr int ZS = D;                           // the zero slot of a published column
static_assert(3 * D * D % RED_PER_WG == 0 && THREADS == 2 * D, "reduce tiling");

__global__ __launch_bounds__(THREADS) void reduce_kernel(ResidualArgs r) {
    __shared__ double xm[D], rm[D];
    const size_t bh = blockIdx.y;
    const int tid = threadIdx.x;
    const double M = static_cast<double>(r.N_pad / BLK);
    const double* P = r.part + bh * NSPLIT * PSTRIDE;
    {
        double v = 0.0;
        for (int s = 0; s < NSPLIT; ++s) v += P[s * PSTRIDE + 3 * D * D + tid];
        if (tid < D) xm[tid] = v / M;
        else rm[tid - D] = v / M;
    }
    __syncthreads();
    double* G = r.mat + bh * 3 * D * D;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int e = blockIdx.x * RED_PER_WG + u * THREADS + tid;
        double v = 0.0;
#pragma unroll
        for (int s = 0; s < NSPLIT; ++s) v += P[s * PSTRIDE + e];
        const int m = e / (D * D), i = (e / D) % D, j = e % D;
        if (m == 0) v -= M * xm[i] * xm[j];
        else if (m == 1) v -= M * xm[i] * rm[j];
        G[e] = v;
    }
}

// ---- 4b. fit: one workgroup per head ----
typedef __attribute__((ext_vector_type(2))) double f64x2;

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

// 1/x and 1/sqrt(x) for normal x > 0: the hardware estimate and two Newton steps
__device__ __forceinline__ double rcp64(double x) {
    double y = __builtin_amdgcn_rcp(x);
    y = fma(y, fma(-x, y, 1.0), y);
    y = fma(y, fma(-x, y, 1.0), y);
    return y;
}
__device__ __forceinline__ double rsq64(double x) {
    double y = __builtin_amdgcn_rsq(x);
    const double h = 0.5 * x;
    y = y * fma(-h * y, y, 1.5);
    y = y * fma(-h * y, y, 1.5);
    return y;
}

__device__ __forceinline__ double readlane64(double v, int lane) {
    const unsigned long long b = static_cast<unsigned long long>(__double_as_longlong(v));
    const unsigned lo = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(b & 0xFFFFFFFFull), lane));
    const unsigned hi = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(b >> 32), lane));
    return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo));
}

// From the KSUB x KSUB Gram matrix (row-major), the inverse Mi = L^{-1} of
// its Cholesky factor (lower triangle of Mi).  Every thread computes it.
__device__ __forceinline__ void chol_inv8(const double* Gs, double (&Mi)[KSUB][KSUB]) {
    double L[KSUB][KSUB], rs[KSUB];
#pragma unroll
    for (int i = 0; i < KSUB; ++i)
#pragma unroll
        for (int j = 0; j <= i; ++j) L[i][j] = Gs[i * KSUB + j];
#pragma unroll
    for (int k = 0; k < KSUB; ++k) {
        double d = L[k][k];
#pragma unroll
        for (int t = 0; t < k; ++t) d = fma(-L[k][t], L[k][t], d);
        rs[k] = rsq64(fmax(d, 1e-300));                   // 1 / L_kk
#pragma unroll
        for (int i = k + 1; i < KSUB; ++i) {
            double v = L[i][k];
#pragma unroll
            for (int t = 0; t < k; ++t) v = fma(-L[i][t], L[k][t], v);
            L[i][k] = v * rs[k];
        }
    }
#pragma unroll
    for (int i = 0; i < KSUB; ++i) {
        Mi[i][i] = rs[i];
#pragma unroll
        for (int j = 0; j < i; ++j) {
            double v = 0.0;
#pragma unroll
            for (int t = j; t < i; ++t) v = fma(L[i][t], Mi[t][j], v);
            Mi[i][j] = -v * rs[i];
        }
    }
}

// Step 16 KB + kk of the elimination (see ldl_columns).
template <int KB>
__device__ __forceinline__ void ldl_step(int kk, double (&A)[8][8], const double (&x)[8], const double (&cu)[8],
                                         double nrinv, double (&xn)[8], double (&cn)[8], double& nrn,
                                         double (*col)[D + 1], int p, int q) {
    constexpr int NB = KB < 7 ? KB + 1 : KB;
    const int k = 16 * KB + kk;
    double u[8];                                           // minus the multipliers of step k
#pragma unroll
    for (int b = KB; b < 8; ++b) u[b] = cu[b] * nrinv;
    if (k + 1 < D && q == ((k + 1) & 15)) {
        double* cw = col[(k + 1) & 1];
        if (kk < 15) {
#pragma unroll
            for (int a = KB; a < 8; ++a) A[a][KB] = fma(x[a], u[KB], A[a][KB]);
#pragma unroll
            for (int a = KB; a < 8; ++a) cw[16 * a + p] = A[a][KB];
            u[KB] = 0.0;
        } else {
#pragma unroll
            for (int a = NB; a < 8; ++a) A[a][NB] = fma(x[a], u[NB], A[a][NB]);
#pragma unroll
            for (int a = NB; a < 8; ++a) cw[16 * a + p] = A[a][NB];
            u[NB] = 0.0;
        }
    }
    __syncthreads();
    // column k + 1 (read past the end on the last step, then unused); the
    // update below does not wait for these reads
    const double* ck = col[(k + 1) & 1];
    const double dn = ck[k + 1];
#pragma unroll
    for (int a = KB; a < 8; ++a) xn[a] = ck[16 * a + p > k + 1 ? 16 * a + p : ZS];
#pragma unroll
    for (int bb = KB; bb < 8; ++bb) cn[bb] = ck[16 * bb + q > k + 1 ? 16 * bb + q : ZS];
#pragma unroll
    for (int bb = KB; bb < 8; ++bb)
#pragma unroll
        for (int a = bb; a < 8; ++a) A[a][bb] = fma(x[a], u[bb], A[a][bb]);
    nrn = -rcp64(fmax(dn, 1e-300));
}

// Columns 16 KB .. 16 KB + 15 of the right-looking LDL^T elimination.
// Thread (p, q) holds A[a][b] = entry (16 a + p, 16 b + q) for a >= b.
// Entering step k, x and cu hold column k's entries of the thread's rows and
// columns, zero for rows / columns <= k (so finished entries are left alone),
// and nrinv minus the reciprocal pivot.  Step k: the owners of column k + 1
// (q == (k + 1) % 16) apply step k to it and publish it in col[(k + 1) % 2];
// after the barrier every thread reads column k + 1 and applies the rest of
// step k, the reads overlapping the update.  Two register sets alternate
// between the steps.  Blocks left of column block KB are finished and skipped.
template <int KB>
__device__ __forceinline__ void ldl_columns(double (&A)[8][8], double (&x)[8], double (&cu)[8], double& nrinv,
                                            double (*col)[D + 1], int p, int q) {
    double x2[8], c2[8], nr2;
#pragma unroll 1
    for (int kk = 0; kk < 16; kk += 2) {
        ldl_step<KB>(kk, A, x, cu, nrinv, x2, c2, nr2, col, p, q);
        ldl_step<KB>(kk + 1, A, x2, c2, nr2, x, cu, nrinv, col, p, q);
    }
}

// Eigen-decomposition of the symmetric KSUB x KSUB matrix Hs (row-major, in
// LDS) by cyclic Jacobi on one wave: each round applies 4 disjoint plane
// rotations (round-robin pairing of the 8 indices, 7 rounds a sweep), the 64
// entries of H and of the eigenvector matrix Es updated one per lane.  The
// rotation for (p, q) zeroes H[p][q] (Golub and Van Loan's symmetric 2 x 2
// Schur decomposition).  On return Hs holds the eigenvalues on its diagonal
// and the columns of Es the eigenvectors.
constexpr int JACOBI_SWEEPS = 6;
__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
__device__ __forceinline__ int rr_partner(int x, int r) {     // round r pairing of 0..7
    if (x == 7) return r;
    if (x == r) return 7;
    return ((2 * r - x) % 7 + 7) % 7;
}
__device__ void jacobi8(double* Hs, double* Es, double* cs, int lane) {
    const int i = lane >> 3, j = lane & 7;
    Es[lane] = i == j ? 1.0 : 0.0;
    wave_sync_lds();
    for (int sweep = 0; sweep < JACOBI_SWEEPS; ++sweep) {
        for (int r = 0; r < 7; ++r) {
            if (lane < KSUB) {                     // lane x: the rotation of its pair, from the lower index
                const int x = lane, y = rr_partner(x, r);
                const int pp = min(x, y), qq = max(x, y);
                const double hpq = Hs[pp * KSUB + qq];
                double c = 1.0, sn = 0.0;
                if (hpq != 0.0) {
                    const double tau = (Hs[qq * KSUB + qq] - Hs[pp * KSUB + pp]) / (2.0 * hpq);
                    const double t = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
                    c = 1.0 / sqrt(1.0 + t * t);
                    sn = t * c;
                }
                cs[2 * x] = c;                     // J[x][x] = c, J[partner][x] = sigma_x
                cs[2 * x + 1] = x == pp ? -sn : sn;
            }
            wave_sync_lds();
            const int pi = rr_partner(i, r), pj = rr_partner(j, r);
            const double ci = cs[2 * i], si = cs[2 * i + 1], cj = cs[2 * j], sj = cs[2 * j + 1];
            const double h = ci * (cj * Hs[i * KSUB + j] + sj * Hs[i * KSUB + pj]) +
                             si * (cj * Hs[pi * KSUB + j] + sj * Hs[pi * KSUB + pj]);
            const double e = cj * Es[i * KSUB + j] + sj * Es[i * KSUB + pj];
            wave_sync_lds();
            Hs[lane] = h;
            Es[lane] = e;
            wave_sync_lds();
        }
    }
}

// With V_r the top right singular vectors of R, W = B P = Z V_r^T with
// Z = (G + lambda I)^{-1} (C V_r), and c = b P = (rm V_r - xm Z) V_r^T, so
// only `rank` right-hand sides are solved.  The subspace and the factor of
// G + lambda I do not depend on each other, so they run side by side:
//   fit_factor_kernel, workgroups (0, head) and (1, head):
//     0: simultaneous iteration on S = R^T R (fp32 copy in LDS, fp64
//        products), KSUB columns, Cholesky QR after every product, 16 to 32
//        steps (until the leading rank columns' span settles), then
//        Rayleigh-Ritz; V_r (fp64) into the workspace;
//     1: LDL^T of G + lambda I by right-looking elimination in registers,
//        thread (p, q) of a 16 x 16 grid holding the entries (16 a + p,
//        16 b + q), one barrier per column, the column published through
//        LDS; the packed factor (stored column k = L_.k D_kk) into the
//        workspace.
//   fit_solve_kernel, one workgroup per head: T = C V_r, the forward and back
//     substitutions with the unit triangular factors (a wave per two
//     right-hand sides, the pivot row's values read across lanes), then W, c
//     and the factors Z, V_r (fp32) for the apply pass.
// Both write into the Gram partial sums' space past the reduction (V_r at 0,
// the factor after it; the column sums further on stay untouched).
constexpr int LPK = D * (D + 1) / 2;                        // packed lower triangle, row i at i (i + 1) / 2
static_assert(D * KSUB + LPK + 1 <= 3 * D * D, "the fit's scratch stays below the column sums");

__global__ __launch_bounds__(THREADS) void fit_factor_kernel(ResidualArgs r) {
    constexpr int SP = D + 4;                               // fp32 row stride of S in LDS
    constexpr int POOL = D * SP / 2;
    __shared__ __attribute__((aligned(16))) double pool[POOL];   // S (fp32)
    __shared__ __attribute__((aligned(16))) double B0[D * KSUB], B1[D * KSUB], Qp[D * KSUB];
    __shared__ __attribute__((aligned(16))) double Pt[4 * D * KSUB];   // partial products, one per wave
    __shared__ double col[2][D + 1];                       // slot D holds 0
    __shared__ double Gs[KSUB * KSUB], Es[KSUB * KSUB], jcs[2 * KSUB];
    __shared__ double red[THREADS / 64];
    const size_t bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int rk = r.rank;
    const double* G = r.mat + bh * 3 * D * D;              // centred X^T X
    const double* S = G + 2 * D * D;                       // R^T R
    double* scratch = r.part + bh * NSPLIT * PSTRIDE;
    if (blockIdx.x == 0) {
        const int ri = tid >> 1, rc = 4 * (tid & 1);       // row, first of four columns
        float* Sf = reinterpret_cast<float*>(pool);
#pragma unroll 1
        for (int e0 = 0; e0 < D * D; e0 += 16 * 2 * THREADS) {     // 16 pairs in flight per thread
            f64x2 v[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = *reinterpret_cast<const f64x2*>(S + e0 + 2 * (j * THREADS + tid));
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int e = e0 + 2 * (j * THREADS + tid);
                Sf[(e / D) * SP + e % D] = static_cast<float>(v[j][0]);
                Sf[(e / D) * SP + e % D + 1] = static_cast<float>(v[j][1]);
            }
        }
        for (int e = tid; e < D * KSUB; e += THREADS) {
            const int i = e / KSUB, c = e % KSUB;
            B0[e] = static_cast<double>(((i * 7 + c * 13 + 3) % 17) - 8) + (i == c ? 16.0 : 0.0);
        }
        __syncthreads();
        // ---- top-rank subspace of S ----
        auto cholqr = [&](const double* Yin, double* Qout) __attribute__((always_inline)) {
            {   // Gram entry tid / 4 over rows i = tid % 4 (mod 4), four lanes combined
                const int g = tid >> 2, a = g / KSUB, b = g % KSUB, i0 = tid & 3;
                double v0 = 0.0, v1 = 0.0, v2 = 0.0, v3 = 0.0;
#pragma unroll
                for (int i = i0; i < D; i += 16) {
                    v0 = fma(Yin[i * KSUB + a], Yin[i * KSUB + b], v0);
                    v1 = fma(Yin[(i + 4) * KSUB + a], Yin[(i + 4) * KSUB + b], v1);
                    v2 = fma(Yin[(i + 8) * KSUB + a], Yin[(i + 8) * KSUB + b], v2);
                    v3 = fma(Yin[(i + 12) * KSUB + a], Yin[(i + 12) * KSUB + b], v3);
                }
                double v = (v0 + v1) + (v2 + v3);
                v += __shfl_xor(v, 1);
                v += __shfl_xor(v, 2);
                if ((tid & 3) == 0) Gs[g] = v;
            }
            __syncthreads();
            double Mi[KSUB][KSUB];
            chol_inv8(Gs, Mi);
            double y[KSUB];
#pragma unroll
            for (int t = 0; t < KSUB; t += 2) {
                const f64x2 w = *reinterpret_cast<const f64x2*>(Yin + ri * KSUB + t);
                y[t] = w[0];
                y[t + 1] = w[1];
            }
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {                     // q_c = sum_{t <= c} Mi[c][t] y_t
                double v = 0.0;
#pragma unroll
                for (int t = 0; t <= 4 + cc; ++t) {             // rc is 0 or 4
                    const double m = rc ? Mi[4 + cc][t] : (t <= cc ? Mi[cc][t] : 0.0);
                    v = fma(m, y[t], v);
                }
                Qout[ri * KSUB + rc + cc] = v;
            }
            __syncthreads();
        };
        // Y = S Q: wave w takes the terms m in [32 w, 32 w + 32); lane l the
        // rows l / 2 + 32 r (r < 4) and columns rc .. rc + 3; the four partial
        // products are summed in wave order.
        auto product = [&](const double* Q, double* Y) __attribute__((always_inline)) {
            const int g = lane >> 1, kc = 32 * wv;
            double y[4][4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) y[rr][cc] = 0.0;
            const float* s0 = Sf + g * SP + kc;
#pragma unroll 2
            for (int m = 0; m < 32; m += 4) {
                f32x4 sv[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) sv[rr] = *reinterpret_cast<const f32x4*>(s0 + 32 * rr * SP + m);
#pragma unroll
                for (int mm = 0; mm < 4; ++mm) {
                    const double* qr = Q + (kc + m + mm) * KSUB + rc;
                    const f64x2 qa = *reinterpret_cast<const f64x2*>(qr);
                    const f64x2 qb = *reinterpret_cast<const f64x2*>(qr + 2);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const double sd = static_cast<double>(sv[rr][mm]);
                        y[rr][0] = fma(sd, qa[0], y[rr][0]);
                        y[rr][1] = fma(sd, qa[1], y[rr][1]);
                        y[rr][2] = fma(sd, qb[0], y[rr][2]);
                        y[rr][3] = fma(sd, qb[1], y[rr][3]);
                    }
                }
            }
            double* pw = Pt + wv * D * KSUB;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                *reinterpret_cast<f64x2*>(pw + (g + 32 * rr) * KSUB + rc) = f64x2{y[rr][0], y[rr][1]};
                *reinterpret_cast<f64x2*>(pw + (g + 32 * rr) * KSUB + rc + 2) = f64x2{y[rr][2], y[rr][3]};
            }
            __syncthreads();
            f64x2 o01 = {0.0, 0.0}, o23 = {0.0, 0.0};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                o01 += *reinterpret_cast<const f64x2*>(Pt + w * D * KSUB + ri * KSUB + rc);
                o23 += *reinterpret_cast<const f64x2*>(Pt + w * D * KSUB + ri * KSUB + rc + 2);
            }
            *reinterpret_cast<f64x2*>(Y + ri * KSUB + rc) = o01;
            *reinterpret_cast<f64x2*>(Y + ri * KSUB + rc + 2) = o23;
            __syncthreads();
        };
        cholqr(B0, B1);
        cholqr(B1, B0);
        for (int e = tid; e < D * KSUB; e += THREADS) Qp[e] = B0[e];
        // Stop once the span of the leading `rank` columns moved by less than
        // SUB_TOL (sum of squared sines of the principal angles, rank minus
        // the squared Frobenius norm of Qp_r^T Q_r) over SUB_CHECK steps.
        for (int it = 0; it < SUB_MAX; ++it) {
            product(B0, B1);
            cholqr(B1, B0);
            if (it % SUB_CHECK == SUB_CHECK - 1) {
                const int g = tid >> 2, a = g / KSUB, b = g % KSUB, i0 = tid & 3;
                double v = 0.0;
                for (int i = i0; i < D; i += 4) v = fma(Qp[i * KSUB + a], B0[i * KSUB + b], v);
                v += __shfl_xor(v, 1);
                v += __shfl_xor(v, 2);
                double o = ((tid & 3) == 0 && a < rk && b < rk) ? v * v : 0.0;
                o = wave_sum(o);
                if (lane == 0) red[wv] = o;
                __syncthreads();
                const double moved = rk - ((red[0] + red[1]) + (red[2] + red[3]));
                if (it + 1 >= SUB_MIN && moved < SUB_TOL) break;      // the same decision in every thread
                for (int e = tid; e < D * KSUB; e += THREADS) Qp[e] = B0[e];
                __syncthreads();
            }
        }
        cholqr(B0, B1);                                        // Q, orthonormal, in B1
        // ---- Rayleigh-Ritz: H = Q^T S Q, H = E diag(l) E^T; V = Q E with the
        // columns ordered by decreasing eigenvalue, the first rank kept ----
        product(B1, B0);                                       // B0 = S Q
        {
            const int g = tid >> 2, a = g / KSUB, b = g % KSUB, i0 = tid & 3;
            double v0 = 0.0, v1 = 0.0, v2 = 0.0, v3 = 0.0;
#pragma unroll
            for (int i = i0; i < D; i += 16) {
                v0 = fma(B1[i * KSUB + a], B0[i * KSUB + b], v0);
                v1 = fma(B1[(i + 4) * KSUB + a], B0[(i + 4) * KSUB + b], v1);
                v2 = fma(B1[(i + 8) * KSUB + a], B0[(i + 8) * KSUB + b], v2);
                v3 = fma(B1[(i + 12) * KSUB + a], B0[(i + 12) * KSUB + b], v3);
            }
            double v = (v0 + v1) + (v2 + v3);
            v += __shfl_xor(v, 1);
            v += __shfl_xor(v, 2);
            if ((tid & 3) == 0) Gs[g] = v;
        }
        __syncthreads();
        if (wv == 0) {
            // symmetrise (the two halves come from different sums) and diagonalise
            const int i = lane >> 3, j = lane & 7;
            const double hs = 0.5 * (Gs[i * KSUB + j] + Gs[j * KSUB + i]);
            wave_sync_lds();
            Gs[lane] = hs;
            wave_sync_lds();
            jacobi8(Gs, Es, jcs, lane);
        }
        __syncthreads();
        double* V = B1;
        {
            double qrow[KSUB], ev[KSUB];
#pragma unroll
            for (int t = 0; t < KSUB; ++t) qrow[t] = V[ri * KSUB + t];
#pragma unroll
            for (int t = 0; t < KSUB; ++t) ev[t] = Gs[t * (KSUB + 1)];
            __syncthreads();
#pragma unroll
            for (int jc = 0; jc < KSUB; ++jc) {                 // eigenvector jc goes to column rank(jc)
                int pos = 0;
#pragma unroll
                for (int t = 0; t < KSUB; ++t) pos += (ev[t] > ev[jc]) || (ev[t] == ev[jc] && t < jc);
                if (pos >= rc && pos < rc + 4) {
                    double v = 0.0;
#pragma unroll
                    for (int t = 0; t < KSUB; ++t) v = fma(qrow[t], Es[t * KSUB + jc], v);
                    V[ri * KSUB + pos] = pos < rk ? v : 0.0;
                }
            }
        }
        __syncthreads();

        for (int e = tid; e < D * KSUB; e += THREADS) scratch[e] = V[e];
        return;
    }
    // ---- LDL^T of G + lambda I ----
    {
        double tr = tid < D ? G[tid * (D + 1)] : 0.0;
        tr = wave_sum(tr);
        if (lane == 0) red[wv] = tr;
        if (tid < 2) col[tid][ZS] = 0.0;
    }
    __syncthreads();
    const double lam = static_cast<double>(r.ridge) * (red[0] + red[1] + red[2] + red[3]) / D;
    const int p = tid >> 4, q = tid & 15;
    double A[8][8];                                        // a >= b used
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b <= a; ++b) {
            const int i = 16 * a + p, j = 16 * b + q;
            A[a][b] = G[i * D + j] + (i == j ? lam : 0.0);
        }
    if (q == 0) {
#pragma unroll
        for (int a = 0; a < 8; ++a) col[0][16 * a + p] = A[a][0];
    }
    __syncthreads();
    double x[8], cu[8], nrinv;
    nrinv = -rcp64(fmax(col[0][0], 1e-300));
#pragma unroll
    for (int a = 0; a < 8; ++a) x[a] = col[0][16 * a + p > 0 ? 16 * a + p : ZS];
#pragma unroll
    for (int b = 0; b < 8; ++b) cu[b] = col[0][16 * b + q > 0 ? 16 * b + q : ZS];
    ldl_columns<0>(A, x, cu, nrinv, col, p, q);
    ldl_columns<1>(A, x, cu, nrinv, col, p, q);
    ldl_columns<2>(A, x, cu, nrinv, col, p, q);
    ldl_columns<3>(A, x, cu, nrinv, col, p, q);
    ldl_columns<4>(A, x, cu, nrinv, col, p, q);
    ldl_columns<5>(A, x, cu, nrinv, col, p, q);
    ldl_columns<6>(A, x, cu, nrinv, col, p, q);
    ldl_columns<7>(A, x, cu, nrinv, col, p, q);
    double* F = scratch + D * KSUB;
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b <= a; ++b) {
            const int i = 16 * a + p, j = 16 * b + q;
            if (i >= j) F[i * (i + 1) / 2 + j] = A[a][b];
        }
    if (tid == 0) F[LPK] = 0.0;                            // zero slot for the substitutions
}

__global__ __launch_bounds__(THREADS) void fit_solve_kernel(ResidualArgs r) {
    __shared__ __attribute__((aligned(16))) double Lp[LPK + 1];
    __shared__ __attribute__((aligned(16))) double B1[D * KSUB], B2[D * KSUB];
    __shared__ double xm[D], rm[D], s8[KSUB];
    const size_t bh = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int rk = r.rank;
    const double M = static_cast<double>(r.N_pad / BLK);
    const double* P = r.part + bh * NSPLIT * PSTRIDE;
    const double* C = r.mat + bh * 3 * D * D + D * D;      // centred X^T R
    {
        double v = 0.0;
        for (int s = 0; s < NSPLIT; ++s) v += P[s * PSTRIDE + 3 * D * D + tid];
        if (tid < D) xm[tid] = v / M;
        else rm[tid - D] = v / M;
    }
    for (int e = tid; e < D * KSUB; e += THREADS) B1[e] = P[e];
    for (int e = tid; e < LPK + 1; e += THREADS) Lp[e] = P[D * KSUB + e];
    __syncthreads();
    const int ri = tid >> 1, rc = 4 * (tid & 1);
    double* V = B1;
    // ---- T = C V_r into B2 ----
    {
        const double* crow = C + ri * D;
        double t0 = 0.0, t1 = 0.0, t2 = 0.0, t3 = 0.0;
#pragma unroll 4
        for (int l = 0; l < D; l += 2) {
            const f64x2 cv = *reinterpret_cast<const f64x2*>(crow + l);
#pragma unroll
            for (int ll = 0; ll < 2; ++ll) {
                const f64x2 va = *reinterpret_cast<const f64x2*>(V + (l + ll) * KSUB + rc);
                const f64x2 vb = *reinterpret_cast<const f64x2*>(V + (l + ll) * KSUB + rc + 2);
                t0 = fma(cv[ll], va[0], t0);
                t1 = fma(cv[ll], va[1], t1);
                t2 = fma(cv[ll], vb[0], t2);
                t3 = fma(cv[ll], vb[1], t3);
            }
        }
        *reinterpret_cast<f64x2*>(B2 + ri * KSUB + rc) = f64x2{t0, t1};
        *reinterpret_cast<f64x2*>(B2 + ri * KSUB + rc + 2) = f64x2{t2, t3};
    }
    __syncthreads();


    // ---- L y = T (unit lower), then L^T Z = D^{-1} y (unit upper): wave w
    // solves columns 2w, 2w + 1, lane the rows 2 lane, 2 lane + 1 ----
    {
        const int c0 = 2 * wv, j0 = 2 * lane;
        if (c0 < rk) {
            double u00 = B2[j0 * KSUB + c0], u01 = B2[j0 * KSUB + c0 + 1];
            double u10 = B2[(j0 + 1) * KSUB + c0], u11 = B2[(j0 + 1) * KSUB + c0 + 1];
            const double rd0 = rcp64(fmax(Lp[j0 * (j0 + 1) / 2 + j0], 1e-300));
            const double rd1 = rcp64(fmax(Lp[(j0 + 1) * (j0 + 2) / 2 + j0 + 1], 1e-300));
            // forward: y_j final at step j; rows i > j lose a_ij y_j / d_j
#pragma unroll 2
            for (int j = 0; j < D; ++j) {
                const int o = j >> 1;
                const bool odd = j & 1;
                const double rdj = readlane64(odd ? rd1 : rd0, o);
                const double w0 = readlane64(odd ? u10 : u00, o) * rdj;
                const double w1 = readlane64(odd ? u11 : u01, o) * rdj;
                const double a0 = Lp[j0 > j ? j0 * (j0 + 1) / 2 + j : LPK];
                const double a1 = Lp[j0 + 1 > j ? (j0 + 1) * (j0 + 2) / 2 + j : LPK];
                u00 = fma(-a0, w0, u00);
                u01 = fma(-a0, w1, u01);
                u10 = fma(-a1, w0, u10);
                u11 = fma(-a1, w1, u11);
            }
            // back: z_i = u_i / d_i at step i; rows j < i lose a_ij z_i
#pragma unroll 2
            for (int i = D - 1; i >= 0; --i) {
                const int o = i >> 1;
                const bool odd = i & 1;
                const double rdi = readlane64(odd ? rd1 : rd0, o);
                const double z0 = readlane64(odd ? u10 : u00, o) * rdi;
                const double z1 = readlane64(odd ? u11 : u01, o) * rdi;
                const double l0 = Lp[j0 < i ? i * (i + 1) / 2 + j0 : LPK];
                const double l1 = Lp[j0 + 1 < i ? i * (i + 1) / 2 + j0 + 1 : LPK];
                u00 = fma(-l0, z0, u00);
                u01 = fma(-l0, z1, u01);
                u10 = fma(-l1, z0, u10);
                u11 = fma(-l1, z1, u11);
            }
            *reinterpret_cast<f64x2*>(B2 + j0 * KSUB + c0) = f64x2{u00 * rd0, u01 * rd0};
            *reinterpret_cast<f64x2*>(B2 + (j0 + 1) * KSUB + c0) = f64x2{u10 * rd1, u11 * rd1};
        }
    }
    __syncthreads();

    // ---- outputs: Z (B2) and V_r (B1), W = Z V_r^T, c = (rm V_r - xm Z) V_r^T ----
    const double* Z = B2;
    float* zvo = r.zv + bh * 2 * D * KSUB;
    for (int e = tid; e < D * KSUB; e += THREADS) {
        zvo[e] = static_cast<float>(Z[e]);
        zvo[D * KSUB + e] = static_cast<float>(V[e]);
    }
    float* Wo = r.wc + bh * (D * D + D);
    {
        double zr[KSUB];
#pragma unroll
        for (int t = 0; t < KSUB; ++t) zr[t] = Z[ri * KSUB + t];
        const int j0 = 64 * (tid & 1);
#pragma unroll 2
        for (int j = j0; j < j0 + 64; j += 4) {
            f32x4 w;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                double v = 0.0;
#pragma unroll
                for (int t = 0; t < KSUB; ++t) v = fma(zr[t], V[(j + jj) * KSUB + t], v);
                w[jj] = static_cast<float>(v);
            }
            *reinterpret_cast<f32x4*>(Wo + ri * D + j) = w;
        }
    }
    {
        const int t = tid >> 5, part = tid & 31;
        double v = 0.0;
        for (int l = part; l < D; l += 32) v += rm[l] * V[l * KSUB + t] - xm[l] * Z[l * KSUB + t];
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        if (part == 0) s8[t] = v;
    }
    __syncthreads();
    if (tid < D) {
        double v = 0.0;
#pragma unroll
        for (int t = 0; t < KSUB; ++t) v = fma(s8[t], V[tid * KSUB + t], v);
        Wo[D * D + tid] = static_cast<float>(v);
    }
}

// ---- 5. apply: o <- o + c + (o Z) V_r^T; a row per 16 lanes, 8 columns per lane ----
constexpr int APPLY_ROWS = 256;                     // rows per workgroup

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// sum over the 16 lanes of a DPP row: quad swaps, then the half-row and row mirrors
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f32<0xB1>(x);
    x += dpp_f32<0x4E>(x);
    x += dpp_f32<0x141>(x);
    x += dpp_f32<0x140>(x);
    return x;
}

__global__ __launch_bounds__(THREADS) void apply_kernel(ResidualArgs r) {
    constexpr int RU = 4;                           // rows in flight per lane group
    const size_t bh = blockIdx.y;
    const int tid = threadIdx.x, c0 = 8 * (tid & 15), g = tid >> 4;
    const float* zv = r.zv + bh * 2 * D * KSUB;
    const float* cg = r.wc + bh * (D * D + D) + D * D;
    float z[8][KSUB], vr[8][KSUB], cc[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
#pragma unroll
        for (int h = 0; h < KSUB; h += 4) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(zv + (c0 + u) * KSUB + h);
            const f32x4 b = *reinterpret_cast<const f32x4*>(zv + D * KSUB + (c0 + u) * KSUB + h);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                z[u][h + e] = a[e];
                vr[u][h + e] = b[e];
            }
        }
        cc[u] = cg[c0 + u];
    }
    uint16_t* O = static_cast<uint16_t*>(r.out) + bh * r.N_pad * D;
    const int row0 = static_cast<int>(blockIdx.x) * APPLY_ROWS;
    for (int base = row0; base < row0 + APPLY_ROWS; base += RU * (THREADS / 16)) {
        u32x4 w[RU];
#pragma unroll
        for (int s = 0; s < RU; ++s) {
            const int row = base + g + s * (THREADS / 16);
            w[s] = row < r.N_pad ? *reinterpret_cast<const u32x4*>(O + static_cast<size_t>(row) * D + c0)
                                 : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int s = 0; s < RU; ++s) {
            const int row = base + g + s * (THREADS / 16);
            float o[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o[2 * e] = bf16_to_f32(static_cast<uint16_t>(w[s][e] & 0xFFFFu));
                o[2 * e + 1] = bf16_to_f32(static_cast<uint16_t>(w[s][e] >> 16));
            }
            float sv[KSUB];
#pragma unroll
            for (int t = 0; t < KSUB; ++t) {
                float a = 0.0f;
#pragma unroll
                for (int u = 0; u < 8; ++u) a = fmaf(o[u], z[u][t], a);
                sv[t] = row16_sum(a);
            }
            float res[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                float a = o[u] + cc[u];
#pragma unroll
                for (int t = 0; t < KSUB; ++t) a = fmaf(sv[t], vr[u][t], a);
                res[u] = a;
            }
            if (row < r.N_pad) {
                const int blk = row / BLK;
                if (row < r.N && row == probe_row(blk, r.N, r.phase)) {
                    const float* od = r.od + (bh * r.Mp + blk) * D + c0;
#pragma unroll
                    for (int u = 0; u < 8; ++u) res[u] = od[u];
                }
                u32x4 pk;
#pragma unroll
                for (int e = 0; e < 4; ++e) pk[e] = row < r.N ? pack_bf16x2(res[2 * e], res[2 * e + 1]) : 0u;
                *reinterpret_cast<u32x4*>(O + static_cast<size_t>(row) * D + c0) = pk;
            }
        }
    }
}

}  // namespace

int residual_key_chunks(int N_pad) { return min(8, N_pad / BLK); }

size_t residual_workspace_bytes(int B, int H, int N_pad) {
    const size_t bh = static_cast<size_t>(B) * H;
    const size_t mp = BLK * ((N_pad / BLK + BLK - 1) / BLK);
    const size_t kc = residual_key_chunks(N_pad);
    const size_t f64 = bh * (NSPLIT * (3 * D * D + 2 * D) + 3 * D * D);
    const size_t f32 = bh * (2 * mp * D + D * D + D) + kc * bh * mp * (D + 1) + bh * 2 * D * KSUB;
    const size_t b16 = bh * mp * D + bh * static_cast<size_t>(N_pad) * D;
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
    r.qp = reinterpret_cast<uint16_t*>(p);  p += bh * mp * D * 2;
    r.zv = reinterpret_cast<float*>(p);    p += bh * 2 * D * KSUB * 4;
    r.v16 = reinterpret_cast<uint16_t*>(p);
}

hipError_t launch_residual(const ResidualArgs& r, hipStream_t s) {
    const int bh = r.B * r.H;
    hipError_t e;
    hipLaunchKernelGGL(probe_gather_kernel, dim3((r.Mp * (D / 8) + THREADS - 1) / THREADS, bh), dim3(THREADS), 0, s, r);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const size_t chunks = static_cast<size_t>(bh) * r.N_pad * (D / 8);
    hipLaunchKernelGGL(value_f16_kernel, dim3(static_cast<unsigned>((chunks + THREADS - 1) / THREADS)), dim3(THREADS),
                       0, s, r);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // dense attention of the gathered probe queries (every key block exact, fp32 out)
    FwdArgs f{};
    f.B = r.B; f.H = r.H; f.N = r.N; f.N_pad = r.N_pad; f.d = D;
    f.comp = -1; f.scale = r.scale;
    f.q = r.qp; f.k = r.k; f.v = r.v; f.v16 = r.v16;
    f.out = r.odp; f.lse = r.lsep;
    f.Nq = r.N_pad / BLK; f.Nq_pad = r.Mp;
    f.dense = r.kchunks; f.out_f32 = 1;
    if ((e = launch_fwd_bf16(f, s)) != hipSuccess) return e;
    hipLaunchKernelGGL(combine_kernel, dim3((r.Mp * D + THREADS - 1) / THREADS, bh), dim3(THREADS), 0, s, r);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(gram_kernel, dim3(NSPLIT, 3, bh), dim3(THREADS), 0, s, r);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(reduce_kernel, dim3(3 * D * D / RED_PER_WG, bh), dim3(THREADS), 0, s, r);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(fit_factor_kernel, dim3(2, bh), dim3(THREADS), 0, s, r);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(fit_solve_kernel, dim3(bh), dim3(THREADS), 0, s, r);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(apply_kernel, dim3((r.N_pad + APPLY_ROWS - 1) / APPLY_ROWS, bh), dim3(THREADS), 0, s, r);
    return hipGetLastError();
}

}  // namespace sa
