// fp32 compensated block-sparse attention forward (d = 64), vector-ALU path.
//
// One wave per (b, h, query block); lane t owns query row t of the block and
// keeps its q row, output accumulator and one tile of 64 logits in
// registers.  Exact key blocks are staged through LDS (broadcast reads), then
// the centroid pseudo-keys q.k_bar_j + ln n_j with values v_bar_j (zeroth-
// order compensation of every unselected block) go through the same online
// softmax, so numerator and denominator share one normalisation (PISA,
// "PISA: Piecewise Sparse Attention Is Wiser for Efficient Diffusion
// Transformers", section 2, "Algorithme Central"; SVG-EAR section 2A).
#include "common.h"
#include "launch.h"

namespace sa {

namespace {

constexpr int D = 64;

__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) void fwd_f32_kernel(FwdArgs a) {
    __shared__ float ks[BLK][D + 1];
    __shared__ float vs[BLK][D + 1];
    __shared__ uint32_t kept[128];                     // nb <= 4096

    const int nq = a.N_pad / BLK, nb = nq;
    const int blk = blockIdx.x % nq;
    const size_t bh = blockIdx.x / nq;
    const int lane = threadIdx.x;
    const int row = blk * BLK + lane;
    const bool valid = row < a.N;
    const float* Q = static_cast<const float*>(a.q) + bh * a.N_pad * D;
    const float* K = static_cast<const float*>(a.k) + bh * a.N_pad * D;
    const float* V = static_cast<const float*>(a.v) + bh * a.N_pad * D;
    const float sc = a.scale;

    float q[D], o[D];
#pragma unroll
    for (int i = 0; i < D; ++i) { q[i] = valid ? Q[static_cast<size_t>(row) * D + i] : 0.f; o[i] = 0.f; }
    float m = -INFINITY, l = 0.f;

    const size_t rowid = bh * nq + blk;
    const int cntE = a.cap > 0 ? min(a.cnt[rowid], a.cap) : 0;
    const int32_t* list = a.idx + rowid * a.cap;
    for (int x = lane; x < 128; x += 64) kept[x] = 0u;
    __syncthreads();
    for (int e = lane; e < cntE; e += 64) {
        const int j = list[e];
        atomicOr(&kept[j >> 5], 1u << (j & 31));
    }
    __syncthreads();

    auto tile_update = [&](int nvalid, const float* bias) __attribute__((always_inline)) {
        float s[BLK];
        float mx = -INFINITY;
#pragma unroll
        for (int n = 0; n < BLK; ++n) {
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < D; ++i) acc = fmaf(q[i], ks[n][i], acc);
            float x = acc * sc + bias[n];
            if (n >= nvalid) x = -INFINITY;
            s[n] = x;
            mx = fmaxf(mx, x);
        }
        if (mx == -INFINITY) return;
        const float mnew = fmaxf(m, mx);
        const float corr = expf(m - mnew);
        l *= corr;
#pragma unroll
        for (int i = 0; i < D; ++i) o[i] *= corr;
#pragma unroll
        for (int n = 0; n < BLK; ++n) {
            const float p = expf(s[n] - mnew);
            l += p;
#pragma unroll
            for (int i = 0; i < D; ++i) o[i] = fmaf(p, vs[n][i], o[i]);
        }
        m = mnew;
    };

    __shared__ float bias[BLK];
    // exact blocks
    for (int e = 0; e < cntE; ++e) {
        const int j = list[e];
        const int nj = min(BLK, a.N - BLK * j);
        __syncthreads();
        for (int x = lane; x < BLK * D / 4; x += 64) {
            const int r = x / (D / 4), c4 = (x % (D / 4)) * 4;
            float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
            if (r < nj) {
                kv = *reinterpret_cast<const float4*>(K + (static_cast<size_t>(j) * BLK + r) * D + c4);
                vv = *reinterpret_cast<const float4*>(V + (static_cast<size_t>(j) * BLK + r) * D + c4);
            }
            ks[r][c4] = kv.x; ks[r][c4 + 1] = kv.y; ks[r][c4 + 2] = kv.z; ks[r][c4 + 3] = kv.w;
            vs[r][c4] = vv.x; vs[r][c4 + 1] = vv.y; vs[r][c4 + 2] = vv.z; vs[r][c4 + 3] = vv.w;
        }
        bias[lane] = 0.f;
        __syncthreads();
        tile_update(nj, bias);
    }
    // centroid pseudo-keys of every unselected block
    if (a.comp >= 0) {
        for (int c0 = 0; c0 < nb; c0 += BLK) {
            __syncthreads();
            for (int x = lane; x < BLK * D / 4; x += 64) {
                const int r = x / (D / 4), c4 = (x % (D / 4)) * 4;
                const int jj = c0 + r;
                float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
                if (jj < nb) {
                    kv = *reinterpret_cast<const float4*>(a.kbar + (bh * nb + jj) * D + c4);
                    vv = *reinterpret_cast<const float4*>(a.vbar + (bh * nb + jj) * D + c4);
                }
                ks[r][c4] = kv.x; ks[r][c4 + 1] = kv.y; ks[r][c4 + 2] = kv.z; ks[r][c4 + 3] = kv.w;
                vs[r][c4] = vv.x; vs[r][c4 + 1] = vv.y; vs[r][c4 + 2] = vv.z; vs[r][c4 + 3] = vv.w;
            }
            {
                const int jj = c0 + lane;
                float bv = -INFINITY;
                if (jj < nb && !((kept[jj >> 5] >> (jj & 31)) & 1u)) bv = logf(static_cast<float>(a.kcount[jj]));
                bias[lane] = bv;
            }
            __syncthreads();
            tile_update(BLK, bias);
        }
    }
    float* O = static_cast<float*>(a.out) + bh * a.N_pad * D;
    const float inv = valid ? 1.0f / l : 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) O[static_cast<size_t>(row) * D + i] = o[i] * inv;
    if (a.lse) a.lse[bh * a.N_pad + row] = valid ? m + logf(l) : 0.f;
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) {
    const int nq = a.N_pad / BLK;
    dim3 grid(nq * a.H * a.B);
    hipLaunchKernelGGL(fwd_f32_kernel, grid, dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace sa
