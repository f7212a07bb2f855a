// fp32 compensated block-sparse attention forward (d = 64) on the fp32
// matrix cores (v_mfma_f32_32x32x2_f32).
//
// One wave per (b, h, query block).  Exact key blocks, then the centroid
// pseudo-keys q.k_bar_j + ln n_j with values v_bar_j (zeroth-order
// compensation of every unselected block), go through one online softmax,
// so numerator and denominator share one normalisation (PISA, "PISA:
// Piecewise Sparse Attention Is Wiser for Efficient Diffusion
// Transformers", section 2, "Algorithme Central"; SVG-EAR section 2A).
//
// Per 64-key tile, S^T = K Q^T is four 32x32 accumulators (key half kh x
// query half qh), each the sum of 32 rank-2 MFMAs: step t pairs dimension t
// (lanes 0-31) with dimension 32 + t (lanes 32-63), so a lane's operands are
// 32 consecutive dimensions of one key row (LDS) or one query row
// (registers).  Lane l holds the logits of query column l % 32 against keys
// 32 kh + 8 (r / 4) + 4 (l / 32) + r % 4 (accumulator entry r); lane l ^ 32
// holds that query's other 32 keys.  O^T = V^T P^T walks the keys in that
// same order (step 16 kh + r takes key 32 kh + 8 (r / 4) + 4 (l / 32) + r % 4
// on lane half l / 32), so P^T's operand is the lane's own weight and V^T's
// is V[that key][32 dh + l % 32], read from LDS.
#include "common.h"
#include "launch.h"

namespace sa {

namespace {

constexpr int D = 64;
constexpr int KEPT_WORDS = 128;                    // nb <= 4096

// accumulator entry r of lane half h: key 8 (r / 4) + 4 h + r % 4 of a 32-key half
__device__ __forceinline__ int acc_key(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

__global__ __launch_bounds__(64) void fwd_f32_kernel(FwdArgs a) {
    __shared__ float ks[BLK][D + 1];               // padded rows: column reads hit 32 banks
    __shared__ float vs[BLK][D + 1];
    __shared__ float bias[BLK];
    __shared__ uint32_t kept[KEPT_WORDS];

    const int nq = a.N_pad / BLK, nb = nq;
    const int blk = blockIdx.x % nq;
    const size_t bh = blockIdx.x / nq;
    const int l = threadIdx.x, h = l >> 5, l32 = l & 31;
    const float* Q = static_cast<const float*>(a.q) + bh * a.N_pad * D;
    const float* K = static_cast<const float*>(a.k) + bh * a.N_pad * D;
    const float* V = static_cast<const float*>(a.v) + bh * a.N_pad * D;
    const float sc = a.scale;

    // Q^T operands: qo[qh][t] = Q[64 blk + 32 qh + l % 32][32 h + t] (pad rows 0)
    float qo[2][32];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
        const int row = blk * BLK + 32 * qh + l32;
        const bool valid = row < a.N;
#pragma unroll
        for (int t4 = 0; t4 < 8; ++t4) {
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            if (valid) x = *reinterpret_cast<const float4*>(Q + static_cast<size_t>(row) * D + 32 * h + 4 * t4);
            qo[qh][4 * t4 + 0] = x.x;
            qo[qh][4 * t4 + 1] = x.y;
            qo[qh][4 * t4 + 2] = x.z;
            qo[qh][4 * t4 + 3] = x.w;
        }
    }
    f32x16 o[2][2];                                // O^T[d half dh][query half qh]
#pragma unroll
    for (int dh = 0; dh < 2; ++dh)
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) o[dh][qh] = f32x16{};
    float m[2] = {-INFINITY, -INFINITY};           // running max of query l % 32 of each half
    float ls[2] = {0.f, 0.f};                      // this lane's part of its row sums

    const size_t rowid = bh * nq + blk;
    const int cntE = a.cap > 0 ? min(a.cnt[rowid], a.cap) : 0;
    const int32_t* list = a.idx + rowid * a.cap;
    for (int x = l; x < KEPT_WORDS; x += 64) kept[x] = 0u;
    __syncthreads();
    for (int e = l; e < cntE; e += 64) {
        const int j = list[e];
        atomicOr(&kept[j >> 5], 1u << (j & 31));
    }
    __syncthreads();

    // rows 0 .. nrows-1 of the 64-row tile from src (row-major, d = 64), zero beyond
    auto stage = [&](float (*dst)[D + 1], const float* src, int nrows) __attribute__((always_inline)) {
        for (int x = l; x < BLK * D / 4; x += 64) {
            const int r = x / (D / 4), c4 = (x % (D / 4)) * 4;
            float4 w = make_float4(0.f, 0.f, 0.f, 0.f);
            if (r < nrows) w = *reinterpret_cast<const float4*>(src + static_cast<size_t>(r) * D + c4);
            dst[r][c4] = w.x;
            dst[r][c4 + 1] = w.y;
            dst[r][c4 + 2] = w.z;
            dst[r][c4 + 3] = w.w;
        }
    };

    // one 64-key tile staged in ks / vs with per-key bias (-inf: no key)
    auto tile_update = [&]() __attribute__((always_inline)) {
        f32x16 s[2][2];                            // S^T[key half kh][query half qh]
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int qh = 0; qh < 2; ++qh) s[kh][qh] = f32x16{};
#pragma unroll
        for (int t = 0; t < 32; ++t)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const float ka = ks[32 * kh + l32][32 * h + t];
#pragma unroll
                for (int qh = 0; qh < 2; ++qh)
                    s[kh][qh] = __builtin_amdgcn_mfma_f32_32x32x2f32(ka, qo[qh][t], s[kh][qh], 0, 0, 0);
            }
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
            float mx = -INFINITY;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float x = s[kh][qh][r] * sc + bias[32 * kh + acc_key(r, h)];
                    s[kh][qh][r] = x;
                    mx = fmaxf(mx, x);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mnew = fmaxf(m[qh], mx);
            const bool none = mnew == -INFINITY;   // no key of this query so far
            const float corr = none ? 1.0f : expf(m[qh] - mnew);
            ls[qh] *= corr;
#pragma unroll
            for (int dh = 0; dh < 2; ++dh)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dh][qh][r] *= corr;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = none ? 0.f : expf(s[kh][qh][r] - mnew);
                    s[kh][qh][r] = p;
                    ls[qh] += p;
                }
            m[qh] = mnew;
        }
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 32 * kh + acc_key(r, h);
#pragma unroll
                for (int dh = 0; dh < 2; ++dh) {
                    const float va = vs[key][32 * dh + l32];
#pragma unroll
                    for (int qh = 0; qh < 2; ++qh)
                        o[dh][qh] = __builtin_amdgcn_mfma_f32_32x32x2f32(va, s[kh][qh][r], o[dh][qh], 0, 0, 0);
                }
            }
    };

    // exact blocks (keys past the sequence end drop out)
    for (int e = 0; e < cntE; ++e) {
        const int j = list[e];
        const int nj = min(BLK, a.N - BLK * j);
        __syncthreads();
        stage(ks, K + static_cast<size_t>(j) * BLK * D, nj);
        stage(vs, V + static_cast<size_t>(j) * BLK * D, nj);
        bias[l] = l < nj ? 0.f : -INFINITY;
        __syncthreads();
        tile_update();
    }
    // centroid pseudo-keys of every unselected block, 64 per tile
    if (a.comp >= 0) {
        for (int c0 = 0; c0 < nb; c0 += BLK) {
            const int nc = min(BLK, nb - c0);
            __syncthreads();
            stage(ks, a.kbar + (bh * nb + c0) * D, nc);
            stage(vs, a.vbar + (bh * nb + c0) * D, nc);
            const int jj = c0 + l;
            float bv = -INFINITY;
            if (jj < nb && !((kept[jj >> 5] >> (jj & 31)) & 1u)) bv = logf(static_cast<float>(a.kcount[jj]));
            bias[l] = bv;
            __syncthreads();
            tile_update();
        }
    }

    // O = O^T / l: lane l writes query 32 qh + l % 32, dimensions
    // 32 dh + 8 (r / 4) + 4 h .. + 3 as float4s; pad rows 0
    float* O = static_cast<float*>(a.out) + bh * a.N_pad * D;
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
        const int row = blk * BLK + 32 * qh + l32;
        const bool valid = row < a.N;
        const float lt = ls[qh] + __shfl_xor(ls[qh], 32);
        const float inv = valid ? 1.0f / lt : 0.f;
#pragma unroll
        for (int dh = 0; dh < 2; ++dh)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 w = make_float4(o[dh][qh][4 * g] * inv, o[dh][qh][4 * g + 1] * inv,
                                             o[dh][qh][4 * g + 2] * inv, o[dh][qh][4 * g + 3] * inv);
                *reinterpret_cast<float4*>(O + static_cast<size_t>(row) * D + 32 * dh + 8 * g + 4 * h) = w;
            }
        if (a.lse && h == 0) a.lse[bh * a.N_pad + row] = valid ? m[qh] + logf(lt) : 0.f;
    }
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) {
    const int nq = a.N_pad / BLK;
    dim3 grid(nq * a.H * a.B);
    hipLaunchKernelGGL(fwd_f32_kernel, grid, dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace sa
