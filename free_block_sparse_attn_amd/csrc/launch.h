// Internal kernel argument blocks and launchers (host side of each .hip file).
// The public C ABI in include/sparse_attn.h validates arguments and calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace sa {

struct PoolArgs {
    int B, H, N, N_pad, d;
    const void* q;
    const void* k;
    const void* v;
    float* qbar;
    float* kbar;
    float* vbar;
    int32_t* kcount;
    void* cent;       // fp16 [B,H,4,nbc,d] centroid planes, or null
    uint16_t* v16;    // fp16 [B,H,N_pad,d] copy of V, or null
    void* kmom;       // fp16 [B,H,nb,d*d] in MFMA operand order (scaled by 2^-kmom_exp), or null
    int8_t* kmom_exp; // [B,H,nb] exponent of each kmom block (with kmom)
    float* hbar;      // fp32 [B,H,d,d] value-major mean moment, or null
    float* hbar_ws;   // fp32 [B,H,64,d,d] partial sums (with hbar)
    float* kcov;      // fp32 [B,H,nb] ln ||H_j - H_bar||_2 (with hbar), or null
    float* klam;      // [B,H,nb] or null
    uint8_t* q8;      // e4m3 copies or null (all or none)
    uint8_t* k8;
    uint8_t* v8;
    int8_t* exp8;     // [B,H,nb,3]
    uint8_t* q4;      // MXFP4 copies or null (all six or none): packed E2M1 codes
    uint8_t* k4;
    uint8_t* v4;
    uint8_t* qs4;     // E8M0 scales: [B,H,N_pad,d/32] for q4 / k4, [B,H,nb,d] for v4
    uint8_t* ks4;
    uint8_t* vs4;
};
hipError_t launch_pool(const PoolArgs& a, bool bf16, hipStream_t s);
// (b, h) pairs whose H_bar partial sums fit the library-owned scratch
constexpr int POOL_STATIC_HEADS = 32;
// That scratch on the current device (resolved once per device), or null.
float* pool_static_scratch();

struct RouteArgs {
    int B, H, nb, d;
    int N;                    // valid tokens (error-aware mode)
    int mode;
    int topk;
    const int32_t* frame_lo;
    const int32_t* frame_hi;
    int window, anchors, anchor_phase, step;
    int n_keep, n_refine;
    float scale;
    const float* qbar;
    const float* kbar;
    const int32_t* kcount;
    const float* klam;        // per-block log term: lambda_j (Triage) or ln M_j (covariance top-k)
    const void* keys;         // bf16 [B,H,N_pad,d] token keys (error-aware mode)
    float* ekey;              // fp32 [B,H,nb(key),nb(query)] error logs (error-aware mode)
    int32_t* idx;
    int32_t* cnt;
    int cap;
    int32_t* idx2;
    int32_t* cnt2;
    int cap2;
};
hipError_t launch_route(const RouteArgs& a, hipStream_t s);

struct FwdArgs {
    int B, H, N, N_pad, d;
    int comp;                 // -1, 0, 1
    float scale;
    const void* q;
    const void* k;
    const void* v;
    const float* kbar;
    const float* vbar;
    const void* cent;         // fp16 centroid planes (bf16 path)
    const void* v16;          // fp16 copy of V (bf16 path)
    const int32_t* kcount;
    const void* kmom;         // fp16 moments, block j scaled by 2^-kmom_exp[j] (comp 1)
    const int8_t* kmom_exp;
    const float* hbar;        // fp32 [B,H,d,d] value-major (comp 2)
    const uint8_t* q8;
    const uint8_t* k8;
    const uint8_t* v8;
    const int8_t* exp8;
    const uint8_t* q4;        // MXFP4 skim copies (skim_fmt 1)
    const uint8_t* k4;
    const uint8_t* v4;
    const uint8_t* qs4;
    const uint8_t* ks4;
    const uint8_t* vs4;
    int skim_fmt;             // 0 e4m3, 1 MXFP4
    const int32_t* idx;
    const int32_t* cnt;
    int cap;
    const int32_t* idx2;
    const int32_t* cnt2;
    int cap2;
    void* out;
    float* lse;
    // query rows: Nq valid of Nq_pad (= N, N_pad for attention over the same
    // sequence); dense > 0: every key block is exact (no lists), split into
    // `dense` consecutive chunks of key blocks, chunk c writing its own
    // normalised O and lse at out / lse + c * B H Nq_pad (d) elements;
    // out_f32: write O in fp32 (bf16 path)
    int Nq, Nq_pad;
    int dense;
    int out_f32;
};
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s);

struct ResidualArgs {
    int B, H, N, N_pad;
    int Mp;                   // probe rows padded to a multiple of 64 (one probe per query block)
    int phase, rank;
    float scale, ridge;
    const void* q;            // bf16 [B,H,N_pad,128]
    const void* k;
    const void* v;
    void* out;                // bf16 [B,H,N_pad,128], corrected in place
    // carved from the caller's workspace (residual_carve)
    int kchunks;              // key chunks of the dense probe pass
    float* odp;               // [kchunks,B,H,Mp,d] dense output per key chunk
    float* lsep;              // [kchunks,B,H,Mp] its natural-log normaliser
    double* part;             // [B,H,8,3*d*d + 2*d] Gram partial sums
    double* mat;              // [B,H,3,d,d] X^T X, X^T R (then B), R^T R
    float* xp;                // [B,H,Mp,d] sparse output at the probes
    float* od;                // [B,H,Mp,d] dense output at the probes
    float* wc;                // [B,H,d*d + d] W, c
    uint16_t* qp;             // [B,H,Mp,d] gathered probe queries
    float* zv;                // [B,H,2,d,8] the factors Z and V_r of W = Z V_r^T
    uint16_t* v16;            // [B,H,N_pad,d] fp16 copy of V (dense probe pass)
};
size_t residual_workspace_bytes(int B, int H, int N_pad);
void residual_carve(ResidualArgs& r, void* ws);
hipError_t launch_residual(const ResidualArgs& r, hipStream_t s);

}  // namespace sa
