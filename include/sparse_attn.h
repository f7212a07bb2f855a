/*
 * sparse_attn.h - C ABI of the MI355X (gfx950) compensated block-sparse
 * attention library: pool -> route -> fused forward.
 *
 * The method.  Self-attention over a video token sequence is cut into
 * 64-token blocks.  For every query block only some key blocks are computed
 * exactly; every other key block is not dropped but compensated inside the
 * same softmax normalisation:
 *   - zeroth order: the block's n_j keys and values are replaced by their
 *     means, i.e. a pseudo-logit q.k_bar_j + ln n_j with value v_bar_j
 *     (page "SVG-EAR: Parameter-Free Linear Compensation for Sparse Video
 *     Generation via Error-aware Routing", section 2A; page "PISA: Piecewise
 *     Sparse Attention Is Wiser for Efficient Diffusion Transformers",
 *     section 2 "Algorithme Central", zeroth-order block term
 *     alpha_{t,j} * sum_n v_{j,n} with alpha_{t,j} = exp(q_t k_bar_j));
 *   - first order (optional): PISA's block Taylor term
 *     exp(q.k_bar_j) * (q^T H_j) with the per-block moment
 *     H_j = sum_n (k_n - k_bar_j) v_n^T (PISA section 2, per-block
 *     first-order matrices);
 *   - a low-precision tier (optional): key blocks computed from fp8 e4m3
 *     copies (page "Triage: Skip, Skim, or Refine Attention Tiles in Video
 *     Diffusion Transformers", the skim tier of its per-tile choice).
 * Routing chooses the exact blocks by top-k on pooled block scores (PISA),
 * by LVSA's local window plus rotating global anchors (page "LVSA:
 * Training-Free Sparse Attention for Long Video Diffusion", section 2
 * "Mecanisme Central"), or by Triage's three tiers.
 *
 * Conventions shared by every call
 *   - Tensors are dense, contiguous, row-major device buffers owned by the
 *     caller; the library never allocates, frees or retains them and keeps
 *     no state between calls.
 *   - Token tensors are [B, H, N_pad, d] with N_pad = 64 * ceil(N / 64);
 *     tokens N .. N_pad-1 are padding: they are never read into a result
 *     and their contents may be anything.  nb = N_pad / 64 blocks; block j
 *     holds n_j = min(64, N - 64 j) valid tokens.
 *   - Every argument is validated on the host before any HIP call.  On a
 *     validation error nothing is launched and no output is touched.
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream).
 *     Launch failures return SA_ERR_HIP; faults inside kernels surface at
 *     the caller's next synchronisation, as for any HIP library.
 *   - Every device pointer must be 16-byte aligned.
 *   - B == 0, H == 0 or N == 0 is a valid empty problem: nothing is
 *     launched and SA_OK is returned.
 *   - Calls are thread-safe; the last-error text is thread-local.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPARSE_ATTN_ABI_VERSION 9
#define SPARSE_ATTN_BLOCK 64

typedef enum {
    SA_OK = 0,
    SA_ERR_INVALID_ARG = 1,   /* a null, misaligned, negative or inconsistent argument */
    SA_ERR_UNSUPPORTED = 2,   /* a valid request this build does not implement */
    SA_ERR_HIP = 3            /* a HIP launch failed; see sparse_attn_last_error() */
} sa_status;

typedef enum {
    SA_F32 = 0,               /* fp32 token tensors */
    SA_BF16 = 1               /* bf16 token tensors (the MFMA path) */
} sa_dtype;

typedef enum {
    SA_COMP_DROP = -1,        /* unselected blocks contribute nothing */
    SA_COMP_ORDER0 = 0,       /* centroid term n_j exp(q.k_bar_j) v_bar_j */
    SA_COMP_ORDER1_BLOCK = 1, /* centroid term + per-block Taylor term with H_j */
    SA_COMP_ORDER1_GLOBAL = 2 /* centroid term + PISA's global Taylor term with H_bar */
} sa_comp;

typedef enum {
    SA_ROUTE_TOPK = 0,
    SA_ROUTE_LVSA = 1,
    SA_ROUTE_TRIAGE = 2,
    SA_ROUTE_TOPK_COV = 3,
    SA_ROUTE_ERROR = 4
} sa_route_mode;

typedef enum {
    SA_SKIM_E4M3 = 0,         /* skim tier in fp8 e4m3, one scale per block and tensor */
    SA_SKIM_MXFP4 = 1         /* skim tier in MXFP4 (fp4 E2M1, E8M0 scales per 32 values) */
} sa_skim_format;

/* Problem shape.  d must be 64 or 128. */
typedef struct {
    int32_t B, H, N, N_pad, d;
} sa_shape;

/*
 * sparse_attn_pool - per-block statistics (the precompute step of PISA's
 * fused pipeline, section 2 "Implementation Materielle": centroids, value
 * sums and first-order matrices are computed before the attention pass).
 *
 * Inputs  q, k, v        dtype [B,H,N_pad,d]
 * Outputs (required)
 *   qbar, kbar, vbar     fp32 [B,H,nb,d]  block means over valid tokens.
 *                        Contract: fp64 sum of the valid tokens in increasing
 *                        token order from +0.0, fp64 division by n_j, then
 *                        round-to-nearest-even to fp32.  These are the
 *                        routing features; they are bit-reproducible.
 *   kcount               int32 [nb]       n_j (same for every b, h).
 * Outputs (optional, NULL to skip)
 *   cent                 fp16 [B,H,4,nbc,d], nbc = 64 * ceil(nb / 64): the
 *                        centroids in the form the bf16 forward pass reads.
 *                        With m the fp32 mean above, hi = fp16_rne(m) and
 *                        lo = fp16_rne(m - hi) (the difference is exact in
 *                        fp32), so hi + lo carries m to about 22 bits:
 *                        plane 0 hi(k_bar), 1 lo(k_bar), 2 hi(v_bar),
 *                        3 lo(v_bar); rows nb .. nbc-1 are 0.  bf16 inputs
 *                        with d == 128 only.
 *   v16                  fp16 [B,H,N_pad,d]  fp16_rne(v), the value operand of
 *                        the bf16 forward pass (exact for bf16 values of
 *                        magnitude 2^-14 .. 65504; below, rounded to fp16's
 *                        subnormal step 2^-24; beyond 65504, inf).  Pad rows
 *                        are 0.  bf16 inputs with d == 128 only.
 *   kmom, kmom_exp       fp16 [B,H,nb,d*d] and int8 [B,H,nb], together: the
 *                        moment of block j, G[o][i] = sum_n (k_n[i] -
 *                        k_bar_j[i]) v_n[o] (H_j transposed), stored as
 *                        fp16_rne(G 2^-e_j) with e_j = kmom_exp[j] chosen so
 *                        that the largest |entry| lands in [2^14, 2^15) (0 for
 *                        an all-zero block), in the forward pass's MFMA
 *                        operand order: G[o][i] at element
 *                        ((o/32 * 8 + i/16) * 64 + o%32 + 32 * ((i/8) % 2)) * 8
 *                        + i%8 of the block.  bf16 inputs with d == 128 only.
 *   hbar                 fp32 [B,H,d,d]  PISA's global first-order statistic
 *                        H_bar = (1/nb) sum_j H_j over all blocks of the head
 *                        (section 2, "Algorithme Central": the mean of the
 *                        per-block first-order matrices), stored value-major
 *                        like kmom's G: hbar[..., o, i] = H_bar[i][o].  Needs
 *                        hbar_ws, fp32 [B,H,64,d,d] caller-owned scratch
 *                        (64 partial sums per head, summed in a fixed order,
 *                        so the result is bit-reproducible).  bf16 inputs with
 *                        d == 128 only.
 *   kcov                 fp32 [B,H,nb]  ln M_j, M_j = ||H_j - H_bar||_2 (the
 *                        largest singular value of the block's deviation from
 *                        the mean moment): the statistic of PISA's
 *                        covariance-aware top-k (section 2, "Routage Sensible
 *                        a la Covariance").  H_j is rebuilt in fp32 (never
 *                        stored); M_j^2 is the largest eigenvalue of
 *                        A = (H_j - H_bar) (H_j - H_bar)^T (that of the
 *                        product in the other order), taken from up to
 *                        32 Lanczos steps on A (fixed start vector, partial
 *                        sums combined in a fixed order, so deterministic;
 *                        the steps stop once the top Ritz value moved by at
 *                        most 2^-15 of itself over 8 steps) and
 *                        64-point multisection of the Lanczos tridiagonal
 *                        with Sturm counts; the Ritz value approaches M_j^2
 *                        from below and lands within fp32 rounding of it even
 *                        where the two top singular values are within a few
 *                        percent.  -inf when M_j = 0.  Needs hbar (and
 *                        hbar_ws).
 *   klam                 fp32 [B,H,nb]  lambda_j = ln(r_k r_v),
 *                        r_x^2 = sum_n ||x_n - x_bar_j||^2 (Triage router's
 *                        omission-error statistic); -inf for 1-token blocks.
 *   q8, k8, v8, exp8     fp8 e4m3 (OCP) copies with one power-of-two scale
 *                        per block and tensor: x8 = e4m3_rne(x * 2^-e), e =
 *                        smallest integer with amax_block * 2^-e <= 448;
 *                        exp8 int8 [B,H,nb,3] holds e for (q, k, v).
 *                        q8, k8: uint8 [B,H,N_pad,d] row-major.
 *                        v8: uint8 [B,H,nb,d,64] block-transposed: entry
 *                        (j, i, p) is value dimension i of key 64 j + kappa(p),
 *                        kappa(p) = 32((p%32)/16) + 8((p%16)/4) + 4(p/32) + p%4
 *                        (the key order of the forward pass's fp8 P operand).
 *                        Pad keys are written as 0.  All
 *                        four pointers or none.  bf16 inputs only.
 *   q4, k4, v4, qs4, ks4, vs4  MXFP4 copies for the 4-bit skim tier (Triage's
 *                        fast tier in the page's own 4 bits, "Triage: Skip,
 *                        Skim, or Refine Attention Tiles in Video Diffusion
 *                        Transformers").  Elements are OCP E2M1 codes (nearest,
 *                        ties to the even code, magnitude 0 as +0) of x 2^-e,
 *                        e the smallest integer with amax 2^-e <= 6 over the
 *                        scale's group (at least -127); scales are E8M0 bytes
 *                        e + 127.  Two codes per byte, the even element in
 *                        the low nibble.
 *                        q4, k4: uint8 [B,H,N_pad,d/2] row-major; qs4, ks4:
 *                        uint8 [B,H,N_pad,d/32], one scale per token and 32
 *                        dimensions (the reduction axis of Q K^T).
 *                        v4: uint8 [B,H,nb,d,32] block-transposed in the
 *                        position order of v8 (kappa above); vs4: uint8
 *                        [B,H,nb,d], one scale per block and dimension over
 *                        the block's valid keys (the reduction axis of P V).
 *                        Pad tokens are code 0 with scale byte 127.  All six
 *                        pointers or none.  bf16 inputs with d == 128 only.
 */
sa_status sparse_attn_pool(const sa_shape* shape, sa_dtype dtype,
                           const void* q, const void* k, const void* v,
                           float* qbar, float* kbar, float* vbar, int32_t* kcount,
                           void* cent, void* v16, void* kmom, int8_t* kmom_exp,
                           float* hbar, float* hbar_ws, float* kcov, float* klam,
                           uint8_t* q8, uint8_t* k8, uint8_t* v8, int8_t* exp8,
                           uint8_t* q4, uint8_t* k4, uint8_t* v4, uint8_t* qs4, uint8_t* ks4, uint8_t* vs4,
                           hipStream_t stream);

/*
 * sparse_attn_pool_static - sparse_attn_pool for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments and results without
 * hbar_ws.  The H_bar partial sums go to a scratch array the library owns,
 * SPARSE_ATTN_POOL_STATIC_HEADS * 64 * d * d fp32 (128 MiB at d = 128), one
 * copy per GPU the library runs on, held until the process ends.  Requests
 * with hbar and B * H > SPARSE_ATTN_POOL_STATIC_HEADS return
 * SA_ERR_UNSUPPORTED and launch nothing.  Nothing in the scratch carries over
 * from one call to the next (every partial a call reads it wrote first), but
 * all calls on one GPU share it: calls that overlap in time on one GPU race
 * and must be ordered by the caller (one stream, or events).  Calls no
 * allocating routine.
 */
#define SPARSE_ATTN_POOL_STATIC_HEADS 32
sa_status sparse_attn_pool_static(const sa_shape* shape, sa_dtype dtype,
                                  const void* q, const void* k, const void* v,
                                  float* qbar, float* kbar, float* vbar, int32_t* kcount,
                                  void* cent, void* v16, void* kmom, int8_t* kmom_exp,
                                  float* hbar, float* kcov, float* klam,
                                  uint8_t* q8, uint8_t* k8, uint8_t* v8, int8_t* exp8,
                                  uint8_t* q4, uint8_t* k4, uint8_t* v4, uint8_t* qs4, uint8_t* ks4, uint8_t* vs4,
                                  hipStream_t stream);

/* Routing request.  Unused fields are ignored by the other modes. */
typedef struct {
    int32_t mode;                 /* sa_route_mode */
    /* SA_ROUTE_TOPK, SA_ROUTE_TOPK_COV, SA_ROUTE_ERROR: keep `topk` (1..nb)
       key blocks per query block. */
    int32_t topk;
    /* SA_ROUTE_LVSA: device int32 [nb] first/last latent frame of each block. */
    const int32_t* frame_lo;
    const int32_t* frame_hi;
    int32_t window;               /* +- frames around the query block's frames */
    int32_t anchors;              /* rotating anchor key blocks (0..nb) */
    int32_t anchor_phase;         /* seeded offset o >= 0 */
    int32_t step;                 /* denoising step s >= 0 */
    /* SA_ROUTE_TRIAGE: tiers per query block. */
    int32_t n_keep;               /* refine + skim blocks (1..nb) */
    int32_t n_refine;             /* refine blocks (0..n_keep) */
    float scale;                  /* softmax scale in the keys (TRIAGE, TOPK_COV, ERROR) */
    /* SA_ROUTE_ERROR */
    const void* keys;             /* device bf16 [B,H,N_pad,d] token keys (d == 128) */
    float* ekey;                  /* device fp32 [B,H,nb,nb] caller workspace; on return
                                     ekey[b,h,j,a] = L(a, j) (key block j, query block a) */
} sa_route_spec;

/*
 * sparse_attn_route - choose the key blocks of every query block.
 *
 * Scores (TOPK, TOPK_COV, TRIAGE, ERROR): s(a, j) = sum_i qbar[a,i] * kbar[j,i], fp64,
 * accumulated in i = 0..d-1 order (products of fp32 values are exact in
 * fp64).  Selections use the total order (-key, j): ties go to the lower
 * block index.  Lists are written ascending, padded with -1 up to `cap`.
 *
 *   TOPK   idx/cnt = the topk best blocks by s (PISA's top-k critical set);
 *          cap >= topk.  idx2/cnt2 unused (may be NULL).
 *   TOPK_COV  PISA's covariance-aware top-k (section 2, "Routage Sensible
 *          a la Covariance"): key = fl(fl(scale s) + kterm_j) (fp64) with
 *          kterm = ln M_j (sparse_attn_pool's kcov); the first topk blocks
 *          by (-key, j).  The key is the log of the bound
 *          exp(scale q.k_bar_j) |q| M_j on the first-order error a skipped
 *          block leaves after the global H_bar term, up to the row's |q|.
 *          cap >= topk.  Needs kterm.
 *   ERROR  SVG-EAR error-aware routing ("SVG-EAR: Parameter-Free Linear
 *          Compensation for Sparse Video Generation via Error-aware Routing",
 *          section 2B).  With the query-block centroid qbar_a as the proxy
 *          of its queries, E(a, j) = sum_n (e^{scale qbar_a.k_n} -
 *          e^{scale qbar_a.kbar_j})^2 is the squared error of its attention
 *          weights when block j's keys are replaced by their centroid.  A
 *          streaming pass over all keys writes L(a, j) = ln sum_n
 *          expm1(scale qbar_a.(k_n - kbar_j))^2 to ekey (fp32; the product
 *          is formed from bf16 high + low parts of both factors, three MFMA
 *          passes, fp32 sums); then key = fl(fl(2 fl(scale s) + L) - ln n_j)
 *          = ln(E / n_j) (fp64) and the first topk blocks by (-key, j) are
 *          kept: the greedy error-to-cost choice with one tile per block.
 *          cap >= topk.  Needs kcount, spec->keys, spec->ekey; d == 128.
 *   LVSA   idx/cnt = {j : [lo_j, hi_j] meets [lo_a - window, hi_a + window]}
 *          U {((phase + step) mod P) + i P : i < anchors}, P = nb / anchors.
 *          A row longer than cap is truncated to its first cap blocks while
 *          cnt holds the full length; sparse_attn_lvsa_capacity() gives the
 *          cap that avoids truncation.
 *   TRIAGE e_skip = fl(fl(scale s) + lambda_j), w = fl(fl(scale s) + ln n_j)
 *          (fp64).  The first n_keep blocks by (-e_skip, j) are kept; of
 *          those the first n_refine by (-w, j) go to idx/cnt (refine, exact
 *          bf16, cap >= n_refine) and the rest to idx2/cnt2 (skim, fp8,
 *          cap2 >= n_keep - n_refine).  Needs kterm = lambda_j
 *          (sparse_attn_pool's klam) and kcount.
 *
 * qbar, kbar  fp32 [B,H,nb,d] (sparse_attn_pool outputs)
 * kcount      int32 [nb]      (TRIAGE, ERROR)
 * kterm       fp32 [B,H,nb]   per-block log term (TRIAGE: lambda_j; TOPK_COV: ln M_j)
 * idx         int32 [B,H,nb,cap]   cnt int32 [B,H,nb]
 * idx2        int32 [B,H,nb,cap2]  cnt2 int32 [B,H,nb]  (TRIAGE)
 */
sa_status sparse_attn_route(const sa_shape* shape, const sa_route_spec* spec,
                            const float* qbar, const float* kbar,
                            const int32_t* kcount, const float* kterm,
                            int32_t* idx, int32_t* cnt, int32_t cap,
                            int32_t* idx2, int32_t* cnt2, int32_t cap2,
                            hipStream_t stream);

/* Host helper: the longest LVSA row for host copies of the frame ranges. */
int32_t sparse_attn_lvsa_capacity(const int32_t* frame_lo_host, const int32_t* frame_hi_host,
                                  int32_t nb, int32_t window, int32_t anchors);

/*
 * sparse_attn_fwd - fused compensated block-sparse attention forward.
 *
 * For query t in block a with exact list E (idx), skim list M (idx2) and
 * the remaining blocks U, computes o_t = N_t / D_t in one online softmax
 * (PISA section 2: the approximations enter numerator and denominator of a
 * single normalisation):
 *   exact   sum_{j in E} sum_n e^{scale q.k_n} (v_n)              bf16 MFMA
 *   skim    sum_{j in M} low-precision logits and P V via the block-scaled
 *           MFMA: skim_fmt SA_SKIM_E4M3 takes the e4m3 copies (one scale per
 *           block and tensor), SA_SKIM_MXFP4 the MXFP4 copies (per-lane E8M0
 *           scales of 32 values); P is e4m3 in both, quantised per row and
 *           tile against a power of two 2^ceil(max L); D takes the
 *           unquantised weights
 *   order0  sum_{j in U} n_j e^{scale q.k_bar_j} (v_bar_j)         comp >= 0
 *   order1  sum_{j in U} e^{scale q.k_bar_j} scale q^T H_j  (N only)  comp == 1
 *   global  scale (sum_{j in U} e^{scale q.k_bar_j}) q^T H_bar (N only) comp == 2
 *           (PISA section 2, "Algorithme Central": the hybrid-order form,
 *           one d x d statistic for every skipped block)
 * Precision (SA_BF16): logits of the exact tiles come from bf16 MFMA on
 * q and k (exact products, fp32 sums).  The exact and centroid weights enter
 * the value products rounded to fp16 (11 significant bits) against the fp16
 * copy of v, and D sums those same rounded weights in fp32, so their
 * rounding cancels in o (every comp); lse = ln D is within 2^-11 relative of
 * the sum of the unrounded weights.  The centroid logits and the first-order
 * products run in fp16 MFMA (q converted once; centroid means as fp16 high +
 * low parts; moments with their block exponents).  Skim weights enter D
 * unquantised (see skim).  Domain: q, k and v within fp16's range
 * (|x| <= 65504); beyond it the fp16 operands overflow and the rows that use
 * them are undefined.
 *
 * scale      softmax scale, finite and > 0
 * q, k, v    dtype [B,H,N_pad,d]
 * kbar, vbar fp32 [B,H,nb,d] centroids (SA_F32 with comp >= 0; unused by
 *            SA_BF16, may be NULL there)
 * cent       fp16 [B,H,4,nbc,d] centroid planes from sparse_attn_pool
 *            (SA_BF16 with comp >= 0; unused by SA_F32)
 * v16        fp16 [B,H,N_pad,d] copy of v from sparse_attn_pool (SA_BF16:
 *            the value operand of the exact tiles)
 * kcount     int32 [nb]
 * kmom, kmom_exp  fp16 moments and their block exponents (comp == 1)
 * hbar       fp32 [B,H,d,d] from sparse_attn_pool (comp == 2, SA_BF16)
 * q8, k8, v8, exp8                      from sparse_attn_pool (skim, SA_SKIM_E4M3)
 * skim_fmt   sa_skim_format of the skim tier
 * q4, k4, v4, qs4, ks4, vs4             from sparse_attn_pool (skim, SA_SKIM_MXFP4)
 * idx, cnt, cap     exact lists (ascending, entries in [0, nb))
 * idx2, cnt2, cap2  skim lists, or NULL / 0 when there is no skim tier
 * out        dtype [B,H,N_pad,d]: fp32 accumulation rounded to the output
 *            dtype (RNE); pad rows are written as 0.
 * lse        fp32 [B,H,N_pad] natural-log normaliser ln D_t, or NULL;
 *            pad rows are written as 0.
 * A row's count is clamped to its cap.  Every row must hold at least one
 * exact or skim block when comp == SA_COMP_DROP.
 * Supported: SA_F32 with d == 64 (comp <= 0, no skim); SA_BF16 with
 * d == 128 (every comp).
 */
sa_status sparse_attn_fwd(const sa_shape* shape, sa_dtype dtype, sa_comp comp, float scale,
                          const void* q, const void* k, const void* v,
                          const float* kbar, const float* vbar, const void* cent,
                          const void* v16, const int32_t* kcount, const void* kmom, const int8_t* kmom_exp,
                          const float* hbar,
                          const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                          const int8_t* exp8, sa_skim_format skim_fmt,
                          const uint8_t* q4, const uint8_t* k4, const uint8_t* v4,
                          const uint8_t* qs4, const uint8_t* ks4, const uint8_t* vs4,
                          const int32_t* idx, const int32_t* cnt, int32_t cap,
                          const int32_t* idx2, const int32_t* cnt2, int32_t cap2,
                          void* out, float* lse, hipStream_t stream);

/*
 * sparse_attn_residual - SparsePR's probe-fitted residual reconstruction
 * ("Partition the Support, Reconstruct the Residual: ...", section 2B), a
 * post-pass that corrects the output of sparse_attn_fwd in place.
 *
 * One probe row per query block a, row 64 a + ((phase + 37 a) mod n_a), is
 * computed by dense attention (every key block exact, fp32).  With X the
 * sparse outputs and R = O_dense - X at the probes, the residual is fitted as
 * R ~ b + X B by ridge regression on the centred probes (lambda = ridge *
 * tr(Xc^T Xc) / d, intercept not penalised; fp64 normal equations solved by
 * an LDL^T elimination) and restricted to the span of the top `rank` right
 * singular vectors of R (simultaneous iteration on R^T R, 8 columns, Cholesky
 * QR after each of 16 to 32 steps, stopping early once the leading `rank`
 * columns' span moves by less than 1e-10 (squared sines) over 4 steps; then
 * Rayleigh-Ritz on the 8-column span, the leading `rank` Ritz vectors):
 * W = B P, c = b P.  Every valid
 * row then gets o + c + o W, evaluated in fp32 as o + c + (o Z) V_r^T with
 * W = Z V_r^T, each probe row its dense output (RNE to bf16); pad rows 0.
 *
 * dtype      SA_BF16; d == 128
 * scale      the softmax scale of the forward call, finite and > 0
 * q, k, v    bf16 [B,H,N_pad,d]
 * out        bf16 [B,H,N_pad,d]: the sparse output on entry, corrected on return
 * phase      >= 0, picks the probe rows; ridge finite >= 0; rank in [1, 8]
 * workspace  device memory of at least sparse_attn_residual_workspace()
 *            bytes, 16-byte aligned, laid out as (Mp = 64 ceil(nb / 64)):
 *              fp64 [B,H,8,3 d d + 2 d]  Gram partial sums
 *              fp64 [B,H,3,d,d]          X^T X, then B; X^T R; R^T R
 *              fp32 [B,H,Mp,d]           X (sparse output at the probes)
 *              fp32 [B,H,Mp,d]           dense output at the probes
 *              fp32 [B,H,d d + d]        W (row-major, o W), then c
 *              fp32 [K,B,H,Mp,d], fp32 [K,B,H,Mp]  the dense probe output and
 *                                        lse per chunk of key blocks,
 *                                        K = min(8, nb)
 *              bf16 [B,H,Mp,d]           gathered probe queries
 *              fp32 [B,H,2,d,8]          Z = (Xc^T Xc + lambda I)^{-1} Xc^T Rc V_r
 *                                        and V_r (columns >= rank zero), the
 *                                        factors W = Z V_r^T is applied by
 *              fp16 [B,H,N_pad,d]        fp16 copy of v (the dense probes'
 *                                        value operand)
 */
size_t sparse_attn_residual_workspace(const sa_shape* shape);
sa_status sparse_attn_residual(const sa_shape* shape, sa_dtype dtype, float scale,
                               const void* q, const void* k, const void* v, void* out,
                               int32_t phase, float ridge, int32_t rank,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static text for a status code. */
const char* sparse_attn_status_string(sa_status status);
/* Detail of the calling thread's last failure ("" if none). */
const char* sparse_attn_last_error(void);
/* SPARSE_ATTN_ABI_VERSION of the loaded library. */
int32_t sparse_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
