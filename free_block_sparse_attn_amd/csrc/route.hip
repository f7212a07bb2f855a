// Block routing kernels: pooled-score top-k, Triage tiers, LVSA mask.
//
// Scores follow one arithmetic contract so the selection is reproducible bit
// for bit: s(a, j) = sum_i qbar[a,i] * kbar[j,i] with fp64 fused multiply-adds
// in i order (the fp32 x fp32 products are exact in fp64, so the fusion does
// not change a bit).  A selection takes the first k elements of the total
// order (-key, j): keys are mapped to order-preserving 64-bit integers and a
// wave finds the k-th key bit by bit with ballots over keys held in registers;
// ties at that key go to the lowest block indices.  Lists are
// written ascending by ballot compaction.
//
// Page basis: PISA's top-k critical set per query block ("PISA: Piecewise
// Sparse Attention Is Wiser for Efficient Diffusion Transformers", section 2,
// "Algorithme Central"); Triage's router choosing skip / skim / refine from
// block statistics ("Triage: Skip, Skim, or Refine Attention Tiles in Video
// Diffusion Transformers", "Un routage fonde sur l'erreur estimee"); LVSA's
// A(t) = G_s U W(t) ("LVSA: Training-Free Sparse Attention for Long Video
// Diffusion", section 2, "Mecanisme Central").
#include "common.h"
#include "launch.h"

namespace sa {

namespace {

constexpr int THREADS = 256;
constexpr int WAVES = THREADS / 64;

__device__ __forceinline__ uint64_t order_key(double s) {
    if (s == 0.0) s = 0.0;                                  // -0 sorts as +0
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(s));
    return (b >> 63) ? ~b : (b | (1ull << 63));
}

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct Threshold {
    uint64_t key;     // the k-th key in the order (-key, j)
    int need;         // how many elements equal to `key` are taken (lowest j first)
};

__device__ __forceinline__ uint64_t wave_and64(uint64_t x) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x &= static_cast<uint64_t>(__shfl_xor(static_cast<long long>(x), off));
    return x;
}
__device__ __forceinline__ uint64_t wave_or64(uint64_t x) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x |= static_cast<uint64_t>(__shfl_xor(static_cast<long long>(x), off));
    return x;
}

// k-th largest key among candidates (key != 0 when `cand_nonzero`), k >= 1,
// k <= number of candidates.  One wave; lane l holds keys l + 64 t (t < KPL)
// in registers.  The threshold is found bit by bit from the highest bit in
// which the candidates differ: bit b is set when at least k keys are >= the
// threshold with it set (one 64-bit compare and one ballot per key and bit,
// no LDS traffic).  The search ends at the first bit where exactly k keys
// are >= the candidate; it returns {candidate - 1, 0} then, which selects
// the same keys.  Real keys are never 0 (order_key of a non-NaN value), so
// 0 marks missing entries.
template <int KPL, typename KeyOf>
__device__ Threshold threshold_select(KeyOf keys, int nb, int k, bool cand_nonzero) {
    const int lane = lane_id();
    uint64_t kr[KPL];
    uint64_t kand = ~0ull, kor = 0ull;
#pragma unroll
    for (int t = 0; t < KPL; ++t) {
        const int j = lane + 64 * t;
        uint64_t key = j < nb ? keys(j) : 0ull;
        if (!cand_nonzero && j < nb) { kand &= key; kor |= key; }
        if (cand_nonzero && key != 0ull) { kand &= key; kor |= key; }
        kr[t] = key;
    }
    kand = wave_and64(kand);
    kor = wave_or64(kor);
    const uint64_t diff = kand ^ kor;                 // bits in which candidates differ
    const int top = diff ? 63 - __builtin_clzll(diff) : -1;
    // the bits above `top` are common to every candidate; lower bits start at 0
    uint64_t T = top < 0 ? kand : (top == 63 ? 0ull : (kand & ~((2ull << top) - 1ull)));
    for (int b = top; b >= 0; --b) {
        const uint64_t cand = T | (1ull << b);
        int c = 0;
#pragma unroll
        for (int t = 0; t < KPL; ++t) c += __popcll(__ballot(kr[t] >= cand));
        // exactly k keys at or above cand: they are the selection (the k-th
        // and (k+1)-th keys first differ in bit b), whatever the lower bits
        if (c == k) return Threshold{cand - 1ull, 0};
        if (c > k) T = cand;
    }
    int gt = 0;
#pragma unroll
    for (int t = 0; t < KPL; ++t) gt += __popcll(__ballot(kr[t] > T));
    return Threshold{T, k - gt};
}

// The same search for long rows, forming the keys again at every bit.
template <typename KeyOf>
__device__ Threshold threshold_select_lds(KeyOf keys, int nb, int k, bool cand_nonzero) {
    const int lane = lane_id();
    uint64_t kand = ~0ull, kor = 0ull;
    for (int j = lane; j < nb; j += 64) {
        const uint64_t key = keys(j);
        if (!cand_nonzero || key != 0ull) { kand &= key; kor |= key; }
    }
    kand = wave_and64(kand);
    kor = wave_or64(kor);
    const uint64_t diff = kand ^ kor;
    const int top = diff ? 63 - __builtin_clzll(diff) : -1;
    uint64_t T = top < 0 ? kand : (top == 63 ? 0ull : (kand & ~((2ull << top) - 1ull)));
    for (int b = top; b >= 0; --b) {
        const uint64_t cand = T | (1ull << b);
        int c = 0;
        for (int j0 = 0; j0 < nb; j0 += 64) {
            const int j = j0 + lane;
            c += __popcll(__ballot(j < nb && keys(j) >= cand));
        }
        if (c == k) return Threshold{cand - 1ull, 0};   // as in threshold_select
        if (c > k) T = cand;
    }
    int gt = 0;
    for (int j0 = 0; j0 < nb; j0 += 64) {
        const int j = j0 + lane;
        gt += __popcll(__ballot(j < nb && keys(j) > T));
    }
    return Threshold{T, k - gt};
}

template <typename KeyOf>
__device__ __forceinline__ Threshold select_kth(KeyOf keys, int nb, int k, bool cand_nonzero) {
    const int kpl = (nb + 63) / 64;
    if (kpl <= 2) return threshold_select<2>(keys, nb, k, cand_nonzero);
    if (kpl <= 4) return threshold_select<4>(keys, nb, k, cand_nonzero);
    if (kpl <= 8) return threshold_select<8>(keys, nb, k, cand_nonzero);
    if (kpl <= 16) return threshold_select<16>(keys, nb, k, cand_nonzero);
    if (kpl <= 32) return threshold_select<32>(keys, nb, k, cand_nonzero);
    return threshold_select_lds(keys, nb, k, cand_nonzero);
}

// Writes the selected indices ascending into out[0..cap), -1 after, returns the count.
// `excl` (optional): a second threshold whose selected elements are excluded.
__device__ int compact_selection(const uint64_t* keys, int nb, Threshold t, bool cand_nonzero,
                                 int32_t* out, int cap, bool none) {
    const int lane = lane_id();
    const uint64_t lt = (1ull << lane) - 1ull;
    int base = 0, eqseen = 0;
    for (int j0 = 0; j0 < nb; j0 += 64) {
        const int j = j0 + lane;
        const uint64_t key = (j < nb) ? keys[j] : 0ull;
        const bool cand = (j < nb) && (!cand_nonzero || key != 0ull) && !none;
        const bool gt = cand && key > t.key;
        const bool eq = cand && key == t.key;
        const uint64_t eqm = __ballot(eq);
        const int eqrank = eqseen + __popcll(eqm & lt);
        const bool sel = gt || (eq && eqrank < t.need);
        const uint64_t selm = __ballot(sel);
        const int pos = base + __popcll(selm & lt);
        if (sel && pos < cap) out[pos] = j;
        base += __popcll(selm);
        eqseen += __popcll(eqm);
    }
    for (int p = base + lane; p < cap; p += 64) out[p] = -1;
    return base;
}

// fp64 scores of R query blocks against all key blocks, row-major in LDS as keys.
template <int R>
__device__ void score_rows(const RouteArgs& a, size_t bh, int row0, double* qs, uint64_t* keyE, int nbp) {
    const int d = a.d, nb = a.nb, tid = threadIdx.x;
    for (int x = tid; x < R * d; x += THREADS) {
        const int r = x / d, i = x % d;
        const int row = row0 + r;
        qs[x] = (row < nb) ? static_cast<double>(a.qbar[(bh * nb + row) * d + i]) : 0.0;
    }
    __syncthreads();
    const bool triage = a.mode == 2, cov = a.mode == 3, err = a.mode == 4;
    const double sc = static_cast<double>(a.scale);
    for (int j = tid; j < nb; j += THREADS) {
        double acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.0;
        const float4* kr = reinterpret_cast<const float4*>(a.kbar + (bh * nb + j) * d);
        for (int i4 = 0; i4 < d / 4; ++i4) {
            const float4 kv = kr[i4];
            const double kd[4] = {static_cast<double>(kv.x), static_cast<double>(kv.y),
                                  static_cast<double>(kv.z), static_cast<double>(kv.w)};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
#pragma unroll
                for (int r = 0; r < R; ++r) acc[r] = fma(qs[r * d + 4 * i4 + u], kd[u], acc[r]);
            }
        }
        if (err) {
            // ln(E / n_j) = 2 scale s + L - ln n_j; the R error logs of key block j are contiguous
            const float* el = a.ekey + (bh * nb + j) * static_cast<size_t>(nb) + row0;
            const double lgn = log(static_cast<double>(a.kcount[j]));
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const double L = (row0 + r < nb) ? static_cast<double>(el[r]) : 0.0;
                keyE[r * nbp + j] = order_key(__dadd_rn(__dadd_rn(2.0 * __dmul_rn(sc, acc[r]), L), -lgn));
            }
        } else if (cov) {
            const double lm = static_cast<double>(a.klam[bh * nb + j]);
#pragma unroll
            for (int r = 0; r < R; ++r) keyE[r * nbp + j] = order_key(__dadd_rn(__dmul_rn(sc, acc[r]), lm));
        } else if (!triage) {
#pragma unroll
            for (int r = 0; r < R; ++r) keyE[r * nbp + j] = order_key(acc[r]);
        } else {
            // Triage: the scaled score itself; both tier keys are formed from
            // it during the selection (one LDS array per row instead of two)
#pragma unroll
            for (int r = 0; r < R; ++r)
                keyE[r * nbp + j] = static_cast<uint64_t>(__double_as_longlong(__dmul_rn(sc, acc[r])));
        }
    }
    __syncthreads();
}

template <int R>
__global__ __launch_bounds__(THREADS) void route_scored_kernel(RouteArgs a) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int nbp = (a.nb + 63) & ~63;
    const bool triage = a.mode == 2;
    double* qs = reinterpret_cast<double*>(smem);                            // R * d
    uint64_t* keyE = reinterpret_cast<uint64_t*>(qs + R * a.d);              // R * nbp

    const int row0 = blockIdx.x * R;
    const size_t bh = static_cast<size_t>(blockIdx.z) * a.H + blockIdx.y;
    score_rows<R>(a, bh, row0, qs, keyE, nbp);

    const int w = threadIdx.x >> 6;
    for (int r = w; r < R; r += WAVES) {
        const int row = row0 + r;
        if (row >= a.nb) break;
        const size_t rowid = bh * a.nb + row;
        uint64_t* kE = keyE + r * nbp;
        const auto from_lds = [kE](int j) { return kE[j]; };
        if (!triage) {
            const Threshold t = select_kth(from_lds, a.nb, a.topk, false);
            const int c = compact_selection(kE, a.nb, t, false, a.idx + rowid * a.cap, a.cap, false);
            if (lane_id() == 0) a.cnt[rowid] = c;
        } else {
            // kE holds the scaled scores ss; e_skip = fl(ss + lambda_j),
            // w = fl(ss + ln n_j) (n_j = 64 except for the last block)
            const float* lam = a.klam + bh * a.nb;
            const double lgn64 = log(64.0);
            const double lgnl = log(static_cast<double>(a.kcount[a.nb - 1]));
            const auto eskip = [kE, lam](int j) {
                return order_key(__dadd_rn(__longlong_as_double(static_cast<long long>(kE[j])),
                                           static_cast<double>(lam[j])));
            };
            // kept = first n_keep by e_skip; then kE[j] becomes the w-key of a
            // kept block and 0 for the others
            const Threshold tk = select_kth(eskip, a.nb, a.n_keep, false);
            {
                const int lane = lane_id();
                const uint64_t lt = (1ull << lane) - 1ull;
                int eqseen = 0;
                for (int j0 = 0; j0 < a.nb; j0 += 64) {
                    const int j = j0 + lane;
                    const uint64_t key = (j < a.nb) ? eskip(j) : 0ull;
                    const bool eq = (j < a.nb) && key == tk.key;
                    const uint64_t eqm = __ballot(eq);
                    const int eqrank = eqseen + __popcll(eqm & lt);
                    const bool kept = (j < a.nb) && (key > tk.key || (eq && eqrank < tk.need));
                    if (j < a.nb) {
                        const double ss = __longlong_as_double(static_cast<long long>(kE[j]));
                        kE[j] = kept ? order_key(__dadd_rn(ss, j == a.nb - 1 ? lgnl : lgn64)) : 0ull;
                    }
                    eqseen += __popcll(eqm);
                }
                wave_sync();
            }
            uint64_t* kW = kE;
            const auto wkey = [kW](int j) { return kW[j]; };
            // refine = first n_refine of the kept blocks by w
            const bool none = a.n_refine == 0;
            Threshold tr{~0ull, 0};
            if (!none) tr = select_kth(wkey, a.nb, a.n_refine, true);
            const int c1 = compact_selection(kW, a.nb, tr, true, a.idx + rowid * a.cap, a.cap, none);
            // skim = kept and not refine: blank the refine keys, take every remaining candidate
            {
                const int lane = lane_id();
                const uint64_t lt = (1ull << lane) - 1ull;
                int eqseen = 0;
                for (int j0 = 0; j0 < a.nb; j0 += 64) {
                    const int j = j0 + lane;
                    const uint64_t key = (j < a.nb) ? kW[j] : 0ull;
                    const bool cand = (j < a.nb) && key != 0ull && !none;
                    const bool eq = cand && key == tr.key;
                    const uint64_t eqm = __ballot(eq);
                    const int eqrank = eqseen + __popcll(eqm & lt);
                    const bool ref = cand && (key > tr.key || (eq && eqrank < tr.need));
                    if (ref) kW[j] = 0ull;
                    eqseen += __popcll(eqm);
                }
                wave_sync();
            }
            const Threshold all{1ull, 0};             // every candidate has key > 1
            const int c2 = compact_selection(kW, a.nb, all, true, a.idx2 + rowid * a.cap2, a.cap2, false);
            if (lane_id() == 0) { a.cnt[rowid] = c1; a.cnt2[rowid] = c2; }
        }
        wave_sync();
    }
}

// LVSA: the mask depends only on the frame ranges, the anchors and the step,
// so every (b, h) gets the same lists.  One wave per query block scans the
// key blocks from LDS copies of the frame ranges and an anchor bitmap and
// writes its list for every (b, h).  Pure integer work.
constexpr int LVSA_ROWS = 4;      // query blocks per workgroup (one per wave)

__global__ __launch_bounds__(64 * LVSA_ROWS) void route_lvsa_kernel(RouteArgs a) {
    __shared__ int32_t flo[4096], fhi[4096];
    __shared__ uint32_t anchor_bits[128];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int nb = a.nb;
    for (int j = tid; j < nb; j += 64 * LVSA_ROWS) {
        flo[j] = a.frame_lo[j];
        fhi[j] = a.frame_hi[j];
    }
    for (int x = tid; x < 128; x += 64 * LVSA_ROWS) anchor_bits[x] = 0u;
    __syncthreads();
    const int P = a.anchors > 0 ? nb / a.anchors : 0;
    if (P > 0) {
        for (int i = tid; i < a.anchors; i += 64 * LVSA_ROWS) {
            const int j = (a.anchor_phase + a.step) % P + i * P;    // < anchors * P <= nb
            atomicOr(&anchor_bits[j >> 5], 1u << (j & 31));
        }
    }
    __syncthreads();
    const int row = blockIdx.x * LVSA_ROWS + w;
    if (row >= nb) return;
    const uint64_t lt = (1ull << lane) - 1ull;
    const int lo = flo[row] - a.window, hi = fhi[row] + a.window;
    const int BH = a.B * a.H;
    int base = 0;
    for (int j0 = 0; j0 < nb; j0 += 64) {
        const int j = j0 + lane;
        bool sel = false;
        if (j < nb) sel = (flo[j] <= hi && fhi[j] >= lo) || ((anchor_bits[j >> 5] >> (j & 31)) & 1u);
        const uint64_t m = __ballot(sel);
        const int pos = base + __popcll(m & lt);
        if (sel && pos < a.cap)
            for (int bh = 0; bh < BH; ++bh) a.idx[(static_cast<size_t>(bh) * nb + row) * a.cap + pos] = j;
        base += __popcll(m);
    }
    for (int p = base + lane; p < a.cap; p += 64)
        for (int bh = 0; bh < BH; ++bh) a.idx[(static_cast<size_t>(bh) * nb + row) * a.cap + p] = -1;
    if (lane == 0)
        for (int bh = 0; bh < BH; ++bh) a.cnt[static_cast<size_t>(bh) * nb + row] = base;
}

// SVG-EAR error estimate ("SVG-EAR: Parameter-Free Linear Compensation for
// Sparse Video Generation via Error-aware Routing", section 2B): for every
// query-block centroid a (the proxy of its queries) and key block j,
//   L(a, j) = ln sum_n expm1(delta_n)^2,  delta_n = scale qbar_a . (k_n - kbar_j),
// the log of the squared error of the proxy's attention weights when the
// block's keys are replaced by their centroid, without the factor e^{2c}
// (c = scale qbar_a . kbar_j) that the selection adds from the fp64 score.
// Streaming: a workgroup holds 64 centroids and walks ERR_CHUNK key blocks;
// the logits never leave the chip.  Each key block is centred in fp32 and
// staged in LDS as bf16 high + low parts, the centroids sit in registers as
// high + low MFMA operands, and delta = (kc_hi + kc_lo) . (q_hi + q_lo) less
// the lo.lo term (three MFMA passes, about 16 bits per factor).  Wave w takes
// key half w / 2 and centroid half w % 2 of the 64 x 64 tile.  Sums use a
// per-lane max shift, sum expm1(delta)^2 = e^{2m} sum (expm1(delta) e^{-m})^2,
// so no term overflows.
constexpr int ERR_CHUNK = 64;          // key blocks per workgroup
constexpr int ERR_PITCH = 128 + 8;     // staged key row pitch (bf16), 16-byte multiple

__device__ __forceinline__ void lse2_combine(float& m, float& s, float mo, float so) {
    // (m, s) represents e^{2m} s
    const float mn = fmaxf(m, mo);
    s = s * __expf(2.0f * (m - mn)) + so * __expf(2.0f * (mo - mn));
    m = mn;
}

__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(3, 3))) void route_err_kernel(RouteArgs a) {
    constexpr int D = 128;
    __shared__ __attribute__((aligned(16))) uint16_t khi[BLK * ERR_PITCH], klo[BLK * ERR_PITCH];
    __shared__ float xch[2][2][2][32];    // [parity][centroid half][m, s][lane]
    const int nb = a.nb;
    const int nct = (nb + BLK - 1) / BLK;
    const int ct = blockIdx.x % nct, ch = blockIdx.x / nct;
    const size_t bh = static_cast<size_t>(blockIdx.z) * a.H + blockIdx.y;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, hl = l >> 5, l32 = l & 31;
    const int kw = w >> 1, cw = w & 1;
    const int j0 = ch * ERR_CHUNK, j1 = min(nb, j0 + ERR_CHUNK);
    const float sc = a.scale;
    // centroid operands: B[k = d][n = centroid], lane holds d = 16 ks + 8 hl .. + 7 of centroid l32
    bf16x8 qh[8], ql[8];
    {
        const int c = BLK * ct + 32 * cw + l32;
        const float* qr = a.qbar + (bh * nb + min(c, nb - 1)) * D;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(qr + 16 * ks + 8 * hl);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(qr + 16 * ks + 8 * hl + 4);
            const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = c < nb ? x[e] : 0.0f;
                const __bf16 h = static_cast<__bf16>(v);
                qh[ks][e] = h;
                ql[ks][e] = static_cast<__bf16>(v - static_cast<float>(h));
            }
        }
    }
    // staging: chunk p of thread t covers key row (t + 256 p) / 16, columns 8 ((t + 256 p) % 16) .. + 7
    const uint16_t* K = static_cast<const uint16_t*>(a.keys) + bh * static_cast<size_t>(nb) * BLK * D;
    u32x4 kreg[4];
    auto load_block = [&](int j) __attribute__((always_inline)) {
        const int n = min(BLK, a.N - BLK * j);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int chunk = tid + THREADS * p, row = chunk >> 4, col0 = (chunk & 15) * 8;
            u32x4 z = {0u, 0u, 0u, 0u};
            if (row < n) z = *reinterpret_cast<const u32x4*>(K + (static_cast<size_t>(j) * BLK + row) * D + col0);
            kreg[p] = z;
        }
    };
    auto stage_block = [&](int j) __attribute__((always_inline)) {
        const int n = min(BLK, a.N - BLK * j);
        const float* kb = a.kbar + (bh * nb + j) * D;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int chunk = tid + THREADS * p, row = chunk >> 4, col0 = (chunk & 15) * 8;
            const f32x4 m0 = *reinterpret_cast<const f32x4*>(kb + col0);
            const f32x4 m1 = *reinterpret_cast<const f32x4*>(kb + col0 + 4);
            const float mb[8] = {m0[0], m0[1], m0[2], m0[3], m1[0], m1[1], m1[2], m1[3]};
            u32x4 hi, lo;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                float c[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int e = 2 * e2 + t;
                    const uint32_t wd = kreg[p][e2];
                    const float kv = __uint_as_float(t ? (wd & 0xFFFF0000u) : (wd << 16));
                    c[t] = row < n ? kv - mb[e] : 0.0f;           // pad keys contribute delta = 0
                }
                hi[e2] = pack_bf16x2(c[0], c[1]);
                lo[e2] = pack_bf16x2(c[0] - bf16_to_f32(static_cast<uint16_t>(hi[e2] & 0xFFFFu)),
                                     c[1] - bf16_to_f32(static_cast<uint16_t>(hi[e2] >> 16)));
            }
            *reinterpret_cast<u32x4*>(khi + row * ERR_PITCH + col0) = hi;
            *reinterpret_cast<u32x4*>(klo + row * ERR_PITCH + col0) = lo;
        }
    };
    float pm = 0.0f, ps = 0.0f;             // wave kw = 0: this lane's (m, s) of the previous block
    auto finish = [&](int j, int par) __attribute__((always_inline)) {
        // wave kw = 0, lanes 0..31: combine with the other key half, write L(a, j)
        if (kw == 0 && hl == 0) {
            float m = pm, s = ps;
            lse2_combine(m, s, xch[par][cw][0][l32], xch[par][cw][1][l32]);
            const int c = BLK * ct + 32 * cw + l32;
            if (c < nb) a.ekey[(bh * nb + j) * static_cast<size_t>(nb) + c] = s > 0.0f ? 2.0f * m + __logf(s) : -INFINITY;
        }
    };
    if (j0 < j1) load_block(j0);
    for (int j = j0; j < j1; ++j) {
        __syncthreads();                      // the previous block's operands are read; xch of j - 1 visible
        if (j > j0) finish(j - 1, (j - 1) & 1);
        stage_block(j);
        if (j + 1 < j1) load_block(j + 1);
        __syncthreads();
        f32x16 acc = f32x16{};
        const uint16_t* ah = khi + (32 * kw + l32) * ERR_PITCH + 8 * hl;
        const uint16_t* al = klo + (32 * kw + l32) * ERR_PITCH + 8 * hl;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const bf16x8 xh = *reinterpret_cast<const bf16x8*>(ah + 16 * ks);
            const bf16x8 xl = *reinterpret_cast<const bf16x8*>(al + 16 * ks);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, qh[ks], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, ql[ks], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xl, qh[ks], acc, 0, 0, 0);
        }
        // this lane: 16 keys of the half for centroid l32
        float dl[16];
        float m = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dl[r] = sc * acc[r];
            m = fmaxf(m, dl[r]);
        }
        // t = expm1(delta) e^{-m}: expm1 keeps small deviations exact when m
        // is small; for m > 1 the form e^{delta - m} - e^{-m} cannot overflow
        // One exponential per value (the lane's m picks the form): e^{delta - m}
        // when m > 1; otherwise e^delta, or for |delta| < 0.5 the Taylor series
        // of expm1 up to delta^7 (first omitted term below 2.5e-7 of the result).
        const float em = __expf(-m);
        const bool big = m > 1.0f;
        const float shift = big ? m : 0.0f;
        float s = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float x = dl[r];
            const float e = __expf(x - shift);
            float p = fmaf(x, 1.0f / 5040.0f, 1.0f / 720.0f);
            p = fmaf(x, p, 1.0f / 120.0f);
            p = fmaf(x, p, 1.0f / 24.0f);
            p = fmaf(x, p, 1.0f / 6.0f);
            p = fmaf(x, p, 0.5f);
            p = fmaf(x, p, 1.0f);
            const float em1 = fabsf(x) < 0.5f ? x * p : e - 1.0f;
            const float t = big ? e - em : em1 * em;
            s = fmaf(t, t, s);
        }
        // the other 16 keys of the half sit in lane l ^ 32
        {
            const auto pmv = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
            const auto psv = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
            const float mo = __uint_as_float(hl ? static_cast<uint32_t>(pmv[0]) : static_cast<uint32_t>(pmv[1]));
            const float so = __uint_as_float(hl ? static_cast<uint32_t>(psv[0]) : static_cast<uint32_t>(psv[1]));
            lse2_combine(m, s, mo, so);
        }
        if (kw == 1 && hl == 0) {
            xch[j & 1][cw][0][l32] = m;
            xch[j & 1][cw][1][l32] = s;
        }
        pm = m;
        ps = s;
    }
    if (j0 < j1) {
        __syncthreads();
        finish(j1 - 1, (j1 - 1) & 1);
    }
}

// ---- scores on the fp64 matrix cores (d = 64 or 128, nb <= 2048) ----
//
// v_mfma_f64_16x16x4_f64 adds its four products to the accumulator one fused
// multiply-add at a time, in k order, so a chain of them over k = 0, 4, 8, ...
// gives the same bits as the sequential fp64 FMA contract above (the operands
// are fp32 values, whose products fp64 holds exactly).  A workgroup takes 16
// query blocks, the MFMA's N, and walks the key blocks 16 at a time, its M: in
// round p wave w scores key tile 8p + w against the 16 rows, and the tiles go
// through LDS to the waves that own the rows (wave w owns rows w and w + 8).
// Those waves keep their rows' keys in registers, lane l holding key blocks
// l + 64 t, so 16 rows need no LDS key arrays and the selection makes no LDS
// traffic.  Key 0 marks a missing entry (no real key is 0).
typedef __attribute__((ext_vector_type(4))) double f64x4;
constexpr int MROWS = 16;          // query blocks per workgroup (the MFMA's N)
constexpr int MWAVES = 8;

// Threshold search of threshold_select on keys already in registers; the
// candidates are the nonzero keys (slots past nb hold 0, which no compare
// against a candidate >= 1 counts, so every slot takes part).
template <int KPL>
__device__ __forceinline__ Threshold threshold_regs(const uint64_t (&kr)[KPL], int k) {
    uint64_t kand = ~0ull, kor = 0ull;
#pragma unroll
    for (int t = 0; t < KPL; ++t)
        if (kr[t] != 0ull) { kand &= kr[t]; kor |= kr[t]; }
    kand = wave_and64(kand);
    kor = wave_or64(kor);
    const uint64_t diff = kand ^ kor;
    const int top = diff ? 63 - __builtin_clzll(diff) : -1;
    uint64_t T = top < 0 ? kand : (top == 63 ? 0ull : (kand & ~((2ull << top) - 1ull)));
    for (int b = top; b >= 0; --b) {
        const uint64_t cand = T | (1ull << b);
        int c = 0;
#pragma unroll
        for (int t = 0; t < KPL; ++t) c += __popcll(__ballot(kr[t] >= cand));
        if (c == k) return Threshold{cand - 1ull, 0};
        if (c > k) T = cand;
    }
    int gt = 0;
#pragma unroll
    for (int t = 0; t < KPL; ++t) gt += __popcll(__ballot(kr[t] > T));
    return Threshold{T, k - gt};
}

// compact_selection over register keys (slot t covers blocks 64 t .. 64 t + 63)
template <int KPL>
__device__ __forceinline__ int compact_regs(const uint64_t (&kr)[KPL], Threshold t, int32_t* out, int cap, bool none) {
    const int lane = lane_id();
    const uint64_t lt = (1ull << lane) - 1ull;
    int base = 0, eqseen = 0;
#pragma unroll
    for (int s = 0; s < KPL; ++s) {
        const uint64_t key = kr[s];
        const bool cand = key != 0ull && !none;
        const bool gt = cand && key > t.key;
        const bool eq = cand && key == t.key;
        const uint64_t eqm = __ballot(eq);
        const int eqrank = eqseen + __popcll(eqm & lt);
        const bool sel = gt || (eq && eqrank < t.need);
        const uint64_t selm = __ballot(sel);
        const int pos = base + __popcll(selm & lt);
        if (sel && pos < cap) out[pos] = 64 * s + lane;
        base += __popcll(selm);
        eqseen += __popcll(eqm);
    }
    for (int p = base + lane; p < cap; p += 64) out[p] = -1;
    return base;
}

// The selection of one row from its register keys: top-k modes take kr as
// the order keys (0 past nb); Triage takes kr as the scaled scores ss.
template <int KPL, int MODE>
__device__ __forceinline__ void select_row(const RouteArgs& a, size_t bh, int row, const uint64_t (&kr)[KPL]) {
    const int nb = a.nb, lane = lane_id();
    const size_t rowid = bh * nb + row;
    if constexpr (MODE != 2) {
        const Threshold t = threshold_regs(kr, a.topk);
        const int c = compact_regs(kr, t, a.idx + rowid * a.cap, a.cap, false);
        if (lane == 0) a.cnt[rowid] = c;
        return;
    }
    // Triage: kept = first n_keep by e_skip = fl(ss + lambda_j); of those,
    // refine = first n_refine by w = fl(ss + ln n_j); skim = kept, not refine
    const float* lam = a.klam + bh * nb;
    const double lgn64 = log(64.0);
    const double lgnl = log(static_cast<double>(a.kcount[nb - 1]));
    uint64_t ek[KPL];
#pragma unroll
    for (int s = 0; s < KPL; ++s) {
        const int j = 64 * s + lane;
        ek[s] = j < nb ? order_key(__dadd_rn(__longlong_as_double(static_cast<long long>(kr[s])), static_cast<double>(lam[j])))
                       : 0ull;
    }
    const Threshold tk = threshold_regs(ek, a.n_keep);
    {
        const uint64_t lt = (1ull << lane) - 1ull;
        int eqseen = 0;
#pragma unroll
        for (int s = 0; s < KPL; ++s) {
            const int j = 64 * s + lane;
            const uint64_t key = ek[s];
            const bool eq = key != 0ull && key == tk.key;
            const uint64_t eqm = __ballot(eq);
            const int eqrank = eqseen + __popcll(eqm & lt);
            const bool kept = key != 0ull && (key > tk.key || (eq && eqrank < tk.need));
            const double ss = __longlong_as_double(static_cast<long long>(kr[s]));
            ek[s] = kept ? order_key(__dadd_rn(ss, j == nb - 1 ? lgnl : lgn64)) : 0ull;
            eqseen += __popcll(eqm);
        }
    }
    const bool none = a.n_refine == 0;
    Threshold tr{~0ull, 0};
    if (!none) tr = threshold_regs(ek, a.n_refine);
    const int c1 = compact_regs(ek, tr, a.idx + rowid * a.cap, a.cap, none);
    {
        const uint64_t lt = (1ull << lane) - 1ull;
        int eqseen = 0;
#pragma unroll
        for (int s = 0; s < KPL; ++s) {
            const uint64_t key = ek[s];
            const bool cand = key != 0ull && !none;
            const bool eq = cand && key == tr.key;
            const uint64_t eqm = __ballot(eq);
            const int eqrank = eqseen + __popcll(eqm & lt);
            const bool ref = cand && (key > tr.key || (eq && eqrank < tr.need));
            if (ref) ek[s] = 0ull;
            eqseen += __popcll(eqm);
        }
    }
    const Threshold all{1ull, 0};
    const int c2 = compact_regs(ek, all, a.idx2 + rowid * a.cap2, a.cap2, false);
    if (lane == 0) { a.cnt[rowid] = c1; a.cnt2[rowid] = c2; }
}

template <int D, int KPL, int MODE>
__global__ __launch_bounds__(64 * MWAVES) void route_mfma_kernel(RouteArgs a) {
    constexpr int KP = D + 4;          // staged row pitch (floats)
    constexpr int NS = D / 4;          // MFMA steps
    constexpr int PL = D / 16;         // 16-byte loads per lane per 16-row tile
    constexpr int SP = MROWS + 1;      // score staging pitch (doubles)
    // scoring: key tiles kt[MWAVES][MROWS * KP] (fp32) and score tiles
    // st[2][MWAVES][MROWS * SP] (fp64); selection: row B's keys while row A
    // is selected, [MWAVES][KPL][64]
    constexpr int KT_BYTES = MWAVES * MROWS * KP * 4;
    constexpr int ST_BYTES = 2 * MWAVES * MROWS * SP * 8;
    constexpr int STASH_BYTES = MWAVES * KPL * 64 * 8;
    constexpr int LDS_BYTES = KT_BYTES + ST_BYTES > STASH_BYTES ? KT_BYTES + ST_BYTES : STASH_BYTES;
    __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
    float (*kt)[MROWS * KP] = reinterpret_cast<float (*)[MROWS * KP]>(lds);
    double (*st)[MWAVES][MROWS * SP] = reinterpret_cast<double (*)[MWAVES][MROWS * SP]>(lds + KT_BYTES);

    const int nb = a.nb;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int row0 = blockIdx.x * MROWS;
    const size_t bh = static_cast<size_t>(blockIdx.z) * a.H + blockIdx.y;
    const float* Kb = a.kbar + bh * nb * D;
    float* my = kt[w];
    const double sc = static_cast<double>(a.scale);

    // rows r0 .. r0 + 15 of a block-major [nb][D] array, zero past nb
    auto load16 = [&](const float* src, int r0, f32x4 (&buf)[PL]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < PL; ++u) {
            const int x = 64 * u + l, r = x / (D / 4), c4 = x % (D / 4);
            buf[u] = (r0 + r < nb) ? *reinterpret_cast<const f32x4*>(src + static_cast<size_t>(r0 + r) * D + 4 * c4)
                                   : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    };
    auto put16 = [&](const f32x4 (&buf)[PL]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < PL; ++u) {
            const int x = 64 * u + l, r = x / (D / 4), c4 = x % (D / 4);
            *reinterpret_cast<f32x4*>(my + r * KP + 4 * c4) = buf[u];
        }
    };
    // MFMA operand of step s for this lane: row l % 16, dimension 4 s + l / 16
    const int opo = (l & 15) * KP + (l >> 4);

    // B operands: the 16 query rows
    float qv[NS];
    f32x4 pre[PL];
    load16(a.qbar + bh * nb * D, row0, pre);
    put16(pre);
    wave_sync();
#pragma unroll
    for (int s = 0; s < NS; ++s) qv[s] = my[opo + 4 * s];
    wave_sync();

    const int rA = w, rB = w + MWAVES;
    uint64_t kA[KPL], kB[KPL];
    load16(Kb, MROWS * w, pre);
#pragma unroll
    for (int p = 0; p < KPL / 2; ++p) {
        kA[2 * p] = kA[2 * p + 1] = kB[2 * p] = kB[2 * p + 1] = 0ull;
        if (128 * p >= nb) continue;                       // uniform
        const int j0 = MROWS * (MWAVES * p + w);
        put16(pre);
        if (128 * (p + 1) < nb) load16(Kb, j0 + 128, pre);
        wave_sync();
        f64x4 acc = {0.0, 0.0, 0.0, 0.0};
        if (j0 < nb) {
#pragma unroll
            for (int s = 0; s < NS; ++s)
                acc = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(my[opo + 4 * s]),
                                                           static_cast<double>(qv[s]), acc, 0, 0, 0);
        }
        // accumulator entry i: key j0 + 4 i + l / 16, query row l % 16
        double* sp = st[p & 1][w];
#pragma unroll
        for (int i = 0; i < 4; ++i) sp[(l & 15) * SP + 4 * i + (l >> 4)] = acc[i];
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int c = 64 * u + l, j = 128 * p + c;
            if (j >= nb) continue;
            const double* sq = st[p & 1][c >> 4];
            const double vA = sq[rA * SP + (c & 15)], vB = sq[rB * SP + (c & 15)];
            uint64_t xA, xB;
            if constexpr (MODE == 2) {
                xA = static_cast<uint64_t>(__double_as_longlong(__dmul_rn(sc, vA)));
                xB = static_cast<uint64_t>(__double_as_longlong(__dmul_rn(sc, vB)));
            } else if constexpr (MODE == 3) {
                const double lm = static_cast<double>(a.klam[bh * nb + j]);
                xA = order_key(__dadd_rn(__dmul_rn(sc, vA), lm));
                xB = order_key(__dadd_rn(__dmul_rn(sc, vB), lm));
            } else if constexpr (MODE == 4) {
                // ln(E / n_j) = 2 scale s + L - ln n_j
                const double lgn = log(static_cast<double>(a.kcount[j]));
                const float* el = a.ekey + (bh * nb + j) * static_cast<size_t>(nb);
                const double LA = row0 + rA < nb ? static_cast<double>(el[row0 + rA]) : 0.0;
                const double LB = row0 + rB < nb ? static_cast<double>(el[row0 + rB]) : 0.0;
                xA = order_key(__dadd_rn(__dadd_rn(2.0 * __dmul_rn(sc, vA), LA), -lgn));
                xB = order_key(__dadd_rn(__dadd_rn(2.0 * __dmul_rn(sc, vB), LB), -lgn));
            } else {
                xA = order_key(vA);
                xB = order_key(vB);
            }
            kA[2 * p + u] = xA;
            kB[2 * p + u] = xB;
        }
    }
    // row B's keys wait in LDS (the tiles are no longer read) while row A is
    // selected; one copy of the selection code serves both rows
    __syncthreads();
    uint64_t* stash = reinterpret_cast<uint64_t*>(lds) + w * KPL * 64 + l;
#pragma unroll
    for (int t = 0; t < KPL; ++t) stash[64 * t] = kB[t];
#pragma unroll 1
    for (int rr = 0; rr < 2; ++rr) {
        if (rr == 1) {
            wave_sync();
#pragma unroll
            for (int t = 0; t < KPL; ++t) kA[t] = stash[64 * t];
        }
        const int row = row0 + w + MWAVES * rr;
        if (row < nb) select_row<KPL, MODE>(a, bh, row, kA);
    }
}

template <int D, int MODE>
hipError_t launch_mfma(const RouteArgs& a, hipStream_t s) {
    dim3 grid((a.nb + MROWS - 1) / MROWS, a.H, a.B);
    if (a.nb <= 512) hipLaunchKernelGGL((route_mfma_kernel<D, 8, MODE>), grid, dim3(64 * MWAVES), 0, s, a);
    else if (a.nb <= 1024) hipLaunchKernelGGL((route_mfma_kernel<D, 16, MODE>), grid, dim3(64 * MWAVES), 0, s, a);
    else hipLaunchKernelGGL((route_mfma_kernel<D, 32, MODE>), grid, dim3(64 * MWAVES), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_mfma_modes(const RouteArgs& a, hipStream_t s) {
    switch (a.mode) {
        case 2: return launch_mfma<D, 2>(a, s);
        case 3: return launch_mfma<D, 3>(a, s);
        case 4: return launch_mfma<D, 4>(a, s);
        default: return launch_mfma<D, 0>(a, s);
    }
}

template <int R>
hipError_t launch_scored(const RouteArgs& a, hipStream_t s) {
    const int nbp = (a.nb + 63) & ~63;
    const size_t lds = R * a.d * sizeof(double) + R * nbp * sizeof(uint64_t);
    dim3 grid((a.nb + R - 1) / R, a.H, a.B);
    hipLaunchKernelGGL((route_scored_kernel<R>), grid, dim3(THREADS), lds, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
    if (a.mode == 4) {
        const int nct = (a.nb + BLK - 1) / BLK, nch = (a.nb + ERR_CHUNK - 1) / ERR_CHUNK;
        hipLaunchKernelGGL(route_err_kernel, dim3(nct * nch, a.H, a.B), dim3(THREADS), 0, s, a);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
    if (a.mode == 1) {
        dim3 grid((a.nb + LVSA_ROWS - 1) / LVSA_ROWS);
        hipLaunchKernelGGL(route_lvsa_kernel, grid, dim3(64 * LVSA_ROWS), 0, s, a);
        return hipGetLastError();
    }
    if ((a.d == 64 || a.d == 128) && a.nb <= 2048)
        return a.d == 128 ? launch_mfma_modes<128>(a, s) : launch_mfma_modes<64>(a, s);
    // rows per workgroup: as many as fit a 64 KiB key budget, at most 16, then
    // halved while the grid has fewer than 1024 workgroups (four per CU), so
    // that the waves' global k_bar loads overlap (Wan-size layer: 16 rows per
    // workgroup took 101 us, 4 rows 80 us)
    const int nbp = (a.nb + 63) & ~63;
    const size_t per_row = nbp * sizeof(uint64_t);
    const size_t budget = 64 * 1024;
    int R = 16;
    while (R > 1 && per_row * R > budget) R >>= 1;
    while (R > 1 && static_cast<long long>((a.nb + R - 1) / R) * a.H * a.B < 1024) R >>= 1;
    switch (R) {
        case 16: return launch_scored<16>(a, s);
        case 8: return launch_scored<8>(a, s);
        case 4: return launch_scored<4>(a, s);
        case 2: return launch_scored<2>(a, s);
        default: return launch_scored<1>(a, s);
    }
}

}  // namespace sa
