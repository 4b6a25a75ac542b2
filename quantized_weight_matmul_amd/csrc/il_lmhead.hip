// il_lmhead.hip -- centroid-masked LM head: the argmax token over a
// centroid-selected subset of the vocabulary (the end of `Drafter::step` on
// the oxinfer 0.0.1 src/drafter.rs page).  For each row x of a batch:
//   1. logits of the C centroids (bf16 rows) -- the decode GEMV of this
//      library, into scratch;
//   2. the k centroids of largest logit, visited by decreasing logit and,
//      among equal logits, increasing index (the page's select_nth_unstable
//      leaves both open; this is the reading taken);
//   3. the score embed[tok] . x of every token of those clusters
//      (token_ordering[c * per + j], per = V / C), and the first token of
//      largest score in visiting order (clusters in step-2 order, tokens in
//      j order), as the page's strict ">" scan picks it.  Ordering entries
//      >= V are skipped (never read, never chosen); a row whose candidates
//      are all skipped gets token -1.
// Launches after the GEMV: select_score_kernel on a grid of (k, rows) --
// every workgroup finds the row's top k (the k-th largest logit by a radix
// select over order-preserving 32-bit keys, a byte at a time from the top:
// an LDS histogram of the keys that still match, then the byte whose bin
// holds the k-th; then every logit above it and the lowest-index ties at it,
// placed by prefix sums; then a bitonic sort of those k into visiting
// order, in one wave's registers when k <= 64), takes its own cluster and
// scores its `per` tokens, each wave 16 at a time (their ordering entries,
// then their rows, fetched together; the 16 partial dots reduced by a
// transposed butterfly), keeping the first maximum -- then final_kernel,
// one wave per row, which takes the first maximum over the k clusters in
// visiting order.  The histogram counts are the only atomics and integer:
// results are deterministic.
#include "il_internal.h"

namespace il {
namespace {

constexpr int kSelThreads = 512;

// (a before b) in visiting order: larger logit first, equal logits by index.
__device__ __forceinline__ bool before(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// Order-preserving 32-bit key of a finite float (-0 counted as +0, so that
// equal keys are equal floats).
__device__ __forceinline__ uint32_t order_key(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct LmParams {  // (n_pow2: the next power of two >= k, the size of the final sort)
    const float *x;         // [t][h]
    const float *cl;        // [t][C] centroid logits
    const uint16_t *embed;  // bf16 [V][h]
    const uint32_t *ordering;
    float *part_score;      // [t][k]
    int *part_token;        // [t][k]
    int *clusters;          // [t][k] or null
    int h, n_c, n_pow2, per, k, vocab;
};

// v of the lane at `src` (wave-uniform).
__device__ __forceinline__ int read_lane(int v, int src) { return __builtin_amdgcn_readlane(v, src); }

__global__ __launch_bounds__(kSelThreads) void select_score_kernel(LmParams p) {
    constexpr int kWaves = kSelThreads / 64;
    extern __shared__ float4 smem4[];
    float *xs = reinterpret_cast<float *>(smem4);     // [h] this row of x (16-byte aligned)
    float *lv = xs + p.h;                             // [C] the row's logits
    float *sv = lv + p.n_c;                           // [n_pow2] logits of the chosen
    int *si = reinterpret_cast<int *>(sv + p.n_pow2);  // [n_pow2] their cluster ids
    __shared__ int hist[4][256];                         // one histogram per radix pass
    __shared__ uint32_t wsum[kWaves];
    __shared__ int chosen;                               // this workgroup's cluster
    __shared__ float wbest[kWaves];                      // per wave: best score, its token and j
    __shared__ int wtok[kWaves], wj[kWaves];

    const int i = blockIdx.x;    // rank of this workgroup's cluster in visiting order
    const int row = blockIdx.y;  // row of x
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float *cl = p.cl + (int64_t)row * p.n_c;
    for (int e = tid; e < p.n_c; e += kSelThreads) lv[e] = cl[e];
    for (int e = tid; e < p.h; e += kSelThreads) xs[e] = p.x[(int64_t)row * p.h + e];
    for (int e = tid; e < 4 * 256; e += kSelThreads) hist[e >> 8][e & 255] = 0;
    __syncthreads();

    // ---- the k-th largest key tau, a byte per pass from the top ----
    // Thread tid owns logits [tid * pt, tid * pt + pt): index order is thread
    // order, which the tie rule below relies on.  Invariant: tau is the
    // krem-th largest of the keys that match the bytes of tau found so far,
    // and 1 <= krem <= their number.  Every wave reads the pass's histogram
    // and finds the byte itself, so a pass needs one barrier.
    const int pt = (p.n_c + kSelThreads - 1) / kSelThreads;
    const int e0 = min(p.n_c, tid * pt), e1 = min(p.n_c, e0 + pt);
    uint32_t tau = 0u;
    int krem = p.k;
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int e = e0; e < e1; ++e) {
            const uint32_t kk = order_key(lv[e]);
            if (pass == 0 || (kk >> (shift + 8)) == (tau >> (shift + 8)))
                atomicAdd(&hist[pass][(kk >> shift) & 0xFFu], 1);
        }
        __syncthreads();
        // lane l holds bins 255 - 4l ... 252 - 4l (descending); the keys in
        // higher bins belong to the lanes below it (inclusive scan)
        int cnt[4], s4 = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) s4 += cnt[q] = hist[pass][255 - 4 * lane - q];
        int inc = s4;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(inc, off, 64);
            if (lane >= off) inc += o;
        }
        int above = inc - s4, dig = 0, kr = 0;
        bool found = false;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (above < krem && krem <= above + cnt[q]) found = true, dig = 255 - 4 * lane - q, kr = krem - above;
            above += cnt[q];
        }
        const int src = __builtin_ctzll(__ballot(found));  // exactly one lane finds it
        tau |= (uint32_t)read_lane(dig, src) << shift;
        krem = read_lane(kr, src);
    }
    // now #keys > tau < k <= #keys >= tau

    // ---- the chosen: every key > tau, then keys == tau by increasing index,
    // placed by a prefix sum of (count > tau) | (count == tau) << 16 ----
    int n_gt = 0, n_eq = 0;
    for (int e = e0; e < e1; ++e) {
        const uint32_t kk = order_key(lv[e]);
        n_gt += kk > tau;
        n_eq += kk == tau;
    }
    const uint32_t packed = (uint32_t)n_gt | ((uint32_t)n_eq << 16);  // both fields <= C < 2^16
    uint32_t inc = packed;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(inc, off, 64);
        if (lane >= off) inc += o;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    uint32_t base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        base += w < wave ? wsum[w] : 0;
        tot += wsum[w];
    }
    const uint32_t excl = base + inc - packed;
    const int tot_gt = (int)(tot & 0xFFFFu);
    int gpos = (int)(excl & 0xFFFFu), epos = (int)(excl >> 16);
    for (int e = e0; e < e1; ++e) {
        const uint32_t kk = order_key(lv[e]);
        if (kk > tau) {
            sv[gpos] = lv[e], si[gpos] = e, ++gpos;
        } else if (kk == tau) {
            if (tot_gt + epos < p.k) sv[tot_gt + epos] = lv[e], si[tot_gt + epos] = e;
            ++epos;
        }
    }
    for (int e = p.k + tid; e < p.n_pow2; e += kSelThreads) sv[e] = -INFINITY, si[e] = p.n_c + e;
    __syncthreads();

    // ---- bitonic sort of the chosen (logit, index) into visiting order ----
    if (p.n_pow2 <= 64) {
        // in one wave's registers, lane l holding element l
        if (wave == 0) {
            float v = lane < p.n_pow2 ? sv[lane] : -INFINITY;
            int ix = lane < p.n_pow2 ? si[lane] : p.n_c + lane;
            for (int size = 2; size <= p.n_pow2; size <<= 1) {
                for (int stride = size >> 1; stride > 0; stride >>= 1) {
                    const float ov = __shfl_xor(v, stride, 64);
                    const int oi = __shfl_xor(ix, stride, 64);
                    const bool want_first = ((lane & stride) == 0) == ((lane & size) == 0);
                    if (before(ov, oi, v, ix) == want_first) v = ov, ix = oi;
                }
            }
            if (lane == i) chosen = ix;
            if (i == 0 && p.clusters && lane < p.k) p.clusters[(int64_t)row * p.k + lane] = ix;
        }
    } else {
        // in LDS, a barrier per stage
        for (int size = 2; size <= p.n_pow2; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int e = tid; e < p.n_pow2 / 2; e += kSelThreads) {
                    const int lo = 2 * e - (e & (stride - 1));  // first of the pair (bit `stride` clear)
                    const int hi = lo + stride;
                    const bool asc = (lo & size) == 0;          // this run sorts into visiting order
                    const float va = sv[lo], vb = sv[hi];
                    const int ia = si[lo], ib = si[hi];
                    if (before(vb, ib, va, ia) == asc) {
                        sv[lo] = vb, sv[hi] = va;
                        si[lo] = ib, si[hi] = ia;
                    }
                }
                __syncthreads();
            }
        }
        if (tid == 0) chosen = si[i];
        if (i == 0 && p.clusters)
            for (int e = tid; e < p.k; e += kSelThreads) p.clusters[(int64_t)row * p.k + e] = si[e];
    }
    __syncthreads();
    // padding indices sort last for finite logits; should one not, it
    // contributes no candidates
    const int c = chosen < p.n_c ? chosen : -1;

    // ---- score the cluster's tokens: wave w takes j = w, w + 8, ..., kBatch
    // tokens at a time so that their ordering entries, then their rows, are
    // fetched together; a lane covers 4 consecutive elements of each
    // 256-element slice of a row.  The kBatch partial sums are reduced by a
    // transposed butterfly: after it, the 4 lanes 4m .. 4m + 3 hold the score
    // of token slot bt(m), the bits of m reversed ----
    constexpr int kBatch = 16;
    const int bt = ((lane >> 5) & 1) * 8 + ((lane >> 4) & 1) * 4 + ((lane >> 3) & 1) * 2 + ((lane >> 2) & 1);
    float best = -INFINITY;
    int best_tok = -1, best_j = 0x7FFFFFFF;
    for (int j0 = wave; c >= 0 && j0 < p.per; j0 += kWaves * kBatch) {
        uint32_t tk[kBatch];
        bool ok[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int j = j0 + kWaves * b;
            ok[b] = j < p.per;
            tk[b] = ok[b] ? p.ordering[(int64_t)c * p.per + j] : 0u;
            ok[b] = ok[b] && tk[b] < (uint32_t)p.vocab;  // out of range: never read nor chosen
        }
        float acc[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) acc[b] = 0.f;
        for (int e = 4 * lane; e < p.h; e += 256) {
            uint2 w[kBatch];
#pragma unroll
            for (int b = 0; b < kBatch; ++b)
                w[b] = ok[b] ? *reinterpret_cast<const uint2 *>(p.embed + (int64_t)tk[b] * p.h + e) : make_uint2(0u, 0u);
            const float4 xv = *reinterpret_cast<const float4 *>(xs + e);
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                acc[b] = fmaf(__builtin_bit_cast(float, w[b].x << 16), xv.x, acc[b]);
                acc[b] = fmaf(__builtin_bit_cast(float, w[b].x & 0xFFFF0000u), xv.y, acc[b]);
                acc[b] = fmaf(__builtin_bit_cast(float, w[b].y << 16), xv.z, acc[b]);
                acc[b] = fmaf(__builtin_bit_cast(float, w[b].y & 0xFFFF0000u), xv.w, acc[b]);
            }
        }
        // halving steps: the lane with bit `off` set keeps the upper half
#pragma unroll
        for (int n = kBatch, off = 32; n > 1; n >>= 1, off >>= 1) {
            const bool upper = (lane & off) != 0;
#pragma unroll
            for (int b = 0; b < n / 2; ++b) {
                const float give = upper ? acc[b] : acc[b + n / 2];
                const float keep = upper ? acc[b + n / 2] : acc[b];
                acc[b] = keep + __shfl_xor(give, off, 64);
            }
        }
        float sc = acc[0];
        sc += __shfl_xor(sc, 2, 64);
        sc += __shfl_xor(sc, 1, 64);
        uint32_t my_tk = 0u;
        bool my_ok = false;
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
            if (b == bt) my_tk = tk[b], my_ok = ok[b];
        // a lane's slot advances in j with j0: the first maximum is kept
        if (my_ok && (best_tok < 0 || sc > best)) best = sc, best_tok = (int)my_tk, best_j = j0 + kWaves * bt;
    }
    // the wave's first maximum: larger score, then smaller j
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float ob = __shfl_xor(best, off, 64);
        const int ot = __shfl_xor(best_tok, off, 64), oj = __shfl_xor(best_j, off, 64);
        if (ot >= 0 && (best_tok < 0 || ob > best || (ob == best && oj < best_j))) best = ob, best_tok = ot, best_j = oj;
    }
    if (lane == 0) wbest[wave] = best, wtok[wave] = best_tok, wj[wave] = best_j;
    __syncthreads();
    if (tid == 0) {
        float b = wbest[0];
        int btk = wtok[0], bj = wj[0];
        for (int w = 1; w < kWaves; ++w)
            if (wtok[w] >= 0 && (btk < 0 || wbest[w] > b || (wbest[w] == b && wj[w] < bj)))
                b = wbest[w], btk = wtok[w], bj = wj[w];
        p.part_score[(int64_t)row * p.k + i] = b;
        p.part_token[(int64_t)row * p.k + i] = btk;
    }
}

// One wave per row: lane l takes clusters l, l + 64, ... (keeping its first
// maximum), then the lanes' bests meet by larger score, then earlier
// cluster: the first maximum in visiting order.
__global__ __launch_bounds__(64) void final_kernel(const float *part_score, const int *part_token, int k,
                                                   int *token, float *score) {
    const int row = blockIdx.x, lane = threadIdx.x;
    float b = -INFINITY;
    int bt = -1, bi = 0x7FFFFFFF;
    for (int i = lane; i < k; i += 64) {
        const float s = part_score[(int64_t)row * k + i];
        const int tk = part_token[(int64_t)row * k + i];
        if (tk >= 0 && (bt < 0 || s > b)) b = s, bt = tk, bi = i;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float ob = __shfl_xor(b, off, 64);
        const int obt = __shfl_xor(bt, off, 64), obi = __shfl_xor(bi, off, 64);
        if (obt >= 0 && (bt < 0 || ob > b || (ob == b && obi < bi))) b = ob, bt = obt, bi = obi;
    }
    if (lane == 0) {
        token[row] = bt;
        if (score) score[row] = b;
    }
}

}  // namespace

// Dynamic LDS of the select kernel: x (h), the row's logits (C) and the
// sort of the k chosen (2 x next power of two >= k).
size_t lm_head_lds_bytes(int n_c, int h, int k) {
    int n_pow2 = 1;
    while (n_pow2 < k) n_pow2 <<= 1;
    return (size_t)(2 * n_pow2 + h + n_c) * 4;
}

size_t lm_head_workspace_bytes(int t, int n_c, int k) { return (size_t)t * (n_c + 2 * k) * 4; }

hipError_t launch_lm_head(const float *x, int t, int h, const KJob &centroids, const uint16_t *embed, int vocab,
                          const uint32_t *ordering, int k, int *token, int *clusters, float *score, void *workspace,
                          int cu_count, hipStream_t s) {
    const int n_c = centroids.n_out;
    if (t < 1 || t > kGemvMaxT || h % kBlock || n_c < 1 || vocab % n_c || k < 1 || k > n_c) return hipErrorInvalidValue;
    if (lm_head_lds_bytes(n_c, h, k) > kLmHeadMaxLds) return hipErrorInvalidValue;
    LmParams p{};
    p.x = x;
    p.embed = embed;
    p.ordering = ordering;
    p.clusters = clusters;
    p.h = h;
    p.n_c = n_c;
    p.n_pow2 = 1;
    while (p.n_pow2 < k) p.n_pow2 <<= 1;
    p.per = vocab / n_c;
    p.k = k;
    p.vocab = vocab;
    // scratch: logits [t][C], partial results [t][k]: the caller's workspace,
    // else stream-ordered
    const size_t cl_bytes = (size_t)t * n_c * 4, part_bytes = (size_t)t * k * 4;
    void *scratch = workspace;
    hipError_t e = hipSuccess;
    if (!scratch) e = hipMallocAsync(&scratch, cl_bytes + 2 * part_bytes, s);
    if (e != hipSuccess) return e;
    float *cl = static_cast<float *>(scratch);
    p.cl = cl;
    p.part_score = reinterpret_cast<float *>(static_cast<char *>(scratch) + cl_bytes);
    p.part_token = reinterpret_cast<int *>(static_cast<char *>(scratch) + cl_bytes + part_bytes);
    KJob cj = centroids;
    cj.y = cl;
    e = launch_gemv(FMT_BF16, x, t, h, &cj, 1, cu_count, s);
    if (e == hipSuccess) {
        const size_t lds = lm_head_lds_bytes(n_c, h, k);
        if (lds > 64 * 1024)
            e = hipFuncSetAttribute(reinterpret_cast<const void *>(select_score_kernel),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e == hipSuccess) {
            hipLaunchKernelGGL(select_score_kernel, dim3(k, t), dim3(kSelThreads), lds, s, p);
            e = hipGetLastError();
        }
    }
    if (e == hipSuccess) {
        hipLaunchKernelGGL(final_kernel, dim3(t), dim3(64), 0, s, p.part_score, p.part_token, k, token, score);
        e = hipGetLastError();
    }
    hipError_t fe = workspace ? hipSuccess : hipFreeAsync(scratch, s);
    return e != hipSuccess ? e : fe;
}

}  // namespace il
