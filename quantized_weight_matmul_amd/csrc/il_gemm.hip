// il_gemm.hip -- prefill GEMM for t > 8 on the gfx950 bf16 matrix cores.
//
// Computes y[t][n_out] = bf16(x)[t][n_in] * W^T with f32 accumulation for
// every job of one format in one launch (the batch of `struct Job`s over one
// shared x that Backend::matmul on the oxinfer 0.0.0 src/gpu.rs page submits
// at once).  x is rounded to bf16 (round-to-nearest-even) by a pre-pass into
// a scratch buffer the caller supplies; bf16 weights are used as stored.
// Q8/Q4 weights enter the matrix cores as their exact integer codes (Q8 q,
// Q4 16 * (code - 8); both are bf16 numbers), and each 32-element block's f32
// partial sum is multiplied by that block's scale (Q4: the f16 scale / 16,
// exact) before it is added to the output: no dequantised weight is rounded,
// so the only rounding of an input is that of x.
//
// One launch holds two kinds of work unit (both on 8 waves, two per SIMD):
//   bf16 weights: whole rounds of 256 x 256 tiles (256 tokens x 256 weight
//     rows, the waves a 2 x 4 grid of 128 x 64), then the tiles left over as
//     128 x 128 quarters (a 4 x 2 grid of 32 x 64), so the last round is
//     short instead of mostly idle;
//   Q8/Q4 weights: whole rounds of 256 x 128 halves (a 4 x 2 grid of 64 x 64),
//     then the rest as 128 x 128 quarters (32 x 64 per wave).
// Workgroups are dispatched in block order, the big units first, so CUs that
// finish their last big unit pick up the small ones.  Every unit walks K in
// steps of 64 through two LDS stages, with 32x32x16 bf16 MFMAs (one wave
// issuing them keeps the matrix core near its peak, which 16x16x32 does
// not); two waves per SIMD let one wave's MFMAs cover the other's waits.
//   bf16 tiles: each K step's x and W tiles go from L2 straight into the LDS
//     stage the MFMAs are not reading (buffer loads with the LDS bit: no
//     staging registers, no LDS write instructions), issued at the start of
//     the step before by four of the eight waves (one per SIMD, so that the
//     other wave there keeps the matrix core busy while the issuing one
//     waits on the load unit); one barrier per step.
//   Q8/Q4 tiles: x's tile is copied into LDS the same way; the weight codes
//     are fetched into registers two steps ahead, converted to bf16 there and
//     written to the idle stage with the step's block scales.
// Q8/Q4 weights at 32 < t <= 128 run the mid-size plan instead: units of
// all t tokens by 128 weight rows, so that every weight is read and
// converted once (Q4 at t <= 64 on 4-wave units, below).
// Rows of 64 bf16 (8 chunks of 16 bytes) are stored with the chunk index
// XOR-swizzled by the row, so that the fragment reads (and the staging
// writes) are free of LDS bank conflicts.  Workgroups are mapped to units
// XCD by XCD (consecutive workgroup ids go to different XCDs), so that each
// XCD works on one contiguous range of units and its L2 holds the operand
// slices its workgroups share.
#include "il_internal.h"

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <type_traits>
#include <utility>

namespace il {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kBigM = 256;  // tokens per tile row of the unit grid
constexpr int BK = 64;
constexpr int kXcds = 8;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr uint32_t kBufFlags = 0x00020000u;
constexpr uint32_t kOut = 0x7FFFFFF0u;  // a buffer offset past every range: reads 0

// Output columns of a big unit: bf16 256 x 256 tiles, Q8/Q4 256 x 128
// halves; with gate/up pairs (GLU) half as many outputs per weight rows.
constexpr int big_cols(int fmt, bool glu) { return (fmt == FMT_BF16 ? 256 : 128) / (glu ? 2 : 1); }

// One launch: big units [0, n_big) of the unit grid (unit = tn * tiles_m +
// tm), then n_small small units covering big units small_lo, small_lo + 1,
// ... (bf16: four 128 x 128 quarters each, Q8/Q4: two 128-token halves).
struct GemmParams {
    const uint16_t *xb;  // bf16 x [t][n_in]
    int t;
    int n_in;
    int n_jobs;
    int tiles_m;        // 256-token rows of the unit grid
    int n_big;          // big units
    int big_per_xcd;    // ceil(n_big / kXcds)
    int n_small;        // small units
    int small_per_xcd;  // ceil(n_small / kXcds)
    int small_lo;       // first big unit the small units split
    KJob job[kMaxJobs];
    int tn0[kMaxJobs + 1];  // prefix sums of unit-grid columns per job
    // mid-size plan (Q8/Q4, 32 < t <= 128; mid_bm = 0 otherwise): units of
    // mid_bm tokens x 128 weight rows; the big units are run whole, the
    // n_small small ones are chunk c = u % n_chunks of unit n_big + u / n_chunks
    int mid_bm;
    int nk;        // K steps of BK
    int n_chunks;  // K chunks every mid unit sums separately, in order
    int chunk_hi[16];  // chunk c = steps [chunk_hi[c - 1], chunk_hi[c]) (chunk_hi[-1] = 0)
    float *part;   // [unit - n_big][chunk][mid_bm * 128] chunk sums of the split units
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, kBufFlags);
}

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));  // RNE
}

// Swizzle of the 16-byte chunk index within an LDS row of 64 bf16.  Rows r
// and the 8 chunks c: slot = c ^ ((r & 7) ^ ((r >> 3) & 1)).  Any 16
// consecutive rows read at one chunk land in 16 distinct (bank-half, slot)
// pairs (64-bank LDS), and any 8 in 8 distinct slots (32-bank LDS).
__device__ __forceinline__ int swz_key(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// s_waitcnt vmcnt(N) (gfx9 encoding; the other counters are not waited for).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the release fence of __syncthreads, which would
// wait for every load in flight; callers wait for what must have landed
// first.  The signal fences keep the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at
// dst + 16 l (dst is wave-uniform); reads past the buffer write zeros.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, uint16_t *dst, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, off, 0, 0, 0);
}

// Unit -> (first token, first output column, job).  Returns false for a unit
// whose sub-tile lies past the edge of x or of its job.
struct Place {
    int m0, n0, j;
};
template <bool GLU>
__device__ __forceinline__ bool place(const GemmParams &p, int unit, int cols, int sub_m, int sub_n, int sub_cols,
                                      Place &pl) {
    const int tn_all = unit / p.tiles_m;
    const int tm = unit - tn_all * p.tiles_m;
    int j = 0;
    if constexpr (!GLU) {
#pragma unroll
        for (int jj = 1; jj < kMaxJobs; ++jj)
            if (jj < p.n_jobs && tn_all >= p.tn0[jj]) j = jj;
    }
    pl.j = j;
    pl.m0 = tm * kBigM + sub_m;
    pl.n0 = (tn_all - p.tn0[j]) * cols + sub_n * sub_cols;
    return pl.m0 < p.t && pl.n0 < p.job[j].n_out;
}

// Which unit this workgroup runs: blocks [0, 8 * big_per_xcd) the big units,
// the rest the small ones, each range mapped XCD by XCD.  Returns -1 (no
// work), 0 (big unit *u) or 1 (small unit *u).
__device__ __forceinline__ int unit_of(const GemmParams &p, int *u) {
    const int b = blockIdx.x;
    const int big_blocks = kXcds * p.big_per_xcd;
    if (b < big_blocks) {
        *u = (b % kXcds) * p.big_per_xcd + b / kXcds;
        return *u < p.n_big ? 0 : -1;
    }
    const int bb = b - big_blocks;
    *u = (bb % kXcds) * p.small_per_xcd + bb / kXcds;
    return *u < p.n_small ? 1 : -1;
}

// ---- epilogue: 32x32 tile, lane holds rows 8 (i / 4) + 4 (lane / 32) + i % 4
//      of column lane % 32; GLU: tile 0 of a wave is the gate, tile 1 the up
//      projection of the same outputs ----
template <int TM, int TN, bool GLU>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[TM][TN], const KJob &jb, int t, int row0, int col0,
                                           int lane) {
    if constexpr (GLU) {
#pragma unroll
        for (int a = 0; a < TM; ++a) {
            const int col = col0 + (lane & 31);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = row0 + a * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
                if (row < t && col < jb.n_out) jb.y[(int64_t)row * jb.n_out + col] = gelu(acc[a][0][i]) * acc[a][1][i];
            }
        }
    } else {
#pragma unroll
        for (int a = 0; a < TM; ++a) {
#pragma unroll
            for (int n = 0; n < TN; ++n) {
                const int col = col0 + n * 32 + (lane & 31);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = row0 + a * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
                    if (row < t && col < jb.n_out) jb.y[(int64_t)row * jb.n_out + col] = acc[a][n][i];
                }
            }
        }
    }
}

// x f32 -> bf16 (RNE) pre-pass: groups of 8 elements (32 bytes in, 16 out).
// A grid of at most kPreWgPerCu workgroups per compute unit strides over the
// groups, kPreGroups * 256 consecutive ones per workgroup and round (thread i
// the groups i, i + 256, ...); each thread loads its next round's groups
// before it stores this round's, so reads and writes overlap (50 MB on the
// 2048-token prefill: 14.1 against 15.8-16.0 us with one round per
// workgroup, by HIP events).
constexpr int kPreGroups = 2;
constexpr int kPreWgPerCu = 8;
__global__ __launch_bounds__(256) void x_to_bf16_kernel(const float *__restrict__ x, uint4 *__restrict__ xb,
                                                        int64_t n8) {
    const float4 *x4 = reinterpret_cast<const float4 *>(x);
    const int64_t stride = (int64_t)gridDim.x * (256 * kPreGroups);
    int64_t g0 = (int64_t)blockIdx.x * (256 * kPreGroups) + threadIdx.x;
    float4 a[kPreGroups], b[kPreGroups];
#pragma unroll
    for (int u = 0; u < kPreGroups; ++u) {
        const int64_t g = g0 + u * 256;
        if (g < n8) {
            a[u] = x4[2 * g];
            b[u] = x4[2 * g + 1];
        }
    }
    while (g0 < n8) {
        const int64_t gn = g0 + stride;
        float4 a2[kPreGroups], b2[kPreGroups];
#pragma unroll
        for (int u = 0; u < kPreGroups; ++u) {
            const int64_t g = gn + u * 256;
            if (g < n8) {
                a2[u] = x4[2 * g];
                b2[u] = x4[2 * g + 1];
            }
        }
#pragma unroll
        for (int u = 0; u < kPreGroups; ++u) {
            const int64_t g = g0 + u * 256;
            if (g < n8)
                xb[g] = make_uint4(pack_bf16(a[u].x, a[u].y), pack_bf16(a[u].z, a[u].w), pack_bf16(b[u].x, b[u].y),
                                   pack_bf16(b[u].z, b[u].w));
        }
#pragma unroll
        for (int u = 0; u < kPreGroups; ++u) {
            a[u] = a2[u];
            b[u] = b2[u];
        }
        g0 = gn;
    }
}

// ----------------------------------------------------------- Q8 / Q4 units
// A BM x 128 unit (BM = 256: a half; 128: a quarter, on 8 waves in a 4 x 2
// grid of (BM / 4) x 64; 64: on a 2 x 4 grid of 32 x 32) over K steps
// [ks_lo, ks_hi).  Per K step (64 = two quantisation blocks) each wave's
// 32x32 tiles get one MFMA chain per block, started from zero, whose f32
// result is scaled by the block's scale of the tile's weight row (one per
// lane: a lane holds one output column) and added to the accumulator.
// CHUNKED: the accumulator restarts from zero at each of the n_chunks chunk
// boundaries of K (chunk c = steps [nk c / n_chunks, nk (c + 1) / n_chunks))
// and the chunk sums are added, in chunk order, into the total, so that a
// unit computed whole and one whose chunks ran in separate workgroups give
// the same bits.  fin(acc, wm, wn, lane) takes the result.
// GLU: B-tile rows come in groups of 32 alternating between the gate and up
// projections (virtual row v is row (v / 64) * 32 + v % 32 of the gate if
// (v / 32) is even, of the up projection if odd), so a wave's two 32-column
// tiles are the gate and up sums of the same outputs.
template <int FMT, int BM, bool GLU, bool CHUNKED, class Fin>
__device__ __forceinline__ void q_unit(const GemmParams &p, uint16_t *lds, float *scl, int m0, int n0, const KJob &jb,
                                       int ks_lo, int ks_hi, Fin &&fin) {
    constexpr int BN = 128, WM = BM == 64 ? 2 : 4, WN = kWaves / WM;
    constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
    constexpr int kCols = GLU ? BN / 2 : BN;  // output columns of the unit
    constexpr int kChunksA = BM * BK / 8 / kThreads;  // 16-byte chunks per thread, A tile
    constexpr int TPR = kThreads / BN;                // staging threads per B row
    constexpr int EPT = BK / TPR;                     // codes of a B row per thread and step
    constexpr int kStage = (BM + BN) * BK;            // bf16 elements per LDS stage
    static_assert(TM >= 1 && TN >= 1 && EPT == 16 && kChunksA >= 1, "unit shape");
    static_assert(!GLU || TN == 2, "GLU pairs the two 32-column tiles of a wave");
    const int n_in = p.n_in;
    const int nb = n_in / kBlock;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // ---- operand descriptors: exactly the unit's valid rows ----
    const int a_rows = min(BM, p.t - m0);
    const int b_rows = min(kCols, jb.n_out - n0);
    const uint32_t row2 = (uint32_t)n_in * 2u;
    const __amdgpu_buffer_rsrc_t ars = make_rsrc(p.xb + (int64_t)m0 * n_in, (uint32_t)a_rows * row2);
    auto b_rsrc = [&](const KJob &k, __amdgpu_buffer_rsrc_t &c, __amdgpu_buffer_rsrc_t &sc) {
        if constexpr (FMT == FMT_Q8) {
            c = make_rsrc(static_cast<const int8_t *>(k.codes) + (int64_t)n0 * n_in, (uint32_t)b_rows * (uint32_t)n_in);
            sc = make_rsrc(static_cast<const float *>(k.scales) + (int64_t)n0 * nb, (uint32_t)b_rows * (uint32_t)nb * 4u);
        } else {
            // tile-major plane; n0 is a multiple of 16, so the unit's rows
            // start at a 16-row tile of the plane
            c = make_rsrc(static_cast<const uint8_t *>(k.codes) + (n0 >> 4) * q4_plane_bytes(16, nb),
                          (uint32_t)q4_plane_bytes(b_rows, nb));
            sc = make_rsrc(static_cast<const uint16_t *>(k.scales) + (int64_t)n0 * nb,
                           (uint32_t)b_rows * (uint32_t)nb * 2u);
        }
    };
    __amdgpu_buffer_rsrc_t brs, bss, brs2, bss2;
    b_rsrc(jb, brs, bss);
    if constexpr (GLU) b_rsrc(p.job[1], brs2, bss2);
    else brs2 = brs, bss2 = bss;

    // weight staging: TPR threads per B row; this thread owns row qr and
    // codes EPT qh .. EPT qh + EPT - 1 of the step (half of block qh / 2)
    const int qr = tid / TPR, qh = tid % TPR;
    const int qkey = swz_key(qr);
    // a wave stages 16 B rows, inside one 32-row group: whether they are
    // gate or up rows is the same for the whole wave (taken from the wave
    // index, so that the descriptor choice is scalar)
    static_assert(64 / TPR == 16, "a wave stages 16 rows");
    const bool up = GLU && ((wave >> 1) & 1);
    const int wr = GLU ? (qr >> 6) * 32 + (qr & 31) : qr;
    const __amdgpu_buffer_rsrc_t crs = up ? brs2 : brs, srs = up ? bss2 : bss;
    // two register sets: the codes of step k are fetched into set k & 1 two
    // steps before they are stored, which covers the HBM latency of a step
    uint4 sb[2];
    uint32_t sbits[2] = {0u, 0u};  // the block scales' bits (Q8 f32, Q4 f16), converted in store()
    auto fetch = [&](int k0, auto set_c) {
        constexpr int S = decltype(set_c)::value;
        const int kh = k0 + EPT * qh;
        const bool ok = kh < n_in && wr < b_rows;
        if constexpr (FMT == FMT_Q8) {
            sb[S] = bload16(crs, ok ? (uint32_t)wr * (uint32_t)n_in + (uint32_t)kh : kOut);
            sbits[S] = __builtin_amdgcn_raw_buffer_load_b32(srs, ok ? ((uint32_t)wr * nb + kh / kBlock) * 4u : kOut, 0, 0);
        } else {
            const uint32_t qoff = (uint32_t)q4_block_offset(wr, kh / kBlock, nb) + (uint32_t)((kh % kBlock) / 2);
            const uint2 h = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(crs, ok ? qoff : kOut, 0, 0));
            sb[S] = make_uint4(h.x, h.y, 0u, 0u);
            sbits[S] = __builtin_amdgcn_raw_buffer_load_b16(srs, ok ? ((uint32_t)wr * nb + kh / kBlock) * 2u : kOut, 0, 0);
        }
    };
    // the codes as exact bf16 numbers into stage st, and the block's scale
    auto store = [&](int st, auto set_c) {
        constexpr int S = decltype(set_c)::value;
        uint16_t *Bs = lds + st * kStage + BM * BK;
        uint32_t o[8];
        if constexpr (FMT == FMT_Q8) {
            const uint32_t w[4] = {sb[S].x, sb[S].y, sb[S].z, sb[S].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                o[2 * i] = pack_bf16((float)(int8_t)(w[i]), (float)(int8_t)(w[i] >> 8));
                o[2 * i + 1] = pack_bf16((float)(int8_t)(w[i] >> 16), (float)(int8_t)(w[i] >> 24));
            }
        } else {
            const uint32_t w[2] = {sb[S].x, sb[S].y};
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint32_t lo = (w[i] << 4) & 0xF0F0F0F0u;  // elements 0, 2, 4, 6: 16 (code - 8)
                const uint32_t hi = w[i] & 0xF0F0F0F0u;         // elements 1, 3, 5, 7
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[4 * i + e] = pack_bf16((float)(int8_t)(lo >> (8 * e)), (float)(int8_t)(hi >> (8 * e)));
            }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
            *reinterpret_cast<uint4 *>(Bs + qr * BK + ((2 * qh + i) ^ qkey) * 8) =
                make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
        if ((qh & 1) == 0) {
            const float ssc = FMT == FMT_Q8 ? __builtin_bit_cast(float, sbits[S])
                                            : (float)__builtin_bit_cast(_Float16, (uint16_t)sbits[S]) * 0.0625f;  // Q4 codes carry * 16; exact
            scl[(st * BN + qr) * 2 + (qh >> 1)] = ssc;
        }
    };

    f32x16 acc[TM][TN], tot[CHUNKED ? TM : 1][CHUNKED ? TN : 1];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int n = 0; n < TN; ++n) acc[a][n] = (f32x16){};
    if constexpr (CHUNKED) {
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
            for (int n = 0; n < TN; ++n) tot[a][n] = (f32x16){};
    }
    int chunk = 0;
    const auto chunk_end = [&](int c) { return (int)((int64_t)p.nk * (c + 1) / p.n_chunks); };
    int next_fold = CHUNKED ? chunk_end(0) : 0;

    // 32x32x16 fragments: lane reads row (lane & 31) of a 32-row tile, 16-byte
    // chunk 2 kk + lane / 32; every fragment row of this lane shares one
    // swizzle key because tile offsets are multiples of 32
    const int frow = lane & 31;
    const int fkey = swz_key(frow);
    const int a_base = (wm * (BM / WM) + frow) * BK;
    const int b_base = (wn * (BN / WN) + frow) * BK;
    auto compute = [&](int st) {
        const uint16_t *As = lds + st * kStage, *Bs = As + BM * BK;
        // this lane's output columns are B rows wn * 64 + 32 n + lane % 32
        f32x2 s[TN];
#pragma unroll
        for (int n = 0; n < TN; ++n) s[n] = *reinterpret_cast<const f32x2 *>(scl + (st * BN + wn * (BN / WN) + n * 32 + frow) * 2);
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            f32x16 part[TM][TN];
#pragma unroll
            for (int kk2 = 0; kk2 < 2; ++kk2) {
                const int slot = ((2 * blk + kk2) * 2 + (lane >> 5)) ^ fkey;
                bf16x8 fa[TM], fb[TN];
#pragma unroll
                for (int a = 0; a < TM; ++a) fa[a] = *reinterpret_cast<const bf16x8 *>(As + a_base + a * 32 * BK + slot * 8);
#pragma unroll
                for (int n = 0; n < TN; ++n) fb[n] = *reinterpret_cast<const bf16x8 *>(Bs + b_base + n * 32 * BK + slot * 8);
#pragma unroll
                for (int a = 0; a < TM; ++a)
#pragma unroll
                    for (int n = 0; n < TN; ++n)
                        part[a][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[n], kk2 ? part[a][n] : (f32x16){},
                                                                              0, 0, 0);
            }
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int n = 0; n < TN; ++n)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[a][n][i] = fmaf(s[n][blk], part[a][n][i], acc[a][n][i]);
        }
    };

    const int nk = ks_hi;
    uint32_t offa[kChunksA];
    int ka[kChunksA];
#pragma unroll
    for (int i = 0; i < kChunksA; ++i) {
        const int u = (wave * kChunksA + i) * 64 + lane, r = u >> 3;
        ka[i] = ((u & 7) ^ swz_key(r)) * 8;
        offa[i] = (uint32_t)r * row2 + (uint32_t)ka[i] * 2u;
    }
    auto issue_a = [&](int st, int k0) {
        uint16_t *As = lds + st * kStage;
#pragma unroll
        for (int i = 0; i < kChunksA; ++i)
            lds_load16(ars, As + (wave * kChunksA + i) * 64 * 8, k0 + ka[i] < n_in ? offa[i] + (uint32_t)k0 * 2u : kOut);
    };
    // B register loads per fetch (codes, then the scale).  A step first
    // writes the codes of the next step (fetched two steps before) into the
    // idle stage, then issues that stage's x copy and the fetch of the step
    // three ahead, then computes: the one wait for the copy is at the end of
    // the step, behind all of its MFMAs and FMAs, and leaves the newest fetch
    // in flight.  (Writing the codes after the copy is issued makes the
    // compiler wait for the copy there: it cannot tell the two LDS ranges
    // apart.)
    constexpr int kBLoads = 2;
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    const int k0 = ks_lo * BK;
    issue_a(0, k0);
    fetch(k0, S0{});
    if (ks_lo + 1 < nk) fetch(k0 + BK, S1{});
    store(0, S0{});
    if (ks_lo + 2 < nk) fetch(k0 + 2 * BK, S0{});
    wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this thread's LDS writes are done
    lds_barrier();
    // step ks computes stage (ks - ks_lo) & 1; the codes of step ks + 1 are
    // in set (ks + 1 - ks_lo) & 1
    auto step = [&](int ks, auto cur_c) {
        constexpr int cur = decltype(cur_c)::value;
        using Next = std::integral_constant<int, cur ^ 1>;
        bool fetched = false;
        if (ks + 1 < nk) {
            store(cur ^ 1, Next{});  // B of step ks + 1
            issue_a(cur ^ 1, (ks + 1) * BK);
            if (ks + 3 < nk) fetch((ks + 3) * BK, Next{}), fetched = true;
        }
        compute(cur);
        if constexpr (CHUNKED) {
            if (ks + 1 == next_fold) {  // the last step of chunk `chunk`
#pragma unroll
                for (int a = 0; a < TM; ++a)
#pragma unroll
                    for (int n = 0; n < TN; ++n) {
                        tot[a][n] += acc[a][n];
                        acc[a][n] = (f32x16){};
                    }
                ++chunk;
                next_fold = chunk < p.n_chunks ? chunk_end(chunk) : -1;
            }
        }
        if (fetched) wait_vmcnt<kBLoads>(); else wait_vmcnt<0>();
        __builtin_amdgcn_s_waitcnt(0xC07F);
        lds_barrier();
    };
    for (int ks = ks_lo; ks < nk; ks += 2) {
        step(ks, S0{});
        if (ks + 1 < nk) step(ks + 1, S1{});
    }
    if constexpr (CHUNKED) fin(tot, wm, wn, lane);
    else fin(acc, wm, wn, lane);
}

// The same BM x 128 Q8/Q4 unit for mid-size t (BM = 64 or 128 holds every
// token; Q4 with 64 tokens and no gate/up pair runs the 4-wave unit further
// down instead), with longer K steps and a deeper pipeline: with BM small a K step
// of 64 has little arithmetic, and its fixed costs (the barrier, the waits,
// all eight waves reading LDS at once) dominated.  Here a step is kMidBK =
// 128 (four quantisation blocks; one block's codes per staging thread), every
// thread keeps kMidDepth steps of its codes in flight in a ring of registers,
// and x's tile is copied mid_a_stages - 1 steps ahead into a ring of LDS
// stages; the codes of the next step are converted into one of two B
// stages.  Every step issues the same loads (past the unit's range they read
// nothing: out-of-range offsets), so the number of loads behind any given
// one is fixed and one wait count serves every step.  The loop is unrolled
// kMidDepth times so that ring indices are constants.  An LDS row holds 128
// bf16 as 16 chunks of 16 bytes, chunk c of row r at slot c ^ (r & 15).
// f(integral_constant<int, J>) for J = 0 .. N - 1 in order, while it returns true.
template <class F, int... J>
__device__ __forceinline__ void unrolled_while(F &&f, std::integer_sequence<int, J...>) {
    (void)(f(std::integral_constant<int, J>{}) && ...);
}

constexpr int kMidBK = 128;   // K per step of a mid unit
constexpr int kMidDepth = 4;  // steps of codes in flight per thread
template <int BM>
constexpr int mid_a_stages() { return BM == 64 ? 4 : 2; }  // LDS stages of x's tile
template <int BM>
constexpr int mid_lds_elems() {  // bf16 elements: A ring, two B stages, then the scales
    return mid_a_stages<BM>() * BM * kMidBK + 2 * 128 * kMidBK + 2 * 128 * 4 * 2;
}

template <int FMT, int BM, bool GLU, bool CHUNKED, class Fin>
__device__ __forceinline__ void q_mid_unit(const GemmParams &p, uint16_t *lds, int m0, int n0, const KJob &jb,
                                           int ks_lo, int ks_hi, Fin &&fin) {
    constexpr int BN = 128, BKM = kMidBK, WM = BM == 64 ? 2 : 4, WN = kWaves / WM;
    constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
    constexpr int kCols = GLU ? BN / 2 : BN;
    constexpr int kRowChunks = BKM / 8;                           // 16-byte chunks per LDS row
    constexpr int kChunksA = BM * kRowChunks / kThreads;          // A copies per thread and step
    constexpr int TPR = kThreads / BN, EPT = BKM / TPR;           // staging threads per B row, codes each
    constexpr int kF = FMT == FMT_Q8 ? 3 : 2;                     // loads per fetch
    constexpr int D = kMidDepth, NA = mid_a_stages<BM>();
    static_assert(TM >= 1 && TN >= 1 && EPT == kBlock && kChunksA >= 1 && kRowChunks == 16, "unit shape");
    static_assert(!GLU || TN == 2, "GLU pairs the two 32-column tiles of a wave");
    static_assert(D % NA == 0 && D % 2 == 0, "ring sizes divide the unroll");
    uint16_t *const Aring = lds;
    uint16_t *const Bst = lds + NA * BM * BKM;
    float *const scl = reinterpret_cast<float *>(Bst + 2 * BN * BKM);  // [stage][B row][block of the step]
    const int n_in = p.n_in;
    const int nb = n_in / kBlock;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    const int a_rows = min(BM, p.t - m0);
    const int b_rows = min(kCols, jb.n_out - n0);
    const uint32_t row2 = (uint32_t)n_in * 2u;
    const __amdgpu_buffer_rsrc_t ars = make_rsrc(p.xb + (int64_t)m0 * n_in, (uint32_t)a_rows * row2);
    // the codes, and the scales from the tiled plane (rows padded to 16 and
    // blocks to 4 with zero scales), so that a block past the end of K, or a
    // row past the job's last, is multiplied by 0; rows past the padding lie
    // outside the descriptors and read 0
    const int nb4 = (nb + 3) / 4;
    constexpr uint32_t kSclBytes = FMT == FMT_Q8 ? 4u : 2u;
    auto b_rsrc = [&](const KJob &k, __amdgpu_buffer_rsrc_t &c, __amdgpu_buffer_rsrc_t &sc) {
        if constexpr (FMT == FMT_Q8)
            c = make_rsrc(static_cast<const int8_t *>(k.codes) + (int64_t)n0 * n_in, (uint32_t)b_rows * (uint32_t)n_in);
        else
            c = make_rsrc(static_cast<const uint8_t *>(k.codes) + (n0 >> 4) * q4_plane_bytes(16, nb),
                          (uint32_t)q4_plane_bytes(b_rows, nb));
        sc = make_rsrc(static_cast<const uint8_t *>(k.scales_t) + (int64_t)(n0 >> 4) * nb4 * 64 * kSclBytes,
                       (uint32_t)tiled_scale_count(b_rows, nb) * kSclBytes);
    };
    __amdgpu_buffer_rsrc_t brs, bss, brs2, bss2;
    b_rsrc(jb, brs, bss);
    if constexpr (GLU) b_rsrc(p.job[1], brs2, bss2);
    else brs2 = brs, bss2 = bss;

    // staging of the codes: TPR threads per B row, each one quantisation
    // block (block qh of the step) of row qr
    const int qr = tid / TPR, qh = tid % TPR;
    const int qkey = qr & 15;
    // gate or up rows: the same for the whole wave (16 rows of one 32-row
    // group), taken from the wave index so that the descriptor choice is scalar
    static_assert(64 / TPR == 16, "a wave stages 16 rows");
    const bool up = GLU && ((wave >> 1) & 1);
    const int wr = GLU ? (qr >> 6) * 32 + (qr & 31) : qr;
    const __amdgpu_buffer_rsrc_t crs = up ? brs2 : brs, srs = up ? bss2 : bss;
    uint4 cq[D][FMT == FMT_Q8 ? 2 : 1];
    uint32_t cs[D];
    // this thread's block of step ks is block 4 ks + qh of row wr: its codes
    // at c_base + ks * c_step, its scale at s_base + ks * s_step.  Past the
    // end of K (the fetches that run ahead of the last steps) these read
    // padding, the next tile's codes or nothing; the results are never used.
    const uint32_t c_base = FMT == FMT_Q8 ? (uint32_t)wr * (uint32_t)n_in + (uint32_t)qh * kBlock
                                          : (uint32_t)q4_block_offset(wr, qh, nb);
    constexpr uint32_t c_step = FMT == FMT_Q8 ? BKM : 1024u;  // Q4: one 64-byte segment per row and step
    const uint32_t s_base = (uint32_t)tiled_scale_index(wr, qh, nb4) * kSclBytes;
    constexpr uint32_t s_step = 64u * kSclBytes;
    auto fetch = [&](int ks, auto slot_c) {
        constexpr int S = decltype(slot_c)::value;
        const uint32_t co = c_base + (uint32_t)ks * c_step, so = s_base + (uint32_t)ks * s_step;
        if constexpr (FMT == FMT_Q8) {
            cq[S][0] = bload16(crs, co);
            cq[S][1] = bload16(crs, co + 16u);
            cs[S] = __builtin_amdgcn_raw_buffer_load_b32(srs, so, 0, 0);
        } else {
            cq[S][0] = bload16(crs, co);
            cs[S] = __builtin_amdgcn_raw_buffer_load_b16(srs, so, 0, 0);
        }
    };
    // ring slot S as exact bf16 codes into B stage st, with the block's scale
    auto store = [&](int st, auto slot_c) {
        constexpr int S = decltype(slot_c)::value;
        uint16_t *Bs = Bst + st * BN * BKM;
        uint32_t o[16];
        if constexpr (FMT == FMT_Q8) {
            const uint32_t w[8] = {cq[S][0].x, cq[S][0].y, cq[S][0].z, cq[S][0].w,
                                   cq[S][1].x, cq[S][1].y, cq[S][1].z, cq[S][1].w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                o[2 * i] = pack_bf16((float)(int8_t)(w[i]), (float)(int8_t)(w[i] >> 8));
                o[2 * i + 1] = pack_bf16((float)(int8_t)(w[i] >> 16), (float)(int8_t)(w[i] >> 24));
            }
        } else {
            const uint32_t w[4] = {cq[S][0].x, cq[S][0].y, cq[S][0].z, cq[S][0].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t lo = (w[i] << 4) & 0xF0F0F0F0u;  // elements 0, 2, 4, 6: 16 (code - 8)
                const uint32_t hi = w[i] & 0xF0F0F0F0u;         // elements 1, 3, 5, 7
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[4 * i + e] = pack_bf16((float)(int8_t)(lo >> (8 * e)), (float)(int8_t)(hi >> (8 * e)));
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<uint4 *>(Bs + qr * BKM + ((4 * qh + i) ^ qkey) * 8) =
                make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
        scl[(st * BN + qr) * 4 + qh] = FMT == FMT_Q8 ? __builtin_bit_cast(float, cs[S])
                                                     : (float)__builtin_bit_cast(_Float16, (uint16_t)cs[S]) * 0.0625f;  // Q4 codes carry * 16; exact
    };
    uint32_t offa[kChunksA];
    int ka[kChunksA];
#pragma unroll
    for (int i = 0; i < kChunksA; ++i) {
        const int u = (wave * kChunksA + i) * 64 + lane, r = u / kRowChunks;
        ka[i] = ((u % kRowChunks) ^ (r & 15)) * 8;
        offa[i] = (uint32_t)r * row2 + (uint32_t)ka[i] * 2u;
    }
    // x's tile of step ks into A stage st; a step that ends past n_in reads
    // zeros there (not the next row of x).  The copies that run ahead of the
    // last steps land in stages that are never read.
    auto issue_a = [&](int st, int ks) {
        uint16_t *As = Aring + st * BM * BKM;
        const int k0 = ks * BKM;
        if (k0 + BKM <= n_in) {
#pragma unroll
            for (int i = 0; i < kChunksA; ++i)
                lds_load16(ars, As + (wave * kChunksA + i) * 64 * 8, offa[i] + (uint32_t)k0 * 2u);
        } else {
#pragma unroll
            for (int i = 0; i < kChunksA; ++i)
                lds_load16(ars, As + (wave * kChunksA + i) * 64 * 8, k0 + ka[i] < n_in ? offa[i] + (uint32_t)k0 * 2u : kOut);
        }
    };

    f32x16 acc[TM][TN], tot[CHUNKED ? TM : 1][CHUNKED ? TN : 1];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int n = 0; n < TN; ++n) acc[a][n] = (f32x16){};
    if constexpr (CHUNKED) {
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
            for (int n = 0; n < TN; ++n) tot[a][n] = (f32x16){};
    }
    int chunk = 0;
    int next_fold = CHUNKED ? p.chunk_hi[0] : 0;

    const int frow = lane & 31;
    const int fkey = frow & 15;
    const int a_base = (wm * (BM / WM) + frow) * BKM;
    const int b_base = (wn * (BN / WN) + frow) * BKM;
    // With one 32x32 tile per wave (BM = 64), a block's scaled sum is added
    // to the accumulator only after the next block's MFMAs are issued, so
    // that the FMAs do not wait for the MFMA results they consume: block b's
    // MFMA results go to buffer b & 1 (four blocks per step, so the last
    // block of a step is always in buffer 1) and are added while block b + 1
    // computes into the other.  (Before the first block, buffer 1 holds a
    // zero product.)  With two tiles per wave (BM = 128) the second buffer
    // does not fit in registers: each block's sum is added right after its
    // MFMAs, and the other wave on the SIMD covers the wait.  Either way the
    // additions into acc come block by block, in order.
    static_assert((BKM / kBlock) % 2 == 0, "blocks alternate between the two buffers");
    constexpr bool kDefer = TM * TN == 1;
    f32x16 part[kDefer ? 2 : 1][TM][TN];
    float part_s[2][TN];
    auto clear1 = [&]() {
        if constexpr (kDefer) {
#pragma unroll
            for (int n = 0; n < TN; ++n) {
                part_s[1][n] = 0.f;
#pragma unroll
                for (int a = 0; a < TM; ++a) part[1][a][n] = (f32x16){};
            }
        }
    };
    clear1();
    auto flush = [&](auto buf_c) {
        if constexpr (!kDefer) return;
        constexpr int B = kDefer ? decltype(buf_c)::value : 0;
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
            for (int n = 0; n < TN; ++n)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[a][n][i] = fmaf(part_s[B][n], part[B][a][n][i], acc[a][n][i]);
    };
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    auto compute = [&](int sa, int sb) {
        const uint16_t *As = Aring + sa * BM * BKM, *Bs = Bst + sb * BN * BKM;
        f32x4 s[TN];
#pragma unroll
        for (int n = 0; n < TN; ++n) s[n] = *reinterpret_cast<const f32x4 *>(scl + (sb * BN + wn * (BN / WN) + n * 32 + frow) * 4);
        auto block = [&](int blk, auto buf_c) {
            constexpr int B = kDefer ? decltype(buf_c)::value : 0;
#pragma unroll
            for (int kk2 = 0; kk2 < 2; ++kk2) {
                const int slot = ((2 * blk + kk2) * 2 + (lane >> 5)) ^ fkey;
                bf16x8 fa[TM], fb[TN];
#pragma unroll
                for (int a = 0; a < TM; ++a) fa[a] = *reinterpret_cast<const bf16x8 *>(As + a_base + a * 32 * BKM + slot * 8);
#pragma unroll
                for (int n = 0; n < TN; ++n) fb[n] = *reinterpret_cast<const bf16x8 *>(Bs + b_base + n * 32 * BKM + slot * 8);
#pragma unroll
                for (int a = 0; a < TM; ++a)
#pragma unroll
                    for (int n = 0; n < TN; ++n)
                        part[B][a][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[n],
                                                                                 kk2 ? part[B][a][n] : (f32x16){}, 0, 0, 0);
            }
            if constexpr (kDefer) {
                flush(std::integral_constant<int, B ^ 1>{});  // the previous block
#pragma unroll
                for (int n = 0; n < TN; ++n) part_s[B][n] = s[n][blk];
            } else {
#pragma unroll
                for (int a = 0; a < TM; ++a)
#pragma unroll
                    for (int n = 0; n < TN; ++n)
#pragma unroll
                        for (int i = 0; i < 16; ++i) acc[a][n][i] = fmaf(s[n][blk], part[0][a][n][i], acc[a][n][i]);
            }
        };
#pragma unroll
        for (int blk = 0; blk < BKM / kBlock; blk += 2) {
            block(blk, B0{});
            block(blk + 1, B1{});
        }
    };

    // Loads issued per step: kChunksA copies, then a fetch of kF loads.
    // Before step ks + 1 the copy of its x tile (issued at step ks + 2 - NA)
    // and the codes of step ks + 2 (fetched at step ks + 1 - D, stored at step
    // ks + 1) must have landed: the wait allows what was issued after the
    // later of them.
    // (In the first step fewer loads follow the codes of step ks_lo + 2,
    // fetched in the prologue after the tiles: (D - 2) fetches and one step.)
    constexpr int kPer = kChunksA + kF;
    constexpr int kAfterA = kF + (NA - 2) * kPer, kAfterF = (D - 1) * kPer, kFirst = (D - 2) * kF + kPer;
    constexpr int kWait0 = kAfterA < kAfterF ? kAfterA : kAfterF;
    constexpr int kWait = kWait0 < kFirst ? kWait0 : kFirst;
    static_assert(kWait >= 0 && kWait < 64, "vmcnt range");
    using Z = std::integral_constant<int, 0>;
    // prologue: the codes of step ks_lo first (they are converted before the
    // loop), then x's tiles of steps ks_lo .. ks_lo + NA - 2, then the codes
    // of steps ks_lo + 1 .. ks_lo + D - 1, and once slot 0 is converted, the
    // codes of step ks_lo + D into it (step j refills the slot it converts,
    // that of step j + 1, with the codes of step j + 1 + D)
    fetch(ks_lo, Z{});
#pragma unroll
    for (int j = 0; j < NA - 1; ++j) issue_a(j, ks_lo + j);
    unrolled_while(
        [&](auto j_c) {
            constexpr int J = decltype(j_c)::value;
            fetch(ks_lo + 1 + J, std::integral_constant<int, 1 + J>{});
            return true;
        },
        std::make_integer_sequence<int, D - 1>{});
    wait_vmcnt<(NA - 1) * kChunksA + (D - 1) * kF>();
    store(0, Z{});
    fetch(ks_lo + D, Z{});
    // x's tile of step ks_lo and the codes of step ks_lo + 1 (converted by
    // the first step), the later of which was followed by D - 1 fetches
    wait_vmcnt<(D - 1) * kF>();
    static_assert((D - 1) * kF <= (NA - 2) * kChunksA + D * kF, "the codes come after the tile");
    __builtin_amdgcn_s_waitcnt(0xC07F);
    lds_barrier();
    // step ks = ks_lo + i: A stage i % NA, B stage i % 2, its codes were in
    // ring slot i % D
    auto step = [&](int ks, auto i_c) {
        constexpr int I = decltype(i_c)::value;
        store((I + 1) & 1, std::integral_constant<int, (I + 1) % D>{});  // step ks + 1
        issue_a((I + NA - 1) % NA, ks + NA - 1);
        fetch(ks + 1 + D, std::integral_constant<int, (I + 1) % D>{});
        compute(I % NA, I & 1);
        if constexpr (CHUNKED) {
            if (ks + 1 == next_fold) {  // the last step of chunk `chunk`
                flush(B1{});
#pragma unroll
                for (int a = 0; a < TM; ++a)
#pragma unroll
                    for (int n = 0; n < TN; ++n) {
                        tot[a][n] += acc[a][n];
                        acc[a][n] = (f32x16){};
                    }
                clear1();
                ++chunk;
                next_fold = chunk < p.n_chunks ? p.chunk_hi[chunk] : -1;
            }
        }
        wait_vmcnt<kWait>();
        __builtin_amdgcn_s_waitcnt(0xC07F);
        lds_barrier();
    };
    for (int ks = ks_lo; ks < ks_hi; ks += D) {
        unrolled_while(
            [&](auto i_c) {
                if (ks + decltype(i_c)::value >= ks_hi) return false;
                step(ks + decltype(i_c)::value, i_c);
                return true;
            },
            std::make_integer_sequence<int, D>{});
    }
    wait_vmcnt<0>();  // the copies past the range write LDS; nothing may be in flight at the end
    if constexpr (CHUNKED) {
        fin(tot, wm, wn, lane);  // the last chunk's end flushed the pending block
    } else {
        flush(B1{});
        fin(acc, wm, wn, lane);
    }
}

// The finisher that writes a unit's result to y: wave (wm, wn) holds rows
// m0 + wm * BM / WM and columns n0 + wn * (BN / WN) (GLU: half as many).
template <int BM, bool GLU>
struct StoreY {
    const GemmParams &p;
    const KJob &jb;
    int m0, n0;
    template <int TM, int TN>
    __device__ __forceinline__ void operator()(const f32x16 (&acc)[TM][TN], int wm, int wn, int lane) const {
        constexpr int WM = BM == 64 ? 2 : 4, WN = kWaves / WM;
        store_tile<TM, TN, GLU>(acc, jb, p.t, m0 + wm * (BM / WM), n0 + wn * (128 / WN) / (GLU ? 2 : 1), lane);
    }
};

template <int FMT, bool GLU>
__global__ __launch_bounds__(kThreads, 1) void gemm_q_kernel(GemmParams p) {
    static_assert(FMT == FMT_Q8 || FMT == FMT_Q4, "bf16 weights use gemm_bf16_kernel");
    // one LDS object: the two operand stages, then the block scales of each
    // stage's B rows ([stage][B row][block of the step], f32).  A second
    // __shared__ object would give the LDS accesses alias scopes under which
    // every fragment read waits for the copies in flight.
    __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * (256 + 128) * BK + 2 * 128 * 2 * 2];
    float *scl = reinterpret_cast<float *>(lds + 2 * (256 + 128) * BK);
    int u;
    const int kind = unit_of(p, &u);
    if (kind < 0) return;
    constexpr int cols = big_cols(FMT, GLU);
    Place pl;
    if (kind == 0) {
        if (!place<GLU>(p, u, cols, 0, 0, cols, pl)) return;
        q_unit<FMT, 256, GLU, false>(p, lds, scl, pl.m0, pl.n0, p.job[pl.j], 0, p.nk,
                                     StoreY<256, GLU>{p, p.job[pl.j], pl.m0, pl.n0});
    } else {
        if (!place<GLU>(p, p.small_lo + (u >> 1), cols, (u & 1) * 128, 0, cols, pl)) return;
        q_unit<FMT, 128, GLU, false>(p, lds, scl, pl.m0, pl.n0, p.job[pl.j], 0, p.nk,
                                     StoreY<128, GLU>{p, p.job[pl.j], pl.m0, pl.n0});
    }
}

// Mid-size t (32 < t <= 128): every unit is BM (64 or 128) tokens -- all of
// them -- by 128 weight rows, summed over K in p.n_chunks chunks (q_mid_unit,
// CHUNKED).  The big units run whole, one workgroup each.  When the units
// are one whole round of the compute units plus a few (272 units of the Q4
// verify shape on 256 CUs), those few are split: one workgroup per chunk,
// each writing its chunk sum to p.part in its registers' order; a second,
// small launch (mid_fixup_kernel) adds each split unit's chunk sums in chunk
// order and writes y.  The last round is then 1/n_chunks of a unit long
// instead of a whole unit.  (Completing the units inside the GEMM launch,
// by whichever workgroup finishes a unit's last chunk, needs a device-wide
// release and acquire per workgroup, which write back and invalidate the
// L2: that measured ~50 us per call on the Q4 verify shape.)
// Layout of a chunk sum: float4 ((wave * kQ + (a * TN + n) * 4 + q) * 64 + lane)
// holds acc[a][n][4 q .. 4 q + 3] of that wave and lane, kQ = TM * TN * 4.
template <int BM>
struct PartFin {
    const GemmParams &p;
    int su, chunk;
    template <int TM, int TN>
    __device__ __forceinline__ void operator()(const f32x16 (&acc)[TM][TN], int, int, int lane) const {
        constexpr int kQ = TM * TN * 4;
        const int wave = threadIdx.x >> 6;
        float4 *mine = reinterpret_cast<float4 *>(p.part) + ((int64_t)su * p.n_chunks + chunk) * (BM * 128 / 4) +
                       (wave * kQ) * 64 + lane;
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
            for (int n = 0; n < TN; ++n)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    mine[((a * TN + n) * 4 + q) * 64] =
                        make_float4(acc[a][n][4 * q], acc[a][n][4 * q + 1], acc[a][n][4 * q + 2], acc[a][n][4 * q + 3]);
    }
};

// The split units' chunk sums added in chunk order, starting from zero as
// the whole units' totals do, and stored as the GEMM's wave would have
// stored them.  One thread per float4 of a chunk sum (GLU: the gate's and
// the up projection's float4 of the same outputs), its n_chunks loads issued
// before the additions; 64-thread workgroups, one per (split unit, wave, a,
// n, q) of the chunk-sum layout.
template <int BM, bool GLU>
__global__ __launch_bounds__(64) void mid_fixup_kernel(GemmParams p) {
    constexpr int WM = BM == 64 ? 2 : 4, WN = kWaves / WM;
    constexpr int TM = BM / WM / 32, TN = 128 / WN / 32, kQ = TM * TN * 4;
    constexpr int kGroups = GLU ? kQ / 2 : kQ;  // GLU: n = 0 and n = 1 in one thread
    constexpr int kMaxChunks = 16;
    static_assert(!GLU || TN == 2, "GLU pairs the two 32-column tiles of a wave");
    const int lane = threadIdx.x;
    int g = blockIdx.x;
    const int grp = g % kGroups;
    g /= kGroups;
    const int wave = g % kWaves, su = g / kWaves;
    // grp -> (a, n, q) of the layout (GLU: n = 0 here, n = 1 its partner)
    const int q = grp & 3, an = grp >> 2;
    const int a = GLU ? an : an / TN, n = GLU ? 0 : an % TN;
    Place pl;
    if (!place<GLU>(p, p.n_big + su, big_cols(FMT_Q4, GLU), 0, 0, big_cols(FMT_Q4, GLU), pl)) return;
    const float4 *src = reinterpret_cast<const float4 *>(p.part) + (int64_t)su * p.n_chunks * (BM * 128 / 4) +
                        (wave * kQ) * 64 + lane;
    const int off0 = ((a * TN + n) * 4 + q) * 64, off1 = ((a * TN + 1) * 4 + q) * 64;
    float4 v0[kMaxChunks], v1[kMaxChunks];
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c)
        if (c < p.n_chunks) {
            v0[c] = src[(int64_t)c * (BM * 128 / 4) + off0];
            if constexpr (GLU) v1[c] = src[(int64_t)c * (BM * 128 / 4) + off1];
        }
    float s0[4] = {0.f, 0.f, 0.f, 0.f}, s1[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c)
        if (c < p.n_chunks) {
            s0[0] += v0[c].x, s0[1] += v0[c].y, s0[2] += v0[c].z, s0[3] += v0[c].w;
            if constexpr (GLU) s1[0] += v1[c].x, s1[1] += v1[c].y, s1[2] += v1[c].z, s1[3] += v1[c].w;
        }
    // rows and column of accumulator elements 4 q .. 4 q + 3 (see store_tile)
    const int wm = wave / WN, wn = wave % WN;
    const KJob &jb = p.job[pl.j];
    const int row0 = pl.m0 + wm * (BM / WM) + a * 32 + q * 8 + (lane >> 5) * 4;
    const int col = pl.n0 + wn * (128 / WN) / (GLU ? 2 : 1) + (GLU ? 0 : n * 32) + (lane & 31);
    if (col >= jb.n_out) return;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int row = row0 + e;
        if (row < p.t) jb.y[(int64_t)row * jb.n_out + col] = GLU ? gelu(s0[e]) * s1[e] : s0[e];
    }
}

template <int FMT, int BM, bool GLU>
__global__ __launch_bounds__(kThreads, 1) void gemm_q_mid_kernel(GemmParams p) {
    static_assert(FMT == FMT_Q8 || FMT == FMT_Q4, "bf16 weights use gemm_bf16_kernel");
    // one LDS object, as in gemm_q_kernel
    __shared__ __attribute__((aligned(1024))) uint16_t lds[mid_lds_elems<BM>()];
    int u;
    const int kind = unit_of(p, &u);
    if (kind < 0) return;
    constexpr int cols = big_cols(FMT, GLU);
    Place pl;
    if (kind == 0) {
        if (!place<GLU>(p, u, cols, 0, 0, cols, pl)) return;
        q_mid_unit<FMT, BM, GLU, true>(p, lds, pl.m0, pl.n0, p.job[pl.j], 0, p.nk,
                                       StoreY<BM, GLU>{p, p.job[pl.j], pl.m0, pl.n0});
    } else {
        const int su = u / p.n_chunks, c = u - su * p.n_chunks;
        if (!place<GLU>(p, p.n_big + su, cols, 0, 0, cols, pl)) return;
        const int lo = c ? p.chunk_hi[c - 1] : 0, hi = p.chunk_hi[c];
        q_mid_unit<FMT, BM, GLU, false>(p, lds, pl.m0, pl.n0, p.job[pl.j], lo, hi, PartFin<BM>{p, su, c});
    }
}

// ------------------------------------------------ Q4 mid units on 4 waves
// The Q4 mid unit of 64 tokens x 128 weight rows, laid out like the
// matrix-core decode kernel's operands: four waves, wave w the unit's rows
// 32 w .. 32 w + 31 as two 16-row weight tiles, 16x16x32 MFMAs (K = 32 = one
// quantisation block).  Every K step (128 elements: one 1 KiB segment of the
// tile-major code plane per weight tile) goes into LDS by buffer-load DMA
// only -- x's tile, the wave's two code segments and their tiled scales --
// so no global load returns into registers and every wait for a copy is
// the explicit one before the step's barrier; the copies run two steps
// ahead through three stages.  A wave reads its codes back (lane 16 g + n:
// row n, block g of the segment), transposes dwords across the lane groups
// so that group g holds elements 8 g .. 8 g + 7 of every block, converts
// them to exact bf16 (16 (code - 8)) and issues one MFMA per (16-token tile,
// weight tile, block); each block's f32 result is multiplied by its scale
// (f16 / 16, exact) into the accumulators.  A wave reads each x fragment
// once per step and uses it for both of its weight tiles: the LDS reads per
// MFMA are half those of the 8-wave unit above, whose fragment reads kept
// the LDS busy over half of the kernel's cycles; and at 75 KiB of LDS two
// workgroups share a CU.  Like the 8-wave unit, a whole unit sums K in
// p.n_chunks chunks and adds them in order, which is what the fixup does
// for the split units, so a unit's result does not depend on the split.
constexpr int kM2Waves = 4;  // waves across a unit's 128 weight rows (32 each)
constexpr int kM2Threads = 64 * kM2Waves;
constexpr int kM2Stages = 3;  // LDS stages: the copies of step ks + 2 land while step ks computes
constexpr int kM2CodeBytes = kM2Waves * 2 * 1024;  // per stage: each wave's two code segments
constexpr int kM2SclBytes = kM2Waves * 2 * 128;    // per stage: their 16 x 4 tiled scales
// The stages are six LDS objects: x's tile of stage i, and the codes then
// the scales of stage i.  Separate objects give each access an alias scope,
// so the compiler waits before a read of one stage only for the copies into
// that stage (which the step's own wait has covered), not for the copies in
// flight into the others.
template <int BM>
struct M2Lds {
    uint8_t *a[kM2Stages];  // BM x kMidBK bf16
    uint8_t *c[kM2Stages];  // kM2CodeBytes of codes, then kM2SclBytes of scales
};

// Dword d of lane group m -> dword m of lane group d (lanes keep l % 16).
__device__ __forceinline__ void xpose4(uint32_t &d0, uint32_t &d1, uint32_t &d2, uint32_t &d3) {
    // lanes 32..63 of the first operand trade places with lanes 0..31 of the second
    const auto a = __builtin_amdgcn_permlane32_swap(d0, d2, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(d1, d3, false, false);
    // odd 16-lane rows of the first operand trade places with even rows of the second
    const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    const auto e = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    d0 = c[0];
    d1 = c[1];
    d2 = e[0];
    d3 = e[1];
}

// 8 Q4 codes of one dword (element 2 e in the low nibble of byte e, stored
// as the 4-bit two's complement of code - 8) -> bf16 16 (code - 8), in order.
__device__ __forceinline__ bf16x8 q4_dword_bf16(uint32_t d) {
    const uint32_t lo = (d << 4) & 0xF0F0F0F0u;  // byte e: 16 (code 2 e - 8) as an int8
    const uint32_t hi = d & 0xF0F0F0F0u;         // byte e: 16 (code 2 e + 1 - 8)
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack_bf16((float)(int8_t)(lo >> (8 * e)), (float)(int8_t)(hi >> (8 * e)));
    return __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
}

// 16 / 4 bytes per lane from a buffer straight into LDS: lane l's bytes land
// at dst + 16 l / 4 l (dst wave-uniform); reads past the buffer write zeros.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint8_t *dst, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t r, uint8_t *dst, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 4, off, 0, 0, 0);
}

template <int BM, bool CHUNKED, class Fin>
__device__ __forceinline__ void q4_mid2_unit(const GemmParams &p, const M2Lds<BM> &lds, int m0, int n0,
                                             const KJob &jb, int ks_lo, int ks_hi, Fin &&fin) {
    constexpr int BKM = kMidBK;
    constexpr int TMT = BM / 16;                                 // 16-token tiles
    constexpr int kChunksA = BM * (BKM / 8) / kM2Threads;        // x copies per thread and step
    constexpr int kPer = kChunksA + 3;                           // copies per thread and step
    static_assert(BM == 64 && kChunksA >= 1 && BKM == 128 && kPer < 64, "unit shape");
    const int n_in = p.n_in;
    const int nb = n_in / kBlock, nb4 = (nb + 3) / 4;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // weight rows 32 wave ..
    const int ln = lane & 15, lg = lane >> 4;

    const int a_rows = min(BM, p.t - m0);
    const int b_rows = min(128, jb.n_out - n0);
    const uint32_t row2 = (uint32_t)n_in * 2u;
    const __amdgpu_buffer_rsrc_t ars = make_rsrc(p.xb + (int64_t)m0 * n_in, (uint32_t)a_rows * row2);
    // the unit's 8 weight tiles of codes and of tiled scales (past the job's
    // last tile, and past the last segment of the last tile, the copies read 0)
    const __amdgpu_buffer_rsrc_t crs =
        make_rsrc(static_cast<const uint8_t *>(jb.codes) + (n0 >> 4) * q4_plane_bytes(16, nb),
                  (uint32_t)q4_plane_bytes(b_rows, nb));
    const __amdgpu_buffer_rsrc_t srs =
        make_rsrc(static_cast<const uint8_t *>(jb.scales_t) + (int64_t)(n0 >> 4) * nb4 * 64 * 2,
                  (uint32_t)tiled_scale_count(b_rows, nb) * 2u);
    // this wave's segment of tile j and step ks: (2 wave + j) nb4 + ks; lane
    // 16 g + n copies row n, block g (16 bytes) of it
    const uint32_t code_lane = ((uint32_t)ln << 6) + ((uint32_t)lg << 4);
    const uint32_t seg0 = (uint32_t)(2 * wave) * (uint32_t)nb4;
    // scales: lanes 0..31 copy tile 0's 128 bytes, lanes 32..63 tile 1's
    const uint32_t scl_lane = ((seg0 + (uint32_t)(lane >> 5) * (uint32_t)nb4) << 7) + ((uint32_t)(lane & 31) << 2);
    // x's tile: copy i of this thread is 16-byte chunk u = (wave kChunksA +
    // i) 64 + lane of the stage, row u / 16, holding chunk (u % 16) ^ (row % 16)
    uint32_t offa[kChunksA];
    int ka[kChunksA];
#pragma unroll
    for (int i = 0; i < kChunksA; ++i) {
        const int u = (wave * kChunksA + i) * 64 + lane, r = u >> 4;
        ka[i] = ((u & 15) ^ (r & 15)) * 8;
        offa[i] = (uint32_t)r * row2 + (uint32_t)ka[i] * 2u;
    }
    auto issue = [&](int ks, auto st_c) {
        constexpr int ST = decltype(st_c)::value;
        uint8_t *sa = lds.a[ST];
        const int k0 = ks * BKM;
        // (a select, not a branch around two sets of copies: copies issued on
        // two paths make the compiler's wait counts after the join conservative)
#pragma unroll
        for (int i = 0; i < kChunksA; ++i)
            lds_dma16(ars, sa + (wave * kChunksA + i) * 1024, k0 + ka[i] < n_in ? offa[i] + (uint32_t)k0 * 2u : kOut);
        uint8_t *cb = lds.c[ST] + wave * 2048;
        lds_dma16(crs, cb, ((seg0 + (uint32_t)ks) << 10) + code_lane);
        lds_dma16(crs, cb + 1024, ((seg0 + (uint32_t)nb4 + (uint32_t)ks) << 10) + code_lane);
        lds_dma4(srs, lds.c[ST] + kM2CodeBytes + wave * 256, scl_lane + ((uint32_t)ks << 7));
    };

    f32x4 acc[TMT][2], tot[CHUNKED ? TMT : 1][CHUNKED ? 2 : 1];
#pragma unroll
    for (int i = 0; i < TMT; ++i) acc[i][0] = acc[i][1] = (f32x4){};
    if constexpr (CHUNKED) {
#pragma unroll
        for (int i = 0; i < TMT; ++i) tot[i][0] = tot[i][1] = (f32x4){};
    }
    int chunk = 0;
    int next_fold = CHUNKED ? p.chunk_hi[0] : 0;

    auto compute = [&](auto st_c) {
        constexpr int ST = decltype(st_c)::value;
        const uint16_t *As = reinterpret_cast<const uint16_t *>(lds.a[ST]);
        const uint4 *cw = reinterpret_cast<const uint4 *>(lds.c[ST] + wave * 2048);
        uint4 c0 = cw[lane], c1 = cw[64 + lane];
        const uint2 *sw = reinterpret_cast<const uint2 *>(lds.c[ST] + kM2CodeBytes + wave * 256);
        const uint2 h0 = sw[ln], h1 = sw[16 + ln];  // row n's four block scales of each tile (f16)
        xpose4(c0.x, c0.y, c0.z, c0.w);
        xpose4(c1.x, c1.y, c1.z, c1.w);
        const uint32_t cd[2][4] = {{c0.x, c0.y, c0.z, c0.w}, {c1.x, c1.y, c1.z, c1.w}};
        const uint32_t hd[2][2] = {{h0.x, h0.y}, {h1.x, h1.y}};
        f32x4 part[2][TMT][2];
        float sc[2][2];
        // block b: the MFMAs into part[b & 1], then block b - 1's scaling,
        // whose MFMA results are ready by then
        auto scale_in = [&](int pb) {
#pragma unroll
            for (int i = 0; i < TMT; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][j][e] = fmaf(sc[pb][j], part[pb][i][j][e], acc[i][j][e]);
        };
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const bf16x8 bq0 = q4_dword_bf16(cd[0][b]), bq1 = q4_dword_bf16(cd[1][b]);
#pragma unroll
            for (int i = 0; i < TMT; ++i) {
                const int r = 16 * i + ln;
                const bf16x8 fa = *reinterpret_cast<const bf16x8 *>(As + r * BKM + (((4 * b + lg) ^ ln) << 3));
                part[b & 1][i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, bq0, (f32x4){}, 0, 0, 0);
                part[b & 1][i][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, bq1, (f32x4){}, 0, 0, 0);
            }
            if (b > 0) scale_in((b - 1) & 1);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint32_t h = hd[j][b >> 1] >> ((b & 1) * 16);
                sc[b & 1][j] = (float)__builtin_bit_cast(_Float16, (uint16_t)h) * 0.0625f;  // codes carry * 16; exact
            }
        }
        scale_in(1);
    };

    // step ks = ks_lo + 3 q + I uses stage I; the loop is unrolled three
    // times so that every stage offset is a constant (with run-time offsets
    // the compiler cannot tell the copies' LDS range from the one a step
    // reads, and waits for every copy in flight before the first read)
    auto step = [&](int ks, auto i_c) {
        constexpr int I = decltype(i_c)::value;
        wait_vmcnt<kPer>();  // this step's copies have landed (the next step's may not)
        lds_barrier();       // ... every wave's; and every wave is done with step ks - 1
        issue(ks + 2, std::integral_constant<int, (I + 2) % kM2Stages>{});  // into step ks - 1's stage
        compute(i_c);
        if constexpr (CHUNKED) {
            if (ks + 1 == next_fold) {  // the last step of chunk `chunk`
#pragma unroll
                for (int i = 0; i < TMT; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        tot[i][j] += acc[i][j];
                        acc[i][j] = (f32x4){};
                    }
                ++chunk;
                next_fold = chunk < p.n_chunks ? p.chunk_hi[chunk] : -1;
            }
        }
    };
    issue(ks_lo, std::integral_constant<int, 0>{});
    issue(ks_lo + 1, std::integral_constant<int, 1>{});
    // (a partial last round leaves the loop rather than going round to its
    // head, so that the head is reached from one place in the loop only)
    for (int ks = ks_lo;; ks += kM2Stages) {
        bool more = true;
        unrolled_while(
            [&](auto i_c) {
                if (ks + decltype(i_c)::value >= ks_hi) return more = false;
                step(ks + decltype(i_c)::value, i_c);
                return true;
            },
            std::make_integer_sequence<int, kM2Stages>{});
        if (!more) break;
    }
    wait_vmcnt<0>();  // the copies past the range write LDS; nothing may be in flight at the end
    if constexpr (CHUNKED) fin(tot, wave, lane);
    else fin(acc, wave, lane);
}

// y from a 4-wave unit: tile (i, j) of wave w, lane l holds rows
// m0 + 16 i + 4 (l / 16) + e of column n0 + 32 w + 16 j + l % 16.
template <int BM>
struct StoreY2 {
    const GemmParams &p;
    const KJob &jb;
    int m0, n0;
    template <int TMT>
    __device__ __forceinline__ void operator()(const f32x4 (&acc)[TMT][2], int wave, int lane) const {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + 32 * wave + 16 * j + (lane & 15);
            if (col >= jb.n_out) continue;
#pragma unroll
            for (int i = 0; i < TMT; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = m0 + 16 * i + 4 * (lane >> 4) + e;
                    if (row < p.t) jb.y[(int64_t)row * jb.n_out + col] = acc[i][j][e];
                }
        }
    }
};

// A split 4-wave unit's chunk sum: float4 ((wave * TMT + i) * 2 + j) * 64 + lane
// of the chunk's BM * 128 floats holds acc[i][j] of that wave and lane.
template <int BM>
struct PartFin2 {
    const GemmParams &p;
    int su, chunk;
    template <int TMT>
    __device__ __forceinline__ void operator()(const f32x4 (&acc)[TMT][2], int wave, int lane) const {
        float4 *mine = reinterpret_cast<float4 *>(p.part) + ((int64_t)su * p.n_chunks + chunk) * (BM * 128 / 4) +
                       (wave * TMT * 2) * 64 + lane;
#pragma unroll
        for (int i = 0; i < TMT; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                mine[(i * 2 + j) * 64] = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
    }
};

// The split 4-wave units' chunk sums added in chunk order from zero, as a
// whole unit adds its chunks, and stored as StoreY2 would have.  One thread
// per float4 of a chunk sum; one 64-thread workgroup per (split unit, wave,
// i, j).
template <int BM>
__global__ __launch_bounds__(64) void mid2_fixup_kernel(GemmParams p) {
    constexpr int TMT = BM / 16, kGroups = TMT * 2, kMaxChunks = 16;
    const int lane = threadIdx.x;
    int g = blockIdx.x;
    const int grp = g % kGroups;
    g /= kGroups;
    const int wave = g % kM2Waves, su = g / kM2Waves;
    const int i = grp >> 1, j = grp & 1;
    Place pl;
    if (!place<false>(p, p.n_big + su, big_cols(FMT_Q4, false), 0, 0, big_cols(FMT_Q4, false), pl)) return;
    const float4 *src = reinterpret_cast<const float4 *>(p.part) + (int64_t)su * p.n_chunks * (BM * 128 / 4) +
                        (wave * kGroups + grp) * 64 + lane;
    float4 v[kMaxChunks];
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c)
        if (c < p.n_chunks) v[c] = src[(int64_t)c * (BM * 128 / 4)];
    float sum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c)
        if (c < p.n_chunks) sum[0] += v[c].x, sum[1] += v[c].y, sum[2] += v[c].z, sum[3] += v[c].w;
    const KJob &jb = p.job[pl.j];
    const int col = pl.n0 + 32 * wave + 16 * j + (lane & 15);
    if (col >= jb.n_out) return;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int row = pl.m0 + 16 * i + 4 * (lane >> 4) + e;
        if (row < p.t) jb.y[(int64_t)row * jb.n_out + col] = sum[e];
    }
}

template <int BM>
__global__ __launch_bounds__(kM2Threads, 2) void gemm_q4_mid2_kernel(GemmParams p) {
    constexpr int kA = BM * kMidBK * 2, kC = kM2CodeBytes + kM2SclBytes;
    __shared__ __attribute__((aligned(1024))) uint8_t a0[kA], a1[kA], a2[kA];
    __shared__ __attribute__((aligned(1024))) uint8_t c0[kC], c1[kC], c2[kC];
    static_assert(kM2Stages == 3, "three stages");
    const M2Lds<BM> lds{{a0, a1, a2}, {c0, c1, c2}};
    int u;
    const int kind = unit_of(p, &u);
    if (kind < 0) return;
    constexpr int cols = big_cols(FMT_Q4, false);
    Place pl;
    if (kind == 0) {
        if (!place<false>(p, u, cols, 0, 0, cols, pl)) return;
        q4_mid2_unit<BM, true>(p, lds, pl.m0, pl.n0, p.job[pl.j], 0, p.nk, StoreY2<BM>{p, p.job[pl.j], pl.m0, pl.n0});
    } else {
        const int su = u / p.n_chunks, c = u - su * p.n_chunks;
        if (!place<false>(p, p.n_big + su, cols, 0, 0, cols, pl)) return;
        const int lo = c ? p.chunk_hi[c - 1] : 0, hi = p.chunk_hi[c];
        q4_mid2_unit<BM, false>(p, lds, pl.m0, pl.n0, p.job[pl.j], lo, hi, PartFin2<BM>{p, su, c});
    }
}

// --------------------------------------------------------------- bf16 units
// A BM x BN tile of bf16 weights on 8 waves (WM x WN grid); both operand
// tiles copied from L2 into LDS by the load unit.  A stage holds the A tile
// (BM rows) then the B tile (BN rows) of one K step, 16-byte chunks swizzled
// as above; instruction i of an issuing wave w fills chunks
// (w * kLoads + i) * 64 + lane of a tile, whose global address each lane
// computes once.
template <int BM, int BN, int WM, int WN, bool GLU>
__device__ __forceinline__ void bf16_unit(const GemmParams &p, uint16_t *lds, int m0, int n0, const KJob &jb) {
    static_assert(WM * WN == kWaves, "8 waves");
    constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
    constexpr int kCols = GLU ? BN / 2 : BN;
    constexpr int kStage = (BM + BN) * BK;  // bf16 elements
    static_assert(!GLU || TN == 2, "GLU pairs the two 32-column tiles of a wave");
    // Who copies: a wave stalls while the CU's load unit drains the copies it
    // issues (~850 cycles of a ~3400-cycle K step when all 8 waves issue
    // theirs at once after the barrier), and its SIMD's matrix core idles
    // if the other wave there is stalled too.  So only waves 0..3, one per
    // SIMD, issue the copies while waves 4..7 start on their MFMAs: 3459 ->
    // 3159 cycles per K step on the 256 x 256 tile.
    constexpr int kIssuers = 4;
    constexpr int kLA = BM * BK / 8 / 64 / kIssuers, kLB = BN * BK / 8 / 64 / kIssuers;
    static_assert(kLA >= 1 && kLB >= 1, "copy split");
    const int n_in = p.n_in;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    const uint32_t row2 = (uint32_t)n_in * 2u;
    const int a_rows = min(BM, p.t - m0), b_rows = min(kCols, jb.n_out - n0);
    const __amdgpu_buffer_rsrc_t ars = make_rsrc(p.xb + (int64_t)m0 * n_in, (uint32_t)a_rows * row2);
    const __amdgpu_buffer_rsrc_t brs =
        make_rsrc(static_cast<const uint16_t *>(jb.codes) + (int64_t)n0 * n_in, (uint32_t)b_rows * row2);
    const __amdgpu_buffer_rsrc_t brs2 =
        GLU ? make_rsrc(static_cast<const uint16_t *>(p.job[1].codes) + (int64_t)n0 * n_in, (uint32_t)b_rows * row2)
            : brs;

    // this lane's chunk of each load: tile row r (8 chunks per row), chunk
    // c = slot ^ key(r); GLU: B-tile row v is row (v / 64) 32 + v % 32 of the
    // gate ((v / 32) even) or up projection -- 8-row blocks never straddle
    // a 32-row group, so the choice is uniform per instruction
    const bool issuer = wave < kIssuers;
    const int iw = issuer ? wave : 0;
    uint32_t offa[kLA], offb[kLB];
    int ka[kLA], kb[kLB];
#pragma unroll
    for (int i = 0; i < kLA; ++i) {
        const int u = (iw * kLA + i) * 64 + lane, r = u >> 3;
        ka[i] = ((u & 7) ^ swz_key(r)) * 8;
        offa[i] = (uint32_t)r * row2 + (uint32_t)ka[i] * 2u;
    }
#pragma unroll
    for (int i = 0; i < kLB; ++i) {
        const int u = (iw * kLB + i) * 64 + lane, v = u >> 3;
        kb[i] = ((u & 7) ^ swz_key(v)) * 8;
        const int wr = GLU ? (v >> 6) * 32 + (v & 31) : v;
        offb[i] = (uint32_t)wr * row2 + (uint32_t)kb[i] * 2u;
    }
    auto issue = [&](int st, int k0) {
        if (!issuer) return;
        uint16_t *As = lds + st * kStage, *Bs = As + BM * BK;
#pragma unroll
        for (int i = 0; i < kLA; ++i)
            lds_load16(ars, As + (iw * kLA + i) * 64 * 8, k0 + ka[i] < n_in ? offa[i] + (uint32_t)k0 * 2u : kOut);
#pragma unroll
        for (int i = 0; i < kLB; ++i) {
            const bool up = GLU && ((((iw * kLB + i) * 8) >> 5) & 1);
            lds_load16(up ? brs2 : brs, Bs + (iw * kLB + i) * 64 * 8,
                       k0 + kb[i] < n_in ? offb[i] + (uint32_t)k0 * 2u : kOut);
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int n = 0; n < TN; ++n) acc[a][n] = (f32x16){};
    const int frow = lane & 31;
    const int fkey = swz_key(frow);
    const int a_base = (wm * (BM / WM) + frow) * BK;
    const int b_base = (wn * (BN / WN) + frow) * BK;
    auto compute = [&](int st) {
        const uint16_t *As = lds + st * kStage, *Bs = As + BM * BK;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int slot = (kk * 2 + (lane >> 5)) ^ fkey;
            bf16x8 fa[TM], fb[TN];
#pragma unroll
            for (int a = 0; a < TM; ++a) fa[a] = *reinterpret_cast<const bf16x8 *>(As + a_base + a * 32 * BK + slot * 8);
#pragma unroll
            for (int n = 0; n < TN; ++n) fb[n] = *reinterpret_cast<const bf16x8 *>(Bs + b_base + n * 32 * BK + slot * 8);
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int n = 0; n < TN; ++n)
                    acc[a][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[n], acc[a][n], 0, 0, 0);
        }
    };

    // step ks computes stage ks & 1 while step ks + 1's tiles land in the
    // other; the wait + barrier at the end of a step publishes them and
    // frees the stage just read for the next issue
    const int nk = (n_in + BK - 1) / BK;
    issue(0, 0);
    wait_vmcnt<0>();
    lds_barrier();
    for (int ks = 0; ks < nk; ++ks) {
        if (ks + 1 < nk) issue((ks + 1) & 1, (ks + 1) * BK);
        compute(ks & 1);
        wait_vmcnt<0>();
        lds_barrier();
    }
    store_tile<TM, TN, GLU>(acc, jb, p.t, m0 + wm * (BM / WM), n0 + wn * (BN / WN) / (GLU ? 2 : 1), lane);
}

template <bool GLU>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(GemmParams p) {
    __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * (256 + 256) * BK];
    int u;
    const int kind = unit_of(p, &u);
    if (kind < 0) return;
    constexpr int cols = big_cols(FMT_BF16, GLU);
    Place pl;
    if (kind == 0) {
        if (!place<GLU>(p, u, cols, 0, 0, cols, pl)) return;
        bf16_unit<256, 256, 2, 4, GLU>(p, lds, pl.m0, pl.n0, p.job[pl.j]);
    } else {
        // quarter q of big tile small_lo + u / 4: tokens (q / 2) * 128, columns (q % 2) * cols / 2
        const int q = u & 3;
        if (!place<GLU>(p, p.small_lo + (u >> 2), cols, (q >> 1) * 128, q & 1, cols / 2, pl)) return;
        bf16_unit<128, 128, 4, 2, GLU>(p, lds, pl.m0, pl.n0, p.job[pl.j]);
    }
}

template <int FMT, bool GLU>
hipError_t launch_plan(GemmParams p, int cu_count, hipStream_t s) {
    const int units = p.tiles_m * p.tn0[kMaxJobs];
    // Whole rounds of big units (one per compute unit at a time); what is
    // left over, less than one round, runs as small units so that the last
    // round is short instead of mostly idle.  With fewer big units than
    // compute units: bf16 runs them all as quarters; Q8/Q4 as halves, or as
    // quarters when those still fit in one round (the Q4 prefill's 224
    // halves ran in ~92 us against ~101 us for 448 quarters in 1.75 rounds).
    constexpr int split = FMT == FMT_BF16 ? 4 : 2;  // small units per big one
    if (units >= cu_count) {
        p.n_big = units / cu_count * cu_count;
        p.small_lo = p.n_big;
        p.n_small = split * (units - p.n_big);
    } else if (FMT == FMT_BF16 || split * units <= cu_count) {
        p.n_big = 0;
        p.small_lo = 0;
        p.n_small = split * units;
    } else {
        p.n_big = units;
        p.small_lo = units;
        p.n_small = 0;
    }
    p.big_per_xcd = (p.n_big + kXcds - 1) / kXcds;
    p.small_per_xcd = (p.n_small + kXcds - 1) / kXcds;
    const dim3 grid(kXcds * (p.big_per_xcd + p.small_per_xcd));
    if (grid.x == 0) return hipSuccess;
    if constexpr (FMT == FMT_BF16)
        hipLaunchKernelGGL((gemm_bf16_kernel<GLU>), grid, dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((gemm_q_kernel<FMT, GLU>), grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

// t <= kVerifyMaxT runs the matrix-core decode kernel's wide mode, which
// rounds x itself up to kWideF32MaxT tokens and reads the bf16 copy of x
// beyond.  Q8/Q4 at kVerifyMaxT < t <= kMidMaxT run the mid plan (units that
// hold every token); larger t and bf16 weights the big/small tile plan.
// IL_PREFILL pins the kernel: gemm (the GEMM the shape would take: mid plan
// or tiles), tiles (the big/small tile plan even where the mid plan would
// run), verify (wide mode; up to kVerifySliceMaxT tokens as even slices of at
// most kVerifyMaxT).
struct Route {
    bool verify;
    int slice;   // tokens per wide-mode launch
    int mid_bm;  // GEMM of mid-size t: tokens per unit (64 or 128), else 0
};
Route route(int fmt, int t, int n_in, const KJob *jobs, int n_jobs, bool glu) {
    bool verify = t <= kVerifyMaxT, tiles = false;
    if (const char *force = getenv("IL_PREFILL")) {
        if (!strcmp(force, "gemm")) verify = false;
        if (!strcmp(force, "tiles")) verify = false, tiles = true;
        if (!strcmp(force, "verify")) verify = t <= kVerifySliceMaxT;
    }
    const int n_slices = (t + kVerifyMaxT - 1) / kVerifyMaxT;
    const int slice = (t + n_slices - 1) / n_slices;  // > kWideF32MaxT when t > kVerifyMaxT
    verify = verify && verify_mfma_fits(fmt, slice, n_in, jobs, n_jobs);
    int mid_bm = 0;
    if (!verify && !tiles && fmt != FMT_BF16 && t <= kMidMaxT) mid_bm = t <= 64 && !glu ? 64 : 128;
    return {verify, slice, mid_bm};
}

// The mid plan's scratch after the bf16 copy of x: the split units' chunk
// sums (after 256 bytes kept free).
constexpr int kMidChunks = 16;   // K chunks of a mid unit (fewer when K has fewer steps)
constexpr int kMidMaxSplit = 16;  // units split per launch, at most
size_t mid_extra_bytes(int mid_bm) { return 256 + (size_t)kMidMaxSplit * kMidChunks * mid_bm * 128 * 4; }
size_t xb_bytes(int t, int n_in) { return ((size_t)t * (size_t)n_in * 2 + 255) / 256 * 256; }

template <int FMT, bool GLU>
hipError_t launch_mid(GemmParams p, int mid_bm, int cu_count, hipStream_t s) {
    // units: one 128-row column of a job each (tiles_m == 1); whole rounds of
    // units run whole, and a last partial round of at most cu_count /
    // n_chunks units is split into chunks
    const int units = p.tn0[kMaxJobs];
    const int left = units % cu_count;
    const int n_split = left > 0 && left * p.n_chunks <= cu_count && left <= kMidMaxSplit && units >= cu_count ? left : 0;
    p.mid_bm = mid_bm;
    p.n_big = units - n_split;
    p.small_lo = p.n_big;
    p.n_small = n_split * p.n_chunks;
    p.big_per_xcd = (p.n_big + kXcds - 1) / kXcds;
    p.small_per_xcd = (p.n_small + kXcds - 1) / kXcds;
    const dim3 grid(kXcds * (p.big_per_xcd + p.small_per_xcd));
    if (grid.x == 0) return hipSuccess;
    // the fixup's workgroups: (split unit, wave, float4 group of the chunk-sum layout)
    const int groups = mid_bm == 64 ? 4 : (GLU ? 4 : 8);
    const dim3 fix((unsigned)(n_split * kWaves * groups));
    if (mid_bm == 64) {
        if constexpr (FMT == FMT_Q4 && !GLU) {
            // the 4-wave units; their fixup: (split unit, wave, tile pair)
            hipLaunchKernelGGL((gemm_q4_mid2_kernel<64>), grid, dim3(kM2Threads), 0, s, p);
            if (n_split)
                hipLaunchKernelGGL((mid2_fixup_kernel<64>), dim3((unsigned)(n_split * kM2Waves * 8)), dim3(64), 0, s, p);
        } else if constexpr (!GLU) {
            hipLaunchKernelGGL((gemm_q_mid_kernel<FMT, 64, false>), grid, dim3(kThreads), 0, s, p);
            if (n_split) hipLaunchKernelGGL((mid_fixup_kernel<64, false>), fix, dim3(64), 0, s, p);
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        hipLaunchKernelGGL((gemm_q_mid_kernel<FMT, 128, GLU>), grid, dim3(kThreads), 0, s, p);
        if (n_split) hipLaunchKernelGGL((mid_fixup_kernel<128, GLU>), fix, dim3(64), 0, s, p);
    }
    return hipGetLastError();
}

// The buffer of il_matmul_noalloc's prefill path: one per device, for
// callers that cannot allocate.  `scratch` names the host-side stand-in of
// the array; kernels get its device address from static_scratch().
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
constexpr int kMaxScratchDevices = 64;
struct StaticScratch {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};
StaticScratch g_static_scratch[kMaxScratchDevices];

}  // namespace

size_t static_scratch_bytes() { return kStaticScratchBytes; }

hipError_t static_scratch(int device, void **ptr) {
    *ptr = nullptr;
    if (device < 0 || device >= kMaxScratchDevices) return hipErrorInvalidDevice;
    StaticScratch &st = g_static_scratch[device];
    // once per device, with that device current (the caller's)
    std::call_once(st.once, [&] { st.err = hipGetSymbolAddress(&st.ptr, HIP_SYMBOL(scratch)); });
    if (st.err == hipSuccess) *ptr = st.ptr;
    return st.err;
}

size_t gemm_scratch_bytes(int fmt, int t, int n_in, const KJob *jobs, int n_jobs, bool glu) {
    if (t <= kGemvMaxT || n_jobs < 1) return 0;
    const Route r = route(fmt, t, n_in, jobs, n_jobs, glu);
    if (r.verify && t <= kWideF32MaxT) return 0;
    return xb_bytes(t, n_in) + (r.mid_bm ? mid_extra_bytes(r.mid_bm) : 0);
}

hipError_t launch_gemm(int fmt, const float *x, void *xb_scratch, int t, int n_in, const KJob *jobs, int n_jobs,
                       int cu_count, hipStream_t s, bool glu, hipEvent_t after_prepass) {
    if (t < 1 || n_jobs < 1 || n_jobs > kMaxJobs || n_in % kBlock || cu_count < 1) return hipErrorInvalidValue;
    if (glu && (n_jobs != 2 || jobs[0].n_out != jobs[1].n_out)) return hipErrorInvalidValue;
    // every buffer descriptor (256 rows of x or of a weight) must stay below 2^31 bytes
    if ((int64_t)kBigM * n_in * 2 >= (1ll << 31)) return hipErrorInvalidValue;
    const Route r = route(fmt, t, n_in, jobs, n_jobs, glu);
    if (r.verify && t <= kWideF32MaxT) return launch_verify_mfma(fmt, x, nullptr, t, n_in, jobs, n_jobs, cu_count, s, glu);
    if (!xb_scratch) return hipErrorInvalidValue;

    // x -> bf16 into the caller's scratch
    const int64_t n8 = (int64_t)t * n_in / 8;
    uint16_t *xb = static_cast<uint16_t *>(xb_scratch);
    const int64_t pre_wgs = std::min<int64_t>((n8 + 256 * kPreGroups - 1) / (256 * kPreGroups),
                                              (int64_t)cu_count * kPreWgPerCu);
    hipLaunchKernelGGL(x_to_bf16_kernel, dim3((unsigned)pre_wgs), dim3(256), 0, s, x, reinterpret_cast<uint4 *>(xb), n8);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && after_prepass) e = hipEventRecord(after_prepass, s);
    if (e != hipSuccess) return e;
    if (r.verify) {
        // one launch per slice of tokens; slice i's x rows and y rows start
        // slice * i rows in
        for (int t0 = 0; t0 < t && e == hipSuccess; t0 += r.slice) {
            const int tt = min(r.slice, t - t0);
            KJob js[kMaxJobs];
            for (int j = 0; j < n_jobs; ++j) {
                js[j] = jobs[j];
                js[j].y = jobs[j].y + (int64_t)t0 * jobs[j].n_out;
            }
            e = launch_verify_mfma(fmt, x + (int64_t)t0 * n_in, xb + (int64_t)t0 * n_in, tt, n_in, js, n_jobs,
                                   cu_count, s, glu);
        }
        return e;
    }
    GemmParams p{};
    p.xb = xb;
    p.t = t;
    p.n_in = n_in;
    p.n_jobs = n_jobs;
    p.tiles_m = (t + kBigM - 1) / kBigM;
    p.nk = r.mid_bm ? (n_in + kMidBK - 1) / kMidBK : (n_in + BK - 1) / BK;
    p.n_chunks = p.nk < kMidChunks ? p.nk : kMidChunks;
    for (int c = 0; c < p.n_chunks; ++c) p.chunk_hi[c] = (int)((int64_t)p.nk * (c + 1) / p.n_chunks);
    if (r.mid_bm) p.part = reinterpret_cast<float *>(static_cast<uint8_t *>(xb_scratch) + xb_bytes(t, n_in) + 256);
    const int cols = big_cols(fmt, glu);
    int tn = 0;
    for (int j = 0; j < n_jobs; ++j) {
        p.job[j] = jobs[j];
        p.tn0[j] = tn;
        // GLU: units over the gate's rows only (each also covers the up rows)
        if (!glu || j == 0) tn += (jobs[j].n_out + cols - 1) / cols;
    }
    for (int j = glu ? 1 : n_jobs; j <= kMaxJobs; ++j) p.tn0[j] = tn;
    if (r.mid_bm) {
        switch (fmt) {
            case FMT_Q8: return glu ? launch_mid<FMT_Q8, true>(p, r.mid_bm, cu_count, s) : launch_mid<FMT_Q8, false>(p, r.mid_bm, cu_count, s);
            case FMT_Q4: return glu ? launch_mid<FMT_Q4, true>(p, r.mid_bm, cu_count, s) : launch_mid<FMT_Q4, false>(p, r.mid_bm, cu_count, s);
            default: return hipErrorInvalidValue;
        }
    }
    switch (fmt) {
        case FMT_BF16: return glu ? launch_plan<FMT_BF16, true>(p, cu_count, s) : launch_plan<FMT_BF16, false>(p, cu_count, s);
        case FMT_Q8: return glu ? launch_plan<FMT_Q8, true>(p, cu_count, s) : launch_plan<FMT_Q8, false>(p, cu_count, s);
        case FMT_Q4: return glu ? launch_plan<FMT_Q4, true>(p, cu_count, s) : launch_plan<FMT_Q4, false>(p, cu_count, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace il
