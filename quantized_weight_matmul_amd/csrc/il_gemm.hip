// il_gemm.hip -- prefill GEMM for t > 8 on the gfx950 bf16 matrix cores.
//
// Computes y[t][n_out] = bf16(x)[t][n_in] * W^T with f32 accumulation for
// every job of one format in one launch (the batch of `struct Job`s over one
// shared x that Backend::matmul on the oxinfer 0.0.0 src/gpu.rs page submits
// at once).  x is rounded to bf16 (round-to-nearest-even) by a pre-pass into
// a stream-ordered scratch buffer; bf16 weights are used as stored; Q8/Q4
// weights are dequantised to their exact f32 value (Q8: q*scale rounded to
// f32, Q4: (code-8)*scale, exact) and rounded to bf16 as they are written to
// LDS, ahead of the MFMAs.
//
// Tiling: a workgroup of 8 waves (two per SIMD) owns a 256 x 256 output tile
// (256 tokens x 256 weight rows) of one job and walks K in steps of 64.  The
// waves form a 2 x 4 grid; each owns 128 x 64 = 4 x 2 MFMA 32x32x16 tiles
// (128 f32 accumulators per lane).  The 32x32x16 bf16 MFMA is used because
// one wave issuing it keeps the matrix core near its peak, which 16x16x32
// does not; two waves per SIMD let one wave's MFMAs cover the other's waits.
// bf16 weights (gemm_bf16_kernel): each K step's x and W tiles go from L2
// straight into the LDS stage the MFMAs are not reading (buffer loads with
// the LDS bit: no staging registers, no LDS write instructions), issued at
// the start of the step before, on the 256 x 256 tile by four of its eight
// waves (one per SIMD, so that the other wave there keeps the matrix core
// busy while the issuing one waits on the load unit); two 64 KiB stages,
// one barrier per step.
// Q8/Q4 weights (gemm_kernel): x's tile is copied into LDS the same way;
// the weight tile is fetched into registers two steps ahead, dequantised
// there, then written to the idle stage.  With fewer 256 x 256 tiles than
// compute units, Q8/Q4 run 256 x 128 halves on 8 waves (the other formats
// and the leftover of whole rounds run 128 x 128 quarters on 4).  Rows
// of 64 bf16 (8 chunks of 16 bytes) are stored with the chunk index
// XOR-swizzled by the row, so that the fragment reads (and the staging
// writes) are free of LDS bank conflicts.  Workgroups are mapped to tiles XCD by XCD
// (consecutive workgroup ids go to different XCDs), so that each XCD works on
// one contiguous range of weight-row tiles and its L2 holds the operand slices
// its workgroups share.
#include "il_internal.h"

#include <cstdlib>
#include <cstring>

namespace il {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kBig = 256;  // side of the work tiles the job table is cut into
constexpr int BK = 64;
constexpr int kXcds = 8;
constexpr uint32_t kBufFlags = 0x00020000u;
constexpr uint32_t kOut = 0x7FFFFFF0u;  // a buffer offset past every range: reads 0

// One launch covers big tiles [tile_lo, tile_lo + n_units) of the
// kBig x kBig tile grid (tile = tn * tiles_m + tm), or, for the 128 x 128
// kernel, the four quarters of each of them (unit = 4 * tile + quarter).
struct GemmParams {
    const uint16_t *xb;  // bf16 x [t][n_in]
    int t;
    int n_in;
    int n_jobs;
    int tiles_m;        // kBig-row tiles of x
    int tile_lo;        // first big tile of this launch
    int n_units;        // work units (workgroups with work) of this launch
    int units_per_xcd;  // ceil(n_units / kXcds)
    KJob job[kMaxJobs];
    int tn0[kMaxJobs + 1];  // prefix sums of kBig-column tiles per job
    int half;               // Q8/Q4 small units: 256 x 128 halves instead of quarters
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

// x f32 -> bf16 (RNE) pre-pass: 8 elements per thread.
__global__ __launch_bounds__(256) void x_to_bf16_kernel(const float *__restrict__ x, uint4 *__restrict__ xb,
                                                        int64_t n8) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const float4 a = reinterpret_cast<const float4 *>(x)[2 * i];
    const float4 b = reinterpret_cast<const float4 *>(x)[2 * i + 1];
    xb[i] = make_uint4(pack_bf16(a.x, a.y), pack_bf16(a.z, a.w), pack_bf16(b.x, b.y), pack_bf16(b.z, b.w));
}

// Q8/Q4 weights.  x's tile goes from L2 straight into LDS (buffer loads with
// the LDS bit, issued at the start of the step before); the weight tile is
// fetched into registers two steps ahead, dequantised, and written to the
// idle LDS stage after the MFMAs.  Steps end with explicit waits and a
// fence-free barrier, so the register prefetch stays in flight across it.
// GLU: jobs 0 and 1 are the gate and up projections.  A tile covers BN / 2
// output columns; B-tile rows come in groups of 32 alternating between the
// two weights (virtual row v holds row (v / 64) * 32 + v % 32 of the gate if
// (v / 32) is even, of the up projection if odd), so every wave's two 32-column
// MFMA tiles are the gate and up sums of the same outputs and the epilogue
// writes GELU(gate) * up from registers.
template <int FMT, int BM, int BN, int WM, int WN, bool GLU = false>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_kernel(GemmParams p) {
    static_assert(FMT == FMT_Q8 || FMT == FMT_Q4, "bf16 weights use gemm_bf16_kernel");
    constexpr int kThreads = 64 * WM * WN;
    constexpr int kChunksA = BM * BK / 8 / kThreads;  // 16-byte chunks per thread, A tile
    constexpr int TM = BM / WM / 32, TN = BN / WN / 32;  // 32x32 MFMA tiles per wave
    constexpr int kCols = GLU ? BN / 2 : BN;  // output columns of a tile
    static_assert(!GLU || TN == 2, "GLU pairs the two 32-column tiles of a wave");
    constexpr int TPR = kThreads / BN;  // Q8/Q4 staging threads per B row
    static_assert(TPR == 2 || TPR == 4, "Q8/Q4 staging: two or four threads per B row");
    constexpr int EPT = BK / TPR;       // elements of a B row per thread and step
    constexpr int kSplitM = kBig / BM, kSplitN = (GLU ? kBig / 2 : kBig) / kCols;  // units per big tile
    static_assert(kChunksA >= 1, "staging shape");
    __shared__ __attribute__((aligned(1024))) uint16_t lds[2][2][(BM > BN ? BM : BN) * BK];  // [stage][A|B]

    // ---- workgroup -> work unit, XCD by XCD ----
    const int b = blockIdx.x;
    const int unit = (b % kXcds) * p.units_per_xcd + b / kXcds;
    if (unit >= p.n_units) return;
    const int tile = p.tile_lo + unit / (kSplitM * kSplitN);
    const int q = unit % (kSplitM * kSplitN);
    const int tn_all = tile / p.tiles_m;
    const int tm = tile - tn_all * p.tiles_m;
    int j = 0;
    if constexpr (!GLU) {
#pragma unroll
        for (int jj = 1; jj < kMaxJobs; ++jj)
            if (jj < p.n_jobs && tn_all >= p.tn0[jj]) j = jj;
    }
    const KJob jb = p.job[j];
    const int m0 = tm * kBig + (q / kSplitN) * BM;
    const int n0 = (tn_all - p.tn0[j]) * (GLU ? kBig / 2 : kBig) + (q % kSplitN) * kCols;
    if (m0 >= p.t || n0 >= jb.n_out) return;  // a quarter past the edge of x or W
    const int n_in = p.n_in;
    const int nb = n_in / kBlock;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;  // WM x WN wave grid

    // ---- operand descriptors: exactly the tile's valid rows ----
    const int a_rows = min(BM, p.t - m0);
    const int b_rows = min(kCols, jb.n_out - n0);
    const uint32_t row2 = (uint32_t)n_in * 2u;
    const __amdgpu_buffer_rsrc_t ars = make_rsrc(p.xb + (int64_t)m0 * n_in, (uint32_t)a_rows * row2);
    // B descriptors over the tile's weight rows [n0, n0 + b_rows) of job k
    auto b_rsrc = [&](const KJob &k, __amdgpu_buffer_rsrc_t &c, __amdgpu_buffer_rsrc_t &sc) {
        if constexpr (FMT == FMT_Q8) {
            c = make_rsrc(static_cast<const int8_t *>(k.codes) + (int64_t)n0 * n_in,
                          (uint32_t)b_rows * (uint32_t)n_in);
            sc = make_rsrc(static_cast<const float *>(k.scales) + (int64_t)n0 * nb,
                           (uint32_t)b_rows * (uint32_t)nb * 4u);
        } else {
            // tile-major plane; n0 is a multiple of 16, so the tile's rows
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
    // elements EPT qh .. EPT qh + EPT - 1 of the step (a quantisation block
    // or half of one)
    const int qr = tid / TPR, qh = tid % TPR;
    const int qkey = swz_key(qr);

    uint4 sb[FMT == FMT_Q8 ? EPT / 16 : 1];
    float ssc = 0.f;
    auto fetch = [&](int k0) {
        {
            const int kh = k0 + EPT * qh;
            const bool ok = kh < n_in;
            // GLU: B-tile row qr is row wr of the gate ((qr / 32) even) or up
            const bool up = GLU && ((qr >> 5) & 1);
            const int wr = GLU ? (qr >> 6) * 32 + (qr & 31) : qr;
            const __amdgpu_buffer_rsrc_t crs = up ? brs2 : brs, srs = up ? bss2 : bss;
            if constexpr (FMT == FMT_Q8) {
                const uint32_t off = ok ? (uint32_t)wr * (uint32_t)n_in + (uint32_t)kh : kOut;
#pragma unroll
                for (int c = 0; c < EPT / 16; ++c) sb[c] = bload16(crs, ok ? off + 16u * c : kOut);
                ssc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                    srs, ok ? ((uint32_t)wr * nb + kh / kBlock) * 4u : kOut, 0, 0));
            } else {
                const uint32_t qoff = (uint32_t)q4_block_offset(wr, kh / kBlock, nb) + (uint32_t)((kh % kBlock) / 2);
                if constexpr (EPT == 32) {
                    sb[0] = bload16(crs, ok && wr < b_rows ? qoff : kOut);
                } else {
                    const uint2 h = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(crs, ok && wr < b_rows ? qoff : kOut, 0, 0));
                    sb[0] = make_uint4(h.x, h.y, 0u, 0u);
                }
                const uint16_t bits = __builtin_amdgcn_raw_buffer_load_b16(
                    srs, ok ? ((uint32_t)wr * nb + kh / kBlock) * 2u : kOut, 0, 0);
                ssc = (float)__builtin_bit_cast(_Float16, bits) * 0.0625f;  // values carry *16
            }
        }
    };
    auto store = [&](uint16_t *Bs) {
        {
            uint32_t o[EPT / 2];
            if constexpr (FMT == FMT_Q8) {
                uint32_t w[EPT / 4];
#pragma unroll
                for (int c = 0; c < EPT / 16; ++c)
                    w[4 * c] = sb[c].x, w[4 * c + 1] = sb[c].y, w[4 * c + 2] = sb[c].z, w[4 * c + 3] = sb[c].w;
#pragma unroll
                for (int i = 0; i < EPT / 4; ++i) {
                    o[2 * i] = pack_bf16((float)(int8_t)(w[i]) * ssc, (float)(int8_t)(w[i] >> 8) * ssc);
                    o[2 * i + 1] = pack_bf16((float)(int8_t)(w[i] >> 16) * ssc, (float)(int8_t)(w[i] >> 24) * ssc);
                }
            } else {
                const uint32_t w[4] = {sb[0].x, sb[0].y, sb[0].z, sb[0].w};
#pragma unroll
                for (int i = 0; i < EPT / 8; ++i) {
                    const uint32_t lo = (w[i] << 4) & 0xF0F0F0F0u;  // elements 0, 2, 4, 6 (code ^ 8)
                    const uint32_t hi = w[i] & 0xF0F0F0F0u;         // elements 1, 3, 5, 7
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        o[4 * i + e] = pack_bf16((float)(int8_t)(lo >> (8 * e)) * ssc, (float)(int8_t)(hi >> (8 * e)) * ssc);
                }
            }
#pragma unroll
            for (int i = 0; i < EPT / 8; ++i)
                *reinterpret_cast<uint4 *>(Bs + qr * BK + (((EPT / 8) * qh + i) ^ qkey) * 8) =
                    make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int n = 0; n < TN; ++n) acc[a][n] = (f32x16){};

    // 32x32x16 fragments: lane reads row (lane & 31) of a 32-row tile, 16-byte
    // chunk 2 kk + lane / 32; every fragment row of this lane shares one
    // swizzle key because tile offsets are multiples of 32
    const int frow = lane & 31;
    const int fkey = swz_key(frow);
    const int a_base = (wm * (BM / WM) + frow) * BK;
    const int b_base = (wn * (BN / WN) + frow) * BK;
    auto compute = [&](const uint16_t *As, const uint16_t *Bs) {
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

    const int nk = (n_in + BK - 1) / BK;
    uint32_t offa[kChunksA];
    int ka[kChunksA];
#pragma unroll
    for (int i = 0; i < kChunksA; ++i) {
        const int u = (wave * kChunksA + i) * 64 + lane, r = u >> 3;
        ka[i] = ((u & 7) ^ swz_key(r)) * 8;
        offa[i] = (uint32_t)r * row2 + (uint32_t)ka[i] * 2u;
    }
    auto issue_a = [&](uint16_t *As, int k0) {
#pragma unroll
        for (int i = 0; i < kChunksA; ++i)
            lds_load16(ars, As + (wave * kChunksA + i) * 64 * 8, k0 + ka[i] < n_in ? offa[i] + (uint32_t)k0 * 2u : kOut);
    };
    // B register loads per fetch (codes, then the scale): the waits below let
    // these, issued after a step's x copy, stay in flight across the barrier
    constexpr int kBLoads = FMT == FMT_Q8 ? EPT / 16 + 1 : 2;
    issue_a(lds[0][0], 0);
    fetch(0);
    store(lds[0][1]);
    const bool f1 = nk > 1;
    if (f1) fetch(BK);
    if (f1) wait_vmcnt<kBLoads>(); else wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this thread's LDS writes are done
    lds_barrier();
    for (int ks = 0; ks < nk; ++ks) {
        const int cur = ks & 1;
        if (ks + 1 < nk) issue_a(lds[cur ^ 1][0], (ks + 1) * BK);
        compute(lds[cur][0], lds[cur][1]);
        bool fetched = false;
        if (ks + 1 < nk) {
            store(lds[cur ^ 1][1]);  // B of step ks + 1 (its loads were in flight)
            if (ks + 2 < nk) fetch((ks + 2) * BK), fetched = true;
        }
        if (fetched) wait_vmcnt<kBLoads>(); else wait_vmcnt<0>();
        __builtin_amdgcn_s_waitcnt(0xC07F);
        lds_barrier();
    }

    // ---- epilogue: 32x32 tile, lane holds rows 8 (i / 4) + 4 (lane / 32) + i % 4
    //      of column lane % 32 ----
    if constexpr (GLU) {
#pragma unroll
        for (int a = 0; a < TM; ++a) {
            const int col = n0 + wn * (BN / WN) / 2 + (lane & 31);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = m0 + wm * (BM / WM) + a * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
                if (row < p.t && col < jb.n_out)
                    jb.y[(int64_t)row * jb.n_out + col] = gelu(acc[a][0][i]) * acc[a][1][i];
            }
        }
    } else {
#pragma unroll
        for (int a = 0; a < TM; ++a) {
#pragma unroll
            for (int n = 0; n < TN; ++n) {
                const int col = n0 + wn * (BN / WN) + n * 32 + (lane & 31);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = m0 + wm * (BM / WM) + a * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
                    if (row < p.t && col < jb.n_out) jb.y[(int64_t)row * jb.n_out + col] = acc[a][n][i];
                }
            }
        }
    }
}

// bf16 weights: the tiling, fragments and epilogue of gemm_kernel, with both
// operand tiles copied from L2 into LDS by the load unit.  A stage holds the
// A tile (BM rows) then the B tile (BN rows) of one K step, 16-byte chunks
// swizzled as above; instruction i of wave w fills chunks
// (w * kLoads + i) * 64 + lane of a tile, whose global address each lane
// computes once.
template <int BM, int BN, int WM, int WN, bool GLU>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_bf16_kernel(GemmParams p) {
    constexpr int kThreads = 64 * WM * WN;
    constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
    constexpr bool kQuarter = BM < kBig;
    constexpr int kCols = GLU ? BN / 2 : BN;
    constexpr int kLoadsA = BM * BK / 8 / kThreads, kLoadsB = BN * BK / 8 / kThreads;
    constexpr int kStage = (BM + BN) * BK;  // bf16 elements
    static_assert(!GLU || TN == 2, "GLU pairs the two 32-column tiles of a wave");
    static_assert(kLoadsA >= 1 && kLoadsB >= 1, "staging shape");
    __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * kStage];

    const int b = blockIdx.x;
    const int unit = (b % kXcds) * p.units_per_xcd + b / kXcds;
    if (unit >= p.n_units) return;
    const int tile = p.tile_lo + (kQuarter ? unit >> 2 : unit);
    const int q = kQuarter ? unit & 3 : 0;
    const int tn_all = tile / p.tiles_m;
    const int tm = tile - tn_all * p.tiles_m;
    int j = 0;
    if constexpr (!GLU) {
#pragma unroll
        for (int jj = 1; jj < kMaxJobs; ++jj)
            if (jj < p.n_jobs && tn_all >= p.tn0[jj]) j = jj;
    }
    const KJob jb = p.job[j];
    const int m0 = tm * kBig + (q >> 1) * BM;
    const int n0 = (tn_all - p.tn0[j]) * (GLU ? kBig / 2 : kBig) + (q & 1) * kCols;
    if (m0 >= p.t || n0 >= jb.n_out) return;  // a quarter past the edge of x or W
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
    // Who copies: a wave stalls while the CU's load unit drains the copies it
    // issues (~850 cycles of a ~3400-cycle K step when all 8 waves issue
    // theirs at once after the barrier), and its SIMD's matrix core idles
    // if the other wave there is stalled too.  So on the 8-wave tile only
    // waves 0..3, one per SIMD, issue the copies (twice as many each) while
    // waves 4..7 start on their MFMAs: 3459 -> 3159 cycles per K step.
    constexpr int kIssuers = kQuarter ? WM * WN : 4;
    constexpr int kLA = kLoadsA * WM * WN / kIssuers, kLB = kLoadsB * WM * WN / kIssuers;
    static_assert(kLA * kIssuers == kLoadsA * WM * WN && kLB * kIssuers == kLoadsB * WM * WN, "copy split");
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

    // ---- epilogue (as gemm_kernel) ----
    if constexpr (GLU) {
#pragma unroll
        for (int a = 0; a < TM; ++a) {
            const int col = n0 + wn * (BN / WN) / 2 + (lane & 31);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = m0 + wm * (BM / WM) + a * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
                if (row < p.t && col < jb.n_out)
                    jb.y[(int64_t)row * jb.n_out + col] = gelu(acc[a][0][i]) * acc[a][1][i];
            }
        }
    } else {
#pragma unroll
        for (int a = 0; a < TM; ++a) {
#pragma unroll
            for (int n = 0; n < TN; ++n) {
                const int col = n0 + wn * (BN / WN) + n * 32 + (lane & 31);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = m0 + wm * (BM / WM) + a * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
                    if (row < p.t && col < jb.n_out) jb.y[(int64_t)row * jb.n_out + col] = acc[a][n][i];
                }
            }
        }
    }
}

template <int FMT, bool GLU>
hipError_t launch_units(GemmParams p, bool quarter, int tile_lo, int n_units, hipStream_t s) {
    p.tile_lo = tile_lo;
    p.n_units = n_units;
    p.units_per_xcd = (n_units + kXcds - 1) / kXcds;
    const dim3 grid(kXcds * p.units_per_xcd);
    if constexpr (FMT == FMT_BF16) {
        if (quarter)
            hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, 2, 2, GLU>), grid, dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((gemm_bf16_kernel<kBig, kBig, 2, 4, GLU>), grid, dim3(512), 0, s, p);
    } else {
        if constexpr (!GLU) {
            if (quarter && p.half) {
                hipLaunchKernelGGL((gemm_kernel<FMT, 256, 128, 2, 4, false>), grid, dim3(512), 0, s, p);
                return hipGetLastError();
            }
        }
        if (quarter)
            hipLaunchKernelGGL((gemm_kernel<FMT, 128, 128, 2, 2, GLU>), grid, dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((gemm_kernel<FMT, kBig, kBig, 2, 4, GLU>), grid, dim3(512), 0, s, p);
    }
    return hipGetLastError();
}

template <int FMT, bool GLU = false>
hipError_t launch_plan(const GemmParams &p, int tiles, int cu_count, hipStream_t s) {
    // Whole rounds of big tiles (one per compute unit at a time); what is
    // left over, less than one round, runs as quarter tiles so that the last
    // round is short instead of mostly idle.
    const int full = tiles >= cu_count ? tiles / cu_count * cu_count : 0;
    hipError_t e = hipSuccess;
    if (full > 0) e = launch_units<FMT, GLU>(p, false, 0, full, s);
    // Q8/Q4 with fewer big tiles than compute units: 256 x 128 halves on 8
    // waves (the Q4 prefill's 112 tiles: 224 halves in one round, 92 us,
    // against 448 quarters in 1.75 rounds, ~101 us) -- whole rounds of them,
    // and the tiles left over as quarters
    if (FMT != FMT_BF16 && !GLU && full == 0) {
        const int halves = 2 * tiles;
        const int h = halves <= cu_count ? halves : halves / cu_count * cu_count / 2 * 2;
        GemmParams q = p;
        q.half = 1;
        e = launch_units<FMT, GLU>(q, true, 0, h, s);
        if (e == hipSuccess && h < halves) e = launch_units<FMT, GLU>(p, true, h / 2, 4 * (tiles - h / 2), s);
        return e;
    }
    if (e == hipSuccess && tiles > full) e = launch_units<FMT, GLU>(p, true, full, 4 * (tiles - full), s);
    return e;
}

}  // namespace

hipError_t launch_gemm(int fmt, const float *x, int t, int n_in, const KJob *jobs, int n_jobs,
                       int cu_count, hipStream_t s, bool glu) {
    if (t < 1 || n_jobs < 1 || n_jobs > kMaxJobs || n_in % kBlock || cu_count < 1) return hipErrorInvalidValue;
    if (glu && (n_jobs != 2 || jobs[0].n_out != jobs[1].n_out)) return hipErrorInvalidValue;
    // every buffer descriptor (kBig rows of x or of a weight) must stay below 2^31 bytes
    if ((int64_t)kBig * n_in * 2 >= (1ll << 31)) return hipErrorInvalidValue;
    GemmParams p{};
    p.t = t;
    p.n_in = n_in;
    p.n_jobs = n_jobs;
    p.tiles_m = (t + kBig - 1) / kBig;
    int tn = 0;
    for (int j = 0; j < n_jobs; ++j) {
        p.job[j] = jobs[j];
        p.tn0[j] = tn;
        // GLU: tiles of kBig / 2 output columns over the gate's rows only
        if (!glu) tn += (jobs[j].n_out + kBig - 1) / kBig;
        else if (j == 0) tn += (jobs[j].n_out + kBig / 2 - 1) / (kBig / 2);
    }
    for (int j = glu ? 1 : n_jobs; j <= kMaxJobs; ++j) p.tn0[j] = tn;
    const int tiles = p.tiles_m * tn;

    // mid-size t: the matrix-core decode kernel's wide mode, which rounds x
    // itself up to kWideF32MaxT tokens and reads the bf16 copy made below
    // beyond.  Q4 weights take it up to kVerifySliceMaxT tokens, as even
    // slices of at most kVerifyMaxT (the Q4 GEMM tiles are dequantised by
    // few waves and measured ~220 us per call on 2 x [17408, 5120] from
    // t = 33 to 128).  IL_PREFILL=gemm|verify pins the kernel.
    bool verify = t <= kVerifyMaxT || (fmt == FMT_Q4 && t <= kVerifySliceMaxT);
    if (const char *force = getenv("IL_PREFILL")) {
        if (!strcmp(force, "gemm")) verify = false;
        if (!strcmp(force, "verify")) verify = t <= kVerifySliceMaxT;
    }
    const int n_slices = (t + kVerifyMaxT - 1) / kVerifyMaxT;
    const int slice = (t + n_slices - 1) / n_slices;  // tokens per slice, > kWideF32MaxT when t > kVerifyMaxT
    verify = verify && verify_mfma_fits(fmt, slice, n_in, jobs, n_jobs);
    if (verify && t <= kWideF32MaxT)
        return launch_verify_mfma(fmt, x, nullptr, t, n_in, jobs, n_jobs, cu_count, s, glu);

    // x -> bf16 into stream-ordered scratch, freed after the GEMM on the same stream
    const int64_t n8 = (int64_t)t * n_in / 8;
    void *xb = nullptr;
    hipError_t e = hipMallocAsync(&xb, (size_t)n8 * 16, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(x_to_bf16_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, x,
                       static_cast<uint4 *>(xb), n8);
    e = hipGetLastError();
    if (e == hipSuccess) {
        p.xb = static_cast<const uint16_t *>(xb);
        if (verify) {
            // one launch per slice of tokens; slice i's x rows and y rows
            // start slice * i rows in
            for (int t0 = 0; t0 < t && e == hipSuccess; t0 += slice) {
                const int tt = min(slice, t - t0);
                KJob js[kMaxJobs];
                for (int j = 0; j < n_jobs; ++j) {
                    js[j] = jobs[j];
                    js[j].y = jobs[j].y + (int64_t)t0 * jobs[j].n_out;
                }
                e = launch_verify_mfma(fmt, x + (int64_t)t0 * n_in, p.xb + (int64_t)t0 * n_in, tt, n_in, js, n_jobs,
                                       cu_count, s, glu);
            }
        } else switch (fmt) {
            case FMT_BF16: e = glu ? launch_plan<FMT_BF16, true>(p, tiles, cu_count, s)
                                   : launch_plan<FMT_BF16>(p, tiles, cu_count, s); break;
            case FMT_Q8: e = glu ? launch_plan<FMT_Q8, true>(p, tiles, cu_count, s)
                                 : launch_plan<FMT_Q8>(p, tiles, cu_count, s); break;
            case FMT_Q4: e = glu ? launch_plan<FMT_Q4, true>(p, tiles, cu_count, s)
                                 : launch_plan<FMT_Q4>(p, tiles, cu_count, s); break;
            default: e = hipErrorInvalidValue;
        }
    }
    hipError_t fe = hipFreeAsync(xb, s);
    return e != hipSuccess ? e : fe;
}

}  // namespace il
