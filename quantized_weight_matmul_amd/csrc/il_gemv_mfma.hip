// il_gemv_mfma.hip -- decode GEMV on the bf16 matrix cores (t <= 8),
// and its "wide" mode for mid-size t (speculative-verify batches, 8 < t <= 32
// per launch; the prefill dispatch runs Q4 weights in slices of up to 32
// tokens to t = 128).
//
// Computes the same sums as the streaming decode kernel,
//   y[i][r] = sum_b s_rb * sum_{k in block b} (q_rk - z) * x_ik
// (bf16: s = 1, z = 0, q = w; Q8: z = 0; Q4: z = 8), i.e. the matmul of the
// `struct Job` doc comment (oxinfer 0.0.0 src/gpu.rs page) for every job of
// one format over the shared x of one submission (Backend::matmul on the
// same page).  With t tokens every weight element feeds 2t flops; once that
// outgrows the f32 vector units' budget per byte of Q4/Q8 weights, the
// contraction is moved onto v_mfma_f32_16x16x32_bf16, while HBM streaming of
// the weights stays the bound.
//
// Operands of one MFMA (16 x 16 output, K = 32 = one quantisation block):
//   * B = 16 weight rows x one block, as exact bf16 values: bf16 weights as
//     stored; Q8 codes converted through f32 (|q| <= 127 is exact in bf16);
//     Q4 codes come from a table in LDS: each byte of the code plane (two
//     nibbles, stored as the 4-bit two's complement of code - 8) indexes
//     256 precomputed pairs of exact bf16 values; the table holds one copy
//     per lane, so the 64 lookups of a wave hit 64 distinct banks and the
//     byte-to-address step is a single v_perm.  No
//     offset is folded out of a sum, so every product of A and B is exact
//     and the rounding of a result is relative to the sum of |x * w|.
//   * A = x as 16 rows: row i < t holds bf16(x_i), rounded to nearest even
//     as on the GEMM path (relative error at most 2^-8 / (1 + 2^-8), about
//     3.89e-3, per element; with the f32 sums, whose tree is a few hundred
//     additions deep, inside the 4e-3 * sum |x * w| bound), and every product
//     of A and B is exact in f32.  Rows of tokens >= t read zeros.  Each wave builds these operands
//     itself from x (f32, a few KiB that stay in L2), one step ahead, in the
//     per-lane order of the MFMA.
//   * The per-block scale multiplies the 16 x 16 f32 result (one FMA per
//     accumulator element), so no rounding of a dequantised weight occurs.
//   * Wide mode (8 < t <= 32): A rows are 16 tokens of bf16(x) per group
//     (round-to-nearest-even, as on the GEMM path), and one converted B
//     operand feeds one or two groups of MFMAs, so the weight conversion is
//     shared by up to 32 tokens.  With one group x is rounded from f32 in
//     registers; two groups read the bf16 copy of x that the GEMM's pre-pass
//     makes, since f32 x for 32 tokens would not fit in registers beside six
//     tiles.
//
// Loads: a wave fetches 16 bytes per lane, 64 bytes of each of 16 rows (one
// bf16 block, two Q8 blocks or four Q4 blocks per row: one "step"; for Q4,
// whose code plane is tile-major, one contiguous KiB).  Lane
// group g (lanes 16g..16g+15) holds row bytes [16g, 16g + 16) of the step;
// the MFMA wants lane group g to hold the g-th quarter of each block, which
// for Q8/Q4 is a 4 x 4 transpose of dwords across the lane groups (two
// permlane32 and two permlane16 swaps).  The K order inside a block that
// results is mirrored in the layout of the A operand, so A and B agree slot
// by slot.
//
// Work split: a workgroup of 8 waves owns a contiguous range of 16-row tiles
// (an equal share of all jobs' tiles), taken in chunks of up to 9 tiles (6 with two
// A row groups) of one job whose accumulators stay in registers.  Wave w streams steps w,
// w + 8, w + 16, ... of every tile of the chunk, so the workgroup reads 512
// contiguous bytes of each row at a time.  Each tile has its own register
// slot, refilled with the next step's 16 bytes as soon as it has been
// consumed, so a whole step of loads stays in flight.  At the end of a chunk
// the eight partial 16 x 16 results per tile are summed through LDS in a
// fixed order, so results are bitwise reproducible (no atomics).
#include "il_internal.h"

#include <type_traits>

namespace il {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 16;                    // weight rows per MFMA tile
// tiles accumulated in registers at once (fewer with two A row groups, whose
// accumulators and x operands take twice the registers)
// (with gate/up pairs an even count: 4 pairs, or 2 with two A row groups)
constexpr int chunk_tiles(int ng, bool glu) { return ng >= 2 ? (glu ? 4 : 6) : (glu ? 8 : 9); }
constexpr uint32_t kBufFlags = 0x00020000u;  // gfx9 raw buffer: 32-bit data format
constexpr uint32_t kOut = 0x7FFFFFF0u;       // a buffer offset past every range: reads 0
// A uniform offset base past every range: every plane and every per-lane
// offset is below 2^31, so base + lane offset stays past the plane and below
// 2^32 (no wrap).  The choice between a tile's base and this one is a scalar
// select, and the load's address costs one vector add.
constexpr uint32_t kOutBase = 0x80000000u;

// Blocks of one row covered by a wave's 16-byte-per-lane step (64 bytes/row).
template <int FMT>
struct Mfma;
template <>
struct Mfma<FMT_BF16> {
    static constexpr int BPS = 1;
    static constexpr int ROW_BYTES_PER_K = 2;
};
template <>
struct Mfma<FMT_Q8> {
    static constexpr int BPS = 2;
    static constexpr int ROW_BYTES_PER_K = 1;
};
template <>
struct Mfma<FMT_Q4> {
    static constexpr int BPS = 4;
    static constexpr int ROW_BYTES_PER_K = 0;  // half a byte: handled explicitly
};

template <int FMT>
__host__ __device__ constexpr int64_t mfma_row_bytes(int64_t n_in) {
    return FMT == FMT_Q4 ? n_in / 2 : n_in * Mfma<FMT>::ROW_BYTES_PER_K;
}

// Index within its block of the code that MFMA operand slot j (0..7) of lane
// group g holds after the loads, transposes and conversions below.
template <int FMT>
__device__ __forceinline__ int slot_code(int g, int j) {
    if constexpr (FMT == FMT_BF16) {
        return 8 * g + j;
    } else if constexpr (FMT == FMT_Q8) {
        return (j < 4) ? 4 * g + j : 16 + 4 * g + (j - 4);
    } else {
        return 8 * g + j;
    }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, kBufFlags);
}

// bit-cast whole vectors: clang 22 turns bit casts of single ext_vector
// elements into copies of element 0
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));  // RNE
}


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

// Q4 code table in LDS: entry (byte b, lane l) at byte offset 256 b + 4 l
// holds the two codes of b (stored as code ^ 8, element 2i in the low nibble
// of byte i) as exact bf16 values code - 8, low nibble first.
constexpr int kQ4LutWords = 256 * 64;

__device__ __forceinline__ uint32_t q4_pair_bf16(int b) {
    const int lo = ((b & 15) ^ 8) - 8, hi = ((b >> 4) ^ 8) - 8;
    return pack_bf16((float)lo, (float)hi);
}

// 8 Q4 codes of one dword -> 8 exact bf16 values, in order: v_perm puts
// byte i of d next to this lane's column offset, which is the table address.
__device__ __forceinline__ bf16x8 q4_to_bf16(const uint32_t *lut, uint32_t d, uint32_t lane4) {
    const char *lb = reinterpret_cast<const char *>(lut);
    uint4 o;
    o.x = *reinterpret_cast<const uint32_t *>(lb + __builtin_amdgcn_perm(d, lane4, 0x0C0C0400u));
    o.y = *reinterpret_cast<const uint32_t *>(lb + __builtin_amdgcn_perm(d, lane4, 0x0C0C0500u));
    o.z = *reinterpret_cast<const uint32_t *>(lb + __builtin_amdgcn_perm(d, lane4, 0x0C0C0600u));
    o.w = *reinterpret_cast<const uint32_t *>(lb + __builtin_amdgcn_perm(d, lane4, 0x0C0C0700u));
    return __builtin_bit_cast(bf16x8, o);
}

// 8 signed Q8 codes (4 per dword) -> 8 exact bf16 values, in order.
__device__ __forceinline__ bf16x8 q8_to_bf16(uint32_t a, uint32_t b) {
    uint4 o;
    o.x = pack_bf16((float)(int8_t)a, (float)(int8_t)(a >> 8));
    o.y = pack_bf16((float)(int8_t)(a >> 16), (float)(int8_t)(a >> 24));
    o.z = pack_bf16((float)(int8_t)b, (float)(int8_t)(b >> 8));
    o.w = pack_bf16((float)(int8_t)(b >> 16), (float)(int8_t)(b >> 24));
    return __builtin_bit_cast(bf16x8, o);
}

__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}


// A operand of one block: the lane's 8 x values (two 16-byte loads) rounded
// to bf16 (round-to-nearest-even, as on the GEMM path).  Whole-vector bit
// casts (see bload16).
__device__ __forceinline__ bf16x8 x_bf16(const uint4 &p, const uint4 &q) {
    const f32x4 a = __builtin_bit_cast(f32x4, p);
    const f32x4 b = __builtin_bit_cast(f32x4, q);
    return __builtin_bit_cast(bf16x8, make_uint4(pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]),
                                                 pack_bf16(b[0], b[1]), pack_bf16(b[2], b[3])));
}

struct MfmaParams {
    const float *x;      // [t][n_in] (narrow mode, wide mode with one group)
    const uint16_t *xb;  // bf16(x) [t][n_in] (wide mode with two groups)
    int t;
    int n_in;
    int nb;     // blocks per row
    int steps;  // ceil(nb / BPS)
    int n_jobs;
    int tiles_total;
    KJob job[kMaxJobs];
    int tile0[kMaxJobs + 1];  // prefix sums of 16-row tiles per job
};

// A run of at most TC consecutive tiles of one job: the unit of register
// accumulation and of the LDS reduction.
struct Chunk {
    int start;  // first tile (global index); >= the workgroup's end: none
    int cnt;    // tiles in the chunk (0: none)
    int j;      // job
    int lrow0;  // job-local row of the chunk's first row
};

// NG = 0: "narrow" mode, t <= 8, A rows 0..t-1 = bf16(x) (f32 in memory),
// rows 8..15 zero, so the outputs sit in lanes 0..31 (rows 0..7).
// NG >= 1: "wide" mode, t <= 16 NG, NG groups of 16 tokens per B operand,
// A rows = bf16(x): rounded from the f32 x as it is loaded (NG = 1) or read
// from the pre-pass's bf16 copy (NG = 2).
// GLU: jobs 0 and 1 are the gate and up projections (same rows); a chunk
// holds TC / 2 tiles of each, slot r < TC / 2 gate tile r and slot TC / 2 + r
// the up tile with the same rows, and the reduction writes
// GELU(gate) * up to job 0's y.
// TE: accumulator elements per lane that hold a token (lane group g, element
// e holds A row 4g + e): all 4 in wide mode; in narrow mode row i of token
// i < t, so min(t, 4) -- the block scale is applied to those only (the
// others stay 0 and are never read).
template <int FMT, int TC, int NG, bool GLU, int TE>
__global__ __launch_bounds__(kThreads) void gemv_mfma_kernel(MfmaParams p) {
    constexpr int BPS = Mfma<FMT>::BPS;
    constexpr int TCh = GLU ? TC / 2 : TC;  // tiles of one job in a chunk
    static_assert(!GLU || TC % 2 == 0, "gate/up tile pairs");
    constexpr bool kWide = NG > 0;
    constexpr int NA = kWide ? NG : 1;  // A row groups per B operand
    __shared__ f32x4 red[kWaves][TC][kWide ? 64 : 32];
    __shared__ uint32_t lut[FMT == FMT_Q4 ? kQ4LutWords : 1];

    const int lane = (int)threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int n = lane & 15;  // weight row within the tile (B column) = A row
    const int g = lane >> 4;  // lane group: quarter of the K slice

    const int t = p.t, nb = p.nb, n_in = p.n_in;
    const int nb4 = (nb + 3) / 4;
    const int64_t row_bytes = mfma_row_bytes<FMT>(n_in);

    // A operand row n of group q is token 16 q + n; rows of tokens >= t read
    // zeros (narrow mode: t <= 8, so rows 8..15 always do).
    const int tok = n;
    constexpr bool kXb16 = NG >= 2;  // x given as bf16
    constexpr int esz = kXb16 ? 2 : 4;
    const __amdgpu_buffer_rsrc_t xrs =
        kXb16 ? make_rsrc(p.xb, (uint32_t)(t * n_in * 2)) : make_rsrc(p.x, (uint32_t)(t * n_in * 4));
    // the lane's 8 x values of a block are two runs of 4 elements
    const uint32_t xoff0 = (uint32_t)((tok * n_in + slot_code<FMT>(g, 0)) * esz);
    const uint32_t xoff1 = (uint32_t)((tok * n_in + slot_code<FMT>(g, 4)) * esz);

    // this workgroup's tiles and this wave's K steps
    const int T = p.tiles_total, G = (int)gridDim.x;
    const int ta = (int)((int64_t)blockIdx.x * T / G);
    const int tb = (int)((int64_t)(blockIdx.x + 1) * T / G);
    // wave w takes steps w, w + 8, ...: at any time the workgroup reads 8
    // consecutive 64-byte steps (512 contiguous bytes) of every row, so the
    // two halves of a 128-byte line are requested together
    const int S = p.steps;
    const int Sw = wave < S ? (S - wave + kWaves - 1) / kWaves : 0;

    auto chunk_at = [&](int start) {
        Chunk c;
        c.start = start;
        c.j = 0;
        if constexpr (!GLU) {
#pragma unroll
            for (int q = 1; q < kMaxJobs; ++q)
                if (q < p.n_jobs && start >= p.tile0[q]) c.j = q;
        }
        c.cnt = start < tb ? min(TCh, min(tb, p.tile0[c.j + 1]) - start) : 0;
        c.lrow0 = (start - p.tile0[c.j]) * kTile;
        return c;
    };

    // ---- register ring: one step of every tile of a chunk, plus x ----
    uint4 wc[TC];
    // Q4: the f16 scales of blocks 4s..4s+3 of the lane's row (one 8-byte
    // load); Q8: the f32 scale of the lane's block
    typename std::conditional<FMT == FMT_Q4, uint2, uint32_t>::type ws[TC];
    uint4 xr[kXb16 ? 1 : NA][BPS][2];  // 8 f32 of x per block (and token group)
    uint4 xw[kXb16 ? NA : 1][BPS];     // two groups: 8 bf16 of x per block and group

    // issue side: chunk, step and the chunk's buffer descriptors
    Chunk ic = chunk_at(ta);
    int is = wave;
    __amdgpu_buffer_rsrc_t crs, srs, crs2, srs2;  // *2: the up projection (GLU)
    auto set_rsrc = [&]() {
        const KJob &jb = p.job[ic.j];
        const int64_t rows = ic.cnt > 0 ? jb.n_out : 0;
        const uint32_t sbytes = (uint32_t)(tiled_scale_count(rows, nb) * (FMT == FMT_Q8 ? 4 : 2));
        const uint32_t cbytes = (uint32_t)(FMT == FMT_Q4 ? q4_plane_bytes(rows, nb) : rows * row_bytes);
        crs = make_rsrc(jb.codes, cbytes);
        srs = make_rsrc(jb.scales_t, sbytes);
        if constexpr (GLU) {
            crs2 = make_rsrc(p.job[1].codes, cbytes);
            srs2 = make_rsrc(p.job[1].scales_t, sbytes);
        }
    };
    set_rsrc();
    auto issue_x = [&]() {
#pragma unroll
        for (int jb = 0; jb < BPS; ++jb) {
            const int b = BPS * is + jb;
#pragma unroll
            for (int q = 0; q < NA; ++q) {
                const bool ok = 16 * q + tok < t && ic.cnt > 0 && b < nb;
                const uint32_t o = (uint32_t)(q * 16 * n_in * esz) + (uint32_t)(b * 32 * esz);
                if constexpr (kXb16 && FMT != FMT_Q8) {
                    xw[q][jb] = bload16(xrs, ok ? xoff0 + o : kOut);  // slots 0..7 are one run
                } else if constexpr (kXb16) {
                    const uint2 lo = __builtin_bit_cast(
                        uint2, __builtin_amdgcn_raw_buffer_load_b64(xrs, ok ? xoff0 + o : kOut, 0, 0));
                    const uint2 hi = __builtin_bit_cast(
                        uint2, __builtin_amdgcn_raw_buffer_load_b64(xrs, ok ? xoff1 + o : kOut, 0, 0));
                    xw[q][jb] = make_uint4(lo.x, lo.y, hi.x, hi.y);
                } else {
                    xr[q][jb][0] = bload16(xrs, ok ? xoff0 + o : kOut);
                    xr[q][jb][1] = bload16(xrs, ok ? xoff1 + o : kOut);
                }
            }
        }
    };
    // Q4: a lane's code and scale offsets are a uniform segment index (tile
    // of the plane * nb4 + step) shifted, plus these per-lane constants
    const uint32_t q4_code_lane = ((uint32_t)n << 6) + ((uint32_t)g << 4);
    const uint32_t q4_scale_lane = (uint32_t)n << 3;
    // bf16 / Q8: a lane's code offset is the tile's first row + the step's 64
    // bytes (uniform) plus its row and 16-byte chunk; its Q8 scale index the
    // tiled plane's uniform part plus row n and block half g / 2
    const uint32_t rm_code_lane = (uint32_t)n * (uint32_t)row_bytes + ((uint32_t)g << 4);
    const uint32_t q8_scale_lane = ((uint32_t)n << 2) + (uint32_t)(g >> 1);
    auto issue_w = [&](int r) {
        const int rt = r % TCh;     // tile of its job
        const bool up = GLU && r >= TCh;
        const __amdgpu_buffer_rsrc_t wrs = up ? crs2 : crs, qrs = up ? srs2 : srs;
        if constexpr (FMT == FMT_Q4) {
            // The code plane and the tiled scale plane are padded to whole
            // 16-row tiles and 4-block segments (zero codes decode to 0,
            // padded scales are 0), so no lane needs a row or block check:
            // only whether the chunk has this tile.  The step's segment of
            // the tile is one 1 KiB run of codes and one 128-byte run of
            // scales (16 rows x 4 blocks x 2 bytes).
            const bool ok = rt < ic.cnt;
            const uint32_t seg = (uint32_t)((ic.lrow0 >> 4) + rt) * (uint32_t)nb4 + (uint32_t)is;
            wc[r] = bload16(wrs, (ok ? seg << 10 : kOutBase) + q4_code_lane);
            ws[r] = __builtin_bit_cast(
                uint2, __builtin_amdgcn_raw_buffer_load_b64(qrs, (ok ? seg << 7 : kOutBase) + q4_scale_lane, 0, 0));
            return;
        }
        // bf16 / Q8, row-major planes: no per-lane checks either.  A row past
        // the job's last lies past its plane's descriptor and reads zeros; a
        // Q8 chunk past the end of a row (the last step, when the row has an
        // odd number of blocks) reads the next row's codes, which meet zero x
        // (x past n_in reads zeros) and the zero padded scale, so it adds 0.
        const bool ok = rt < ic.cnt;
        const uint32_t row0 = (uint32_t)(ic.lrow0 + kTile * rt);
        wc[r] = bload16(wrs, (ok ? row0 * (uint32_t)row_bytes + ((uint32_t)is << 6) : kOutBase) + rm_code_lane);
        if constexpr (FMT == FMT_Q8) {
            // this lane's 16 bytes are half of block 2s + g/2: scale index
            // ((tile * nb4 + s/2) * 64) + 4 n + 2 (s % 2) + g/2 in the tiled plane
            const uint32_t tq = ((row0 >> 4) * (uint32_t)nb4 + ((uint32_t)is >> 1)) * 64u + (((uint32_t)is & 1u) << 1);
            ws[r] = __builtin_amdgcn_raw_buffer_load_b32(qrs, (ok ? tq * 4u : kOutBase) + q8_scale_lane * 4u, 0, 0);
        }
    };
    auto advance = [&](Chunk &c, int &s) {
        s += kWaves;
        if (s >= S) {
            s = wave;
            c = chunk_at(c.start + max(c.cnt, 1));
        }
    };

    f32x4 acc[TC][NA];
#pragma unroll
    for (int r = 0; r < TC; ++r)
#pragma unroll
        for (int q = 0; q < NA; ++q) acc[r][q] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // ---- end of a chunk: sum the 8 waves' partials per tile through LDS ----
    auto reduce = [&](const Chunk &c) {
        const KJob &jb = p.job[c.j];
        const float *redf = reinterpret_cast<const float *>(&red[0][0][0]);
        constexpr int kLanes = kWide ? 64 : 32;  // lanes holding distinct outputs
#pragma unroll
        for (int q = 0; q < NA; ++q) {
#pragma unroll
            for (int r = 0; r < TC; ++r) {
                if (r % TCh < c.cnt) {
                    // narrow mode: rows 0..7 are lanes 0..31
                    if (kWide || lane < 32) red[wave][r][lane] = acc[r][q];
                }
                acc[r][q] = (f32x4){0.f, 0.f, 0.f, 0.f};
            }
            __syncthreads();
            for (int r = wave; r < c.cnt; r += kWaves) {
#pragma unroll
                for (int h = 0; h < (kWide ? 4 : 2); ++h) {
                    const int i = 4 * h + (lane >> 4);  // token within the group
                    const int row = c.lrow0 + kTile * r + n;
                    const int token = 16 * q + i;
                    if (token < t && row < jb.n_out) {
                        // token i, row n sits in lane 16 * (i / 4) + n, element i % 4
                        const int slot = 16 * (i >> 2) + n, e = i & 3;
                        float sum = 0.f;
#pragma unroll
                        for (int w = 0; w < kWaves; ++w) sum += redf[((w * TC + r) * kLanes + slot) * 4 + e];
                        if constexpr (GLU) {
                            float su = 0.f;
#pragma unroll
                            for (int w = 0; w < kWaves; ++w)
                                su += redf[((w * TC + TCh + r) * kLanes + slot) * 4 + e];
                            sum = gelu(sum) * su;
                        }
                        jb.y[(int64_t)token * jb.n_out + row] = sum;
                    }
                }
            }
            __syncthreads();  // red is rewritten next
        }
    };

    // ---- one step of one tile ----
    auto consume = [&](int r, const bf16x8 (&a)[NA][BPS]) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        if constexpr (FMT == FMT_BF16) {
#pragma unroll
            for (int q = 0; q < NA; ++q) acc[r][q] = mfma(a[q][0], __builtin_bit_cast(bf16x8, wc[r]), acc[r][q]);
        } else if constexpr (FMT == FMT_Q8) {
            uint32_t d0 = wc[r].x, d1 = wc[r].y, d2 = wc[r].z, d3 = wc[r].w;
            xpose4(d0, d1, d2, d3);
            // lane groups 0,1 hold block 2s's scale, groups 2,3 block 2s+1's
            const auto sc = __builtin_amdgcn_permlane32_swap(ws[r], ws[r], false, false);
            const f32x2 scf = __builtin_bit_cast(f32x2, sc);  // whole-vector cast (see bload16)
            const bf16x8 b0 = q8_to_bf16(d0, d1), b1 = q8_to_bf16(d2, d3);
            f32x4 p0[NA], p1[NA];
#pragma unroll
            for (int q = 0; q < NA; ++q) {
                p0[q] = mfma(a[q][0], b0, z);
                p1[q] = mfma(a[q][1], b1, z);
            }
            // all MFMAs issue before the first read of a result
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < NA; ++q)
#pragma unroll
                for (int e = 0; e < TE; ++e) acc[r][q][e] = fmaf(scf[1], p1[q][e], fmaf(scf[0], p0[q][e], acc[r][q][e]));
        } else {
            uint32_t d[4] = {wc[r].x, wc[r].y, wc[r].z, wc[r].w};
            xpose4(d[0], d[1], d[2], d[3]);
            const uint32_t sb[4] = {ws[r].x, ws[r].x >> 16, ws[r].y, ws[r].y >> 16};
            f32x4 pj[NA][4];
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) {
                const bf16x8 bq = q4_to_bf16(lut, d[jb], (uint32_t)lane << 2);
#pragma unroll
                for (int q = 0; q < NA; ++q) pj[q][jb] = mfma(a[q][jb], bq, z);
            }
            // all MFMAs issue before the first read of a result, so the
            // scaling of block 0 overlaps the matrix core's work on 1..3
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) {
                const float sf = (float)__builtin_bit_cast(_Float16, (uint16_t)sb[jb]);
#pragma unroll
                for (int q = 0; q < NA; ++q)
#pragma unroll
                    for (int e = 0; e < TE; ++e) acc[r][q][e] = fmaf(sf, pj[q][jb][e], acc[r][q][e]);
            }
        }
    };

    // Units (chunk, step) in order; the loads of the next unit are issued
    // while the current one is consumed: x first, then each tile's weights
    // right after that tile's registers are consumed.  No branch surrounds a
    // load in the loop, so the in-order vector-memory counter keeps a whole
    // step of loads in flight.  The first unit's loads go out before the Q4
    // code table is built, so that building it overlaps their latency.
    if (Sw > 0) {
        issue_x();
#pragma unroll
        for (int r = 0; r < TC; ++r) issue_w(r);
    }
    if constexpr (FMT == FMT_Q4) {
        // the code table: wave w fills byte values w, w + 8, ..., one column
        // per lane; then this wave's LDS writes are waited for and the
        // workgroup meets at a barrier without __syncthreads' release fence,
        // which would also wait for the loads above
#pragma unroll 4
        for (int i = 0; i < 32; ++i) lut[(8 * i + wave) * 64 + lane] = q4_pair_bf16(8 * i + wave);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    if (Sw == 0) {
        for (Chunk c = chunk_at(ta); c.cnt > 0; c = chunk_at(c.start + c.cnt)) reduce(c);
        return;
    }
    Chunk cc = ic;
    int cs = is;
    advance(ic, is);
    set_rsrc();
    while (cc.cnt > 0) {
        bf16x8 a[NA][BPS];
#pragma unroll
        for (int jb = 0; jb < BPS; ++jb) {
            if constexpr (kXb16) {
#pragma unroll
                for (int q = 0; q < NA; ++q) a[q][jb] = __builtin_bit_cast(bf16x8, xw[q][jb]);
            } else {
                a[0][jb] = x_bf16(xr[0][jb][0], xr[0][jb][1]);
            }
        }
        issue_x();
#pragma unroll
        for (int r = 0; r < TC; ++r) {
            if (r % TCh < cc.cnt) consume(r, a);
            issue_w(r);
        }
        const bool chunk_end = cs + kWaves >= S;
        if (chunk_end) reduce(cc);
        cc = ic;
        cs = is;
        advance(ic, is);
        set_rsrc();
    }
}

}  // namespace

namespace {

// every buffer offset a lane forms stays below 2^31: with row-major planes
// that includes the rows of a job's last tile past n_out (16-row padding) and
// the 32 bytes a Q8 row's last step reads past its end
bool mfma_fits(int fmt, int64_t x_bytes, int n_in, const KJob *jobs, int n_jobs) {
    if (n_in <= 0 || n_in % kBlock || x_bytes >= (1ll << 31) || n_jobs < 1 || n_jobs > kMaxJobs) return false;
    const int64_t rb = fmt == FMT_BF16 ? 2ll * n_in : (int64_t)n_in;
    const int64_t sb = fmt == FMT_Q8 ? 4 : 2;
    for (int j = 0; j < n_jobs; ++j) {
        const int64_t rows16 = (jobs[j].n_out + kTile - 1) / kTile * kTile;
        if ((fmt == FMT_Q4 ? q4_plane_bytes(jobs[j].n_out, n_in / kBlock) : rows16 * rb + 64) >= (1ll << 31) ||
            tiled_scale_count(jobs[j].n_out, n_in / kBlock) * sb >= (1ll << 31))
            return false;
    }
    return true;
}

// With glu the tile range is job 0's (the gate); each tile also stands for
// the up projection's tile with the same rows.
bool fill_params(MfmaParams &p, int fmt, int t, int n_in, const KJob *jobs, int n_jobs, bool glu) {
    p.t = t;
    p.n_in = n_in;
    p.nb = n_in / kBlock;
    const int bps = fmt == FMT_BF16 ? 1 : fmt == FMT_Q8 ? 2 : 4;
    p.steps = (p.nb + bps - 1) / bps;
    p.n_jobs = n_jobs;
    int tiles = 0;
    for (int j = 0; j < n_jobs; ++j) {
        p.job[j] = jobs[j];
        p.tile0[j] = tiles;
        if (!glu || j == 0) tiles += (jobs[j].n_out + kTile - 1) / kTile;
    }
    for (int j = glu ? 1 : n_jobs; j <= kMaxJobs; ++j) p.tile0[j] = tiles;
    p.tiles_total = tiles;
    return tiles > 0;
}

template <int FMT, int NG, bool GLU, int TE>
hipError_t launch_te(const MfmaParams &p, int grid, hipStream_t s) {
    hipLaunchKernelGGL((gemv_mfma_kernel<FMT, chunk_tiles(NG, GLU), NG, GLU, TE>), dim3(grid), dim3(kThreads), 0,
                       s, p);
    return hipGetLastError();
}

template <int FMT, int NG, bool GLU>
hipError_t launch_mode(const MfmaParams &p, int cu_count, hipStream_t s) {
    // one workgroup per compute unit at most, each an equal share of the tiles
    const int grid = p.tiles_total < cu_count ? p.tiles_total : cu_count;
    if constexpr (NG == 0) {
        if (p.t == 1) return launch_te<FMT, NG, GLU, 1>(p, grid, s);
        if (p.t == 2) return launch_te<FMT, NG, GLU, 2>(p, grid, s);
    }
    return launch_te<FMT, NG, GLU, 4>(p, grid, s);
}

template <int NG>
hipError_t launch_fmt_mode(int fmt, const MfmaParams &p, int cu_count, hipStream_t s, bool glu) {
    switch (fmt) {
        case FMT_BF16: return glu ? launch_mode<FMT_BF16, NG, true>(p, cu_count, s)
                                  : launch_mode<FMT_BF16, NG, false>(p, cu_count, s);
        case FMT_Q8: return glu ? launch_mode<FMT_Q8, NG, true>(p, cu_count, s)
                                : launch_mode<FMT_Q8, NG, false>(p, cu_count, s);
        case FMT_Q4: return glu ? launch_mode<FMT_Q4, NG, true>(p, cu_count, s)
                                : launch_mode<FMT_Q4, NG, false>(p, cu_count, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool gemv_mfma_fits(int fmt, int t, int n_in, const KJob *jobs, int n_jobs) {
    return t >= 1 && t <= kGemvMaxT && mfma_fits(fmt, 4ll * t * n_in, n_in, jobs, n_jobs);
}

hipError_t launch_gemv_mfma(int fmt, const float *x, int t, int n_in, const KJob *jobs, int n_jobs,
                            int cu_count, hipStream_t s, bool glu) {
    if (!gemv_mfma_fits(fmt, t, n_in, jobs, n_jobs)) return hipErrorInvalidValue;
    if (glu && (n_jobs != 2 || jobs[0].n_out != jobs[1].n_out)) return hipErrorInvalidValue;
    MfmaParams p{};
    p.x = x;
    if (!fill_params(p, fmt, t, n_in, jobs, n_jobs, glu)) return hipSuccess;
    return launch_fmt_mode<0>(fmt, p, cu_count, s, glu);
}

bool verify_mfma_fits(int fmt, int t, int n_in, const KJob *jobs, int n_jobs) {
    return t > kGemvMaxT && t <= kVerifyMaxT && mfma_fits(fmt, 4ll * t * n_in, n_in, jobs, n_jobs);
}

hipError_t launch_verify_mfma(int fmt, const float *x, const uint16_t *xb, int t, int n_in, const KJob *jobs,
                              int n_jobs, int cu_count, hipStream_t s, bool glu) {
    if (!verify_mfma_fits(fmt, t, n_in, jobs, n_jobs)) return hipErrorInvalidValue;
    if (glu && (n_jobs != 2 || jobs[0].n_out != jobs[1].n_out)) return hipErrorInvalidValue;
    if (t > kWideF32MaxT && xb == nullptr) return hipErrorInvalidValue;
    MfmaParams p{};
    p.x = x;
    p.xb = xb;
    if (!fill_params(p, fmt, t, n_in, jobs, n_jobs, glu)) return hipSuccess;
    return t <= kWideF32MaxT ? launch_fmt_mode<1>(fmt, p, cu_count, s, glu)
                             : launch_fmt_mode<2>(fmt, p, cu_count, s, glu);
}

}  // namespace il
