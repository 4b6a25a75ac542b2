// il_gemv.hip -- decode GEMV for t <= 8: every job of one format in one launch.
//
// Computes, for each job, y[i][r] = sum_b s_rb * sum_{k in block b} q_rk * x_ik
// (bf16: s = 1, q = w), i.e. y[t][n_out] = x[t][n_in] * W^T from the doc
// comment of `struct Job` (oxinfer 0.0.0 src/gpu.rs page), for a batch of jobs
// sharing x "in a single submission" (Backend::matmul on the same page).
//
// Shape of the kernel (HBM-bound: every weight byte is read exactly once):
//   * a workgroup is 4 waves; each wave owns R consecutive output rows (the
//     rows of all jobs are numbered consecutively, so a wave may straddle two
//     jobs) and walks the whole K range of those rows;
//   * per step a lane fetches 16 contiguous weight bytes of each of its R rows
//     (one global_load_dwordx4; the 64 lanes of a wave cover 1 KiB of a row),
//     the next step's loads are issued before the current step's math;
//   * x is staged once per workgroup in LDS as f32, permuted so that every
//     lane's ds_read_b128 is a contiguous, conflict-free 1 KiB wave access;
//     x larger than the LDS budget is staged in K chunks;
//   * dequantisation happens in registers and is exact: bf16 -> f32 is a
//     shift, Q8 codes are sign-extended bytes, Q4 nibbles (stored code ^ 8) are
//     moved to the top of a byte and sign-extended (16 * (code - 8)); the
//     block scale multiplies each lane's per-block partial sum;
//   * f32 FMAs accumulate per lane, a wave reduction finishes each output, and
//     lane 0 stores it: each y element is written once, no atomics, so results
//     are bitwise reproducible.
#include "il_internal.h"

#include <atomic>
#include <cstdlib>
#include <cstring>

namespace il {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kXLdsBytes = 64 * 1024;  // LDS budget for x per workgroup

template <int FMT>
struct FmtTraits;
template <>
struct FmtTraits<FMT_BF16> {
    static constexpr int E = 8;  // elements per 16-byte lane load
};
template <>
struct FmtTraits<FMT_Q8> {
    static constexpr int E = 16;
};
template <>
struct FmtTraits<FMT_Q4> {
    static constexpr int E = 32;
};

struct GemvParams {
    const float *x;
    int t;
    int n_in;
    int n_jobs;
    int total_rows;
    int kc;        // K elements per LDS chunk (multiple of 64*E)
    int n_chunks;  // ceil(n_in / kc)
    KJob job[kMaxJobs];
    int row0[kMaxJobs + 1];  // prefix sums of n_out
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Byte offset of element k within a bf16 / Q8 code row.
template <int FMT>
__device__ __forceinline__ int64_t code_byte(int64_t k) {
    if constexpr (FMT == FMT_BF16) return 2 * k;
    if constexpr (FMT == FMT_Q8) return k;
    return k / 2;
}

template <int FMT>
__device__ __forceinline__ int64_t row_bytes(int64_t n_in) {
    return code_byte<FMT>(n_in);
}

// Byte offset of the 16 bytes a lane fetches at element k (a multiple of the
// lane's elements) of row `local` of a job: row-major for bf16 / Q8, the
// tile-major block place for Q4.
template <int FMT>
__device__ __forceinline__ int64_t code_offset(int64_t local, int64_t k, int64_t n_in) {
    if constexpr (FMT == FMT_Q4) return q4_block_offset(local, k / kBlock, n_in / kBlock);
    else return local * row_bytes<FMT>(n_in) + code_byte<FMT>(k);
}

// Element j (0 <= j < 4) of 4-element group g of a 16-byte weight vector, as
// an exact f32.  Q4 values come out multiplied by 16 (folded into the scale).
template <int FMT>
__device__ __forceinline__ void dequant4(const uint4 &v, int g, float out[4]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    if constexpr (FMT == FMT_BF16) {
        // 8 bf16: group g = words 2g, 2g+1
        uint32_t a = w[2 * g], b = w[2 * g + 1];
        out[0] = __builtin_bit_cast(float, a << 16);
        out[1] = __builtin_bit_cast(float, a & 0xFFFF0000u);
        out[2] = __builtin_bit_cast(float, b << 16);
        out[3] = __builtin_bit_cast(float, b & 0xFFFF0000u);
    } else if constexpr (FMT == FMT_Q8) {
        // 16 int8: group g = word g
        uint32_t a = w[g];
        out[0] = (float)(int8_t)(a);
        out[1] = (float)(int8_t)(a >> 8);
        out[2] = (float)(int8_t)(a >> 16);
        out[3] = (float)(int8_t)(a >> 24);
    } else {
        // 32 nibbles, 8 per word: group g = elements 4g..4g+3 = the low (g even)
        // or high (g odd) two bytes of word g/2.  Moving each nibble to the top
        // of a byte makes the signed byte equal 16 * (code - 8).
        uint32_t a = w[g / 2];
        uint32_t lo = (a << 4) & 0xF0F0F0F0u;  // word elements 0, 2, 4, 6
        uint32_t hi = a & 0xF0F0F0F0u;         // word elements 1, 3, 5, 7
        const int sh = 16 * (g & 1);
        out[0] = (float)(int8_t)(lo >> sh);
        out[1] = (float)(int8_t)(hi >> sh);
        out[2] = (float)(int8_t)(lo >> (sh + 8));
        out[3] = (float)(int8_t)(hi >> (sh + 8));
    }
}

template <int FMT>
__device__ __forceinline__ float load_scale(const void *scales, int64_t idx) {
    if constexpr (FMT == FMT_Q8) {
        return static_cast<const float *>(scales)[idx];
    } else {
        uint16_t bits = static_cast<const uint16_t *>(scales)[idx];
        return (float)__builtin_bit_cast(_Float16, bits) * 0.0625f;  // Q4 values carry *16
    }
}

template <int FMT, int T, int R>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvParams p) {
    constexpr int E = FmtTraits<FMT>::E;
    constexpr int STEP = 64 * E;  // K elements a wave covers per step
    constexpr int G = E / 4;      // float4 groups per lane per step
    extern __shared__ float4 xs[];  // [T][kc/4], permuted per step

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n_in = p.n_in;
    const int rows_per_block = kWaves * R;
    const int n_groups = (p.total_rows + rows_per_block - 1) / rows_per_block;
    const int kc4 = p.kc / 4;
    bool staged = false;

    for (int group = blockIdx.x; group < n_groups; group += gridDim.x) {
        // ---- this wave's rows: (job, local row) and base pointers ----
        const uint8_t *crow[R];  // the job's code plane
        int lrow[R];             // row within the job
        const void *srow[R];
        float *yrow[R];
        int ystride[R];
        bool valid[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            int g = group * rows_per_block + wave * R + r;
            valid[r] = g < p.total_rows;
            int j = 0;
#pragma unroll
            for (int q = 1; q < kMaxJobs; ++q)
                if (q < p.n_jobs && g >= p.row0[q]) j = q;
            int local = valid[r] ? g - p.row0[j] : 0;
            crow[r] = static_cast<const uint8_t *>(p.job[j].codes);
            lrow[r] = local;
            srow[r] = p.job[j].scales;
            if constexpr (FMT == FMT_Q8)
                srow[r] = static_cast<const float *>(p.job[j].scales) + (int64_t)local * (n_in / kBlock);
            if constexpr (FMT == FMT_Q4)
                srow[r] = static_cast<const uint16_t *>(p.job[j].scales) + (int64_t)local * (n_in / kBlock);
            yrow[r] = p.job[j].y + local;
            ystride[r] = p.job[j].n_out;
        }

        float acc[R][T];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int i = 0; i < T; ++i) acc[r][i] = 0.f;

        for (int c = 0; c < p.n_chunks; ++c) {
            const int k0 = c * p.kc;
            const int klen = min(p.kc, n_in - k0);
            // ---- stage x[:, k0 : k0+klen) into LDS (once if it all fits) ----
            if (p.n_chunks > 1 || !staged) {
                if (staged) __syncthreads();  // previous chunk fully consumed
                const int n4 = klen / 4;
                for (int idx = threadIdx.x; idx < T * n4; idx += kThreads) {
                    int i = idx / n4;
                    int f = idx - i * n4;
                    int k = 4 * f;
                    int s = k / STEP;
                    int rem = k - s * STEP;
                    int l = rem / E;
                    int g4 = (rem - l * E) / 4;
                    float4 v = *reinterpret_cast<const float4 *>(p.x + (int64_t)i * n_in + k0 + k);
                    xs[i * kc4 + (s * G + g4) * 64 + l] = v;
                }
                __syncthreads();
                staged = true;
            }

            const int steps = (klen + STEP - 1) / STEP;
            // prefetch step 0
            uint4 wv[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                int k = k0 + lane * E;
                bool act = valid[r] && (lane * E < klen);
                wv[r] = act ? *reinterpret_cast<const uint4 *>(crow[r] + code_offset<FMT>(lrow[r], k, n_in))
                            : make_uint4(0, 0, 0, 0);
            }
            for (int s = 0; s < steps; ++s) {
                const int kl = s * STEP + lane * E;  // chunk-local k of this lane
                const bool act = kl < klen;
                // issue the next step's loads before this step's math
                uint4 nv[R];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    int kn = kl + STEP;
                    bool a2 = valid[r] && (kn < klen);
                    nv[r] = a2 ? *reinterpret_cast<const uint4 *>(crow[r] + code_offset<FMT>(lrow[r], k0 + kn, n_in))
                               : make_uint4(0, 0, 0, 0);
                }
                if (act) {
                    float part[R][T];
#pragma unroll
                    for (int r = 0; r < R; ++r)
#pragma unroll
                        for (int i = 0; i < T; ++i) part[r][i] = 0.f;
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        float w[R][4];
#pragma unroll
                        for (int r = 0; r < R; ++r) dequant4<FMT>(wv[r], g, w[r]);
#pragma unroll
                        for (int i = 0; i < T; ++i) {
                            float4 xv = xs[i * kc4 + (s * G + g) * 64 + lane];
#pragma unroll
                            for (int r = 0; r < R; ++r) {
                                part[r][i] = fmaf(w[r][0], xv.x, part[r][i]);
                                part[r][i] = fmaf(w[r][1], xv.y, part[r][i]);
                                part[r][i] = fmaf(w[r][2], xv.z, part[r][i]);
                                part[r][i] = fmaf(w[r][3], xv.w, part[r][i]);
                            }
                        }
                    }
                    if constexpr (FMT == FMT_BF16) {
#pragma unroll
                        for (int r = 0; r < R; ++r)
#pragma unroll
                            for (int i = 0; i < T; ++i) acc[r][i] += part[r][i];
                    } else {
                        const int blk = (k0 + kl) / kBlock;
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            float sc = valid[r] ? load_scale<FMT>(srow[r], blk) : 0.f;
#pragma unroll
                            for (int i = 0; i < T; ++i) acc[r][i] = fmaf(sc, part[r][i], acc[r][i]);
                        }
                    }
                }
#pragma unroll
                for (int r = 0; r < R; ++r) wv[r] = nv[r];
            }
        }

        // ---- finish: wave reductions, lane 0 stores ----
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int i = 0; i < T; ++i) {
                float v = wave_sum(acc[r][i]);
                if (lane == 0 && valid[r] && i < p.t) yrow[r][(int64_t)i * ystride[r]] = v;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Streaming variant, used whenever all of x fits in LDS.  Each wave owns R
// rows and keeps P steps x R rows of 16-byte weight loads in flight in a
// register ring: a slot is refilled with the load P steps ahead as soon as it
// has been consumed, so HBM sees a continuous stream of requests.  All global
// reads are buffer loads whose descriptor spans exactly one row (or x):
// reads past the end return 0 without touching memory, so the main loop has
// no branches around loads and the in-order vector-memory counter lets the
// whole ring stay in flight.  x goes straight from L2 to LDS (buffer loads
// with the LDS bit, issued before the first weight loads; padding slots past
// n_in read as zeros), so staging x overlaps the start of the weight stream.
constexpr int kStreamWaves = 8;
constexpr int kStreamThreads = 64 * kStreamWaves;
constexpr int kStreamMaxLds = 160 * 1024;     // gfx950 LDS per workgroup
constexpr uint32_t kBufFlags = 0x00020000u;   // gfx9 raw buffer: 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, kBufFlags);
}

// bit-cast whole vectors: clang 22 turns bit casts of single ext_vector
// elements into copies of element 0
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <int FMT>
__device__ __forceinline__ float buf_scale(__amdgpu_buffer_rsrc_t r, uint32_t blk) {
    if constexpr (FMT == FMT_Q8) {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, blk * 4u, 0, 0));
    } else {
        const uint16_t bits = __builtin_amdgcn_raw_buffer_load_b16(r, blk * 2u, 0, 0);
        return (float)__builtin_bit_cast(_Float16, bits) * 0.0625f;  // Q4 values carry *16
    }
}

// Sum over the 64 lanes of a wave, result in every lane: DPP within each row
// of 16 lanes, then two cross-row exchanges.
__device__ __forceinline__ float wave_sum_dpp(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));  // row_half_mirror
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));  // row_mirror
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

// Steps (of 64*E elements) per x row in LDS: n_in rounded up to whole rings.
template <int FMT, int P>
__host__ __device__ constexpr int stream_steps(int n_in) {
    constexpr int STEP = 64 * FmtTraits<FMT>::E;
    return (n_in + STEP * P - 1) / (STEP * P) * P;
}

// GLU: the R rows of a wave are R / 2 output rows of the gate projection
// (jobs[0]) followed by the same R / 2 rows of the up projection (jobs[1]);
// the epilogue writes GELU(gate) * up to jobs[0].y.
template <int FMT, int T, int R, int P, bool GLU>
__global__ __launch_bounds__(kStreamThreads) void gemv_stream_kernel(GemvParams p) {
    constexpr int RO = GLU ? R / 2 : R;  // output rows per wave
    static_assert(!GLU || R % 2 == 0, "gate/up pairs");
    constexpr int E = FmtTraits<FMT>::E;
    constexpr int STEP = 64 * E;
    constexpr int G = E / 4;
    constexpr int SLOTS_PER_STEP = STEP / 4;  // float4 slots per step per x row
    constexpr int LOG_SPS = (E == 8) ? 7 : (E == 16) ? 8 : 9;
    static_assert((1 << LOG_SPS) == SLOTS_PER_STEP, "slot math");
    extern __shared__ float4 xs[];  // [T][steps_pad * SLOTS_PER_STEP]

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n_in = p.n_in;
    const int steps_pad = stream_steps<FMT, P>(n_in);
    const int xrow4 = steps_pad * SLOTS_PER_STEP;
    const int n_slots = T * xrow4;
    const int nb = n_in / kBlock;

    // ---- 1. x: L2 -> LDS, one 1 KiB wave access per instruction ----
    // slot q (float4) = row i, step s, group g4, lane l, holding
    // x[i][s*STEP + l*E + 4*g4 .. +4]; slots past n_in read zeros.
    {
        const __amdgpu_buffer_rsrc_t xrs = make_rsrc(p.x, (uint32_t)(T * n_in * 4));
        for (int q0 = wave * 64; q0 < n_slots; q0 += kStreamThreads) {
            const int q = q0 + lane;
            int i = 0, rem = q;
#pragma unroll
            for (int ii = 1; ii < T; ++ii)
                if (rem >= xrow4) rem -= xrow4, ++i;
            const int s = rem >> LOG_SPS;
            const int g4 = (rem & (SLOTS_PER_STEP - 1)) >> 6;
            const int k = s * STEP + (rem & 63) * E + g4 * 4;
            const uint32_t off = (k < n_in) ? (uint32_t)((i * n_in + k) * 4) : 0x7FFFFFF0u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xrs, (__attribute__((address_space(3))) void *)(xs + q0), 16, off, 0, 0, 0);
        }
    }

    // ---- 2. this wave's rows: one buffer descriptor per row ----
    __amdgpu_buffer_rsrc_t crs[R], srs[R];
    float *yrow[R];
    int ystride[R];
    bool valid[R];
    uint32_t rsub[R];  // Q4: the row's 64-byte slot within a segment
    const int row_base = ((int)blockIdx.x * kStreamWaves + wave) * RO;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int g = row_base + (GLU ? r % RO : r);
        valid[r] = g < p.total_rows;
        int j = GLU ? r / RO : 0;
        if constexpr (!GLU) {
#pragma unroll
            for (int q = 1; q < kMaxJobs; ++q)
                if (q < p.n_jobs && g >= p.row0[q]) j = q;
        }
        const int local = valid[r] ? g - p.row0[j] : 0;
        if constexpr (FMT == FMT_Q4) {
            // the row's 16-row tile; its segments sit 1 KiB apart
            const int64_t tb = q4_plane_bytes(16, nb);
            crs[r] = make_rsrc(static_cast<const uint8_t *>(p.job[j].codes) + (int64_t)(local >> 4) * tb,
                               valid[r] ? (uint32_t)tb : 0u);
            rsub[r] = (uint32_t)(local & 15) << 6;
        } else {
            const uint32_t rb = valid[r] ? (uint32_t)row_bytes<FMT>(n_in) : 0u;
            crs[r] = make_rsrc(static_cast<const uint8_t *>(p.job[j].codes) + (int64_t)local * row_bytes<FMT>(n_in),
                               rb);
        }
        if constexpr (FMT == FMT_Q8)
            srs[r] = make_rsrc(static_cast<const float *>(p.job[j].scales) + (int64_t)local * nb,
                               valid[r] ? (uint32_t)(nb * 4) : 0u);
        else if constexpr (FMT == FMT_Q4)
            srs[r] = make_rsrc(static_cast<const uint16_t *>(p.job[j].scales) + (int64_t)local * nb,
                               valid[r] ? (uint32_t)(nb * 2) : 0u);
        else
            srs[r] = crs[r];
        yrow[r] = p.job[j].y + local;
        ystride[r] = p.job[j].n_out;
    }

    // ---- 3. prologue: P steps of weight (and scale) loads in flight ----
    uint4 buf[P][R];
    float sbuf[P][R];
    auto issue = [&](int u, int s) {
        const int k = s * STEP + lane * E;  // reads at k >= n_in return zeros
        const uint32_t off = (uint32_t)code_byte<FMT>(k);
        const int blk = k / kBlock;  // Q4: one block per lane
        const uint32_t qoff = ((uint32_t)(blk >> 2) << 10) + ((uint32_t)(blk & 3) << 4);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if constexpr (FMT == FMT_Q4)
                buf[u][r] = buf_load16(crs[r], blk < nb ? qoff + rsub[r] : 0x7FFFFFF0u);
            else
                buf[u][r] = buf_load16(crs[r], off);
            if constexpr (FMT != FMT_BF16) sbuf[u][r] = buf_scale<FMT>(srs[r], (uint32_t)(k / kBlock));
        }
    };
#pragma unroll
    for (int u = 0; u < P; ++u) issue(u, u);
    __syncthreads();  // x is in LDS (the compiler waits for the LDS loads only)

    // ---- 4. main loop: ring of P slots, no branches around loads ----
    float acc[R][T];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < T; ++i) acc[r][i] = 0.f;

    for (int s0 = 0; s0 < steps_pad; s0 += P) {
#pragma unroll
        for (int u = 0; u < P; ++u) {
            const int s = s0 + u;
            float part[R][T];
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int i = 0; i < T; ++i) part[r][i] = 0.f;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float w[R][4];
#pragma unroll
                for (int r = 0; r < R; ++r) dequant4<FMT>(buf[u][r], g, w[r]);
#pragma unroll
                for (int i = 0; i < T; ++i) {
                    const float4 xv = xs[i * xrow4 + (s * G + g) * 64 + lane];
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        part[r][i] = fmaf(w[r][0], xv.x, part[r][i]);
                        part[r][i] = fmaf(w[r][1], xv.y, part[r][i]);
                        part[r][i] = fmaf(w[r][2], xv.z, part[r][i]);
                        part[r][i] = fmaf(w[r][3], xv.w, part[r][i]);
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int i = 0; i < T; ++i) {
                    if constexpr (FMT == FMT_BF16)
                        acc[r][i] += part[r][i];
                    else
                        acc[r][i] = fmaf(sbuf[u][r], part[r][i], acc[r][i]);
                }
            issue(u, s + P);  // refill this slot P steps ahead
        }
    }

    // ---- 5. wave reductions; lane 0 stores ----
    if constexpr (GLU) {
#pragma unroll
        for (int r = 0; r < RO; ++r) {
#pragma unroll
            for (int i = 0; i < T; ++i) {
                const float vg = wave_sum_dpp(acc[r][i]);
                const float vu = wave_sum_dpp(acc[RO + r][i]);
                if (lane == 0 && valid[r]) yrow[r][(int64_t)i * ystride[r]] = gelu(vg) * vu;
            }
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int i = 0; i < T; ++i) {
                const float v = wave_sum_dpp(acc[r][i]);
                if (lane == 0 && valid[r]) yrow[r][(int64_t)i * ystride[r]] = v;
            }
        }
    }
}

template <int FMT, int P>
size_t stream_lds_bytes(int t, int n_in) {
    constexpr int STEP = 64 * FmtTraits<FMT>::E;
    return (size_t)t * stream_steps<FMT, P>(n_in) * STEP * sizeof(float);
}

template <int FMT, int T, int R, int P, bool GLU>
hipError_t launch_stream(const GemvParams &p, hipStream_t s) {
    const size_t lds = stream_lds_bytes<FMT, P>(T, p.n_in);
    auto kern = gemv_stream_kernel<FMT, T, R, P, GLU>;
    if (lds > 64 * 1024) {
        // the attribute belongs to the kernel on the current device: raised
        // once per device (bit d of `raised`; a benign race, it is idempotent)
        static std::atomic<uint64_t> raised{0};
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
        if (!bit || !(raised.load(std::memory_order_relaxed) & bit)) {
            e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                    kStreamMaxLds);
            if (e != hipSuccess) return e;
            raised.fetch_or(bit, std::memory_order_relaxed);
        }
    }
    const int rows_per_block = kStreamWaves * (GLU ? R / 2 : R);
    const int grid = (p.total_rows + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kStreamThreads), lds, s, p);
    return hipGetLastError();
}

// Ring depth for a row of `steps` 16-byte lane loads: 4 where it divides the
// steps, else 2 (rows are padded to whole rings with zero reads).  Measured
// under graph replay: the fused bf16 decode (8 steps) 11.0 us with 8 loads in
// flight per row, 10.4 with 4, 11.6 with 2; the Q8 down projection (14
// steps) 16.5 us with 8, 15.8 with 2.
inline int stream_ring(int steps) { return steps % 4 == 0 ? 4 : 2; }

constexpr int kStreamLongRow = 8192;  // inputs per row from which bf16 / Q8 rows go two per wave

template <int FMT, int T, bool GLU = false>
hipError_t try_stream(const GemvParams &p, hipStream_t s, bool *taken) {
    constexpr int STEP = 64 * FmtTraits<FMT>::E;
    const int steps = (p.n_in + STEP - 1) / STEP;
    const int P = stream_ring(steps);
    // bytes of every buffer descriptor (x and one row) stay far below 2^31
    *taken = (int64_t)T * p.n_in * 4 < (1ll << 31);
    // rows per wave: Q4 rows are short, so 4 give a workgroup enough weight
    // bytes next to its copy of x; bf16 and Q8 take one (Q8 gate/up shape
    // under graph replay: 28.0 us with one row per wave, 28.7 with two;
    // four were ~25 % slower) -- with GLU at least one gate/up pair.  Rows
    // of kStreamLongRow inputs or more take two, which halves the copies of
    // the (long) x per weight row: the Q8 down projection [4096 x 14336]
    // 15.6 -> 14.95 us; four rows 19.5 us.
    constexpr int R0 = (FMT == FMT_Q4) ? 4 : 1;
    constexpr int R = GLU && R0 < 2 ? 2 : R0;
    if (!*taken) return hipSuccess;
    if constexpr (R == 1) {
        if (p.n_in >= kStreamLongRow) {
            if (P == 4 && stream_lds_bytes<FMT, 4>(T, p.n_in) <= kStreamMaxLds)
                return launch_stream<FMT, T, 2, 4, GLU>(p, s);
            if (P == 2 && stream_lds_bytes<FMT, 2>(T, p.n_in) <= kStreamMaxLds)
                return launch_stream<FMT, T, 2, 2, GLU>(p, s);
        }
    }
    if (P == 4 && stream_lds_bytes<FMT, 4>(T, p.n_in) <= kStreamMaxLds)
        return launch_stream<FMT, T, R, 4, GLU>(p, s);
    if (P == 2 && stream_lds_bytes<FMT, 2>(T, p.n_in) <= kStreamMaxLds)
        return launch_stream<FMT, T, R, 2, GLU>(p, s);
    *taken = false;
    return hipSuccess;
}

// The gate/up step on the streaming kernel; *taken is false when x does not
// fit in LDS (the caller then uses the matrix-core kernel).
template <int FMT>
hipError_t try_stream_glu(const GemvParams &p, hipStream_t s, bool *taken) {
    switch (p.t) {
        case 1: return try_stream<FMT, 1, true>(p, s, taken);
        case 2: return try_stream<FMT, 2, true>(p, s, taken);
        case 3: return try_stream<FMT, 3, true>(p, s, taken);
        case 4: return try_stream<FMT, 4, true>(p, s, taken);
        case 5: return try_stream<FMT, 5, true>(p, s, taken);
        case 6: return try_stream<FMT, 6, true>(p, s, taken);
        case 7: return try_stream<FMT, 7, true>(p, s, taken);
        case 8: return try_stream<FMT, 8, true>(p, s, taken);
        default: *taken = false; return hipErrorInvalidValue;
    }
}

template <int FMT, int T>
hipError_t launch_t(const GemvParams &p, int cu_count, hipStream_t s) {
    constexpr int R = (T <= 2) ? 4 : 2;
    const int rows_per_block = kWaves * R;
    const int n_groups = (p.total_rows + rows_per_block - 1) / rows_per_block;
    const size_t lds = (size_t)T * p.kc * sizeof(float);
    // One chunk: persistent grid (x staged once per workgroup).  Several
    // chunks: one row group per workgroup.
    int grid = n_groups;
    if (p.n_chunks == 1) grid = min(n_groups, cu_count * 8);
    hipLaunchKernelGGL((gemv_kernel<FMT, T, R>), dim3(grid), dim3(kThreads), lds, s, p);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(GemvParams &p, int cu_count, hipStream_t s) {
    constexpr int STEP = 64 * FmtTraits<FMT>::E;
    {
        bool taken = false;
        hipError_t e = hipSuccess;
        switch (p.t) {
            case 1: e = try_stream<FMT, 1>(p, s, &taken); break;
            case 2: e = try_stream<FMT, 2>(p, s, &taken); break;
            case 3: e = try_stream<FMT, 3>(p, s, &taken); break;
            case 4: e = try_stream<FMT, 4>(p, s, &taken); break;
            case 5: e = try_stream<FMT, 5>(p, s, &taken); break;
            case 6: e = try_stream<FMT, 6>(p, s, &taken); break;
            case 7: e = try_stream<FMT, 7>(p, s, &taken); break;
            case 8: e = try_stream<FMT, 8>(p, s, &taken); break;
            default: break;
        }
        if (taken || e != hipSuccess) return e;
    }
    // K chunk: as much of x as the LDS budget allows, in whole steps.
    int kc = kXLdsBytes / (int)(p.t * sizeof(float));
    kc = (kc / STEP) * STEP;
    if (kc < STEP) kc = STEP;
    if (kc >= p.n_in) kc = ((p.n_in + STEP - 1) / STEP) * STEP;
    p.kc = kc;
    p.n_chunks = (p.n_in + kc - 1) / kc;
    switch (p.t) {
        case 1: return launch_t<FMT, 1>(p, cu_count, s);
        case 2: return launch_t<FMT, 2>(p, cu_count, s);
        case 3: return launch_t<FMT, 3>(p, cu_count, s);
        case 4: return launch_t<FMT, 4>(p, cu_count, s);
        case 5: return launch_t<FMT, 5>(p, cu_count, s);
        case 6: return launch_t<FMT, 6>(p, cu_count, s);
        case 7: return launch_t<FMT, 7>(p, cu_count, s);
        case 8: return launch_t<FMT, 8>(p, cu_count, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Which decode kernel a call takes.  The streaming kernel's f32 vector work
// per weight byte (2t flops per element plus the dequantisation) grows with
// t; the matrix-core kernel's does not, but it keeps a whole step of loads in
// flight only across the 16-row tiles a workgroup owns, so with few tiles
// per compute unit (short or few jobs) it streams slowly.  Measured per call
// (us, streaming / matrix-core, one box):
//   Q4 2 x [17408, 5120] (136 rows per CU): t = 1 36.5 / 25.4, t = 8 337 / 26.0
//   Q4 [4096 + 1024 + 1024, 4096] (24):     t = 1 8.7 / 20.0, t = 8 19.7 / 22.9
//   Q4 [4096, 14336] (16):                   t = 2 22.0 / 31.7, t = 4 38.2 / 33.5
//   Q4 [1024, 4096] (4):                     t = 4 11.6 / 13.2, t = 8 18.6 / 14.1
//   Q8 2 x [14336, 4096] (112):              t = 2 31.3 / 32.8, t = 4 44.3 / 32.9
//   Q8 [4096, 14336] (16):                   t = 4 41.8 / 55.0, t = 8 65.9 / 57.8
//   Q8 2 x [1024, 4096] (8):                 t = 8 10.7 / 19.5
// bf16 always streams (its vector work is a shift and an FMA per element).
static bool decode_on_matrix_cores(int fmt, int t, int n_in, const KJob *jobs, int n_jobs, int cu_count) {
    int64_t rows = 0;
    for (int j = 0; j < n_jobs; ++j) rows += jobs[j].n_out;
    const int64_t per_cu = rows / (cu_count > 0 ? cu_count : 1);
    if (fmt == FMT_Q4) return per_cu >= 64 || (t >= 4 && n_in >= 8192) || (t >= 8 && per_cu <= 8);
    if (fmt == FMT_Q8) return (per_cu >= 64 && t >= 4) || (t >= 8 && n_in >= 8192);
    return false;
}

hipError_t launch_gemv(int fmt, const float *x, int t, int n_in, const KJob *jobs, int n_jobs,
                       int cu_count, hipStream_t s, bool glu) {
    if (t < 1 || t > kGemvMaxT || n_jobs < 1 || n_jobs > kMaxJobs) return hipErrorInvalidValue;
    if (glu && (n_jobs != 2 || jobs[0].n_out != jobs[1].n_out)) return hipErrorInvalidValue;
    // IL_DECODE=valu|mfma pins the kernel family (both compute the same sums)
    bool use_mfma = decode_on_matrix_cores(fmt, t, n_in, jobs, n_jobs, cu_count);
    if (const char *force = getenv("IL_DECODE")) {
        if (!strcmp(force, "mfma")) use_mfma = true;
        if (!strcmp(force, "valu")) use_mfma = false;
    }
    if (use_mfma && gemv_mfma_fits(fmt, t, n_in, jobs, n_jobs))
        return launch_gemv_mfma(fmt, x, t, n_in, jobs, n_jobs, cu_count, s, glu);
    GemvParams p{};
    p.x = x;
    p.t = t;
    p.n_in = n_in;
    p.n_jobs = n_jobs;
    if (glu) {
        // both projections are numbered from row 0; the pairs are the rows
        p.job[0] = jobs[0];
        p.job[1] = jobs[1];
        for (int j = 0; j <= kMaxJobs; ++j) p.row0[j] = 0;
        p.total_rows = jobs[0].n_out;
        bool taken = false;
        hipError_t e = hipSuccess;
        switch (fmt) {
            case FMT_BF16: e = try_stream_glu<FMT_BF16>(p, s, &taken); break;
            case FMT_Q8: e = try_stream_glu<FMT_Q8>(p, s, &taken); break;
            case FMT_Q4: e = try_stream_glu<FMT_Q4>(p, s, &taken); break;
            default: return hipErrorInvalidValue;
        }
        if (taken || e != hipSuccess) return e;
        if (!gemv_mfma_fits(fmt, t, n_in, jobs, n_jobs)) return hipErrorInvalidValue;
        return launch_gemv_mfma(fmt, x, t, n_in, jobs, n_jobs, cu_count, s, true);
    }
    int rows = 0;
    for (int j = 0; j < n_jobs; ++j) {
        p.job[j] = jobs[j];
        p.row0[j] = rows;
        rows += jobs[j].n_out;
    }
    for (int j = n_jobs; j <= kMaxJobs; ++j) p.row0[j] = rows;
    p.total_rows = rows;
    switch (fmt) {
        case FMT_BF16: return launch_fmt<FMT_BF16>(p, cu_count, s);
        case FMT_Q8: return launch_fmt<FMT_Q8>(p, cu_count, s);
        case FMT_Q4: return launch_fmt<FMT_Q4>(p, cu_count, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace il
