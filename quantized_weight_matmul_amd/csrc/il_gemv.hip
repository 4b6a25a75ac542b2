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

// Byte offset of element k within a code row.
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
        const uint8_t *crow[R];
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
            crow[r] = static_cast<const uint8_t *>(p.job[j].codes) + (int64_t)local * row_bytes<FMT>(n_in);
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
                wv[r] = act ? *reinterpret_cast<const uint4 *>(crow[r] + code_byte<FMT>(k))
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
                    nv[r] = a2 ? *reinterpret_cast<const uint4 *>(crow[r] + code_byte<FMT>(k0 + kn))
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

hipError_t launch_gemv(int fmt, const float *x, int t, int n_in, const KJob *jobs, int n_jobs,
                       int cu_count, hipStream_t s) {
    if (t < 1 || t > kGemvMaxT || n_jobs < 1 || n_jobs > kMaxJobs) return hipErrorInvalidValue;
    GemvParams p{};
    p.x = x;
    p.t = t;
    p.n_in = n_in;
    p.n_jobs = n_jobs;
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
