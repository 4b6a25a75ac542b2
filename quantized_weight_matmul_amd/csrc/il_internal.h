// il_internal.h -- declarations shared by the library's translation units.
//
// Device layouts (written by the upload/repack stage, read by every kernel):
//   BF16 : codes  = uint16 [n_out][n_in]          (the host layout, row-major)
//   Q8   : codes  = int8   [n_out][n_in]          (row-major, K contiguous)
//          scales = float  [n_out][n_in/32]
//   Q4   : codes  = uint8, tile-major: tiles of 16 rows, each a run of
//                  64-byte segments per row (128 elements, 4 blocks):
//                  block b of row r (16 bytes) at q4_block_offset(r, b, nb);
//                  element 2j of a block in the low nibble of its byte j,
//                  stored as code ^ 8, i.e. the 4-bit two's complement of
//                  code - 8; rows padded to 16 and blocks to 4 with zero
//                  bytes (= code 8, value 0)
//          scales = uint16 [n_out][n_in/32]       (f16 bits)
// Every bf16 / Q8 code row starts 16-byte aligned (n_in % 32 == 0), so one
// lane can fetch 16 bytes of a row with a single global_load_dwordx4.  A Q4
// tile's 16 rows x 64 bytes of one segment are one contiguous 1 KiB: the
// matrix-core decode kernel's wave fetches it with one instruction.
// Q8/Q4 also keep a second copy of the scales in tiles of 16 rows x 4 blocks
// (the order the matrix-core decode kernel reads them in, one 128- or
// 256-byte run per tile and step):
//   scales_t[((row / 16) * nb4 + b / 4) * 64 + (row % 16) * 4 + b % 4],
//   nb4 = ceil(nb / 4), rows padded to a multiple of 16 (padding is zero).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace il {

enum : int { FMT_BF16 = 0, FMT_Q8 = 1, FMT_Q4 = 2 };
constexpr int kBlock = 32;     // quantisation block (elements)
constexpr int kMaxJobs = 8;    // jobs per kernel launch (kernarg table)
constexpr int kGemvMaxT = 8;   // t <= kGemvMaxT runs the decode kernels
constexpr int kVerifyMaxT = 32;  // largest t the matrix-core decode kernel takes in wide mode
constexpr int kVerifySliceMaxT = 128;  // Q4 under IL_PREFILL=verify: wide mode in slices of <= kVerifyMaxT tokens up to here
constexpr int kMidMaxT = 128;  // Q8/Q4 GEMM with all tokens in one unit (the mid-size plan) up to here

struct Weight {
    int fmt;
    int device;
    int64_t n_out;
    int64_t n_in;
    int64_t host_bytes;  // WeightRef::bytes of the host format
    void *alloc;         // single device allocation holding both planes
    const void *codes;
    const void *scales;    // nullptr for BF16
    const void *scales_t;  // tiled copy of the scales; nullptr for BF16
};

// Index of the scale of (row, block b) in the tiled scale plane.
__host__ __device__ inline int64_t tiled_scale_index(int64_t row, int64_t b, int64_t nb4) {
    return (((row >> 4) * nb4 + (b >> 2)) << 6) + ((row & 15) << 2) + (b & 3);
}
__host__ __device__ inline int64_t tiled_scale_count(int64_t n_out, int64_t nb) {
    return (n_out + 15) / 16 * ((nb + 3) / 4) * 64;
}

// Byte offset of Q4 block b of row r (16 bytes) in the tile-major code plane,
// and the plane's size (nb = blocks per row).
__host__ __device__ inline int64_t q4_block_offset(int64_t r, int64_t b, int64_t nb) {
    return (((r >> 4) * ((nb + 3) >> 2) + (b >> 2)) << 10) + ((r & 15) << 6) + ((b & 3) << 4);
}
__host__ __device__ inline int64_t q4_plane_bytes(int64_t n_out, int64_t nb) {
    return (n_out + 15) / 16 * ((nb + 3) / 4) * 1024;
}

// GELU(v) = v * Phi(v) = 0.5 v (1 + erf(v / sqrt 2)), the activation of the
// fused gate/up step (gelu_mul on the oxinfer 0.0.1 src/drafter.rs page,
// which does not print it; this is the plain definition).
__device__ __forceinline__ float gelu(float v) { return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f)); }

// One job as the kernels see it.
struct KJob {
    const void *codes;
    const void *scales;
    const void *scales_t;
    float *y;
    int n_out;
};

// ---- upload / repack (il_repack.hip) ----
enum : int { SRC_F32 = 0, SRC_BF16 = 1 };  // element type of a weight to quantise
// f32 / bf16 [n_out][n_in] (device) -> the Q8 / Q4 device planes.
hipError_t launch_quantize(int fmt, int src_type, const void *src, uint8_t *codes, void *scales, void *scales_t,
                           int64_t n_out, int64_t n_in, hipStream_t s);
// Q8 / Q4 device planes -> host-format blocks in `out` (device memory).
hipError_t launch_unrepack(int fmt, const void *codes, const void *scales, uint8_t *out, int64_t n_out,
                           int64_t n_in, hipStream_t s);
hipError_t launch_repack_q8(const uint8_t *staging, int8_t *codes, float *scales, float *scales_t,
                            int64_t n_out, int64_t n_in, hipStream_t s);
hipError_t launch_repack_q4(const uint8_t *staging, uint8_t *codes, uint16_t *scales, uint16_t *scales_t,
                            int64_t n_out, int64_t n_in, hipStream_t s);

// Every launcher below takes `glu`: when set, jobs[0] and jobs[1] are the
// gate and up projections of one feed-forward step (same fmt and n_out,
// n_jobs == 2) and the launch writes y = GELU(x G^T) * (x U^T) into
// jobs[0].y only; g and u never reach memory.

// ---- decode GEMV, t <= kGemvMaxT (il_gemv.hip) ----
// All jobs share fmt, x and n_in; n_jobs <= kMaxJobs.
hipError_t launch_gemv(int fmt, const float *x, int t, int n_in, const KJob *jobs, int n_jobs,
                       int cu_count, hipStream_t s, bool glu = false);

// ---- decode GEMV on the bf16 matrix cores, t <= kGemvMaxT (il_gemv_mfma.hip) ----
// Same contract as launch_gemv.  gemv_mfma_fits says whether the kernel's
// 32-bit buffer offsets cover x and every job's weight planes.
bool gemv_mfma_fits(int fmt, int t, int n_in, const KJob *jobs, int n_jobs);
hipError_t launch_gemv_mfma(int fmt, const float *x, int t, int n_in, const KJob *jobs, int n_jobs,
                            int cu_count, hipStream_t s, bool glu = false);

// ---- mid-size t (kGemvMaxT < t <= kVerifyMaxT) on the same kernel, "wide"
// mode: up to 32 tokens per weight operand.  For t <= kWideF32MaxT the kernel
// rounds x (f32, row-major [t][n_in]) to bf16 as it loads it and xb may be
// null; above, xb must be bf16(x) (row-major, from the GEMM's pre-pass) ----
constexpr int kWideF32MaxT = 16;
bool verify_mfma_fits(int fmt, int t, int n_in, const KJob *jobs, int n_jobs);
hipError_t launch_verify_mfma(int fmt, const float *x, const uint16_t *xb, int t, int n_in, const KJob *jobs,
                              int n_jobs, int cu_count, hipStream_t s, bool glu = false);

// ---- prefill GEMM, t > kGemvMaxT (il_gemm.hip) ----
// Bytes of device scratch launch_gemm needs for this call (the bf16 copy of
// x its units read; for Q8/Q4 at kVerifyMaxT < t <= kMidMaxT also the
// counters and chunk sums of the units it splits over K), 0 when the call
// takes a path that rounds x itself.
size_t gemm_scratch_bytes(int fmt, int t, int n_in, const KJob *jobs, int n_jobs, bool glu = false);
// xb_scratch: gemm_scratch_bytes(...) bytes of device memory, 256-byte
// aligned, that nothing else uses until the stream has passed this call (may
// be null when that size is 0).  Enqueues the x -> bf16 pre-pass and one GEMM
// launch (or the wide-mode launches of mid-size t).
// after_prepass: when not null, recorded on s between the pre-pass and the
// GEMM launch (device timing of the two kernels apart).
hipError_t launch_gemm(int fmt, const float *x, void *xb_scratch, int t, int n_in, const KJob *jobs, int n_jobs,
                       int cu_count, hipStream_t s, bool glu = false, hipEvent_t after_prepass = nullptr);
// The device's static scratch of il_matmul_noalloc (static_scratch_bytes()
// bytes, 256-byte aligned, shared by every call on that device): its device
// address, looked up on the first call for the device, which must be current.
size_t static_scratch_bytes();
hipError_t static_scratch(int device, void **ptr);

// ---- plain streaming read of device memory (il_probe.hip) ----
// Workgroups of `waves` waves each read `chunk` bytes (16 per lane per load,
// `depth` loads in flight per lane); sink gets one word per workgroup.
hipError_t launch_read_probe(const void *buf, int64_t bytes, int64_t chunk, int waves, int depth, uint32_t *sink,
                             hipStream_t s);

// ---- centroid-masked LM head (il_lmhead.hip) ----
// x [t][h] (t <= kGemvMaxT); centroids: a bf16 job [C][h]; embed bf16 [V][h]
// with V % C == 0; ordering [V] (entries < V); 1 <= k <= C.  Writes token[t]
// and, when not null, clusters[t][k] (visiting order) and score[t].
// Dynamic LDS budget of the select kernel: 160 KiB less 8 KiB kept for its
// static arrays (histograms and per-wave results, about 4.2 KiB).
constexpr size_t kLmHeadMaxLds = 152 * 1024;
size_t lm_head_lds_bytes(int n_c, int h, int k);
// workspace: lm_head_workspace_bytes(t, C, k) bytes of device memory, or
// null for a stream-ordered allocation.
size_t lm_head_workspace_bytes(int t, int n_c, int k);
hipError_t launch_lm_head(const float *x, int t, int h, const KJob &centroids, const uint16_t *embed, int vocab,
                          const uint32_t *ordering, int k, int *token, int *clusters, float *score, void *workspace,
                          int cu_count, hipStream_t s);

}  // namespace il
