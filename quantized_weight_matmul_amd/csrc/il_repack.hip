// il_repack.hip -- the upload/repack stage (Backend::upload on the oxinfer
// 0.0.0 src/gpu.rs page: "prepares device-side state for a weight matrix").
//
// The host bytes are first copied to a device staging buffer; these kernels
// then split the packed array-of-blocks formats into a code plane (Q8 row-major,
// Q4 tile-major) and a separate scale plane, plus a tiled copy of the scales
// (layouts in il_internal.h).  Integer byte moves only: every value is preserved bit for
// bit.  BF16 needs no kernel, its host layout is already the device layout.
// Also here: the quantiser that builds the Q8 / Q4 planes from f32 or bf16
// weights on upload, and the inverse repack that writes a weight back in its
// host format.
#include "il_internal.h"

namespace il {
namespace {

// One thread per 36-byte Q8 block {f32 scale; int8 q[32]}.  Blocks start
// 4-byte aligned (36 = 9 dwords), so the block is read as 9 dwords.
__global__ void repack_q8_kernel(const uint32_t *__restrict__ staging,
                                 uint4 *__restrict__ codes, float *__restrict__ scales,
                                 float *__restrict__ scales_t, int64_t n_blocks, int64_t nb) {
    int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= n_blocks) return;
    const uint32_t *src = staging + b * 9;
    uint32_t d[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) d[i] = src[i];
    scales[b] = __builtin_bit_cast(float, d[0]);
    scales_t[tiled_scale_index(b / nb, b % nb, (nb + 3) / 4)] = __builtin_bit_cast(float, d[0]);
    // block b covers codes[b*32 .. b*32+31]: two 16-byte stores
    codes[2 * b] = make_uint4(d[1], d[2], d[3], d[4]);
    codes[2 * b + 1] = make_uint4(d[5], d[6], d[7], d[8]);
}

// One thread per 18-byte Q4 block {u16 f16 scale; u8 qs[16]}.  Blocks start
// 2-byte aligned, so the block is read as 9 halfwords.  Each nibble is stored
// XOR 8 (two's complement of code - 8), which lets the kernels sign-extend it
// with one byte-select conversion; the 16 code bytes go to the block's place
// in the tile-major plane.
__global__ void repack_q4_kernel(const uint16_t *__restrict__ staging,
                                 uint8_t *__restrict__ codes, uint16_t *__restrict__ scales,
                                 uint16_t *__restrict__ scales_t, int64_t n_blocks, int64_t nb) {
    int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= n_blocks) return;
    const uint16_t *src = staging + b * 9;
    uint16_t h[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) h[i] = src[i];
    scales[b] = h[0];
    scales_t[tiled_scale_index(b / nb, b % nb, (nb + 3) / 4)] = h[0];
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        w[i] = ((uint32_t)h[1 + 2 * i] | ((uint32_t)h[2 + 2 * i] << 16)) ^ 0x88888888u;
    *reinterpret_cast<uint4 *>(codes + q4_block_offset(b / nb, b % nb, nb)) = make_uint4(w[0], w[1], w[2], w[3]);
}

// ---- quantise on upload: full-precision weights -> the Q8 / Q4 planes ----
// Per 32-element block of a row, with amax = max |w| over the block
// (symmetric absmax scaling; the pages import QMatrix / Q4Matrix without
// showing how they are built, so this rule is a reading):
//   Q8: s = amax / 127 (f32); q = rint(w / s) clamped to [-127, 127];
//   Q4: s = binary16(amax / 7), round to nearest even, saturated at 65504;
//       q = rint(w / s) clamped to [-8, 7] against that stored scale, and the
//       nibble holds q's 4-bit two's complement (= code ^ 8, code = q + 8);
//   a zero scale stores 0 and all-zero values.
// Divisions are the correctly rounded f32 division, rint rounds half to even.
// One thread per block, all 32 of its elements (eight 16-byte loads of f32,
// four of bf16), so amax needs no lane exchanges.  Q8: in row order, so that
// a wave's code stores are one contiguous 2 KiB run (8 lanes per block, 4
// elements each, measured 64.9 against 63.6 us on f32 [14336, 4096]).
template <int SRC>
__device__ __forceinline__ void load_block(const void *__restrict__ src, int64_t e0, float (&v)[kBlock]) {
    if constexpr (SRC == SRC_F32) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 f = static_cast<const float4 *>(src)[e0 / 4 + i];
            v[4 * i] = f.x, v[4 * i + 1] = f.y, v[4 * i + 2] = f.z, v[4 * i + 3] = f.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 h = static_cast<const uint4 *>(src)[e0 / 8 + i];  // bf16 -> f32 is exact
            const uint32_t w[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                v[8 * i + 2 * k] = __builtin_bit_cast(float, w[k] << 16);
                v[8 * i + 2 * k + 1] = __builtin_bit_cast(float, w[k] & 0xFFFF0000u);
            }
        }
    }
}

template <int SRC>
__global__ __launch_bounds__(256) void quantize_q8_kernel(const void *__restrict__ src, int8_t *__restrict__ codes,
                                                          float *__restrict__ scales, float *__restrict__ scales_t,
                                                          int64_t n_blocks, int64_t nb) {
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= n_blocks) return;
    const int64_t e0 = b * kBlock;
    float v[kBlock];
    load_block<SRC>(src, e0, v);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < kBlock; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const float s = amax / 127.0f;
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t packed = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float q = 0.f;
            if (s != 0.f) q = fminf(fmaxf(rintf(v[4 * j + i] / s), -127.f), 127.f);
            packed |= (uint32_t)(uint8_t)(int8_t)q << (8 * i);
        }
        w[j] = packed;
    }
    uint4 *dst = reinterpret_cast<uint4 *>(codes + e0);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    scales[b] = s;
    scales_t[tiled_scale_index(b / nb, b % nb, (nb + 3) / 4)] = s;
}

// Q4, in the order of the tile-major plane: workgroup (16-row tile, group of
// 4 segments); wave w takes segment 4 group + w, lane l the block of row l / 4
// and segment slot l % 4, all 32 of its elements (one thread per block, amax
// without lane exchanges), so that the wave's code stores are one contiguous
// 1 KiB run of the plane and its tiled scales one 128-byte run (in row
// order the stores landed in 64-byte runs: 101 against 88 us on f32
// [17408, 5120]).
template <int SRC>
__global__ __launch_bounds__(256) void quantize_q4_kernel(const void *__restrict__ src, uint8_t *__restrict__ codes,
                                                          uint16_t *__restrict__ scales, uint16_t *__restrict__ scales_t,
                                                          int64_t n_out, int64_t nb) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t nb4 = (nb + 3) / 4;
    const int64_t ngroups = (nb4 + 3) / 4;
    const int64_t tile = blockIdx.x / ngroups, grp = blockIdx.x - tile * ngroups;
    const int64_t seg = grp * 4 + wave;
    const int64_t row = tile * 16 + (lane >> 2);
    const int64_t blk = seg * 4 + (lane & 3);
    if (seg >= nb4 || row >= n_out || blk >= nb) return;  // padding: the planes were cleared
    const int64_t e0 = (row * nb + blk) * kBlock;
    float v[kBlock];
    load_block<SRC>(src, e0, v);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < kBlock; ++i) amax = fmaxf(amax, fabsf(v[i]));
    uint16_t sb = __builtin_bit_cast(uint16_t, (_Float16)(amax / 7.0f));
    if (sb == 0x7C00u) sb = 0x7BFFu;
    const float sc = (float)__builtin_bit_cast(_Float16, sb);
    // element 2j in the low nibble of byte j; the nibble is q's 4-bit two's
    // complement (= code ^ 8)
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < kBlock; ++i) {
        float q = 0.f;
        if (sc != 0.f) q = fminf(fmaxf(rintf(v[i] / sc), -8.f), 7.f);
        w[i >> 3] |= ((uint32_t)(int)q & 0xFu) << (4 * (i & 7));
    }
    *reinterpret_cast<uint4 *>(codes + q4_block_offset(row, blk, nb)) = make_uint4(w[0], w[1], w[2], w[3]);
    scales[row * nb + blk] = sb;
    scales_t[tiled_scale_index(row, blk, nb4)] = sb;
}

// ---- download: the device planes back to the host block formats ----
// One thread per block, the inverse of the repack kernels above.
__global__ void unrepack_q8_kernel(const uint4 *__restrict__ codes, const float *__restrict__ scales,
                                   uint32_t *__restrict__ out, int64_t n_blocks) {
    int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= n_blocks) return;
    const uint4 c0 = codes[2 * b], c1 = codes[2 * b + 1];
    uint32_t *dst = out + b * 9;
    dst[0] = __builtin_bit_cast(uint32_t, scales[b]);
    dst[1] = c0.x, dst[2] = c0.y, dst[3] = c0.z, dst[4] = c0.w;
    dst[5] = c1.x, dst[6] = c1.y, dst[7] = c1.z, dst[8] = c1.w;
}

__global__ void unrepack_q4_kernel(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
                                   uint16_t *__restrict__ out, int64_t n_blocks, int64_t nb) {
    int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= n_blocks) return;
    const uint4 c = *reinterpret_cast<const uint4 *>(codes + q4_block_offset(b / nb, b % nb, nb));
    const uint32_t w[4] = {c.x ^ 0x88888888u, c.y ^ 0x88888888u, c.z ^ 0x88888888u, c.w ^ 0x88888888u};
    uint16_t *dst = out + b * 9;
    dst[0] = scales[b];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        dst[1 + 2 * i] = (uint16_t)w[i];
        dst[2 + 2 * i] = (uint16_t)(w[i] >> 16);
    }
}

}  // namespace

hipError_t launch_quantize(int fmt, int src_type, const void *src, uint8_t *codes, void *scales, void *scales_t,
                           int64_t n_out, int64_t n_in, hipStream_t s) {
    const int64_t n_blocks = n_out * (n_in / kBlock);
    const int64_t nb = n_in / kBlock;
    const dim3 t(256);
    if (fmt == FMT_Q8 && (src_type == SRC_F32 || src_type == SRC_BF16)) {
        const dim3 g((unsigned)((n_blocks + 255) / 256));
        int8_t *c = reinterpret_cast<int8_t *>(codes);
        float *sc = static_cast<float *>(scales), *sct = static_cast<float *>(scales_t);
        if (src_type == SRC_F32)
            hipLaunchKernelGGL((quantize_q8_kernel<SRC_F32>), g, t, 0, s, src, c, sc, sct, n_blocks, nb);
        else
            hipLaunchKernelGGL((quantize_q8_kernel<SRC_BF16>), g, t, 0, s, src, c, sc, sct, n_blocks, nb);
    } else if (fmt == FMT_Q4 && (src_type == SRC_F32 || src_type == SRC_BF16)) {
        // one workgroup per (16-row tile, group of 4 segments)
        const int64_t nb4 = (nb + 3) / 4, tiles = (n_out + 15) / 16;
        const dim3 gq((unsigned)(tiles * ((nb4 + 3) / 4)));
        uint16_t *sc = static_cast<uint16_t *>(scales), *sct = static_cast<uint16_t *>(scales_t);
        if (src_type == SRC_F32)
            hipLaunchKernelGGL((quantize_q4_kernel<SRC_F32>), gq, t, 0, s, src, codes, sc, sct, n_out, nb);
        else
            hipLaunchKernelGGL((quantize_q4_kernel<SRC_BF16>), gq, t, 0, s, src, codes, sc, sct, n_out, nb);
    } else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_unrepack(int fmt, const void *codes, const void *scales, uint8_t *out, int64_t n_out,
                           int64_t n_in, hipStream_t s) {
    const int64_t n_blocks = n_out * (n_in / kBlock);
    const dim3 g((unsigned)((n_blocks + 255) / 256)), t(256);
    if (fmt == FMT_Q8)
        hipLaunchKernelGGL(unrepack_q8_kernel, g, t, 0, s, static_cast<const uint4 *>(codes),
                           static_cast<const float *>(scales), reinterpret_cast<uint32_t *>(out), n_blocks);
    else if (fmt == FMT_Q4)
        hipLaunchKernelGGL(unrepack_q4_kernel, g, t, 0, s, static_cast<const uint8_t *>(codes),
                           static_cast<const uint16_t *>(scales), reinterpret_cast<uint16_t *>(out), n_blocks,
                           n_in / kBlock);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_repack_q8(const uint8_t *staging, int8_t *codes, float *scales, float *scales_t,
                            int64_t n_out, int64_t n_in, hipStream_t s) {
    const int64_t n_blocks = n_out * (n_in / kBlock);
    const int64_t grid = (n_blocks + 255) / 256;
    hipLaunchKernelGGL(repack_q8_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                       reinterpret_cast<const uint32_t *>(staging), reinterpret_cast<uint4 *>(codes), scales,
                       scales_t, n_blocks, n_in / kBlock);
    return hipGetLastError();
}

hipError_t launch_repack_q4(const uint8_t *staging, uint8_t *codes, uint16_t *scales, uint16_t *scales_t,
                            int64_t n_out, int64_t n_in, hipStream_t s) {
    const int64_t n_blocks = n_out * (n_in / kBlock);
    const int64_t grid = (n_blocks + 255) / 256;
    hipLaunchKernelGGL(repack_q4_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                       reinterpret_cast<const uint16_t *>(staging), codes, scales, scales_t, n_blocks,
                       n_in / kBlock);
    return hipGetLastError();
}

}  // namespace il
