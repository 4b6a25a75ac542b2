// il_repack.hip -- the upload/repack stage (Backend::upload on the oxinfer
// 0.0.0 src/gpu.rs page: "prepares device-side state for a weight matrix").
//
// The host bytes are first copied to a device staging buffer; these kernels
// then split the packed array-of-blocks formats into a K-contiguous code plane
// and a separate scale plane, plus a tiled copy of the scales (layouts in
// il_internal.h).  Integer byte moves
// only: every value is preserved bit for bit.  BF16 needs no kernel, its host
// layout is already the device layout.
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
// with one byte-select conversion.
__global__ void repack_q4_kernel(const uint16_t *__restrict__ staging,
                                 uint4 *__restrict__ codes, uint16_t *__restrict__ scales,
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
    codes[b] = make_uint4(w[0], w[1], w[2], w[3]);
}

}  // namespace

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
                       reinterpret_cast<const uint16_t *>(staging), reinterpret_cast<uint4 *>(codes), scales,
                       scales_t, n_blocks, n_in / kBlock);
    return hipGetLastError();
}

}  // namespace il
