// il_probe.hip -- a plain streaming read of device memory, the reference
// against which the decode kernels' weight bandwidth is judged: the weight
// GB/s of `WeightRef::bytes` (oxinfer 0.0.0 src/gpu.rs page) that a kernel
// reading each byte once can reach on this part, with no arithmetic beside
// the loads.
//
// Shape: workgroups of `waves` waves; workgroup g reads bytes
// [g * chunk, (g + 1) * chunk) of the buffer (the last one less), each lane
// 16 bytes per load, `depth` loads in flight per lane (issued back to back,
// then consumed in order while the next ones go out).  The loaded words are
// folded with XOR into one word per workgroup, written to `sink`, so the
// loads cannot be removed.  Every load goes through a buffer descriptor that
// spans exactly the workgroup's range, so a ragged tail reads zeros.
#include "il_internal.h"

namespace il {
namespace {

constexpr uint32_t kBufFlags = 0x00020000u;
constexpr uint32_t kOut = 0x7FFFFFF0u;

template <int DEPTH>
__global__ __launch_bounds__(1024) void read_probe_kernel(const uint8_t *__restrict__ buf, int64_t bytes,
                                                          int64_t chunk, uint32_t *__restrict__ sink) {
    const int64_t base = (int64_t)blockIdx.x * chunk;
    const int64_t len = bytes - base < chunk ? bytes - base : chunk;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(buf + base), (short)0, (uint32_t)len, kBufFlags);
    const uint32_t stride = blockDim.x * 16u;  // bytes one load of the workgroup covers
    const uint32_t n = (uint32_t)((len + stride - 1) / stride);
    uint32_t off = threadIdx.x * 16u;
    uint4 ring[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
        ring[d] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)d < n ? off + d * stride : kOut, 0, 0));
    uint32_t acc = 0;
    for (uint32_t i = 0; i < n; i += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            acc ^= ring[d].x ^ ring[d].y ^ ring[d].z ^ ring[d].w;
            const uint32_t nx = i + DEPTH + d;
            ring[d] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, nx < n ? off + nx * stride : kOut, 0, 0));
        }
    }
    // one word per workgroup: wave reduction by XOR, then the first wave's lanes
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
    if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void *buf, int64_t bytes, int64_t chunk, int waves, int depth, uint32_t *sink,
                             hipStream_t s) {
    if (!buf || bytes <= 0 || chunk < 1024 || chunk % 16 || chunk >= (1ll << 31) || waves < 1 || waves > 16)
        return hipErrorInvalidValue;
    const int64_t grid = (bytes + chunk - 1) / chunk;
    if (grid > (1ll << 31) - 1) return hipErrorInvalidValue;
    const dim3 g((unsigned)grid), b((unsigned)(64 * waves));
    const uint8_t *p = static_cast<const uint8_t *>(buf);
    switch (depth) {
        case 1: hipLaunchKernelGGL(read_probe_kernel<1>, g, b, 0, s, p, bytes, chunk, sink); break;
        case 2: hipLaunchKernelGGL(read_probe_kernel<2>, g, b, 0, s, p, bytes, chunk, sink); break;
        case 4: hipLaunchKernelGGL(read_probe_kernel<4>, g, b, 0, s, p, bytes, chunk, sink); break;
        case 8: hipLaunchKernelGGL(read_probe_kernel<8>, g, b, 0, s, p, bytes, chunk, sink); break;
        case 16: hipLaunchKernelGGL(read_probe_kernel<16>, g, b, 0, s, p, bytes, chunk, sink); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace il
