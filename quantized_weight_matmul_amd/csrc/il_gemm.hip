// il_gemm.hip -- prefill GEMM for t > 8 on the gfx950 bf16 matrix cores.
//
// Computes y[t][n_out] = bf16(x)[t][n_in] * W^T with f32 accumulation for
// every job of one format in one launch (the batch of `struct Job`s over one
// shared x that Backend::matmul on the oxinfer 0.0.0 src/gpu.rs page submits
// at once).  x is rounded to bf16 (round-to-nearest-even); bf16 weights are
// used as stored; Q8/Q4 weights are dequantised to their exact f32 value
// (Q8: q*scale rounded to f32, Q4: (code-8)*scale, exact) and then rounded to
// bf16 as they are written to LDS, ahead of the MFMAs.
//
// Tiling: a workgroup owns a BM x BN output tile (BM tokens x BN weight rows)
// of one job and walks K in BK steps.  Four waves in a 2 x 2 grid each own a
// 64 x 64 sub-tile = 4 x 4 MFMA 16x16x32 tiles.  Global tiles for step k+1 are
// fetched into registers while step k runs from LDS.
#include "il_internal.h"

namespace il {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // bf16 elements per LDS row (pad: no bank conflicts)
constexpr int kThreads = 256;

struct GemmParams {
    const float *x;
    int t;
    int n_in;
    int n_jobs;
    int tiles_m;
    KJob job[kMaxJobs];
    int tile0[kMaxJobs + 1];  // prefix sums of tiles_m * tiles_n per job
};

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    f32x2 v = {a, b};
    bf16x2 h = __builtin_convertvector(v, bf16x2);  // v_cvt_pk_bf16_f32: RNE
    return __builtin_bit_cast(uint32_t, h);
}

// Weight tile staging: each thread owns one row (n) and one 32-element half
// (h) of the BN x BK tile: 32 elements -> 4 x 16 bytes of bf16.
template <int FMT>
struct BStage {
    uint4 raw[4];  // bf16 uses all four, Q8 two, Q4 one
    float scale;
};

template <int FMT>
__device__ __forceinline__ void load_b(BStage<FMT> &st, const KJob &jb, int n_in, int n, int k) {
    // k: first element of this thread's 32-element half (a block boundary)
    const bool ok = n < jb.n_out;
    if constexpr (FMT == FMT_BF16) {
        const uint4 *src = reinterpret_cast<const uint4 *>(
            static_cast<const uint16_t *>(jb.codes) + (int64_t)n * n_in + k);
#pragma unroll
        for (int i = 0; i < 4; ++i) st.raw[i] = ok ? src[i] : make_uint4(0, 0, 0, 0);
    } else if constexpr (FMT == FMT_Q8) {
        const uint4 *src = reinterpret_cast<const uint4 *>(
            static_cast<const int8_t *>(jb.codes) + (int64_t)n * n_in + k);
        st.raw[0] = ok ? src[0] : make_uint4(0, 0, 0, 0);
        st.raw[1] = ok ? src[1] : make_uint4(0, 0, 0, 0);
        st.scale = ok ? static_cast<const float *>(jb.scales)[(int64_t)n * (n_in / kBlock) + k / kBlock]
                      : 0.f;
    } else {
        const uint4 *src = reinterpret_cast<const uint4 *>(
            static_cast<const uint8_t *>(jb.codes) + (int64_t)n * (n_in / 2) + k / 2);
        st.raw[0] = ok ? src[0] : make_uint4(0, 0, 0, 0);
        uint16_t bits = ok ? static_cast<const uint16_t *>(jb.scales)[(int64_t)n * (n_in / kBlock) + k / kBlock]
                           : (uint16_t)0;
        st.scale = (float)__builtin_bit_cast(_Float16, bits) * 0.0625f;  // values carry *16
    }
}

// Convert the staged half-row to 32 bf16 and store at dst (16-byte aligned).
template <int FMT>
__device__ __forceinline__ void store_b(const BStage<FMT> &st, uint16_t *dst) {
    uint4 *d = reinterpret_cast<uint4 *>(dst);
    if constexpr (FMT == FMT_BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) d[i] = st.raw[i];
    } else if constexpr (FMT == FMT_Q8) {
        const uint32_t w[8] = {st.raw[0].x, st.raw[0].y, st.raw[0].z, st.raw[0].w,
                               st.raw[1].x, st.raw[1].y, st.raw[1].z, st.raw[1].w};
        uint32_t o[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float a = (float)(int8_t)(w[i]) * st.scale;
            float b = (float)(int8_t)(w[i] >> 8) * st.scale;
            float c = (float)(int8_t)(w[i] >> 16) * st.scale;
            float e = (float)(int8_t)(w[i] >> 24) * st.scale;
            o[2 * i] = pack_bf16(a, b);
            o[2 * i + 1] = pack_bf16(c, e);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) d[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
    } else {
        const uint32_t w[4] = {st.raw[0].x, st.raw[0].y, st.raw[0].z, st.raw[0].w};
        uint32_t o[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // word i holds elements 8i..8i+7; nibbles stored code ^ 8
            uint32_t lo = (w[i] << 4) & 0xF0F0F0F0u;  // elements 0, 2, 4, 6
            uint32_t hi = w[i] & 0xF0F0F0F0u;         // elements 1, 3, 5, 7
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                float ev = (float)(int8_t)(lo >> (8 * b)) * st.scale;
                float od = (float)(int8_t)(hi >> (8 * b)) * st.scale;
                o[4 * i + b] = pack_bf16(ev, od);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) d[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
    }
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDS_STRIDE];

    // ---- tile -> (job, m tile, n tile) ----
    const int tile = blockIdx.x;
    int j = 0;
#pragma unroll
    for (int q = 1; q < kMaxJobs; ++q)
        if (q < p.n_jobs && tile >= p.tile0[q]) j = q;
    const KJob jb = p.job[j];
    const int local = tile - p.tile0[j];
    const int tm = local % p.tiles_m;
    const int tn = local / p.tiles_m;
    const int m0 = tm * BM, n0 = tn * BN;
    const int n_in = p.n_in;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;

    // staging roles: thread -> (row, 32-element half) of the A and B tiles
    const int sr = tid >> 1, sh = tid & 1;
    const int am = m0 + sr;
    const bool a_ok = am < p.t;
    const float *arow = p.x + (int64_t)(a_ok ? am : 0) * n_in + sh * 32;

    f32x4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = (f32x4){0.f, 0.f, 0.f, 0.f};

    float4 areg[8];
    BStage<FMT> breg;
    // Fetch this thread's halves of the A and B tiles at K offset k0; a half
    // that lies past n_in (n_in % 64 == 32 on the last step) is zero-filled.
    auto load_tiles = [&](int k0) {
        const bool k_ok = k0 + sh * 32 < n_in;
        const float4 *src = reinterpret_cast<const float4 *>(arow + k0);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            areg[i] = (a_ok && k_ok) ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        if (k_ok) {
            load_b<FMT>(breg, jb, n_in, n0 + sr, k0 + sh * 32);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) breg.raw[i] = make_uint4(0, 0, 0, 0);
            breg.scale = 0.f;
        }
    };
    auto store_tiles = [&]() {
        uint4 *ad = reinterpret_cast<uint4 *>(As + sr * LDS_STRIDE + sh * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 u = areg[2 * i], v = areg[2 * i + 1];
            ad[i] = make_uint4(pack_bf16(u.x, u.y), pack_bf16(u.z, u.w), pack_bf16(v.x, v.y),
                               pack_bf16(v.z, v.w));
        }
        store_b<FMT>(breg, Bs + sr * LDS_STRIDE + sh * 32);
    };

    const int ksteps = n_in / BK + ((n_in % BK) ? 1 : 0);
    load_tiles(0);
    for (int ks = 0; ks < ksteps; ++ks) {
        __syncthreads();  // previous step's MFMAs are done reading LDS
        store_tiles();
        __syncthreads();
        if (ks + 1 < ksteps) load_tiles((ks + 1) * BK);
#pragma unroll
        for (int kk = 0; kk < BK / 32; ++kk) {
            bf16x8 af[4], bfr[4];
            const int kcol = kk * 32 + (lane >> 4) * 8;
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int row = wm * 64 + a * 16 + (lane & 15);
                af[a] = *reinterpret_cast<const bf16x8 *>(As + row * LDS_STRIDE + kcol);
            }
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int row = wn * 64 + b * 16 + (lane & 15);
                bfr[b] = *reinterpret_cast<const bf16x8 *>(Bs + row * LDS_STRIDE + kcol);
            }
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
        }
    }

    // ---- epilogue: lane holds rows 4*(lane/16)+e of column lane%16 ----
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int n = n0 + wn * 64 + b * 16 + (lane & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + wm * 64 + a * 16 + (lane >> 4) * 4 + e;
                if (m < p.t && n < jb.n_out) jb.y[(int64_t)m * jb.n_out + n] = acc[a][b][e];
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm(int fmt, const float *x, int t, int n_in, const KJob *jobs, int n_jobs,
                       int cu_count, hipStream_t s) {
    (void)cu_count;
    if (t < 1 || n_jobs < 1 || n_jobs > kMaxJobs || n_in % kBlock) return hipErrorInvalidValue;
    GemmParams p{};
    p.x = x;
    p.t = t;
    p.n_in = n_in;
    p.n_jobs = n_jobs;
    p.tiles_m = (t + BM - 1) / BM;
    int tiles = 0;
    for (int j = 0; j < n_jobs; ++j) {
        p.job[j] = jobs[j];
        p.tile0[j] = tiles;
        tiles += p.tiles_m * ((jobs[j].n_out + BN - 1) / BN);
    }
    for (int j = n_jobs; j <= kMaxJobs; ++j) p.tile0[j] = tiles;
    switch (fmt) {
        case FMT_BF16: hipLaunchKernelGGL(gemm_kernel<FMT_BF16>, dim3(tiles), dim3(kThreads), 0, s, p); break;
        case FMT_Q8: hipLaunchKernelGGL(gemm_kernel<FMT_Q8>, dim3(tiles), dim3(kThreads), 0, s, p); break;
        case FMT_Q4: hipLaunchKernelGGL(gemm_kernel<FMT_Q4>, dim3(tiles), dim3(kThreads), 0, s, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace il
