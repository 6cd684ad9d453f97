// Measurement probes: the device's attainable dense bf16 matrix rate and streaming-copy bandwidth, so
// that roofline fractions can be stated against peaks measured on the same device beside the vendor's.
//
// peak_mfma_kernel: every wave keeps four independent 32x32x16 bf16 MFMA accumulation chains busy from
// register operands (no memory traffic in the loop), then folds its accumulators into one float per
// lane so the work cannot be dropped.  peak_copy_kernel: a grid-stride copy in 16-byte pieces with four
// pieces in flight per thread, reading and writing each byte once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lola.h"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f16v;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPeakChains = 4;

__global__ __launch_bounds__(256) void peak_mfma_kernel(int iters, float* __restrict__ out) {
    const int tid = threadIdx.x;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(1.0f + 1e-3f * (float)((tid + e) & 7));
        b[e] = (__bf16)(1.0f - 1e-3f * (float)((tid * 3 + e) & 7));
    }
    f16v acc[kPeakChains];
#pragma unroll
    for (int j = 0; j < kPeakChains; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < kPeakChains; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kPeakChains; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    out[(int64_t)blockIdx.x * 256 + tid] = s;
}

__global__ __launch_bounds__(256) void peak_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        int64_t pieces) {
    constexpr int UN = 4;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x; i0 < pieces; i0 += stride * UN) {
        u32x4 v[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int64_t i = i0 + stride * u;
            v[u] = src[i < pieces ? i : i0];
        }
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int64_t i = i0 + stride * u;
            if (i < pieces) dst[i] = v[u];
        }
    }
}

}  // namespace

extern "C" {

lola_status lola_peak_mfma_bf16(int32_t workgroups, int32_t iters, float* out, void* stream) {
    if (workgroups <= 0 || iters <= 0 || !out || ((uintptr_t)out & 15u) != 0) return LOLA_EINVAL;
    hipLaunchKernelGGL(peak_mfma_kernel, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream, iters, out);
    return hipGetLastError() == hipSuccess ? LOLA_OK : LOLA_EDEVICE;
}

lola_status lola_peak_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (!src || !dst || bytes == 0 || (bytes & 15u) != 0 || ((uintptr_t)src & 15u) != 0 ||
        ((uintptr_t)dst & 15u) != 0)
        return LOLA_EINVAL;
    const int64_t pieces = (int64_t)(bytes / 16);
    int64_t blocks = (pieces + 256 * 4 - 1) / (256 * 4);
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(peak_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<const u32x4*>(src), reinterpret_cast<u32x4*>(dst), pieces);
    return hipGetLastError() == hipSuccess ? LOLA_OK : LOLA_EDEVICE;
}

}  // extern "C"
