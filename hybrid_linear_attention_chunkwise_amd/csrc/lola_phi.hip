// Feature map phi(k) for every token a prefill call may score: the call's input keys, the initial
// cache members and the initial window ring (LoLA notes 2.2; the map is fixed per layer).  The
// features do not depend on the state, so they are computed here in parallel, once, and the serial
// allocation chain only reads them.  Output row r of phi_store uses the source index of
// lola_internal.hpp.  One workgroup: 64 rows, four waves of one 16-row MFMA tile each.
#include "lola_common.hpp"
#include "lola_internal.hpp"

namespace lola {

namespace {

template <typename T>
__device__ __forceinline__ void store4p(T* dst, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4p<float>(float* dst, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
}
template <>
__device__ __forceinline__ void store4p<bf16>(bf16* dst, float a, float b, float c, float d) {
    bf16x4 v;
    v[0] = (bf16)a; v[1] = (bf16)b; v[2] = (bf16)c; v[3] = (bf16)d;
    *reinterpret_cast<bf16x4*>(dst) = v;
}

template <typename T, int DK, int PHI>
__global__ __launch_bounds__(256) void phi_kernel(PrefillArgs A) {
    constexpr int D = kFeat, DW = (PHI == kPhiSoftmaxPM) ? D / 2 : D, WT_LD = DK + 4;
    __shared__ __align__(16) T wt[DW * WT_LD];
    const int bh = blockIdx.y;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c = l & 15;
    const int n = A.n, lam = A.lam, eta = A.eta;
    const int rows = n + lam + eta;
    stage_wt<T, DK, DW, 256>(wt, WT_LD, A.W);
    __syncthreads();
    const int r = blockIdx.x * 64 + w * 16 + c;
    const T* rk = nullptr;
    if (r < n) rk = reinterpret_cast<const T*>(A.k) + ((int64_t)bh * n + r) * DK;
    else if (r < n + lam) {
        if (A.cache_pos[(int64_t)bh * lam + (r - n)] >= 0)
            rk = reinterpret_cast<const T*>(A.cache_k) + ((int64_t)bh * lam + (r - n)) * DK;
    } else if (r < rows) {
        rk = reinterpret_cast<const T*>(A.win_k) + ((int64_t)bh * eta + (r - n - lam)) * DK;
    }
    Frag8<T> xf[DK / 32];
#pragma unroll
    for (int ss = 0; ss < DK / 32; ++ss) xf[ss] = rk ? load_frag(rk, ss, g) : frag_zero<T>();
    float ph[D / 16][4];
    phi_tile<T, DK, PHI>(wt, WT_LD, xf, ph);
    if (rk) {
        T* out = reinterpret_cast<T*>(A.ws + (int64_t)bh * A.L.per_bh + A.L.phi_store) + (int64_t)r * D;
#pragma unroll
        for (int ft = 0; ft < D / 16; ++ft) store4p<T>(out + 16 * ft + 4 * g, ph[ft][0], ph[ft][1], ph[ft][2], ph[ft][3]);
    }
}

}  // namespace

template <typename T, int DK, int PHI>
hipError_t launch_phi_t(const PrefillArgs& a, hipStream_t stream) {
    const int rows = a.n + a.lam + a.eta;
    dim3 grid((rows + 63) / 64, a.BH);
    hipLaunchKernelGGL((phi_kernel<T, DK, PHI>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

template hipError_t launch_phi_t<float, 64, 0>(const PrefillArgs&, hipStream_t);
template hipError_t launch_phi_t<float, 64, 1>(const PrefillArgs&, hipStream_t);
template hipError_t launch_phi_t<float, 128, 0>(const PrefillArgs&, hipStream_t);
template hipError_t launch_phi_t<float, 128, 1>(const PrefillArgs&, hipStream_t);
template hipError_t launch_phi_t<bf16, 64, 0>(const PrefillArgs&, hipStream_t);
template hipError_t launch_phi_t<bf16, 64, 1>(const PrefillArgs&, hipStream_t);
template hipError_t launch_phi_t<bf16, 128, 0>(const PrefillArgs&, hipStream_t);
template hipError_t launch_phi_t<bf16, 128, 1>(const PrefillArgs&, hipStream_t);

}  // namespace lola
