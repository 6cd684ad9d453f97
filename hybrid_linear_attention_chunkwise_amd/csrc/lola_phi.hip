// Feature map phi(k) for every token a prefill call may score: the call's input keys, the initial
// cache members and the initial window ring (LoLA notes 2.2; the map is fixed per layer).  The
// features do not depend on the state, so they are computed here in parallel, once, and the serial
// allocation chain only reads them.  Output row r of phi_store uses the source index of
// lola_internal.hpp.  Under a query-accumulated scoring rule the call's queries follow, rows
// n + lam + eta + i = phi(q_i), for the score kernel.  One workgroup: kPhiBlocks blocks of 64 rows,
// four waves of one 16-row MFMA tile each per block.
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

// Rows per workgroup: W^T is staged once and used for kPhiBlocks blocks of 64 rows; the next block's
// keys are in flight while the current one is mapped.
constexpr int kPhiBlocks = 4;

template <typename T, int DK, int PHI>
__global__ __launch_bounds__(256) void phi_kernel(PrefillArgs A) {
    constexpr int D = kFeat, DW = (PHI == kPhiSoftmaxPM) ? D / 2 : D, WT_LD = DK + 4;
    __shared__ __align__(16) T wt[DW * WT_LD];
    const int bh = blockIdx.y;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c = l & 15;
    const int n = A.n, lam = A.lam, eta = A.eta;
    const int rows = n + lam + eta + (A.score_rule != kScoreSre ? n : 0);
    T* out0 = reinterpret_cast<T*>(A.ws + (int64_t)bh * A.L.per_bh + A.L.phi_store);
    // key row of phi_store row r (source index), or nullptr: no key (an empty initial cache slot)
    auto key_row = [&](int r) -> const T* {
        if (r < n) return reinterpret_cast<const T*>(A.k) + ((int64_t)bh * n + r) * DK;
        if (r < n + lam)
            return A.cache_pos[(int64_t)bh * lam + (r - n)] >= 0
                       ? reinterpret_cast<const T*>(A.cache_k) + ((int64_t)bh * lam + (r - n)) * DK : nullptr;
        if (r < n + lam + eta)
            return reinterpret_cast<const T*>(A.win_k) + ((int64_t)bh * eta + (r - n - lam)) * DK;
        if (r < rows) return reinterpret_cast<const T*>(A.q) + ((int64_t)bh * n + (r - n - lam - eta)) * DK;
        return nullptr;
    };
    Frag8<T> xf[DK / 32], xn[DK / 32];
    const int r0 = blockIdx.x * 64 * kPhiBlocks + w * 16 + c;
    const T* rk = key_row(r0);
#pragma unroll
    for (int ss = 0; ss < DK / 32; ++ss) xf[ss] = rk ? load_frag(rk, ss, g) : frag_zero<T>();
    stage_wt<T, DK, DW, 256>(wt, WT_LD, A.W);
    __syncthreads();
    for (int blk = 0; blk < kPhiBlocks; ++blk) {
        const int r = r0 + 64 * blk;
        if (r - c >= rows) break;                      // wave-uniform: the whole tile is past the end
        const T* rkn = blk + 1 < kPhiBlocks ? key_row(r + 64) : nullptr;
#pragma unroll
        for (int ss = 0; ss < DK / 32; ++ss) xn[ss] = rkn ? load_frag(rkn, ss, g) : frag_zero<T>();
        float ph[D / 16][4];
        phi_tile<T, DK, PHI>(wt, WT_LD, xf, ph);
        if (rk) {
            T* out = out0 + (int64_t)r * D;
#pragma unroll
            for (int ft = 0; ft < D / 16; ++ft) store4p<T>(out + 16 * ft + 4 * g, ph[ft][0], ph[ft][1], ph[ft][2], ph[ft][3]);
        }
        rk = rkn;
#pragma unroll
        for (int ss = 0; ss < DK / 32; ++ss) xf[ss] = xn[ss];
    }
}

}  // namespace

template <typename T, int DK, int PHI>
hipError_t launch_phi_t(const PrefillArgs& a, hipStream_t stream) {
    const int rows = a.n + a.lam + a.eta + (a.score_rule != kScoreSre ? a.n : 0);
    dim3 grid((rows + 64 * kPhiBlocks - 1) / (64 * kPhiBlocks), a.BH);
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
