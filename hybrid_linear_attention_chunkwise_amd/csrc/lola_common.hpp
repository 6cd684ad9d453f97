// Device-side building blocks shared by the LoLA kernels (gfx950, wave64).
//
// MFMA fragments.  Every contraction in this library is built from 16x16 output tiles and a
// reduction dimension walked in "super-steps" of 32.  Within a super-step ss, lane l (lane group
// g = l / 16, column c = l % 16) feeds eight reduction indices, always in this order:
//     k(ss, g, e) = 32*ss + 16*(e/4) + 4*g + (e%4),   e = 0..7
// For bf16 the eight values form one v_mfma_f32_16x16x32_bf16 operand (the instruction sums over
// its own k = 8g + e, so any bijection applied to both operands gives the same product).  For fp32
// the eight values drive eight v_mfma_f32_16x16x4_f32 steps (step e uses k = value e of each group).
// The point of this order: the 16x16 accumulator layout (lane l holds rows 4g + r, r = 0..3, of
// column c) of two stacked tiles is exactly a fragment, so an accumulator can feed the next
// contraction as an operand without a trip through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lola {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f4;

constexpr int kFeat = 128;          // feature dimension D (fixed in v1)
constexpr int kPhiElu1 = 0;
constexpr int kPhiSoftmaxPM = 1;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ f4 zero4() { return f4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }

// exp via the hardware base-2 exponential (one v_exp_f32; results below the normal range flush to 0,
// which only ever meets weights that are negligible next to the largest one).
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
// Hardware reciprocal (about 1 ulp), for normalisers.
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// ---------------------------------------------------------------------------------------------
// Fragments
// ---------------------------------------------------------------------------------------------
template <typename T> struct Frag8;
template <> struct Frag8<float> { float v[8]; };
template <> struct Frag8<bf16> { bf16x8 v; };

template <typename T> __device__ __forceinline__ Frag8<T> frag_zero();
template <> __device__ __forceinline__ Frag8<float> frag_zero<float>() {
    Frag8<float> f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = 0.f;
    return f;
}
template <> __device__ __forceinline__ Frag8<bf16> frag_zero<bf16>() {
    Frag8<bf16> f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = (bf16)0.f;
    return f;
}

// Eight reduction-order values of one row: row[32ss + 4g .. +3] and row[32ss + 16 + 4g .. +3].
__device__ __forceinline__ Frag8<float> load_frag(const float* row, int ss, int g) {
    const float4 lo = *reinterpret_cast<const float4*>(row + 32 * ss + 4 * g);
    const float4 hi = *reinterpret_cast<const float4*>(row + 32 * ss + 16 + 4 * g);
    Frag8<float> f;
    f.v[0] = lo.x; f.v[1] = lo.y; f.v[2] = lo.z; f.v[3] = lo.w;
    f.v[4] = hi.x; f.v[5] = hi.y; f.v[6] = hi.z; f.v[7] = hi.w;
    return f;
}
__device__ __forceinline__ Frag8<bf16> load_frag(const bf16* row, int ss, int g) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + 32 * ss + 4 * g);
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 32 * ss + 16 + 4 * g);
    Frag8<bf16> f;
    f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return f;
}
// The contiguous variant of the order: lane group g feeds row[32ss + 8g .. +7], one 16-byte load.
// Usable wherever both operands of a product are loaded from memory in that same order (the MFMA
// sums over its eight k values per group in any order).
__device__ __forceinline__ Frag8<bf16> load_frag_contig(const bf16* row, int ss, int g) {
    Frag8<bf16> f;
    f.v = *reinterpret_cast<const bf16x8*>(row + 32 * ss + 8 * g);
    return f;
}
__device__ __forceinline__ Frag8<float> load_frag_contig(const float* row, int ss, int g) {
    const float4 lo = *reinterpret_cast<const float4*>(row + 32 * ss + 8 * g);
    const float4 hi = *reinterpret_cast<const float4*>(row + 32 * ss + 8 * g + 4);
    Frag8<float> f;
    f.v[0] = lo.x; f.v[1] = lo.y; f.v[2] = lo.z; f.v[3] = lo.w;
    f.v[4] = hi.x; f.v[5] = hi.y; f.v[6] = hi.z; f.v[7] = hi.w;
    return f;
}

// fp32 source converted to the operand type (used for fp32 state feeding bf16 MFMA).
template <typename T> __device__ __forceinline__ Frag8<T> load_frag_cvt(const float* row, int ss, int g);
template <> __device__ __forceinline__ Frag8<float> load_frag_cvt<float>(const float* row, int ss, int g) {
    return load_frag(row, ss, g);
}
template <> __device__ __forceinline__ Frag8<bf16> load_frag_cvt<bf16>(const float* row, int ss, int g) {
    const Frag8<float> x = load_frag(row, ss, g);
    Frag8<bf16> f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = (bf16)x.v[e];
    return f;
}

// Two stacked accumulator tiles (rows 0..15 in lo, 16..31 in hi) as a fragment.
template <typename T> __device__ __forceinline__ Frag8<T> frag_from_acc(const f4& lo, const f4& hi);
template <> __device__ __forceinline__ Frag8<float> frag_from_acc<float>(const f4& lo, const f4& hi) {
    Frag8<float> f;
#pragma unroll
    for (int r = 0; r < 4; ++r) { f.v[r] = lo[r]; f.v[4 + r] = hi[r]; }
    return f;
}
template <> __device__ __forceinline__ Frag8<bf16> frag_from_acc<bf16>(const f4& lo, const f4& hi) {
    Frag8<bf16> f;
#pragma unroll
    for (int r = 0; r < 4; ++r) { f.v[r] = (bf16)lo[r]; f.v[4 + r] = (bf16)hi[r]; }
    return f;
}

__device__ __forceinline__ float frag_get(const Frag8<float>& f, int e) { return f.v[e]; }
__device__ __forceinline__ float frag_get(const Frag8<bf16>& f, int e) { return (float)f.v[e]; }

// acc (16x16) += A (16 rows x 32) * B (32 x 16 columns) in the reduction order above.
__device__ __forceinline__ void mma32(f4& acc, const Frag8<float>& a, const Frag8<float>& b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
}
__device__ __forceinline__ void mma32(f4& acc, const Frag8<bf16>& a, const Frag8<bf16>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}

// ---------------------------------------------------------------------------------------------
// Cross-lane reductions inside a wave.
// ---------------------------------------------------------------------------------------------
// Over the four lane groups (lanes c, c+16, c+32, c+48): a column of an accumulator tile.  The gfx950
// lane-swap instructions pair each lane with lane ^ 16 (then ^ 32) in VALU registers, without the LDS
// crossbar; the two halves returned are the lane's own value and its partner's.
__device__ __forceinline__ void pair16(float x, float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair32(float x, float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_groups(float x) {
    float a, b;
    pair16(x, a, b);
    pair32(a + b, a, b);
    return a + b;
}
__device__ __forceinline__ float max_groups(float x) {
    float a, b;
    pair16(x, a, b);
    pair32(fmaxf(a, b), a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float min_groups(float x) {
    float a, b;
    pair16(x, a, b);
    pair32(fminf(a, b), a, b);
    return fminf(a, b);
}
// Inclusive sum over the 16 lanes of a lane group with DPP row shifts (VALU only, no LDS): lane 15
// of each group (c == 15) ends with the group's total.
template <int CTRL>
__device__ __forceinline__ float dpp_shr(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float sum_cols_last(float x) {
    x += dpp_shr<0x111>(x);   // row_shr:1
    x += dpp_shr<0x112>(x);   // row_shr:2
    x += dpp_shr<0x114>(x);   // row_shr:4
    x += dpp_shr<0x118>(x);   // row_shr:8
    return x;
}
// Whole-wave sum / max, every lane gets the result: quad and row rotations by DPP, then the lane
// swaps across the four rows (VALU only).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
    x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
    x += dpp_mov<0x124>(x);   // row_ror:4
    x += dpp_mov<0x128>(x);   // row_ror:8
    return sum_groups(x);
}
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_mov<0xB1>(x));
    x = fmaxf(x, dpp_mov<0x4E>(x));
    x = fmaxf(x, dpp_mov<0x124>(x));
    x = fmaxf(x, dpp_mov<0x128>(x));
    return max_groups(x);
}
__device__ __forceinline__ float wave_min(float x) {
    x = fminf(x, dpp_mov<0xB1>(x));
    x = fminf(x, dpp_mov<0x4E>(x));
    x = fminf(x, dpp_mov<0x124>(x));
    x = fminf(x, dpp_mov<0x128>(x));
    return min_groups(x);
}
// Inclusive prefix sum over the whole wave: row_shr steps inside each 16-lane row, then the totals
// of the earlier rows (VALU and scalar reads only, no LDS).
template <int CTRL>
__device__ __forceinline__ int dpp_shr_i(int x) {
    return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ int wave_inclusive_sum(int x) {
    x += dpp_shr_i<0x111>(x);
    x += dpp_shr_i<0x112>(x);
    x += dpp_shr_i<0x114>(x);
    x += dpp_shr_i<0x118>(x);
    const int row = lane_id() >> 4;
    const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
              r2 = __builtin_amdgcn_readlane(x, 47);
    return x + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}
// Over the 16 columns of one lane group: a row of an accumulator tile.
__device__ __forceinline__ float sum_cols(float x) {
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 8);
    return x;
}

// ---------------------------------------------------------------------------------------------
// Feature map phi on a 16-row tile (section 2.2; the two fixed forms of the library).
//   x frags: xf[ss] holds row c = lane % 16 of the 16 inputs, reduction over d_k (in the standard
//   order, or the contiguous one when CONTIG; W^T is then read in the same order).
//   wt: W transposed in LDS, [DW][wt_ld] (row j = column j of W).
//   out[ft][r] = phi(x_c)[16*ft + 4*g + r], ft = 0..7 (D = 128).
// ---------------------------------------------------------------------------------------------
template <typename T, int DK, int PHI, bool CONTIG = false>
__device__ __forceinline__ void phi_tile(const T* wt, int wt_ld, const Frag8<T> (&xf)[DK / 32],
                                         float (&out)[kFeat / 16][4]) {
    constexpr int DW = (PHI == kPhiSoftmaxPM) ? kFeat / 2 : kFeat;
    const int l = lane_id(), g = l >> 4, c = l & 15;
    f4 pre[DW / 16];
#pragma unroll
    for (int ft = 0; ft < DW / 16; ++ft) {
        pre[ft] = zero4();
#pragma unroll
        for (int ss = 0; ss < DK / 32; ++ss) {
            const Frag8<T> a = CONTIG ? load_frag_contig(wt + (16 * ft + c) * wt_ld, ss, g)
                                      : load_frag(wt + (16 * ft + c) * wt_ld, ss, g);
            mma32(pre[ft], a, xf[ss]);
        }
    }
    if constexpr (PHI == kPhiSoftmaxPM) {
        float mx = -INFINITY, mn = INFINITY;
#pragma unroll
        for (int ft = 0; ft < DW / 16; ++ft)
#pragma unroll
            for (int r = 0; r < 4; ++r) { mx = fmaxf(mx, pre[ft][r]); mn = fminf(mn, pre[ft][r]); }
        mx = max_groups(mx);
        mn = min_groups(mn);
        float sp = 0.f, sm = 0.f;
#pragma unroll
        for (int ft = 0; ft < DW / 16; ++ft)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ep = fast_exp(pre[ft][r] - mx);
                const float em = fast_exp(mn - pre[ft][r]);
                out[ft][r] = ep;
                out[ft + DW / 16][r] = em;
                sp += ep;
                sm += em;
            }
        sp = sum_groups(sp);
        sm = sum_groups(sm);
        const float ip = fast_rcp(sp), im = fast_rcp(sm);
#pragma unroll
        for (int ft = 0; ft < DW / 16; ++ft)
#pragma unroll
            for (int r = 0; r < 4; ++r) { out[ft][r] *= ip; out[ft + DW / 16][r] *= im; }
    } else {
#pragma unroll
        for (int ft = 0; ft < DW / 16; ++ft)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float z = pre[ft][r];
                out[ft][r] = z > 0.f ? z + 1.f : fast_exp(z);
            }
    }
}

// Stage W^T (T) in LDS: wt[j * wt_ld + d] = W[d][j], W fp32 [DK][DW] row-major.  All of a thread's
// 16-byte loads are issued before any store, so the copy costs one memory latency.
template <typename T, int DK, int DW, int NT>
__device__ __forceinline__ void stage_wt(T* wt, int wt_ld, const float* __restrict__ W) {
    constexpr int N4 = DK * DW / 4;
    constexpr int PER = (N4 + NT - 1) / NT;
    float4 v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int i4 = threadIdx.x + NT * u;
        if (i4 < N4) v[u] = reinterpret_cast<const float4*>(W)[i4];
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int i4 = threadIdx.x + NT * u;
        if (i4 < N4) {
            const int i = 4 * i4, d = i / DW, j = i - d * DW;
            wt[(j + 0) * wt_ld + d] = from_f<T>(v[u].x);
            wt[(j + 1) * wt_ld + d] = from_f<T>(v[u].y);
            wt[(j + 2) * wt_ld + d] = from_f<T>(v[u].z);
            wt[(j + 3) * wt_ld + d] = from_f<T>(v[u].w);
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Block-wide exclusive scan of int values in LDS (in place).  All threads of the block must call
// it.  tmp needs blockDim.x / 64 + 1 ints.  Returns the total.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ int block_exclusive_scan(int* arr, int n, int* tmp) {
    const int nt = blockDim.x, tid = threadIdx.x;
    const int per = (n + nt - 1) / nt;
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    int local = 0;
    for (int i = lo; i < hi; ++i) local += arr[i];
    // inclusive scan of `local` across the block
    const int l = lane_id(), w = tid >> 6;
    int x = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (l >= o) x += y;
    }
    if (l == 63) tmp[w] = x;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int i = 0; i < nt / 64; ++i) { const int v = tmp[i]; tmp[i] = run; run += v; }
        tmp[nt / 64] = run;
    }
    __syncthreads();
    int run = tmp[w] + x - local;
    for (int i = lo; i < hi; ++i) { const int v = arr[i]; arr[i] = run; run += v; }
    const int total = tmp[nt / 64];
    __syncthreads();
    return total;
}

// ---------------------------------------------------------------------------------------------
// Exclusive prefix counts of a predicate over rows 0..N-1 without LDS scans or barriers: every wave
// ballots all 64-row chunks (cheap) and writes the prefix of the chunks it owns (chunk k belongs to
// wave k % nwaves).  pred(row) must read data that is already visible to the whole block.  Returns
// the total count (the same in every lane).
// ---------------------------------------------------------------------------------------------
template <typename Pred>
__device__ __forceinline__ int ballot_prefix(int N, int nwaves, Pred pred, int* out) {
    const int l = lane_id(), w = threadIdx.x >> 6;
    const unsigned long long lt = l ? (~0ull >> (64 - l)) : 0ull;
    int base = 0;
    for (int k = 0; k * 64 < N; ++k) {
        const int r = k * 64 + l;
        const bool p = r < N && pred(r);
        const unsigned long long m = __ballot(p);
        if (k % nwaves == w && r < N) out[r] = base + __popcll(m & lt);
        base += __popcll(m);
    }
    return base;
}

// Row pointer helpers for element types stored as raw bytes.
template <typename T>
__device__ __forceinline__ const T* row_ptr(const void* base, int64_t row, int ld) {
    return reinterpret_cast<const T*>(base) + row * (int64_t)ld;
}
template <typename T>
__device__ __forceinline__ T* row_ptr_w(void* base, int64_t row, int ld) {
    return reinterpret_cast<T*>(base) + row * (int64_t)ld;
}

}  // namespace lola
