// SRE collision map of one prefill call (LoLA notes, 4.4 Fig. 3; relative form Fig. 10, Eq. (26)).
//
// Row r of the map is the state (H_r, s_r) at the end of chunk r of the call.  For r < nchunks - 1
// that is the chunk-start snapshot of chunk r + 1 the allocation chain left in the workspace (H^T in
// MFMA fragment order, s in fp32); the last row is the state the call left behind.  Entry (r, i) is
// SRE(phi(k_i), v_i | H_r, s_r) (Eq. (10)) for each input token i folded in chunk r or before, and 0
// for a token the state does not hold yet (still in the window or the cache, or never folded).
//
// Every entry is a slice of the product H_r^T Phi^T over the call's tokens, so the map is MFMA work:
// one workgroup takes one row and a block of tokens, stages H_r^T in LDS in operand order, and each
// wave forms the recall of two 16-token tiles at a time (H_r^T from LDS as the A operand, the tokens'
// features from the feature kernel's store as the B operand, so each A fragment read serves two
// products).  The SRE epilogue (normaliser phi^T s, difference to v, norm) runs on the accumulators.
// Workgroups of one (sequence, head) go to one XCD, so its tokens are read from that XCD's L2.
// The relative form is a second pass that subtracts, from each token's column, its entry at the row
// of its own fold.
#include "lola_common.hpp"
#include "lola_internal.hpp"

namespace lola {

namespace {

template <typename T, int DK>
struct CollideCfg {
    static constexpr int D = kFeat;
    static constexpr int DV = DK;
    static constexpr int VT = DV / 16;                  // 16-row tiles of H^T (value rows)
    static constexpr int SS = D / 32;                   // 32-wide reduction slices
    static constexpr int NW = 4;                        // waves per workgroup
    static constexpr int NT = 64 * NW;
    static constexpr int HFR = VT * SS * 64 * 8;        // H^T elements, fragment order
    static constexpr int TT = sizeof(T) == 2 ? 2 : 1;   // token tiles per wave and step
    static constexpr int HW = VT >= 8 ? VT / 2 : VT;    // value tiles accumulated at a time
};

// Token tile operands of one lane: features of token c (B operand, all of D) and the value entries
// that meet the lane's accumulator rows (4 per 16-row value tile).
template <typename T> struct VQuad;
template <> struct VQuad<float> { using type = f4; };
template <> struct VQuad<bf16> { using type = bf16x4; };
template <typename T, int D, int VT>
struct TokTile {
    Frag8<T> f[D / 32];
    typename VQuad<T>::type v[VT];
};

template <typename T, int DK>
__global__ __launch_bounds__(256) void collide_kernel(CollideArgs A) {
    using Cfg = CollideCfg<T, DK>;
    constexpr int D = Cfg::D, DV = Cfg::DV, VT = Cfg::VT, SS = Cfg::SS, NT = Cfg::NT, HFR = Cfg::HFR,
                  TT = Cfg::TT, HW = Cfg::HW, NW = Cfg::NW;
    static_assert(NT == 256, "launch bound");
    __shared__ __align__(16) T hT[HFR];
    __shared__ __align__(16) float sS[D];

    // block -> (sequence-head, row, token block), with the blocks of one XCD (bid mod 8) taking a
    // contiguous stretch of that order
    const int R = A.nchunks, n = A.n, nblk = A.nblk;
    const int64_t G = (int64_t)A.BH * R * nblk;
    const int64_t G8 = G & ~int64_t(7);
    const int64_t bid = blockIdx.x;
    const int64_t lin = bid < G8 ? (bid & 7) * (G8 >> 3) + (bid >> 3) : bid;
    const int blk = (int)(lin % nblk);
    const int r = (int)((lin / nblk) % R);
    const int bh = (int)(lin / ((int64_t)nblk * R));

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c = l & 15;
    const int i0 = blk * A.tok_per_block;
    const int iend = min(n, i0 + A.tok_per_block);
    // tokens folded in chunk r or before left the window by the end of chunk r: i < (r + 1) C - eta
    const int64_t lim64 = (int64_t)(r + 1) * A.C - A.eta;
    const int ilim = (int)max((int64_t)i0, min((int64_t)iend, lim64));
    float* orow = A.out + ((int64_t)bh * R + r) * n;
    for (int i = ilim + tid; i < iend; i += NT) orow[i] = 0.f;
    if (ilim <= i0) return;   // whole workgroup: nothing of the block is in this state

    const char* wsb = A.ws + (int64_t)bh * A.L.per_bh;
    if (r + 1 < R) {
        const char* rec = wsb + A.L.chunk0 + (int64_t)(r + 1) * A.L.per_chunk;
        const uint4* src = reinterpret_cast<const uint4*>(rec + A.L.c_snap_h);
        uint4* dst = reinterpret_cast<uint4*>(hT);
        constexpr int NP = HFR * (int)sizeof(T) / 16;
        static_assert(NP % NT == 0, "whole pieces per thread");
#pragma unroll
        for (int j = 0; j < NP / NT; ++j) dst[tid + NT * j] = src[tid + NT * j];
        const float* ss = reinterpret_cast<const float*>(rec + A.L.c_snap_s);
        for (int d = tid; d < D; d += NT) sS[d] = ss[d];
    } else {
        const float* Hb = A.H + (int64_t)bh * DV * D;   // H^T: row = value, D features
        static_assert(VT * SS * 64 % NT == 0, "whole fragments per thread");
#pragma unroll
        for (int j = 0; j < VT * SS * 64 / NT; ++j) {
            const int p = tid + NT * j;
            const int u = p / (SS * 64), s_ = (p / 64) % SS, ln = p % 64;
            *reinterpret_cast<Frag8<T>*>(hT + (int64_t)p * 8) =
                load_frag_cvt<T>(Hb + (int64_t)(16 * u + (ln & 15)) * D, s_, ln >> 4);
        }
        for (int d = tid; d < D; d += NT) sS[d] = A.s[(int64_t)bh * D + d];
    }

    const T* phiStore = reinterpret_cast<const T*>(wsb + A.L.phi_store);
    const T* vin = reinterpret_cast<const T*>(A.v) + (int64_t)bh * n * DV;
    const int32_t* fa = A.fold_at + (int64_t)bh * n;

    // step k of wave w: tiles (k * NW + w) * TT .. + TT - 1 of the block (16 tokens each)
    const int ntile = (ilim - i0 + 15) >> 4;
    const int nstep = (ntile + NW * TT - 1) / (NW * TT);
    auto load = [&](TokTile<T, D, VT> (&t)[TT], bool (&live)[TT], int step) {
#pragma unroll
        for (int z = 0; z < TT; ++z) {
            const int tile = (step * NW + w) * TT + z;
            const int i = i0 + 16 * tile + c;
            const bool in = tile < ntile && i < ilim;
            const int f = in ? fa[i] : -1;
            const bool act = f >= 0 && f <= r;
            live[z] = __ballot(act) != 0;
            const int ii = act ? i : i0;                 // an inactive lane reads a valid row
            const T* pr = phiStore + (int64_t)ii * D;
#pragma unroll
            for (int s_ = 0; s_ < SS; ++s_) t[z].f[s_] = load_frag(pr, s_, g);
            const T* vr = vin + (int64_t)ii * DV + 4 * g;
#pragma unroll
            for (int u = 0; u < VT; ++u)
                t[z].v[u] = *reinterpret_cast<const typename VQuad<T>::type*>(vr + 16 * u);
        }
    };

    TokTile<T, D, VT> cur[TT], nxt[TT];
    bool liveC[TT], liveN[TT];
    if (nstep > 0) load(cur, liveC, 0);
    __syncthreads();

    for (int step = 0; step < nstep; ++step) {
        if (step + 1 < nstep) load(nxt, liveN, step + 1);
        bool any = false;
#pragma unroll
        for (int z = 0; z < TT; ++z) any |= liveC[z];
        if (any) {
            float den[TT], sq[TT];
#pragma unroll
            for (int z = 0; z < TT; ++z) {
                float dd = 0.f;
#pragma unroll
                for (int s_ = 0; s_ < SS; ++s_) {
                    const f4 slo = *reinterpret_cast<const f4*>(sS + 32 * s_ + 4 * g);
                    const f4 shi = *reinterpret_cast<const f4*>(sS + 32 * s_ + 16 + 4 * g);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        dd += frag_get(cur[z].f[s_], e) * slo[e] + frag_get(cur[z].f[s_], 4 + e) * shi[e];
                }
                dd = sum_groups(dd);
                den[z] = dd != 0.f ? __builtin_amdgcn_rcpf(dd) : 0.f;   // empty state: recall 0
                sq[z] = 0.f;
            }
#pragma unroll
            for (int u0 = 0; u0 < VT; u0 += HW) {
                f4 acc[TT][HW];
#pragma unroll
                for (int z = 0; z < TT; ++z)
#pragma unroll
                    for (int u = 0; u < HW; ++u) acc[z][u] = zero4();
#pragma unroll
                for (int s_ = 0; s_ < SS; ++s_) {
#pragma unroll
                    for (int u = 0; u < HW; ++u) {
                        const Frag8<T> a = *reinterpret_cast<const Frag8<T>*>(hT + (((u0 + u) * SS + s_) * 64 + l) * 8);
#pragma unroll
                        for (int z = 0; z < TT; ++z) mma32(acc[z][u], a, cur[z].f[s_]);
                    }
                }
#pragma unroll
                for (int z = 0; z < TT; ++z)
#pragma unroll
                    for (int u = 0; u < HW; ++u)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float x = acc[z][u][e] * den[z] - to_f(cur[z].v[u0 + u][e]);
                            sq[z] += x * x;
                        }
            }
#pragma unroll
            for (int z = 0; z < TT; ++z) {
                const float tot = sum_groups(sq[z]);
                const int tile = (step * NW + w) * TT + z;
                const int i = i0 + 16 * tile + c;
                if (g == 0 && tile < ntile && i < ilim) {
                    const int f = fa[i];
                    orow[i] = (f >= 0 && f <= r) ? __builtin_amdgcn_sqrtf(tot) : 0.f;
                }
            }
        } else {
#pragma unroll
            for (int z = 0; z < TT; ++z) {
                const int tile = (step * NW + w) * TT + z;
                const int i = i0 + 16 * tile + c;
                if (g == 0 && tile < ntile && i < ilim) orow[i] = 0.f;
            }
        }
        if (step + 1 < nstep) {
#pragma unroll
            for (int z = 0; z < TT; ++z) { cur[z] = nxt[z]; liveC[z] = liveN[z]; }
        }
    }
}

// Relative form: out[r][i] -= out[f][i] for r >= f, f the row of token i's fold.  One thread per
// token walks its column, so the subtracted entry is read before it is overwritten.
__global__ __launch_bounds__(256) void collide_relative_kernel(float* out, const int32_t* fold_at, int BH,
                                                               int R, int n) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)BH * n) return;
    const int bh = (int)(idx / n), i = (int)(idx % n);
    const int f = fold_at[idx];
    if (f < 0 || f >= R) return;
    float* col = out + (int64_t)bh * R * n + i;
    const float base = col[(int64_t)f * n];
    for (int rr = f; rr < R; ++rr) col[(int64_t)rr * n] -= base;
}

template <typename T, int DK>
hipError_t launch_collide_t(const CollideArgs& a, hipStream_t stream) {
    const int64_t G = (int64_t)a.BH * a.nchunks * a.nblk;
    hipLaunchKernelGGL((collide_kernel<T, DK>), dim3((unsigned)G), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.relative) return e;
    const int64_t nt = (int64_t)a.BH * a.n;
    hipLaunchKernelGGL(collide_relative_kernel, dim3((unsigned)((nt + 255) / 256)), dim3(256), 0, stream, a.out,
                       a.fold_at, a.BH, a.nchunks, a.n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_collide(const CollideArgs& a, int dtype, int d, hipStream_t stream) {
    if (dtype == 0) return d == 64 ? launch_collide_t<float, 64>(a, stream) : launch_collide_t<float, 128>(a, stream);
    return d == 64 ? launch_collide_t<bf16, 64>(a, stream) : launch_collide_t<bf16, 128>(a, stream);
}

}  // namespace lola
