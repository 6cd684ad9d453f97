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
    static constexpr int SFR = SS * 64 * 8;             // normaliser tile elements
    static constexpr int TT = 1;                        // token tiles per wave and step
    static constexpr int HW = VT >= 8 ? VT / 2 : VT;    // value tiles accumulated at a time
};

// Operand layout.  The tokens' features and values are read with one 16-byte load per lane and
// 32-wide slice: lane (g, c) takes features 32 ss + 8 g .. + 7 of token c (the contiguous reduction
// order of lola_common.hpp), and for each pair p of value tiles the values 32 p + 8 g .. + 7.  So that
// the pairs meet the accumulator rows, value tile u holds the value rows
//     val(u, m) = 32 (u / 2) + 8 (m / 4) + 4 (u % 2) + m % 4,   m = 0..15 (the tile's row),
// which puts rows 4 g .. 4 g + 3 of tiles 2p and 2p + 1 (lane group g's accumulator rows) on values
// 32 p + 8 g .. + 7.  H^T is put in this row order and reduction order when it is staged in LDS.
__device__ __forceinline__ int val_row(int u, int m) { return 32 * (u >> 1) + 8 * (m >> 2) + 4 * (u & 1) + (m & 3); }

template <typename T, int D, int VT>
struct TokTile {
    Frag8<T> f[D / 32];   // features, contiguous reduction order
    Frag8<T> v[VT / 2];   // values of tile pair p: element 4 q + r is row r of tile 2 p + q
};

// Four consecutive elements of an operand.
template <typename T> struct Piece;
template <> struct Piece<float> { using type = f4; };
template <> struct Piece<bf16> { using type = bf16x4; };
template <typename T> __device__ __forceinline__ Frag8<T> join_pieces(const typename Piece<T>::type& a,
                                                                     const typename Piece<T>::type& b) {
    Frag8<T> f;
    __builtin_memcpy(&f, &a, sizeof(a));
    __builtin_memcpy(reinterpret_cast<char*>(&f) + sizeof(a), &b, sizeof(b));
    return f;
}

// Normaliser tile: a 16 x D operand whose product with the features gives phi(k)^T s in its first
// rows.  bf16 operands carry s as two rows, s_hi = bf16(s) and s_lo = bf16(s - s_hi), so the sum
// of the two rows keeps s to about 16 bits; fp32 operands carry s in row 0.  Lane (g, c), slice ss,
// contiguous reduction order.
template <typename T> __device__ __forceinline__ Frag8<T> norm_frag(const float* s, int ss, int g, int c);
template <> __device__ __forceinline__ Frag8<float> norm_frag<float>(const float* s, int ss, int g, int c) {
    return c == 0 ? load_frag_contig(s, ss, g) : frag_zero<float>();
}
template <> __device__ __forceinline__ Frag8<bf16> norm_frag<bf16>(const float* s, int ss, int g, int c) {
    if (c > 1) return frag_zero<bf16>();
    const Frag8<float> x = load_frag_contig(s, ss, g);
    Frag8<bf16> f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const bf16 hi = (bf16)x.v[e];
        f.v[e] = c == 0 ? hi : (bf16)(x.v[e] - (float)hi);
    }
    return f;
}

// H^T fragment (tile u, slice ss, lane (g, c)) of the staged layout from fp32 H^T rows.
template <typename T> __device__ __forceinline__ Frag8<T> staged_from_rows(const float* Ht, int u, int ss, int g, int c);
template <> __device__ __forceinline__ Frag8<float> staged_from_rows<float>(const float* Ht, int u, int ss, int g, int c) {
    return load_frag_contig(Ht + (int64_t)val_row(u, c) * kFeat, ss, g);
}
template <> __device__ __forceinline__ Frag8<bf16> staged_from_rows<bf16>(const float* Ht, int u, int ss, int g, int c) {
    const Frag8<float> x = load_frag_contig(Ht + (int64_t)val_row(u, c) * kFeat, ss, g);
    Frag8<bf16> f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = (bf16)x.v[e];
    return f;
}

template <typename T, int DK, int RB>
__global__ __launch_bounds__(256) void collide_kernel(CollideArgs A) {
    using Cfg = CollideCfg<T, DK>;
    constexpr int D = Cfg::D, DV = Cfg::DV, VT = Cfg::VT, SS = Cfg::SS, NT = Cfg::NT, HFR = Cfg::HFR,
                  SFR = Cfg::SFR, TT = Cfg::TT, HW = Cfg::HW, NW = Cfg::NW;
    static_assert(NT == 256, "launch bound");
    static_assert(SS * 64 == NT, "one normaliser fragment per thread");
    static_assert(VT % 2 == 0, "value tiles come in pairs");
    __shared__ __align__(16) T hT[RB][HFR + SFR];   // H^T tiles, then the normaliser tile

    // block -> (sequence-head, group of RB rows, token block), with the blocks of one XCD (bid mod 8)
    // taking a contiguous stretch of that order
    const int R = A.nchunks, n = A.n, nblk = A.nblk, nrg = (R + RB - 1) / RB;
    const int64_t G = (int64_t)A.BH * nrg * nblk;
    const int64_t G8 = G & ~int64_t(7);
    const int64_t bid = blockIdx.x;
    const int64_t lin = bid < G8 ? (bid & 7) * (G8 >> 3) + (bid >> 3) : bid;
    const int blk = (int)(lin % nblk);
    const int r0 = (int)((lin / nblk) % nrg) * RB;
    const int bh = (int)(lin / ((int64_t)nblk * nrg));
    const int nr = min(RB, R - r0);

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c = l & 15;
    const int i0 = blk * A.tok_per_block;
    const int iend = min(n, i0 + A.tok_per_block);
    // tokens folded in chunk r or before left the window by the end of chunk r: i < (r + 1) C - eta.
    // Row r's entries from ilim[r] on are 0 without looking at them.
    int ilim[RB];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
        const int64_t lim = (int64_t)(r0 + rr + 1) * A.C - A.eta;
        ilim[rr] = rr < nr ? (int)max((int64_t)i0, min((int64_t)iend, lim)) : i0;
        float* orow = A.out + ((int64_t)bh * R + r0 + rr) * n;
        if (rr < nr)
            for (int i = ilim[rr] + tid; i < iend; i += NT) orow[i] = 0.f;
    }
    int itop = i0;   // rows' limits grow with r, but take the maximum anyway
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) itop = max(itop, ilim[rr]);
    if (itop <= i0) return;   // whole workgroup: nothing of the block is in these states

    const char* wsb = A.ws + (int64_t)bh * A.L.per_bh;
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
        const int r = r0 + rr;
        if (rr >= nr || ilim[rr] <= i0) continue;
        const float* sr;
        static_assert(VT * SS * 64 % NT == 0, "whole fragments per thread");
        if (r + 1 < R) {
            // the snapshot is in the chain's fragment order: tile w, slice ss, lane (G, c') holds
            // H^T[16 w + c'][32 ss + 16 h + 4 G + e], h = 0, 1, e = 0..3.  Staged fragment (u, ss,
            // (g, c)) needs H^T[val(u, c)][32 ss + 8 g .. + 7]: the h = g / 2 halves of lanes
            // G = 2 (g % 2) and G + 1 of row val(u, c).
            const char* rec = wsb + A.L.chunk0 + (int64_t)(r + 1) * A.L.per_chunk;
            const T* snap = reinterpret_cast<const T*>(rec + A.L.c_snap_h);
            using PT = typename Piece<T>::type;
#pragma unroll
            for (int j = 0; j < VT * SS * 64 / NT; ++j) {
                const int p = tid + NT * j;
                const int u = p / (SS * 64), s_ = (p / 64) % SS, gg = (p >> 4) & 3, cc = p & 15;
                const int val = val_row(u, cc);
                const int G0 = 2 * (gg & 1), h = gg >> 1;
                const T* sb = snap + ((int64_t)((val >> 4) * SS + s_) * 64 + (val & 15)) * 8 + 4 * h;
                const PT a = *reinterpret_cast<const PT*>(sb + G0 * 16 * 8);
                const PT b = *reinterpret_cast<const PT*>(sb + (G0 + 1) * 16 * 8);
                *reinterpret_cast<Frag8<T>*>(hT[rr] + (int64_t)p * 8) = join_pieces<T>(a, b);
            }
            sr = reinterpret_cast<const float*>(rec + A.L.c_snap_s);
        } else {
            const float* Hb = A.H + (int64_t)bh * DV * D;   // H^T: row = value, D features
#pragma unroll
            for (int j = 0; j < VT * SS * 64 / NT; ++j) {
                const int p = tid + NT * j;
                const int u = p / (SS * 64), s_ = (p / 64) % SS, ln = p % 64;
                *reinterpret_cast<Frag8<T>*>(hT[rr] + (int64_t)p * 8) =
                    staged_from_rows<T>(Hb, u, s_, ln >> 4, ln & 15);
            }
            sr = A.s + (int64_t)bh * D;
        }
        *reinterpret_cast<Frag8<T>*>(hT[rr] + HFR + (int64_t)tid * 8) = norm_frag<T>(sr, w, g, c);
    }

    const T* phiStore = reinterpret_cast<const T*>(wsb + A.L.phi_store);
    const T* vin = reinterpret_cast<const T*>(A.v) + (int64_t)bh * n * DV;
    const int32_t* fa = A.fold_at + (int64_t)bh * n;

    // step k of wave w: tiles (k * NW + w) * TT .. + TT - 1 of the block (16 tokens each)
    const int ntile = (itop - i0 + 15) >> 4;
    const int nstep = (ntile + NW * TT - 1) / (NW * TT);
    // fold chunk of this lane's token in each tile (-1: past the block's live range)
    auto load = [&](TokTile<T, D, VT> (&t)[TT], int (&fz)[TT], int step) {
#pragma unroll
        for (int z = 0; z < TT; ++z) {
            const int tile = (step * NW + w) * TT + z;
            const int i = i0 + 16 * tile + c;
            const bool in = tile < ntile && i < itop;
            fz[z] = in ? fa[i] : -1;
            // the operand addresses do not wait for the fold chunk (a lane past the live range reads
            // a valid row), so the fold-chunk load and the operand loads are in flight together
            const int ii = in ? i : i0;
            const T* pr = phiStore + (int64_t)ii * D;
#pragma unroll
            for (int s_ = 0; s_ < SS; ++s_) t[z].f[s_] = load_frag_contig(pr, s_, g);
            const T* vr = vin + (int64_t)ii * DV;
#pragma unroll
            for (int p = 0; p < VT / 2; ++p) t[z].v[p] = load_frag_contig(vr, p, g);
        }
    };

    // Every step starts by taking the operands loaded during the previous step (the first ones are
    // loaded before the barrier), then issues the next step's loads, so each loop iteration is entered
    // with the same loads outstanding and no step waits for the loads it has just issued.
    TokTile<T, D, VT> cur[TT], nxt[TT];
    int fC[TT], fN[TT];
    if (nstep > 0) load(nxt, fN, 0);
    __syncthreads();

    for (int step = 0; step < nstep; ++step) {
#pragma unroll
        for (int z = 0; z < TT; ++z) { cur[z] = nxt[z]; fC[z] = fN[z]; }
        if (step + 1 < nstep) load(nxt, fN, step + 1);
        float vf[TT][VT][4];   // the values in fp32 by accumulator tile and row, once for all rows
#pragma unroll
        for (int z = 0; z < TT; ++z)
#pragma unroll
            for (int u = 0; u < VT; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e) vf[z][u][e] = frag_get(cur[z].v[u >> 1], 4 * (u & 1) + e);
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) {
            const int r = r0 + rr;
            if (rr >= nr) break;
            const T* hr = hT[rr];
            bool act[TT];
            bool any = false;
#pragma unroll
            for (int z = 0; z < TT; ++z) {
                const int tile = (step * NW + w) * TT + z;
                const int i = i0 + 16 * tile + c;
                act[z] = fC[z] >= 0 && fC[z] <= r && i < ilim[rr];
                any |= __ballot(act[z]) != 0;
            }
            float sre[TT];
#pragma unroll
            for (int z = 0; z < TT; ++z) sre[z] = 0.f;
            if (any) {
                // normaliser phi(k)^T s from the normaliser tile (its rows sum to s)
                float inv[TT], sq[TT];
                {
                    f4 accS[TT];
#pragma unroll
                    for (int z = 0; z < TT; ++z) accS[z] = zero4();
#pragma unroll
                    for (int s_ = 0; s_ < SS; ++s_) {
                        const Frag8<T> a = *reinterpret_cast<const Frag8<T>*>(hr + HFR + (s_ * 64 + l) * 8);
#pragma unroll
                        for (int z = 0; z < TT; ++z) mma32(accS[z], a, cur[z].f[s_]);
                    }
#pragma unroll
                    for (int z = 0; z < TT; ++z) {
                        const float dd = sum_groups((accS[z][0] + accS[z][1]) + (accS[z][2] + accS[z][3]));
                        inv[z] = dd != 0.f ? __builtin_amdgcn_rcpf(dd) : 0.f;   // empty state: recall 0
                        sq[z] = 0.f;
                    }
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
                            const Frag8<T> a =
                                *reinterpret_cast<const Frag8<T>*>(hr + (((u0 + u) * SS + s_) * 64 + l) * 8);
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
                                const float x = acc[z][u][e] * inv[z] - vf[z][u0 + u][e];
                                sq[z] += x * x;
                            }
                }
#pragma unroll
                for (int z = 0; z < TT; ++z) sre[z] = act[z] ? __builtin_amdgcn_sqrtf(sum_groups(sq[z])) : 0.f;
            }
            float* orow = A.out + ((int64_t)bh * R + r) * n;
#pragma unroll
            for (int z = 0; z < TT; ++z) {
                const int tile = (step * NW + w) * TT + z;
                const int i = i0 + 16 * tile + c;
                if (g == 0 && tile < ntile && i < ilim[rr]) orow[i] = sre[z];
            }
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
    constexpr int RB = kCollideRows;
    const int64_t G = (int64_t)a.BH * ((a.nchunks + RB - 1) / RB) * a.nblk;
    hipLaunchKernelGGL((collide_kernel<T, DK, RB>), dim3((unsigned)G), dim3(256), 0, stream, a);
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
