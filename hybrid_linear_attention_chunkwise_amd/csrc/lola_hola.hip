// HOLA variant: Gated DeltaNet state plus an exact KV cache chosen by write magnitude.
//
// HOLA reading notes (cc.laoqi.cc, paper 2607.02303 v1), part 2 ("Method"):
//   3.1 Eq. (1), 3.5  state: e_t = v_t - alpha_t S_{t-1}^T k_t,  S_t = alpha_t S_{t-1} + beta_t k_t e_t^T,
//                     with unit-norm keys and queries; read-out o_t = S_t^T q_t;
//   3.3 Eqs. (5)-(6)  write magnitude m_t = beta_t ||e_t||, fixed at write time; the persistent cache keeps
//                     the w largest; a query of chunk c sees that cache (built from the earlier chunks),
//                     the chunk's tokens up to itself, and a null sink;
//   3.4 Eq. (7)       the cache path reads with RMS-normalised, gamma-scaled q and k, temperature 1;
//   3.2 Eq. (3)       y_t = o_t + sigmoid(gate) * cache read-out.
//
// Kernels, in launch order:
//   prep   one pass over the tokens: the inverse L2 norms of q and k (the state path normalises with
//          them while it stages rows) and the cache path's normalised q, k (storage type), one 16-byte
//          piece per lane;
//   block  the delta rule over blocks of 16 tokens is linear in the state at the block start: per
//          block, in parallel, the matrices that do not depend on the state (T = (I + A)^{-1}, the
//          masked query-key products, the decay vectors), one wave per block;
//   scan   serial in the blocks, separable in the value dimension: one workgroup per (sequence, head,
//          16 columns of S) holds S in MFMA accumulators and applies a whole block with fp32 MFMAs
//          (E = T (V - diag(gam) K S), O = diag(gam) Q S + M E, S = glast S + K^T diag(wgt) E),
//          the next block's operands loaded while one is applied;
//   top    m_t = beta_t ||e_t|| (the scan leaves each token's e^2 summed over every 16 columns) and
//          each chunk's own w largest magnitudes, all chunks in parallel;
//   cache  the persistent cache at every chunk start, serial in the chunks: one wave per (sequence,
//          head) merges each chunk's list into the current cache by rank (ties: older);
//   read   one workgroup per (sequence, head, chunk, 64 queries): softmax over the chunk's persistent
//          cache and the chunk's tokens up to each query, with the sink as the initial state of the
//          running softmax; QK^T and PV^T on MFMA with key blocks staged in LDS one block ahead; adds
//          the state read-out.
#include <algorithm>

#include "lola_common.hpp"
#include "lola_internal.hpp"

namespace lola {

namespace {

constexpr float kHolaRmsEps = 1e-6f;

// ---------------- prep ----------------
// One row per D / (16 / sizeof(T)) lanes, each lane one 16-byte piece of q and of k.
template <typename T, int D>
__global__ __launch_bounds__(256) void hola_prep_kernel(HolaArgs A) {
    constexpr int EPV = 16 / (int)sizeof(T), LPR = D / EPV, RPB = 256 / LPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;   // over B*h*n rows
    const int lane = threadIdx.x % LPR;
    if (row >= (int64_t)A.BH * A.n) return;                             // no barrier in this kernel
    const int head = (int)((row / A.n) % A.heads);
    char* wsb = A.ws;
#pragma unroll
    for (int which = 0; which < 2; ++which) {                           // 0: queries, 1: keys
        const uint4 raw = *reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(which ? A.k : A.q) + row * D + lane * EPV);
        const T* xp = reinterpret_cast<const T*>(&raw);
        float x[EPV];
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < EPV; ++i) {
            x[i] = to_f(xp[i]);
            ss += x[i] * x[i];
        }
#pragma unroll
        for (int sh = 1; sh < LPR; sh <<= 1) ss += __shfl_xor(ss, sh, LPR);
        const float inv_l2 = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;        // a zero row stays zero
        const float inv_rms = 1.0f / sqrtf(ss / (float)D + kHolaRmsEps);
        const float* gam = (which ? A.gamma_k : A.gamma_q) + (int64_t)head * D + lane * EPV;
        uint4 til;
        T* tp = reinterpret_cast<T*>(&til);
#pragma unroll
        for (int i = 0; i < EPV; ++i) tp[i] = from_f<T>(gam[i] * x[i] * inv_rms);
        *reinterpret_cast<uint4*>(reinterpret_cast<T*>(wsb + (which ? A.L.ktil : A.L.qtil)) + row * D + lane * EPV) = til;
        if (lane == 0) reinterpret_cast<float*>(wsb + (which ? A.L.kinv : A.L.qinv))[row] = inv_l2;
    }
}

// ---------------- blocked delta rule ----------------
// 16x16x4 fp32 MFMA: acc += A (16 x 4) B (4 x 16); lane (g, r) gives A[r][g], lane (g, c) gives B[g][c],
// and lane (g, c) of the accumulator holds rows 4g .. 4g + 3 of column c.  A product over 16 (or more)
// k indices runs as steps s = 0..3 with k = 4g + s, so an accumulator's element s is directly the B
// operand of step s.
__device__ __forceinline__ void mfma4(f4& acc, float a, float b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

// Per-block matrices, all blocks in parallel: one wave per block of 16 tokens.  Gram products K K^T and
// Q K^T on MFMA (the 16 x 4 pieces of a row serve as both operands), decay products taken directly
// (no ratio of prefix products, which could underflow), T by forward substitution, one column per lane.
template <typename T, int D>
__global__ __launch_bounds__(256) void hola_block_kernel(HolaArgs A) {
    constexpr int BT = kHolaBT;
    __shared__ float sM[4][2][BT][BT + 1];                              // per wave: A, then T; Mq
    __shared__ float sAB[4][2][BT];                                      // alpha, beta
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, g = l >> 4, c = l & 15;
    const int64_t gb = (int64_t)blockIdx.x * 4 + w;                     // (sequence-head, block)
    if (gb >= (int64_t)A.BH * A.nblk) return;                           // whole wave; no workgroup barrier below
    const int bh = (int)(gb / A.nblk), ib = (int)(gb % A.nblk);
    const int n = A.n, t0 = ib * BT;
    const T* kin = reinterpret_cast<const T*>(A.k) + (int64_t)bh * n * D;
    const T* qin = reinterpret_cast<const T*>(A.q) + (int64_t)bh * n * D;
    const float* kinv = reinterpret_cast<const float*>(A.ws + A.L.kinv) + (int64_t)bh * n;
    const float* qinv = reinterpret_cast<const float*>(A.ws + A.L.qinv) + (int64_t)bh * n;
    // token c of the block: unit key and query, pieces 16 kk + 4g .. + 3
    const int tc = t0 + c;
    const bool in = tc < n;
    const int tv = in ? tc : n - 1;
    const float kn = in ? kinv[tv] : 0.f, qn = in ? qinv[tv] : 0.f;
    f4 G = zero4(), QK = zero4();
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        float kx[4], qx[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            kx[s] = to_f(kin[(int64_t)tv * D + 16 * kk + 4 * g + s]) * kn;
            qx[s] = to_f(qin[(int64_t)tv * D + 16 * kk + 4 * g + s]) * qn;
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            mfma4(G, kx[s], kx[s]);                                     // G[i][j] = k_i . k_j
            mfma4(QK, qx[s], kx[s]);                                    // QK[i][j] = q_i . k_j
        }
    }
    if (l < BT) {
        sAB[w][0][l] = t0 + l < n ? A.alpha[(int64_t)bh * n + t0 + l] : 1.f;   // past n: no decay, no write
        sAB[w][1][l] = t0 + l < n ? A.beta[(int64_t)bh * n + t0 + l] : 0.f;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    // ratio(i, j) = prod_{j < l <= i} alpha_l;  lane (g, c) holds rows i = 4g + e, column j = c
    // one running product over the block: run = prod_{c < l <= m} alpha_l (1 for m <= c), captured at
    // the lane's rows m = 4g .. 4g + 3
    float rr[4] = {1.f, 1.f, 1.f, 1.f};
    {
        float run = 1.f;
#pragma unroll
        for (int m = 0; m < BT; ++m) {
            run = m > c ? run * sAB[w][0][m] : 1.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) rr[e] = m == 4 * g + e ? run : rr[e];
        }
    }
    const float bj = sAB[w][1][c];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = 4 * g + e, j = c;
        sM[w][0][i][j] = j < i ? rr[e] * bj * G[e] : 0.f;              // A (strictly lower)
        sM[w][1][i][j] = j <= i ? rr[e] * bj * QK[e] : 0.f;            // Mq (lower, with the diagonal)
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    HolaBlock* out = reinterpret_cast<HolaBlock*>(A.ws + A.L.blk) + gb;
    // T = (I + A)^{-1}: lane c < 16 solves column c by forward substitution
    float tcol[BT];
    if (l < BT) {
#pragma unroll
        for (int i = 0; i < BT; ++i) {
            float x = i == l ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < i; ++j) x = fmaf(-sM[w][0][i][j], tcol[j], x);
            tcol[i] = x;
        }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    if (l < BT) {
#pragma unroll
        for (int i = 0; i < BT; ++i) sM[w][0][i][l] = tcol[i];         // T overwrites A
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    // operand layout: lane (g, r) holds row r, columns 4g .. 4g + 3
    *reinterpret_cast<float4*>(out->Tp[l]) =
        make_float4(sM[w][0][c][4 * g], sM[w][0][c][4 * g + 1], sM[w][0][c][4 * g + 2], sM[w][0][c][4 * g + 3]);
    *reinterpret_cast<float4*>(out->Mp[l]) =
        make_float4(sM[w][1][c][4 * g], sM[w][1][c][4 * g + 1], sM[w][1][c][4 * g + 2], sM[w][1][c][4 * g + 3]);
    if (l < BT) {
        float gm = 1.f, wt = sAB[w][1][l];
        for (int m = 0; m <= l; ++m) gm *= sAB[w][0][m];
        for (int m = l + 1; m < BT; ++m) wt *= sAB[w][0][m];
        out->gam[l] = gm;
        out->wgt[l] = wt;
        if (l == BT - 1) out->glast = gm;
    }
}

// The serial part, block by block: one workgroup of four waves per (sequence, head, 16 value columns),
// S[:, columns] in MFMA accumulators, each wave holding d / 64 tiles of 16 rows.  Per block, each wave
// forms its rows' share of K S and Q S; the shares meet in LDS (the one barrier of the block); then
// every wave forms E and O (the same arithmetic in each, so all hold identical values) and updates
// its own rows of S.  A block's operands are loaded into registers while the previous block runs.
template <typename T, int D, int NW>
__global__ __launch_bounds__(64 * NW) void hola_scan_kernel(HolaArgs A) {
    constexpr int BT = kHolaBT, TPW = D / 16 / NW;                     // row tiles per wave
    static_assert(TPW >= 1 && TPW * NW * 16 == D, "scan waves");
    __shared__ f4 sX[2][NW][2][64];                                     // [parity][wave][K S | Q S][lane]
    __shared__ float sKT[NW][BT][TPW * 16 + 4];                         // each wave's unit keys, its rows
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, g = l >> 4, c = l & 15;
    const int bh = blockIdx.x / (D / 16), cb = 16 * (blockIdx.x % (D / 16));
    const int n = A.n, nblk = A.nblk;
    const T* kin = reinterpret_cast<const T*>(A.k) + (int64_t)bh * n * D;
    const T* qin = reinterpret_cast<const T*>(A.q) + (int64_t)bh * n * D;
    const T* vin = reinterpret_cast<const T*>(A.v) + (int64_t)bh * n * D;
    const float* kinv = reinterpret_cast<const float*>(A.ws + A.L.kinv) + (int64_t)bh * n;
    const float* qinv = reinterpret_cast<const float*>(A.ws + A.L.qinv) + (int64_t)bh * n;
    const HolaBlock* blk = reinterpret_cast<const HolaBlock*>(A.ws + A.L.blk) + (int64_t)bh * nblk;
    float* oo = reinterpret_cast<float*>(A.ws + A.L.o) + (int64_t)bh * n * D;
    float* esq = reinterpret_cast<float*>(A.ws + A.L.esq) + (int64_t)bh * n * (D / 16);
    float* sink = reinterpret_cast<float*>(A.ws + A.L.sink);

    // a block's operands as loaded (raw storage type; converted where they are used, so that the loads
    // of the next block stay in flight while a block runs)
    // four elements of a row as 32-bit words: 2 (bf16) or 4 (fp32)
    constexpr int NWD = 4 * (int)sizeof(T) / 4;
    struct alignas(4 * sizeof(T)) Raw4 { uint32_t u[NWD]; };
    auto elem = [](const Raw4& r, int s) {
        if constexpr (sizeof(T) == 2) return __uint_as_float(s & 1 ? r.u[s >> 1] & 0xFFFF0000u : r.u[s >> 1] << 16);
        else return __uint_as_float(r.u[s]);
    };
    struct Ops {
        Raw4 ka[TPW], qa[TPW];                                          // token c: k, q at rows 16 rt + 4g ..
        float kn, qn;                                                   // its inverse norms
        T v[4];                                                         // V[4g + e][column c]
        float4 tp, mp, gam, wgt;
        float glast;
    };
    auto fetch = [&](int ib, Ops& o) {
        const int t0 = ib * BT, tc = t0 + c;
        const int tv = tc < n ? tc : n - 1;                             // always a valid row
        o.kn = kinv[tv];
        o.qn = qinv[tv];
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp) {
            const int r0 = 16 * (w * TPW + tp) + 4 * g;
            o.ka[tp] = *reinterpret_cast<const Raw4*>(kin + (int64_t)tv * D + r0);
            o.qa[tp] = *reinterpret_cast<const Raw4*>(qin + (int64_t)tv * D + r0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = t0 + 4 * g + e;
            o.v[e] = vin[(int64_t)(t < n ? t : n - 1) * D + cb + c];
        }
        const HolaBlock* b = blk + ib;
        o.tp = *reinterpret_cast<const float4*>(b->Tp[l]);
        o.mp = *reinterpret_cast<const float4*>(b->Mp[l]);
        o.gam = *reinterpret_cast<const float4*>(&b->gam[4 * g]);
        o.wgt = *reinterpret_cast<const float4*>(&b->wgt[4 * g]);
        o.glast = b->glast;
    };

    f4 S[TPW];
#pragma unroll
    for (int tp = 0; tp < TPW; ++tp) S[tp] = zero4();
    auto step = [&](int ib, const Ops& cur) {
        // this wave's rows of K S and Q S; its unit keys go to LDS for K^T below
        const bool cin = ib * BT + c < n;                               // token c exists
        const float kn = cin ? cur.kn : 0.f, qn = cin ? cur.qn : 0.f;
        f4 R = zero4(), QS = zero4();
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp) {
            float ka[4], qa[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                ka[s] = elem(cur.ka[tp], s) * kn;                       // unit key and query
                qa[s] = elem(cur.qa[tp], s) * qn;
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                mfma4(R, ka[s], S[tp][s]);
                mfma4(QS, qa[s], S[tp][s]);
            }
            *reinterpret_cast<float4*>(&sKT[w][c][16 * tp + 4 * g]) = make_float4(ka[0], ka[1], ka[2], ka[3]);
        }
        sX[ib & 1][w][0][l] = R;
        sX[ib & 1][w][1][l] = QS;
        __syncthreads();
        f4 Rt = zero4(), Qt = zero4();
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            Rt += sX[ib & 1][ww][0][l];
            Qt += sX[ib & 1][ww][1][l];
        }
        const float gm[4] = {cur.gam.x, cur.gam.y, cur.gam.z, cur.gam.w};
        const float wg[4] = {cur.wgt.x, cur.wgt.y, cur.wgt.z, cur.wgt.w};
        const float tpv[4] = {cur.tp.x, cur.tp.y, cur.tp.z, cur.tp.w};
        const float mpv[4] = {cur.mp.x, cur.mp.y, cur.mp.z, cur.mp.w};
        // E = T (V - diag(gam) K S);  O = diag(gam) Q S + M E
        f4 E = zero4(), O;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const float vv = ib * BT + 4 * g + s < n ? to_f(cur.v[s]) : 0.f;
            mfma4(E, tpv[s], fmaf(-gm[s], Rt[s], vv));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) O[e] = gm[e] * Qt[e];
#pragma unroll
        for (int s = 0; s < 4; ++s) mfma4(O, mpv[s], E[s]);
        // S = glast S + K^T diag(wgt) E on this wave's rows
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp) {
            S[tp] *= cur.glast;
#pragma unroll
            for (int s = 0; s < 4; ++s) mfma4(S[tp], sKT[w][4 * g + s][16 * tp + c], wg[s] * E[s]);
        }
        // every wave holds the same E and O: wave w stores rows 4g + w, without a branch (a token past n
        // writes to the sink), so the waits for the next block's loads stay exact
        float ov = O[0], ev = E[0];
#pragma unroll
        for (int e = 1; e < 4; ++e) {
            ov = (w & 3) == e ? O[e] : ov;
            ev = (w & 3) == e ? E[e] : ev;
        }
        const int t = ib * BT + 4 * g + (w & 3);                        // waves w and w + 4 store alike
        // the write magnitude's share from these 16 columns: e^2 summed over the 16 lanes of the row
        // (a DPP row is exactly the lanes of one g), stored by the lane of column 0
        float q2 = ev * ev;
        q2 += dpp_mov<0x128>(q2);                                       // row_ror:8
        q2 += dpp_mov<0x124>(q2);                                       // row_ror:4
        q2 += dpp_mov<0x122>(q2);                                       // row_ror:2
        q2 += dpp_mov<0x121>(q2);                                       // row_ror:1
        float* po = t < n ? oo + (int64_t)t * D + cb + c : sink + l;
        float* pe = t < n && c == 0 ? esq + (int64_t)t * (D / 16) + cb / 16 : sink + 64 + l;
        *po = ov;
        *pe = q2;
    };
    // two operand sets in turn: a block's loads were issued one block earlier, with no copies between.
    // The loads are unconditional (past the last block they repeat it), so the waits for them stay exact.
    Ops o0, o1;
    fetch(0, o0);
    for (int ib = 0; ib < nblk; ib += 2) {
        fetch(min(ib + 1, nblk - 1), o1);
        __builtin_amdgcn_sched_barrier(0);                              // issue the loads before the step
        step(ib, o0);
        if (ib + 1 >= nblk) break;
        fetch(min(ib + 2, nblk - 1), o0);
        __builtin_amdgcn_sched_barrier(0);
        step(ib + 1, o1);
    }
    if (A.S_out) {
        float* so = A.S_out + (int64_t)bh * D * D;
#pragma unroll
        for (int tp = 0; tp < TPW; ++tp)
#pragma unroll
            for (int e = 0; e < 4; ++e) so[(int64_t)(16 * (w * TPW + tp) + 4 * g + e) * D + cb + c] = S[tp][e];
    }
}

// ---------------- persistent cache per chunk ----------------
// Ranking key: larger = kept first; equal magnitudes rank the older position higher.  The magnitude's
// bits are mapped so that unsigned order is float order (with -0 taken as +0).
__device__ __forceinline__ unsigned ordered_bits(float m) {
    const unsigned u = __float_as_uint(m);
    return m == 0.f ? 0x80000000u : (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_mag(unsigned long long key) {
    const unsigned u = (unsigned)(key >> 32);
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}
__device__ __forceinline__ unsigned long long hola_key(float m, int pos) {
    return ((unsigned long long)ordered_bits(m) << 32) | (unsigned long long)(0xFFFFFFFFu - (unsigned)pos);
}
__device__ __forceinline__ int key_pos(unsigned long long key) { return (int)(0xFFFFFFFFu - (unsigned)key); }

// Each chunk's own ranking, all chunks in parallel: the w largest keys of the chunk's tokens, largest
// first.  The persistent cache at any chunk start is the top w of the union of these lists over the
// earlier chunks, since a token outside its own chunk's top w has w larger keys before it anyway.
// The magnitudes m_t = beta_t ||e_t|| are formed here from the scan's per-16-column sums of e^2, added
// in column order.
template <int D>
__global__ __launch_bounds__(256) void hola_chunk_top_kernel(HolaArgs A) {
    constexpr int NG = D / 16;
    __shared__ unsigned long long sKey[kHolaMaxC];
    const int bh = blockIdx.x / A.nchunks, ch = blockIdx.x % A.nchunks, tid = threadIdx.x;
    const int n = A.n, C = A.C, a = ch * C, nx = min(C, n - a), keep = min(A.w, nx);
    const int ls = min(kHolaMaxW, C);                                   // list stride
    const float* esq = reinterpret_cast<const float*>(A.ws + A.L.esq) + (int64_t)bh * n * NG;
    const float* beta = A.beta + (int64_t)bh * n;
    unsigned long long* out = reinterpret_cast<unsigned long long*>(A.ws + A.L.tlist) + ((int64_t)bh * A.nchunks + ch) * ls;
    for (int i = tid; i < nx; i += 256) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < NG; ++j) ss += esq[(int64_t)(a + i) * NG + j];
        sKey[i] = hola_key(beta[a + i] * sqrtf(ss), a + i);
    }
    __syncthreads();
    for (int i = tid; i < nx; i += 256) {
        const unsigned long long ki = sKey[i];
        int above = 0;
#pragma unroll 16
        for (int j = 0; j < nx; ++j) above += sKey[j] > ki;
        if (above < keep) out[above] = ki;
    }
}

// Number of entries of a list sorted largest first that exceed x (x is in neither list twice).
__device__ __forceinline__ int count_above(const unsigned long long* L, int len, unsigned long long x) {
    int lo = 0, hi = len;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (L[mid] > x) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

// The persistent cache at every chunk start, serial in the chunks: one wave per (sequence, head) keeps
// the current cache as a key list sorted largest first and merges each chunk's own list into it by
// rank (an entry's new index is its index plus the number of entries of the other list above it);
// the chunk lists are loaded eight chunks at a time, one batch ahead.
__global__ __launch_bounds__(64) void hola_cache_kernel(HolaArgs A) {
    constexpr int NB = 8;
    __shared__ unsigned long long sCur[2][kHolaMaxW];
    __shared__ unsigned long long sL[NB][kHolaMaxW];
    const int bh = blockIdx.x, lane = threadIdx.x;
    const int n = A.n, C = A.C, w = A.w, nchunks = A.nchunks, ls = min(kHolaMaxW, C);
    const unsigned long long* tl = reinterpret_cast<const unsigned long long*>(A.ws + A.L.tlist) + (int64_t)bh * nchunks * ls;
    int* clist = reinterpret_cast<int*>(A.ws + A.L.clist) + (int64_t)bh * (nchunks + 1) * kHolaMaxW;
    auto count_of = [&](int ch) { return min(w, min(C, n - ch * C)); };
    unsigned long long rb[NB];
    auto fetch = [&](int c0) {
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int ch = c0 + u;
            rb[u] = ch < nchunks && lane < count_of(ch) ? tl[(int64_t)ch * ls + lane] : 0ull;
        }
    };
    int ncur = 0, cb = 0;
    fetch(0);
    for (int c0 = 0; c0 < nchunks; c0 += NB) {
        __syncthreads();                                                // the previous batch is used up
#pragma unroll
        for (int u = 0; u < NB; ++u) sL[u][lane] = rb[u];
        __syncthreads();
        if (c0 + NB < nchunks) fetch(c0 + NB);
        for (int u = 0; u < NB && c0 + u < nchunks; ++u) {
            const int ch = c0 + u, nl = count_of(ch);
            clist[(int64_t)ch * kHolaMaxW + lane] = lane < ncur ? key_pos(sCur[cb][lane]) : -1;   // the cache now
            const unsigned long long* L = sL[u];
            if (lane < ncur) {
                const unsigned long long x = sCur[cb][lane];
                const int r = lane + count_above(L, nl, x);
                if (r < w) sCur[cb ^ 1][r] = x;
            }
            if (lane < nl) {
                const unsigned long long y = L[lane];
                const int r = lane + count_above(sCur[cb], ncur, y);
                if (r < w) sCur[cb ^ 1][r] = y;
            }
            __syncthreads();
            cb ^= 1;
            ncur = min(w, ncur + nl);
        }
    }
    // the final cache: in rank order after the chunk lists, and sorted by position with its magnitudes
    clist[(int64_t)nchunks * kHolaMaxW + lane] = lane < ncur ? key_pos(sCur[cb][lane]) : -1;
    if (lane < ncur) {
        const unsigned long long x = sCur[cb][lane];
        const int p = key_pos(x);
        int before = 0;
        for (int j = 0; j < ncur; ++j) before += key_pos(sCur[cb][j]) < p;
        if (A.cache_pos_out) A.cache_pos_out[(int64_t)bh * w + before] = p;
        if (A.cache_score_out) A.cache_score_out[(int64_t)bh * w + before] = key_mag(x);
    }
    for (int i = ncur + lane; i < w; i += 64) {
        if (A.cache_pos_out) A.cache_pos_out[(int64_t)bh * w + i] = -1;
        if (A.cache_score_out) A.cache_score_out[(int64_t)bh * w + i] = 0.f;
    }
}

// ---------------- cache read ----------------
template <typename T, int D>
__global__ __launch_bounds__(256) void hola_read_kernel(HolaArgs A) {
    constexpr int KB = 64, EPV = 16 / (int)sizeof(T), K_LD = D + EPV, VT_LD = KB + EPV, JT = D / 16;
    __shared__ __align__(16) T sK[KB * K_LD];
    __shared__ __align__(16) T sVT[D * VT_LD];
    __shared__ int sPos[KB];
    __shared__ int sList[kHolaMaxW];
    const int nqt = A.nqt;
    const int bid = blockIdx.x;
    const int qt = bid % nqt;
    const int ch = (bid / nqt) % A.nchunks;
    const int bh = bid / (nqt * A.nchunks);
    const int n = A.n, C = A.C;
    const int a = ch * C, b = min(a + C, n);
    const int q0 = a + 64 * qt;
    if (q0 >= b) return;                                                // whole workgroup: ragged last chunk
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c = l & 15;
    const int head = bh % A.heads;
    const T* ktil = reinterpret_cast<const T*>(A.ws + A.L.ktil) + (int64_t)bh * n * D;
    const T* qtil = reinterpret_cast<const T*>(A.ws + A.L.qtil) + (int64_t)bh * n * D;
    const T* vin = reinterpret_cast<const T*>(A.v) + (int64_t)bh * n * D;
    const float* ost = reinterpret_cast<const float*>(A.ws + A.L.o) + (int64_t)bh * n * D;
    const int* clist = reinterpret_cast<const int*>(A.ws + A.L.clist) + ((int64_t)bh * (A.nchunks + 1) + ch) * kHolaMaxW;
    for (int j = tid; j < kHolaMaxW; j += 256) sList[j] = clist[j];
    __syncthreads();
    int nA = 0;
    static_assert(kHolaMaxW == 64, "one list entry per lane");
    nA = __popcll(__ballot(sList[l] >= 0));                             // valid entries come first
    const int hi = min(q0 + 63, b - 1);                                 // last chunk key any query here needs
    const int NK = nA + (hi - a + 1);
    auto key_pos = [&](int kk) { return kk < nA ? sList[kk] : a + (kk - nA); };

    const int tq = q0 + 16 * w + c;                                     // this lane's query (column c)
    const bool qvalid = tq < b;
    Frag8<T> qf[D / 32];
#pragma unroll
    for (int ss = 0; ss < D / 32; ++ss) qf[ss] = qvalid ? load_frag(qtil + (int64_t)tq * D, ss, g) : frag_zero<T>();
    const float scale = 1.0f / sqrtf((float)D);
    // the null sink starts the running softmax: logit sink, weight 1 at its own maximum, value 0
    float m_run = A.sink[head], l_part = 0.f;
    f4 O[JT];
#pragma unroll
    for (int J = 0; J < JT; ++J) O[J] = zero4();

    // key blocks are staged through registers one block ahead: keys row-major in 16-byte pieces;
    // values transposed (dimension-major, the A operand of PV^T), each thread loading KPW = 4 / sizeof(T)
    // keys' pieces of the same dimensions so that their elements pair into 32-bit LDS words
    constexpr int KPW = 4 / (int)sizeof(T), PC = D / EPV;              // keys per word, pieces per row
    constexpr int KPT = KB * PC / 256;                                  // key pieces per thread
    constexpr int VPT = KB / KPW * PC / 256;                            // (key word, piece) items per thread
    static_assert(KPT >= 1 && VPT >= 1, "read staging");
    uint4 rk[KPT], rv[VPT][KPW];
    auto clamp_pos = [&](int kk) { return key_pos(kk < NK ? kk : NK - 1); };   // NK >= 1
    auto fetch = [&](int kb) {
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            const int i = tid + 256 * u, kk = kb * KB + i / PC;
            const uint4 x = *reinterpret_cast<const uint4*>(ktil + (int64_t)clamp_pos(kk) * D + (i % PC) * EPV);
            rk[u] = kk < NK ? x : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int i = tid + 256 * u, jw = i % (KB / KPW), p = i / (KB / KPW);
#pragma unroll
            for (int h = 0; h < KPW; ++h) {
                const int kk = kb * KB + KPW * jw + h;
                const uint4 x = *reinterpret_cast<const uint4*>(vin + (int64_t)clamp_pos(kk) * D + p * EPV);
                rv[u][h] = kk < NK ? x : make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto stash = [&](int kb) {
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            const int i = tid + 256 * u;
            *reinterpret_cast<uint4*>(sK + (i / PC) * K_LD + (i % PC) * EPV) = rk[u];
        }
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int i = tid + 256 * u, jw = i % (KB / KPW), p = i / (KB / KPW);
            const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&rv[u][0]);
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                uint32_t word;
                if constexpr (KPW == 2) {
                    const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&rv[u][1]);
                    const uint32_t lo = (w0[e / 2] >> (16 * (e % 2))) & 0xFFFFu;   // key 2 jw, dimension p EPV + e
                    const uint32_t hi = (w1[e / 2] >> (16 * (e % 2))) & 0xFFFFu;   // key 2 jw + 1
                    word = lo | (hi << 16);
                } else {
                    word = w0[e];
                }
                *reinterpret_cast<uint32_t*>(sVT + (p * EPV + e) * VT_LD + KPW * jw) = word;
            }
        }
        for (int j = tid; j < KB; j += 256) sPos[j] = kb * KB + j < NK ? key_pos(kb * KB + j) : -1;
    };

    const int nkb = (NK + KB - 1) / KB;
    fetch(0);
    for (int kb = 0; kb < nkb; ++kb) {
        __syncthreads();                                                // the previous block is used up
        stash(kb);
        __syncthreads();
        if (kb + 1 < nkb) fetch(kb + 1);
        if (q0 + 16 * w < b) {
            f4 st[KB / 16];
#pragma unroll
            for (int kt = 0; kt < KB / 16; ++kt) {
                st[kt] = zero4();
#pragma unroll
                for (int ss = 0; ss < D / 32; ++ss) mma32(st[kt], load_frag(sK + (16 * kt + c) * K_LD, ss, g), qf[ss]);
            }
            float bmax = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < KB / 16; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int pos = sPos[16 * kt + 4 * g + r];
                    const bool ok = pos >= 0 && pos <= tq;              // persistent entries precede the chunk
                    const float sc = ok ? st[kt][r] * scale : -INFINITY;
                    st[kt][r] = sc;
                    bmax = fmaxf(bmax, sc);
                }
            bmax = max_groups(bmax);
            const float m_new = fmaxf(m_run, bmax);
            const float alpha = fast_exp(m_run - m_new);
#pragma unroll
            for (int J = 0; J < JT; ++J)
#pragma unroll
                for (int r = 0; r < 4; ++r) O[J][r] *= alpha;
            l_part *= alpha;
#pragma unroll
            for (int kt = 0; kt < KB / 16; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = st[kt][r] != -INFINITY ? fast_exp(st[kt][r] - m_new) : 0.f;
                    st[kt][r] = p;
                    l_part += p;
                }
            m_run = m_new;
#pragma unroll
            for (int k2 = 0; k2 < KB / 32; ++k2) {
                const Frag8<T> bp = frag_from_acc<T>(st[2 * k2], st[2 * k2 + 1]);
#pragma unroll
                for (int J = 0; J < JT; ++J) mma32(O[J], load_frag(sVT + (16 * J + c) * VT_LD, k2, g), bp);
            }
        }
    }
    // denominator: the keys' weights (summed over the lane groups) plus the sink's exp(sink - m)
    const float lsum = sum_groups(l_part) + expf(A.sink[head] - m_run);
    if (qvalid) {
        const float gsc = 1.0f / (1.0f + expf(-A.gate[head]));
        const float inv = gsc / lsum;
        T* yrow = reinterpret_cast<T*>(A.y) + ((int64_t)bh * n + tq) * D;
        const float* orow = ost + (int64_t)tq * D;
#pragma unroll
        for (int J = 0; J < JT; ++J)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = 16 * J + 4 * g + r;
                yrow[d] = from_f<T>(orow[d] + O[J][r] * inv);
            }
    }
}

// ---------------- decode memory after a prefill ----------------
// The memory a decode step continues from: the persistent cache at the start of the open chunk (the
// last chunk's list, or the final cache when the call ends on a chunk boundary), sorted by position,
// with magnitudes formed as the ranking formed them, and the open chunk's tokens.  Keys and values are
// copied raw (the cache path normalises them when it reads).  One workgroup per (sequence, head).
template <typename T, int D>
__global__ __launch_bounds__(256) void hola_state_kernel(HolaArgs A) {
    constexpr int NG = D / 16, EPV = 16 / (int)sizeof(T), PPR = D / EPV;
    __shared__ int sPos[kHolaMaxW];
    __shared__ int sIdx[kHolaMaxW];
    const int bh = blockIdx.x, tid = threadIdx.x;
    const int n = A.n, C = A.C, w = A.w, nchunks = A.nchunks;
    const int nopen = n % C, cs = n - nopen;
    const int* clist = reinterpret_cast<const int*>(A.ws + A.L.clist) +
                       ((int64_t)bh * (nchunks + 1) + (nopen > 0 ? nchunks - 1 : nchunks)) * kHolaMaxW;
    const float* esq = reinterpret_cast<const float*>(A.ws + A.L.esq) + (int64_t)bh * n * NG;
    const float* beta = A.beta + (int64_t)bh * n;
    auto mag = [&](int p) {                       // as the chunk ranking forms it
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < NG; ++j) ss += esq[(int64_t)p * NG + j];
        return beta[p] * sqrtf(ss);
    };
    if (tid < kHolaMaxW) sPos[tid] = tid < w ? clist[tid] : -1;
    __syncthreads();
    if (tid < w) {                                // valid entries come first in rank order
        const int p = sPos[tid];
        int idx = tid;
        if (p >= 0) {
            idx = 0;
            for (int j = 0; j < w; ++j) idx += (sPos[j] >= 0 && sPos[j] < p) ? 1 : 0;
        }
        sIdx[tid] = idx;
        A.st_cache_pos[(int64_t)bh * w + idx] = p;
        A.st_cache_score[(int64_t)bh * w + idx] = p >= 0 ? mag(p) : 0.f;
    }
    __syncthreads();
    const T* kin = reinterpret_cast<const T*>(A.k) + (int64_t)bh * n * D;
    const T* vin = reinterpret_cast<const T*>(A.v) + (int64_t)bh * n * D;
    T* ck = reinterpret_cast<T*>(A.st_cache_k) + (int64_t)bh * w * D;
    T* cv = reinterpret_cast<T*>(A.st_cache_v) + (int64_t)bh * w * D;
    for (int it = tid; it < w * PPR; it += 256) {
        const int e = it / PPR, pc = it % PPR, p = sPos[e];
        if (p >= 0) {
            const int idx = sIdx[e];
            *reinterpret_cast<uint4*>(ck + (int64_t)idx * D + pc * EPV) = *reinterpret_cast<const uint4*>(kin + (int64_t)p * D + pc * EPV);
            *reinterpret_cast<uint4*>(cv + (int64_t)idx * D + pc * EPV) = *reinterpret_cast<const uint4*>(vin + (int64_t)p * D + pc * EPV);
        }
    }
    T* ok = reinterpret_cast<T*>(A.st_open_k) + (int64_t)bh * C * D;
    T* ov = reinterpret_cast<T*>(A.st_open_v) + (int64_t)bh * C * D;
    for (int it = tid; it < nopen * PPR; it += 256) {
        const int i = it / PPR, pc = it % PPR;
        *reinterpret_cast<uint4*>(ok + (int64_t)i * D + pc * EPV) = *reinterpret_cast<const uint4*>(kin + (int64_t)(cs + i) * D + pc * EPV);
        *reinterpret_cast<uint4*>(ov + (int64_t)i * D + pc * EPV) = *reinterpret_cast<const uint4*>(vin + (int64_t)(cs + i) * D + pc * EPV);
    }
    for (int i = tid; i < nopen; i += 256) A.st_open_score[(int64_t)bh * C + i] = mag(cs + i);
}

// ---------------- decode ----------------
// N consecutive elements of a row, 16-byte aligned, in 16-byte pieces (8 bytes when that is all).
template <typename T, int N>
__device__ __forceinline__ void load_row_piece(const T* p, T (&out)[N]) {
    constexpr int BYTES = N * (int)sizeof(T);
    static_assert(BYTES % 8 == 0, "whole 8-byte pieces");
    if constexpr (BYTES >= 16) {
#pragma unroll
        for (int u = 0; u < BYTES / 16; ++u) {
            const uint4 x = reinterpret_cast<const uint4*>(p)[u];
            __builtin_memcpy(reinterpret_cast<char*>(out) + 16 * u, &x, 16);
        }
    } else {
        const uint2 x = *reinterpret_cast<const uint2*>(p);
        __builtin_memcpy(out, &x, 8);
    }
}

// Sum over a workgroup of NT threads (every thread gets it); red holds NT / 64 floats.
template <int NT>
__device__ __forceinline__ float block_sum(float x, float* red) {
    x = wave_sum(x);
    __syncthreads();                              // red is free (its previous use is complete)
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) t += red[i];
    return t;
}
template <int NT>
__device__ __forceinline__ float block_max(float x, float* red) {
    x = wave_max(x);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    float t = -INFINITY;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) t = fmaxf(t, red[i]);
    return t;
}

// One token for every (sequence, head): one workgroup of 4D threads, thread (row group rg, column j)
// holding rows rg D/4 .. + D/4 - 1 of column j of S in registers.
//   1. unit-norm q, k for the state, the RMS-normalised, gamma-scaled query of the cache path;
//   2. S^T k and S^T q in one pass over S; e = v - alpha S^T k, m = beta |e|,
//      S <- alpha S + beta k e^T (written back), o = S_new^T q = alpha S^T q + beta (k.q) e;
//   3. the cache path over the persistent cache, the open chunk's earlier tokens and the token, with
//      the sink: logits by 16-lane groups, one row each, then the weighted sum of the value rows;
//   4. y = o + sigmoid(gate) * read-out; the token joins the open chunk; a token that closes its chunk
//      merges the chunk into the cache (top w by magnitude, ties to the older, sorted by position).
template <typename T, int D>
__global__ __launch_bounds__(4 * D) void hola_decode_kernel(HolaDecodeArgs A) {
    constexpr int NT = 4 * D, NG16 = NT / 16, EPL = D / 16;
    constexpr int EPV = 16 / (int)sizeof(T), PPR = D / EPV;
    constexpr int MAXE = kHolaMaxW + kHolaMaxC;
    constexpr int SRG = NT / (D / 4), SR = D / SRG;      // state: row groups of float4 columns, rows each
    constexpr int CPL = 8, VRG = NT / (D / CPL);         // value rows: 8 columns a thread, row groups
    static_assert(SRG == 16 && VRG == 32, "the reduction buffer holds 32 row groups");
    __shared__ float sQ[D], sK[D], sKr[D], sV[D], sU[D], sE[D];
    __shared__ __align__(16) float sPart[32][D];
    __shared__ float sRed[NT / 64];
    __shared__ float sLg[MAXE];
    __shared__ unsigned long long sKey[MAXE];
    __shared__ int sKeep[kHolaMaxW];              // kept candidates in position order
    const int bh = blockIdx.x, tid = threadIdx.x, head = bh % A.heads;
    const int w = A.w, C = A.C, nopen = A.nopen;
    const int j = tid % D;
    const float alpha = A.alpha[bh], beta = A.beta[bh];

    // 1. the token
    float qx = 0.f, kx = 0.f;
    if (tid < D) {
        qx = to_f(reinterpret_cast<const T*>(A.q)[(int64_t)bh * D + tid]);
        kx = to_f(reinterpret_cast<const T*>(A.k)[(int64_t)bh * D + tid]);
        sV[tid] = to_f(reinterpret_cast<const T*>(A.v)[(int64_t)bh * D + tid]);
        sKr[tid] = kx;
    }
    const float qq = block_sum<NT>(qx * qx, sRed);
    const float kk = block_sum<NT>(kx * kx, sRed);
    const float kq = block_sum<NT>(kx * qx, sRed);
    const float iq = qq > 0.f ? 1.0f / sqrtf(qq) : 0.f, ik = kk > 0.f ? 1.0f / sqrtf(kk) : 0.f;
    if (tid < D) {
        sQ[tid] = qx * iq;
        sK[tid] = kx * ik;
        const float qt = A.gamma_q[(int64_t)head * D + tid] * qx * (1.0f / sqrtf(qq / (float)D + kHolaRmsEps));
        sU[tid] = A.gamma_k[(int64_t)head * D + tid] * qt * (1.0f / sqrtf((float)D));
    }
    __syncthreads();

    // 2. the state: thread (row group sg, columns 4 jc .. + 3) holds D / 16 rows of four columns (in
    // registers up to d = 128, read again for the update at d = 256), as 16-byte pieces
    constexpr bool KEEP = SR <= 8;
    const int jc = tid % (D / 4), sg = tid / (D / 4);
    float* Sg = A.S + (int64_t)bh * D * D;
    f4 sr[KEEP ? SR : 1];
    f4 pk = zero4(), pq = zero4();
#pragma unroll 8
    for (int r = 0; r < SR; ++r) {
        const int i = sg * SR + r;
        const float4 v4 = *reinterpret_cast<const float4*>(Sg + (int64_t)i * D + 4 * jc);
        const f4 sv = f4{v4.x, v4.y, v4.z, v4.w};
        if (KEEP) sr[KEEP ? r : 0] = sv;
        pk += sv * sK[i];
        pq += sv * sQ[i];
    }
    *reinterpret_cast<float4*>(&sPart[sg][4 * jc]) = make_float4(pk[0], pk[1], pk[2], pk[3]);
    *reinterpret_cast<float4*>(&sPart[16 + sg][4 * jc]) = make_float4(pq[0], pq[1], pq[2], pq[3]);
    __syncthreads();
    float e = 0.f, o = 0.f;
    if (tid < D) {
        float stk = 0.f, stq = 0.f;
#pragma unroll
        for (int g2 = 0; g2 < SRG; ++g2) {
            stk += sPart[g2][j];
            stq += sPart[16 + g2][j];
        }
        e = sV[j] - alpha * stk;
        o = alpha * stq + beta * (kq * iq * ik) * e;
        sE[j] = e;
    }
    const float m = beta * sqrtf(block_sum<NT>(e * e, sRed));   // its barriers also publish sE
    {
        const f4 e4 = f4{sE[4 * jc], sE[4 * jc + 1], sE[4 * jc + 2], sE[4 * jc + 3]};
#pragma unroll 8
        for (int r = 0; r < SR; ++r) {
            const int i = sg * SR + r;
            f4 sv;
            if (KEEP) {
                sv = sr[KEEP ? r : 0];
            } else {
                const float4 v4 = *reinterpret_cast<const float4*>(Sg + (int64_t)i * D + 4 * jc);
                sv = f4{v4.x, v4.y, v4.z, v4.w};
            }
            const f4 nw = alpha * sv + (beta * sK[i]) * e4;
            *reinterpret_cast<float4*>(Sg + (int64_t)i * D + 4 * jc) = make_float4(nw[0], nw[1], nw[2], nw[3]);
        }
    }

    // 3. the cache path: entries = cache (valid slots first), open tokens, the token
    const int* cpos = A.cache_pos + (int64_t)bh * w;
    int nv = 0;
    for (int i = 0; i < w; ++i) nv += cpos[i] >= 0 ? 1 : 0;
    const int NE = nv + nopen + 1;
    const T* ck = reinterpret_cast<const T*>(A.cache_k) + (int64_t)bh * w * D;
    const T* cvv = reinterpret_cast<const T*>(A.cache_v) + (int64_t)bh * w * D;
    T* okp = reinterpret_cast<T*>(A.open_k) + (int64_t)bh * C * D;
    T* ovp = reinterpret_cast<T*>(A.open_v) + (int64_t)bh * C * D;
    {
        const int grp = tid >> 4, gl = tid & 15;
        for (int en = grp; en < NE; en += NG16) {
            float dot = 0.f, ss = 0.f;
            if (en < nv + nopen) {
                const T* kr = (en < nv ? ck + (int64_t)en * D : okp + (int64_t)(en - nv) * D) + gl * EPL;
                T kb[EPL];
                load_row_piece<T, EPL>(kr, kb);
#pragma unroll
                for (int x = 0; x < EPL; ++x) {
                    const float kv = to_f(kb[x]);
                    dot += kv * sU[gl * EPL + x];
                    ss += kv * kv;
                }
            } else {
#pragma unroll
                for (int x = 0; x < EPL; ++x) {
                    const float kv = sKr[gl * EPL + x];
                    dot += kv * sU[gl * EPL + x];
                    ss += kv * kv;
                }
            }
#pragma unroll
            for (int sh = 8; sh >= 1; sh >>= 1) {
                dot += __shfl_xor(dot, sh, 16);
                ss += __shfl_xor(ss, sh, 16);
            }
            if (gl == 0) sLg[en] = dot / sqrtf(ss / (float)D + kHolaRmsEps);
        }
    }
    __syncthreads();
    const float sink = A.sink[head];
    float lmax = -INFINITY;
    for (int en = tid; en < NE; en += NT) lmax = fmaxf(lmax, sLg[en]);
    const float mx = fmaxf(block_max<NT>(lmax, sRed), sink);
    float psum = 0.f;
    for (int en = tid; en < NE; en += NT) {
        const float p = expf(sLg[en] - mx);
        sLg[en] = p;
        psum += p;
    }
    const float den = block_sum<NT>(psum, sRed) + expf(sink - mx);   // its barriers also publish sLg
    // the value rows: thread (row group vg, columns 8 vc .. + 7), rows vg, vg + 32, ...
    {
        const int vc = tid % (D / CPL), vg = tid / (D / CPL);
        float acc[CPL];
#pragma unroll
        for (int x = 0; x < CPL; ++x) acc[x] = 0.f;
        for (int en = vg; en < NE; en += VRG) {
            const float p = sLg[en];
            if (en < nv + nopen) {
                const T* vr = (en < nv ? cvv + (int64_t)en * D : ovp + (int64_t)(en - nv) * D) + CPL * vc;
                T vb[CPL];
                load_row_piece<T, CPL>(vr, vb);
#pragma unroll
                for (int x = 0; x < CPL; ++x) acc[x] += p * to_f(vb[x]);
            } else {
#pragma unroll
                for (int x = 0; x < CPL; ++x) acc[x] += p * sV[CPL * vc + x];
            }
        }
        __syncthreads();                          // sPart is free
#pragma unroll
        for (int x = 0; x < CPL; ++x) sPart[vg][CPL * vc + x] = acc[x];
    }
    __syncthreads();

    // 4. output, the open chunk, the chunk close
    if (tid < D) {
        float rsum = 0.f;
#pragma unroll
        for (int g2 = 0; g2 < VRG; ++g2) rsum += sPart[g2][j];
        const float rd = rsum / den;
        const float gsig = 1.0f / (1.0f + expf(-A.gate[head]));
        reinterpret_cast<T*>(A.y)[(int64_t)bh * D + j] = from_f<T>(o + gsig * rd);
        okp[(int64_t)nopen * D + j] = from_f<T>(sKr[j]);
        ovp[(int64_t)nopen * D + j] = from_f<T>(sV[j]);
    }
    if (tid == 0) A.open_score[(int64_t)bh * C + nopen] = m;
    if (nopen + 1 < C || w == 0) return;           // uniform: the chunk stays open, or nothing is kept

    __syncthreads();                              // the token's row and magnitude are written
    const int N = nv + nopen + 1;
    const int64_t cs = A.t - nopen;               // first position of the closing chunk
    float* cscore = A.cache_score + (int64_t)bh * w;
    const float* oscore = A.open_score + (int64_t)bh * C;
    for (int c = tid; c < N; c += NT)
        sKey[c] = c < nv ? hola_key(cscore[c], cpos[c]) : hola_key(oscore[c - nv], (int)(cs + (c - nv)));
    __syncthreads();
    const int keep = min(w, N);
    for (int c = tid; c < N; c += NT) {
        const unsigned long long kc = sKey[c];
        int above = 0;
        for (int c2 = 0; c2 < N; ++c2) above += sKey[c2] > kc ? 1 : 0;
        sLg[c] = above < keep ? 1.f : 0.f;        // kept flag
    }
    __syncthreads();
    // kept candidates in position order: cache entries come before open ones and are sorted already
    for (int c = tid; c < N; c += NT)
        if (sLg[c] != 0.f) {
            int idx = 0;
            for (int c2 = 0; c2 < c; ++c2) idx += sLg[c2] != 0.f ? 1 : 0;
            sKeep[idx] = c;
        }
    __syncthreads();
    // rows: every source piece is read before any slot is written (a kept cache entry moves down)
    constexpr int NP = (kHolaMaxW * PPR * 2 + NT - 1) / NT;
    uint4 buf[NP];
#pragma unroll
    for (int u = 0; u < NP; ++u) {
        const int it = tid + u * NT;              // over [keep][k, v][PPR]
        buf[u] = make_uint4(0u, 0u, 0u, 0u);
        if (it < keep * 2 * PPR) {
            const int slot = it / (2 * PPR), which = (it / PPR) & 1, pc = it % PPR;
            const int c = sKeep[slot];
            const T* src = c < nv ? (which ? cvv : ck) + (int64_t)c * D : (which ? ovp : okp) + (int64_t)(c - nv) * D;
            buf[u] = *reinterpret_cast<const uint4*>(src + pc * EPV);
        }
    }
    int newpos = -1;
    float newscore = 0.f;
    if (tid < keep) {
        const int c = sKeep[tid];
        newpos = c < nv ? cpos[c] : (int)(cs + (c - nv));
        newscore = c < nv ? cscore[c] : oscore[c - nv];
    }
    __syncthreads();
    T* ckw = reinterpret_cast<T*>(A.cache_k) + (int64_t)bh * w * D;
    T* cvw = reinterpret_cast<T*>(A.cache_v) + (int64_t)bh * w * D;
#pragma unroll
    for (int u = 0; u < NP; ++u) {
        const int it = tid + u * NT;
        if (it < keep * 2 * PPR) {
            const int slot = it / (2 * PPR), which = (it / PPR) & 1, pc = it % PPR;
            *reinterpret_cast<uint4*>((which ? cvw : ckw) + (int64_t)slot * D + pc * EPV) = buf[u];
        }
    }
    if (tid < w) {
        A.cache_pos[(int64_t)bh * w + tid] = tid < keep ? newpos : -1;
        cscore[tid] = tid < keep ? newscore : 0.f;
    }
}

// An empty memory: S = 0, every cache slot empty.
__global__ __launch_bounds__(256) void hola_init_kernel(HolaInitArgs A) {
    const int64_t nS = (int64_t)A.BH * A.d * A.d, nc = (int64_t)A.BH * A.w;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nS; i += (int64_t)gridDim.x * 256) A.S[i] = 0.f;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nc; i += (int64_t)gridDim.x * 256) {
        A.cache_pos[i] = -1;
        A.cache_score[i] = 0.f;
    }
}

template <typename T, int D>
hipError_t launch_hola_t(const HolaArgs& a, hipStream_t stream) {
    const int64_t rows = (int64_t)a.BH * a.n;
    constexpr int prep_rows = 256 / (D / (16 / (int)sizeof(T)));         // rows per prep workgroup
    const unsigned rgrid = (unsigned)((rows + prep_rows - 1) / prep_rows);
    hipLaunchKernelGGL((hola_prep_kernel<T, D>), dim3(rgrid), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((hola_block_kernel<T, D>), dim3((unsigned)(((int64_t)a.BH * a.nblk + 3) / 4)), dim3(256), 0,
                       stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // four waves (one per SIMD); eight, with one row tile each, measured 22% slower at d = 128
    hipLaunchKernelGGL((hola_scan_kernel<T, D, 4>), dim3(a.BH * (D / 16)), dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.w > 0) {
        hipLaunchKernelGGL((hola_chunk_top_kernel<D>), dim3((unsigned)((int64_t)a.BH * a.nchunks)), dim3(256), 0, stream,
                           a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(hola_cache_kernel, dim3(a.BH), dim3(64), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((hola_read_kernel<T, D>), dim3((unsigned)((int64_t)a.BH * a.nchunks * a.nqt)), dim3(256), 0,
                       stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.st_open_k) {
        hipLaunchKernelGGL((hola_state_kernel<T, D>), dim3(a.BH), dim3(256), 0, stream, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename T, int D>
hipError_t launch_hola_decode_t(const HolaDecodeArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((hola_decode_kernel<T, D>), dim3(a.BH), dim3(4 * D), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_hola_decode(const HolaDecodeArgs& a, int dtype, int d, hipStream_t stream) {
    if (dtype == 0)
        return d == 64 ? launch_hola_decode_t<float, 64>(a, stream)
                       : d == 128 ? launch_hola_decode_t<float, 128>(a, stream) : launch_hola_decode_t<float, 256>(a, stream);
    return d == 64 ? launch_hola_decode_t<bf16, 64>(a, stream)
                   : d == 128 ? launch_hola_decode_t<bf16, 128>(a, stream) : launch_hola_decode_t<bf16, 256>(a, stream);
}

hipError_t launch_hola_init(const HolaInitArgs& a, hipStream_t stream) {
    const int64_t tot = (int64_t)a.BH * a.d * a.d;
    const unsigned grid = (unsigned)std::min<int64_t>(2048, (tot + 255) / 256);
    hipLaunchKernelGGL(hola_init_kernel, dim3(grid > 0 ? grid : 1), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_hola(const HolaArgs& a, int dtype, int d, hipStream_t stream) {
    if (dtype == 0)
        return d == 64 ? launch_hola_t<float, 64>(a, stream)
                       : d == 128 ? launch_hola_t<float, 128>(a, stream) : launch_hola_t<float, 256>(a, stream);
    return d == 64 ? launch_hola_t<bf16, 64>(a, stream)
                   : d == 128 ? launch_hola_t<bf16, 128>(a, stream) : launch_hola_t<bf16, 256>(a, stream);
}

}  // namespace lola
