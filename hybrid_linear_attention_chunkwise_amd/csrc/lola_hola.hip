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
//          them while it stages rows) and the cache path's normalised q, k (storage type), 32 lanes per row;
//   scan   the delta rule, serial in t but separable in the value dimension: one workgroup per
//          (sequence, head, 256 / L columns of S), L = 8, 16 or 32 lanes per column (d / L of its rows
//          per lane, in registers), so S^T k and S^T q close with a few DPP steps.  Keys, queries, values
//          and gates are staged in LDS 32 tokens at a time, the next block loaded while one is scanned;
//   mag    m_t = beta_t ||e_t||, 32 lanes per row;
//   top    each chunk's own w largest magnitudes, all chunks in parallel;
//   cache  the persistent cache at every chunk start, serial in the chunks: one wave per (sequence,
//          head) merges each chunk's list into the current cache by rank (ties: older);
//   read   one workgroup per (sequence, head, chunk, 64 queries): softmax over the chunk's persistent
//          cache and the chunk's tokens up to each query, with the sink as the initial state of the
//          running softmax; QK^T and PV^T on MFMA with key blocks staged in LDS one block ahead; adds
//          the state read-out.
#include "lola_common.hpp"
#include "lola_internal.hpp"

#include <type_traits>

namespace lola {

namespace {

constexpr float kHolaRmsEps = 1e-6f;

template <typename T, int PER>
__device__ __forceinline__ void load_row_piece(const T* p, float (&x)[PER]) {
#pragma unroll
    for (int i = 0; i < PER; ++i) x[i] = to_f(p[i]);
}

// ---------------- prep ----------------
template <typename T, int D>
__global__ __launch_bounds__(256) void hola_prep_kernel(HolaArgs A) {
    constexpr int PER = D / 32;
    const int64_t row = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);   // over B*h*n rows
    const int lane = threadIdx.x & 31;
    if (row >= (int64_t)A.BH * A.n) return;                             // no barrier in this kernel
    const int head = (int)((row / A.n) % A.heads);
    char* wsb = A.ws;
#pragma unroll
    for (int which = 0; which < 2; ++which) {                           // 0: queries, 1: keys
        const T* src = reinterpret_cast<const T*>(which ? A.k : A.q) + row * D + lane * PER;
        float x[PER];
        load_row_piece<T, PER>(src, x);
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < PER; ++i) ss += x[i] * x[i];
#pragma unroll
        for (int sh = 1; sh < 32; sh <<= 1) ss += __shfl_xor(ss, sh, 32);
        const float inv_l2 = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;        // a zero row stays zero
        const float inv_rms = 1.0f / sqrtf(ss / (float)D + kHolaRmsEps);
        T* til = reinterpret_cast<T*>(wsb + (which ? A.L.ktil : A.L.qtil)) + row * D + lane * PER;
        const float* gam = (which ? A.gamma_k : A.gamma_q) + (int64_t)head * D + lane * PER;
#pragma unroll
        for (int i = 0; i < PER; ++i) til[i] = from_f<T>(gam[i] * x[i] * inv_rms);
        if (lane == 0) reinterpret_cast<float*>(wsb + (which ? A.L.kinv : A.L.qinv))[row] = inv_l2;
    }
}

// ---------------- scan ----------------

// The delta rule is serial in t but separable in the value dimension: column c of S only needs k, q,
// alpha, beta and v_c.  One workgroup of four waves takes 256 / LPC columns of one (sequence, head); a
// column belongs to LPC lanes of one wave, each lane holding d / LPC of its rows in registers, so S^T k
// and S^T q close with a few DPP steps and the per-token chain stays short.  S = scl * P: the decay
// multiplies the scalar scl, so the write costs one FMA per element (P += (beta e / scl) k); P is
// rescaled into S before scl gets small.  Tokens are staged in LDS TB at a time; the next block's
// operands are loaded into registers while the current block is scanned, and the outputs of a block
// leave through LDS as whole rows.
template <typename T, int D, int LPC>
__global__ __launch_bounds__(256) void hola_scan_kernel(HolaArgs A) {
    constexpr int TB = 32;                                              // tokens staged at a time
    constexpr int NT = 256;
    constexpr int CPW = NT / LPC;                                       // columns per workgroup
    constexpr int RP = D / LPC;                                         // rows per lane
    constexpr int EPV = 16 / (int)sizeof(T), PC = D / EPV;              // elements per 16-byte piece, per row
    constexpr int KVP = TB * PC / NT;                                   // pieces of k (and of q) per thread
    constexpr int VV = TB * CPW / NT;                                   // values per thread
    constexpr int OV = TB * CPW / NT;                                   // outputs per thread and array
    static_assert(LPC == 8 || LPC == 16 || LPC == 32, "lanes per column");
    static_assert(RP % 2 == 0 && KVP >= 1 && VV >= 1 && D % CPW == 0, "scan tiling");
    __shared__ __align__(16) float sK[TB][D];
    __shared__ __align__(16) float sQ[TB][D];
    __shared__ float sV[TB][CPW];
    __shared__ float sO[TB][CPW], sE[TB][CPW];
    __shared__ float sJunk[2][NT];                                      // the stores of the other lanes
    __shared__ float sAl[TB], sBe[TB];
    const int bh = blockIdx.x / (D / CPW), cb = CPW * (blockIdx.x % (D / CPW));   // first column of the part
    const int tid = threadIdx.x;
    const int cl = tid / LPC;                                           // column within the part
    const int part = tid % LPC;
    const int col = cb + cl, row0 = part * RP;
    // a column's lanes: half a DPP row, one row, or two rows paired by a lane swap; every lane gets the sum
    auto col_sum = [](float x) {
        if constexpr (LPC == 8) {
            x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
            x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
            x += dpp_mov<0x141>(x);   // row_half_mirror: the other quad of the eight lanes
        } else {
            x += dpp_mov<0x128>(x);   // row_ror:8
            x += dpp_mov<0x124>(x);   // row_ror:4
            x += dpp_mov<0x122>(x);   // row_ror:2
            x += dpp_mov<0x121>(x);   // row_ror:1
            if constexpr (LPC == 32) {
                float a, b;
                pair16(x, a, b);
                x = a + b;
            }
        }
        return x;
    };
    const int n = A.n;
    const T* kin = reinterpret_cast<const T*>(A.k) + (int64_t)bh * n * D;
    const T* qin = reinterpret_cast<const T*>(A.q) + (int64_t)bh * n * D;
    const float* kinv = reinterpret_cast<const float*>(A.ws + A.L.kinv) + (int64_t)bh * n;
    const float* qinv = reinterpret_cast<const float*>(A.ws + A.L.qinv) + (int64_t)bh * n;
    const T* vin = reinterpret_cast<const T*>(A.v) + (int64_t)bh * n * D;
    const float* al = A.alpha + (int64_t)bh * n;
    const float* be = A.beta + (int64_t)bh * n;
    float* oo = reinterpret_cast<float*>(A.ws + A.L.o) + (int64_t)bh * n * D;
    float* ee = reinterpret_cast<float*>(A.ws + A.L.e) + (int64_t)bh * n * D;

    // next block's operands in registers (raw k and q rows in 16-byte pieces with their tokens' inverse
    // norms); a token past n reads as zero
    uint4 rk[KVP], rq[KVP];
    float rkn[KVP], rqn[KVP];
    float rv[VV], ra = 0.f, rb = 0.f;
    auto fetch = [&](int t0) {
#pragma unroll
        for (int i = 0; i < KVP; ++i) {
            const int f = tid + i * NT, tk = f / PC;
            const bool in = t0 + tk < n;
            const int tt = in ? t0 + tk : n - 1;                        // always a valid row
            const int64_t off = (int64_t)tt * D + (f % PC) * EPV;
            rk[i] = *reinterpret_cast<const uint4*>(kin + off);
            rq[i] = *reinterpret_cast<const uint4*>(qin + off);
            rkn[i] = in ? kinv[tt] : 0.f;
            rqn[i] = in ? qinv[tt] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < VV; ++i) {
            const int f = tid + i * NT, tk = f / CPW;
            const bool in = t0 + tk < n;
            const float x = to_f(vin[(int64_t)(in ? t0 + tk : n - 1) * D + cb + f % CPW]);
            rv[i] = in ? x : 0.f;
        }
        if (tid < TB && t0 + tid < n) { ra = al[t0 + tid]; rb = be[t0 + tid]; }
    };
    auto stash = [&]() {
#pragma unroll
        for (int i = 0; i < KVP; ++i) {
            const int f = tid + i * NT;
            const T* kp = reinterpret_cast<const T*>(&rk[i]);
            const T* qp = reinterpret_cast<const T*>(&rq[i]);
#pragma unroll
            for (int e4 = 0; e4 < EPV; e4 += 4) {                        // unit-norm rows: x / ||x||
                *reinterpret_cast<float4*>(&sK[0][0] + f * EPV + e4) =
                    make_float4(to_f(kp[e4]) * rkn[i], to_f(kp[e4 + 1]) * rkn[i], to_f(kp[e4 + 2]) * rkn[i],
                                to_f(kp[e4 + 3]) * rkn[i]);
                *reinterpret_cast<float4*>(&sQ[0][0] + f * EPV + e4) =
                    make_float4(to_f(qp[e4]) * rqn[i], to_f(qp[e4 + 1]) * rqn[i], to_f(qp[e4 + 2]) * rqn[i],
                                to_f(qp[e4 + 3]) * rqn[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < VV; ++i) (&sV[0][0])[tid + i * NT] = rv[i];
        if (tid < TB) { sAl[tid] = ra; sBe[tid] = rb; }
    };
    auto flush = [&](int t0) {                                          // block t0's outputs, whole rows
#pragma unroll
        for (int i = 0; i < OV; ++i) {
            const int f = tid + i * NT, tk = f / CPW;
            if (t0 + tk < n) {
                const int64_t off = (int64_t)(t0 + tk) * D + cb + f % CPW;
                oo[off] = (&sO[0][0])[f];
                ee[off] = (&sE[0][0])[f];
            }
        }
    };

    float P[RP];                                                        // P[r] = S(row0 + r, col) / scl
#pragma unroll
    for (int r = 0; r < RP; ++r) P[r] = 0.f;
    float scl = 1.f;
    // one token: returns the column's read-out o and residual e.  FOLD: check whether scl must be folded
    // into P first (a block whose scales all stay above the threshold skips the check, which keeps its
    // tokens in one basic block)
    auto token = [&](int j, float& o, float& e, auto fold_tag) {
        constexpr bool FOLD = decltype(fold_tag)::value;
        float kc[RP], qc[RP];
#pragma unroll
        for (int r = 0; r < RP; r += 2) {
            const float2 k2 = *reinterpret_cast<const float2*>(&sK[j][row0 + r]);
            const float2 q2 = *reinterpret_cast<const float2*>(&sQ[j][row0 + r]);
            kc[r] = k2.x; kc[r + 1] = k2.y;
            qc[r] = q2.x; qc[r + 1] = q2.y;
        }
        const float vc = sV[j][cl], ac = sAl[j], bc = sBe[j];
        float u2[2] = {0.f, 0.f};
#pragma unroll
        for (int r = 0; r < RP; ++r) u2[r & 1] = fmaf(P[r], kc[r], u2[r & 1]);
        const float sp = ac * scl;                                      // alpha S^T k = sp * (P^T k)
        if constexpr (FOLD) {
            if (sp < 1e-20f) {                                          // fold the scale into P (S unchanged)
#pragma unroll
                for (int r = 0; r < RP; ++r) P[r] *= scl;
                scl = 1.f;
            }
        }
        const float sd = ac * scl;                                      // scale of the decayed state
        const float rs = bc * __builtin_amdgcn_rcpf(sd);                // off the chain: beta / scale
        e = fmaf(-sp, col_sum(u2[0] + u2[1]), vc);                      // v - alpha S^T k
        const float wr = rs * e;                                        // the write in P's scale
        float o2[2] = {0.f, 0.f};
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            P[r] = fmaf(wr, kc[r], P[r]);
            o2[r & 1] = fmaf(P[r], qc[r], o2[r & 1]);
        }
        o = sd * col_sum(o2[0] + o2[1]);
        scl = sd;
    };

    fetch(0);
    for (int t0 = 0; t0 < n; t0 += TB) {
        const int nb = min(TB, n - t0);
        __syncthreads();                                                // the previous block is used up
        if (t0 > 0) flush(t0 - TB);
        stash();
        __syncthreads();
        if (t0 + TB < n) fetch(t0 + TB);
        // the scales this block reaches if nothing folds: the last is the smallest
        float s = scl;
        for (int j = 0; j < nb; ++j) s = sAl[j] * s;
        if (nb == TB && s >= 1e-20f) {
            // lane `part` of a column keeps the outputs of tokens part, part + LPC, ... in registers, so
            // the block's loop writes no LDS and the next tokens' reads can run ahead
            float mo[TB / LPC], me[TB / LPC];
#pragma unroll
            for (int u = 0; u < TB / LPC; ++u) mo[u] = me[u] = 0.f;
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                float o, e;
                token(j, o, e, std::false_type{});
                mo[j / LPC] = part == j % LPC ? o : mo[j / LPC];
                me[j / LPC] = part == j % LPC ? e : me[j / LPC];
            }
#pragma unroll
            for (int u = 0; u < TB / LPC; ++u) {
                sO[part + LPC * u][cl] = mo[u];
                sE[part + LPC * u][cl] = me[u];
            }
        } else {
            for (int j = 0; j < nb; ++j) {
                float o, e;
                token(j, o, e, std::true_type{});
                float* po = part == 0 ? &sO[j][cl] : &sJunk[0][tid];    // one lane per column keeps it
                float* pe = part == 0 ? &sE[j][cl] : &sJunk[1][tid];
                *po = o;
                *pe = e;
            }
        }
    }
    __syncthreads();
    flush((n - 1) / TB * TB);
    if (A.S_out) {
        float* so = A.S_out + (int64_t)bh * D * D;
#pragma unroll
        for (int r = 0; r < RP; ++r) so[(int64_t)(row0 + r) * D + col] = P[r] * scl;
    }
}

// ---------------- write magnitude ----------------
template <int D>
__global__ __launch_bounds__(256) void hola_mag_kernel(HolaArgs A) {
    constexpr int PER = D / 32;
    const int64_t row = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
    const int lane = threadIdx.x & 31;
    if (row >= (int64_t)A.BH * A.n) return;                             // no barrier in this kernel
    const float* e = reinterpret_cast<const float*>(A.ws + A.L.e) + row * D + lane * PER;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) ss += e[i] * e[i];
#pragma unroll
    for (int sh = 1; sh < 32; sh <<= 1) ss += __shfl_xor(ss, sh, 32);
    if (lane == 0) reinterpret_cast<float*>(A.ws + A.L.m)[row] = A.beta[row] * sqrtf(ss);
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
__global__ __launch_bounds__(256) void hola_chunk_top_kernel(HolaArgs A) {
    __shared__ unsigned long long sKey[kHolaMaxC];
    const int bh = blockIdx.x / A.nchunks, ch = blockIdx.x % A.nchunks, tid = threadIdx.x;
    const int n = A.n, C = A.C, a = ch * C, nx = min(C, n - a), keep = min(A.w, nx);
    const int ls = min(kHolaMaxW, C);                                   // list stride
    const float* m = reinterpret_cast<const float*>(A.ws + A.L.m) + (int64_t)bh * n;
    unsigned long long* out = reinterpret_cast<unsigned long long*>(A.ws + A.L.tlist) + ((int64_t)bh * A.nchunks + ch) * ls;
    for (int i = tid; i < nx; i += 256) sKey[i] = hola_key(m[a + i], a + i);
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
    int* clist = reinterpret_cast<int*>(A.ws + A.L.clist) + (int64_t)bh * nchunks * kHolaMaxW;
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
    // the final cache, sorted by position, with its magnitudes
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
    const int* clist = reinterpret_cast<const int*>(A.ws + A.L.clist) + ((int64_t)bh * A.nchunks + ch) * kHolaMaxW;
    for (int j = tid; j < kHolaMaxW; j += 256) sList[j] = clist[j];
    __syncthreads();
    int nA = 0;
    while (nA < kHolaMaxW && sList[nA] >= 0) ++nA;
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
            const float alpha = expf(m_run - m_new);
#pragma unroll
            for (int J = 0; J < JT; ++J)
#pragma unroll
                for (int r = 0; r < 4; ++r) O[J][r] *= alpha;
            l_part *= alpha;
#pragma unroll
            for (int kt = 0; kt < KB / 16; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = st[kt][r] != -INFINITY ? expf(st[kt][r] - m_new) : 0.f;
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

template <typename T, int D>
hipError_t launch_hola_t(const HolaArgs& a, hipStream_t stream) {
    const int64_t rows = (int64_t)a.BH * a.n;
    const unsigned rgrid = (unsigned)((rows + 7) / 8);
    hipLaunchKernelGGL((hola_prep_kernel<T, D>), dim3(rgrid), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // lanes per column of S: the fewest (least reduction work per token) whose grid still covers the
    // compute units; each workgroup takes 256 / lanes columns
    const int ncu = device_cus();
    if ((int64_t)a.BH * (D / 32) >= ncu)
        hipLaunchKernelGGL((hola_scan_kernel<T, D, 8>), dim3(a.BH * (D / 32)), dim3(256), 0, stream, a);
    else if ((int64_t)a.BH * (D / 16) >= ncu)
        hipLaunchKernelGGL((hola_scan_kernel<T, D, 16>), dim3(a.BH * (D / 16)), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((hola_scan_kernel<T, D, 32>), dim3(a.BH * (D / 8)), dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((hola_mag_kernel<D>), dim3(rgrid), dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.w > 0) {
        hipLaunchKernelGGL(hola_chunk_top_kernel, dim3((unsigned)((int64_t)a.BH * a.nchunks)), dim3(256), 0, stream, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(hola_cache_kernel, dim3(a.BH), dim3(64), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((hola_read_kernel<T, D>), dim3((unsigned)((int64_t)a.BH * a.nchunks * a.nqt)), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_hola(const HolaArgs& a, int dtype, int d, hipStream_t stream) {
    if (dtype == 0) return d == 64 ? launch_hola_t<float, 64>(a, stream) : launch_hola_t<float, 128>(a, stream);
    return d == 64 ? launch_hola_t<bf16, 64>(a, stream) : launch_hola_t<bf16, 128>(a, stream);
}

}  // namespace lola
