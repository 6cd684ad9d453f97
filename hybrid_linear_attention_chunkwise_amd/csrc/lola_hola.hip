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
//   prep   one pass over the tokens: unit-norm q, k for the state (fp32) and the cache path's
//          normalised q, k (storage type), 32 lanes per row;
//   scan   the delta rule, serial in t but separable in the value dimension: one workgroup per
//          (sequence, head, 16 columns of S), a 16-lane row per column (d/16 of its rows per lane, in
//          registers), so S^T k and S^T q close with DPP rotations.  Keys, queries, values and gates
//          are staged in LDS 32 tokens at a time;
//   mag    m_t = beta_t ||e_t||, 32 lanes per row;
//   cache  the persistent cache at every chunk start, serial in the chunks: one workgroup per (sequence,
//          head) keeps the current cache and merges each chunk into it by exact rank (ties: older);
//   read   one workgroup per (sequence, head, chunk, 64 queries): softmax over the chunk's persistent
//          cache and the chunk's tokens up to each query, with the sink as the initial state of the
//          running softmax; QK^T and PV^T on MFMA with key blocks staged in LDS; adds the state read-out.
#include "lola_common.hpp"
#include "lola_internal.hpp"

namespace lola {

namespace {

constexpr float kHolaRmsEps = 1e-6f;
constexpr int kHolaScanLanes = 32;   // lanes per column of S in the scan

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
        float* hat = reinterpret_cast<float*>(wsb + (which ? A.L.khat : A.L.qhat)) + row * D + lane * PER;
        T* til = reinterpret_cast<T*>(wsb + (which ? A.L.ktil : A.L.qtil)) + row * D + lane * PER;
        const float* gam = (which ? A.gamma_k : A.gamma_q) + (int64_t)head * D + lane * PER;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            hat[i] = x[i] * inv_l2;
            til[i] = from_f<T>(gam[i] * x[i] * inv_rms);
        }
    }
}

// ---------------- scan ----------------
// Sum over the 16 lanes of a DPP row (every lane gets the total): rotations by 8, 4, 2, 1.
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp_mov<0x128>(x);   // row_ror:8
    x += dpp_mov<0x124>(x);   // row_ror:4
    x += dpp_mov<0x122>(x);   // row_ror:2
    x += dpp_mov<0x121>(x);   // row_ror:1
    return x;
}

// The delta rule is serial in t but separable in the value dimension: column c of S only needs k, q,
// alpha, beta and v_c.  One workgroup of four waves takes 16 columns of one (sequence, head); a column
// belongs to one 16-lane row of a wave, each lane holding d/16 of its rows in registers, so S^T k and
// S^T q close with four DPP rotations and the per-token chain stays short.  S = scl * P: the decay
// multiplies the scalar scl, so the write costs one FMA per element (P += (beta e / scl) k); P is
// rescaled into S before scl gets small.
template <typename T, int D>
__global__ __launch_bounds__(256) void hola_scan_kernel(HolaArgs A) {
    constexpr int TB = 32;                                              // tokens staged at a time
    constexpr int LPC = kHolaScanLanes;                                 // lanes per column: 16 or 32
    constexpr int CPW = 256 / LPC;                                      // columns per workgroup
    constexpr int RP = D / LPC;                                         // rows per lane
    constexpr int NT = 256;
    __shared__ __align__(16) float sK[TB][D];
    __shared__ __align__(16) float sQ[TB][D];
    __shared__ __align__(16) float sV[TB][CPW];
    __shared__ float sAl[TB], sBe[TB];
    const int bh = blockIdx.x / (D / CPW), cb = CPW * (blockIdx.x % (D / CPW));   // first column of the part
    const int tid = threadIdx.x;
    const int cl = tid / LPC;                                           // column within the part
    const int part = tid % LPC;
    const int col = cb + cl, row0 = part * RP;
    // a column's lanes: one 16-lane DPP row, or two rows paired by a lane swap
    auto col_sum = [](float x) {
        x = row_sum16(x);
        if constexpr (LPC == 32) {
            float a, b;
            pair16(x, a, b);
            x = a + b;
        }
        return x;
    };
    const int n = A.n;
    const float* kh = reinterpret_cast<const float*>(A.ws + A.L.khat) + (int64_t)bh * n * D;
    const float* qh = reinterpret_cast<const float*>(A.ws + A.L.qhat) + (int64_t)bh * n * D;
    const T* vin = reinterpret_cast<const T*>(A.v) + (int64_t)bh * n * D;
    const float* al = A.alpha + (int64_t)bh * n;
    const float* be = A.beta + (int64_t)bh * n;
    float* oo = reinterpret_cast<float*>(A.ws + A.L.o) + (int64_t)bh * n * D;
    float* ee = reinterpret_cast<float*>(A.ws + A.L.e) + (int64_t)bh * n * D;
    float P[RP];                                                        // P[r] = S(row0 + r, col) / scl
#pragma unroll
    for (int r = 0; r < RP; ++r) P[r] = 0.f;
    float scl = 1.f;
    for (int t0 = 0; t0 < n; t0 += TB) {
        const int nb = min(TB, n - t0);
        __syncthreads();                                                // the previous block is used up
        for (int i = tid; i < nb * D; i += NT) {
            sK[i / D][i % D] = kh[(int64_t)t0 * D + i];
            sQ[i / D][i % D] = qh[(int64_t)t0 * D + i];
        }
        for (int i = tid; i < nb * CPW; i += NT) sV[i / CPW][i % CPW] = to_f(vin[(int64_t)(t0 + i / CPW) * D + cb + i % CPW]);
        if (tid < nb) { sAl[tid] = al[t0 + tid]; sBe[tid] = be[t0 + tid]; }
        __syncthreads();
        // the next token's operands are read from LDS while the current one is computed
        float kc[RP], qc[RP];
#pragma unroll
        for (int r = 0; r < RP; ++r) { kc[r] = sK[0][row0 + r]; qc[r] = sQ[0][row0 + r]; }
        float vc = sV[0][cl], ac = sAl[0], bc = sBe[0];
        for (int j = 0; j < nb; ++j) {
            const int jn = j + 1 < nb ? j + 1 : j;
            float kn[RP], qn[RP];
#pragma unroll
            for (int r = 0; r < RP; ++r) { kn[r] = sK[jn][row0 + r]; qn[r] = sQ[jn][row0 + r]; }
            const float vn = sV[jn][cl], an = sAl[jn], bnx = sBe[jn];
            float u2[2] = {0.f, 0.f};
#pragma unroll
            for (int r = 0; r < RP; ++r) u2[r & 1] = fmaf(P[r], kc[r], u2[r & 1]);
            const float stk = scl * col_sum(u2[0] + u2[1]);             // (S^T k)_col
            if (ac * scl < 1e-20f) {                                    // fold the scale into P (S unchanged)
#pragma unroll
                for (int r = 0; r < RP; ++r) P[r] *= scl;
                scl = 1.f;
            }
            const float sd = ac * scl;                                  // scale of the decayed state
            const float e = vc - ac * stk;                              // residual of the decayed prediction
            const float wr = bc * e / sd;                               // the write in P's scale
            float o2[2] = {0.f, 0.f};
#pragma unroll
            for (int r = 0; r < RP; ++r) {
                P[r] = fmaf(wr, kc[r], P[r]);
                o2[r & 1] = fmaf(P[r], qc[r], o2[r & 1]);
            }
            const float o = sd * col_sum(o2[0] + o2[1]);
            scl = sd;
            if (part == 0) {
                oo[(int64_t)(t0 + j) * D + col] = o;
                ee[(int64_t)(t0 + j) * D + col] = e;
            }
#pragma unroll
            for (int r = 0; r < RP; ++r) { kc[r] = kn[r]; qc[r] = qn[r]; }
            vc = vn; ac = an; bc = bnx;
        }
    }
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
// Ranking key: larger = kept first; equal magnitudes rank the older position higher.
__device__ __forceinline__ unsigned long long hola_key(float m, int pos) {
    return ((unsigned long long)__float_as_uint(m) << 32) | (unsigned long long)(0xFFFFFFFFu - (unsigned)pos);
}

__global__ __launch_bounds__(256) void hola_cache_kernel(HolaArgs A) {
    __shared__ int sCur[kHolaMaxW];
    __shared__ int sCand[kHolaMaxW + kHolaMaxC];
    __shared__ unsigned long long sKey[kHolaMaxW + kHolaMaxC];
    __shared__ int sCount;
    const int bh = blockIdx.x, tid = threadIdx.x;
    const int n = A.n, C = A.C, w = A.w, nchunks = A.nchunks;
    const float* m = reinterpret_cast<const float*>(A.ws + A.L.m) + (int64_t)bh * n;
    int* clist = reinterpret_cast<int*>(A.ws + A.L.clist) + (int64_t)bh * nchunks * kHolaMaxW;
    int ncur = 0;
    for (int ch = 0; ch <= nchunks; ++ch) {
        // the cache at the start of chunk ch (after the last chunk: the final cache)
        if (ch < nchunks)
            for (int j = tid; j < kHolaMaxW; j += 256) clist[(int64_t)ch * kHolaMaxW + j] = j < ncur ? sCur[j] : -1;
        else {
            // final cache, sorted by position, with its magnitudes
            for (int i = tid; i < ncur; i += 256) {
                const int p = sCur[i];
                int before = 0;
                for (int j = 0; j < ncur; ++j) before += sCur[j] < p;
                if (A.cache_pos_out) A.cache_pos_out[(int64_t)bh * w + before] = p;
                if (A.cache_score_out) A.cache_score_out[(int64_t)bh * w + before] = m[p];
            }
            for (int i = ncur + tid; i < w; i += 256) {
                if (A.cache_pos_out) A.cache_pos_out[(int64_t)bh * w + i] = -1;
                if (A.cache_score_out) A.cache_score_out[(int64_t)bh * w + i] = 0.f;
            }
            break;
        }
        // candidates: the current cache and this chunk's tokens; keep the w largest
        const int a = ch * C, nx = min(C, n - a);
        const int nc = ncur + nx;
        for (int i = tid; i < nc; i += 256) {
            const int p = i < ncur ? sCur[i] : a + (i - ncur);
            sCand[i] = p;
            sKey[i] = hola_key(m[p], p);
        }
        if (tid == 0) sCount = 0;
        __syncthreads();
        const int keep = min(w, nc);
        for (int i = tid; i < nc; i += 256) {
            const unsigned long long ki = sKey[i];
            int above = 0;
#pragma unroll 16
            for (int j = 0; j < nc; ++j) above += sKey[j] > ki;    // unrolled: the LDS reads overlap
            if (above < keep) sCur[atomicAdd(&sCount, 1)] = sCand[i];
        }
        __syncthreads();
        ncur = keep;
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

    for (int kb = 0; kb * KB < NK; ++kb) {
        __syncthreads();                                                // the previous block is used up
        for (int i = tid; i < KB * (D / EPV); i += 256) {              // keys, 16-byte pieces
            const int j = i / (D / EPV), p = i % (D / EPV);
            const int kk = kb * KB + j;
            uint4 x = make_uint4(0, 0, 0, 0);
            if (kk < NK) x = *reinterpret_cast<const uint4*>(ktil + (int64_t)key_pos(kk) * D + p * EPV);
            *reinterpret_cast<uint4*>(sK + j * K_LD + p * EPV) = x;
        }
        for (int i = tid; i < KB * D; i += 256) {                      // values, transposed
            const int j = i % KB, d = i / KB;
            const int kk = kb * KB + j;
            sVT[d * VT_LD + j] = kk < NK ? vin[(int64_t)key_pos(kk) * D + d] : from_f<T>(0.f);
        }
        for (int j = tid; j < KB; j += 256) sPos[j] = kb * KB + j < NK ? key_pos(kb * KB + j) : -1;
        __syncthreads();
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
    hipLaunchKernelGGL((hola_scan_kernel<T, D>), dim3(a.BH * (D / (256 / kHolaScanLanes))), dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((hola_mag_kernel<D>), dim3(rgrid), dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(hola_cache_kernel, dim3(a.BH), dim3(256), 0, stream, a);
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
