// Query-accumulated cache scores of a prefill call (LoLA notes 4.5, Table 4; the rules of App. F).
//
// Under these rules a key's score gathers, from every query t whose window holds it (pos <= t <=
// pos + eta - 1), one term of e = exp(q_t.k / sqrt(d_k)) and p = phi(q_t).phi(k):
//   kernel_sq (e - p)^2,  kernel_abs |e - p|,  ratio p / e,  attn e.
// An allocation at a chunk start a uses the terms of the queries t < a; the score is fixed once the key
// leaves the window.  The terms do not depend on the state, so this kernel computes every key's sums
// for the whole call in parallel before the allocation chain runs, two per key:
//   score_alloc  the queries before the start of the chunk in which the key leaves the window (what its
//                own allocation sees; for a key that does not leave during the call, every query);
//   score_full   every query of the call (what later allocations and the next call see).
// Both start from the score the state carried (a window token's partial sum from earlier calls).
// The initial cache members' final scores are copied to their source rows.
//
// One workgroup: 32 keys of one (sequence, head) in position order (the initial ring tokens, then the
// call's keys).  Every wave holds all the keys and their features as A operands; the
// waves split the 16-query tiles of the band, so each query tile is loaded once per workgroup and
// serves every key tile.  e and p come from two MFMA products, the rule and the band mask run on the
// accumulators, and each key's sums are reduced over columns and then over waves at the end.
#include "lola_common.hpp"
#include "lola_internal.hpp"

namespace lola {

namespace {

__device__ __forceinline__ float rule_term(int rule, float e, float p) {
    switch (rule) {
        case kScoreKernelSq: { const float d = e - p; return d * d; }
        case kScoreKernelAbs: return fabsf(e - p);
        case kScoreRatio: return p / e;
        default: return e;   // kScoreAttn
    }
}

template <typename T> struct QsCfg {
    static constexpr int KT = 2;                         // 16-key tiles per workgroup (each wave holds all)
    static constexpr int KEYS = 16 * KT;
};

template <typename T, int DK>
__global__ __launch_bounds__(256) void qscore_kernel(PrefillArgs A) {
    constexpr int D = kFeat, KT = QsCfg<T>::KT, KEYS = QsCfg<T>::KEYS, NW = 4;
    __shared__ float sPart[2][NW][KEYS];                      // per-wave partial sums (alloc, full)
    const int bh = blockIdx.y;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c = l & 15;
    const int n = A.n, lam = A.lam, eta = A.eta, C = A.C, rule = A.score_rule;
    const int64_t t0 = A.t0, tend = t0 + n;                   // the call's queries: [t0, tend)
    const int nr = (int)(t0 < (int64_t)eta ? t0 : (int64_t)eta);   // initial ring tokens present
    char* wsb = A.ws + (int64_t)bh * A.L.per_bh;
    const T* phiStore = reinterpret_cast<const T*>(wsb + A.L.phi_store);
    const T* phiQ = phiStore + (int64_t)(n + lam + eta) * D;
    float* sAlloc = reinterpret_cast<float*>(wsb + A.L.score_alloc);
    float* sFull = reinterpret_cast<float*>(wsb + A.L.score_full);
    const T* kin = reinterpret_cast<const T*>(A.k) + (int64_t)bh * n * DK;
    const T* qin = reinterpret_cast<const T*>(A.q) + (int64_t)bh * n * DK;
    const T* ringK = eta > 0 ? reinterpret_cast<const T*>(A.win_k) + (int64_t)bh * eta * DK : nullptr;

    if (blockIdx.x == 0 && lam > 0)   // initial cache members: their final scores, as they are
        for (int j = tid; j < lam; j += 256) {
            const float v = A.cache_score[(int64_t)bh * lam + j];
            sAlloc[n + j] = v;
            sFull[n + j] = v;
        }

    const int nkeys = nr + n;
    const int kb = blockIdx.x * KEYS;                         // the workgroup's first key
    // key j (position order) -> position, source, key row
    const int64_t p0 = t0 - nr;
    auto key_of = [&](int j, int64_t& pos, int& src, const T*& row) {
        pos = p0 + j;
        if (pos >= t0) { src = (int)(pos - t0); row = kin + (int64_t)src * DK; }
        else {
            const int slot = (int)(pos % eta);
            src = n + lam + slot;
            row = ringK + (int64_t)slot * DK;
        }
    };
    // A operands: row c of key tile kt is key kb + 16 kt + c (a lane past the keys reads key kb)
    Frag8<T> kf[KT][DK / 32], pk[KT][D / 32];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        const int j = kb + 16 * kt + c;
        int64_t pos;
        int src;
        const T* row;
        key_of(j < nkeys ? j : kb, pos, src, row);
#pragma unroll
        for (int ss = 0; ss < DK / 32; ++ss) kf[kt][ss] = load_frag_contig(row, ss, g);
#pragma unroll
        for (int ss = 0; ss < D / 32; ++ss) pk[kt][ss] = load_frag_contig(phiStore + (int64_t)src * D, ss, g);
    }
    // per accumulator row (key 16 kt + 4g + r), as offsets from t0: band [pos, pos + eta) of queries,
    // and the first query its own allocation does not see (the start of the chunk in which it leaves
    // the window)
    int kpos[KT][4], kalloc[KT][4];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = kb + 16 * kt + 4 * g + r;
            kpos[kt][r] = j - nr;
            const int x = kpos[kt][r] + eta;                  // exit time
            kalloc[kt][r] = (j < nkeys && x < n) ? (x / C) * C : n;
        }
    const int64_t plast = p0 + min(kb + KEYS - 1, nkeys - 1);
    const int64_t qlo = max(p0 + kb, t0);
    const int64_t qhi = min(plast + eta, tend);               // exclusive
    const float scale = 1.0f / sqrtf((float)DK);
    float accA[KT][4], accF[KT][4];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) accA[kt][r] = accF[kt][r] = 0.f;

    // wave w takes query tiles w, w + 4, ... of the band; the next one's loads are in flight while
    // one is used, and each query tile serves all KT key tiles
    Frag8<T> qf[DK / 32], pq[D / 32], qn[DK / 32], pn[D / 32];
    auto load_q = [&](Frag8<T> (&a)[DK / 32], Frag8<T> (&b)[D / 32], int64_t tq0) {
        const int64_t t = tq0 + c < tend ? tq0 + c : tend - 1;   // a lane past the end reads a valid row
        const int i = (int)(t - t0);
#pragma unroll
        for (int ss = 0; ss < DK / 32; ++ss) a[ss] = load_frag_contig(qin + (int64_t)i * DK, ss, g);
#pragma unroll
        for (int ss = 0; ss < D / 32; ++ss) b[ss] = load_frag_contig(phiQ + (int64_t)i * D, ss, g);
    };
    const int64_t first = qlo + 16 * w;
    if (kb < nkeys && first < qhi) load_q(qn, pn, first);
    for (int64_t tq0 = first; kb < nkeys && tq0 < qhi; tq0 += 16 * NW) {
#pragma unroll
        for (int ss = 0; ss < DK / 32; ++ss) qf[ss] = qn[ss];
#pragma unroll
        for (int ss = 0; ss < D / 32; ++ss) pq[ss] = pn[ss];
        if (tq0 + 16 * NW < qhi) load_q(qn, pn, tq0 + 16 * NW);
        const int t = (int)(tq0 - t0) + c;                    // this lane's query (column c), from t0
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            f4 sacc = zero4(), pacc = zero4();
#pragma unroll
            for (int ss = 0; ss < DK / 32; ++ss) mma32(sacc, kf[kt][ss], qf[ss]);
#pragma unroll
            for (int ss = 0; ss < D / 32; ++ss) mma32(pacc, pk[kt][ss], pq[ss]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool in = t < n && t >= kpos[kt][r] && t < kpos[kt][r] + eta;
                const float f = in ? rule_term(rule, fast_exp(sacc[r] * scale), pacc[r]) : 0.f;
                accF[kt][r] += f;
                accA[kt][r] += t < kalloc[kt][r] ? f : 0.f;
            }
        }
    }
    // column sums (lane (g, 15) ends with rows 4g .. 4g + 3 of each key tile), then across waves
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float a = sum_cols_last(accA[kt][r]);
            const float f = sum_cols_last(accF[kt][r]);
            if (c == 15) {
                sPart[0][w][16 * kt + 4 * g + r] = a;
                sPart[1][w][16 * kt + 4 * g + r] = f;
            }
        }
    __syncthreads();
    for (int jj = tid; jj < KEYS; jj += 256) {
        const int j = kb + jj;
        if (j >= nkeys) continue;
        float a = 0.f, f = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) { a += sPart[0][ww][jj]; f += sPart[1][ww][jj]; }
        int64_t pos;
        int src;
        const T* row;
        key_of(j, pos, src, row);
        const float prior = pos < t0 ? A.win_score[(int64_t)bh * eta + (src - n - lam)] : 0.f;
        sAlloc[src] = prior + a;
        sFull[src] = prior + f;
    }
}

}  // namespace

template <typename T, int DK>
hipError_t launch_qscore_t(const PrefillArgs& a, hipStream_t stream) {
    const int64_t nr = a.t0 < (int64_t)a.eta ? a.t0 : (int64_t)a.eta;
    const int64_t nkeys = nr + a.n;
    constexpr int KEYS = QsCfg<T>::KEYS;
    dim3 grid((unsigned)((nkeys + KEYS - 1) / KEYS), a.BH);
    hipLaunchKernelGGL((qscore_kernel<T, DK>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

template hipError_t launch_qscore_t<float, 64>(const PrefillArgs&, hipStream_t);
template hipError_t launch_qscore_t<float, 128>(const PrefillArgs&, hipStream_t);
template hipError_t launch_qscore_t<bf16, 64>(const PrefillArgs&, hipStream_t);
template hipError_t launch_qscore_t<bf16, 128>(const PrefillArgs&, hipStream_t);

}  // namespace lola
