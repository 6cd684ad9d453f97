// Prefill read-out: one workgroup per (sequence/head, chunk, 64-query tile); four waves of 16 queries.
//
// Eq. (14) of the LoLA notes (2.5) with the chunk schedule the chain kernel recorded:
//   linear part  L(t) = H_c^T phi(q_t) + sum_{i in S_c, tau_i <= t} (phi(q_t).phi(k_i)) v_i
//   exact part   E(t) = sum_{i in window(t) U cache_c, i not linear} exp(q_t.k_i / sqrt(d_k)) v_i
//   y_t = (L + E) / (L_den + E_den), one shared denominator.
// H_c is the chunk-start snapshot; S_c the tokens folded by chunk c (tau_i = max(i + eta, chunk start));
// cache_c the cache after chunk c's allocation.  A cache key that is still inside query t's window is
// read through the window, so no key is counted twice.
//
// Contractions run on MFMA in the transposed orientation (values x queries): the score tile K Q^T
// comes out with the key index along the accumulator rows, which is the layout the P V^T product
// needs for its B operand, so probabilities never leave registers.  Key and value blocks of 64 are
// staged once per workgroup in LDS (values transposed) and shared by the four waves; the next
// block's 16-byte loads are in flight while the current block is used.
#include "lola_common.hpp"
#include "lola_internal.hpp"

#include <algorithm>
#include <type_traits>

namespace lola {

namespace {

template <typename T>
__device__ __forceinline__ void store4o(T* dst, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4o<float>(float* dst, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
}
template <>
__device__ __forceinline__ void store4o<bf16>(bf16* dst, float a, float b, float c, float d) {
    bf16x4 v;
    v[0] = (bf16)a; v[1] = (bf16)b; v[2] = (bf16)c; v[3] = (bf16)d;
    *reinterpret_cast<bf16x4*>(dst) = v;
}

template <typename T>
__device__ __forceinline__ Frag8<T> frag_from_rows(const float (&lo)[4], const float (&hi)[4]) {
    return frag_from_acc<T>(f4{lo[0], lo[1], lo[2], lo[3]}, f4{hi[0], hi[1], hi[2], hi[3]});
}

// NB: key blocks in flight.  1 keeps the registers low enough for two workgroups per CU (the bulk of
// the read-out, beside the chain); 2 is for the last chunk range, whose workgroups run alone.
template <typename T, int DK, int PHI, int NB>
__global__ __launch_bounds__(256) void readout_kernel(PrefillArgs A) {
    constexpr int D = kFeat, DV = DK, JT = DV / 16;
    constexpr int DW = (PHI == kPhiSoftmaxPM) ? D / 2 : D;
    constexpr int EPV = 16 / (int)sizeof(T);
    constexpr int WT_LD = DK + 4, KB = 64, K_LD = DK + EPV, VT_LD = KB + EPV;
    constexpr int CPK = DK / EPV;                   // 16-byte pieces per key row
    constexpr int KPT = KB * CPK / 256;             // key pieces per thread per block
    constexpr int TPW = 4 / (int)sizeof(T);         // keys packed per 32-bit LDS word
    constexpr int NCG = 256 * TPW / KB;             // value column groups
    constexpr int VD = DV / NCG;                    // value columns per thread
    constexpr int VPT = VD / EPV;                   // value pieces per key and thread
    __shared__ __align__(16) T wt[DW * WT_LD];
    __shared__ __align__(16) T sK[KB * K_LD];
    __shared__ __align__(16) T sVT[DV * VT_LD];
    __shared__ float sS[D];
    __shared__ int sKeyPos[KB];
    __shared__ int sKeyBand[KB];
    __shared__ int sFoldPos[128];
    __shared__ int sFoldSrc[128];
    __shared__ int sCachePos[kMaxLambda];
    __shared__ int sCacheSrc[kMaxLambda];

    const int nqt = A.nqt, nseg = A.c_end - A.c_begin;
    const int bid = blockIdx.x;
    const int qt = bid % nqt;
    const int ch = A.c_begin + (bid / nqt) % nseg;
    const int bh = bid / (nqt * nseg);
    const int n = A.n, C = A.C, eta = A.eta, lam = A.lam;
    const int64_t t0 = A.t0;
    const int64_t a = t0 + (int64_t)ch * C;
    const int64_t b = min(a + (int64_t)C, t0 + (int64_t)n);
    const int64_t q0 = a + 64 * qt;
    if (q0 >= b) return;   // whole workgroup: ragged last chunk

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c = l & 15;
    const char* rec = A.ws + (int64_t)bh * A.L.per_bh + A.L.chunk0 + (int64_t)ch * A.L.per_chunk;
    const T* snapH = reinterpret_cast<const T*>(rec + A.L.c_snap_h);
    const float* snapS = reinterpret_cast<const float*>(rec + A.L.c_snap_s);
    const int* cachePos = reinterpret_cast<const int*>(rec + A.L.c_cache_pos);
    const int* cacheSrc = reinterpret_cast<const int*>(rec + A.L.c_cache_src);
    const int nf = *reinterpret_cast<const int*>(rec + A.L.c_fold_n);
    const int* foldPos = reinterpret_cast<const int*>(rec + A.L.c_fold_pos);
    const int* foldSrc = reinterpret_cast<const int*>(rec + A.L.c_fold_src);
    const T* phiStore = reinterpret_cast<const T*>(A.ws + (int64_t)bh * A.L.per_bh + A.L.phi_store);
    const T* foldVT = reinterpret_cast<const T*>(rec + A.L.c_fold_vt);
    const int cpv = A.L.c_pad64;

    const T* qin = reinterpret_cast<const T*>(A.q) + (int64_t)bh * n * DK;
    const T* kin = reinterpret_cast<const T*>(A.k) + (int64_t)bh * n * DK;
    const T* vin = reinterpret_cast<const T*>(A.v) + (int64_t)bh * n * DV;
    const T* ringK = eta > 0 ? reinterpret_cast<const T*>(A.win_k) + (int64_t)bh * eta * DK : nullptr;
    const T* ringV = eta > 0 ? reinterpret_cast<const T*>(A.win_v) + (int64_t)bh * eta * DV : nullptr;
    const T* cK = lam > 0 ? reinterpret_cast<const T*>(A.cache_k) + (int64_t)bh * lam * DK : nullptr;
    const T* cV = lam > 0 ? reinterpret_cast<const T*>(A.cache_v) + (int64_t)bh * lam * DV : nullptr;
    T* yout = reinterpret_cast<T*>(A.y) + (int64_t)bh * n * DV;

    // exact keys of this query tile: its window band, then the chunk's cache list
    const int64_t blo = max((int64_t)0, q0 - eta + 1);
    const int64_t bhi = min(q0 + 63, b - 1);
    const int nb = (eta > 0 && bhi >= blo) ? (int)(bhi - blo + 1) : 0;
    const int NK = nb + ((A.read_mask & kReadSparse) ? lam : 0);   // a hidden cache adds no keys
    const int blo_slot = eta > 0 ? (int)(blo % eta) : 0;    // ring slot of the first band key
    const int nblk = (NK + KB - 1) / KB;
    // key kk -> (position, band?, K row, V row); position -1 = no key.  The chunk's cache list is read
    // from memory for the first block and from its LDS copy after that (one memory latency per block).
    auto key_rows = [&](int kk, int& pos, int& band, const T*& rk, const T*& rv, auto fromLds) {
        pos = -1; band = 0; rk = nullptr; rv = nullptr;
        if (kk < nb) {
            const int64_t ps = blo + kk;
            pos = (int)ps;
            band = 1;
            if (ps >= t0) { rk = kin + (ps - t0) * DK; rv = vin + (ps - t0) * DV; }
            else {
                const int sl = (int)((blo_slot + kk) % eta);
                rk = ringK + sl * DK;
                rv = ringV + sl * DV;
            }
        } else if (kk < NK) {
            const int jj = kk - nb;
            const int p = decltype(fromLds)::value ? sCachePos[jj] : cachePos[jj];
            if (p >= 0) {
                pos = p;
                const int src = decltype(fromLds)::value ? sCacheSrc[jj] : cacheSrc[jj];
                if (src < n) { rk = kin + (int64_t)src * DK; rv = vin + (int64_t)src * DV; }
                else if (src < n + lam) { rk = cK + (int64_t)(src - n) * DK; rv = cV + (int64_t)(src - n) * DV; }
                else { rk = ringK + (int64_t)(src - n - lam) * DK; rv = ringV + (int64_t)(src - n - lam) * DV; }
            }
        }
    };
    // A key block in flight: its key pieces, value pieces, positions and band flags.  NB buffers, so
    // the loads of the next NB blocks are in flight while a block is used.
    struct KVBuf {
        uint4 k[KPT];
        uint4 v[TPW][VPT];
        int pos[TPW], band[TPW];
    };
    auto prefetch = [&](KVBuf& bf, int kb, auto fromLds) {
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            const int q = tid + 256 * u;
            const int j = q / CPK, p = q % CPK;
            int pos, band;
            const T* rk;
            const T* rv;
            key_rows(kb * KB + j, pos, band, rk, rv, fromLds);
            bf.k[u] = rk ? *reinterpret_cast<const uint4*>(rk + p * EPV) : make_uint4(0, 0, 0, 0);
        }
        {   // values: thread -> (TPW consecutive keys, one column group)
            const int j0 = (tid % (KB / TPW)) * TPW, cg = tid / (KB / TPW);
#pragma unroll
            for (int z = 0; z < TPW; ++z) {
                const T* rk;
                const T* rv;
                key_rows(kb * KB + j0 + z, bf.pos[z], bf.band[z], rk, rv, fromLds);
#pragma unroll
                for (int u = 0; u < VPT; ++u)
                    bf.v[z][u] = rv ? *reinterpret_cast<const uint4*>(rv + cg * VD + u * EPV) : make_uint4(0, 0, 0, 0);
            }
        }
    };
    KVBuf bufs[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i)
        if (i < nblk) prefetch(bufs[i], i, std::false_type{});

    stage_wt<T, DK, DW, 256>(wt, WT_LD, A.W);
    for (int d = tid; d < D; d += 256) sS[d] = snapS[d];
    for (int i = tid; i < nf; i += 256) { sFoldPos[i] = foldPos[i]; sFoldSrc[i] = foldSrc[i]; }
    for (int j = tid; j < lam; j += 256) { sCachePos[j] = cachePos[j]; sCacheSrc[j] = cacheSrc[j]; }
    __syncthreads();

    const int64_t tq = q0 + 16 * w + c;          // this lane's query (column c of the wave's tile)
    const bool qvalid = tq < b;
    const bool wave_active = q0 + 16 * w < b;

    // queries as B operand (column c = query), and their features
    Frag8<T> qf[DK / 32];
#pragma unroll
    for (int ss = 0; ss < DK / 32; ++ss) qf[ss] = qvalid ? load_frag(qin + (tq - t0) * DK, ss, g) : frag_zero<T>();
    // exact part: blocks of KB keys staged in LDS (keys row-major, values transposed)
    const float scale = 1.0f / sqrtf((float)DK);
    float m_run = -INFINITY, l_part = 0.f;
    f4 O[JT];
#pragma unroll
    for (int J = 0; J < JT; ++J) O[J] = zero4();

    auto stage = [&](const KVBuf& bf) {
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            const int q = tid + 256 * u;
            const int j = q / CPK, p = q % CPK;
            *reinterpret_cast<uint4*>(sK + j * K_LD + p * EPV) = bf.k[u];
        }
        {   // transposed value block: whole 32-bit words, consecutive threads -> consecutive words
            const int j0 = (tid % (KB / TPW)) * TPW, cg = tid / (KB / TPW);
#pragma unroll
            for (int u = 0; u < VPT; ++u)
#pragma unroll
                for (int x = 0; x < EPV; ++x) {
                    T word[TPW];
#pragma unroll
                    for (int z = 0; z < TPW; ++z) word[z] = reinterpret_cast<const T*>(&bf.v[z][u])[x];
                    *reinterpret_cast<uint32_t*>(sVT + (cg * VD + u * EPV + x) * VT_LD + j0) =
                        *reinterpret_cast<const uint32_t*>(word);
                }
            if (cg == 0)
#pragma unroll
                for (int z = 0; z < TPW; ++z) { sKeyPos[j0 + z] = bf.pos[z]; sKeyBand[j0 + z] = bf.band[z]; }
        }
    };
    auto compute = [&]() {
        if (wave_active) {
            f4 st[KB / 16];
#pragma unroll
            for (int kt = 0; kt < KB / 16; ++kt) {
                st[kt] = zero4();
#pragma unroll
                for (int ss = 0; ss < DK / 32; ++ss) mma32(st[kt], load_frag(sK + (16 * kt + c) * K_LD, ss, g), qf[ss]);
            }
            float bmax = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < KB / 16; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * kt + 4 * g + r;
                    const int pos = sKeyPos[j];
                    bool ok;
                    if (sKeyBand[j]) ok = pos >= 0 && (int64_t)pos <= tq && (int64_t)pos >= tq - eta + 1;
                    else ok = pos >= 0 && (int64_t)pos <= tq - eta;
                    const float sc = ok ? st[kt][r] * scale : -INFINITY;
                    st[kt][r] = sc;
                    bmax = fmaxf(bmax, sc);
                }
            bmax = max_groups(bmax);
            const float m_new = fmaxf(m_run, bmax);
            const bool any = m_new != -INFINITY;
            const float alpha = (any && m_run != -INFINITY) ? fast_exp(m_run - m_new) : (any ? 0.f : 1.f);
#pragma unroll
            for (int J = 0; J < JT; ++J)
#pragma unroll
                for (int r = 0; r < 4; ++r) O[J][r] *= alpha;
            l_part *= alpha;
#pragma unroll
            for (int kt = 0; kt < KB / 16; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = (st[kt][r] != -INFINITY) ? fast_exp(st[kt][r] - m_new) : 0.f;
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
    };
    for (int kb0 = 0; kb0 < nblk; kb0 += NB) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int kb = kb0 + i;
            if (kb < nblk) {
                stage(bufs[i]);
                __syncthreads();
                if (kb + NB < nblk) prefetch(bufs[i], kb + NB, std::true_type{});
                compute();
                __syncthreads();
            }
        }
    }

    // linear part (skipped when the read mask hides the state: no terms in numerator or denominator)
    f4 L[JT];
#pragma unroll
    for (int J = 0; J < JT; ++J) L[J] = zero4();
    float lden = 0.f;
    if (A.read_mask & kReadState) {
        // linear part, after the exact loop so its registers are not live during it
        float ph[D / 16][4];
        phi_tile<T, DK, PHI>(wt, WT_LD, qf, ph);
        Frag8<T> pf[D / 32];
#pragma unroll
        for (int ss = 0; ss < D / 32; ++ss) pf[ss] = frag_from_rows<T>(ph[2 * ss], ph[2 * ss + 1]);

        // linear part: H_c^T phi(Q)^T (snapshot stored in fragment order) and phi(Q) s_c
#pragma unroll
        for (int ss = 0; ss < D / 32; ++ss)
#pragma unroll
            for (int J = 0; J < JT; ++J)
                mma32(L[J], *reinterpret_cast<const Frag8<T>*>(snapH + ((int64_t)(J * (D / 32) + ss) * 64 + l) * 8), pf[ss]);
#pragma unroll
        for (int ft = 0; ft < D / 16; ++ft)
#pragma unroll
            for (int r = 0; r < 4; ++r) lden += ph[ft][r] * sS[16 * ft + 4 * g + r];
        lden = sum_groups(lden);

        // tokens folded by this chunk become linear at tau = max(exit time, chunk start).  fold_group
        // handles FG groups of 32 folded tokens: every load of the groups (their features and transposed
        // values) is issued before any of it is used.  The last-range variant takes 64 tokens per round
        // trip; the bulk variant 32, which keeps its registers within two workgroups per CU.
        float lden_f = 0.f;
        auto fold_group = [&](int fb0, auto fgc) {
            constexpr int FG = decltype(fgc)::value;
            Frag8<T> af[FG][2][D / 32], vf[FG][JT];
#pragma unroll
            for (int f2 = 0; f2 < FG; ++f2) {
                const int fb = fb0 + f2;
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const int i = 32 * fb + 16 * h2 + c;
                    const T* prow = i < nf ? phiStore + (int64_t)sFoldSrc[i] * D : nullptr;
#pragma unroll
                    for (int ss = 0; ss < D / 32; ++ss) af[f2][h2][ss] = prow ? load_frag(prow, ss, g) : frag_zero<T>();
                }
#pragma unroll
                for (int J = 0; J < JT; ++J)
                    vf[f2][J] = fb * 32 < nf ? load_frag(foldVT + (int64_t)(16 * J + c) * cpv, fb, g) : frag_zero<T>();
            }
#pragma unroll
            for (int f2 = 0; f2 < FG; ++f2) {
                const int fb = fb0 + f2;
                f4 sp[2];
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    sp[h2] = zero4();
#pragma unroll
                    for (int ss = 0; ss < D / 32; ++ss) mma32(sp[h2], af[f2][h2][ss], pf[ss]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int ii = 32 * fb + 16 * h2 + 4 * g + r;
                        bool ok = false;
                        if (ii < nf) {
                            const int64_t tau = max((int64_t)sFoldPos[ii] + eta, a);
                            ok = tau <= tq;
                        }
                        sp[h2][r] = ok ? sp[h2][r] : 0.f;
                        lden_f += sp[h2][r];
                    }
                }
                const Frag8<T> bw = frag_from_acc<T>(sp[0], sp[1]);
#pragma unroll
                for (int J = 0; J < JT; ++J) mma32(L[J], vf[f2][J], bw);
            }
        };
        constexpr int FG = NB >= 2 ? 2 : 1;
        for (int fb0 = 0; fb0 * 32 < nf; fb0 += FG) fold_group(fb0, std::integral_constant<int, FG>{});
        lden += sum_groups(lden_f);
    }

    // joint normalisation with a common scale exp(-cmax), cmax = max(m, log L_den)
    const float lsum = sum_groups(l_part);
    if (qvalid) {
        float cm;
        if (lden > 0.f) cm = (m_run != -INFINITY) ? fmaxf(m_run, logf(lden)) : logf(lden);
        else cm = m_run;
        const float sl = lden > 0.f ? fast_exp(-cm) : 0.f;
        const float se = m_run != -INFINITY ? fast_exp(m_run - cm) : 0.f;
        const float inv = 1.f / (lden * sl + lsum * se);
        T* yrow = yout + (tq - t0) * DV;
#pragma unroll
        for (int J = 0; J < JT; ++J)
            store4o<T>(yrow + 16 * J + 4 * g, (L[J][0] * sl + O[J][0] * se) * inv, (L[J][1] * sl + O[J][1] * se) * inv,
                       (L[J][2] * sl + O[J][2] * se) * inv, (L[J][3] * sl + O[J][3] * se) * inv);
    }
}

// Commit, one workgroup per (sequence, head), in two phases split by a barrier:
//  1. the final cache members' K/V into the state's slots (a member may come from the initial window
//     ring, so this completes before the ring is overwritten), and the slots' positions;
//  2. the last eta input tokens into the window ring.
// Rows move as 16-byte pieces; each thread has UN loads in flight.
constexpr int kCommitThreads = 1024;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));   // 16 bytes, a native vector

template <typename T, int DK>
__global__ __launch_bounds__(kCommitThreads) void commit_kernel(PrefillArgs A) {
    constexpr int DV = DK, EPV = 16 / (int)sizeof(T), CPR = DK / EPV, UN = 4, NTH = kCommitThreads;
    const int bh = blockIdx.x, tid = threadIdx.x;
    const int n = A.n, eta = A.eta, lam = A.lam;
    const int64_t t0 = A.t0;
    const T* kin = reinterpret_cast<const T*>(A.k) + (int64_t)bh * n * DK;
    const T* vin = reinterpret_cast<const T*>(A.v) + (int64_t)bh * n * DV;
    T* ringK = eta > 0 ? reinterpret_cast<T*>(A.win_k) + (int64_t)bh * eta * DK : nullptr;
    T* ringV = eta > 0 ? reinterpret_cast<T*>(A.win_v) + (int64_t)bh * eta * DV : nullptr;
    if (lam > 0) {
        const char* wsb = A.ws + (int64_t)bh * A.L.per_bh;
        const int* fp = reinterpret_cast<const int*>(wsb + A.L.slot_pos);
        const int* fs = reinterpret_cast<const int*>(wsb + A.L.slot_src);
        T* cK = reinterpret_cast<T*>(A.cache_k) + (int64_t)bh * lam * DK;
        T* cV = reinterpret_cast<T*>(A.cache_v) + (int64_t)bh * lam * DV;
        int32_t* cpos = A.cache_pos + (int64_t)bh * lam;
        const int items = lam * 2 * CPR;                 // (slot, K or V, piece)
        // UN items per thread in flight, without branches around the loads (an item that copies nothing
        // reads row 0 of the call's keys instead), so the values stay in registers
        for (int i0 = tid; i0 < items; i0 += NTH * UN) {
            u32x4 val[UN];
            T* dst[UN];
            bool ok[UN];
#pragma unroll
            for (int u = 0; u < UN; ++u) {
                const int it = i0 + NTH * u;
                const bool in = it < items;
                const int itc = in ? it : 0;
                const int j = itc / (2 * CPR), rem = itc % (2 * CPR), isv = rem / CPR, pc = rem % CPR;
                const int src = fs[j];
                ok[u] = in && src >= 0 && src != n + j;   // not empty, and not a member that kept its slot
                const T* row = kin;
                if (src >= 0 && src < n) row = (isv ? vin : kin) + (int64_t)src * DK;
                else if (src >= n + lam) row = (isv ? ringV : ringK) + (int64_t)(src - n - lam) * DK;
                val[u] = *reinterpret_cast<const u32x4*>((ok[u] ? row : kin) + (ok[u] ? pc * EPV : 0));
                dst[u] = (isv ? cV : cK) + (int64_t)j * DK + pc * EPV;
            }
#pragma unroll
            for (int u = 0; u < UN; ++u)
                if (ok[u]) *reinterpret_cast<u32x4*>(dst[u]) = val[u];
        }
        for (int j = tid; j < lam; j += NTH) cpos[j] = fp[j];
    }
    __syncthreads();                                     // every read of the old ring is done
    if (eta > 0) {
        const int64_t plo = max(t0, t0 + n - eta);
        const int cnt = (int)(t0 + n - plo);
        const int slot0 = (int)(plo % eta);             // ring slot of plo; later ones follow (x < eta)
        const int items = cnt * 2 * CPR;
        for (int i0 = tid; i0 < items; i0 += NTH * UN) {
            u32x4 val[UN];
            T* dst[UN];
            bool ok[UN];
#pragma unroll
            for (int u = 0; u < UN; ++u) {
                const int it = i0 + NTH * u;
                ok[u] = it < items;
                const int itc = ok[u] ? it : 0;
                const int x = itc / (2 * CPR), rem = itc % (2 * CPR), isv = rem / CPR, pc = rem % CPR;
                const int64_t pos = plo + x;
                const int slot = slot0 + x >= eta ? slot0 + x - eta : slot0 + x;
                val[u] = *reinterpret_cast<const u32x4*>((isv ? vin : kin) + (pos - t0) * DK + pc * EPV);
                dst[u] = (isv ? ringV : ringK) + (int64_t)slot * DK + pc * EPV;
            }
#pragma unroll
            for (int u = 0; u < UN; ++u)
                if (ok[u]) *reinterpret_cast<u32x4*>(dst[u]) = val[u];
        }
    }
    if (A.score_rule != kScoreSre) {
        // query-accumulated scores: each final cache member's, and each window token's so far (the
        // window at the end of the call, old ring tokens included when the call is shorter than eta)
        const char* wsb = A.ws + (int64_t)bh * A.L.per_bh;
        const float* scFull = reinterpret_cast<const float*>(wsb + A.L.score_full);
        if (lam > 0) {
            const int* fs = reinterpret_cast<const int*>(wsb + A.L.slot_src);
            for (int j = tid; j < lam; j += NTH) {
                const int src = fs[j];
                A.cache_score[(int64_t)bh * lam + j] = src >= 0 ? scFull[src] : 0.f;
            }
        }
        if (eta > 0) {
            const int64_t plo = max((int64_t)0, t0 + n - eta);
            for (int64_t pos = plo + tid; pos < t0 + n; pos += NTH) {
                const int slot = (int)(pos % eta);
                const int src = pos >= t0 ? (int)(pos - t0) : n + lam + slot;
                A.win_score[(int64_t)bh * eta + slot] = scFull[src];
            }
        }
    }
}

template <typename T, int DK>
static hipError_t launch_commit(const PrefillArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((commit_kernel<T, DK>), dim3(a.BH), dim3(kCommitThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

template <typename T, int DK, int PHI>
hipError_t launch_chain_t(const PrefillArgs& a, hipStream_t stream);

// The overlapped schedule walks the chain in at most kMaxSegments chunk ranges; it takes one event per
// range boundary plus one to join the second stream back (kOverlapEvents in all), all the caller's.
constexpr int kMaxSegments = kOverlapEvents - 1;
constexpr int kOverlapMinChunks = 8;

static hipError_t record(hipEvent_t const* ev, int i, hipStream_t stream) {
    if (!ev || !ev[i]) return hipSuccess;
    return hipEventRecord(ev[i], stream);
}

template <typename T, int DK, int PHI>
static hipError_t launch_readout(PrefillArgs a, int c0, int c1, hipStream_t stream, bool last_range = false) {
    a.c_begin = c0;
    a.c_end = c1;
    if (std::is_same<T, bf16>::value && readout_fast_fits(a, 1)) return launch_readout_fast(a, DK, PHI, c0, c1, stream);
    const int64_t blocks = (int64_t)a.BH * (c1 - c0) * a.nqt;
    if (last_range)
        hipLaunchKernelGGL((readout_kernel<T, DK, PHI, 2>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((readout_kernel<T, DK, PHI, 1>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int DK, int PHI>
static hipError_t launch_chain_range(PrefillArgs a, int c0, int c1, hipStream_t stream) {
    a.c_begin = c0;
    a.c_end = c1;
    if (chain_fast_fits(a, (int)sizeof(T), DK)) return launch_chain_fast(a, stream);
    return launch_chain_t<T, DK, PHI>(a, stream);
}

// Chunk ranges for the overlapped schedule.  Only the read-out of the last range is not hidden behind
// the chain, and a read-out workgroup takes about as long however many run beside it, so the last
// range holds as many chunks as one wave of workgroups covers (ncu / per_chunk, at least 2).  Going
// backwards each range doubles: the read-out of a range (on the compute units the chain leaves free)
// then still finishes before the chain finishes the next one, and there are few launches.
static int split_chunks(int nchunks, int per_chunk, int ncu, int* bounds, int max_seg) {
    int sizes[kMaxSegments];
    int k = 0, sum = 0;
    int sz = per_chunk > 0 ? (ncu + per_chunk - 1) / per_chunk : 2;
    sz = sz < 2 ? 2 : sz;
    while (k < max_seg && sum < nchunks) {               // from the last range backwards
        const int take = sz < nchunks - sum ? sz : nchunks - sum;
        sizes[k++] = take;
        sum += take;
        sz *= 2;
    }
    if (sum < nchunks) sizes[k - 1] += nchunks - sum;   // out of ranges: the first one takes the rest
    if (k >= 2 && sizes[k - 1] < sizes[k - 2]) {         // a short remainder joins its neighbour
        sizes[k - 2] += sizes[k - 1];
        --k;
    }
    bounds[0] = 0;
    for (int i = 0; i < k; ++i) bounds[i + 1] = bounds[i] + sizes[k - 1 - i];
    return k;
}

// Ranges when the read-outs beside the chain are cut into launches that fit the free compute units:
// those read-outs run behind the chain, so the first range is short (they start early), the ranges then
// double, and the last range, whose read-out runs on the whole device after the chain, takes
// last_pct percent of the units.
static int split_capped(int units, int last_pct, int* bounds, int max_seg) {
    constexpr int first = 2;
    int last = (units * last_pct + 50) / 100;
    last = last < 1 ? 1 : last;
    if (units < 2 || max_seg < 2) { bounds[0] = 0; bounds[1] = units; return 1; }
    if (last > units - 1) last = units - 1;
    const int rest = units - last;
    int k = 0, sum = 0, sz = first;
    bounds[0] = 0;
    while (sum < rest && k < max_seg - 2) {
        const int take = sz < rest - sum ? sz : rest - sum;
        sum += take;
        bounds[++k] = sum;
        sz *= 2;
    }
    if (sum < rest) bounds[++k] = rest;
    bounds[++k] = units;
    return k;
}

int device_cus() {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
        return v;
    (void)hipGetLastError();
    return 256;
}

template <typename T, int DK, int PHI>
hipError_t launch_prefill_t(const PrefillArgs& a0, hipStream_t stream, hipEvent_t const* ev, const Overlap* ov) {
    PrefillArgs a = a0;
    hipError_t e;
    const Overlap* side = (ev == nullptr && a.nchunks >= kOverlapMinChunks) ? ov : nullptr;
    if (side == nullptr) {
        // one chain launch, then the read-out: used when timing the kernels one by one
        if ((e = record(ev, 0, stream)) != hipSuccess) return e;
        a.c_begin = 0;
        a.c_end = a.nchunks;
        if ((e = launch_phi_t<T, DK, PHI>(a, stream)) != hipSuccess) return e;
        if (a.score_rule != kScoreSre && (e = launch_qscore_t<T, DK>(a, stream)) != hipSuccess) return e;
        if ((e = record(ev, 1, stream)) != hipSuccess) return e;
        if ((e = launch_chain_range<T, DK, PHI>(a, 0, a.nchunks, stream)) != hipSuccess) return e;
        if ((e = record(ev, 2, stream)) != hipSuccess) return e;
        if ((e = launch_readout<T, DK, PHI>(a, 0, a.nchunks, stream)) != hipSuccess) return e;
        if ((e = record(ev, 3, stream)) != hipSuccess) return e;
        if ((e = launch_commit<T, DK>(a, stream)) != hipSuccess) return e;
        return record(ev, 4, stream);
    }
    // Overlapped: the chain walks the chunk ranges on the caller's stream; the read-out of a range
    // runs on the caller's second stream as soon as the chain has finished it, beside the next range's
    // chain.  The second stream forks from and joins back into the call's stream through the caller's
    // events (one per range boundary, one for the join), so the call stays ordered as one unit.
    int bounds[kMaxSegments + 1];
    // The read-out's unit of work: chunks it takes in one workgroup (the bf16 kernel for C = 64 covers
    // two chunks per tile, so ranges are cut between tiles) and workgroups per unit.
    const bool fastro = std::is_same<T, bf16>::value && readout_fast_fits(a, 1);
    const int cpu = fastro ? (a.C == 64 ? 2 : 1) : 1;
    const int nunits = (a.nchunks + cpu - 1) / cpu;
    const int ncu = device_cus();
    // When the chain holds a quarter of the compute units or more, its read-outs take about as long as
    // the chain itself, and a read-out launch whose workgroups wait for free units holds up the dispatch
    // of the chain's next range behind it until its last workgroup is placed.  The read-outs beside the
    // chain are then cut into launches of at most cap units: three rounds of the workgroups the free
    // units hold, so a chain range waits at most about one read-out workgroup's time.
    const int cap = (fastro && 4 * a.BH >= ncu && a.BH < ncu)
                        ? std::max(1, 3 * readout_fast_groups_per_cu() * (ncu - a.BH) / a.BH) : 0;
    const int nseg = cap > 0 ? split_capped(nunits, 40, bounds, kMaxSegments)
                             : split_chunks(nunits, fastro ? a.BH : a.BH * a.nqt, ncu, bounds, kMaxSegments);
    for (int i = 0; i <= nseg; ++i) bounds[i] = bounds[i] * cpu < a.nchunks ? bounds[i] * cpu : a.nchunks;
    if ((e = launch_phi_t<T, DK, PHI>(a, stream)) != hipSuccess) return e;
    if (a.score_rule != kScoreSre && (e = launch_qscore_t<T, DK>(a, stream)) != hipSuccess) return e;
    // The last range's read-out follows the chain on the caller's stream, so it starts without a
    // cross-stream hop; the earlier ranges' read-outs run on the side stream.
    for (int i = 0; i < nseg; ++i) {
        if ((e = launch_chain_range<T, DK, PHI>(a, bounds[i], bounds[i + 1], stream)) != hipSuccess) return e;
        if ((e = hipEventRecord(side->ev[i], stream)) != hipSuccess) return e;
        if (i == nseg - 1) break;
        if ((e = hipStreamWaitEvent(side->stream, side->ev[i], 0)) != hipSuccess) return e;
        const int step = cap > 0 ? cap * cpu : bounds[i + 1] - bounds[i];
        for (int c0 = bounds[i]; c0 < bounds[i + 1]; c0 += step) {
            const int c1 = c0 + step < bounds[i + 1] ? c0 + step : bounds[i + 1];
            if ((e = launch_readout<T, DK, PHI>(a, c0, c1, side->stream, false)) != hipSuccess) return e;
        }
    }
    if ((e = launch_readout<T, DK, PHI>(a, bounds[nseg - 1], bounds[nseg], stream, nseg > 1)) != hipSuccess) return e;
    // The commit overwrites the state's cache and window rows.  A call that starts from an empty
    // state (t = 0: no cache member, no window token) never reads those rows in the read-out, so its
    // commit runs on the side stream as soon as the chain is done, beside the last read-out;
    // otherwise it follows every read-out on the caller's stream.  Either way the caller's stream
    // joins the side stream.
    a.c_begin = 0;
    a.c_end = a.nchunks;
    const bool fresh = a.t0 == 0;
    if (fresh) {
        if ((e = hipStreamWaitEvent(side->stream, side->ev[nseg - 1], 0)) != hipSuccess) return e;
        if ((e = launch_commit<T, DK>(a, side->stream)) != hipSuccess) return e;
    }
    if ((e = hipEventRecord(side->ev[kOverlapEvents - 1], side->stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(stream, side->ev[kOverlapEvents - 1], 0)) != hipSuccess) return e;
    if (!fresh) return launch_commit<T, DK>(a, stream);
    return hipSuccess;
}

hipError_t launch_prefill(const PrefillArgs& a, int dtype, int d, int phi_kind, hipStream_t stream,
                          hipEvent_t const* ev, const Overlap* ov) {
    if (dtype == 0) {
        if (d == 64) return phi_kind ? launch_prefill_t<float, 64, 1>(a, stream, ev, ov) : launch_prefill_t<float, 64, 0>(a, stream, ev, ov);
        return phi_kind ? launch_prefill_t<float, 128, 1>(a, stream, ev, ov) : launch_prefill_t<float, 128, 0>(a, stream, ev, ov);
    }
    if (d == 64) return phi_kind ? launch_prefill_t<bf16, 64, 1>(a, stream, ev, ov) : launch_prefill_t<bf16, 64, 0>(a, stream, ev, ov);
    return phi_kind ? launch_prefill_t<bf16, 128, 1>(a, stream, ev, ov) : launch_prefill_t<bf16, 128, 0>(a, stream, ev, ov);
}

}  // namespace lola
