// Prefill read-out for bf16 storage with chunks of 64 or 128 tokens: one workgroup per (sequence/head,
// 128 consecutive queries); four waves of 32 queries (two 16-query MFMA tiles each).
//
// Eq. (14) of the LoLA notes (2.5) with the chunk schedule the chain kernel recorded:
//   linear part  L(t) = H_c^T phi(q_t) + sum_{i in S_c, tau_i <= t} (phi(q_t).phi(k_i)) v_i   (den: phi(q_t).s_c + ...)
//   exact part   E(t) = sum_{i in window(t) U cache_c, i not linear} exp(q_t.k_i / sqrt(d_k)) v_i
//   y_t = (L + E) / (L_den + E_den), one shared denominator.
// The linear part is formed first and seeds the running softmax state as if it were one more term of
// weight L_den: max m = log L_den, accumulator L / L_den, sum 1.  The key loop then only rescales and
// adds, and the output is accumulator / sum; no second accumulator stays live through the loop.
//
// Keys.  The 128 queries share one stream of 64-key blocks staged in LDS (keys row-major, values
// transposed): the window band [q0 - eta + 1, q0 + 127], then the cache list of the first chunk of the
// tile, then (chunks of 64) the slots whose member changed at the second chunk.  Every key carries, per
// query group (the chunk of waves 0-1 and of waves 2-3), the range of queries that read it exactly:
//   band key p: [p, p + eta - 1]; cache member p: [p + eta, inf) (a member still inside a query's window
//   is read through the window); a slot replaced at the second chunk: nothing for its second group;
//   the replacement: nothing for the first group.
// A wave classifies each block against its 32 queries: no key read (skipped), every key read by every
// query (no mask), or mixed (mask from the ranges: one subtraction and one unsigned comparison).
//
// Softmax in base 2 with the scale folded into one FMA; the running max is raised only when a block's
// max exceeds it by more than 8 (wave-uniform), so most blocks skip the accumulator rescale.  Probabilities
// are at most 2^8 and the result is the same up to rounding.  The exact weights of the denominator are
// summed on the matrix cores (an all-ones operand against each bf16 probability fragment), so numerator
// and denominator use the same rounded weights.
//
// Workgroups are ordered so that each XCD (workgroup id mod 8) takes a contiguous run of tiles of the
// same heads: neighbouring chunks share most window and cache keys in that XCD's L2.
#include "lola_common.hpp"
#include "lola_internal.hpp"
#include "lola_readout_common.hpp"

namespace lola {

namespace {

using namespace rd;

constexpr int kRfQ = 128;          // queries per workgroup
constexpr int kRfKB = 64;          // keys per staged block
constexpr int kRfThreads = 256;

template <int DK, int PHI>
struct RfCfg {
    static constexpr int D = kFeat, DV = DK, JT = DV / 16;
    static constexpr int DW = (PHI == kPhiSoftmaxPM) ? D / 2 : D;
    static constexpr int WT_LD = DK + 8;           // 16-byte aligned rows for whole-fragment reads
    static constexpr int CPK = DK / 8;             // 16-byte chunks per key (and value) row
    static constexpr int RPB = 256 / (2 * DK);     // rows per 256 bytes (the 64 LDS banks): 1 or 2
    static constexpr int SEG = DV / 16;            // 32-byte segments per value row
    static constexpr int PPT = kRfKB * CPK / kRfThreads;   // chunks per thread and block (one row)
};

// LDS: two key-block buffers (keys row-major, values transposed; W^T shares the second one, which the
// key loop first fills after the features are formed), the blocks' query ranges, the replaced slots,
// the fold lists, then the five slot tables of lambda entries each (rounded up to 4), whose size is
// set at launch.
struct RfLds {
    size_t k, vt, wt, tlo, span, dpos, dsrc, fpos, fsrc, snaps, repm, misc, tables;
};
constexpr size_t kRfBufBytes = 2 * 2 * (size_t)kRfKB * 128;   // one buffer: keys + values at d = 128
__host__ __device__ constexpr size_t rf_al(size_t x) { return (x + 15) & ~size_t(15); }

template <int DK, int PHI>
__host__ __device__ constexpr RfLds rf_lds() {
    using Cfg = RfCfg<DK, PHI>;
    static_assert(2 * kRfKB * (DK + Cfg::DV) <= (int)kRfBufBytes, "one key block per buffer");
    RfLds o{};
    size_t p = 0;
    o.k = p;     p = rf_al(p + 2 * kRfKB * DK);          // buffer b: keys at k + b * kRfBufBytes
    o.vt = p;    p = rf_al(p + 2 * kRfKB * Cfg::DV);      //           values at vt + b * kRfBufBytes
    o.wt = kRfBufBytes;                                   // from buffer 1 on (elu at d = 128: past it)
    p = 2 * kRfBufBytes;
    p = p > kRfBufBytes + rf_al(2 * Cfg::DW * Cfg::WT_LD) ? p : kRfBufBytes + rf_al(2 * Cfg::DW * Cfg::WT_LD);
    o.tlo = p;   p = rf_al(p + 4 * 2 * 2 * kRfKB);        // [buffer][group][key]
    o.span = p;  p = rf_al(p + 4 * 2 * 2 * kRfKB);
    o.dpos = p;  p = rf_al(p + 4 * kRfKB);
    o.dsrc = p;  p = rf_al(p + 4 * kRfKB);
    o.fpos = p;  p = rf_al(p + 4 * 2 * kMaxChunk);
    o.fsrc = p;  p = rf_al(p + 4 * 2 * kMaxChunk);
    o.snaps = p; p = rf_al(p + 4 * 2 * kFeat);          // s of both chunks' snapshots
    o.repm = p;  p = rf_al(p + 8 * (kMaxLambda / 64));  // replaced-slot masks, one word per 64 slots
    o.misc = p;  p = rf_al(p + 4 * 16);
    o.tables = p;
    return o;
}

template <int DK, int PHI>
__global__ __launch_bounds__(kRfThreads, 2) void readout_fast_kernel(PrefillArgs A, int tiles_per_bh, int u_begin,
                                                                    int ntiles) {
    using T = bf16;
    using Cfg = RfCfg<DK, PHI>;
    constexpr int D = Cfg::D, DV = Cfg::DV, JT = Cfg::JT, DW = Cfg::DW, WT_LD = Cfg::WT_LD, PPT = Cfg::PPT,
                  KB = kRfKB;
    extern __shared__ __align__(16) char smem[];
    constexpr RfLds lo = rf_lds<DK, PHI>();
    constexpr int BUFE = (int)(kRfBufBytes / sizeof(T));   // buffer stride in elements
    T* sK = reinterpret_cast<T*>(smem + lo.k);              // [2 buffers] [KB][DK], swizzled
    T* sV = reinterpret_cast<T*>(smem + lo.vt);             // [2 buffers] [KB][DV], swizzled
    T* wt = reinterpret_cast<T*>(smem + lo.wt);             // shares buffer 1 until the key loop
    int* sTlo = reinterpret_cast<int*>(smem + lo.tlo);      // [2 buffers][2 groups][KB]
    int* sSpan = reinterpret_cast<int*>(smem + lo.span);    // [2 buffers][2 groups][KB]
    const int lam4 = (A.lam + 3) & ~3;
    int* cPos = reinterpret_cast<int*>(smem + lo.tables);   // cache list of the tile's first chunk
    int* cSrc = cPos + lam4;
    int* g1ok = cSrc + lam4;                                // slot unchanged at the second chunk
    int* cPos1 = g1ok + lam4;                               // the second chunk's slot table
    int* cSrc1 = cPos1 + lam4;
    int* dPos = reinterpret_cast<int*>(smem + lo.dpos);     // slots replaced at the second chunk
    int* dSrc = reinterpret_cast<int*>(smem + lo.dsrc);
    int* fPos = reinterpret_cast<int*>(smem + lo.fpos);     // [2][kMaxChunk] fold lists per group
    int* fSrc = reinterpret_cast<int*>(smem + lo.fsrc);
    int* misc = reinterpret_cast<int*>(smem + lo.misc);
    float* snapsL = reinterpret_cast<float*>(smem + lo.snaps);
    unsigned long long* repm = reinterpret_cast<unsigned long long*>(smem + lo.repm);

    // XCD-aware order: workgroup id mod 8 picks a contiguous eighth of the tiles.
    const int G = gridDim.x;
    const int per = G / 8;                          // G is a multiple of 8 (host pads)
    const int tile = (blockIdx.x % 8) * per + blockIdx.x / 8;
    if (tile >= ntiles) return;
    const int bh = tile / tiles_per_bh;
    const int u = u_begin + tile % tiles_per_bh;
    const int n = A.n, C = A.C, eta = A.eta, lam = A.lam;
    const int64_t t0 = A.t0;
    const int64_t q0 = t0 + (int64_t)kRfQ * u;
    const int64_t tend = t0 + n;                    // first position past the call
    const int cpt = kRfQ / C;                       // chunks per tile: 2 (C = 64) or 1 (C = 128)
    const int ch0 = u * cpt;                        // first chunk of the tile
    const bool two = cpt == 2 && ch0 + 1 < A.nchunks && q0 + 64 < tend;   // a second chunk with queries
    const bool sparse = (A.read_mask & kReadSparse) && lam > 0;

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c = l & 15;
    const int grp = cpt == 2 ? (w >> 1) : 0;        // query group (chunk) of this wave
    const int chw = ch0 + grp;
    const int64_t tw0 = q0 + 32 * w;                // first query of this wave
    const bool wave_active = tw0 < tend;

    const char* wsb = A.ws + (int64_t)bh * A.L.per_bh;
    const char* rec0 = wsb + A.L.chunk0 + (int64_t)ch0 * A.L.per_chunk;
    const char* rec1 = two ? rec0 + A.L.per_chunk : rec0;
    const T* phiStore = reinterpret_cast<const T*>(wsb + A.L.phi_store);
    const T* qin = reinterpret_cast<const T*>(A.q) + (int64_t)bh * n * DK;
    const T* kin = reinterpret_cast<const T*>(A.k) + (int64_t)bh * n * DK;
    const T* vin = reinterpret_cast<const T*>(A.v) + (int64_t)bh * n * DV;
    const T* ringK = eta > 0 ? reinterpret_cast<const T*>(A.win_k) + (int64_t)bh * eta * DK : nullptr;
    const T* ringV = eta > 0 ? reinterpret_cast<const T*>(A.win_v) + (int64_t)bh * eta * DV : nullptr;
    const T* cK = lam > 0 ? reinterpret_cast<const T*>(A.cache_k) + (int64_t)bh * lam * DK : nullptr;
    const T* cV = lam > 0 ? reinterpret_cast<const T*>(A.cache_v) + (int64_t)bh * lam * DV : nullptr;
    T* yout = reinterpret_cast<T*>(A.y) + (int64_t)bh * n * DV;

    // ---- key stream of the tile ----
    const int64_t blo = q0 - eta + 1 > 0 ? q0 - eta + 1 : 0;
    const int64_t bhi = (q0 + kRfQ - 1 < tend - 1) ? q0 + kRfQ - 1 : tend - 1;
    const int nb = (eta > 0 && bhi >= blo) ? (int)(bhi - blo + 1) : 0;
    const int ring0 = eta > 0 ? (int)(blo % eta) : 0;       // ring slot of the first band key
    const int nbb = (nb + KB - 1) / KB;
    const int ncb = sparse ? (lam + KB - 1) / KB : 0;

    // The prologue issues its independent loads together: the query fragments (for the features),
    // both chunks' slot tables and fold lists, W^T, then (after the barrier) the first key block; the
    // replaced-slot pass reads the slot tables from LDS.
    Frag8<T> qf[2][DK / 32];
    auto load_q = [&]() {
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
            // a query past the call's end reads the call's first row instead: its lanes' results are
            // never stored, and every row is finite
            const int64_t tq = tw0 + 16 * qq + c;
            const T* qrow = qin + (tq < tend ? tq - t0 : 0) * DK;
#pragma unroll
            for (int ss = 0; ss < DK / 32; ++ss) qf[qq][ss] = load_frag_contig(qrow, ss, g);
        }
    };
    const bool lin = (A.read_mask & kReadState) && wave_active;
    if (lin) load_q();
    if (sparse) {
        const int* p0 = reinterpret_cast<const int*>(rec0 + A.L.c_cache_pos);
        const int* s0 = reinterpret_cast<const int*>(rec0 + A.L.c_cache_src);
        const int* p1 = reinterpret_cast<const int*>(rec1 + A.L.c_cache_pos);
        const int* s1 = reinterpret_cast<const int*>(rec1 + A.L.c_cache_src);
        for (int j = tid; j < lam; j += kRfThreads) {
            const int a0 = p0[j], b0 = s0[j], a1 = p1[j], b1 = s1[j];
            cPos[j] = a0;
            cSrc[j] = b0;
            cPos1[j] = a1;
            cSrc1[j] = b1;
            g1ok[j] = a0 == a1;
        }
    } else if (tid == 0) {
        misc[0] = 0;
    }
    {
        const int nf0 = *reinterpret_cast<const int*>(rec0 + A.L.c_fold_n);
        const int nf1 = two ? *reinterpret_cast<const int*>(rec1 + A.L.c_fold_n) : 0;
        const int* fp0 = reinterpret_cast<const int*>(rec0 + A.L.c_fold_pos);
        const int* fs0 = reinterpret_cast<const int*>(rec0 + A.L.c_fold_src);
        const int* fp1 = reinterpret_cast<const int*>(rec1 + A.L.c_fold_pos);
        const int* fs1 = reinterpret_cast<const int*>(rec1 + A.L.c_fold_src);
        for (int i = tid; i < nf0; i += kRfThreads) { fPos[i] = fp0[i]; fSrc[i] = fs0[i]; }
        for (int i = tid; i < nf1; i += kRfThreads) { fPos[kMaxChunk + i] = fp1[i]; fSrc[kMaxChunk + i] = fs1[i]; }
        if (tid == 0) { misc[1] = nf0; misc[2] = nf1; }
        // The folded tokens' features, gathered into key buffer 0 (free until block 0 is staged after the
        // linear part): 128 rows, those of the second chunk from row 64 (C = 64), half a row a thread.
        // Their loads overlap the ones above; the fold term then reads its operands from LDS.
        if (A.read_mask & kReadState) {
            for (int i = tid; i < 2 * D; i += kRfThreads) {
                const int64_t soff = i >= D ? (int64_t)(rec1 - rec0) : 0;
                snapsL[i] = reinterpret_cast<const float*>(rec0 + soff + A.L.c_snap_s)[i % D];
            }
        }
        if (A.read_mask & kReadState) {
            static_assert(kRfThreads == 256, "two threads a fold row");
            const int row = tid & 127, half = tid >> 7;
            const int gi = cpt == 2 ? row >> 6 : 0, i = cpt == 2 ? row & 63 : row;
            const int64_t goff = gi ? (int64_t)(rec1 - rec0) : 0;     // an offset, not a pointer select
            const int* fsg = reinterpret_cast<const int*>(rec0 + goff + A.L.c_fold_src);
            const int src = i < (gi ? nf1 : nf0) ? fsg[i] : 0;
            const T* prow = phiStore + (int64_t)src * D + 64 * half;
            typedef unsigned u32x4 __attribute__((ext_vector_type(4)));   // a vector value, kept in registers
            u32x4 fr[8];
#pragma unroll
            for (int x = 0; x < 8; ++x) fr[x] = *reinterpret_cast<const u32x4*>(prow + 8 * x);
#pragma unroll
            for (int x = 0; x < 8; ++x)
                *reinterpret_cast<u32x4*>(sK + row * D + kswz<D>(row, 8 * half + x) * 8) = fr[x];
        }
    }
    // W^T in LDS for the query features
    if (A.read_mask & kReadState) stage_wt<T, DK, DW, kRfThreads>(wt, WT_LD, A.W);
    __syncthreads();
    // slots replaced at the second chunk, first step: one ballot mask per 64 slots, the waves taking
    // the groups in turn (the ranks follow after the next barrier, before block 0 is staged)
    const unsigned long long lt = l ? (~0ull >> (64 - l)) : 0ull;
    const int nrg = (lam + 63) >> 6;
    auto replaced = [&](int j) {
        const int a0 = j < lam ? cPos[j] : -1, a1 = j < lam ? cPos1[j] : -1;
        return j < lam && a1 >= 0 && a1 != a0;
    };
    if (sparse)
        for (int gi = w; gi < nrg; gi += kRfThreads / 64) {
            const unsigned long long m = __ballot(replaced(64 * gi + l));
            if (l == 0) repm[gi] = m;
        }
    const int nblk0 = nbb + ncb;                    // blocks known before the replaced-slot pass
    int nd = 0;                                     // replaced slots (known after the next barrier)

    // key kk of block kb -> position, rows, and the query ranges of both groups
    auto key_of = [&](int kb, int j, int& pos, const T*& rk, const T*& rv, unsigned& tl0, unsigned& sp0,
                      unsigned& tl1, unsigned& sp1) {
        pos = -1; rk = kin; rv = vin;
        tl0 = tl1 = kNoKey; sp0 = sp1 = 0u;
        if (kb < nbb) {
            const int kk = kb * KB + j;
            if (kk < nb) {
                const int64_t p = blo + kk;
                pos = (int)p;
                if (p >= t0) { rk = kin + (p - t0) * DK; rv = vin + (p - t0) * DV; }
                else {
                    int sl = ring0 + kk;
                    sl = sl >= eta ? sl - eta : sl;      // kk < eta here (p < t0 <= q0)
                    rk = ringK + (int64_t)sl * DK;
                    rv = ringV + (int64_t)sl * DV;
                }
                tl0 = tl1 = (unsigned)p;
                sp0 = sp1 = (unsigned)(eta - 1);
            }
            return;
        }
        int p = -1, src = -1, ok0 = 0, ok1 = 0;
        if (kb < nbb + ncb) {
            const int jj = (kb - nbb) * KB + j;
            if (jj < lam) { p = cPos[jj]; src = cSrc[jj]; ok0 = 1; ok1 = g1ok[jj]; }
        } else if (j < nd) {
            p = dPos[j]; src = dSrc[j]; ok0 = 0; ok1 = 1;
        }
        if (p < 0) return;
        pos = p;
        if (src < n) { rk = kin + (int64_t)src * DK; rv = vin + (int64_t)src * DV; }
        else if (src < n + lam) { rk = cK + (int64_t)(src - n) * DK; rv = cV + (int64_t)(src - n) * DV; }
        else { rk = ringK + (int64_t)(src - n - lam) * DK; rv = ringV + (int64_t)(src - n - lam) * DV; }
        const unsigned lo_ = (unsigned)(p + eta);
        if (ok0) { tl0 = lo_; sp0 = kNoKey - lo_; }
        if (ok1) { tl1 = lo_; sp1 = kNoKey - lo_; }
    };

    // A block in flight: thread t stages key t / 4 of the block, chunks (t mod 4) * PPT .. + PPT - 1 of
    // its key row and of its value row, and (t mod 4 == 0) the key's query ranges.
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));   // vector values, kept in registers
    u32x4 bufk[PPT], bufv[PPT];
    unsigned btl0, bsp0, btl1, bsp1;
    const int sj = tid >> 2, sq0 = (tid & 3) * PPT;
    auto prefetch = [&](int kb) {
        int pos;
        const T* rk;
        const T* rv;
        key_of(kb, sj, pos, rk, rv, btl0, bsp0, btl1, bsp1);
        // a key slot without a key (pos < 0) loads the call's first row: finite values that every
        // query masks out (its query range is empty), so no branch around the loads
        (void)pos;
#pragma unroll
        for (int x = 0; x < PPT; ++x) {
            bufk[x] = *reinterpret_cast<const u32x4*>(rk + (sq0 + x) * 8);
            bufv[x] = *reinterpret_cast<const u32x4*>(rv + (sq0 + x) * 8);
        }
    };
    auto stage = [&](int b) {
        T* bk = sK + b * BUFE;
        T* bv = sV + b * BUFE;
#pragma unroll
        for (int x = 0; x < PPT; ++x) {
            *reinterpret_cast<u32x4*>(bk + sj * DK + kswz<DK>(sj, sq0 + x) * 8) = bufk[x];
            *reinterpret_cast<u32x4*>(bv + sj * DV + vswz<DK>(sj, sq0 + x) * 8) = bufv[x];
        }
        if ((tid & 3) == 0) {
            int* tl = sTlo + b * 2 * KB;
            int* sp = sSpan + b * 2 * KB;
            tl[sj] = (int)btl0;
            sp[sj] = (int)bsp0;
            tl[KB + sj] = (int)btl1;
            sp[KB + sj] = (int)bsp1;
        }
    };
    // this wave's view of the staged block, from the keys' query ranges (lane l reads key l): none of
    // its queries reads a key, or every query reads every key, or a mask is needed
    const unsigned ta = (unsigned)tw0;
    const unsigned tb = (unsigned)(tw0 + 31 < tend - 1 ? tw0 + 31 : tend - 1);
    auto classify = [&](int b, bool& none, bool& full) {
        const unsigned tl = (unsigned)sTlo[(2 * b + grp) * KB + l], sp = (unsigned)sSpan[(2 * b + grp) * KB + l];
        const unsigned hi = tl == kNoKey ? 0u : tl + sp;
        const bool read_by_none = tl > tb || hi < ta;      // no query of the wave reads key l
        const bool read_by_all = tl <= ta && hi >= tb;     // every query of the wave reads key l
        none = __ballot(!read_by_none) == 0ull;
        full = !none && __ballot(!read_by_all) == 0ull;
    };
    if (nblk0 > 0) prefetch(0);                    // in flight through the linear part

    // ---- the linear part seeding the softmax state ----
    // The query fragments serve the features, are dropped through the linear part and are loaded
    // again from L2 for the key loop.
    constexpr float kLog2e = 1.4426950408889634f;
    const float sl2 = kLog2e / sqrtf((float)DK);       // score -> base-2 logit
    f4 O[JT][2];
    float m_run[2], l_run[2];
    // The exact terms' weights are summed by the matrix cores: an all-ones A operand against the
    // probability fragments gives every lane the sum over a step's 32 keys for its query (the same
    // bf16-rounded weights the value products use).  l_run keeps the linear seed only.
    f4 lsum[2];
    Frag8<T> ones;
#pragma unroll
    for (int i = 0; i < 8; ++i) ones.v[i] = (T)1.f;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
        m_run[qq] = -INFINITY;
        l_run[qq] = 0.f;
        lsum[qq] = zero4();
#pragma unroll
        for (int J = 0; J < JT; ++J) O[J][qq] = zero4();
    }
    if (lin) {
        const char* recw = grp ? rec1 : rec0;
        const T* snapH = reinterpret_cast<const T*>(recw + A.L.c_snap_h);
        const float* snapS = snapsL + grp * D;           // staged in LDS with the prologue's loads
        const T* foldVT = reinterpret_cast<const T*>(recw + A.L.c_fold_vt);
        const int cpv = A.L.c_pad64;
        const int nf = misc[1 + grp];
        const int* fp = fPos + grp * kMaxChunk;
        const int* fs = fSrc + grp * kMaxChunk;
        const int64_t a = t0 + (int64_t)chw * C;       // the wave's chunk start
        Frag8<T> pf[2][D / 32];
        float lden[2];
        // H_c^T phi(Q)^T from the fragment-order snapshot (each fragment serves both query tiles), in
        // batches of four fragments: the next batch is requested before the current one is used.  The
        // first batch is requested before the features are formed.
        constexpr int HB = 4, NHB = JT * (D / 32) / HB;
        Frag8<T> hb[2][HB];
        auto load_hb = [&](int b, Frag8<T> (&dst)[HB]) {
            const int ss = b / (JT / HB), J0 = (b % (JT / HB)) * HB;
#pragma unroll
            for (int jj = 0; jj < HB; ++jj)
                dst[jj] = *reinterpret_cast<const Frag8<T>*>(snapH + ((int64_t)((J0 + jj) * (D / 32) + ss) * 64 + l) * 8);
        };
        load_hb(0, hb[0]);
        phi_pair<DK, PHI>(wt, WT_LD, qf, snapS, pf, lden);
#pragma unroll
        for (int b = 0; b < NHB; ++b) {
            if (b + 1 < NHB) load_hb(b + 1, hb[(b + 1) & 1]);
            const int ss = b / (JT / HB), J0 = (b % (JT / HB)) * HB;
#pragma unroll
            for (int jj = 0; jj < HB; ++jj) {
                mma32(O[J0 + jj][0], hb[b & 1][jj], pf[0][ss]);
                mma32(O[J0 + jj][1], hb[b & 1][jj], pf[1][ss]);
            }
            __builtin_amdgcn_sched_barrier(0);        // bound the snapshot fragments in flight
        }
        // tokens folded by this chunk become linear at tau = max(exit time, chunk start)
        float lf[2] = {0.f, 0.f};
        for (int fb = 0; fb * 32 < nf; ++fb) {
            // the kernel values phi(q_t).phi(k_i) of 32 folded tokens (two halves of 16) and both query
            // tiles, masked by tau_i <= t, then their values (requested first)
            Frag8<T> vfs[JT];
#pragma unroll
            for (int J = 0; J < JT; ++J) vfs[J] = load_frag(foldVT + (int64_t)(16 * J + c) * cpv, fb, g);
            f4 sp[2][2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int i = 32 * fb + 16 * h2 + c;
                const int row = (cpt == 2 ? 64 * grp : 0) + (i < nf ? i : 0);   // the gathered rows in LDS
                const T* fr = sK + row * D + 4 * (g & 1);
                Frag8<T> af[D / 32];
#pragma unroll
                for (int ss = 0; ss < D / 32; ++ss) {
                    af[ss].v = __builtin_shufflevector(*reinterpret_cast<const bf16x4*>(fr + kswz<D>(row, 4 * ss + (g >> 1)) * 8),
                                                       *reinterpret_cast<const bf16x4*>(fr + kswz<D>(row, 4 * ss + 2 + (g >> 1)) * 8),
                                                       0, 1, 2, 3, 4, 5, 6, 7);
                    if (i >= nf) af[ss] = frag_zero<T>();
                }
#pragma unroll
                for (int qq = 0; qq < 2; ++qq) {
                    sp[h2][qq] = zero4();
#pragma unroll
                    for (int ss = 0; ss < D / 32; ++ss) mma32(sp[h2][qq], af[ss], pf[qq][ss]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            Frag8<T> bw[2];
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
                const int64_t tq = tw0 + 16 * qq + c;
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int ii = 32 * fb + 16 * h2 + 4 * g + r;
                        bool ok = false;
                        if (ii < nf) {
                            const int64_t tau = max((int64_t)fp[ii] + eta, a);
                            ok = tau <= tq;
                        }
                        sp[h2][qq][r] = ok ? sp[h2][qq][r] : 0.f;
                        lf[qq] += sp[h2][qq][r];
                    }
                bw[qq] = frag_from_acc<T>(sp[0][qq], sp[1][qq]);
            }
#pragma unroll
            for (int J = 0; J < JT; ++J) {
                const Frag8<T> vf = vfs[J];
                mma32(O[J][0], vf, bw[0]);
                mma32(O[J][1], vf, bw[1]);
                if (J % 4 == 3) __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
            const float den = sum_groups(lden[qq]) + sum_groups(lf[qq]);
            if (den > 0.f) {
                const float inv = 1.f / den;
                m_run[qq] = __builtin_amdgcn_logf(den);            // log2 of the linear weight
                l_run[qq] = g == 0 ? 1.f : 0.f;                   // counted once in the group sum
#pragma unroll
                for (int J = 0; J < JT; ++J)
#pragma unroll
                    for (int r = 0; r < 4; ++r) O[J][qq][r] *= inv;
            } else {
#pragma unroll
                for (int J = 0; J < JT; ++J) O[J][qq] = zero4();
            }
        }
    }

    // ---- exact part: the key blocks ----
    asm volatile("" ::: "memory");                  // a second load, not the first one kept live
    load_q();
    __syncthreads();                                // every wave is past the fold term: buffer 0 is free
    // replaced slots, second step: each group's entries at its rank among all groups
    if (sparse) {
        for (int gi = w; gi < nrg; gi += kRfThreads / 64) {
            int base = 0;
            for (int g2 = 0; g2 < gi; ++g2) base += __popcll(repm[g2]);
            const unsigned long long m = repm[gi];
            const int j = 64 * gi + l;
            const int k = base + __popcll(m & lt);
            if (((m >> l) & 1ull) && k < KB) { dPos[k] = cPos1[j]; dSrc[k] = cSrc1[j]; }
        }
        if (tid == 0) {
            int tot = 0;
            for (int g2 = 0; g2 < nrg; ++g2) tot += __popcll(repm[g2]);
            misc[0] = tot < KB ? tot : KB;
        }
    }
    if (nblk0 > 0) stage(0);
    __syncthreads();                                // block 0 staged, the replaced slots listed
    nd = misc[0];
    const int ndb = (sparse && two && nd > 0) ? 1 : 0;
    const int nblk = nbb + ncb + ndb;
    // Two buffers: block kb + 1 is staged into the other buffer while block kb is read, so one
    // barrier per block orders both (the buffer staged at kb was last read at kb - 1).
    for (int kb = 0; kb < nblk; ++kb) {
        const int cb = kb & 1;
        const T* bK = sK + cb * BUFE;
        const T* bV = sV + cb * BUFE;
        const int* tloG = sTlo + (2 * cb + grp) * KB;
        const int* spanG = sSpan + (2 * cb + grp) * KB;
        bool none, full;
        classify(cb, none, full);
        if (kb + 1 < nblk) prefetch(kb + 1);
        if (wave_active && !none) {
            // K Q^T by reduction step: the eight accumulators of a step are independent, so the matrix
            // cores do not wait on one accumulator's previous product
            f4 S[KB / 16][2];
#pragma unroll
            for (int kt = 0; kt < KB / 16; ++kt) {
                S[kt][0] = zero4();
                S[kt][1] = zero4();
            }
#pragma unroll
            for (int ss = 0; ss < DK / 32; ++ss) {
                Frag8<T> kf[KB / 16];
#pragma unroll
                for (int kt = 0; kt < KB / 16; ++kt) {
                    // the contiguous reduction order (the query fragments use it too): one 16-byte chunk
                    const int row = 16 * kt + c;
                    kf[kt].v = *reinterpret_cast<const bf16x8*>(bK + row * DK + kswz<DK>(row, 4 * ss + g) * 8);
                }
#pragma unroll
                for (int kt = 0; kt < KB / 16; ++kt) {
                    mma32(S[kt][0], kf[kt], qf[0][ss]);
                    mma32(S[kt][1], kf[kt], qf[1][ss]);
                }
                __builtin_amdgcn_sched_barrier(0);            // bound the key fragments in flight
            }
            if (!full) {
#pragma unroll
                for (int kt = 0; kt < KB / 16; ++kt) {
                    const int4 tv = *reinterpret_cast<const int4*>(tloG + 16 * kt + 4 * g);
                    const int4 sv = *reinterpret_cast<const int4*>(spanG + 16 * kt + 4 * g);
                    const unsigned tlr[4] = {(unsigned)tv.x, (unsigned)tv.y, (unsigned)tv.z, (unsigned)tv.w};
                    const unsigned spr[4] = {(unsigned)sv.x, (unsigned)sv.y, (unsigned)sv.z, (unsigned)sv.w};
#pragma unroll
                    for (int qq = 0; qq < 2; ++qq) {
                        const unsigned tq = (unsigned)(tw0 + 16 * qq + c);
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            S[kt][qq][r] = (tq - tlr[r]) <= spr[r] ? S[kt][qq][r] : -INFINITY;
                    }
                }
            }
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
                float bm = -INFINITY;
#pragma unroll
                for (int kt = 0; kt < KB / 16; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) bm = fmaxf(bm, S[kt][qq][r]);
                bm = max_groups(bm) * sl2;
                // raise the running max only when the block's exceeds it by more than 8 (base 2)
                if (__ballot(bm > m_run[qq] + 8.f)) {
                    const float mn_ = fmaxf(m_run[qq], bm);
                    const float alpha = m_run[qq] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[qq] - mn_);
                    l_run[qq] *= alpha;
                    lsum[qq][0] *= alpha;
#pragma unroll
                    for (int J = 0; J < JT; ++J)
#pragma unroll
                        for (int r = 0; r < 4; ++r) O[J][qq][r] *= alpha;
                    m_run[qq] = mn_;
                }
                const float mref = m_run[qq] == -INFINITY ? 0.f : m_run[qq];
#pragma unroll
                for (int kt = 0; kt < KB / 16; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        S[kt][qq][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kt][qq][r], sl2, -mref));
            }
#pragma unroll
            for (int k2 = 0; k2 < KB / 32; ++k2) {
                const Frag8<T> p0 = frag_from_acc<T>(S[2 * k2][0], S[2 * k2 + 1][0]);
                const Frag8<T> p1 = frag_from_acc<T>(S[2 * k2][1], S[2 * k2 + 1][1]);
                mma32(lsum[0], ones, p0);
                mma32(lsum[1], ones, p1);
#pragma unroll
                for (int J = 0; J < JT; ++J) {
                    // value rows 16J + c, keys 32k2 + 4g .. + 3 and 32k2 + 16 + 4g .. + 3, by transposed reads of
                    // the row-major block: lane (g, c) names key 4g + c / 4, values 16J + 4(c mod 4) .. + 3
                    const int ka = 32 * k2 + 4 * g + (c >> 2), kb2 = ka + 16;
                    const int q = 2 * J + ((c >> 1) & 1), off = 4 * (c & 1);
                    Frag8<T> vf;
                    vf.v = __builtin_shufflevector(lds_read_tr(bV + ka * DV + vswz<DK>(ka, q) * 8 + off),
                                                   lds_read_tr(bV + kb2 * DV + vswz<DK>(kb2, q) * 8 + off),
                                                   0, 1, 2, 3, 4, 5, 6, 7);
                    mma32(O[J][0], vf, p0);
                    mma32(O[J][1], vf, p1);
                    if (J % 4 == 3) __builtin_amdgcn_sched_barrier(0);   // bound the value fragments in flight
                }
            }
        }
        if (kb + 1 < nblk) stage(cb ^ 1);
        __syncthreads();
    }

    // ---- output: accumulator / sum ----
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
        const int64_t tq = tw0 + 16 * qq + c;
        // the linear seed (on lane group 0, hence the group sum) and the exact weights (every lane)
        const float tot = sum_groups(l_run[qq]) + lsum[qq][0];
        if (wave_active && tq < tend) {
            const float inv = 1.f / tot;
            T* yrow = yout + (tq - t0) * DV;
#pragma unroll
            for (int J = 0; J < JT; ++J) {
                bf16x4 v4;
                v4[0] = (bf16)(O[J][qq][0] * inv);
                v4[1] = (bf16)(O[J][qq][1] * inv);
                v4[2] = (bf16)(O[J][qq][2] * inv);
                v4[3] = (bf16)(O[J][qq][3] * inv);
                *reinterpret_cast<bf16x4*>(yrow + 16 * J + 4 * g) = v4;
            }
        }
    }
}

}  // namespace

int readout_fast_groups_per_cu() { return 2; }

bool readout_fast_fits(const PrefillArgs& a, int dtype) {
    return dtype == 1 && (a.C == 64 || a.C == 128);
}

template <int DK, int PHI>
hipError_t launch_readout_fast_t(const PrefillArgs& a, int c0, int c1, hipStream_t stream) {
    const size_t lds = rf_lds<DK, PHI>().tables + (size_t)5 * 4 * ((a.lam + 3) & ~3);
    const int cpt = kRfQ / a.C;
    const int u0 = c0 / cpt;
    const int u1 = (c1 + cpt - 1) / cpt;
    if (u1 <= u0) return hipSuccess;
    const int tiles_per_bh = u1 - u0;
    const int64_t ntiles = (int64_t)a.BH * tiles_per_bh;
    const int64_t grid = (ntiles + 7) / 8 * 8;
    auto kern = readout_fast_kernel<DK, PHI>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kRfThreads), lds, stream, a, tiles_per_bh, u0, (int)ntiles);
    return hipGetLastError();
}

hipError_t launch_readout_fast(const PrefillArgs& a, int d, int phi_kind, int c0, int c1, hipStream_t stream) {
    if (d == 64) return phi_kind ? launch_readout_fast_t<64, 1>(a, c0, c1, stream) : launch_readout_fast_t<64, 0>(a, c0, c1, stream);
    return phi_kind ? launch_readout_fast_t<128, 1>(a, c0, c1, stream) : launch_readout_fast_t<128, 0>(a, c0, c1, stream);
}

}  // namespace lola
