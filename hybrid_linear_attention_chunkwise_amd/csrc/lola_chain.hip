// Prefill allocation chain: one workgroup per (sequence, head) walks the chunks in order.
//
// Per chunk (LoLA notes, 2.6 Eq. (15) with 2.3 Eq. (10) and 2.4 Eqs. (11)-(13)):
//   1. snapshot (H, s) at the chunk start for the read-out kernel;
//   2. candidate table: cache slots plus the tokens that leave the window during the chunk (their
//      features were computed beforehand by the parallel feature kernel);
//   3. if cache + leaving tokens exceed lambda: SRE of every candidate against the chunk-start state,
//      then keep the lambda largest (ties: older position);
//   4. free the slots of folded cache members, give them to the leaving tokens that stay;
//   5. record the chunk's cache list and fold list for the read-out kernel;
//   6. fold: H += Phi_S^T V_S, s += sum Phi_S.
//
// H lives in registers for the whole call as MFMA accumulators: one wave per 16 value columns of H
// (D x d_v, feature rows, value columns), all feature rows.  The SRE numerators are computed
// transposed, H^T Phi_E^T, with those accumulators used directly as the MFMA A operand (see
// lola_common.hpp), so each candidate is one accumulator column and its squared error over the
// wave's value rows needs one cross-lane sum.  The wave partials are summed in a fixed order, so
// results are deterministic.  Selection keeps the lambda largest keys with a 256-bin histogram of SRE
// and an exact rank only inside the boundary bin; prefix counts use wave ballots, not LDS scans.
//
// Every token's features are computed once and stored by source index (the same index that locates
// its K/V), so a token that enters the cache is never copied: a slot is just (position, source).
// Candidate rows reach LDS in double-buffered 32 KB batches of 16-byte loads; the first batch of the
// next chunk is fetched while the current chunk folds.
#include "lola_common.hpp"
#include "lola_internal.hpp"

namespace lola {

namespace {

template <typename T, int DK, int PHI>
struct ChainCfg {
    static constexpr int D = kFeat;
    static constexpr int DV = DK;
    static constexpr int NW = DV / 16;                       // waves: one per 16 value columns
    static constexpr int NT = 64 * NW;                       // threads
    static constexpr int IT = D / 16;                        // accumulator tiles along D
    static constexpr int EPV = 16 / (int)sizeof(T);          // elements per 16-byte piece
    static constexpr int ROWB = (D + DV) * (int)sizeof(T);   // bytes of one candidate row (phi | v)
    static constexpr int NB = ROWB <= 512 ? 64 : 32;         // candidate rows per batch
    static constexpr int TPB = NB / 16;                      // tiles per batch
    static constexpr int CPR = ROWB / 16;                    // 16-byte pieces per row
    static constexpr int CPHI = D / EPV;                     // pieces holding phi
    static constexpr int LPT = NB * CPR / NT;                // pieces per thread per batch
    static constexpr int PHI_LD = D + EPV;                   // LDS row strides (keep 16-byte alignment)
    static constexpr int V_LD = DV + EPV;
    static constexpr int BUF = NB * (PHI_LD + V_LD);         // elements per batch buffer
    static constexpr int FB = sizeof(T) == 2 ? 64 : 32;      // tokens per fold batch
    static constexpr int ST_LD = FB + EPV;                   // 16-byte aligned rows
    static constexpr int TPW = 4 / (int)sizeof(T);           // tokens packed per 32-bit LDS word
    static constexpr int FIPT = FB / TPW * CPR / NT;         // fold staging items per thread
    static constexpr int FLPT = FIPT * TPW;                  // pieces per thread per fold batch
    static constexpr int NBIN = 256;                         // selection histogram
    static_assert(NB * CPR % NT == 0 && (FB / (4 / (int)sizeof(T))) * CPR % NT == 0, "batches must split evenly");
    static_assert((D + DV) * ST_LD <= 2 * BUF, "fold staging must fit in the batch buffers");
};

// Rows of the per-candidate arrays: lam + C rounded up to 64 (a whole number of batches).
__host__ __device__ inline int cand_rows(int lam, int C) { return ((lam + C + 63) / 64) * 64; }

struct ChainLds {
    size_t buf, s, slot_pos, slot_src, c_src, c_pos, key, aux, flag, a1, a2, a3, free_list, fold_row,
        part, den, hist, tmp, total;
};

__host__ __device__ inline size_t al16(size_t x) { return (x + 15) & ~size_t(15); }

template <typename T, int DK, int PHI>
__host__ __device__ inline ChainLds chain_lds(int lam, int C) {
    using Cfg = ChainCfg<T, DK, PHI>;
    const int nr = cand_rows(lam, C);
    ChainLds o;
    size_t p = 0;
    o.buf = p;       p = al16(p + sizeof(T) * 2 * Cfg::BUF);
    o.s = p;         p = al16(p + sizeof(float) * Cfg::D);
    o.slot_pos = p;  p = al16(p + sizeof(int) * (lam + 1));
    o.slot_src = p;  p = al16(p + sizeof(int) * (lam + 1));
    o.c_src = p;     p = al16(p + sizeof(int) * nr);
    o.c_pos = p;     p = al16(p + sizeof(int) * nr);
    o.key = p;       p = al16(p + sizeof(unsigned long long) * nr);
    o.aux = p;       p = al16(p + sizeof(int) * nr);
    o.flag = p;      p = al16(p + sizeof(int) * nr);
    o.a1 = p;        p = al16(p + sizeof(int) * nr);
    o.a2 = p;        p = al16(p + sizeof(int) * (lam + 1));
    o.a3 = p;        p = al16(p + sizeof(int) * (C + 1));
    o.free_list = p; p = al16(p + sizeof(int) * (lam + 1));
    o.fold_row = p;  p = al16(p + sizeof(int) * (C + 1));
    o.part = p;      p = al16(p + sizeof(float) * Cfg::NW * nr);
    o.den = p;       p = al16(p + sizeof(float) * nr);
    o.hist = p;      p = al16(p + sizeof(int) * (Cfg::NBIN + 4));
    o.tmp = p;       p = al16(p + sizeof(int) * 32);
    o.total = p;
    return o;
}

// Key ordering the cache: larger = kept first.  SRE >= 0, so its bit pattern orders like the value;
// on equal SRE the older (smaller) position ranks higher.  0 marks an empty row.
__device__ __forceinline__ unsigned long long keep_key(float sre, int pos) {
    return ((unsigned long long)__float_as_uint(sre) << 32) | (unsigned long long)(0xFFFFFFFFu - (unsigned)pos);
}

__device__ __forceinline__ unsigned wave_min_u32(unsigned x) {
    for (int o = 32; o > 0; o >>= 1) x = min(x, (unsigned)__shfl_xor((int)x, o));
    return x;
}
__device__ __forceinline__ unsigned wave_max_u32(unsigned x) {
    for (int o = 32; o > 0; o >>= 1) x = max(x, (unsigned)__shfl_xor((int)x, o));
    return x;
}

// Where a token's V and features live during the call (see the source index in lola_internal.hpp).
template <typename T, int DK>
struct Sources {
    const T* vin;
    const T* cV;
    const T* ringV;
    const T* phi;
    int n, lam;
    __device__ __forceinline__ const T* v_row(int src) const {
        if (src < n) return vin + (int64_t)src * DK;
        if (src < n + lam) return cV + (int64_t)(src - n) * DK;
        return ringV + (int64_t)(src - n - lam) * DK;
    }
    __device__ __forceinline__ const T* phi_row(int src) const { return phi + (int64_t)src * kFeat; }
};

template <typename T, int DK, int PHI>
__global__ __launch_bounds__(4 * DK) void chain_kernel(PrefillArgs A) {
    using Cfg = ChainCfg<T, DK, PHI>;
    constexpr int D = Cfg::D, DV = Cfg::DV, NW = Cfg::NW, NT = Cfg::NT, IT = Cfg::IT, EPV = Cfg::EPV,
                  NB = Cfg::NB, TPB = Cfg::TPB, CPR = Cfg::CPR, CPHI = Cfg::CPHI, LPT = Cfg::LPT,
                  PHI_LD = Cfg::PHI_LD, V_LD = Cfg::V_LD, BUF = Cfg::BUF, FB = Cfg::FB, ST_LD = Cfg::ST_LD,
                  FLPT = Cfg::FLPT, NBIN = Cfg::NBIN, TPW = Cfg::TPW, FIPT = Cfg::FIPT;
    extern __shared__ __align__(16) char smem[];
    const int lam = A.lam, eta = A.eta, n = A.n, C = A.C;
    const ChainLds lo = chain_lds<T, DK, PHI>(lam, C);
    T* bufs = reinterpret_cast<T*>(smem + lo.buf);
    float* sS = reinterpret_cast<float*>(smem + lo.s);
    int* slotPos = reinterpret_cast<int*>(smem + lo.slot_pos);
    int* slotSrc = reinterpret_cast<int*>(smem + lo.slot_src);
    int* cSrc = reinterpret_cast<int*>(smem + lo.c_src);
    int* cPos = reinterpret_cast<int*>(smem + lo.c_pos);
    unsigned long long* key = reinterpret_cast<unsigned long long*>(smem + lo.key);
    int* aux = reinterpret_cast<int*>(smem + lo.aux);
    int* flag = reinterpret_cast<int*>(smem + lo.flag);
    int* a1 = reinterpret_cast<int*>(smem + lo.a1);
    int* a2 = reinterpret_cast<int*>(smem + lo.a2);
    int* a3 = reinterpret_cast<int*>(smem + lo.a3);
    int* freeList = reinterpret_cast<int*>(smem + lo.free_list);
    int* foldRow = reinterpret_cast<int*>(smem + lo.fold_row);
    float* part = reinterpret_cast<float*>(smem + lo.part);
    float* sDen = reinterpret_cast<float*>(smem + lo.den);
    int* hist = reinterpret_cast<int*>(smem + lo.hist);
    int* tmp = reinterpret_cast<int*>(smem + lo.tmp);

    const int bh = blockIdx.x;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c = l & 15;
    const int64_t t0 = A.t0;
    const int nrp = cand_rows(lam, C);

    char* wsb = A.ws + (int64_t)bh * A.L.per_bh;
    Sources<T, DK> src;
    src.vin = reinterpret_cast<const T*>(A.v) + (int64_t)bh * n * DV;
    src.cV = lam > 0 ? reinterpret_cast<const T*>(A.cache_v) + (int64_t)bh * lam * DV : nullptr;
    src.ringV = eta > 0 ? reinterpret_cast<const T*>(A.win_v) + (int64_t)bh * eta * DV : nullptr;
    src.phi = reinterpret_cast<const T*>(wsb + A.L.phi_store);
    src.n = n;
    src.lam = lam;
    const int32_t* cPosState = lam > 0 ? A.cache_pos + (int64_t)bh * lam : nullptr;
    int32_t* foldAt = A.fold_at ? A.fold_at + (int64_t)bh * n : nullptr;

    auto chunk_x = [&](int ch, int64_t& xlo) {           // leaving tokens of chunk ch: [xlo, xlo + nX)
        const int64_t a = t0 + (int64_t)ch * C;
        const int64_t b = min(a + (int64_t)C, t0 + (int64_t)n);
        xlo = a - eta > 0 ? a - eta : 0;
        return b - eta > xlo ? (int)(b - eta - xlo) : 0;
    };
    // candidate table of chunk ch: cache slots (rows 0..lam-1) then leaving tokens (rows lam..)
    auto build_table = [&](int ch) {
        int64_t xlo;
        const int nX = chunk_x(ch, xlo);
        for (int r = tid; r < nrp; r += NT) {
            int s_ = -1, p_ = -1, f = 0;
            if (r < lam) { s_ = slotSrc[r]; p_ = slotPos[r]; f = p_ >= 0; }
            else if (r < lam + nX) {
                const int64_t pos = xlo + (r - lam);
                p_ = (int)pos;
                s_ = pos >= t0 ? (int)(pos - t0) : n + lam + (int)(pos % eta);
                f = 1;
            }
            cSrc[r] = s_;
            cPos[r] = p_;
            flag[r] = f;
        }
    };
    uint4 stage[LPT];
    auto load_batch = [&](int bt, int NR) {
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
            const int q = tid + NT * u;
            const int row = bt * NB + q / CPR, pc = q % CPR;
            uint4 val = make_uint4(0, 0, 0, 0);
            if (row < NR && flag[row]) {
                const int s_ = cSrc[row];
                const T* p_ = pc < CPHI ? src.phi_row(s_) + pc * EPV : src.v_row(s_) + (pc - CPHI) * EPV;
                val = *reinterpret_cast<const uint4*>(p_);
            }
            stage[u] = val;
        }
    };
    auto store_batch = [&](int bi) {
        T* bphi = bufs + bi * BUF;
        T* bv = bphi + NB * PHI_LD;
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
            const int q = tid + NT * u;
            const int r = q / CPR, pc = q % CPR;
            T* dst = pc < CPHI ? bphi + r * PHI_LD + pc * EPV : bv + r * V_LD + (pc - CPHI) * EPV;
            *reinterpret_cast<uint4*>(dst) = stage[u];
        }
    };

    // ---------------- set-up ----------------
    for (int d = tid; d < D; d += NT) sS[d] = A.s[(int64_t)bh * D + d];
    for (int j = tid; j < lam; j += NT) {
        const int p = cPosState[j];
        slotPos[j] = p;
        slotSrc[j] = p >= 0 ? n + j : -1;
    }
    if (foldAt)
        for (int i = tid; i < n; i += NT) foldAt[i] = -1;
    f4 acc[IT];
    {
        const float* Hb = A.H + (int64_t)bh * DV * D;
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const float4 h = *reinterpret_cast<const float4*>(Hb + (16 * w + c) * D + 16 * i + 4 * g);
            acc[i] = f4{h.x, h.y, h.z, h.w};
        }
    }
    __syncthreads();
    int nG = ballot_prefix(lam, NW, [&](int j) { return slotPos[j] >= 0; }, a2);
    build_table(0);
    __syncthreads();
    bool prefetched = false;
    {
        int64_t xlo0;
        const int nX0 = chunk_x(0, xlo0);
        if (lam > 0 && nG + nX0 > lam) { load_batch(0, lam + nX0); prefetched = true; }
    }

    // ---------------- chunk loop ----------------
    for (int ch = 0; ch < A.nchunks; ++ch) {
        int64_t xlo;
        const int nX = chunk_x(ch, xlo);
        const int NR = lam + nX;
        char* rec = wsb + A.L.chunk0 + (int64_t)ch * A.L.per_chunk;

        // (1) snapshot of the chunk-start state, in the fragment order the read-out kernel loads
        {
            T* snapH = reinterpret_cast<T*>(rec + A.L.c_snap_h);
#pragma unroll
            for (int ss = 0; ss < D / 32; ++ss) {
                const Frag8<T> f = frag_from_acc<T>(acc[2 * ss], acc[2 * ss + 1]);
                *reinterpret_cast<Frag8<T>*>(snapH + ((int64_t)(w * (D / 32) + ss) * 64 + l) * 8) = f;
            }
            float* snapS = reinterpret_cast<float*>(rec + A.L.c_snap_s);
            for (int d = tid; d < D; d += NT) snapS[d] = sS[d];
        }

        // (3) decide which candidates are folded
        const bool scoring = lam > 0 && nG + nX > lam;
        if (scoring) {
            float sv[D / 32][8];
#pragma unroll
            for (int ss = 0; ss < D / 32; ++ss)
#pragma unroll
                for (int e = 0; e < 8; ++e) sv[ss][e] = sS[32 * ss + 16 * (e >> 2) + 4 * g + (e & 3)];
            Frag8<T> hb[D / 32];
#pragma unroll
            for (int ss = 0; ss < D / 32; ++ss) hb[ss] = frag_from_acc<T>(acc[2 * ss], acc[2 * ss + 1]);

            const int nbatch = (NR + NB - 1) / NB;
            if (!prefetched) load_batch(0, NR);
            store_batch(0);
            __syncthreads();
            for (int bt = 0; bt < nbatch; ++bt) {
                if (bt + 1 < nbatch) load_batch(bt + 1, NR);
                const T* bphi = bufs + (bt & 1) * BUF;
                const T* bv = bphi + NB * PHI_LD;
                // pass 1: numerators^T (rows = this wave's value columns, columns = 16 candidates);
                // the denominator phi.s of tile t is computed by wave t % NW only
                f4 num[TPB];
#pragma unroll
                for (int tile = 0; tile < TPB; ++tile) {
                    num[tile] = zero4();
                    const bool mine = (tile % NW) == w;
                    float den = 0.f;
#pragma unroll
                    for (int ss = 0; ss < D / 32; ++ss) {
                        const Frag8<T> bf = load_frag(bphi + (tile * 16 + c) * PHI_LD, ss, g);
                        mma32(num[tile], hb[ss], bf);
                        if (mine)
#pragma unroll
                            for (int e = 0; e < 8; ++e) den += frag_get(bf, e) * sv[ss][e];
                    }
                    if (mine) {
                        den = sum_groups(den);
                        if (g == 0) sDen[bt * NB + tile * 16 + c] = den;
                    }
                }
                __syncthreads();
                // pass 2: squared error over the wave's value rows
#pragma unroll
                for (int tile = 0; tile < TPB; ++tile) {
                    const int rr = bt * NB + tile * 16 + c;
                    const float den = sDen[rr];
                    const float inv = den != 0.f ? 1.f / den : 0.f;     // empty state: recall 0
                    const T* vr = bv + (tile * 16 + c) * V_LD + 16 * w + 4 * g;
                    float sq = 0.f;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float x = num[tile][r] * inv - to_f(vr[r]);
                        sq += x * x;
                    }
                    sq = sum_groups(sq);
                    if (g == 0 && rr < NR) part[w * nrp + rr] = sq;
                }
                if (bt + 1 < nbatch) store_batch((bt + 1) & 1);
                __syncthreads();
            }
            // keys, and the SRE range for the histogram
            {
                unsigned mn = 0x7F800000u, mx = 0u;
                for (int r = tid; r < NR; r += NT) {
                    unsigned long long k = 0ull;
                    if (flag[r]) {
                        float s2 = 0.f;
#pragma unroll
                        for (int ww = 0; ww < NW; ++ww) s2 += part[ww * nrp + r];
                        const float sre = sqrtf(s2);
                        k = keep_key(sre, cPos[r]);
                        mn = min(mn, __float_as_uint(sre));
                        mx = max(mx, __float_as_uint(sre));
                    }
                    key[r] = k;
                }
                mn = wave_min_u32(mn);
                mx = wave_max_u32(mx);
                if (l == 0) { tmp[8 + w] = (int)mn; tmp[16 + w] = (int)mx; }
                for (int i = tid; i < NBIN; i += NT) hist[i] = 0;
                if (tid == 0) tmp[4] = 0;
            }
            __syncthreads();
            unsigned umn = 0x7F800000u, umx = 0u;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) { umn = min(umn, (unsigned)tmp[8 + ww]); umx = max(umx, (unsigned)tmp[16 + ww]); }
            const float smin = __uint_as_float(umn), smax = __uint_as_float(umx);
            const float bscale = smax > smin ? (float)NBIN / (smax - smin) : 0.f;
            auto bin_of = [&](unsigned long long k) -> int {
                const float x = __uint_as_float((unsigned)(k >> 32));
                return min(NBIN - 1, (int)((x - smin) * bscale));   // monotone in the key
            };
            for (int r = tid; r < NR; r += NT)
                if (flag[r]) atomicAdd(&hist[bin_of(key[r])], 1);
            __syncthreads();
            const int nF = nG + nX - lam;                     // how many to fold
            {   // boundary bin: cumulative count before it < nF <= cumulative through it
                int v4[4], s4 = 0;
#pragma unroll
                for (int u = 0; u < 4; ++u) { v4[u] = hist[4 * l + u]; s4 += v4[u]; }
                int x = s4;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) { const int y = __shfl_up(x, o); if (l >= o) x += y; }
                int run = x - s4, bstar = -1, need = 0;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (run < nF && nF <= run + v4[u]) { bstar = 4 * l + u; need = nF - run; }
                    run += v4[u];
                }
                // every wave finds the same (bin, need); spread it from the owning lane
                const unsigned long long own = __ballot(bstar >= 0);
                const int srcl = __ffsll((long long)own) - 1;
                bstar = __shfl(bstar, srcl);
                need = __shfl(need, srcl);
                int* blist = aux;                                 // members of the boundary bin
                for (int r = tid; r < NR; r += NT) {
                    if (!flag[r]) continue;
                    const int br = bin_of(key[r]);
                    if (br < bstar) flag[r] = 2;
                    else if (br > bstar) flag[r] = 1;
                    else blist[atomicAdd(&tmp[4], 1)] = r;
                }
                __syncthreads();
                const int nbm = tmp[4];
                for (int i = tid; i < nbm; i += NT) {         // exact rank inside the boundary bin
                    const int r = blist[i];
                    const unsigned long long kr = key[r];
                    int below = 0;
                    for (int j = 0; j < nbm; ++j) below += key[blist[j]] < kr;
                    flag[r] = below < need ? 2 : 1;
                }
            }
            __syncthreads();
        } else if (lam == 0) {
            for (int r = tid; r < NR; r += NT) flag[r] = 2;
            __syncthreads();
        }

        // (4) fold order first, so the fold's loads overlap the rest of the bookkeeping
        const int nS = ballot_prefix(NR, NW, [&](int r) { return flag[r] == 2; }, a1);
        __syncthreads();
        for (int r = tid; r < NR; r += NT)
            if (flag[r] == 2) foldRow[a1[r]] = r;
        __syncthreads();
        uint4 stg[FLPT];
        // fold staging item: TPW consecutive tokens (m0 .. m0+TPW-1) x one 16-byte piece pc, so that
        // the transposed LDS writes below are whole 32-bit words at consecutive addresses
        auto load_fold = [&](int fb) {
#pragma unroll
            for (int u = 0; u < FIPT; ++u) {
                const int q = tid + NT * u;
                const int m0 = (q % (FB / TPW)) * TPW, pc = q / (FB / TPW);
#pragma unroll
                for (int z = 0; z < TPW; ++z) {
                    const int k = fb * FB + m0 + z;
                    uint4 val = make_uint4(0, 0, 0, 0);
                    if (k < nS) {
                        const int s_ = cSrc[foldRow[k]];
                        const T* p_ = pc < CPHI ? src.phi_row(s_) + pc * EPV : src.v_row(s_) + (pc - CPHI) * EPV;
                        val = *reinterpret_cast<const uint4*>(p_);
                    }
                    stg[u * TPW + z] = val;
                }
            }
        };
        if (nS > 0) load_fold(0);
        ballot_prefix(lam, NW, [&](int j) { return slotPos[j] < 0 || flag[j] == 2; }, a2);
        ballot_prefix(nX, NW, [&](int x) { return flag[lam + x] == 1; }, a3);
        __syncthreads();
        for (int j = tid; j < lam; j += NT)
            if ((slotPos[j] < 0) || flag[j] == 2) freeList[a2[j]] = j;
        {
            int* recFoldPos = reinterpret_cast<int*>(rec + A.L.c_fold_pos);
            int* recFoldSrc = reinterpret_cast<int*>(rec + A.L.c_fold_src);
            for (int k = tid; k < nS; k += NT) {
                const int r = foldRow[k];
                const int pos = cPos[r];
                recFoldPos[k] = pos;
                recFoldSrc[k] = cSrc[r];
                if (foldAt && pos >= t0) foldAt[pos - t0] = ch;
            }
            if (tid == 0) *reinterpret_cast<int*>(rec + A.L.c_fold_n) = nS;
        }
        __syncthreads();
        for (int j = tid; j < lam; j += NT)
            if (flag[j] == 2) { slotPos[j] = -1; slotSrc[j] = -1; }
        __syncthreads();
        for (int x = tid; x < nX; x += NT) {
            if (flag[lam + x] != 1) continue;
            const int j = freeList[a3[x]];
            slotPos[j] = cPos[lam + x];
            slotSrc[j] = cSrc[lam + x];
        }
        __syncthreads();
        {
            int* rp = reinterpret_cast<int*>(rec + A.L.c_cache_pos);
            int* rs = reinterpret_cast<int*>(rec + A.L.c_cache_src);
            for (int j = tid; j < lam; j += NT) { rp[j] = slotPos[j]; rs[j] = slotSrc[j]; }
        }
        nG = scoring ? lam : (lam == 0 ? 0 : nG + nX);
        const bool more = ch + 1 < A.nchunks;

        // (6) fold in batches of FB tokens: H += Phi_S^T V_S (MFMA), s += column sums.  Once the last
        // batch is staged, the next chunk's candidate table is built so its first batch can be
        // fetched while this fold runs.
        {
            T* recVT = reinterpret_cast<T*>(rec + A.L.c_fold_vt);
            const int cpv = A.L.c_pad64;
            T* stPhi = bufs;                      // [D][ST_LD]   (reuses the batch buffers)
            T* stV = bufs + D * ST_LD;            // [DV][ST_LD]
            for (int fb = 0; fb * FB < nS; ++fb) {
                if (fb > 0) load_fold(fb);
#pragma unroll
                for (int u = 0; u < FIPT; ++u) {
                    const int q = tid + NT * u;
                    const int m0 = (q % (FB / TPW)) * TPW, pc = q / (FB / TPW);
                    T* dst0 = pc < CPHI ? stPhi + (pc * EPV) * ST_LD + m0 : stV + ((pc - CPHI) * EPV) * ST_LD + m0;
#pragma unroll
                    for (int x = 0; x < EPV; ++x) {
                        T word[TPW];
#pragma unroll
                        for (int z = 0; z < TPW; ++z) word[z] = reinterpret_cast<const T*>(&stg[u * TPW + z])[x];
                        *reinterpret_cast<uint32_t*>(dst0 + x * ST_LD) = *reinterpret_cast<const uint32_t*>(word);
                    }
                }
                __syncthreads();
                if (more && (fb + 1) * FB >= nS) build_table(ch + 1);
#pragma unroll
                for (int kk = 0; kk < FB / 32; ++kk)
#pragma unroll
                    for (int i = 0; i < IT; ++i) {
                        const Frag8<T> af = load_frag(stPhi + (16 * i + c) * ST_LD, kk, g);
                        const Frag8<T> bf = load_frag(stV + (16 * w + c) * ST_LD, kk, g);
                        mma32(acc[i], af, bf);
                    }
                {   // s: NT / D threads per feature row
                    constexpr int TPR = NT / D;
                    const int d = tid / TPR, pr = tid % TPR;
                    float sum = 0.f;
                    const T* row = stPhi + d * ST_LD + pr * (FB / TPR);
#pragma unroll
                    for (int m = 0; m < FB / TPR; ++m) sum += to_f(row[m]);
#pragma unroll
                    for (int o = 1; o < TPR; o <<= 1) sum += __shfl_xor(sum, o);
                    if (pr == 0) sS[d] += sum;
                }
                // values, transposed, for the read-out kernel (16-byte row pieces)
                for (int q = tid; q < DV * (FB / EPV); q += NT) {
                    const int e = q / (FB / EPV), p = q % (FB / EPV);
                    *reinterpret_cast<uint4*>(recVT + (int64_t)e * cpv + fb * FB + p * EPV) =
                        *reinterpret_cast<const uint4*>(stV + e * ST_LD + p * EPV);
                }
                __syncthreads();
            }
            if (more && nS == 0) {
                build_table(ch + 1);
                __syncthreads();
            }
        }
        prefetched = false;
        if (more) {
            int64_t xn;
            const int nXn = chunk_x(ch + 1, xn);
            if (lam > 0 && nG + nXn > lam) { load_batch(0, lam + nXn); prefetched = true; }
        }
    }

    // ---------------- final state ----------------
    {
        float* Hb = A.H + (int64_t)bh * DV * D;
#pragma unroll
        for (int i = 0; i < IT; ++i)
            *reinterpret_cast<float4*>(Hb + (16 * w + c) * D + 16 * i + 4 * g) =
                make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
        for (int d = tid; d < D; d += NT) A.s[(int64_t)bh * D + d] = sS[d];
        int* fp = reinterpret_cast<int*>(wsb + A.L.slot_pos);
        int* fs = reinterpret_cast<int*>(wsb + A.L.slot_src);
        for (int j = tid; j < lam; j += NT) { fp[j] = slotPos[j]; fs[j] = slotSrc[j]; }
    }
}

}  // namespace

template <typename T, int DK, int PHI>
hipError_t launch_chain_t(const PrefillArgs& a, hipStream_t stream) {
    const size_t lds = chain_lds<T, DK, PHI>(a.lam, a.C).total;
    auto kern = chain_kernel<T, DK, PHI>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(a.BH), dim3(ChainCfg<T, DK, PHI>::NT), lds, stream, a);
    return hipGetLastError();
}

size_t chain_lds_bytes(int d, int phi_kind, int esz, int lam, int C) {
    if (esz == 4) {
        if (d == 64) return phi_kind ? chain_lds<float, 64, 1>(lam, C).total : chain_lds<float, 64, 0>(lam, C).total;
        return phi_kind ? chain_lds<float, 128, 1>(lam, C).total : chain_lds<float, 128, 0>(lam, C).total;
    }
    if (d == 64) return phi_kind ? chain_lds<bf16, 64, 1>(lam, C).total : chain_lds<bf16, 64, 0>(lam, C).total;
    return phi_kind ? chain_lds<bf16, 128, 1>(lam, C).total : chain_lds<bf16, 128, 0>(lam, C).total;
}

template hipError_t launch_chain_t<float, 64, 0>(const PrefillArgs&, hipStream_t);
template hipError_t launch_chain_t<float, 64, 1>(const PrefillArgs&, hipStream_t);
template hipError_t launch_chain_t<float, 128, 0>(const PrefillArgs&, hipStream_t);
template hipError_t launch_chain_t<float, 128, 1>(const PrefillArgs&, hipStream_t);
template hipError_t launch_chain_t<bf16, 64, 0>(const PrefillArgs&, hipStream_t);
template hipError_t launch_chain_t<bf16, 64, 1>(const PrefillArgs&, hipStream_t);
template hipError_t launch_chain_t<bf16, 128, 0>(const PrefillArgs&, hipStream_t);
template hipError_t launch_chain_t<bf16, 128, 1>(const PrefillArgs&, hipStream_t);

}  // namespace lola
