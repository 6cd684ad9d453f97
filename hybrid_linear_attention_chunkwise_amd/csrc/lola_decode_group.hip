// Chunked single-token decode: the allocation runs once per group of Cd decode steps (LoLA notes 2.6,
// Eq. (15) and Fig. 2, with 2.4 and Eq. (14) per step), for a decoder that only has one token at a
// time.  Groups cover exit times [a, b) with b the next multiple of Cd after a (so from an aligned
// start every group is Cd steps).
//
// Group start (the first step of a group, at t = a): the candidates are the cache and the tokens that
// leave the window during the group, positions [a - eta, b - eta), all of which are in the ring (or
// the current token) already.  If they exceed lambda, every candidate's SRE against the state at the
// group start ranks them (ties: older kept) and the lambda largest stay exact.  Old cache members
// that lose are folded at once (their tau is the group start); leaving tokens that lose are marked in
// the per-(sequence, head) fold mask (bit = exit time mod Cd) and folded at their own exit step;
// leaving tokens that stay move into the freed slots (slot order, position order).
// Every step: fold the token leaving at this step if it is marked, read out over the window, the cache
// members that have left the window (pos + eta <= t) and the state, and write the token into the ring.
//
// One workgroup per (sequence, head), one wave per 16 value rows of H^T (fp32 registers); H^T in bf16
// fragment order in LDS is the A operand of the candidates' recalls.  Folds are rank-1 updates in fp32
// registers, in batches of 16 tokens whose features come from one MFMA tile.
#include "lola_common.hpp"
#include "lola_internal.hpp"

namespace lola {

namespace {

__host__ __device__ inline size_t al16g(size_t x) { return (x + 15) & ~size_t(15); }
constexpr int kFoldBatch = 16;

template <typename T, int DK, int PHI>
struct GrpCfg {
    static constexpr int D = kFeat, DV = DK;
    static constexpr int DW = (PHI == kPhiSoftmaxPM) ? D / 2 : D;
    static constexpr int NW = DV / 16;
    static constexpr int NT = 64 * NW;
    static constexpr int WT_LD = DK + 4;
    static constexpr int EPV = 16 / (int)sizeof(T);
};

struct GrpLds {
    size_t hb, wt, s, q, phiq, cpos, csrc, key, fold, pre1, pre2, fphi, fv, logit, wlog, red, o, lsum, list, total;
};

// rows: lam cache slots then up to Cd leaving tokens (rounded up to whole 64-row ballot groups)
__host__ __device__ inline int grp_rows(int lam, int cd) { return ((lam + cd + 63) / 64) * 64; }

template <typename T, int DK, int PHI>
__host__ __device__ inline GrpLds grp_lds(int lam, int eta, int cd) {
    using Cfg = GrpCfg<T, DK, PHI>;
    constexpr int D = Cfg::D, DV = Cfg::DV;
    const int nr = grp_rows(lam, cd);
    GrpLds o;
    size_t p = 0;
    o.hb = p;     p = al16g(p + sizeof(T) * DV * D);
    o.wt = p;     p = al16g(p + sizeof(T) * Cfg::DW * Cfg::WT_LD);
    o.s = p;      p = al16g(p + sizeof(float) * D);
    o.q = p;      p = al16g(p + sizeof(float) * DK);
    o.phiq = p;   p = al16g(p + sizeof(float) * D);
    o.cpos = p;   p = al16g(p + sizeof(int) * (lam + 1));        // slot positions after the allocation
    o.csrc = p;   p = al16g(p + sizeof(int) * (lam + 1));        // slot -> candidate row that entered it, or -1
    o.key = p;    p = al16g(p + sizeof(unsigned long long) * nr);
    o.fold = p;   p = al16g(p + sizeof(int) * nr);               // 1: candidate row folded
    o.pre1 = p;   p = al16g(p + sizeof(int) * nr);               // prefix counts (freed slots / entrants)
    o.pre2 = p;   p = al16g(p + sizeof(int) * nr);
    o.fphi = p;   p = al16g(p + sizeof(float) * kFoldBatch * D);
    o.fv = p;     p = al16g(p + sizeof(float) * kFoldBatch * DV);
    o.logit = p;  p = al16g(p + sizeof(float) * (lam + 16));
    o.wlog = p;   p = al16g(p + sizeof(float) * (eta + 16));
    o.red = p;    p = al16g(p + sizeof(unsigned long long) * 32);
    o.o = p;      p = al16g(p + sizeof(float) * Cfg::NW * DV);
    o.lsum = p;   p = al16g(p + sizeof(float) * DV);
    o.list = p;   p = al16g(p + sizeof(int) * (lam + cd + 2));   // rows folded at this step
    o.total = p;
    return o;
}

__device__ __forceinline__ unsigned long long keep_key_g(float sre, int pos) {
    return ((unsigned long long)__float_as_uint(sre) << 32) | (unsigned long long)(0xFFFFFFFFu - (unsigned)pos);
}

template <typename T>
__device__ __forceinline__ void load4g(const T* p, float (&o)[4]);
template <>
__device__ __forceinline__ void load4g<float>(const float* p, float (&o)[4]) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
template <>
__device__ __forceinline__ void load4g<bf16>(const bf16* p, float (&o)[4]) {
    const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
    o[0] = (float)v[0]; o[1] = (float)v[1]; o[2] = (float)v[2]; o[3] = (float)v[3];
}

template <typename T, int DK, int PHI>
__global__ __launch_bounds__(4 * DK) void decode_group_kernel(DecodeArgs A) {
    using Cfg = GrpCfg<T, DK, PHI>;
    constexpr int D = Cfg::D, DV = Cfg::DV, DW = Cfg::DW, NW = Cfg::NW, NT = Cfg::NT, WT_LD = Cfg::WT_LD,
                  EPV = Cfg::EPV, JT = DV / 16, IT = D / 16;
    extern __shared__ __align__(16) char smem[];
    const int lam = A.lam, eta = A.eta, cd = A.dec_chunk;
    const bool gs = A.group_start != 0;
    const GrpLds lo = grp_lds<T, DK, PHI>(lam, eta, cd);
    T* sHb = reinterpret_cast<T*>(smem + lo.hb);
    T* wt = reinterpret_cast<T*>(smem + lo.wt);
    float* sS = reinterpret_cast<float*>(smem + lo.s);
    float* sQ = reinterpret_cast<float*>(smem + lo.q);
    float* sPhiQ = reinterpret_cast<float*>(smem + lo.phiq);
    int* sCpos = reinterpret_cast<int*>(smem + lo.cpos);
    int* sCsrc = reinterpret_cast<int*>(smem + lo.csrc);
    unsigned long long* sKey = reinterpret_cast<unsigned long long*>(smem + lo.key);
    int* sFold = reinterpret_cast<int*>(smem + lo.fold);
    int* sPre1 = reinterpret_cast<int*>(smem + lo.pre1);
    int* sPre2 = reinterpret_cast<int*>(smem + lo.pre2);
    float* sFphi = reinterpret_cast<float*>(smem + lo.fphi);
    float* sFv = reinterpret_cast<float*>(smem + lo.fv);
    float* sLogit = reinterpret_cast<float*>(smem + lo.logit);
    float* sWlog = reinterpret_cast<float*>(smem + lo.wlog);
    unsigned long long* sRed = reinterpret_cast<unsigned long long*>(smem + lo.red);
    float* sO = reinterpret_cast<float*>(smem + lo.o);
    float* sL = reinterpret_cast<float*>(smem + lo.lsum);
    int* sList = reinterpret_cast<int*>(smem + lo.list);
    int* sRedI = reinterpret_cast<int*>(sRed + 8);
    float* sRedF = reinterpret_cast<float*>(sRed + 16);

    const int bh = blockIdx.x;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c = l & 15;
    const int64_t t = A.t;
    const float scale = 1.0f / sqrtf((float)DK);

    float* Hg = A.H + (int64_t)bh * DV * D;
    float* sg = A.s + (int64_t)bh * D;
    const T* qg = reinterpret_cast<const T*>(A.q) + (int64_t)bh * DK;
    const T* kg = reinterpret_cast<const T*>(A.k) + (int64_t)bh * DK;
    const T* vg = reinterpret_cast<const T*>(A.v) + (int64_t)bh * DV;
    T* ringK = eta > 0 ? reinterpret_cast<T*>(A.win_k) + (int64_t)bh * eta * DK : nullptr;
    T* ringV = eta > 0 ? reinterpret_cast<T*>(A.win_v) + (int64_t)bh * eta * DV : nullptr;
    T* cK = lam > 0 ? reinterpret_cast<T*>(A.cache_k) + (int64_t)bh * lam * DK : nullptr;
    T* cV = lam > 0 ? reinterpret_cast<T*>(A.cache_v) + (int64_t)bh * lam * DV : nullptr;
    int32_t* cpos = lam > 0 ? A.cache_pos + (int64_t)bh * lam : nullptr;
    unsigned long long* maskg = A.dec_fold + bh;

    // where position p's K / V live during this step: the current input, or its ring slot
    auto key_row = [&](int64_t p) -> const T* { return (p == t || eta == 0) ? kg : ringK + (int)(p % eta) * DK; };
    auto val_row = [&](int64_t p) -> const T* { return (p == t || eta == 0) ? vg : ringV + (int)(p % eta) * DV; };

    // the group's leaving tokens: exit times [t, t + glen), positions [t - eta, t - eta + glen) >= 0
    const int glen = cd - (int)(t % cd);
    const int64_t xlo = t - eta > 0 ? t - eta : 0;
    const int64_t xhi = t - eta + glen;
    const int nX = (gs && xhi > xlo) ? (int)(xhi - xlo) : 0;
    const int nrow = lam + nX;

    // ---- stage ----
    f4 acc[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const float4 h = *reinterpret_cast<const float4*>(Hg + (16 * w + c) * D + 16 * i + 4 * g);
        acc[i] = f4{h.x, h.y, h.z, h.w};
    }
    stage_wt<T, DK, DW, NT>(wt, WT_LD, A.W);
    for (int d = tid; d < D; d += NT) sS[d] = sg[d];
    for (int d = tid; d < DK; d += NT) sQ[d] = to_f(qg[d]);
    for (int j = tid; j < lam; j += NT) { sCpos[j] = cpos[j]; sCsrc[j] = -1; }
#pragma unroll
    for (int ss = 0; ss < D / 32; ++ss)
        *reinterpret_cast<Frag8<T>*>(sHb + ((w * (D / 32) + ss) * 64 + l) * 8) =
            frag_from_acc<T>(acc[2 * ss], acc[2 * ss + 1]);
    __syncthreads();
    int nG = 0;
    for (int k = 0; k * 64 < lam; ++k) {
        const int j = k * 64 + l;
        nG += __popcll(__ballot(j < lam && sCpos[j] >= 0));
    }
    if (w == 0) {       // features of the query (one tile, the query in column 0)
        Frag8<T> xf[DK / 32];
#pragma unroll
        for (int ss = 0; ss < DK / 32; ++ss) xf[ss] = c == 0 ? load_frag(qg, ss, g) : frag_zero<T>();
        float ph[D / 16][4];
        phi_tile<T, DK, PHI>(wt, WT_LD, xf, ph);
        if (c == 0)
#pragma unroll
            for (int ft = 0; ft < D / 16; ++ft)
#pragma unroll
                for (int r = 0; r < 4; ++r) sPhiQ[16 * ft + 4 * g + r] = ph[ft][r];
    }
    __syncthreads();

    // ---- group start: scoring and allocation ----
    unsigned long long mask = gs ? 0ull : *maskg;
    int nfold_now = 0;                         // rows folded at this step (old members), listed in sList
    if (gs) {
        const bool scoring = lam > 0 && nG + nX > lam;
        // candidate row r: a cache slot (r < lam) or leaving position xlo + (r - lam)
        auto row_valid = [&](int r) { return r < lam ? sCpos[r] >= 0 : r < nrow; };
        auto row_pos = [&](int r) -> int { return r < lam ? sCpos[r] : (int)(xlo + (r - lam)); };
        if (scoring) {
            float sv[D / 32][8];
#pragma unroll
            for (int ss = 0; ss < D / 32; ++ss)
#pragma unroll
                for (int e = 0; e < 8; ++e) sv[ss][e] = sS[32 * ss + 16 * (e >> 2) + 4 * g + (e & 3)];
            for (int tile = w; tile * 16 < nrow; tile += NW) {
                const int row = tile * 16 + c;
                const bool valid = row < nrow && row_valid(row);
                const T* rk = kg;
                const T* rv = vg;
                if (valid) {
                    if (row < lam) { rk = cK + (int64_t)row * DK; rv = cV + (int64_t)row * DV; }
                    else { rk = key_row(xlo + (row - lam)); rv = val_row(xlo + (row - lam)); }
                }
                Frag8<T> kf[DK / 32];
#pragma unroll
                for (int ss = 0; ss < DK / 32; ++ss) kf[ss] = valid ? load_frag(rk, ss, g) : frag_zero<T>();
                float vv[JT][4];
#pragma unroll
                for (int J = 0; J < JT; ++J) {
                    if (valid) load4g<T>(rv + 16 * J + 4 * g, vv[J]);
                    else { vv[J][0] = vv[J][1] = vv[J][2] = vv[J][3] = 0.f; }
                }
                float ph[D / 16][4];
                phi_tile<T, DK, PHI>(wt, WT_LD, kf, ph);
                float den = 0.f;
#pragma unroll
                for (int ss = 0; ss < D / 32; ++ss)
#pragma unroll
                    for (int e = 0; e < 8; ++e) den += ph[2 * ss + (e >> 2)][e & 3] * sv[ss][e];
                den = sum_groups(den);
                const float inv = den != 0.f ? fast_rcp(den) : 0.f;      // empty state: recall 0
                float sq = 0.f;
#pragma unroll
                for (int J = 0; J < JT; ++J) {
                    f4 num = zero4();
#pragma unroll
                    for (int ss = 0; ss < D / 32; ++ss) {
                        const Frag8<T> a = *reinterpret_cast<const Frag8<T>*>(sHb + ((J * (D / 32) + ss) * 64 + l) * 8);
                        const Frag8<T> b = frag_from_acc<T>(f4{ph[2 * ss][0], ph[2 * ss][1], ph[2 * ss][2], ph[2 * ss][3]},
                                                            f4{ph[2 * ss + 1][0], ph[2 * ss + 1][1], ph[2 * ss + 1][2],
                                                               ph[2 * ss + 1][3]});
                        mma32(num, a, b);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float x = num[r] * inv - vv[J][r];
                        sq += x * x;
                    }
                }
                sq = sum_groups(sq);
                if (g == 0 && row < nrow) sKey[row] = valid ? keep_key_g(__builtin_amdgcn_sqrtf(sq), row_pos(row)) : 0ull;
            }
            __syncthreads();
            // exact rank: the nF smallest keys are folded (keys are distinct: positions differ)
            const int nF = nG + nX - lam;
            for (int r = tid; r < nrow; r += NT) {
                int f = 0;
                if (row_valid(r)) {
                    const unsigned long long kr = sKey[r];
                    int below = 0;
                    for (int j = 0; j < nrow; ++j) below += (sKey[j] != 0ull && sKey[j] < kr);
                    f = below < nF;
                }
                sFold[r] = f;
            }
        } else {
            // nothing to score: lambda = 0 folds every leaving token; otherwise all fit and stay
            for (int r = tid; r < nrow; r += NT) sFold[r] = (lam == 0 && r >= lam && row_valid(r)) ? 1 : 0;
        }
        __syncthreads();
        // freed slots (empty, or holding a folded member) in slot order; entrants (kept leaving tokens)
        // in position order; the k-th entrant takes the k-th freed slot
        const int nFree = ballot_prefix(lam, NW, [&](int j) { return sCpos[j] < 0 || sFold[j]; }, sPre1);
        const int nEnt = ballot_prefix(nX, NW, [&](int x) { return !sFold[lam + x]; }, sPre2);
        (void)nFree;
        __syncthreads();
        for (int j = tid; j < lam; j += NT) {
            const bool freed = sCpos[j] < 0 || sFold[j];
            if (!freed) continue;
            const int k = sPre1[j];
            if (k < nEnt) {
                // the k-th entrant: find x with entrant rank k (entrant ranks are the prefix over x)
                int x = -1;
                for (int xx = 0; xx < nX; ++xx)
                    if (!sFold[lam + xx] && sPre2[xx] == k) { x = xx; break; }
                sCsrc[j] = lam + x;
            }
        }
        // old members folded now, and the leaving tokens marked to fold at their exit
        if (tid == 0) {
            int nf = 0;
            for (int j = 0; j < lam; ++j)
                if (sCpos[j] >= 0 && sFold[j]) sList[nf++] = j;
            sRedI[4] = nf;
        }
        for (int x = 0; x < nX; ++x)
            if (sFold[lam + x]) mask |= 1ull << ((xlo + x + eta) % cd);
        __syncthreads();
        nfold_now = sRedI[4];
    } else if (lam == 0) {
        mask = ~0ull;                        // no cache: every leaving token folds at its exit
    }

    // ---- this step's folds: old members (group start) and the token leaving now, if marked ----
    const bool has_e = (eta == 0) || (t >= eta);
    const bool fold_e = has_e && (lam == 0 || ((mask >> (t % cd)) & 1ull));
    const int nfold = nfold_now + (fold_e ? 1 : 0);
    for (int b0 = 0; b0 < nfold; b0 += kFoldBatch) {
        const int nb = nfold - b0 < kFoldBatch ? nfold - b0 : kFoldBatch;
        auto fold_rows = [&](int i, const T*& rk, const T*& rv) {
            const int idx = b0 + i;
            if (idx < nfold_now) {
                const int j = sList[idx];
                rk = cK + (int64_t)j * DK;
                rv = cV + (int64_t)j * DV;
            } else {
                rk = eta == 0 ? kg : ringK + (int)(t % eta) * DK;
                rv = eta == 0 ? vg : ringV + (int)(t % eta) * DV;
            }
        };
        if (w == 0) {
            const T* rk = kg;
            const T* rv = vg;
            const bool ok = c < nb;
            if (ok) fold_rows(c, rk, rv);
            Frag8<T> xf[DK / 32];
#pragma unroll
            for (int ss = 0; ss < DK / 32; ++ss) xf[ss] = ok ? load_frag(rk, ss, g) : frag_zero<T>();
            float ph[D / 16][4];
            phi_tile<T, DK, PHI>(wt, WT_LD, xf, ph);
            if (ok)
#pragma unroll
                for (int ft = 0; ft < D / 16; ++ft)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sFphi[c * D + 16 * ft + 4 * g + r] = ph[ft][r];
        }
        for (int q = tid; q < nb * DV; q += NT) {
            const int i = q / DV, d = q % DV;
            const T* rk;
            const T* rv;
            fold_rows(i, rk, rv);
            sFv[i * DV + d] = to_f(rv[d]);
        }
        __syncthreads();
        for (int i = 0; i < nb; ++i) {
            const float vd = sFv[i * DV + 16 * w + c];
#pragma unroll
            for (int ii = 0; ii < IT; ++ii)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[ii][r] += vd * sFphi[i * D + 16 * ii + 4 * g + r];
        }
        for (int f = tid; f < D; f += NT) {
            float add = 0.f;
            for (int i = 0; i < nb; ++i) add += sFphi[i * D + f];
            sS[f] += add;
        }
        __syncthreads();
    }

    // ---- cache after the allocation: slot j holds position sCpos'[j] whose rows are the cache rows,
    //      or (entered now) the leaving token's ring / input rows ----
    auto slot_pos = [&](int j) -> int {
        if (gs) {
            if (sCsrc[j] >= 0) return (int)(xlo + (sCsrc[j] - lam));
            if (sCpos[j] >= 0 && sFold[j]) return -1;
        }
        return sCpos[j];
    };
    auto slot_k = [&](int j) -> const T* {
        return (gs && sCsrc[j] >= 0) ? key_row(xlo + (sCsrc[j] - lam)) : cK + (int64_t)j * DK;
    };
    auto slot_v = [&](int j) -> const T* {
        return (gs && sCsrc[j] >= 0) ? val_row(xlo + (sCsrc[j] - lam)) : cV + (int64_t)j * DV;
    };
    // a member is read exactly once it has left the window (before that the window holds it)
    auto cache_exact = [&](int j) -> bool {
        if (!(A.read_mask & kReadSparse)) return false;
        const int p = slot_pos(j);
        return p >= 0 && (int64_t)p + eta <= t;
    };

    // ---- logits: cache slots, then the window (positions max(0, t-eta+1) .. t) ----
    for (int tile = w; tile * 16 < lam; tile += NW) {
        const int j = tile * 16 + c;
        const bool valid = j < lam && cache_exact(j);
        const T* rk = valid ? slot_k(j) : kg;
        float lg = 0.f;
#pragma unroll
        for (int ss = 0; ss < DK / 32; ++ss) {
            const Frag8<T> kf = valid ? load_frag(rk, ss, g) : frag_zero<T>();
#pragma unroll
            for (int e = 0; e < 8; ++e) lg += frag_get(kf, e) * sQ[32 * ss + 16 * (e >> 2) + 4 * g + (e & 3)];
        }
        lg = sum_groups(lg) * scale;
        if (g == 0 && j < lam) sLogit[j] = lg;
    }
    const int64_t wlo = max((int64_t)0, t - eta + 1);
    const int nw = eta > 0 ? (int)(t - wlo + 1) : 0;
    for (int tile = w; tile * 16 < nw; tile += NW) {
        const int i = tile * 16 + c;
        const bool valid = i < nw;
        const T* rk = valid ? key_row(wlo + i) : kg;
        float lg = 0.f;
#pragma unroll
        for (int ss = 0; ss < DK / 32; ++ss) {
            const Frag8<T> kf = valid ? load_frag(rk, ss, g) : frag_zero<T>();
#pragma unroll
            for (int e = 0; e < 8; ++e) lg += frag_get(kf, e) * sQ[32 * ss + 16 * (e >> 2) + 4 * g + (e & 3)];
        }
        lg = sum_groups(lg) * scale;
        if (g == 0 && valid) sWlog[i] = lg;
    }
    float Lrow;
    {
        float part_ = 0.f;
#pragma unroll
        for (int i = 0; i < IT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) part_ += acc[i][r] * sPhiQ[16 * i + 4 * g + r];
        Lrow = sum_groups(part_);
    }
    __syncthreads();
    float mloc = -INFINITY;
    for (int i = tid; i < nw; i += NT) mloc = fmaxf(mloc, sWlog[i]);
    for (int j = tid; j < lam; j += NT)
        if (cache_exact(j)) mloc = fmaxf(mloc, sLogit[j]);
    for (int o = 32; o > 0; o >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o));
    if (l == 0) sRedF[w] = mloc;
    __syncthreads();
    float m = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) m = fmaxf(m, sRedF[ww]);

    // ---- weighted values ----
    constexpr int LPR = DV / EPV;
    constexpr int RPW = 64 / LPR;
    const int sub = l / LPR, col = (l % LPR) * EPV;
    float o[EPV];
#pragma unroll
    for (int x = 0; x < EPV; ++x) o[x] = 0.f;
    float lsum = 0.f;
    const int nkeys = nw + lam;
    for (int kk0 = w * RPW; kk0 < nkeys; kk0 += NW * RPW * 4) {
        uint4 raw[4];
        float pw[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int kk = kk0 + u * NW * RPW + sub;
            float lg = -INFINITY;
            const T* rv = nullptr;
            if (kk < nw) {
                lg = sWlog[kk];
                rv = val_row(wlo + kk);
            } else if (kk < nkeys) {
                const int j = kk - nw;
                if (cache_exact(j)) {
                    lg = sLogit[j];
                    rv = slot_v(j);
                }
            }
            pw[u] = rv ? fast_exp(lg - m) : 0.f;
            raw[u] = rv ? *reinterpret_cast<const uint4*>(rv + col) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const T* e = reinterpret_cast<const T*>(&raw[u]);
#pragma unroll
            for (int x = 0; x < EPV; ++x) o[x] += pw[u] * to_f(e[x]);
            if ((l % LPR) == 0) lsum += pw[u];
        }
    }
#pragma unroll
    for (int x = 0; x < EPV; ++x)
        for (int sh = LPR; sh < 64; sh <<= 1) o[x] += __shfl_xor(o[x], sh);
    for (int sh = 1; sh < 64; sh <<= 1) lsum += __shfl_xor(lsum, sh);
    if (sub == 0)
#pragma unroll
        for (int x = 0; x < EPV; ++x) sO[w * DV + col + x] = o[x];
    if (l == 0) sRedF[8 + w] = lsum;
    if (g == 0) sL[16 * w + c] = Lrow;
    __syncthreads();

    // ---- output (Eq. (14), one shared normaliser with a common scale) ----
    {
        const bool rs = (A.read_mask & kReadState) != 0;
        float lden = 0.f;
        if (rs)
            for (int f = 0; f < D; ++f) lden += sPhiQ[f] * sS[f];
        float lsum_all = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) lsum_all += sRedF[8 + ww];
        for (int d = tid; d < DV; d += NT) {
            float Od = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) Od += sO[ww * DV + d];
            const float Ld = rs ? sL[d] : 0.f;
            const bool any = m != -INFINITY;
            float cm;
            if (lden > 0.f) cm = any ? fmaxf(m, logf(lden)) : logf(lden);
            else cm = m;
            const float sl = lden > 0.f ? fast_exp(-cm) : 0.f;
            const float se = any ? fast_exp(m - cm) : 0.f;
            const float yv = (Ld * sl + Od * se) / (lden * sl + lsum_all * se);
            reinterpret_cast<T*>(A.y)[(int64_t)bh * DV + d] = from_f<T>(yv);
        }
    }

    // ---- state write-back: H, s, the entrants' rows into their slots, the mask, then the ring ----
#pragma unroll
    for (int i = 0; i < IT; ++i)
        *reinterpret_cast<float4*>(Hg + (16 * w + c) * D + 16 * i + 4 * g) =
            make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
    for (int f = tid; f < D; f += NT) sg[f] = sS[f];
    if (gs) {
        for (int q = tid; q < lam * (DK + DV); q += NT) {
            const int j = q / (DK + DV), d = q % (DK + DV);
            if (sCsrc[j] < 0) continue;
            const int64_t p = xlo + (sCsrc[j] - lam);
            if (d < DK) cK[(int64_t)j * DK + d] = key_row(p)[d];
            else cV[(int64_t)j * DV + (d - DK)] = val_row(p)[d - DK];
        }
        for (int j = tid; j < lam; j += NT) cpos[j] = slot_pos(j);
        if (tid == 0) *maskg = mask;
    }
    __syncthreads();                           // every read of the ring is done before it is written
    if (eta > 0) {
        const int slot = (int)(t % eta);
        for (int d = tid; d < DK; d += NT) ringK[(int64_t)slot * DK + d] = kg[d];
        for (int d = tid; d < DV; d += NT) ringV[(int64_t)slot * DV + d] = vg[d];
    }
}

}  // namespace

size_t decode_group_lds_bytes(int d, int phi_kind, int esz, int lam, int eta, int cd) {
    if (esz == 4) {
        if (d == 64) return phi_kind ? grp_lds<float, 64, 1>(lam, eta, cd).total : grp_lds<float, 64, 0>(lam, eta, cd).total;
        return phi_kind ? grp_lds<float, 128, 1>(lam, eta, cd).total : grp_lds<float, 128, 0>(lam, eta, cd).total;
    }
    if (d == 64) return phi_kind ? grp_lds<bf16, 64, 1>(lam, eta, cd).total : grp_lds<bf16, 64, 0>(lam, eta, cd).total;
    return phi_kind ? grp_lds<bf16, 128, 1>(lam, eta, cd).total : grp_lds<bf16, 128, 0>(lam, eta, cd).total;
}

template <typename T, int DK, int PHI>
static hipError_t launch_group_t(const DecodeArgs& a, hipStream_t stream) {
    const size_t lds = grp_lds<T, DK, PHI>(a.lam, a.eta, a.dec_chunk).total;
    auto kern = decode_group_kernel<T, DK, PHI>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(a.BH), dim3(GrpCfg<T, DK, PHI>::NT), lds, stream, a);
    return hipGetLastError();
}

hipError_t launch_decode_group(const DecodeArgs& a, int dtype, int d, int phi_kind, hipStream_t stream) {
    if (dtype == 0) {
        if (d == 64) return phi_kind ? launch_group_t<float, 64, 1>(a, stream) : launch_group_t<float, 64, 0>(a, stream);
        return phi_kind ? launch_group_t<float, 128, 1>(a, stream) : launch_group_t<float, 128, 0>(a, stream);
    }
    if (d == 64) return phi_kind ? launch_group_t<bf16, 64, 1>(a, stream) : launch_group_t<bf16, 64, 0>(a, stream);
    return phi_kind ? launch_group_t<bf16, 128, 1>(a, stream) : launch_group_t<bf16, 128, 0>(a, stream);
}

}  // namespace lola
