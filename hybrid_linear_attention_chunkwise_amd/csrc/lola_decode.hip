// Decode step: one workgroup per (sequence, head), one token.  LoLA notes 2.4 (single-token update:
// the token leaving the window joins the cache as a candidate, SRE against the state before the
// update, fold the lowest) followed by Eq. (14) of 2.5.
//
// Memory-bound: every step streams H (read + write), the window ring and the cache.  The workgroup
// has one wave per 16 value rows of H^T; each wave keeps its rows in fp32 registers for the whole
// step (fold and linear read-out happen there) and publishes a bf16 copy in LDS, in MFMA fragment
// order, which all waves read as the A operand of the SRE numerators H^T Phi_E^T.  Candidates (the
// cache slots and the leaving token) are processed in 16-column tiles: keys give both the exact logits
// and the features (one MFMA tile through W^T), values give the squared errors.  Window keys give the
// remaining logits; one pass over window and cache values then forms the exact numerator.
#include "lola_common.hpp"
#include "lola_internal.hpp"

namespace lola {

namespace {

__host__ __device__ inline size_t al16d(size_t x) { return (x + 15) & ~size_t(15); }

template <typename T, int DK, int PHI>
struct DecCfg {
    static constexpr int D = kFeat, DV = DK;
    static constexpr int DW = (PHI == kPhiSoftmaxPM) ? D / 2 : D;
    static constexpr int NW = DV / 16;          // waves: one per 16 value rows of H^T
    static constexpr int NT = 64 * NW;
    static constexpr int WT_LD = DK + 4;
    static constexpr int EPV = 16 / (int)sizeof(T);
};

struct DecLds {
    size_t hb, wt, s, q, phiq, phif, vf, ek, ev, cpos, sre, logit, wlog, red, o, lsum, total;
};

template <typename T, int DK, int PHI>
__host__ __device__ inline DecLds dec_lds(int lam, int eta) {
    using Cfg = DecCfg<T, DK, PHI>;
    constexpr int D = Cfg::D, DV = Cfg::DV;
    DecLds o;
    size_t p = 0;
    o.hb = p;     p = al16d(p + sizeof(T) * DV * D);                 // H^T in fragment order
    o.wt = p;     p = al16d(p + sizeof(T) * Cfg::DW * Cfg::WT_LD);
    o.s = p;      p = al16d(p + sizeof(float) * D);
    o.q = p;      p = al16d(p + sizeof(float) * DK);
    o.phiq = p;   p = al16d(p + sizeof(float) * D);
    o.phif = p;   p = al16d(p + sizeof(float) * D);
    o.vf = p;     p = al16d(p + sizeof(float) * DV);
    o.ek = p;     p = al16d(p + sizeof(T) * DK);
    o.ev = p;     p = al16d(p + sizeof(T) * DV);
    o.cpos = p;   p = al16d(p + sizeof(int) * (lam + 1));
    o.sre = p;    p = al16d(p + sizeof(float) * (lam + 16));
    o.logit = p;  p = al16d(p + sizeof(float) * (lam + 16));
    o.wlog = p;   p = al16d(p + sizeof(float) * (eta + 16));
    o.red = p;    p = al16d(p + sizeof(unsigned long long) * 32);
    o.o = p;      p = al16d(p + sizeof(float) * Cfg::NW * DV);
    o.lsum = p;   p = al16d(p + sizeof(float) * DV);
    o.total = p;
    return o;
}

__device__ __forceinline__ unsigned long long keep_key_d(float sre, int pos) {
    return ((unsigned long long)__float_as_uint(sre) << 32) | (unsigned long long)(0xFFFFFFFFu - (unsigned)pos);
}

template <typename T>
__device__ __forceinline__ void load4f(const T* p, float (&o)[4]);
template <>
__device__ __forceinline__ void load4f<float>(const float* p, float (&o)[4]) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
template <>
__device__ __forceinline__ void load4f<bf16>(const bf16* p, float (&o)[4]) {
    const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
    o[0] = (float)v[0]; o[1] = (float)v[1]; o[2] = (float)v[2]; o[3] = (float)v[3];
}

template <typename T, int DK, int PHI>
__global__ __launch_bounds__(4 * DK) void decode_kernel(DecodeArgs A) {
    using Cfg = DecCfg<T, DK, PHI>;
    constexpr int D = Cfg::D, DV = Cfg::DV, DW = Cfg::DW, NW = Cfg::NW, NT = Cfg::NT, WT_LD = Cfg::WT_LD,
                  EPV = Cfg::EPV, JT = DV / 16, IT = D / 16;
    extern __shared__ __align__(16) char smem[];
    const int lam = A.lam, eta = A.eta;
    const DecLds lo = dec_lds<T, DK, PHI>(lam, eta);
    T* sHb = reinterpret_cast<T*>(smem + lo.hb);
    T* wt = reinterpret_cast<T*>(smem + lo.wt);
    float* sS = reinterpret_cast<float*>(smem + lo.s);
    float* sQ = reinterpret_cast<float*>(smem + lo.q);
    float* sPhiQ = reinterpret_cast<float*>(smem + lo.phiq);
    float* sPhiF = reinterpret_cast<float*>(smem + lo.phif);
    float* sVf = reinterpret_cast<float*>(smem + lo.vf);
    T* sEk = reinterpret_cast<T*>(smem + lo.ek);
    T* sEv = reinterpret_cast<T*>(smem + lo.ev);
    int* sCpos = reinterpret_cast<int*>(smem + lo.cpos);
    float* sSre = reinterpret_cast<float*>(smem + lo.sre);
    float* sLogit = reinterpret_cast<float*>(smem + lo.logit);
    float* sWlog = reinterpret_cast<float*>(smem + lo.wlog);
    unsigned long long* sRed = reinterpret_cast<unsigned long long*>(smem + lo.red);
    float* sO = reinterpret_cast<float*>(smem + lo.o);
    float* sL = reinterpret_cast<float*>(smem + lo.lsum);
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

    // the token that leaves the window at this step (token t itself when eta == 0)
    const bool has_e = (eta == 0) || (t >= eta);
    const int64_t e_pos = t - eta;
    const T* ekg = eta == 0 ? kg : (has_e ? ringK + (t % eta) * DK : nullptr);
    const T* evg = eta == 0 ? vg : (has_e ? ringV + (t % eta) * DV : nullptr);

    // ---- stage: H^T rows of this wave (fp32 registers) and their bf16 copy in fragment order ----
    f4 acc[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const float4 h = *reinterpret_cast<const float4*>(Hg + (16 * w + c) * D + 16 * i + 4 * g);
        acc[i] = f4{h.x, h.y, h.z, h.w};
    }
    stage_wt<T, DK, DW, NT>(wt, WT_LD, A.W);
    for (int d = tid; d < D; d += NT) sS[d] = sg[d];
    for (int d = tid; d < DK; d += NT) {
        sQ[d] = to_f(qg[d]);
        sEk[d] = has_e ? ekg[d] : from_f<T>(0.f);
    }
    for (int d = tid; d < DV; d += NT) sEv[d] = has_e ? evg[d] : from_f<T>(0.f);
    for (int j = tid; j < lam; j += NT) sCpos[j] = cpos[j];
    if (tid == 0) sRed[1] = ~0ull;
#pragma unroll
    for (int ss = 0; ss < D / 32; ++ss)
        *reinterpret_cast<Frag8<T>*>(sHb + ((w * (D / 32) + ss) * 64 + l) * 8) =
            frag_from_acc<T>(acc[2 * ss], acc[2 * ss + 1]);
    __syncthreads();
    // occupied slots and the first empty one, by wave ballots (every wave gets the same answer)
    int nG = 0, first_empty = -1;
    for (int k = 0; k * 64 < lam; ++k) {
        const int j = k * 64 + l;
        const unsigned long long occ = __ballot(j < lam && sCpos[j] >= 0);
        const unsigned long long emp = __ballot(j < lam && sCpos[j] < 0);
        nG += __popcll(occ);
        if (first_empty < 0 && emp) first_empty = k * 64 + __ffsll((long long)emp) - 1;
    }
    // features of the query: wave 0, one tile with the query in column 0
    if (w == 0) {
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
    const bool scoring = has_e && lam > 0 && nG >= lam;

    // ---- candidate tiles: cache slots (rows 0..lam-1) and the leaving token (row lam) ----
    const int nrow = lam + 1;
    float sv[D / 32][8];
#pragma unroll
    for (int ss = 0; ss < D / 32; ++ss)
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[ss][e] = sS[32 * ss + 16 * (e >> 2) + 4 * g + (e & 3)];
    for (int tile = w; tile * 16 < nrow; tile += NW) {
        const int row = tile * 16 + c;
        bool valid;
        const T* rk;
        const T* rv;
        if (row < lam) { valid = sCpos[row] >= 0; rk = cK + (int64_t)row * DK; rv = cV + (int64_t)row * DV; }
        else { valid = (row == lam) && has_e; rk = sEk; rv = sEv; }
        Frag8<T> kf[DK / 32];
#pragma unroll
        for (int ss = 0; ss < DK / 32; ++ss) kf[ss] = valid ? load_frag(rk, ss, g) : frag_zero<T>();
        float vv[JT][4];
        if (scoring) {
#pragma unroll
            for (int J = 0; J < JT; ++J) {
                if (valid) load4f<T>(rv + 16 * J + 4 * g, vv[J]);
                else { vv[J][0] = vv[J][1] = vv[J][2] = vv[J][3] = 0.f; }
            }
        }
        float lg = 0.f;
#pragma unroll
        for (int ss = 0; ss < DK / 32; ++ss)
#pragma unroll
            for (int e = 0; e < 8; ++e) lg += frag_get(kf[ss], e) * sQ[32 * ss + 16 * (e >> 2) + 4 * g + (e & 3)];
        lg = sum_groups(lg) * scale;
        if (g == 0 && row <= lam) sLogit[row] = lg;
        if (scoring) {
            float ph[D / 16][4];
            phi_tile<T, DK, PHI>(wt, WT_LD, kf, ph);
            float den = 0.f;
#pragma unroll
            for (int ss = 0; ss < D / 32; ++ss)
#pragma unroll
                for (int e = 0; e < 8; ++e) den += ph[2 * ss + (e >> 2)][e & 3] * sv[ss][e];
            den = sum_groups(den);
            const float inv = den != 0.f ? fast_rcp(den) : 0.f;     // empty state: recall 0
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
            if (g == 0 && row <= lam) sSre[row] = __builtin_amdgcn_sqrtf(sq);
        }
    }
    __syncthreads();

    // ---- allocation: which candidate is folded (row), and where the leaving token goes (slot) ----
    int f_row = -1;          // row folded into (H, s): 0..lam-1 a cache slot, lam the leaving token
    int e_slot = -1;         // slot that receives the leaving token
    if (scoring) {
        unsigned long long best = ~0ull;
        for (int r = tid; r < nrow; r += NT) {
            const bool valid = r < lam ? sCpos[r] >= 0 : has_e;
            if (!valid) continue;
            const int pos = r < lam ? sCpos[r] : (int)e_pos;
            const unsigned long long k = keep_key_d(sSre[r], pos);
            best = k < best ? k : best;
        }
        for (int o = 32; o > 0; o >>= 1) {
            const unsigned long long y = __shfl_xor(best, o);
            best = y < best ? y : best;
        }
        if (l == 0) atomicMin(&sRed[1], best);
        __syncthreads();
        const unsigned long long kmin = sRed[1];
        const int fpos = (int)(0xFFFFFFFFu - (unsigned)(kmin & 0xFFFFFFFFull));
        if (fpos == (int)e_pos) f_row = lam;
        else {
            if (tid == 0) sRedI[2] = -1;
            __syncthreads();
            for (int r = tid; r < lam; r += NT)
                if (sCpos[r] == fpos) sRedI[2] = r;
            __syncthreads();
            f_row = sRedI[2];
        }
        if (f_row < lam) e_slot = f_row;
    } else if (has_e) {
        if (lam == 0) f_row = lam;
        else e_slot = first_empty;
    }

    // ---- fold: features of the folded token (wave 0, one MFMA tile), then the rank-1 update ----
    if (f_row >= 0) {
        const T* kf_row = f_row < lam ? cK + (int64_t)f_row * DK : sEk;
        const T* vf_row = f_row < lam ? cV + (int64_t)f_row * DV : sEv;
        if (w == 0) {
            Frag8<T> xf[DK / 32];
#pragma unroll
            for (int ss = 0; ss < DK / 32; ++ss) xf[ss] = c == 0 ? load_frag(kf_row, ss, g) : frag_zero<T>();
            float ph[D / 16][4];
            phi_tile<T, DK, PHI>(wt, WT_LD, xf, ph);
            if (c == 0)
#pragma unroll
                for (int ft = 0; ft < D / 16; ++ft)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sPhiF[16 * ft + 4 * g + r] = ph[ft][r];
        }
        for (int d = tid; d < DV; d += NT) sVf[d] = to_f(vf_row[d]);
        __syncthreads();
        const float vd = sVf[16 * w + c];
#pragma unroll
        for (int i = 0; i < IT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][r] += vd * sPhiF[16 * i + 4 * g + r];
        for (int f = tid; f < D; f += NT) sS[f] += sPhiF[f];
    }

    // ---- window logits: positions max(0, t-eta+1) .. t-1 from the ring, t from the input ----
    const int64_t wlo = max((int64_t)0, t - eta + 1);
    const int nw = eta > 0 ? (int)(t - wlo + 1) : 0;
    // ring slot of window position wlo + i (i < nw <= eta), from one 64-bit remainder
    const int wslot0 = eta > 0 ? (int)(wlo % eta) : 0;
    auto wslot = [&](int i) { const int sl = wslot0 + i; return sl >= eta ? sl - eta : sl; };
    for (int tile = w; tile * 16 < nw; tile += NW) {
        const int i = tile * 16 + c;
        const bool valid = i < nw;
        const int64_t p = wlo + i;
        const T* rk = valid ? (p == t ? kg : ringK + wslot(i) * DK) : nullptr;
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
    // linear part (registers): L[d] for this wave's rows, and phi(q).s
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

    // exact set: window + cache after the allocation (occupied slots except a folded one, plus the
    // leaving token unless it was folded)
    auto cache_row_exact = [&](int r) -> bool {
        if (!(A.read_mask & kReadSparse)) return false;   // hidden cache: no exact cache keys
        if (r < lam) return sCpos[r] >= 0 && r != f_row;
        return has_e && f_row != lam && lam > 0;
    };
    float mloc = -INFINITY;
    for (int i = tid; i < nw; i += NT) mloc = fmaxf(mloc, sWlog[i]);
    for (int r = tid; r < nrow; r += NT)
        if (cache_row_exact(r)) mloc = fmaxf(mloc, sLogit[r]);
    for (int o = 32; o > 0; o >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o));
    if (l == 0) sRedF[w] = mloc;
    __syncthreads();
    float m = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) m = fmaxf(m, sRedF[ww]);

    // ---- weighted values: lane group (w, g) takes keys kk = 4*NW*j + 4*w + g; 16 lanes per row,
    //      EPV values per lane ----
    constexpr int LPR = DV / EPV;                 // lanes per value row
    constexpr int RPW = 64 / LPR;                 // rows per wave instruction
    const int sub = l / LPR, col = (l % LPR) * EPV;
    float o[EPV];
#pragma unroll
    for (int x = 0; x < EPV; ++x) o[x] = 0.f;
    float lsum = 0.f;
    const int nkeys = nw + nrow;
    for (int kk0 = w * RPW; kk0 < nkeys; kk0 += NW * RPW * 4) {
        uint4 raw[4];
        float pw[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int kk = kk0 + u * NW * RPW + sub;
            float lg = -INFINITY;
            const T* rv = nullptr;
            if (kk < nw) {
                const int64_t p = wlo + kk;
                lg = sWlog[kk];
                rv = p == t ? vg : ringV + wslot(kk) * DV;
            } else if (kk < nkeys) {
                const int r = kk - nw;
                if (cache_row_exact(r)) {
                    lg = sLogit[r];
                    rv = r < lam ? cV + (int64_t)r * DV : sEv;
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
    // reduce the RPW row groups of the wave, then the waves through LDS
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

    // ---- output ----
    {
        const bool rs = (A.read_mask & kReadState) != 0;   // hidden state: no linear terms
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

    // ---- state write-back ----
#pragma unroll
    for (int i = 0; i < IT; ++i)
        *reinterpret_cast<float4*>(Hg + (16 * w + c) * D + 16 * i + 4 * g) =
            make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
    for (int f = tid; f < D; f += NT) sg[f] = sS[f];
    if (e_slot >= 0) {
        for (int d = tid; d < DK; d += NT) cK[(int64_t)e_slot * DK + d] = sEk[d];
        for (int d = tid; d < DV; d += NT) cV[(int64_t)e_slot * DV + d] = sEv[d];
        if (tid == 0) cpos[e_slot] = (int)e_pos;
    }
    if (eta > 0) {
        const int slot = (int)(t % eta);
        for (int d = tid; d < DK; d += NT) ringK[(int64_t)slot * DK + d] = kg[d];
        for (int d = tid; d < DV; d += NT) ringV[(int64_t)slot * DV + d] = vg[d];
    }
    if (A.folded_pos && tid == 0) {
        int fp = -1;
        if (f_row == lam) fp = (int)e_pos;
        else if (f_row >= 0) fp = sCpos[f_row];
        A.folded_pos[bh] = fp;
    }
}

// Empties the state: H = 0, s = 0, cache_pos = -1 (plain fill kernels, no memset nodes).
__global__ __launch_bounds__(256) void init_kernel(InitArgs A) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t nh = (int64_t)A.BH * A.D * A.d_v, ns = (int64_t)A.BH * A.D, nc = (int64_t)A.BH * A.lam;
    if (i < nh) A.H[i] = 0.f;
    if (i < ns) A.s[i] = 0.f;
    if (i < nc) A.cache_pos[i] = -1;
    if (A.cache_score && i < nc) A.cache_score[i] = 0.f;
    if (A.win_score && i < (int64_t)A.BH * A.eta) A.win_score[i] = 0.f;
}

}  // namespace

template <typename T, int DK, int PHI>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
    const size_t lds = dec_lds<T, DK, PHI>(a.lam, a.eta).total;
    auto kern = decode_kernel<T, DK, PHI>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(a.BH), dim3(DecCfg<T, DK, PHI>::NT), lds, stream, a);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, int d, int phi_kind, hipStream_t stream) {
    if (dtype == 0) {
        if (d == 64) return phi_kind ? launch_decode_t<float, 64, 1>(a, stream) : launch_decode_t<float, 64, 0>(a, stream);
        return phi_kind ? launch_decode_t<float, 128, 1>(a, stream) : launch_decode_t<float, 128, 0>(a, stream);
    }
    if (d == 64) return phi_kind ? launch_decode_t<bf16, 64, 1>(a, stream) : launch_decode_t<bf16, 64, 0>(a, stream);
    return phi_kind ? launch_decode_t<bf16, 128, 1>(a, stream) : launch_decode_t<bf16, 128, 0>(a, stream);
}

size_t decode_lds_bytes(int d, int phi_kind, int esz, int lam) {
    // eta only sizes a small logits array; callers add its bytes separately
    if (esz == 4) {
        if (d == 64) return phi_kind ? dec_lds<float, 64, 1>(lam, 0).total : dec_lds<float, 64, 0>(lam, 0).total;
        return phi_kind ? dec_lds<float, 128, 1>(lam, 0).total : dec_lds<float, 128, 0>(lam, 0).total;
    }
    if (d == 64) return phi_kind ? dec_lds<bf16, 64, 1>(lam, 0).total : dec_lds<bf16, 64, 0>(lam, 0).total;
    return phi_kind ? dec_lds<bf16, 128, 1>(lam, 0).total : dec_lds<bf16, 128, 0>(lam, 0).total;
}

hipError_t launch_init(const InitArgs& a, hipStream_t stream) {
    const int64_t total = (int64_t)a.BH * a.D * a.d_v;
    int64_t mx = total > (int64_t)a.BH * a.lam ? total : (int64_t)a.BH * a.lam;
    if (a.win_score && (int64_t)a.BH * a.eta > mx) mx = (int64_t)a.BH * a.eta;
    const unsigned blocks = (unsigned)((mx + 255) / 256);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(init_kernel, dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lola
