// Decode step, register-resident path for bf16 storage: the same step as decode_kernel (LoLA notes
// 2.4 single-token update, then Eq. (14) of 2.5), organised for memory-level parallelism.
//
// One workgroup per (sequence, head); a wave per 16 value rows of H^T.  Every global load of the step
// is issued at the start: the wave's H^T rows (fp32, kept for the fold, the linear read-out and the
// write-back), its window-key tiles and its candidate tiles (keys and values of up to MT tiles of 16
// cache slots / the leaving token).  Nothing is loaded twice: the candidates' values, held in
// accumulator order for their squared errors, are the same registers the exact numerator is formed
// from, and the folded candidate's features are recomputed from the keys its wave still holds.  The
// window values are fetched once the window keys have been used, while the allocation runs.
//
// Logits come from MFMA with the query as row 0 of the A operand; features through W^T as in the
// other kernels; the SRE numerators H^T phi(k) from the bf16 H^T copy in LDS.  Keys, the query and
// W^T use the contiguous fragment order (one 16-byte load per lane and super-step).
#include "lola_common.hpp"
#include "lola_internal.hpp"

namespace lola {

namespace {

__host__ __device__ constexpr size_t al16f(size_t x) { return (x + 15) & ~size_t(15); }

template <int DK, int PHI>
struct FastCfg {
    static constexpr int D = kFeat, DV = DK;
    static constexpr int DW = (PHI == kPhiSoftmaxPM) ? D / 2 : D;
    static constexpr int NW = DV / 16, NT = 64 * NW, WT_LD = DK + 8, JT = DV / 16;   // 16-byte rows
    static constexpr int MT = 3;                              // candidate tiles per wave
    static constexpr int MW = 2;                              // window-key tiles per wave
    static constexpr int LPR = DV / 8;                        // lanes per value row (8 bf16 each)
    static constexpr int RPW = 64 / LPR;                      // value rows per wave instruction
    static constexpr int MAXW = MW * 16 * NW;                 // window keys the path holds
    static constexpr int UW = MAXW / (NW * RPW);              // value rows per lane
    static constexpr int MAXC = MT * 16 * NW;                 // candidate rows the path holds
};

struct FastLds {
    size_t hb, wt, s, phiq, phif, vf, ek, ev, cpos, sre, logit, wlog, red, o, oc, lrow, total;
};

template <int DK, int PHI>
__host__ __device__ constexpr FastLds fast_lds() {
    using Cfg = FastCfg<DK, PHI>;
    constexpr int D = Cfg::D, DV = Cfg::DV;
    FastLds o{};
    size_t p = 0;
    o.hb = p;     p = al16f(p + sizeof(bf16) * DV * D);             // H^T in fragment order
    o.wt = p;     p = al16f(p + sizeof(bf16) * Cfg::DW * Cfg::WT_LD);
    o.s = p;      p = al16f(p + sizeof(float) * D);
    o.phiq = p;   p = al16f(p + sizeof(float) * D);
    o.phif = p;   p = al16f(p + sizeof(float) * D);
    o.vf = p;     p = al16f(p + sizeof(float) * DV);
    o.ek = p;     p = al16f(p + sizeof(bf16) * DK);
    o.ev = p;     p = al16f(p + sizeof(bf16) * DV);
    o.cpos = p;   p = al16f(p + sizeof(int) * Cfg::MAXC);
    o.sre = p;    p = al16f(p + sizeof(float) * Cfg::MAXC);
    o.logit = p;  p = al16f(p + sizeof(float) * Cfg::MAXC);
    o.wlog = p;   p = al16f(p + sizeof(float) * Cfg::MAXW);
    o.red = p;    p = al16f(p + sizeof(unsigned long long) * 32);
    o.o = p;      p = al16f(p + sizeof(float) * Cfg::NW * DV);
    o.oc = p;     p = al16f(p + sizeof(float) * Cfg::NW * DV);
    o.lrow = p;   p = al16f(p + sizeof(float) * DV);
    o.total = p;
    return o;
}

__device__ __forceinline__ unsigned long long fkey(float sre, int pos) {
    return ((unsigned long long)__float_as_uint(sre) << 32) | (unsigned long long)(0xFFFFFFFFu - (unsigned)pos);
}

template <int DK, int PHI>
__global__ __launch_bounds__(4 * DK) void decode_fast_kernel(DecodeArgs A) {
    using T = bf16;
    using Cfg = FastCfg<DK, PHI>;
    constexpr int D = Cfg::D, DV = Cfg::DV, DW = Cfg::DW, NW = Cfg::NW, NT = Cfg::NT, WT_LD = Cfg::WT_LD,
                  JT = Cfg::JT, IT = D / 16, MT = Cfg::MT, MW = Cfg::MW, LPR = Cfg::LPR, RPW = Cfg::RPW,
                  UW = Cfg::UW;
    extern __shared__ __align__(16) char smem[];
    const int lam = A.lam, eta = A.eta;
    constexpr FastLds lo = fast_lds<DK, PHI>();
    T* sHb = reinterpret_cast<T*>(smem + lo.hb);
    T* wt = reinterpret_cast<T*>(smem + lo.wt);
    float* sS = reinterpret_cast<float*>(smem + lo.s);
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
    float* sOc = reinterpret_cast<float*>(smem + lo.oc);
    float* sL = reinterpret_cast<float*>(smem + lo.lrow);
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
    const int eslot = eta > 0 ? (int)(t % eta) : 0;
    const T* ekg = eta == 0 ? kg : (has_e ? ringK + (int64_t)eslot * DK : kg);
    const T* evg = eta == 0 ? vg : (has_e ? ringV + (int64_t)eslot * DV : vg);
    // the window of query t: positions wlo .. t (t itself from the input)
    const int64_t wlo = max((int64_t)0, t - eta + 1);
    const int nw = eta > 0 ? (int)(t - wlo + 1) : 0;
    const int wslot0 = eta > 0 ? (int)(wlo % eta) : 0;
    auto wrow = [&](int i, const T* ring, const T* cur, int ld) -> const T* {
        if (i >= nw) return cur;                              // no key: any valid row, never used
        if (wlo + i == t) return cur;
        const int sl = wslot0 + i >= eta ? wslot0 + i - eta : wslot0 + i;
        return ring + (int64_t)sl * ld;
    };
    const int ntw = (nw + 15) >> 4;                           // window-key tiles
    const int ntc = (lam + 16) >> 4;                          // candidate tiles: rows 0..lam
    // candidate tile of (wave, group u): the last group runs over the waves backwards, so a wave that
    // gets a last-group tile is not wave 0, which computes the query's features
    auto ctile = [&](int ww, int u) { return u < MT - 1 ? ww + NW * u : NW * u + (NW - 1 - ww); };

    // ---------------- every load of the step ----------------
    // First H^T and the small operands, whose LDS copies are the only stores that wait on memory;
    // then the key and candidate tiles, which stay in flight through the barrier and are consumed
    // in the order they were issued.
    constexpr int WPT = DK * DW / 4 / NT;                     // float4 pieces of W per thread
    static_assert(DK * DW / 4 % NT == 0 && 2 * NT >= Cfg::MAXC && NT >= D, "thread coverage");
    f4 acc[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const float4 h = *reinterpret_cast<const float4*>(Hg + (16 * w + c) * D + 16 * i + 4 * g);
        acc[i] = f4{h.x, h.y, h.z, h.w};
    }
    // every workgroup reads all of W at the same moment: start each one at a different piece so the
    // requests spread over the cache channels instead of queueing on the same lines
    float4 wreg[WPT];
    const int wrot = (bh * 97) & (NT * WPT - 1);
#pragma unroll
    for (int u = 0; u < WPT; ++u) wreg[u] = reinterpret_cast<const float4*>(A.W)[(tid + NT * u + wrot) & (NT * WPT - 1)];
    const float s_in = tid < D ? sg[tid] : 0.f;
    const int cp_in = tid < lam ? cpos[tid] : -1;
    const int cp_in2 = tid + NT < lam ? cpos[tid + NT] : -1;
    T ek_in = from_f<T>(0.f), ev_in = from_f<T>(0.f);
    if (has_e && tid < DK) ek_in = ekg[tid];
    if (has_e && tid < DV) ev_in = evg[tid];
    static_assert((NT * WPT & (NT * WPT - 1)) == 0, "W pieces: a power of two");
#pragma unroll
    for (int u = 0; u < WPT; ++u) {
        const int i = 4 * ((tid + NT * u + wrot) & (NT * WPT - 1)), d = i / DW, j = i - d * DW;
        wt[(j + 0) * WT_LD + d] = from_f<T>(wreg[u].x);
        wt[(j + 1) * WT_LD + d] = from_f<T>(wreg[u].y);
        wt[(j + 2) * WT_LD + d] = from_f<T>(wreg[u].z);
        wt[(j + 3) * WT_LD + d] = from_f<T>(wreg[u].w);
    }
    if (tid < D) sS[tid] = s_in;
    if (tid < lam) sCpos[tid] = cp_in;
    if (tid + NT < lam) sCpos[tid + NT] = cp_in2;
    if (tid < DK) sEk[tid] = ek_in;
    if (tid < DV) sEv[tid] = ev_in;
    if (tid == 0) sRed[1] = ~0ull;
#pragma unroll
    for (int ss = 0; ss < D / 32; ++ss)
        *reinterpret_cast<Frag8<T>*>(sHb + ((w * (D / 32) + ss) * 64 + l) * 8) =
            frag_from_acc<T>(acc[2 * ss], acc[2 * ss + 1]);
    __builtin_amdgcn_sched_barrier(0);                        // the tile loads stay below
    // the query, as row 0 of an A operand (and column 0 of a B operand: the same registers)
    Frag8<T> qa[DK / 32];
#pragma unroll
    for (int ss = 0; ss < DK / 32; ++ss) qa[ss] = c == 0 ? load_frag_contig(qg, ss, g) : frag_zero<T>();
    Frag8<T> wk[MW][DK / 32];
#pragma unroll
    for (int u = 0; u < MW; ++u) {
        const T* rk = wrow(16 * (w + NW * u) + c, ringK, kg, DK);
#pragma unroll
        for (int ss = 0; ss < DK / 32; ++ss) wk[u][ss] = load_frag_contig(rk, ss, g);
    }
    Frag8<T> ck[MT][DK / 32];
    bf16x4 cv[MT][JT];
#pragma unroll
    for (int u = 0; u < MT; ++u) {
        const int r = 16 * ctile(w, u) + c;
        const T* rk = kg;
        const T* rv = vg;
        if (r < lam) { rk = cK + (int64_t)r * DK; rv = cV + (int64_t)r * DV; }
        else if (r == lam) { rk = ekg; rv = evg; }
#pragma unroll
        for (int ss = 0; ss < DK / 32; ++ss) ck[u][ss] = load_frag_contig(rk, ss, g);
#pragma unroll
        for (int J = 0; J < JT; ++J) cv[u][J] = *reinterpret_cast<const bf16x4*>(rv + 16 * J + 4 * g);
    }
    __syncthreads();

    // ---------------- logits (query in row 0; lane (0, c) holds column c) ----------------
#pragma unroll
    for (int u = 0; u < MW; ++u) {
        const int j = w + NW * u;
        if (j < ntw) {
            f4 st = zero4();
#pragma unroll
            for (int ss = 0; ss < DK / 32; ++ss) mma32(st, qa[ss], wk[u][ss]);
            if (g == 0 && 16 * j + c < nw) sWlog[16 * j + c] = st[0] * scale;
        }
    }
#pragma unroll
    for (int u = 0; u < MT; ++u) {
        const int j = ctile(w, u);
        if (j < ntc) {
            f4 st = zero4();
#pragma unroll
            for (int ss = 0; ss < DK / 32; ++ss) mma32(st, qa[ss], ck[u][ss]);
            if (g == 0) sLogit[16 * j + c] = st[0] * scale;
        }
    }
    // occupied slots and the first empty one, by wave ballots (the same answer in every wave)
    int nG = 0, first_empty = -1;
    for (int k = 0; k * 64 < lam; ++k) {
        const int j = k * 64 + l;
        const unsigned long long occ = __ballot(j < lam && sCpos[j] >= 0);
        const unsigned long long emp = __ballot(j < lam && sCpos[j] < 0);
        nG += __popcll(occ);
        if (first_empty < 0 && emp) first_empty = k * 64 + __ffsll((long long)emp) - 1;
    }
    const bool scoring = has_e && lam > 0 && nG >= lam;
    // features of the query: wave 0 (no last-group candidate tile)
    if (w == 0) {
        float ph[D / 16][4];
        phi_tile<T, DK, PHI, true>(wt, WT_LD, qa, ph);
        if (c == 0)
#pragma unroll
            for (int ft = 0; ft < D / 16; ++ft)
#pragma unroll
                for (int r = 0; r < 4; ++r) sPhiQ[16 * ft + 4 * g + r] = ph[ft][r];
    }

    // ---------------- SRE of the candidates against the state before the update ----------------
    if (scoring) {
#pragma unroll
        for (int u = 0; u < MT; ++u) {
            const int j = ctile(w, u);
            if (j >= ntc) continue;
            float ph[D / 16][4];
            phi_tile<T, DK, PHI, true>(wt, WT_LD, ck[u], ph);
            float den = 0.f;
#pragma unroll
            for (int ft = 0; ft < D / 16; ++ft) {
                const f4 sv = *reinterpret_cast<const f4*>(sS + 16 * ft + 4 * g);
#pragma unroll
                for (int r = 0; r < 4; ++r) den += ph[ft][r] * sv[r];
            }
            den = sum_groups(den);
            const float inv = den != 0.f ? fast_rcp(den) : 0.f;   // empty state: recall 0
            Frag8<T> pf[D / 32];
#pragma unroll
            for (int ss = 0; ss < D / 32; ++ss)
                pf[ss] = frag_from_acc<T>(f4{ph[2 * ss][0], ph[2 * ss][1], ph[2 * ss][2], ph[2 * ss][3]},
                                          f4{ph[2 * ss + 1][0], ph[2 * ss + 1][1], ph[2 * ss + 1][2], ph[2 * ss + 1][3]});
            float sq = 0.f;
#pragma unroll
            for (int J = 0; J < JT; ++J) {
                f4 num = zero4();
#pragma unroll
                for (int ss = 0; ss < D / 32; ++ss)
                    mma32(num, *reinterpret_cast<const Frag8<T>*>(sHb + ((J * (D / 32) + ss) * 64 + l) * 8), pf[ss]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float x = num[r] * inv - to_f(cv[u][J][r]);
                    sq += x * x;
                }
            }
            sq = sum_groups(sq);
            if (g == 0) sSre[16 * j + c] = __builtin_amdgcn_sqrtf(sq);
        }
    }
    __syncthreads();

    // window values: fetched now, used after the allocation.  Row kk of the window for lane group
    // (w, sub): kk = RPW * (w + NW * u) + sub; 16-byte pieces, LPR lanes per row
    const int sub = l / LPR, col = (l % LPR) * 8;
    uint4 wvr[UW];
#pragma unroll
    for (int u = 0; u < UW; ++u) {
        const int kk = RPW * (w + NW * u) + sub;
        wvr[u] = *reinterpret_cast<const uint4*>(wrow(kk, ringV, vg, DV) + col);
    }
    // ---------------- allocation: the lowest SRE is folded (ties: the newer position) ----------------
    int f_row = -1;          // folded row: 0..lam-1 a cache slot, lam the leaving token
    int e_slot = -1;         // slot that receives the leaving token
    if (scoring) {
        unsigned long long best = ~0ull;
        for (int r = tid; r <= lam; r += NT) {
            const bool valid = r < lam ? sCpos[r] >= 0 : true;
            if (!valid) continue;
            const int pos = r < lam ? sCpos[r] : (int)e_pos;
            const unsigned long long k = fkey(sSre[r], pos);
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

    // ---------------- fold: the folded candidate's features from the keys its wave holds ----------------
    if (f_row >= 0) {
        const int jf = f_row >> 4, cf = f_row & 15;
        const int uf = jf / NW < MT - 1 ? jf / NW : MT - 1;
        const int wf = uf < MT - 1 ? jf % NW : NW - 1 - (jf - NW * (MT - 1));
        if (w == wf) {
#pragma unroll
            for (int u = 0; u < MT; ++u) {
                if (u != uf) continue;
                float ph[D / 16][4];
                phi_tile<T, DK, PHI, true>(wt, WT_LD, ck[u], ph);
                if (c == cf) {
#pragma unroll
                    for (int ft = 0; ft < D / 16; ++ft)
#pragma unroll
                        for (int r = 0; r < 4; ++r) sPhiF[16 * ft + 4 * g + r] = ph[ft][r];
#pragma unroll
                    for (int J = 0; J < JT; ++J)
#pragma unroll
                        for (int r = 0; r < 4; ++r) sVf[16 * J + 4 * g + r] = to_f(cv[u][J][r]);
                }
            }
        }
        __syncthreads();
        const float vd = sVf[16 * w + c];
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const f4 pf = *reinterpret_cast<const f4*>(sPhiF + 16 * i + 4 * g);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][r] += vd * pf[r];
        }
        for (int f = tid; f < D; f += NT) sS[f] += sPhiF[f];
    }

    // ---------------- exact part of Eq. (14) ----------------
    // exact keys: the window, and the cache after the allocation (the leaving token if it was kept)
    auto cand_exact = [&](int r) -> bool {
        if (!(A.read_mask & kReadSparse)) return false;   // hidden cache: no exact cache keys
        if (r < lam) return sCpos[r] >= 0 && r != f_row;
        return r == lam && has_e && f_row != lam && lam > 0;
    };
    float mloc = -INFINITY;
    for (int i = tid; i < nw; i += NT) mloc = fmaxf(mloc, sWlog[i]);
    for (int r = tid; r <= lam; r += NT)
        if (cand_exact(r)) mloc = fmaxf(mloc, sLogit[r]);
    mloc = wave_max(mloc);
    if (l == 0) sRedF[w] = mloc;
    // linear row of this wave (after the fold), and phi(q).s on wave 0
    {
        float part_ = 0.f;
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const f4 pq = *reinterpret_cast<const f4*>(sPhiQ + 16 * i + 4 * g);
#pragma unroll
            for (int r = 0; r < 4; ++r) part_ += acc[i][r] * pq[r];
        }
        part_ = sum_groups(part_);
        if (g == 0) sL[16 * w + c] = part_;
    }
    __syncthreads();
    float m = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) m = fmaxf(m, sRedF[ww]);
    const bool any = m != -INFINITY;

    // window values
    float o[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) o[x] = 0.f;
    float lsum = 0.f;
#pragma unroll
    for (int u = 0; u < UW; ++u) {
        const int kk = RPW * (w + NW * u) + sub;
        const float p = kk < nw ? fast_exp(sWlog[kk] - m) : 0.f;
        const T* e = reinterpret_cast<const T*>(&wvr[u]);
#pragma unroll
        for (int x = 0; x < 8; ++x) o[x] += p * to_f(e[x]);
        if ((l % LPR) == 0) lsum += p;
    }
    static_assert(LPR == 16 || LPR == 8, "value rows span one or two DPP rows");
#pragma unroll
    for (int x = 0; x < 8; ++x) {
        if (LPR == 8) o[x] += dpp_mov<0x128>(o[x]);          // the two rows of a 16-lane group
        o[x] = sum_groups(o[x]);
    }
    if (sub == 0)
#pragma unroll
        for (int x = 0; x < 8; ++x) sO[w * DV + col + x] = o[x];
    // cache values, from the candidate registers: lane (g, c) adds p_c v_c for its value rows
    f4 oc[JT];
#pragma unroll
    for (int J = 0; J < JT; ++J) oc[J] = zero4();
#pragma unroll
    for (int u = 0; u < MT; ++u) {
        const int j = ctile(w, u);
        if (j >= ntc) continue;
        const int r = 16 * j + c;
        if (any && cand_exact(r)) {         // (an empty slot's registers may hold anything)
            const float p = fast_exp(sLogit[r] - m);
#pragma unroll
            for (int J = 0; J < JT; ++J)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) oc[J][rr] += p * to_f(cv[u][J][rr]);
            if (g == 0) lsum += p;
        }
    }
#pragma unroll
    for (int J = 0; J < JT; ++J)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) oc[J][rr] = sum_cols_last(oc[J][rr]);
    if (c == 15)
#pragma unroll
        for (int J = 0; J < JT; ++J)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) sOc[w * DV + 16 * J + 4 * g + rr] = oc[J][rr];
    lsum = wave_sum(lsum);
    if (l == 0) sRedF[8 + w] = lsum;
    if (w == 0) {   // phi(q).s after the fold
        const float x = wave_sum(sPhiQ[l] * sS[l] + sPhiQ[l + 64] * sS[l + 64]);
        if (l == 0) sRedF[20] = x;
    }
    __syncthreads();

    // ---------------- output, joint normalisation with the common scale exp(-cm) ----------------
    if (tid < DV) {
        const int d = tid;
        const bool rs = (A.read_mask & kReadState) != 0;   // hidden state: no linear terms
        const float lden = rs ? sRedF[20] : 0.f;
        float lsum_all = 0.f, Od = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            lsum_all += sRedF[8 + ww];
            Od += sO[ww * DV + d] + sOc[ww * DV + d];
        }
        const float Ld = rs ? sL[d] : 0.f;
        float cm;
        if (lden > 0.f) cm = any ? fmaxf(m, logf(lden)) : logf(lden);
        else cm = m;
        const float sl = lden > 0.f ? fast_exp(-cm) : 0.f;
        const float se = any ? fast_exp(m - cm) : 0.f;
        const float yv = (Ld * sl + Od * se) / (lden * sl + lsum_all * se);
        reinterpret_cast<T*>(A.y)[(int64_t)bh * DV + d] = from_f<T>(yv);
    }

    // ---------------- state write-back ----------------
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
        for (int d = tid; d < DK; d += NT) ringK[(int64_t)eslot * DK + d] = kg[d];
        for (int d = tid; d < DV; d += NT) ringV[(int64_t)eslot * DV + d] = vg[d];
    }
    if (A.folded_pos && tid == 0) {
        int fp = -1;
        if (f_row == lam) fp = (int)e_pos;
        else if (f_row >= 0) fp = sCpos[f_row];
        A.folded_pos[bh] = fp;
    }
}

}  // namespace

bool decode_fast_fits(int d, int lam, int eta) {
    if (d == 128) return lam + 1 <= FastCfg<128, 1>::MAXC && eta <= FastCfg<128, 1>::MAXW;
    if (d == 64) return lam + 1 <= FastCfg<64, 1>::MAXC && eta <= FastCfg<64, 1>::MAXW;
    return false;
}

size_t decode_fast_lds_bytes(int d, int phi_kind) {
    if (d == 64) return phi_kind ? fast_lds<64, 1>().total : fast_lds<64, 0>().total;
    return phi_kind ? fast_lds<128, 1>().total : fast_lds<128, 0>().total;
}

template <int DK, int PHI>
static hipError_t launch_fast_t(const DecodeArgs& a, hipStream_t stream) {
    constexpr size_t lds = fast_lds<DK, PHI>().total;
    auto kern = decode_fast_kernel<DK, PHI>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(a.BH), dim3(FastCfg<DK, PHI>::NT), lds, stream, a);
    return hipGetLastError();
}

hipError_t launch_decode_fast(const DecodeArgs& a, int d, int phi_kind, hipStream_t stream) {
    if (d == 64) return phi_kind ? launch_fast_t<64, 1>(a, stream) : launch_fast_t<64, 0>(a, stream);
    return phi_kind ? launch_fast_t<128, 1>(a, stream) : launch_fast_t<128, 0>(a, stream);
}

}  // namespace lola
