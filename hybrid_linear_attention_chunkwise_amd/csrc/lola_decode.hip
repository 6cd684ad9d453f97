// Decode step: one workgroup per (sequence, head), one token.  LoLA notes 2.4 (single-token update:
// the token leaving the window joins the cache as a candidate, SRE against the state before the
// update, fold the lowest) followed by Eq. (14) of 2.5.
//
// Memory-bound: every step streams H (read + write), the window ring and the cache.  H is staged once
// in LDS (fp32) and serves the SRE numerators (MFMA, candidates as columns), the fold (rank-1 update)
// and the linear read-out; candidate features come from the cached keys through the same phi tile as
// the prefill path.  Logits of the cache members are produced in the candidate pass, so cache keys
// are read once.
#include "lola_common.hpp"
#include "lola_internal.hpp"

namespace lola {

namespace {

__host__ __device__ inline size_t al16d(size_t x) { return (x + 15) & ~size_t(15); }

struct DecLds {
    size_t ht, wt, s, q, ek, ev, phiq, phif, pre, cpos, sre, logit, wlogit, red, o, total;
};

template <typename T, int DK, int PHI>
__host__ __device__ inline DecLds dec_lds(int lam, int eta) {
    constexpr int D = kFeat, DV = DK, DW = (PHI == kPhiSoftmaxPM) ? D / 2 : D;
    DecLds o;
    size_t p = 0;
    o.ht = p;     p = al16d(p + sizeof(float) * DV * (D + 4));
    o.wt = p;     p = al16d(p + sizeof(T) * DW * (DK + 4));
    o.s = p;      p = al16d(p + sizeof(float) * D);
    o.q = p;      p = al16d(p + sizeof(float) * DK);
    o.ek = p;     p = al16d(p + sizeof(T) * DK);
    o.ev = p;     p = al16d(p + sizeof(T) * DV);
    o.phiq = p;   p = al16d(p + sizeof(float) * D);
    o.phif = p;   p = al16d(p + sizeof(float) * D);
    o.pre = p;    p = al16d(p + sizeof(float) * 2 * DW);
    o.cpos = p;   p = al16d(p + sizeof(int) * (lam + 1));
    o.sre = p;    p = al16d(p + sizeof(float) * (lam + 16));
    o.logit = p;  p = al16d(p + sizeof(float) * (lam + 16));
    o.wlogit = p; p = al16d(p + sizeof(float) * (eta + 16));
    o.red = p;    p = al16d(p + sizeof(unsigned long long) * 16);
    o.o = p;      p = al16d(p + sizeof(float) * 4 * DV);
    o.total = p;
    return o;
}

__device__ __forceinline__ unsigned long long keep_key_d(float sre, int pos) {
    return ((unsigned long long)__float_as_uint(sre) << 32) | (unsigned long long)(0xFFFFFFFFu - (unsigned)pos);
}

template <typename T, int DK, int PHI>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs A) {
    constexpr int D = kFeat, DV = DK, JT = DV / 16;
    constexpr int DW = (PHI == kPhiSoftmaxPM) ? D / 2 : D;
    constexpr int HT_LD = D + 4, WT_LD = DK + 4;
    extern __shared__ __align__(16) char smem[];
    const int lam = A.lam, eta = A.eta;
    const DecLds lo = dec_lds<T, DK, PHI>(lam, eta);
    float* sHT = reinterpret_cast<float*>(smem + lo.ht);
    T* wt = reinterpret_cast<T*>(smem + lo.wt);
    float* sS = reinterpret_cast<float*>(smem + lo.s);
    float* sQ = reinterpret_cast<float*>(smem + lo.q);
    T* sEk = reinterpret_cast<T*>(smem + lo.ek);
    T* sEv = reinterpret_cast<T*>(smem + lo.ev);
    float* sPhiQ = reinterpret_cast<float*>(smem + lo.phiq);
    float* sPhiF = reinterpret_cast<float*>(smem + lo.phif);
    float* sPre = reinterpret_cast<float*>(smem + lo.pre);
    int* sCpos = reinterpret_cast<int*>(smem + lo.cpos);
    float* sSre = reinterpret_cast<float*>(smem + lo.sre);
    float* sLogit = reinterpret_cast<float*>(smem + lo.logit);
    float* sWLogit = reinterpret_cast<float*>(smem + lo.wlogit);
    unsigned long long* sRed = reinterpret_cast<unsigned long long*>(smem + lo.red);
    float* sO = reinterpret_cast<float*>(smem + lo.o);

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

    // ---- stage state and inputs ----
    for (int i = tid; i < DV * D / 4; i += 256) {
        const int d = (4 * i) / D, f = 4 * i - d * D;
        const float4 h = *reinterpret_cast<const float4*>(Hg + 4 * i);
        *reinterpret_cast<float4*>(sHT + d * HT_LD + f) = h;
    }
    stage_wt<T>(wt, WT_LD, A.W, DK, DW);
    for (int d = tid; d < D; d += 256) sS[d] = sg[d];
    for (int d = tid; d < DK; d += 256) {
        sQ[d] = to_f(qg[d]);
        sEk[d] = has_e ? ekg[d] : from_f<T>(0.f);
    }
    for (int d = tid; d < DV; d += 256) sEv[d] = has_e ? evg[d] : from_f<T>(0.f);
    for (int j = tid; j < lam; j += 256) sCpos[j] = cpos[j];
    if (tid == 0) { sRed[0] = 0; sRed[1] = ~0ull; sRed[2] = ~0ull; }
    __syncthreads();
    for (int j = tid; j < lam; j += 256) {
        if (sCpos[j] >= 0) atomicAdd(reinterpret_cast<unsigned long long*>(&sRed[0]), 1ull);
        else atomicMin(&sRed[2], (unsigned long long)j);
    }
    __syncthreads();
    const int nG = (int)sRed[0];
    const int first_empty = sRed[2] == ~0ull ? -1 : (int)sRed[2];
    const bool scoring = has_e && lam > 0 && nG >= lam;

    // ---- candidate pass: cache slots (rows 0..lam-1) and the leaving token (row lam) ----
    // logits for every candidate; SRE only when the cache overflows.
    const int nrow = lam + 1;
    for (int tile = w; tile * 16 < nrow; tile += 4) {
        const int row = tile * 16 + c;
        bool valid;
        const T* rk;
        const T* rv;
        if (row < lam) { valid = sCpos[row] >= 0; rk = cK + (int64_t)row * DK; rv = cV + (int64_t)row * DV; }
        else { valid = (row == lam) && has_e; rk = sEk; rv = sEv; }
        Frag8<T> kf[DK / 32];
        float lg = 0.f;
#pragma unroll
        for (int ss = 0; ss < DK / 32; ++ss) {
            kf[ss] = valid ? load_frag(rk, ss, g) : frag_zero<T>();
#pragma unroll
            for (int e = 0; e < 8; ++e) lg += frag_get(kf[ss], e) * sQ[32 * ss + 16 * (e >> 2) + 4 * g + (e & 3)];
        }
        lg = sum_groups(lg) * scale;
        if (scoring) {
            float ph[D / 16][4];
            phi_tile<T, DK, PHI>(wt, WT_LD, kf, ph);
            float den = 0.f;
#pragma unroll
            for (int ft = 0; ft < D / 16; ++ft)
#pragma unroll
                for (int r = 0; r < 4; ++r) den += ph[ft][r] * sS[16 * ft + 4 * g + r];
            den = sum_groups(den);
            f4 num[JT];
#pragma unroll
            for (int J = 0; J < JT; ++J) num[J] = zero4();
#pragma unroll
            for (int ss = 0; ss < D / 32; ++ss) {
                const Frag8<T> bf = frag_from_acc<T>(f4{ph[2 * ss][0], ph[2 * ss][1], ph[2 * ss][2], ph[2 * ss][3]},
                                                     f4{ph[2 * ss + 1][0], ph[2 * ss + 1][1], ph[2 * ss + 1][2], ph[2 * ss + 1][3]});
#pragma unroll
                for (int J = 0; J < JT; ++J) mma32(num[J], load_frag_cvt<T>(sHT + (16 * J + c) * HT_LD, ss, g), bf);
            }
            const float inv = den != 0.f ? 1.f / den : 0.f;
            float sq = 0.f;
#pragma unroll
            for (int J = 0; J < JT; ++J)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float vv = valid ? to_f(rv[16 * J + 4 * g + r]) : 0.f;
                    const float x = num[J][r] * inv - vv;
                    sq += x * x;
                }
            sq = sum_groups(sq);
            if (g == 0 && row <= lam) sSre[row] = sqrtf(sq);
        }
        if (g == 0 && row <= lam) sLogit[row] = lg;
    }
    __syncthreads();

    // ---- allocation: which candidate is folded (row), and where the leaving token goes (slot) ----
    int f_row = -1;          // row folded into (H, s): 0..lam-1 a cache slot, lam the leaving token
    int e_slot = -1;         // slot that receives the leaving token
    if (scoring) {
        unsigned long long best = ~0ull;
        for (int r = tid; r < nrow; r += 256) {
            const bool valid = r < lam ? sCpos[r] >= 0 : has_e;
            if (!valid) continue;
            const int pos = r < lam ? sCpos[r] : (int)e_pos;
            const unsigned long long k = keep_key_d(sSre[r], pos);
            best = k < best ? k : best;
        }
        atomicMin(&sRed[1], best);
        __syncthreads();
        const unsigned long long kmin = sRed[1];
        // the position in the low word identifies the row
        const int fpos = (int)(0xFFFFFFFFu - (unsigned)(kmin & 0xFFFFFFFFull));
        if (fpos == (int)e_pos) f_row = lam;
        else {
            for (int r = 0; r < lam; ++r)
                if (sCpos[r] == fpos) { f_row = r; break; }
        }
        if (f_row < lam) e_slot = f_row;
    } else if (has_e) {
        if (lam == 0) f_row = lam;
        else e_slot = first_empty;
    }

    // ---- features of the query and of the folded token (VALU; W^T in LDS) ----
    {
        const T* kf = nullptr;
        if (f_row >= 0) kf = f_row < lam ? cK + (int64_t)f_row * DK : sEk;
        for (int i = tid; i < 2 * DW; i += 256) {
            const int which = i / DW, j = i - which * DW;
            float z = 0.f;
            if (which == 0) {
                for (int d = 0; d < DK; ++d) z += sQ[d] * to_f(wt[j * WT_LD + d]);
            } else if (kf) {
                for (int d = 0; d < DK; ++d) z += to_f(kf[d]) * to_f(wt[j * WT_LD + d]);
            }
            sPre[i] = z;
        }
    }
    __syncthreads();
    if (w < 2) {
        // wave 0: query, wave 1: folded token
        float* outp = w == 0 ? sPhiQ : sPhiF;
        const float* pre = sPre + w * DW;
        if (PHI == kPhiSoftmaxPM) {
            float mx = -INFINITY, mn = INFINITY;
            for (int j = l; j < DW; j += 64) { mx = fmaxf(mx, pre[j]); mn = fminf(mn, pre[j]); }
            for (int o = 32; o > 0; o >>= 1) { mx = fmaxf(mx, __shfl_xor(mx, o)); mn = fminf(mn, __shfl_xor(mn, o)); }
            float sp = 0.f, sm = 0.f;
            for (int j = l; j < DW; j += 64) { sp += fast_exp(pre[j] - mx); sm += fast_exp(mn - pre[j]); }
            for (int o = 32; o > 0; o >>= 1) { sp += __shfl_xor(sp, o); sm += __shfl_xor(sm, o); }
            for (int j = l; j < DW; j += 64) {
                outp[j] = fast_exp(pre[j] - mx) / sp;
                outp[DW + j] = fast_exp(mn - pre[j]) / sm;
            }
        } else {
            for (int j = l; j < DW; j += 64) { const float z = pre[j]; outp[j] = z > 0.f ? z + 1.f : fast_exp(z); }
        }
    }
    __syncthreads();

    // ---- fold (rank-1 update of H and s) ----
    if (f_row >= 0) {
        const T* vf = f_row < lam ? cV + (int64_t)f_row * DV : sEv;
        for (int i = tid; i < DV * D; i += 256) {
            const int d = i / D, f = i - d * D;
            sHT[d * HT_LD + f] += to_f(vf[d]) * sPhiF[f];
        }
        for (int f = tid; f < D; f += 256) sS[f] += sPhiF[f];
    }
    __syncthreads();

    // ---- read-out ----
    // window logits: positions max(0, t-eta+1) .. t-1 from the ring, t from the input
    const int64_t wlo = max((int64_t)0, t - eta + 1);
    const int nw = eta > 0 ? (int)(t - wlo + 1) : 0;
    for (int tile = w; tile * 16 < nw; tile += 4) {
        const int i = tile * 16 + c;
        const bool valid = i < nw;
        const int64_t p = wlo + i;
        const T* rk = valid ? (p == t ? kg : ringK + (p % eta) * DK) : nullptr;
        float lg = 0.f;
#pragma unroll
        for (int ss = 0; ss < DK / 32; ++ss) {
            const Frag8<T> kf = valid ? load_frag(rk, ss, g) : frag_zero<T>();
#pragma unroll
            for (int e = 0; e < 8; ++e) lg += frag_get(kf, e) * sQ[32 * ss + 16 * (e >> 2) + 4 * g + (e & 3)];
        }
        lg = sum_groups(lg) * scale;
        if (g == 0 && valid) sWLogit[i] = lg;
    }
    __syncthreads();
    // exact set: window + cache after the allocation (occupied slots except a folded one, plus the
    // leaving token unless it was folded)
    auto cache_row_exact = [&](int r) -> bool {
        if (r < lam) return sCpos[r] >= 0 && r != f_row;
        return has_e && f_row != lam && lam > 0;
    };
    float mloc = -INFINITY;
    for (int i = tid; i < nw; i += 256) mloc = fmaxf(mloc, sWLogit[i]);
    for (int r = tid; r < nrow; r += 256)
        if (cache_row_exact(r)) mloc = fmaxf(mloc, sLogit[r]);
    for (int o = 32; o > 0; o >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o));
    float* sRedF = reinterpret_cast<float*>(sRed + 4);
    if (l == 0) sRedF[w] = mloc;
    __syncthreads();
    const float m = fmaxf(fmaxf(sRedF[0], sRedF[1]), fmaxf(sRedF[2], sRedF[3]));
    // weighted values: wave w takes keys w, w+4, ...; lane handles value columns l, l+64
    float o0 = 0.f, o1 = 0.f, lsum = 0.f;
    const int nkeys = nw + nrow;
    for (int i = w; i < nkeys; i += 4) {
        float lg;
        const T* rv;
        if (i < nw) {
            const int64_t p = wlo + i;
            lg = sWLogit[i];
            rv = p == t ? vg : ringV + (p % eta) * DV;
        } else {
            const int r = i - nw;
            if (!cache_row_exact(r)) continue;
            lg = sLogit[r];
            rv = r < lam ? cV + (int64_t)r * DV : sEv;
        }
        const float p = fast_exp(lg - m);
        lsum += p;
        o0 += p * to_f(rv[l]);
        if (DV > 64) o1 += p * to_f(rv[l + 64]);
    }
    sO[w * DV + l] = o0;
    if (DV > 64) sO[w * DV + l + 64] = o1;
    if (l == 0) sRedF[4 + w] = lsum;
    __syncthreads();
    // linear part and output
    {
        const float lsum_all = sRedF[4] + sRedF[5] + sRedF[6] + sRedF[7];
        // L[d] = sum_f H^T[d][f] phi_q[f]; threads pair up on one row d
        const int d = tid >> 1, half = tid & 1;
        float Ld = 0.f;
        if (d < DV)
            for (int f = half * (D / 2); f < (half + 1) * (D / 2); ++f) Ld += sHT[d * HT_LD + f] * sPhiQ[f];
        Ld += __shfl_xor(Ld, 1);
        float lden = 0.f;
        for (int f = 0; f < D; ++f) lden += sPhiQ[f] * sS[f];
        if (d < DV && half == 0) {
            const float Od = sO[d] + sO[DV + d] + sO[2 * DV + d] + sO[3 * DV + d];
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
    __syncthreads();

    // ---- state write-back ----
    for (int i = tid; i < DV * D / 4; i += 256) {
        const int d = (4 * i) / D, f = 4 * i - d * D;
        *reinterpret_cast<float4*>(Hg + 4 * i) = *reinterpret_cast<const float4*>(sHT + d * HT_LD + f);
    }
    for (int f = tid; f < D; f += 256) sg[f] = sS[f];
    if (e_slot >= 0) {
        for (int d = tid; d < DK; d += 256) cK[(int64_t)e_slot * DK + d] = sEk[d];
        for (int d = tid; d < DV; d += 256) cV[(int64_t)e_slot * DV + d] = sEv[d];
        if (tid == 0) cpos[e_slot] = (int)e_pos;
    }
    if (eta > 0) {
        const int slot = (int)(t % eta);
        for (int d = tid; d < DK; d += 256) ringK[(int64_t)slot * DK + d] = kg[d];
        for (int d = tid; d < DV; d += 256) ringV[(int64_t)slot * DV + d] = vg[d];
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
}

}  // namespace

template <typename T, int DK, int PHI>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
    const size_t lds = dec_lds<T, DK, PHI>(a.lam, a.eta).total;
    auto kern = decode_kernel<T, DK, PHI>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(a.BH), dim3(256), lds, stream, a);
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
    const int64_t mx = total > (int64_t)a.BH * a.lam ? total : (int64_t)a.BH * a.lam;
    const unsigned blocks = (unsigned)((mx + 255) / 256);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(init_kernel, dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lola
