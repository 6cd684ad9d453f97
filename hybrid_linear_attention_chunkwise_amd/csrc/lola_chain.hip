// Prefill allocation chain: one workgroup per (sequence, head) walks the chunks in order.
//
// Per chunk (LoLA notes, 2.6 Eq. (15) with 2.3 Eq. (10) and 2.4 Eqs. (11)-(13)):
//   1. snapshot (H, s) at the chunk start for the read-out kernel;
//   2. features and values of the tokens that leave the window during the chunk;
//   3. if cache + leaving tokens exceed lambda: SRE of every candidate against the chunk-start state,
//      then keep the lambda largest (ties: older position);
//   4. free the slots of folded cache members, give them to the leaving tokens that stay;
//   5. record the chunk's cache list and fold list for the read-out kernel;
//   6. fold: H += Phi_S^T V_S, s += sum Phi_S.
//
// H lives in registers for the whole call as MFMA accumulators: wave w owns the 16x16 tiles of H
// (D x d_v, feature rows, value columns) whose value columns fall in its quarter.  The SRE numerator
// Phi_E * H then uses those accumulators directly as the MFMA B operand (see lola_common.hpp), so the
// scoring pass streams candidate features only.  Each wave produces partial squared errors over its
// value columns; the four partials are summed in a fixed order, so the result is deterministic.
#include "lola_common.hpp"
#include "lola_internal.hpp"

namespace lola {

namespace {

template <typename T, int DK, int PHI>
struct ChainCfg {
    static constexpr int D = kFeat;
    static constexpr int DV = DK;
    static constexpr int DW = (PHI == kPhiSoftmaxPM) ? D / 2 : D;
    static constexpr int WT_LD = DK + 4;     // padded LDS row of W^T
    static constexpr int JT = DV / 16;       // accumulator tiles along d_v
    static constexpr int JW = JT / 4;        // per wave
    static constexpr int IT = D / 16;        // accumulator tiles along D
    static constexpr int FB = 32;            // tokens per fold batch
    static constexpr int ST_LD = FB + 4;     // padded LDS row of a staged fold batch
};

struct ChainLds {
    size_t wt, s, st_phi, st_v, slot_pos, slot_src, key, flag, a1, a2, a3, free_list, ent_slot,
        fold_row, part, tmp, total;
};

__host__ __device__ inline size_t al16(size_t x) { return (x + 15) & ~size_t(15); }

template <typename T, int DK, int PHI>
__host__ __device__ inline ChainLds chain_lds(int lam, int C) {
    using Cfg = ChainCfg<T, DK, PHI>;
    const int nr = ((lam + C + 15) / 16) * 16;
    ChainLds o;
    size_t p = 0;
    o.wt = p;        p = al16(p + sizeof(T) * Cfg::DW * Cfg::WT_LD);
    o.s = p;         p = al16(p + sizeof(float) * Cfg::D);
    o.st_phi = p;    p = al16(p + sizeof(T) * Cfg::D * Cfg::ST_LD);
    o.st_v = p;      p = al16(p + sizeof(T) * Cfg::DV * Cfg::ST_LD);
    o.slot_pos = p;  p = al16(p + sizeof(int) * (lam + 1));
    o.slot_src = p;  p = al16(p + sizeof(int) * (lam + 1));
    o.key = p;       p = al16(p + sizeof(unsigned long long) * nr);
    o.flag = p;      p = al16(p + sizeof(int) * nr);
    o.a1 = p;        p = al16(p + sizeof(int) * nr);
    o.a2 = p;        p = al16(p + sizeof(int) * (lam + 1));
    o.a3 = p;        p = al16(p + sizeof(int) * (C + 1));
    o.free_list = p; p = al16(p + sizeof(int) * (lam + 1));
    o.ent_slot = p;  p = al16(p + sizeof(int) * (C + 1));
    o.fold_row = p;  p = al16(p + sizeof(int) * (C + 1));
    o.part = p;      p = al16(p + sizeof(float) * 4 * nr);
    o.tmp = p;       p = al16(p + sizeof(int) * 16);
    o.total = p;
    return o;
}

template <typename T>
__device__ __forceinline__ void store4(T* dst, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float* dst, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
}
template <>
__device__ __forceinline__ void store4<bf16>(bf16* dst, float a, float b, float c, float d) {
    bf16x4 v;
    v[0] = (bf16)a; v[1] = (bf16)b; v[2] = (bf16)c; v[3] = (bf16)d;
    *reinterpret_cast<bf16x4*>(dst) = v;
}

// Key ordering the cache: larger = kept first.  SRE >= 0, so its bit pattern orders like the value;
// on equal SRE the older (smaller) position ranks higher.
__device__ __forceinline__ unsigned long long keep_key(float sre, int pos) {
    return ((unsigned long long)__float_as_uint(sre) << 32) | (unsigned long long)(0xFFFFFFFFu - (unsigned)pos);
}

template <typename T, int DK, int PHI>
__global__ __launch_bounds__(256) void chain_kernel(PrefillArgs A) {
    using Cfg = ChainCfg<T, DK, PHI>;
    constexpr int D = Cfg::D, DV = Cfg::DV, DW = Cfg::DW, WT_LD = Cfg::WT_LD, JW = Cfg::JW,
                  IT = Cfg::IT, FB = Cfg::FB, ST_LD = Cfg::ST_LD;
    extern __shared__ __align__(16) char smem[];
    const int lam = A.lam, eta = A.eta, n = A.n, C = A.C;
    const ChainLds lo = chain_lds<T, DK, PHI>(lam, C);
    T* wt = reinterpret_cast<T*>(smem + lo.wt);
    float* sS = reinterpret_cast<float*>(smem + lo.s);
    T* stPhi = reinterpret_cast<T*>(smem + lo.st_phi);
    T* stV = reinterpret_cast<T*>(smem + lo.st_v);
    int* slotPos = reinterpret_cast<int*>(smem + lo.slot_pos);
    int* slotSrc = reinterpret_cast<int*>(smem + lo.slot_src);
    unsigned long long* key = reinterpret_cast<unsigned long long*>(smem + lo.key);
    int* flag = reinterpret_cast<int*>(smem + lo.flag);
    int* a1 = reinterpret_cast<int*>(smem + lo.a1);
    int* a2 = reinterpret_cast<int*>(smem + lo.a2);
    int* a3 = reinterpret_cast<int*>(smem + lo.a3);
    int* freeList = reinterpret_cast<int*>(smem + lo.free_list);
    int* entSlot = reinterpret_cast<int*>(smem + lo.ent_slot);
    int* foldRow = reinterpret_cast<int*>(smem + lo.fold_row);
    float* part = reinterpret_cast<float*>(smem + lo.part);
    int* tmp = reinterpret_cast<int*>(smem + lo.tmp);

    const int bh = blockIdx.x;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c = l & 15;
    const int64_t t0 = A.t0;
    const int nrp = ((lam + C + 15) / 16) * 16;

    char* wsb = A.ws + (int64_t)bh * A.L.per_bh;
    T* candPhi = reinterpret_cast<T*>(wsb + A.L.cand_phi);
    T* candV = reinterpret_cast<T*>(wsb + A.L.cand_v);
    const T* kin = reinterpret_cast<const T*>(A.k) + (int64_t)bh * n * DK;
    const T* vin = reinterpret_cast<const T*>(A.v) + (int64_t)bh * n * DV;
    const T* ringK = eta > 0 ? reinterpret_cast<const T*>(A.win_k) + (int64_t)bh * eta * DK : nullptr;
    const T* ringV = eta > 0 ? reinterpret_cast<const T*>(A.win_v) + (int64_t)bh * eta * DV : nullptr;
    const T* cK = lam > 0 ? reinterpret_cast<const T*>(A.cache_k) + (int64_t)bh * lam * DK : nullptr;
    const T* cV = lam > 0 ? reinterpret_cast<const T*>(A.cache_v) + (int64_t)bh * lam * DV : nullptr;
    const int32_t* cPos = lam > 0 ? A.cache_pos + (int64_t)bh * lam : nullptr;
    int32_t* foldAt = A.fold_at ? A.fold_at + (int64_t)bh * n : nullptr;

    // ---------------- set-up ----------------
    stage_wt<T>(wt, WT_LD, A.W, DK, DW);
    for (int d = tid; d < D; d += 256) sS[d] = A.s[(int64_t)bh * D + d];
    for (int j = tid; j < lam; j += 256) {
        const int p = cPos[j];
        slotPos[j] = p;
        slotSrc[j] = p >= 0 ? n + j : -1;
    }
    if (foldAt)
        for (int i = tid; i < n; i += 256) foldAt[i] = -1;

    f4 acc[IT][JW];
    {
        const float* Hb = A.H + (int64_t)bh * DV * D;
#pragma unroll
        for (int i = 0; i < IT; ++i)
#pragma unroll
            for (int jw = 0; jw < JW; ++jw) {
                const int J = w * JW + jw;
                const float4 h = *reinterpret_cast<const float4*>(Hb + (16 * J + c) * D + 16 * i + 4 * g);
                acc[i][jw] = f4{h.x, h.y, h.z, h.w};
            }
    }
    __syncthreads();

    // features and values of the initial cache members -> candidate rows 0..lam-1
    for (int tile = w; tile * 16 < lam; tile += 4) {
        const int row = tile * 16 + c;
        const bool valid = row < lam && slotPos[row] >= 0;
        Frag8<T> xf[DK / 32];
#pragma unroll
        for (int ss = 0; ss < DK / 32; ++ss) xf[ss] = valid ? load_frag(cK + (int64_t)row * DK, ss, g) : frag_zero<T>();
        float ph[D / 16][4];
        phi_tile<T, DK, PHI>(wt, WT_LD, xf, ph);
        if (valid)
#pragma unroll
            for (int ft = 0; ft < D / 16; ++ft)
                store4<T>(candPhi + (int64_t)row * D + 16 * ft + 4 * g, ph[ft][0], ph[ft][1], ph[ft][2], ph[ft][3]);
    }
    for (int i = tid; i < lam * DV; i += 256) {
        const int j = i / DV;
        if (slotPos[j] >= 0) candV[i] = cV[i];
    }
    if (tid == 0) {
        int cnt = 0;
        for (int j = 0; j < lam; ++j) cnt += slotPos[j] >= 0;
        tmp[8] = cnt;
    }
    __syncthreads();
    int nG = tmp[8];
    __syncthreads();

    // ---------------- chunk loop ----------------
    for (int ch = 0; ch < A.nchunks; ++ch) {
        const int64_t a = t0 + (int64_t)ch * C;
        const int64_t b = min(a + (int64_t)C, t0 + (int64_t)n);
        const int64_t xlo = a - eta > 0 ? a - eta : 0;
        const int64_t xhi = b - eta;
        const int nX = xhi > xlo ? (int)(xhi - xlo) : 0;
        char* rec = wsb + A.L.chunk0 + (int64_t)ch * A.L.per_chunk;

        // (1) snapshot of the chunk-start state
        {
            T* snapH = reinterpret_cast<T*>(rec + A.L.c_snap_h);
#pragma unroll
            for (int i = 0; i < IT; ++i)
#pragma unroll
                for (int jw = 0; jw < JW; ++jw) {
                    const int J = w * JW + jw;
                    store4<T>(snapH + (16 * J + c) * D + 16 * i + 4 * g, acc[i][jw][0], acc[i][jw][1],
                              acc[i][jw][2], acc[i][jw][3]);
                }
            float* snapS = reinterpret_cast<float*>(rec + A.L.c_snap_s);
            for (int d = tid; d < D; d += 256) snapS[d] = sS[d];
        }

        // (2) leaving tokens: features -> rows lam.., values -> rows lam..
        for (int tile = w; tile * 16 < nX; tile += 4) {
            const int x = tile * 16 + c;
            const bool valid = x < nX;
            const int64_t pos = xlo + x;
            const T* rk = nullptr;
            if (valid) rk = pos >= t0 ? kin + (pos - t0) * DK : ringK + (pos % eta) * DK;
            Frag8<T> xf[DK / 32];
#pragma unroll
            for (int ss = 0; ss < DK / 32; ++ss) xf[ss] = valid ? load_frag(rk, ss, g) : frag_zero<T>();
            float ph[D / 16][4];
            phi_tile<T, DK, PHI>(wt, WT_LD, xf, ph);
            if (valid)
#pragma unroll
                for (int ft = 0; ft < D / 16; ++ft)
                    store4<T>(candPhi + (int64_t)(lam + x) * D + 16 * ft + 4 * g, ph[ft][0], ph[ft][1], ph[ft][2],
                              ph[ft][3]);
        }
        for (int i = tid; i < nX * DV; i += 256) {
            const int x = i / DV, e = i - x * DV;
            const int64_t pos = xlo + x;
            const T* rv = pos >= t0 ? vin + (pos - t0) * DV : ringV + (pos % eta) * DV;
            candV[(int64_t)(lam + x) * DV + e] = rv[e];
        }
        const int NR = lam + nX;
        for (int r = tid; r < nrp; r += 256) {
            int f = 0;
            if (r < lam) f = slotPos[r] >= 0 ? 1 : 0;
            else if (r < NR) f = 1;
            flag[r] = f;
        }
        __syncthreads();

        // (3) decide which candidates are folded
        const bool scoring = lam > 0 && nG + nX > lam;
        if (scoring) {
            float sv[D / 32][8];
#pragma unroll
            for (int ss = 0; ss < D / 32; ++ss)
#pragma unroll
                for (int e = 0; e < 8; ++e) sv[ss][e] = sS[32 * ss + 16 * (e >> 2) + 4 * g + (e & 3)];
            const int ntile = (NR + 15) / 16;
            for (int tile = 0; tile < ntile; ++tile) {
                const int row = tile * 16 + c;
                const bool valid = row < NR && flag[row] != 0;
                f4 num[JW];
#pragma unroll
                for (int jw = 0; jw < JW; ++jw) num[jw] = zero4();
                float den = 0.f;
#pragma unroll
                for (int ss = 0; ss < D / 32; ++ss) {
                    const Frag8<T> af = valid ? load_frag(candPhi + (int64_t)row * D, ss, g) : frag_zero<T>();
#pragma unroll
                    for (int e = 0; e < 8; ++e) den += frag_get(af, e) * sv[ss][e];
#pragma unroll
                    for (int jw = 0; jw < JW; ++jw) {
                        const Frag8<T> bf = frag_from_acc<T>(acc[2 * ss][jw], acc[2 * ss + 1][jw]);
                        mma32(num[jw], af, bf);
                    }
                }
                den = sum_groups(den);
                float sq[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int rr = tile * 16 + 4 * g + r;
                    const float dr = __shfl(den, 4 * g + r);
                    const float inv = dr != 0.f ? 1.f / dr : 0.f;
                    float acc_sq = 0.f;
                    const bool rv = rr < NR;
#pragma unroll
                    for (int jw = 0; jw < JW; ++jw) {
                        const int J = w * JW + jw;
                        const float vv = rv ? to_f(candV[(int64_t)rr * DV + 16 * J + c]) : 0.f;
                        const float x = num[jw][r] * inv - vv;
                        acc_sq += x * x;
                    }
                    sq[r] = sum_cols(acc_sq);
                }
                if (c == 0)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int rr = tile * 16 + 4 * g + r;
                        if (rr < NR) part[w * nrp + rr] = sq[r];
                    }
            }
            __syncthreads();
            for (int r = tid; r < NR; r += 256) {
                unsigned long long k = 0ull;
                if (flag[r]) {
                    const float sre = sqrtf(part[r] + part[nrp + r] + part[2 * nrp + r] + part[3 * nrp + r]);
                    const int pos = r < lam ? slotPos[r] : (int)(xlo + (r - lam));
                    k = keep_key(sre, pos);
                }
                key[r] = k;
            }
            __syncthreads();
            for (int r = tid; r < NR; r += 256) {
                if (!flag[r]) continue;
                const unsigned long long kr = key[r];
                int rank = 0;
                for (int j = 0; j < NR; ++j) rank += key[j] > kr;
                flag[r] = rank >= lam ? 2 : 1;
            }
            __syncthreads();
        } else if (lam == 0) {
            for (int r = tid; r < NR; r += 256) flag[r] = 2;
            __syncthreads();
        }

        // (4) bookkeeping: fold order, free slots, entrants
        for (int r = tid; r < NR; r += 256) a1[r] = flag[r] == 2;
        for (int j = tid; j < lam; j += 256) a2[j] = (slotPos[j] < 0) || flag[j] == 2;
        for (int x = tid; x < nX; x += 256) a3[x] = flag[lam + x] == 1;
        __syncthreads();
        const int nS = block_exclusive_scan(a1, NR, tmp);
        block_exclusive_scan(a2, lam, tmp);
        const int nEnt = block_exclusive_scan(a3, nX, tmp);
        for (int j = tid; j < lam; j += 256)
            if ((slotPos[j] < 0) || flag[j] == 2) freeList[a2[j]] = j;
        for (int r = tid; r < NR; r += 256)
            if (flag[r] == 2) foldRow[a1[r]] = r;
        __syncthreads();
        int* recFoldPos = reinterpret_cast<int*>(rec + A.L.c_fold_pos);
        for (int k = tid; k < nS; k += 256) {
            const int r = foldRow[k];
            const int pos = r < lam ? slotPos[r] : (int)(xlo + (r - lam));
            recFoldPos[k] = pos;
            if (foldAt && pos >= t0) foldAt[pos - t0] = ch;
        }
        if (tid == 0) *reinterpret_cast<int*>(rec + A.L.c_fold_n) = nS;
        __syncthreads();
        for (int j = tid; j < lam; j += 256)
            if (flag[j] == 2) { slotPos[j] = -1; slotSrc[j] = -1; }
        __syncthreads();
        for (int x = tid; x < nX; x += 256) {
            if (flag[lam + x] != 1) continue;
            const int j = freeList[a3[x]];
            const int64_t pos = xlo + x;
            entSlot[a3[x]] = j;
            slotPos[j] = (int)pos;
            slotSrc[j] = pos >= t0 ? (int)(pos - t0) : n + lam + (int)(pos % eta);
        }
        __syncthreads();
        {
            int* rp = reinterpret_cast<int*>(rec + A.L.c_cache_pos);
            int* rs = reinterpret_cast<int*>(rec + A.L.c_cache_src);
            for (int j = tid; j < lam; j += 256) { rp[j] = slotPos[j]; rs[j] = slotSrc[j]; }
        }

        // (6) fold in batches of FB tokens; also emit the fold list for the read-out kernel
        T* recPhi = reinterpret_cast<T*>(rec + A.L.c_fold_phi);
        T* recVT = reinterpret_cast<T*>(rec + A.L.c_fold_vt);
        const int cp32 = A.L.c_pad32;
        for (int fb = 0; fb * FB < nS; ++fb) {
            for (int i = tid; i < FB * D; i += 256) {
                const int m = i / D, d = i - m * D;
                const int k = fb * FB + m;
                T val = from_f<T>(0.f);
                if (k < nS) {
                    val = candPhi[(int64_t)foldRow[k] * D + d];
                    recPhi[(int64_t)k * D + d] = val;
                }
                stPhi[d * ST_LD + m] = val;
            }
            for (int i = tid; i < FB * DV; i += 256) {
                const int m = i / DV, e = i - m * DV;
                const int k = fb * FB + m;
                const T val = k < nS ? candV[(int64_t)foldRow[k] * DV + e] : from_f<T>(0.f);
                stV[e * ST_LD + m] = val;
                recVT[(int64_t)e * cp32 + fb * FB + m] = val;
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < IT; ++i) {
                const Frag8<T> af = load_frag(stPhi + (16 * i + c) * ST_LD, 0, g);
#pragma unroll
                for (int jw = 0; jw < JW; ++jw) {
                    const int J = w * JW + jw;
                    const Frag8<T> bf = load_frag(stV + (16 * J + c) * ST_LD, 0, g);
                    mma32(acc[i][jw], af, bf);
                }
            }
            for (int d = tid; d < D; d += 256) {
                float sum = 0.f;
                for (int m = 0; m < FB; ++m) sum += to_f(stPhi[d * ST_LD + m]);
                sS[d] += sum;
            }
            __syncthreads();
        }

        // (7) entrants take their slots' candidate rows
        for (int i = tid; i < nEnt * (D + DV); i += 256) {
            const int k = i / (D + DV), e = i - k * (D + DV);
            const int j = entSlot[k];
            // the entrant's candidate row: the k-th kept leaving token
            const int64_t pos = slotPos[j];
            const int x = (int)(pos - xlo);
            if (e < D) candPhi[(int64_t)j * D + e] = candPhi[(int64_t)(lam + x) * D + e];
            else candV[(int64_t)j * DV + (e - D)] = candV[(int64_t)(lam + x) * DV + (e - D)];
        }
        nG = scoring ? lam : (lam == 0 ? 0 : nG + nX);
        __syncthreads();
    }

    // ---------------- final state ----------------
    {
        float* Hb = A.H + (int64_t)bh * DV * D;
#pragma unroll
        for (int i = 0; i < IT; ++i)
#pragma unroll
            for (int jw = 0; jw < JW; ++jw) {
                const int J = w * JW + jw;
                *reinterpret_cast<float4*>(Hb + (16 * J + c) * D + 16 * i + 4 * g) =
                    make_float4(acc[i][jw][0], acc[i][jw][1], acc[i][jw][2], acc[i][jw][3]);
            }
        for (int d = tid; d < D; d += 256) A.s[(int64_t)bh * D + d] = sS[d];
        int* fp = reinterpret_cast<int*>(wsb + A.L.slot_pos);
        int* fs = reinterpret_cast<int*>(wsb + A.L.slot_src);
        for (int j = tid; j < lam; j += 256) { fp[j] = slotPos[j]; fs[j] = slotSrc[j]; }
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
    hipLaunchKernelGGL(kern, dim3(a.BH), dim3(256), lds, stream, a);
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
