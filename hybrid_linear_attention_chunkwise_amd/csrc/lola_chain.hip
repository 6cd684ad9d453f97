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
// (D x d_v, feature rows, value columns), all feature rows.  At each chunk start every wave converts
// its accumulators into operand fragments of H^T (see lola_common.hpp) and writes them twice: to the
// chunk's snapshot for the read-out kernel and to LDS.  Scoring then runs candidate-major: wave w
// takes candidate tiles w, w + NW, ..., reads H^T from LDS as the A operand and the candidates'
// features straight from memory as the B operand, so each candidate's whole recall H^T phi(k), and
// with it the SRE, is formed inside one wave.  Selection keeps the lambda largest keys with a
// 256-bin histogram of SRE and an exact rank only inside the boundary bin; prefix counts use wave
// ballots, not LDS scans.  The fold stages the folded rows transposed in LDS and accumulates
// H += Phi_S^T V_S into the same registers.
//
// Every token's features are computed once and stored by source index (the same index that locates
// its K/V), so a token that enters the cache is never copied: a slot is just (position, source).
// The first scoring tile of the next chunk is fetched while the current chunk folds.
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
    static constexpr int CPR = ROWB / 16;                    // 16-byte pieces per row
    static constexpr int CPHI = D / EPV;                     // pieces holding phi
    static constexpr int FB = sizeof(T) == 2 ? 64 : 32;      // tokens per fold batch
    static constexpr int ST_LD = FB + EPV;                   // 16-byte aligned rows
    static constexpr int STAGE = (D + DV) * ST_LD;           // fold staging elements: [D + DV][ST_LD]
    static constexpr int HFR = NW * (D / 32) * 64 * 8;       // H^T copy, MFMA fragment order
    static constexpr int TPW = 4 / (int)sizeof(T);           // tokens packed per 32-bit LDS word
    static constexpr int FIPT = FB / TPW * CPR / NT;         // fold staging items per thread
    static constexpr int FLPT = FIPT * TPW;                  // pieces per thread per fold batch
    static constexpr int NBIN = 256;                         // selection histogram
    static_assert((FB / (4 / (int)sizeof(T))) * CPR % NT == 0, "fold batches must split evenly");
};

// Four consecutive elements of a value row (one accumulator column's rows 4g .. 4g + 3).
template <typename T> struct Quad;
template <> struct Quad<float> { f4 v; };
template <> struct Quad<bf16> { bf16x4 v; };
__device__ __forceinline__ Quad<float> load_quad(const float* p) { return {*reinterpret_cast<const f4*>(p)}; }
__device__ __forceinline__ Quad<bf16> load_quad(const bf16* p) { return {*reinterpret_cast<const bf16x4*>(p)}; }
__device__ __forceinline__ void store_quad(float* p, const Quad<float>& q) { *reinterpret_cast<f4*>(p) = q.v; }
__device__ __forceinline__ void store_quad(bf16* p, const Quad<bf16>& q) { *reinterpret_cast<bf16x4*>(p) = q.v; }

// One lane's share of a 16-candidate scoring tile: the features of candidate c = lane % 16 as the B
// operand (all of D), and the value entries that meet the lane's accumulator rows (one Quad per
// 16-row tile of H^T).
template <typename T, int D, int NW>
struct CandTile {
    Frag8<T> f[D / 32];
    Quad<T> v[NW];
};

// Candidate table: cache slots in rows 0 .. lam-1, the leaving tokens from row lam16 = lam rounded up
// to 16, so a 16-row scoring tile never mixes the two.  Rows of the per-candidate arrays: lam16 + C
// rounded up to 64 (whole ballot groups and tiles).
__host__ __device__ constexpr int x_base(int lam) { return (lam + 15) & ~15; }
__host__ __device__ constexpr int cand_rows(int lam, int C) { return ((x_base(lam) + C + 63) / 64) * 64; }

struct ChainLds {
    size_t s, slot_pos, slot_src, c_src, c_pos, key, aux, flag, a1, a2, a3, fold_src, ent_row, ent_pos, ent_src, slot_of_x,
        hist, tmp, hcopy, stage, total;
};

__host__ __device__ constexpr size_t al16(size_t x) { return (x + 15) & ~size_t(15); }

// LDS layout, sized for the largest supported cache and chunk so that every offset is a compile-time
// constant (the LDS instructions then carry them as immediates instead of one register per array).
// The small per-row arrays come first, inside the 64 KB immediate range.
template <typename T, int DK, int PHI>
__host__ __device__ constexpr ChainLds chain_lds() {
    using Cfg = ChainCfg<T, DK, PHI>;
    constexpr int lam = kMaxLambda, C = kMaxChunk;
    constexpr int nr = cand_rows(lam, C);
    ChainLds o{};
    size_t p = 0;
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
    o.fold_src = p;  p = al16(p + sizeof(int) * (C + 1));
    o.ent_row = p;   p = al16(p + sizeof(int) * (C + 1));
    o.ent_pos = p;   p = al16(p + sizeof(int) * (C + 1));
    o.ent_src = p;   p = al16(p + sizeof(int) * (C + 1));
    o.slot_of_x = p; p = al16(p + sizeof(int) * (C + 1));
    o.hist = p;      p = al16(p + sizeof(int) * (Cfg::NBIN + 4));
    o.tmp = p;       p = al16(p + sizeof(int) * 32);
    o.hcopy = p;     p = al16(p + sizeof(T) * Cfg::HFR);
    o.stage = p;     p = al16(p + sizeof(T) * Cfg::STAGE);
    o.total = p;
    return o;
}

// Key ordering the cache: larger = kept first.  SRE >= 0, so its bit pattern orders like the value;
// on equal SRE the older (smaller) position ranks higher.  0 marks an empty row.
__device__ __forceinline__ unsigned long long keep_key(float sre, int pos) {
    return ((unsigned long long)__float_as_uint(sre) << 32) | (unsigned long long)(0xFFFFFFFFu - (unsigned)pos);
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

// QS: the candidates are ranked by query-accumulated scores computed before the chain (a separate
// instantiation, so the SRE path is compiled exactly as it would be without the option).
template <typename T, int DK, int PHI, bool QS>
__global__ __launch_bounds__(4 * DK) void chain_kernel(PrefillArgs A) {
    using Cfg = ChainCfg<T, DK, PHI>;
    constexpr int D = Cfg::D, DV = Cfg::DV, NW = Cfg::NW, NT = Cfg::NT, IT = Cfg::IT, EPV = Cfg::EPV,
                  CPHI = Cfg::CPHI, FB = Cfg::FB, ST_LD = Cfg::ST_LD, FLPT = Cfg::FLPT, NBIN = Cfg::NBIN,
                  TPW = Cfg::TPW, FIPT = Cfg::FIPT;
    extern __shared__ __align__(16) char smem[];
    const int lam = A.lam, eta = A.eta, n = A.n, C = A.C;
    constexpr ChainLds lo = chain_lds<T, DK, PHI>();
    T* stage = reinterpret_cast<T*>(smem + lo.stage);
    T* hcopy = reinterpret_cast<T*>(smem + lo.hcopy);
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
    int* foldSrcL = reinterpret_cast<int*>(smem + lo.fold_src);   // source of the k-th folded token
    int* entRow = reinterpret_cast<int*>(smem + lo.ent_row);      // k-th entrant: leaving-token index,
    int* entPos = reinterpret_cast<int*>(smem + lo.ent_pos);      // position
    int* entSrc = reinterpret_cast<int*>(smem + lo.ent_src);      // and source
    int* slotOfX = reinterpret_cast<int*>(smem + lo.slot_of_x);
    int* hist = reinterpret_cast<int*>(smem + lo.hist);
    int* tmp = reinterpret_cast<int*>(smem + lo.tmp);

    const int bh = blockIdx.x;
    // l and c are re-derived at the top of every chunk through an empty asm (see the chunk loop)
    int tid = threadIdx.x, l = tid & 63, g = l >> 4, c = l & 15;
    const int w = tid >> 6;
    const int64_t t0 = A.t0;
    const int nrp = cand_rows(lam, C);
    const int xb = x_base(lam);                           // first leaving-token row of the table
    const int ct = xb >> 4;                               // scoring tiles that hold cache slots

    char* wsb = A.ws + (int64_t)bh * A.L.per_bh;
    Sources<T, DK> src;
    src.vin = reinterpret_cast<const T*>(A.v) + (int64_t)bh * n * DV;
    src.cV = lam > 0 ? reinterpret_cast<const T*>(A.cache_v) + (int64_t)bh * lam * DV : nullptr;
    src.ringV = eta > 0 ? reinterpret_cast<const T*>(A.win_v) + (int64_t)bh * eta * DV : nullptr;
    src.phi = reinterpret_cast<const T*>(wsb + A.L.phi_store);
    T* mirPhi = reinterpret_cast<T*>(wsb + A.L.mir_phi);
    const int mirVoff = (int)((A.L.mir_v - A.L.mir_phi) / (int64_t)sizeof(T));   // mir_v - mir_phi
    src.n = n;
    src.lam = lam;
    const int32_t* cPosState = lam > 0 ? A.cache_pos + (int64_t)bh * lam : nullptr;
    int32_t* foldAt = A.fold_at ? A.fold_at + (int64_t)bh * n : nullptr;

    // ring slot (position mod eta) of a position in [t0 - eta, t0), from one 64-bit remainder:
    // pos = t0 - eta + off with 0 <= off < eta, so pos mod eta = (t0 mod eta + off) mod eta
    const int ring0 = eta > 0 ? (int)(t0 % eta) : 0;
    auto ring_slot = [&](int64_t pos) {
        const int sl = ring0 + (int)(pos - (t0 - eta));
        return sl >= eta ? sl - eta : sl;
    };
    auto chunk_x = [&](int ch, int64_t& xlo) {           // leaving tokens of chunk ch: [xlo, xlo + nX)
        const int64_t a = t0 + (int64_t)ch * C;
        const int64_t b = min(a + (int64_t)C, t0 + (int64_t)n);
        xlo = a - eta > 0 ? a - eta : 0;
        return b - eta > xlo ? (int)(b - eta - xlo) : 0;
    };
    // candidate table of chunk ch: cache slots (rows 0..lam-1) then leaving tokens (rows xb..)
    auto build_table = [&](int ch) {
        int64_t xlo;
        const int nX = chunk_x(ch, xlo);
        for (int r = tid; r < nrp; r += NT) {
            int s_ = -1, p_ = -1, f = 0;
            if (r < lam) { s_ = slotSrc[r]; p_ = slotPos[r]; f = p_ >= 0; }
            else if (r >= xb && r < xb + nX) {
                const int64_t pos = xlo + (r - xb);
                p_ = (int)pos;
                s_ = pos >= t0 ? (int)(pos - t0) : n + lam + ring_slot(pos);
                f = 1;
            }
            cSrc[r] = s_;
            cPos[r] = p_;
            flag[r] = f;
        }
    };
    // Scoring tile j: candidates in table rows 16j .. 16j + 15, one per lane column c.  Cache tiles
    // (j < ct) come from the slot mirror, where features and values already sit in operand and
    // accumulator order (one 16-byte or 8-byte piece per lane and register, contiguous across the
    // wave).  Leaving-token tiles come from their rows; a lane without a candidate reads input row 0
    // instead, so the loads need no branch (its column of the products is never used).
    // Mirror values: a lane's quads of VP consecutive row tiles sit together (one 16-byte piece), so
    // a tile's values take NW / VP loads.
    constexpr int VP = sizeof(T) == 2 ? 2 : 1;
    auto mir_v_off = [&](int tile, int wv, int lane) {
        return mirVoff + (((tile * (NW / VP) + wv / VP) * 64 + lane) * VP + wv % VP) * 4;
    };
    auto load_tile = [&](CandTile<T, D, NW>& t, int j) {
        if (j < ct) {
            const T* b = mirPhi + ((int64_t)j * (D / 32) * 64 + l) * 8;
#pragma unroll
            for (int ss = 0; ss < D / 32; ++ss) t.f[ss] = *reinterpret_cast<const Frag8<T>*>(b + ss * 64 * 8);
            const T* bv = mirPhi + mir_v_off(j, 0, l);
#pragma unroll
            for (int wp = 0; wp < NW / VP; ++wp) {
                if constexpr (VP == 2) {
                    const uint4 x = *reinterpret_cast<const uint4*>(bv + wp * 64 * 8);
                    __builtin_memcpy(&t.v[2 * wp], &x, 8);
                    __builtin_memcpy(&t.v[2 * wp + 1], reinterpret_cast<const char*>(&x) + 8, 8);
                } else {
                    t.v[wp] = load_quad(bv + wp * 64 * 4);
                }
            }
        } else {
            const int row = 16 * j + c;                       // < nrp: tiles never pass the table
            const int f = flag[row], s0 = cSrc[row];
            const int s_ = f != 0 ? s0 : 0;
            const T* pr = src.phi_row(s_);
#pragma unroll
            for (int ss = 0; ss < D / 32; ++ss) t.f[ss] = load_frag(pr, ss, g);
            const T* vr = src.v_row(s_) + 4 * g;
#pragma unroll
            for (int wv = 0; wv < NW; ++wv) t.v[wv] = load_quad(vr + 16 * wv);
        }
    };
    // Lane (g, c) of a tile's registers holds exactly the pieces of candidate c that belong at lane
    // (g, slot % 16) of the slot's mirror tile: this writes them there.
    auto tile_to_slot = [&](const CandTile<T, D, NW>& t, int slot) {
        T* b = mirPhi + ((int64_t)(slot >> 4) * (D / 32) * 64 + g * 16 + (slot & 15)) * 8;
#pragma unroll
        for (int ss = 0; ss < D / 32; ++ss) *reinterpret_cast<Frag8<T>*>(b + ss * 64 * 8) = t.f[ss];
        T* bv = mirPhi + mir_v_off(slot >> 4, 0, g * 16 + (slot & 15));
#pragma unroll
        for (int wp = 0; wp < NW / VP; ++wp) {
            if constexpr (VP == 2) {
                uint4 x;
                __builtin_memcpy(&x, &t.v[2 * wp], 8);
                __builtin_memcpy(reinterpret_cast<char*>(&x) + 8, &t.v[2 * wp + 1], 8);
                *reinterpret_cast<uint4*>(bv + wp * 64 * 8) = x;
            } else {
                store_quad(bv + wp * 64 * 4, t.v[wp]);
            }
        }
    };
    // Copy rows into the slot mirror from their sources: info(e, slot, source) names item e; a
    // negative source skips it.  A row is QPR four-element pieces (features, then values); each
    // thread loads MU pieces before it stores any, so a round costs one memory latency.
    constexpr int QPR = D / 4 + DV / 4;
    constexpr int MU = 4;
    auto rows_to_mirror = [&](int nrows, auto&& info) {
        for (int q0 = 0; q0 < nrows * QPR; q0 += NT * MU) {
            Quad<T> qv[MU];
            int doff[MU];                                     // element offset from mir_phi, -1: none
#pragma unroll
            for (int u = 0; u < MU; ++u) {
                const int q = q0 + tid + NT * u;
                doff[u] = -1;
                if (q < nrows * QPR) {
                    const int e = q / QPR, it = q - e * QPR;
                    int slot, s_;
                    info(e, slot, s_);
                    if (s_ >= 0) {
                        const int tile = slot >> 4, cc = slot & 15;
                        if (it < D / 4) {                     // feature piece (ss, h, gg)
                            const int ss = it >> 3, h = (it >> 2) & 1, gg = it & 3;
                            qv[u] = load_quad(src.phi_row(s_) + 32 * ss + 16 * h + 4 * gg);
                            doff[u] = ((tile * (D / 32) + ss) * 64 + gg * 16 + cc) * 8 + 4 * h;
                        } else {                              // value piece (wv, gg)
                            const int iv = it - D / 4, wv = iv >> 2, gg = iv & 3;
                            qv[u] = load_quad(src.v_row(s_) + 16 * wv + 4 * gg);
                            doff[u] = mir_v_off(tile, wv, gg * 16 + cc);
                        }
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < MU; ++u)
                if (doff[u] >= 0) store_quad(mirPhi + doff[u], qv[u]);
        }
    };
    // bf16 keeps the next tile in flight while a tile is computed; fp32 operands are twice the
    // registers, so there a tile is fetched when its turn comes.
    constexpr bool PREF = sizeof(T) == 2;
    CandTile<T, D, NW> cur, nxt;

    // ---------------- set-up ----------------
    // The call's chunks may be walked in several launches (chunk ranges [c_begin, c_end)); H, s and
    // the slot table carry over through the state and the workspace, the slot mirror stays in place.
    const bool first = A.c_begin == 0;
    for (int d = tid; d < D; d += NT) sS[d] = A.s[(int64_t)bh * D + d];
    if (first) {
        for (int j = tid; j < lam; j += NT) {
            const int p = cPosState[j];
            slotPos[j] = p;
            slotSrc[j] = p >= 0 ? n + j : -1;
        }
        if (foldAt)
            for (int i = tid; i < n; i += NT) foldAt[i] = -1;
    } else {
        const int* fp = reinterpret_cast<const int*>(wsb + A.L.slot_pos);
        const int* fs = reinterpret_cast<const int*>(wsb + A.L.slot_src);
        for (int j = tid; j < lam; j += NT) { slotPos[j] = fp[j]; slotSrc[j] = fs[j]; }
    }
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
    if (first) rows_to_mirror(lam, [&](int e, int& slot, int& s_) { slot = e; s_ = slotSrc[e]; });
    build_table(A.c_begin);
    __syncthreads();
    // The first two tiles of each wave (cur, nxt) are fetched before the chunk starts.
    bool prefetched = false;
    auto prefetch_first = [&](int ch_) {
        int64_t xl;
        const int nX_ = chunk_x(ch_, xl);
        prefetched = false;
        if (!QS && lam > 0 && nG + nX_ > lam) {
            const int nt = (xb + nX_ + 15) / 16;
            if (w < nt) load_tile(cur, w);
            if (PREF && w + NW < nt) load_tile(nxt, w + NW);
            prefetched = true;
        }
    };
    prefetch_first(A.c_begin);

    // ---------------- chunk loop ----------------
    for (int ch = A.c_begin; ch < A.c_end; ++ch) {
        // Opaque to the optimiser: the lane-dependent LDS offsets and row pointers derived from l and c
        // are recomputed in the loop (a few integer operations) instead of being hoisted and kept live
        // across it, which overflowed the 256 registers a wave has here and put about twenty values in
        // scratch memory, reloaded on the chunk's critical path.
        asm volatile("" : "+v"(l), "+v"(c));
        int64_t xlo;
        const int nX = chunk_x(ch, xlo);
        const int NR = xb + nX;
        char* rec = wsb + A.L.chunk0 + (int64_t)ch * A.L.per_chunk;

        // (1) snapshot of the chunk-start state, in the fragment order the read-out kernel loads
        {
            T* snapH = reinterpret_cast<T*>(rec + A.L.c_snap_h);
#pragma unroll
            for (int ss = 0; ss < D / 32; ++ss) {
                const Frag8<T> f = frag_from_acc<T>(acc[2 * ss], acc[2 * ss + 1]);
                *reinterpret_cast<Frag8<T>*>(snapH + ((int64_t)(w * (D / 32) + ss) * 64 + l) * 8) = f;
                *reinterpret_cast<Frag8<T>*>(hcopy + ((w * (D / 32) + ss) * 64 + l) * 8) = f;
            }
            float* snapS = reinterpret_cast<float*>(rec + A.L.c_snap_s);
            for (int d = tid; d < D; d += NT) snapS[d] = sS[d];
        }

        // (3) decide which candidates are folded
        const bool scoring = lam > 0 && nG + nX > lam;
        const int ntile = (NR + 15) >> 4;
        if (scoring) {
            // SRE of every candidate against the chunk-start state.  Each wave takes whole 16-candidate
            // tiles (tile j goes to wave j % NW) and computes their full recall H^T phi(k) from the
            // LDS copy of H^T, so a candidate's error needs no exchange between waves.  The next
            // tile's loads are in flight while the current one is computed.
            __syncthreads();                                  // every wave's part of the H^T copy

            unsigned mn = 0x7F800000u, mx = 0u;
            if constexpr (!QS) {
                if (!prefetched && w < ntile) load_tile(cur, w);
                for (int j = w; j < ntile; j += NW) {
                    const bool has_next = j + NW < ntile;
                    if (PREF && has_next && !(prefetched && j == w)) load_tile(nxt, j + NW);
                    // the recall in two halves of the value rows (the B fragments stay in registers, each A
                    // fragment is still read once), which halves the accumulators held at a time
                    constexpr int HW = NW >= 8 ? NW / 2 : NW;
                    float den = 0.f;
#pragma unroll
                    for (int ss = 0; ss < D / 32; ++ss) {
                        const f4 slo = *reinterpret_cast<const f4*>(sS + 32 * ss + 4 * g);
                        const f4 shi = *reinterpret_cast<const f4*>(sS + 32 * ss + 16 + 4 * g);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            den += frag_get(cur.f[ss], e) * slo[e] + frag_get(cur.f[ss], 4 + e) * shi[e];
                    }
                    den = sum_groups(den);
                    const float inv = den != 0.f ? __builtin_amdgcn_rcpf(den) : 0.f;   // empty state: recall 0
                    float sq = 0.f;
#pragma unroll
                    for (int w0 = 0; w0 < NW; w0 += HW) {
                        f4 rec[HW];
#pragma unroll
                        for (int u = 0; u < HW; ++u) rec[u] = zero4();
#pragma unroll
                        for (int ss = 0; ss < D / 32; ++ss) {
                            Frag8<T> a[HW];
#pragma unroll
                            for (int u = 0; u < HW; ++u)
                                a[u] = *reinterpret_cast<const Frag8<T>*>(hcopy + (((w0 + u) * (D / 32) + ss) * 64 + l) * 8);
#pragma unroll
                            for (int u = 0; u < HW; ++u) mma32(rec[u], a[u], cur.f[ss]);
                            __builtin_amdgcn_sched_barrier(0);        // bound the A fragments in flight
                        }
#pragma unroll
                        for (int u = 0; u < HW; ++u)
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const float x = rec[u][r] * inv - to_f(cur.v[w0 + u].v[r]);
                                sq += x * x;
                            }
                    }
                    sq = sum_groups(sq);
                    const int row = 16 * j + c;
                    if (row < NR) {
                        const bool ok = flag[row] != 0;
                        const float sre = __builtin_amdgcn_sqrtf(sq);
                        if (g == 0) key[row] = ok ? keep_key(sre, cPos[row]) : 0ull;
                        if (ok) { mn = min(mn, __float_as_uint(sre)); mx = max(mx, __float_as_uint(sre)); }
                    }
                    if (has_next) {
                        if (PREF) cur = nxt;
                        else load_tile(cur, j + NW);
                    }
                }
            } else {
                // query-accumulated rule: the scores were computed before the chain; a cache member
                // has its complete score, a leaving token the one its own allocation sees
                const float* scAlloc = reinterpret_cast<const float*>(wsb + A.L.score_alloc);
                const float* scFull = reinterpret_cast<const float*>(wsb + A.L.score_full);
                for (int r = tid; r < NR; r += NT) {
                    unsigned long long kk = 0ull;
                    if (flag[r] != 0) {
                        const float sc = r < lam ? scFull[cSrc[r]] : scAlloc[cSrc[r]];
                        kk = keep_key(sc, cPos[r]);
                        mn = min(mn, __float_as_uint(sc));
                        mx = max(mx, __float_as_uint(sc));
                    }
                    key[r] = kk;
                }
            }
            // the score range for the histogram
            // (non-negative floats order like their bit patterns)
            mn = __float_as_uint(wave_min(__uint_as_float(mn)));
            mx = __float_as_uint(wave_max(__uint_as_float(mx)));
            if (l == 0) { tmp[8 + w] = (int)mn; tmp[16 + w] = (int)mx; }
            for (int i = tid; i < NBIN; i += NT) hist[i] = 0;
            if (tid == 0) tmp[4] = 0;
            __syncthreads();
            unsigned umn = 0x7F800000u, umx = 0u;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) { umn = min(umn, (unsigned)tmp[8 + ww]); umx = max(umx, (unsigned)tmp[16 + ww]); }
            const float smin = __uint_as_float(umn), smax = __uint_as_float(umx);
            const float bscale = smax > smin ? (float)NBIN / (smax - smin) : 0.f;
            // Query-accumulated scores span decades (they hold exponentials), so their bins split the
            // range of the bit patterns, a logarithmic scale; SRE values use linear bins.
            constexpr bool logbins = QS;
            const float lscale = (float)NBIN / ((float)(umx - umn) + 1.f);
            auto bin_of = [&](unsigned long long k) -> int {
                const unsigned b = (unsigned)(k >> 32);
                if (logbins) return min(NBIN - 1, (int)((float)(b - umn) * lscale));
                return min(NBIN - 1, (int)((__uint_as_float(b) - smin) * bscale));   // monotone in the key
            };
            for (int r = tid; r < NR; r += NT)
                if (flag[r]) atomicAdd(&hist[bin_of(key[r])], 1);
            __syncthreads();
            const int nF = nG + nX - lam;                     // how many to fold
            {   // boundary bin: cumulative count before it < nF <= cumulative through it
                int v4[4], s4 = 0;
#pragma unroll
                for (int u = 0; u < 4; ++u) { v4[u] = hist[4 * l + u]; s4 += v4[u]; }
                const int x = wave_inclusive_sum(s4);
                int run = x - s4, bstar = -1, need = 0;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (run < nF && nF <= run + v4[u]) { bstar = 4 * l + u; need = nF - run; }
                    run += v4[u];
                }
                // every wave finds the same (bin, need); spread it from the owning lane
                const unsigned long long own = __ballot(bstar >= 0);
                const int srcl = __ffsll((long long)own) - 1;
                bstar = __builtin_amdgcn_readlane(bstar, srcl);
                need = __builtin_amdgcn_readlane(need, srcl);
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

        // (4) prefix counts, all three in one pass over the table (one LDS read of each row): fold order
        // over the table (a1), freed cache slots (a2), entrants, the kept leaving tokens (a3).  Every
        // wave ballots every 64-row group and writes the prefixes of the groups it owns.
        int nS = 0, nE = 0;
        {
            const unsigned long long lt = l ? (~0ull >> (64 - l)) : 0ull;
            int nFree = 0;
#pragma unroll 2
            for (int k = 0; k * 64 < NR; ++k) {
                const int r = k * 64 + l;
                const int f = r < NR ? flag[r] : 0;
                const bool p2 = r < lam && (slotPos[r] < 0 || f == 2);
                const unsigned long long m1 = __ballot(f == 2), m2 = __ballot(p2), m3 = __ballot(r >= xb && f == 1);
                if (k % NW == w && r < NR) {
                    a1[r] = nS + __popcll(m1 & lt);
                    if (r < lam) a2[r] = nFree + __popcll(m2 & lt);
                    if (r >= xb) a3[r - xb] = nE + __popcll(m3 & lt);
                }
                nS += __popcll(m1);
                nFree += __popcll(m2);
                nE += __popcll(m3);
            }
        }
        __syncthreads();
        // (5) the fold list (recorded for the read-out kernel) and the entrant list
        {
            int* recFoldPos = reinterpret_cast<int*>(rec + A.L.c_fold_pos);
            int* recFoldSrc = reinterpret_cast<int*>(rec + A.L.c_fold_src);
            for (int r = tid; r < NR; r += NT) {
                if (flag[r] != 2) continue;
                const int k = a1[r], pos = cPos[r], sr = cSrc[r];
                foldSrcL[k] = sr;
                recFoldPos[k] = pos;
                recFoldSrc[k] = sr;
                if (foldAt && pos >= t0) foldAt[pos - t0] = ch;
            }
            if (tid == 0) *reinterpret_cast<int*>(rec + A.L.c_fold_n) = nS;
            for (int x = tid; x < nX; x += NT)
                if (flag[xb + x] == 1) {
                    const int k = a3[x];
                    entRow[k] = x;
                    entPos[k] = cPos[xb + x];
                    entSrc[k] = cSrc[xb + x];
                }
        }
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
                        const int s_ = foldSrcL[k];
                        const T* p_ = pc < CPHI ? src.phi_row(s_) + pc * EPV : src.v_row(s_) + (pc - CPHI) * EPV;
                        val = *reinterpret_cast<const uint4*>(p_);
                    }
                    stg[u * TPW + z] = val;
                }
            }
        };
        if (nS > 0) load_fold(0);
        // (6) the k-th freed slot (in slot order) goes to the k-th entrant; the other freed slots empty
        for (int j = tid; j < lam; j += NT) {
            if (slotPos[j] >= 0 && flag[j] != 2) continue;
            const int k = a2[j];
            if (k < nE) {
                slotPos[j] = entPos[k];
                slotSrc[j] = entSrc[k];
                slotOfX[entRow[k]] = j;
            } else {
                slotPos[j] = -1;
                slotSrc[j] = -1;
            }
        }
        __syncthreads();
        // (7) the entrants' features and values into their slots' mirror rows.  After scoring, the
        // leaving-token tiles are the last tile of their waves and still sit in registers (when there
        // are no more of them than waves); otherwise they are copied from their sources.
        if (lam > 0 && nE > 0) {
            if (scoring && ntile - ct <= NW) {
                const int jl = w < ntile ? w + NW * ((ntile - 1 - w) / NW) : -1;
                if (jl >= ct) {
                    const int x = 16 * (jl - ct) + c;
                    if (x < nX && flag[xb + x] == 1) tile_to_slot(cur, slotOfX[x]);
                }
            } else {
                rows_to_mirror(nE, [&](int e, int& slot, int& s_) {
                    slot = slotOfX[entRow[e]];
                    s_ = entSrc[e];
                });
            }
        }
        {
            int* rp = reinterpret_cast<int*>(rec + A.L.c_cache_pos);
            int* rs = reinterpret_cast<int*>(rec + A.L.c_cache_src);
            for (int j = tid; j < lam; j += NT) { rp[j] = slotPos[j]; rs[j] = slotSrc[j]; }
        }
        nG = scoring ? lam : (lam == 0 ? 0 : nG + nX);
        const bool more = ch + 1 < A.c_end;

        // (6) fold in batches of FB tokens: H += Phi_S^T V_S (MFMA), s += column sums.  Once the last
        // batch is staged, the next chunk's candidate table is built so its first batch can be
        // fetched while this fold runs.
        {
            T* recVT = reinterpret_cast<T*>(rec + A.L.c_fold_vt);
            const int cpv = A.L.c_pad64;
            T* stPhi = stage;                     // [D][ST_LD]
            T* stV = stage + D * ST_LD;           // [DV][ST_LD]
            for (int fb = 0; fb * FB < nS; ++fb) {
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
                // the next batch's rows are in flight under this batch's products (the staging
                // registers are free once their pieces are in LDS)
                if ((fb + 1) * FB < nS) load_fold(fb + 1);
                if (more && (fb + 1) * FB >= nS) build_table(ch + 1);
#pragma unroll
                for (int kk = 0; kk < FB / 32; ++kk) {
                    const Frag8<T> bf = load_frag(stV + (16 * w + c) * ST_LD, kk, g);
#pragma unroll
                    for (int i0 = 0; i0 < IT; i0 += 4) {
                        Frag8<T> af[4];
#pragma unroll
                        for (int u = 0; u < 4; ++u) af[u] = load_frag(stPhi + (16 * (i0 + u) + c) * ST_LD, kk, g);
#pragma unroll
                        for (int u = 0; u < 4; ++u) mma32(acc[i0 + u], af[u], bf);
                        __builtin_amdgcn_sched_barrier(0);        // bound the A fragments in flight
                    }
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
        if (more) prefetch_first(ch + 1);
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
    constexpr size_t lds = chain_lds<T, DK, PHI>().total;
    auto kern = a.score_rule != kScoreSre ? chain_kernel<T, DK, PHI, true> : chain_kernel<T, DK, PHI, false>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(a.BH), dim3(ChainCfg<T, DK, PHI>::NT), lds, stream, a);
    return hipGetLastError();
}

size_t chain_lds_bytes(int d, int phi_kind, int esz) {
    if (esz == 4) {
        if (d == 64) return phi_kind ? chain_lds<float, 64, 1>().total : chain_lds<float, 64, 0>().total;
        return phi_kind ? chain_lds<float, 128, 1>().total : chain_lds<float, 128, 0>().total;
    }
    if (d == 64) return phi_kind ? chain_lds<bf16, 64, 1>().total : chain_lds<bf16, 64, 0>().total;
    return phi_kind ? chain_lds<bf16, 128, 1>().total : chain_lds<bf16, 128, 0>().total;
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
