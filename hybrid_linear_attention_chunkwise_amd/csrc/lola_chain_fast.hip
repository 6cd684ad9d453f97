// Prefill allocation chain for bf16 with d_k = d_v = 128, lambda <= 256, C <= 64 and SRE scoring
// (LoLA notes 2.6 Eq. (15) with 2.3 Eq. (10) and 2.4 Eqs. (11)-(13)).  It takes the same decisions and
// writes the same chunk records as the general chain kernel (lola_chain.hip), bit for bit: the
// products, their summation order and the selection rule are the same.  What differs is where the
// data sits, which sets the time a chunk takes on the chain's serial path.
//
// One workgroup of eight waves per (sequence, head), for a whole chunk range:
//   registers  wave w: H's value columns 16w .. 16w + 15 (fp32 accumulators, all 128 feature rows),
//              and the features and values of cache slot tiles w and w + 8 (16 slots a tile, in MFMA
//              operand order), so scoring reads no cache data from memory;
//   LDS        token rows (128 features then 128 values, 512 bytes; 16-byte pieces XOR-swizzled by
//              row): two buffers of leaving tokens, each filled by direct global-to-LDS loads one
//              chunk ahead, the rows of the cache members a chunk folds, and a zero row; H^T in
//              operand order; the slot table (double-buffered by chunk parity); the selection's keys.
//
// Per chunk:
//   1. H^T to LDS, the chunk-start snapshot to the chunk record;                               barrier
//   2. every wave scores its tiles (at most two cache tiles and one leaving-token tile), reading
//      each A fragment of H^T once for all of them;                                            barrier
//   3. all eight waves select the nF smallest keys together: a shared 256-bin histogram of the SRE
//      bits between their extremes, a scan that every wave repeats to find the boundary bin, and an
//      exact rank of that bin's members (its 16-key bucket, or a list when it holds more);
//                                                                                      two barriers
//   4. each wave publishes its tiles' fold and freed-slot counts and entrant masks; after one
//      exchange every slot owner ranks its own slots, writes the fold list and the slot table,
//      stages its folded members' rows and takes its entrants from the leaving buffer;
//                                                                                      two barriers
//   5. fold: H += Phi_S^T V_S, both operands read with transposing LDS reads of the token rows.
#include <stdlib.h>

#include <type_traits>

#include "lola_common.hpp"
#include "lola_internal.hpp"

namespace lola {

namespace {

constexpr int kFcD = 128;                 // features = d_k = d_v
constexpr int kFcNW = 8, kFcNT = 512;
constexpr int kFcMaxLam = 256, kFcMaxC = 64;
constexpr int kFcMaxCand = kFcMaxLam + kFcMaxC;
constexpr int kFcKPL = kFcMaxCand / 64;   // candidates per lane in the selection
constexpr int kFcRowB = 512;              // one token row
constexpr int kFcStageRow = 128;          // rows 0..63 and 64..127: leaving buffers; 128..191: folds
constexpr int kFcZeroRow = 192;
constexpr int kFcRows = 193;
constexpr int kFcBucket = 16;             // keys a histogram bin keeps for the exact rank
static_assert(256 * kFcBucket * 8 <= 64 * kFcRowB, "buckets fit the staging rows");

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct FcLds {
    size_t rows, hcopy, list, spos, ssrc, s, mm, tw, em, frow, hist, misc, total;
};

__host__ __device__ constexpr FcLds fc_lds() {
    FcLds o{};
    size_t p = 0;
    o.rows = p;   p += (size_t)kFcRows * kFcRowB;
    o.hcopy = p;  p += (size_t)kFcNW * (kFcD / 32) * 64 * 16;
    o.list = p;   p += 8 * kFcMaxCand;
    o.spos = p;   p += 4 * 2 * kFcMaxLam;
    o.ssrc = p;   p += 4 * 2 * kFcMaxLam;
    o.s = p;      p += 4 * kFcD;
    o.mm = p;     p += 4 * 2 * kFcNW;
    o.tw = p;     p += 4 * 32;
    o.em = p;     p += 16;
    o.frow = p;   p += 4 * kFcMaxC;
    o.hist = p;   p += 4 * 256;
    o.misc = p;   p += 64;
    o.total = p;
    return o;
}

// A workgroup barrier that orders LDS only: the chain's global stores (chunk records, the fold list)
// are read by later kernels, never by another wave of the same chain, so they stay in flight across it.
// Each wave waits for its own leaving-token loads at the top of a chunk, before the first barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ unsigned long long fc_key(float sre, int pos) {
    // larger = kept first; equal SRE: the older position ranks higher; 0 = no candidate
    return ((unsigned long long)__float_as_uint(sre) << 32) | (unsigned long long)(0xFFFFFFFFu - (unsigned)pos);
}

// byte offset of 8-byte half h of logical 16-byte piece p in LDS token row r
__device__ __forceinline__ int fc_off(int r, int p, int h) { return r * kFcRowB + ((p ^ (r & 15)) << 4) + (h << 3); }

__device__ __forceinline__ bf16x4 fc_tr(const char* p) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (v4s __attribute__((address_space(3)))*)((__attribute__((address_space(3))) char*)p));
    bf16x4 out;
    __builtin_memcpy(&out, &r, sizeof(out));
    return out;
}

__global__ __launch_bounds__(kFcNT) void chain_fast_kernel(PrefillArgs A) {
    constexpr FcLds lo = fc_lds();
    constexpr int D = kFcD;
    extern __shared__ __align__(16) char smem[];
    char* rows = smem + lo.rows;
    bf16* hcopy = reinterpret_cast<bf16*>(smem + lo.hcopy);
    unsigned long long* list = reinterpret_cast<unsigned long long*>(smem + lo.list);  // boundary-bin keys
    int* sPos = reinterpret_cast<int*>(smem + lo.spos);       // [2][kFcMaxLam], by chunk parity
    int* sSrc = reinterpret_cast<int*>(smem + lo.ssrc);
    float* sS = reinterpret_cast<float*>(smem + lo.s);
    unsigned* mm = reinterpret_cast<unsigned*>(smem + lo.mm);  // per wave: min and max SRE bits
    int* tw = reinterpret_cast<int*>(smem + lo.tw);           // per tile: folds | freed slots << 16
    unsigned short* em = reinterpret_cast<unsigned short*>(smem + lo.em);   // entrants by leaving tile
    int* frow = reinterpret_cast<int*>(smem + lo.frow);       // fold rank -> LDS row
    int* hist = reinterpret_cast<int*>(smem + lo.hist);
    int* misc = reinterpret_cast<int*>(smem + lo.misc);

    const int lam = A.lam, eta = A.eta, n = A.n, C = A.C;
    const int bh = blockIdx.x;
    int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, so its branches are scalar
    int l = tid & 63, g = l >> 4, c = l & 15;
    const int64_t t0 = A.t0;
    const int nct = (lam + 15) >> 4;                          // cache tiles
    const int lamp = nct * 16;                                // candidate index of the first leaving token

    char* wsb = A.ws + (int64_t)bh * A.L.per_bh;
    const bf16* phiS = reinterpret_cast<const bf16*>(wsb + A.L.phi_store);
    const bf16* vin = reinterpret_cast<const bf16*>(A.v) + (int64_t)bh * n * D;
    const bf16* cV = lam > 0 ? reinterpret_cast<const bf16*>(A.cache_v) + (int64_t)bh * lam * D : nullptr;
    const bf16* ringV = eta > 0 ? reinterpret_cast<const bf16*>(A.win_v) + (int64_t)bh * eta * D : nullptr;
    const int32_t* cPosState = lam > 0 ? A.cache_pos + (int64_t)bh * lam : nullptr;
    int32_t* foldAt = A.fold_at ? A.fold_at + (int64_t)bh * n : nullptr;

    auto v_row = [&](int src) -> const bf16* {
        if (src < n) return vin + (int64_t)src * D;
        if (src < n + lam) return cV + (int64_t)(src - n) * D;
        return ringV + (int64_t)(src - n - lam) * D;
    };
    auto phi_row = [&](int src) -> const bf16* { return phiS + (int64_t)src * D; };
    const int ring0 = eta > 0 ? (int)(t0 % eta) : 0;
    auto source_of = [&](int64_t pos) -> int {               // input row, or the state's ring slot
        if (pos >= t0) return (int)(pos - t0);
        const int sl = ring0 + (int)(pos - (t0 - eta));
        return n + lam + (sl >= eta ? sl - eta : sl);
    };
    auto chunk_x = [&](int ch, int64_t& xlo) {               // leaving tokens of chunk ch: [xlo, xlo + nX)
        const int64_t a = t0 + (int64_t)ch * C;
        const int64_t b = min(a + (int64_t)C, t0 + (int64_t)n);
        xlo = a - eta > 0 ? a - eta : 0;
        return b - eta > xlo ? (int)(b - eta - xlo) : 0;
    };
    // lane (g, c)'s share of the token in LDS row r, in the register cache's order: features
    // 32ss + 4g .. + 3 and 32ss + 16 + 4g .. + 3, values 16J + 4g .. + 3
    auto row_load = [&](int r, Frag8<bf16> (&F)[4], bf16x4 (&V)[8]) {
#pragma unroll
        for (int ss = 0; ss < 4; ++ss) {
            const bf16x4 a = *reinterpret_cast<const bf16x4*>(rows + fc_off(r, 4 * ss + (g >> 1), g & 1));
            const bf16x4 b = *reinterpret_cast<const bf16x4*>(rows + fc_off(r, 4 * ss + 2 + (g >> 1), g & 1));
            F[ss].v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int J = 0; J < 8; ++J) V[J] = *reinterpret_cast<const bf16x4*>(rows + fc_off(r, 16 + 2 * J + (g >> 1), g & 1));
    };
    auto row_store = [&](int r, const Frag8<bf16> (&F)[4], const bf16x4 (&V)[8]) {
#pragma unroll
        for (int ss = 0; ss < 4; ++ss) {
            *reinterpret_cast<bf16x4*>(rows + fc_off(r, 4 * ss + (g >> 1), g & 1)) =
                __builtin_shufflevector(F[ss].v, F[ss].v, 0, 1, 2, 3);
            *reinterpret_cast<bf16x4*>(rows + fc_off(r, 4 * ss + 2 + (g >> 1), g & 1)) =
                __builtin_shufflevector(F[ss].v, F[ss].v, 4, 5, 6, 7);
        }
#pragma unroll
        for (int J = 0; J < 8; ++J) *reinterpret_cast<bf16x4*>(rows + fc_off(r, 16 + 2 * J + (g >> 1), g & 1)) = V[J];
    };
    // Leaving tokens of chunk ch_ into buffer buf: one instruction fills two rows (lane l: row l / 32,
    // slot l % 32, which holds logical piece slot ^ (row mod 16)).  Nothing reads rows past the chunk's
    // tokens.
    auto prefetch = [&](int ch_, int buf) {
        int64_t xl;
        const int nx = chunk_x(ch_, xl);
        const int rel = (int)(xl - t0);                       // >= -eta: leaving token 0 relative to the call
        if (rel >= 0) {
            // every leaving token is an input token: lanes with l mod 32 < 16 read features, the others
            // values, of consecutive input rows
            const uintptr_t fb = reinterpret_cast<uintptr_t>(phiS + (int64_t)rel * D);
            const uintptr_t vb = reinterpret_cast<uintptr_t>(vin + (int64_t)rel * D);
            const uintptr_t base = (l & 16) ? vb : fb;
            for (int pr = w; 2 * pr < nx; pr += kFcNW) {
                const int x = 2 * pr + (l >> 5);
                const int off = min(x, nx - 1) * (D * 2) + (((l & 15) ^ (x & 15)) << 4);
                __builtin_amdgcn_global_load_lds(
                    reinterpret_cast<const void*>(base + off),
                    (void __attribute__((address_space(3)))*)((__attribute__((address_space(3))) char*)(rows + (64 * buf + 2 * pr) * kFcRowB)),
                    16, 0, 0);
            }
            return;
        }
        for (int pr = w; 2 * pr < nx; pr += kFcNW) {
            const int x = 2 * pr + (l >> 5);
            const int p = (l & 31) ^ ((64 * buf + x) & 15);
            const int r = rel + min(x, nx - 1);               // a row past the chunk's tokens repeats the last
            // an input token (r >= 0) or a token of the state's window ring; both addresses are formed and
            // one selected (a branch here became a table of pointers in private memory)
            int sl = ring0 + r + eta;
            sl = sl >= eta ? sl - eta : sl;
            const bool in_call = r >= 0;
            const int src = in_call ? r : n + lam + sl;
            const bf16* vin_row = vin + (int64_t)(in_call ? r : 0) * D;
            const bf16* ring_row = ringV + (int64_t)(in_call ? 0 : sl) * D;
            const bf16* vrow = in_call ? vin_row : ring_row;
            const bf16* gp = p < 16 ? phiS + (int64_t)src * D + 8 * p : vrow + 8 * (p - 16);
            __builtin_amdgcn_global_load_lds(
                (const void*)gp,
                (void __attribute__((address_space(3)))*)((__attribute__((address_space(3))) char*)(rows + (64 * buf + 2 * pr) * kFcRowB)),
                16, 0, 0);
        }
    };

    // One step of the contiguous case (every leaving token an input token, rows from the input row of
    // the first on): the pair of rows w + 8 it.  The chunk loop spreads the four steps over the first
    // scoring steps, so these loads are not issued in one burst behind the snapshot's stores.
    auto prefetch_step = [&](int nx, uintptr_t base, int buf, int it) {
        const int pr = w + kFcNW * it;
        if (2 * pr < nx) {
            const int x = 2 * pr + (l >> 5);
            const int off = min(x, nx - 1) * (D * 2) + (((l & 15) ^ (x & 15)) << 4);
            __builtin_amdgcn_global_load_lds(
                reinterpret_cast<const void*>(base + off),
                (void __attribute__((address_space(3)))*)((__attribute__((address_space(3))) char*)(rows + (64 * buf + 2 * pr) * kFcRowB)),
                16, 0, 0);
        }
    };

    // ---------------- set-up ----------------
    const int cb0 = A.c_begin & 1;
    const bool first = A.c_begin == 0;
    const int* wsPos = reinterpret_cast<const int*>(wsb + A.L.slot_pos);
    const int* wsSrc = reinterpret_cast<const int*>(wsb + A.L.slot_src);
    for (int j = tid; j < lam; j += kFcNT) {
        int p_, s_;
        if (first) { p_ = cPosState[j]; s_ = p_ >= 0 ? n + j : -1; }
        else { p_ = wsPos[j]; s_ = wsSrc[j]; }
        sPos[cb0 * kFcMaxLam + j] = p_;
        sSrc[cb0 * kFcMaxLam + j] = s_;
    }
    if (first && foldAt)
        for (int i = tid; i < n; i += kFcNT) foldAt[i] = -1;
    for (int d = tid; d < D; d += kFcNT) sS[d] = A.s[(int64_t)bh * D + d];
    for (int e = tid; e < kFcRowB / 4; e += kFcNT) reinterpret_cast<int*>(rows + kFcZeroRow * kFcRowB)[e] = 0;
    f4 acc[8];
    {
        const float* Hb = A.H + (int64_t)bh * D * D;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 h = *reinterpret_cast<const float4*>(Hb + (16 * w + c) * D + 16 * i + 4 * g);
            acc[i] = f4{h.x, h.y, h.z, h.w};
        }
    }
    // the register cache: slot tiles w (u = 0) and w + 8 (u = 1)
    Frag8<bf16> CF[2][4];
    bf16x4 CV[2][8];
    int posR[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int j = 16 * (w + 8 * u) + c;
        int p_ = -1, s_ = -1;
        if (j < lam) {
            if (first) { p_ = cPosState[j]; s_ = p_ >= 0 ? n + j : -1; }
            else { p_ = wsPos[j]; s_ = wsSrc[j]; }
        }
        posR[u] = p_;
        if (s_ >= 0) {
            const bf16* pr = phi_row(s_);
            const bf16* vr = v_row(s_);
#pragma unroll
            for (int ss = 0; ss < 4; ++ss) CF[u][ss] = load_frag(pr, ss, g);
#pragma unroll
            for (int J = 0; J < 8; ++J) CV[u][J] = *reinterpret_cast<const bf16x4*>(vr + 16 * J + 4 * g);
        } else {
#pragma unroll
            for (int ss = 0; ss < 4; ++ss) CF[u][ss] = frag_zero<bf16>();
#pragma unroll
            for (int J = 0; J < 8; ++J) CV[u][J] = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
        }
    }
    int nG = 0;
#pragma unroll
    for (int u = 0; u < 2; ++u) nG += __popcll(__ballot(g == 0 && posR[u] >= 0));
    {   // every wave counted its own tiles; the total goes through LDS once
        if (l == 0) misc[8 + w] = nG;
        __syncthreads();
        nG = 0;
#pragma unroll
        for (int ww = 0; ww < kFcNW; ++ww) nG += misc[8 + ww];
    }
    prefetch(A.c_begin, cb0);

    // ---------------- chunk loop ----------------
    for (int ch = A.c_begin; ch < A.c_end; ++ch) {
        // Opaque to the optimiser: lane-dependent LDS offsets are recomputed in the loop (a few integer
        // operations) instead of being hoisted out of it and kept live across the whole chunk.
        asm volatile("" : "+v"(tid), "+v"(l), "+v"(g), "+v"(c));
        const int cb = ch & 1, nb = cb ^ 1;
        int64_t xlo;
        const int nX = chunk_x(ch, xlo);
        const int nlt = (nX + 15) >> 4;
        char* rec = wsb + A.L.chunk0 + (int64_t)ch * A.L.per_chunk;

        // (1) H^T in operand order: LDS copy and the chunk-start snapshot.  The wait (for this wave's
        // share of the chunk's leaving-token rows) comes first: it also waits for every store the wave
        // has issued, and the snapshot's stores are better left in flight.
        __builtin_amdgcn_s_waitcnt(0);
        {
            bf16* snapH = reinterpret_cast<bf16*>(rec + A.L.c_snap_h);
#pragma unroll
            for (int ss = 0; ss < 4; ++ss) {
                const Frag8<bf16> f = frag_from_acc<bf16>(acc[2 * ss], acc[2 * ss + 1]);
                *reinterpret_cast<Frag8<bf16>*>(snapH + ((int64_t)(w * 4 + ss) * 64 + l) * 8) = f;
                *reinterpret_cast<Frag8<bf16>*>(hcopy + ((w * 4 + ss) * 64 + l) * 8) = f;
            }
        }
        lds_barrier();
        // the next chunk's leaving tokens: the contiguous case in four steps (during scoring, or here
        // when the chunk does not score), any other at once
        int pnx = 0;
        uintptr_t pbase = 0;
        bool pf_steps = false;
        if (ch + 1 < A.c_end) {
            int64_t pxl;
            pnx = chunk_x(ch + 1, pxl);
            const int prel = (int)(pxl - t0);
            if (prel >= 0) {
                pf_steps = true;
                pbase = reinterpret_cast<uintptr_t>(((l & 16) ? vin : phiS) + (int64_t)prel * D);
            } else {
                prefetch(ch + 1, nb);
            }
        }
        {
            float* snapS = reinterpret_cast<float*>(rec + A.L.c_snap_s);
            for (int d = tid; d < D; d += kFcNT) snapS[d] = sS[d];
        }

        // (2) scoring: SRE of every candidate against the chunk-start state.  From here on lane (g, c),
        // g < 3, stands for candidate c of tile w + 8g: a cache slot (tiles below nct) or a leaving
        // token; its key stays in its registers.
        const bool scoring = lam > 0 && nG + nX > lam;
        const int Tg = w + 8 * g;
        const bool lane_c = g < 2 && 16 * Tg + c < lam;
        const int xg = 16 * (Tg - nct) + c;
        const bool lane_x = Tg >= nct && Tg < nct + nlt && xg < nX;
        const int posg = g == 0 ? posR[0] : posR[1];
        bool fold = false;
        if (!scoring && pf_steps) {
#pragma unroll
            for (int it = 0; it < 4; ++it) prefetch_step(pnx, pbase, nb, it);
        }
        if (scoring) {
            const bool h0 = w < nct, h1 = w + 8 < nct;
            int L = -1;
#pragma unroll
            for (int u = 0; u < 3; ++u) {
                const int T = w + 8 * u;
                if (T >= nct && T < nct + nlt) L = T - nct;
            }
            const bool hx = L >= 0;
            // the leaving-token tile's features; its values are read from LDS as each J needs them
            Frag8<bf16> XF[4];
            const int xr = 16 * (hx ? L : 0) + c;
            const int xrow = 64 * cb + xr;
            const bool xok = hx && xr < nX;
#pragma unroll
            for (int ss = 0; ss < 4; ++ss) {
                const bf16x4 a = *reinterpret_cast<const bf16x4*>(rows + fc_off(xrow, 4 * ss + (g >> 1), g & 1));
                const bf16x4 b = *reinterpret_cast<const bf16x4*>(rows + fc_off(xrow, 4 * ss + 2 + (g >> 1), g & 1));
                XF[ss].v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
                if (!xok) XF[ss] = frag_zero<bf16>();
            }
            // recall H^T phi(k) by value-row tile J; each A fragment serves all of the wave's tiles, and
            // the fragments of J + 1 are in flight while J is computed.  Without a leaving-token tile the
            // wave runs the two-tile loop; an absent cache tile has zero operands (its slots are empty).
            float sq[3] = {0.f, 0.f, 0.f};
            float inv[3];
            {   // denominators phi(k) . s
                float den[3] = {0.f, 0.f, 0.f};
#pragma unroll
                for (int ss = 0; ss < 4; ++ss) {
                    const f4 slo = *reinterpret_cast<const f4*>(sS + 32 * ss + 4 * g);
                    const f4 shi = *reinterpret_cast<const f4*>(sS + 32 * ss + 16 + 4 * g);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        den[0] += frag_get(CF[0][ss], e) * slo[e] + frag_get(CF[0][ss], 4 + e) * shi[e];
                        den[1] += frag_get(CF[1][ss], e) * slo[e] + frag_get(CF[1][ss], 4 + e) * shi[e];
                        den[2] += frag_get(XF[ss], e) * slo[e] + frag_get(XF[ss], 4 + e) * shi[e];
                    }
                }
#pragma unroll
                for (int u = 0; u < 3; ++u) {
                    den[u] = sum_groups(den[u]);
                    inv[u] = den[u] != 0.f ? __builtin_amdgcn_rcpf(den[u]) : 0.f;   // empty state: recall 0
                }
            }
            auto recall = [&](auto with_x) {
                constexpr bool WX = decltype(with_x)::value;
                // A fragments and the leaving tile's values of step J + 1 are requested before step J
                // is computed (the values first, so a wait for step J never waits for step J + 1)
                Frag8<bf16> a[2][4];
                bf16x4 xvb[2];
                if (WX) xvb[0] = *reinterpret_cast<const bf16x4*>(rows + fc_off(xrow, 16 + (g >> 1), g & 1));
#pragma unroll
                for (int ss = 0; ss < 4; ++ss)
                    a[0][ss] = *reinterpret_cast<const Frag8<bf16>*>(hcopy + (ss * 64 + l) * 8);
#pragma unroll
                for (int J = 0; J < 8; ++J) {
                    const int cur = J & 1;
                    if (J < 4 && pf_steps) prefetch_step(pnx, pbase, nb, J);
                    if (J + 1 < 8) {
                        if (WX) xvb[cur ^ 1] = *reinterpret_cast<const bf16x4*>(rows + fc_off(xrow, 16 + 2 * (J + 1) + (g >> 1), g & 1));
#pragma unroll
                        for (int ss = 0; ss < 4; ++ss)
                            a[cur ^ 1][ss] = *reinterpret_cast<const Frag8<bf16>*>(hcopy + (((J + 1) * 4 + ss) * 64 + l) * 8);
                    }
                    bf16x4 xv = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
                    if (WX && xok) xv = xvb[cur];
                    f4 r0 = zero4(), r1 = zero4(), r2 = zero4();
#pragma unroll
                    for (int ss = 0; ss < 4; ++ss) {
                        mma32(r0, a[cur][ss], CF[0][ss]);
                        mma32(r1, a[cur][ss], CF[1][ss]);
                        if (WX) mma32(r2, a[cur][ss], XF[ss]);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float x0 = r0[r] * inv[0] - (float)CV[0][J][r];
                        const float x1 = r1[r] * inv[1] - (float)CV[1][J][r];
                        sq[0] += x0 * x0;
                        sq[1] += x1 * x1;
                        if (WX) {
                            const float x2 = r2[r] * inv[2] - (float)xv[r];
                            sq[2] += x2 * x2;
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);        // bound the fragments in flight
                }
            };
            if (hx) recall(std::true_type{});
            else recall(std::false_type{});
            unsigned long long myk = 0ull;
            {
                const float sre0 = __builtin_amdgcn_sqrtf(sum_groups(sq[0]));
                const float sre1 = __builtin_amdgcn_sqrtf(sum_groups(sq[1]));
                const float sre2 = __builtin_amdgcn_sqrtf(sum_groups(sq[2]));
                if (lane_c && posg >= 0) myk = fc_key(g == 0 ? sre0 : sre1, posg);
                else if (lane_x) myk = fc_key(sre2, (int)(xlo + xg));
            }
            // (3) selection by all waves: the nF = nG + nX - lambda smallest keys fold.  A 256-bin
            // histogram over the SRE's bit pattern between the smallest and largest SRE (SRE >= 0, so
            // the bits order like the value: a logarithmic scale on which a bin is monotone in the key)
            // finds the boundary bin; its members are ranked exactly against each other.
            {
                const float kf = __uint_as_float((unsigned)(myk >> 32));
                const float lo_ = wave_min(myk ? kf : INFINITY), hi_ = wave_max(myk ? kf : 0.f);
                if (l == 0) {
                    mm[2 * w] = __float_as_uint(lo_);
                    mm[2 * w + 1] = __float_as_uint(hi_);
                }
                if (l < 32) hist[32 * w + l] = 0;
                if (tid == 0) misc[2] = 0;                    // boundary list length
            }
            lds_barrier();
            unsigned bmn = 0xFFFFFFFFu, bmx = 0u;
#pragma unroll
            for (int k2 = 0; k2 < kFcNW / 2; ++k2) {
                const u32x4 m4 = *reinterpret_cast<const u32x4*>(mm + 4 * k2);
                bmn = min(bmn, min(m4.x, m4.z));
                bmx = max(bmx, max(m4.y, m4.w));
            }
            const float scale = bmx > bmn ? 256.f / ((float)(bmx - bmn) + 1.f) : 0.f;
            const unsigned kb = (unsigned)(myk >> 32);
            const int bin = kb <= bmn ? 0 : min(255, (int)((float)(kb - bmn) * scale));
            // Each key also goes to its bin's bucket (16 keys a bin, in the staging rows, which hold
            // nothing until the slot owners fill them), so a small boundary bin is ranked without a
            // further exchange.
            unsigned long long* bucket = reinterpret_cast<unsigned long long*>(rows + kFcStageRow * kFcRowB);
            if (myk) {
                const int id = atomicAdd(&hist[bin], 1);
                if (id < kFcBucket) bucket[kFcBucket * bin + id] = myk;
            }
            lds_barrier();
            const int need = nG + nX - lam;
            const int4 h4 = *reinterpret_cast<const int4*>(hist + 4 * l);
            const int s4 = h4.x + h4.y + h4.z + h4.w;
            const int cum = wave_inclusive_sum(s4);
            const int lb = __builtin_amdgcn_readfirstlane(__ffsll((long long)__ballot(cum >= need)) - 1);
            int run = cum - s4, bl = 0, bef = 0, hb = 0;
            {
                const int hv[4] = {h4.x, h4.y, h4.z, h4.w};
                bool found = false;
#pragma unroll
                for (int k2 = 0; k2 < 4; ++k2) {
                    if (!found && need <= run + hv[k2]) { bl = 4 * l + k2; bef = run; hb = hv[k2]; found = true; }
                    run += hv[k2];
                }
            }
            const int bstar = __builtin_amdgcn_readlane(bl, lb);
            const int needp = need - __builtin_amdgcn_readlane(bef, lb);   // folds inside the boundary bin
            const int mb = __builtin_amdgcn_readlane(hb, lb);              // its members
            fold = myk != 0ull && bin < bstar;
            const bool member = myk != 0ull && bin == bstar;
            if (mb > needp) {
                // the members' keys: the bin's bucket, or (more than a bucket holds) a list built now
                const unsigned long long* keys = bucket + kFcBucket * bstar;
                if (mb > kFcBucket) {
                    if (member) list[atomicAdd(&misc[2], 1)] = myk;
                    lds_barrier();
                    keys = list;
                }
                if (__ballot(member) != 0ull) {
                    int below = 0;
#pragma unroll 4
                    for (int t = 0; t < mb; t += 2) {
                        typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
                        const u64x2 pk = *reinterpret_cast<const u64x2*>(keys + t);
                        below += (pk.x < myk ? 1 : 0) + (t + 1 < mb && pk.y < myk ? 1 : 0);
                    }
                    fold = fold || (member && below < needp);
                }
            } else {
                fold = fold || member;
            }
        } else if (lam == 0) {
            fold = lane_x;
        }

        // (4) the three candidate sets, in candidate order: folds, freed cache slots (empty, or holding
        // a fold) and entrants (kept leaving tokens).  A member's rank in its set is its fold rank or its
        // freed-slot rank; the freed slot of rank k takes the entrant of rank k.  Each wave publishes its
        // tiles' counts and the leaving tiles' entrant masks; after one exchange every slot owner ranks
        // its own slots, moves their rows and writes the fold list and the slot table.
        const unsigned long long bf = __ballot(fold), br = __ballot(lane_c && (posg < 0 || fold)),
                                 be = __ballot(lane_x && !fold);
        if (c == 0 && g < 3) {
            const unsigned fm = (unsigned)(bf >> (16 * g)) & 0xFFFFu, rm = (unsigned)(br >> (16 * g)) & 0xFFFFu;
            tw[Tg] = __popc(fm) | (__popc(rm) << 16);
            if (Tg >= nct && Tg < nct + nlt) em[Tg - nct] = (unsigned short)((be >> (16 * g)) & 0xFFFFull);
        }
        lds_barrier();
        int nS;
        {
            const int twl = l < 3 * kFcNW ? tw[l] : 0;
            unsigned long long E = *reinterpret_cast<const unsigned long long*>(em);
            E &= nX >= 64 ? ~0ull : ((1ull << nX) - 1ull);
            const int incl = wave_inclusive_sum(twl);
            const int excl = incl - twl;
            nS = __builtin_amdgcn_readlane(incl, 3 * kFcNW - 1) & 0xFFFF;
            const int nE = __popcll(E);
            int P[3];
#pragma unroll
            for (int u = 0; u < 3; ++u) P[u] = __builtin_amdgcn_readlane(excl, w + 8 * u);
            int* recFoldPos = reinterpret_cast<int*>(rec + A.L.c_fold_pos);
            int* recFoldSrc = reinterpret_cast<int*>(rec + A.L.c_fold_src);
            int* rp = reinterpret_cast<int*>(rec + A.L.c_cache_pos);
            int* rs = reinterpret_cast<int*>(rec + A.L.c_cache_src);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int j = 16 * (w + 8 * u) + c;
                if (j < lam) {
                    const unsigned long long lowc = ((1ull << c) - 1ull) << (16 * u);
                    int np = posR[u], ns = sSrc[cb * kFcMaxLam + j];
                    if ((bf >> (16 * u + c)) & 1ull) {
                        const int fr = (P[u] & 0xFFFF) + __popcll(bf & lowc);
                        row_store(kFcStageRow + fr, CF[u], CV[u]);
                        if (g == 0) {
                            frow[fr] = kFcStageRow + fr;
                            recFoldPos[fr] = np;
                            recFoldSrc[fr] = ns;
                            if (foldAt && np >= t0) foldAt[np - t0] = ch;
                        }
                    }
                    if ((br >> (16 * u + c)) & 1ull) {
                        int rk = (P[u] >> 16) + __popcll(br & lowc);
                        if (rk < nE) {
                            // the rk-th set bit of E: the entrant's leaving-token index
                            unsigned long long mk = E;
                            int x = 0;
#pragma unroll
                            for (int wdt = 32; wdt >= 1; wdt >>= 1) {
                                const int cnt = __popcll(mk & ((1ull << wdt) - 1ull));
                                if (rk >= cnt) { rk -= cnt; x += wdt; mk >>= wdt; }
                            }
                            row_load(64 * cb + x, CF[u], CV[u]);
                            np = (int)(xlo + x);
                            ns = source_of(xlo + x);
                        } else {
                            np = -1;
                            ns = -1;
                        }
                    }
                    posR[u] = np;
                    if (g == 0) {
                        sPos[nb * kFcMaxLam + j] = np;
                        sSrc[nb * kFcMaxLam + j] = ns;
                        rp[j] = np;
                        rs[j] = ns;
                    }
                }
            }
            // the folds among the wave's leaving tokens
#pragma unroll
            for (int u = 0; u < 3; ++u) {
                const int T = w + 8 * u;
                if (T >= nct && T < nct + nlt) {
                    const int x = 16 * (T - nct) + c;
                    if (g == 0 && x < nX && ((bf >> (16 * u + c)) & 1ull)) {
                        const int fr = (P[u] & 0xFFFF) + __popcll(bf & (((1ull << c) - 1ull) << (16 * u)));
                        const int64_t pos = xlo + x;
                        frow[fr] = 64 * cb + x;
                        recFoldPos[fr] = (int)pos;
                        recFoldSrc[fr] = source_of(pos);
                        if (foldAt && pos >= t0) foldAt[pos - t0] = ch;
                    }
                }
            }
            if (w == 0 && l >= nS) frow[l] = kFcZeroRow;
            if (tid == 0) *reinterpret_cast<int*>(rec + A.L.c_fold_n) = nS;
        }
        nG = scoring ? lam : (lam == 0 ? 0 : nG + nX);
        lds_barrier();

        // (5) fold: H += Phi_S^T V_S (32 tokens a step), s += column sums; the values, transposed, go
        // to the chunk record for the read-out kernel
        if (nS > 0) {
            bf16* recVT = reinterpret_cast<bf16*>(rec + A.L.c_fold_vt);
            const int cpv = A.L.c_pad64;
            const int q = c & 3;
            const int nkk = (nS + 31) >> 5;
            // lane (g, c) names token 32kk + 4g + c / 4 (and + 16) at elements 4(c mod 4) .. + 3 of a
            // 16-element tile; it receives element c of tokens 32kk + 4g .. + 3 (and + 16 ..).  The
            // value operands (and their record stores) come first, so the stores are old by the time
            // the next chunk waits on its loads.
            int ra[2], rb[2];
            Frag8<bf16> vf[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (kk >= nkk) break;
                ra[kk] = frow[32 * kk + 4 * g + (c >> 2)];
                rb[kk] = frow[32 * kk + 16 + 4 * g + (c >> 2)];
                vf[kk].v = __builtin_shufflevector(fc_tr(rows + fc_off(ra[kk], 16 + 2 * w + (q >> 1), q & 1)),
                                                   fc_tr(rows + fc_off(rb[kk], 16 + 2 * w + (q >> 1), q & 1)),
                                                   0, 1, 2, 3, 4, 5, 6, 7);
                bf16* dst = recVT + (int64_t)(16 * w + c) * cpv + 32 * kk + 4 * g;
                *reinterpret_cast<bf16x4*>(dst) = __builtin_shufflevector(vf[kk].v, vf[kk].v, 0, 1, 2, 3);
                *reinterpret_cast<bf16x4*>(dst + 16) = __builtin_shufflevector(vf[kk].v, vf[kk].v, 4, 5, 6, 7);
            }
            // a step's eight A fragments are requested together, before its products
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (kk >= nkk) break;
                Frag8<bf16> af[8];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    af[i].v = __builtin_shufflevector(fc_tr(rows + fc_off(ra[kk], 2 * i + (q >> 1), q & 1)),
                                                      fc_tr(rows + fc_off(rb[kk], 2 * i + (q >> 1), q & 1)),
                                                      0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                for (int i = 0; i < 8; ++i) mma32(acc[i], af[i], vf[kk]);
                __builtin_amdgcn_sched_barrier(0);
            }
            {   // s: four threads per feature, sixteen tokens each, in the general kernel's order
                const int d = tid >> 2, pr = tid & 3;
                float sum = 0.f;
#pragma unroll
                for (int m = 0; m < 16; ++m) {
                    const int r = frow[16 * pr + m];
                    sum += (float)*reinterpret_cast<const bf16*>(rows + fc_off(r, d >> 3, 0) + 2 * (d & 7));
                }
                sum += __shfl_xor(sum, 1);
                sum += __shfl_xor(sum, 2);
                if (pr == 0) sS[d] += sum;
            }
        }
    }

    // ---------------- final state ----------------
    __builtin_amdgcn_s_waitcnt(0);                    // no load into LDS outlives the workgroup
    __syncthreads();
    {
        float* Hb = A.H + (int64_t)bh * D * D;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<float4*>(Hb + (16 * w + c) * D + 16 * i + 4 * g) =
                make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
        for (int d = tid; d < D; d += kFcNT) A.s[(int64_t)bh * D + d] = sS[d];
        const int fb = A.c_end & 1;
        int* fp = reinterpret_cast<int*>(wsb + A.L.slot_pos);
        int* fs = reinterpret_cast<int*>(wsb + A.L.slot_src);
        for (int j = tid; j < lam; j += kFcNT) {
            fp[j] = sPos[fb * kFcMaxLam + j];
            fs[j] = sSrc[fb * kFcMaxLam + j];
        }
    }
}

}  // namespace

bool chain_fast_fits(const PrefillArgs& a, int esz, int d) {
    return esz == 2 && d == kFcD && a.score_rule == kScoreSre && a.lam <= kFcMaxLam && a.C <= kFcMaxC &&
           !getenv("LOLA_CHAIN_GENERAL");
}

hipError_t launch_chain_fast(const PrefillArgs& a, hipStream_t stream) {
    constexpr size_t lds = fc_lds().total;
    static_assert(lds <= 160 * 1024, "chain LDS");
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(chain_fast_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(chain_fast_kernel, dim3(a.BH), dim3(kFcNT), lds, stream, a);
    return hipGetLastError();
}

}  // namespace lola
