// C ABI of the LoLA library: validation, workspace sizing and launch sequencing.  See include/lola.h.
#include <limits.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/lola.h"
#include "lola_internal.hpp"

namespace {

using lola::WsLayout;
using lola::kMaxLambda;
using lola::kMaxChunk;

constexpr size_t kLdsLimit = 160 * 1024;

inline int64_t rup(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Shape checks shared by every entry point.  Returns LOLA_OK, LOLA_EINVAL or LOLA_EUNSUPPORTED.
lola_status check_shape(const lola_state* st) {
    if (!st) return LOLA_EINVAL;
    if (st->B <= 0 || st->n_heads <= 0 || st->d_k <= 0 || st->d_v <= 0 || st->D <= 0) return LOLA_EINVAL;
    if (st->eta < 0 || st->lambda < 0) return LOLA_EINVAL;
    if (st->dtype != LOLA_F32 && st->dtype != LOLA_BF16) return LOLA_EINVAL;
    if (st->t < 0) return LOLA_EINVAL;
    if (st->d_k != st->d_v || (st->d_k != 64 && st->d_k != 128)) return LOLA_EUNSUPPORTED;
    if (st->D != 128) return LOLA_EUNSUPPORTED;
    if (st->lambda > kMaxLambda) return LOLA_EUNSUPPORTED;
    if ((int64_t)st->B * st->n_heads > INT_MAX / 2) return LOLA_EUNSUPPORTED;
    return LOLA_OK;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

lola_status check_state_ptrs(const lola_state* st) {
    if (!st->H || !st->s || !aligned16(st->H) || !aligned16(st->s)) return LOLA_EINVAL;
    if (st->eta > 0 && (!st->win_k || !st->win_v || !aligned16(st->win_k) || !aligned16(st->win_v)))
        return LOLA_EINVAL;
    if (st->lambda > 0 && (!st->cache_k || !st->cache_v || !st->cache_pos || !aligned16(st->cache_k) ||
                           !aligned16(st->cache_v) || !aligned16(st->cache_pos)))
        return LOLA_EINVAL;
    return LOLA_OK;
}

// Options: mask within the three memories and holding the window; a known rule; zero reserved fields.
// Scores need the state's score arrays.
lola_status check_options(const lola_state* st, const lola_options* opt) {
    if (!opt) return LOLA_OK;
    if ((opt->read_mask & ~LOLA_READ_ALL) != 0 || !(opt->read_mask & LOLA_READ_WINDOW)) return LOLA_EINVAL;
    if (opt->score_rule < LOLA_SCORE_SRE || opt->score_rule > LOLA_SCORE_ATTN) return LOLA_EINVAL;
    if (opt->reserved != 0 || opt->decode_chunk < 0 || opt->decode_chunk > 64) return LOLA_EINVAL;
    if (opt->overlap) {
        if (!opt->overlap->stream) return LOLA_EINVAL;
        for (int i = 0; i < LOLA_OVERLAP_EVENTS; ++i)
            if (!opt->overlap->events[i]) return LOLA_EINVAL;
    }
    if (opt->score_rule != LOLA_SCORE_SRE) {
        if (st->eta > 0 && (!st->win_score || !aligned16(st->win_score))) return LOLA_EINVAL;
        if (st->lambda > 0 && (!st->cache_score || !aligned16(st->cache_score))) return LOLA_EINVAL;
    }
    return LOLA_OK;
}

lola_status check_phi(const lola_state* st, const lola_phi* phi) {
    if (!phi || !phi->W || !aligned16(phi->W)) return LOLA_EINVAL;
    if (phi->kind != LOLA_PHI_ELU1 && phi->kind != LOLA_PHI_SOFTMAX_PM) return LOLA_EINVAL;
    if (phi->d_k != st->d_k || phi->D != st->D) return LOLA_EINVAL;
    return LOLA_OK;
}

WsLayout make_layout(const lola_state* st, int64_t n, int32_t C) {
    const int64_t esz = st->dtype == LOLA_BF16 ? 2 : 4;
    const int64_t D = st->D, dv = st->d_v, lam = st->lambda;
    WsLayout L;
    memset(&L, 0, sizeof(L));
    L.nchunks = (int32_t)((n + C - 1) / C);
    L.c_pad16 = (int32_t)rup(C, 16);
    L.c_pad64 = (int32_t)rup(C, 64);
    int64_t p = 0;
    L.phi_store = p; p = rup(p + (2 * n + lam + st->eta) * D * esz, 256);
    L.score_alloc = p; p = rup(p + (n + lam + st->eta) * 4, 256);
    L.score_full = p;  p = rup(p + (n + lam + st->eta) * 4, 256);
    L.slot_pos = p;  p = rup(p + (lam + 1) * 4, 256);
    L.slot_src = p;  p = rup(p + (lam + 1) * 4, 256);
    L.mir_phi = p;   p = rup(p + rup(lam, 16) * D * esz, 256);
    L.mir_v = p;     p = rup(p + rup(lam, 16) * dv * esz, 256);
    L.chunk0 = p;
    int64_t q = 0;
    L.c_snap_h = q;    q = rup(q + dv * D * esz, 256);
    L.c_snap_s = q;    q = rup(q + D * 4, 256);
    L.c_cache_pos = q; q = rup(q + (lam + 1) * 4, 256);
    L.c_cache_src = q; q = rup(q + (lam + 1) * 4, 256);
    L.c_fold_n = q;    q = rup(q + 4, 256);
    L.c_fold_pos = q;  q = rup(q + L.c_pad16 * 4, 256);
    L.c_fold_src = q;  q = rup(q + L.c_pad16 * 4, 256);
    L.c_fold_vt = q;   q = rup(q + dv * L.c_pad64 * esz, 256);
    L.per_chunk = q;
    L.per_bh = rup(L.chunk0 + (int64_t)L.nchunks * L.per_chunk, 256);
    return L;
}

lola_status check_prefill_config(const lola_state* st, int64_t n, int32_t C) {
    if (n < 0 || C < 1) return LOLA_EINVAL;
    if (st->lambda > 0 && st->eta < C - 1) return LOLA_EINVAL;   // causality of chunk-level promotion
    if (C > kMaxChunk) return LOLA_EUNSUPPORTED;
    if (st->t + n + st->eta >= (int64_t)INT_MAX) return LOLA_EUNSUPPORTED;
    if (n > INT_MAX / 2) return LOLA_EUNSUPPORTED;
    const int esz = st->dtype == LOLA_BF16 ? 2 : 4;
    if (lola::chain_lds_bytes(st->d_k, 1, esz) > kLdsLimit || lola::chain_lds_bytes(st->d_k, 0, esz) > kLdsLimit)
        return LOLA_EUNSUPPORTED;
    return LOLA_OK;
}

}  // namespace

static lola::HolaLayout hola_layout(int64_t BH, int64_t d, int64_t esz, int64_t n, int64_t C, int64_t nchunks) {
    lola::HolaLayout L;
    int64_t p = 0;
    const int64_t rows = BH * n;
    L.qinv = p; p = rup(p + rows * 4, 256);
    L.kinv = p; p = rup(p + rows * 4, 256);
    L.qtil = p; p = rup(p + rows * d * esz, 256);
    L.ktil = p; p = rup(p + rows * d * esz, 256);
    L.o = p;    p = rup(p + rows * d * 4, 256);
    L.esq = p;  p = rup(p + rows * (d / 16) * 4, 256);
    L.clist = p; p = rup(p + BH * (nchunks + 1) * lola::kHolaMaxW * 4, 256);
    L.blk = p;  p = rup(p + BH * ((n + lola::kHolaBT - 1) / lola::kHolaBT) * (int64_t)sizeof(lola::HolaBlock), 256);
    L.sink = p; p = rup(p + 2 * 64 * 4, 256);
    L.tlist = p; p = rup(p + BH * nchunks * (C < lola::kHolaMaxW ? C : lola::kHolaMaxW) * 8, 256);
    L.total = p;
    return L;
}

static lola_status hola_check(int32_t B, int32_t n_heads, int32_t d, int32_t dtype, int64_t n, int32_t C) {
    if (B <= 0 || n_heads <= 0 || n < 0 || C < 1) return LOLA_EINVAL;
    if (dtype != LOLA_F32 && dtype != LOLA_BF16) return LOLA_EINVAL;
    if (d != 64 && d != 128 && d != 256) return LOLA_EUNSUPPORTED;
    if (C > lola::kHolaMaxC || n > INT_MAX / 2 || (int64_t)B * n_heads > INT_MAX / 2) return LOLA_EUNSUPPORTED;
    return LOLA_OK;
}

namespace lola {
// Every check of a prefill call but the workspace's (shared with the allocation-free entry point).
lola_status prefill_checks(const lola_state* st, const lola_phi* phi, const void* q, const void* k, const void* v,
                           int64_t n, int32_t C, const lola_options* opt, const void* y, const int32_t* fold_at,
                           void* stream) {
    lola_status rc = check_shape(st);
    if (rc != LOLA_OK) return rc;
    rc = check_state_ptrs(st);
    if (rc != LOLA_OK) return rc;
    rc = check_phi(st, phi);
    if (rc != LOLA_OK) return rc;
    rc = check_options(st, opt);
    if (rc != LOLA_OK) return rc;
    rc = check_prefill_config(st, n, C);
    if (rc != LOLA_OK) return rc;
    if (st->dec_chunk != 0 || (opt && opt->decode_chunk > 1)) return LOLA_EINVAL;   // a decode group is open
    if (opt && opt->overlap && opt->overlap->stream == stream) return LOLA_EINVAL;
    if (n == 0) return LOLA_OK;
    if (!q || !k || !v || !y || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(y)) return LOLA_EINVAL;
    if (fold_at && !aligned16(fold_at)) return LOLA_EINVAL;
    return LOLA_OK;
}
}  // namespace lola

extern "C" {

const char* lola_status_string(lola_status status) {
    switch (status) {
        case LOLA_OK: return "LOLA_OK";
        case LOLA_EINVAL: return "LOLA_EINVAL: invalid argument";
        case LOLA_EUNSUPPORTED: return "LOLA_EUNSUPPORTED: shape outside the supported set";
        case LOLA_EDEVICE: return "LOLA_EDEVICE: HIP launch or runtime failure";
        default: return "unknown lola_status";
    }
}

size_t lola_workspace_bytes(const lola_state* st, int64_t n_max, int32_t C) {
    if (check_shape(st) != LOLA_OK || n_max < 0 || C < 1 || C > kMaxChunk) return 0;
    if (n_max == 0) return 256;
    const WsLayout L = make_layout(st, n_max, C);
    return (size_t)L.per_bh * (size_t)st->B * (size_t)st->n_heads;
}

lola_status lola_state_init(lola_state* st, void* stream) {
    lola_status rc = check_shape(st);
    if (rc != LOLA_OK) return rc;
    rc = check_state_ptrs(st);
    if (rc != LOLA_OK) return rc;
    lola::InitArgs a;
    a.BH = st->B * st->n_heads;
    a.D = st->D;
    a.d_v = st->d_v;
    a.lam = st->lambda;
    a.eta = st->eta;
    a.H = st->H;
    a.s = st->s;
    a.cache_pos = st->cache_pos;
    a.win_score = st->eta > 0 ? st->win_score : nullptr;
    a.cache_score = st->lambda > 0 ? st->cache_score : nullptr;
    if (lola::launch_init(a, (hipStream_t)stream) != hipSuccess) return LOLA_EDEVICE;
    st->t = 0;
    st->dec_chunk = 0;
    return LOLA_OK;
}


static lola_status prefill_impl(lola_state* st, const lola_phi* phi, const void* q, const void* k,
                                const void* v, int64_t n, int32_t C, const lola_options* opt, void* y,
                                int32_t* fold_at, void* workspace, size_t workspace_bytes, void* stream,
                                void* const* events) {
    const lola_status rc = lola::prefill_checks(st, phi, q, k, v, n, C, opt, y, fold_at, stream);
    if (rc != LOLA_OK || n == 0) return rc;
    const WsLayout L = make_layout(st, n, C);
    const size_t need = (size_t)L.per_bh * (size_t)st->B * (size_t)st->n_heads;
    if (!workspace || ((uintptr_t)workspace & 255u) != 0 || workspace_bytes < need) return LOLA_EINVAL;

    lola::PrefillArgs a;
    a.BH = st->B * st->n_heads;
    a.n = (int)n;
    a.C = C;
    a.eta = st->eta;
    a.lam = st->lambda;
    a.nchunks = L.nchunks;
    a.nqt = (C + 63) / 64;
    a.read_mask = opt ? opt->read_mask : LOLA_READ_ALL;
    a.score_rule = opt ? opt->score_rule : LOLA_SCORE_SRE;
    a.win_score = st->win_score;
    a.cache_score = st->cache_score;
    a.t0 = st->t;
    a.q = q; a.k = k; a.v = v; a.y = y;
    a.W = phi->W;
    a.H = st->H; a.s = st->s;
    a.win_k = st->win_k; a.win_v = st->win_v;
    a.cache_k = st->cache_k; a.cache_v = st->cache_v; a.cache_pos = st->cache_pos;
    a.fold_at = fold_at;
    a.ws = reinterpret_cast<char*>(workspace);
    a.L = L;
    if ((int64_t)a.BH * a.nchunks * a.nqt > (int64_t)INT_MAX) return LOLA_EUNSUPPORTED;
    lola::Overlap ov;
    const bool use_ov = opt && opt->overlap;
    if (use_ov) {
        static_assert(LOLA_OVERLAP_EVENTS == lola::kOverlapEvents, "overlap event count");
        ov.stream = (hipStream_t)opt->overlap->stream;
        for (int i = 0; i < lola::kOverlapEvents; ++i) ov.ev[i] = (hipEvent_t)opt->overlap->events[i];
    }
    const hipError_t e = lola::launch_prefill(a, st->dtype, st->d_k, phi->kind, (hipStream_t)stream,
                                              reinterpret_cast<hipEvent_t const*>(events), use_ov ? &ov : nullptr);
    if (e != hipSuccess) return LOLA_EDEVICE;
    if (getenv("LOLA_DEBUG_SYNC") && hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return LOLA_EDEVICE;
    st->t += n;
    return LOLA_OK;
}

lola_status lola_prefill(lola_state* st, const lola_phi* phi, const void* q, const void* k, const void* v,
                         int64_t n, int32_t C, void* y, int32_t* fold_at, void* workspace,
                         size_t workspace_bytes, void* stream) {
    return prefill_impl(st, phi, q, k, v, n, C, nullptr, y, fold_at, workspace, workspace_bytes, stream, nullptr);
}

lola_status lola_prefill_ex(lola_state* st, const lola_phi* phi, const void* q, const void* k, const void* v,
                            int64_t n, int32_t C, const lola_options* opt, void* y, int32_t* fold_at,
                            void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_impl(st, phi, q, k, v, n, C, opt, y, fold_at, workspace, workspace_bytes, stream, nullptr);
}

lola_status lola_prefill_profiled(lola_state* st, const lola_phi* phi, const void* q, const void* k,
                                  const void* v, int64_t n, int32_t C, void* y, int32_t* fold_at,
                                  void* workspace, size_t workspace_bytes, void* stream,
                                  void* const events[5]) {
    return prefill_impl(st, phi, q, k, v, n, C, nullptr, y, fold_at, workspace, workspace_bytes, stream, events);
}

static lola_status decode_impl(lola_state* st, const lola_phi* phi, const void* q, const void* k, const void* v,
                               const lola_options* opt, void* y, int32_t* folded_pos, void* stream) {
    lola_status rc = check_shape(st);
    if (rc != LOLA_OK) return rc;
    rc = check_state_ptrs(st);
    if (rc != LOLA_OK) return rc;
    rc = check_phi(st, phi);
    if (rc != LOLA_OK) return rc;
    rc = check_options(st, opt);
    if (rc != LOLA_OK) return rc;
    if (opt && opt->score_rule != LOLA_SCORE_SRE) return LOLA_EUNSUPPORTED;
    if (opt && opt->overlap) return LOLA_EINVAL;                         // decode runs one kernel per step
    const int cd = (opt && opt->decode_chunk > 1) ? opt->decode_chunk : 0;
    if (st->dec_chunk != 0 && st->dec_chunk != cd) return LOLA_EINVAL;  // another group is open
    if (!q || !k || !v || !y || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(y)) return LOLA_EINVAL;
    if (folded_pos && !aligned16(folded_pos)) return LOLA_EINVAL;
    if (st->t + 1 + st->eta >= (int64_t)INT_MAX) return LOLA_EUNSUPPORTED;
    const int esz = st->dtype == LOLA_BF16 ? 2 : 4;
    if (cd > 0) {
        if (folded_pos || !st->dec_fold || ((uintptr_t)st->dec_fold & 7u) != 0) return LOLA_EINVAL;
        if (st->lambda > 0 && st->eta < cd - 1) return LOLA_EINVAL;     // causality of the group's allocation
        if (lola::decode_group_lds_bytes(st->d_k, phi->kind, esz, st->lambda, st->eta, cd) > kLdsLimit)
            return LOLA_EUNSUPPORTED;
    } else {
        const size_t lds = lola::decode_lds_bytes(st->d_k, phi->kind, esz, st->lambda) + 4 * (size_t)(st->eta + 16);
        if (lds > kLdsLimit) return LOLA_EUNSUPPORTED;
    }

    lola::DecodeArgs a;
    a.BH = st->B * st->n_heads;
    a.eta = st->eta;
    a.lam = st->lambda;
    a.read_mask = opt ? opt->read_mask : LOLA_READ_ALL;
    a.t = st->t;
    a.q = q; a.k = k; a.v = v; a.y = y;
    a.W = phi->W;
    a.H = st->H; a.s = st->s;
    a.win_k = st->win_k; a.win_v = st->win_v;
    a.cache_k = st->cache_k; a.cache_v = st->cache_v; a.cache_pos = st->cache_pos;
    a.folded_pos = folded_pos;
    a.dec_chunk = cd;
    a.group_start = (cd > 0 && st->dec_chunk == 0) ? 1 : 0;
    a.dec_fold = reinterpret_cast<unsigned long long*>(st->dec_fold);
    hipError_t e;
    if (cd > 0) {
        e = lola::launch_decode_group(a, st->dtype, st->d_k, phi->kind, (hipStream_t)stream);
    } else {
        // bf16 states whose cache and window fit the register-resident kernel take it
        const bool fast = st->dtype == LOLA_BF16 && lola::decode_fast_fits(st->d_k, st->lambda, st->eta) &&
                          lola::decode_fast_lds_bytes(st->d_k, phi->kind) <= kLdsLimit &&
                          !getenv("LOLA_DECODE_GENERAL");
        e = fast ? lola::launch_decode_fast(a, st->d_k, phi->kind, (hipStream_t)stream)
                 : lola::launch_decode(a, st->dtype, st->d_k, phi->kind, (hipStream_t)stream);
    }
    if (e != hipSuccess) return LOLA_EDEVICE;
    if (getenv("LOLA_DEBUG_SYNC") && hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return LOLA_EDEVICE;
    st->t += 1;
    if (cd > 0) st->dec_chunk = (st->t % cd == 0) ? 0 : cd;              // the group's last step closes it
    return LOLA_OK;
}

lola_status lola_decode_step(lola_state* st, const lola_phi* phi, const void* q, const void* k, const void* v,
                             void* y, int32_t* folded_pos, void* stream) {
    return decode_impl(st, phi, q, k, v, nullptr, y, folded_pos, stream);
}

lola_status lola_decode_step_ex(lola_state* st, const lola_phi* phi, const void* q, const void* k, const void* v,
                                const lola_options* opt, void* y, int32_t* folded_pos, void* stream) {
    return decode_impl(st, phi, q, k, v, opt, y, folded_pos, stream);
}

size_t hola_workspace_bytes(int32_t B, int32_t n_heads, int32_t d, int32_t dtype, int64_t n, int32_t C) {
    if (hola_check(B, n_heads, d, dtype, n, C) != LOLA_OK) return 0;
    if (n == 0) return 256;
    const int64_t nchunks = (n + C - 1) / C;
    return (size_t)hola_layout((int64_t)B * n_heads, d, dtype == LOLA_BF16 ? 2 : 4, n, C, nchunks).total;
}

lola_status hola_prefill(int32_t B, int32_t n_heads, int32_t d, int32_t dtype, int64_t n, int32_t C, int32_t w,
                         const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                         const float* gamma_q, const float* gamma_k, const float* sink, const float* gate,
                         void* y, float* S_out, int32_t* cache_pos_out, float* cache_score_out, void* workspace,
                         size_t workspace_bytes, void* stream) {
    lola_status rc = hola_check(B, n_heads, d, dtype, n, C);
    if (rc != LOLA_OK) return rc;
    if (w < 0) return LOLA_EINVAL;
    if (w > lola::kHolaMaxW) return LOLA_EUNSUPPORTED;
    if (n == 0) return LOLA_OK;
    if (!q || !k || !v || !y || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(y)) return LOLA_EINVAL;
    if (!alpha || !beta || !gamma_q || !gamma_k || !sink || !gate) return LOLA_EINVAL;
    const int64_t nchunks = (n + C - 1) / C;
    const int64_t BH = (int64_t)B * n_heads;
    const int nqt = (C + 63) / 64;
    if (BH * nchunks * nqt > (int64_t)INT_MAX || (BH * n + 7) / 8 > (int64_t)INT_MAX) return LOLA_EUNSUPPORTED;
    const lola::HolaLayout L = hola_layout(BH, d, dtype == LOLA_BF16 ? 2 : 4, n, C, nchunks);
    if (!workspace || ((uintptr_t)workspace & 255u) != 0 || workspace_bytes < (size_t)L.total) return LOLA_EINVAL;
    lola::HolaArgs a;
    a.BH = (int)BH;
    a.heads = n_heads;
    a.n = (int)n;
    a.C = C;
    a.w = w;
    a.nchunks = (int)nchunks;
    a.nqt = nqt;
    a.nblk = (int)((n + lola::kHolaBT - 1) / lola::kHolaBT);
    a.q = q; a.k = k; a.v = v;
    a.alpha = alpha; a.beta = beta;
    a.gamma_q = gamma_q; a.gamma_k = gamma_k;
    a.sink = sink; a.gate = gate;
    a.y = y;
    a.S_out = S_out;
    a.cache_pos_out = w > 0 ? cache_pos_out : nullptr;
    a.cache_score_out = w > 0 ? cache_score_out : nullptr;
    a.ws = reinterpret_cast<char*>(workspace);
    a.L = L;
    a.st_cache_pos = nullptr;
    a.st_cache_score = nullptr;
    a.st_cache_k = a.st_cache_v = a.st_open_k = a.st_open_v = nullptr;
    a.st_open_score = nullptr;
    if (lola::launch_hola(a, dtype, d, (hipStream_t)stream) != hipSuccess) return LOLA_EDEVICE;
    if (getenv("LOLA_DEBUG_SYNC") && hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return LOLA_EDEVICE;
    return LOLA_OK;
}

static lola_status hola_state_check(const hola_state* st) {
    if (!st) return LOLA_EINVAL;
    lola_status rc = hola_check(st->B, st->n_heads, st->d, st->dtype, 0, st->C);
    if (rc != LOLA_OK) return rc;
    if (st->w < 0 || st->t < 0) return LOLA_EINVAL;
    if (st->w > lola::kHolaMaxW) return LOLA_EUNSUPPORTED;
    if (!st->S || !aligned16(st->S) || !st->open_k || !st->open_v || !st->open_score || !aligned16(st->open_k) ||
        !aligned16(st->open_v))
        return LOLA_EINVAL;
    if (st->w > 0 && (!st->cache_pos || !st->cache_score || !st->cache_k || !st->cache_v || !aligned16(st->cache_k) ||
                      !aligned16(st->cache_v)))
        return LOLA_EINVAL;
    return LOLA_OK;
}

lola_status hola_state_init(hola_state* st, void* stream) {
    lola_status rc = hola_state_check(st);
    if (rc != LOLA_OK) return rc;
    lola::HolaInitArgs a;
    a.BH = st->B * st->n_heads;
    a.d = st->d;
    a.w = st->w;
    a.S = st->S;
    a.cache_pos = st->cache_pos;
    a.cache_score = st->cache_score;
    if (lola::launch_hola_init(a, (hipStream_t)stream) != hipSuccess) return LOLA_EDEVICE;
    st->t = 0;
    return LOLA_OK;
}

lola_status hola_prefill_state(hola_state* st, int64_t n, const void* q, const void* k, const void* v,
                               const float* alpha, const float* beta, const float* gamma_q, const float* gamma_k,
                               const float* sink, const float* gate, void* y, void* workspace, size_t workspace_bytes,
                               void* stream) {
    lola_status rc = hola_state_check(st);
    if (rc != LOLA_OK) return rc;
    if (n < 0) return LOLA_EINVAL;
    if (st->t != 0) return LOLA_EUNSUPPORTED;
    if (n == 0) return LOLA_OK;
    rc = hola_check(st->B, st->n_heads, st->d, st->dtype, n, st->C);
    if (rc != LOLA_OK) return rc;
    if (!q || !k || !v || !y || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(y)) return LOLA_EINVAL;
    if (!alpha || !beta || !gamma_q || !gamma_k || !sink || !gate) return LOLA_EINVAL;
    const int32_t C = st->C, d = st->d, dtype = st->dtype;
    const int64_t nchunks = (n + C - 1) / C;
    const int64_t BH = (int64_t)st->B * st->n_heads;
    const int nqt = (C + 63) / 64;
    if (BH * nchunks * nqt > (int64_t)INT_MAX || (BH * n + 7) / 8 > (int64_t)INT_MAX) return LOLA_EUNSUPPORTED;
    const lola::HolaLayout L = hola_layout(BH, d, dtype == LOLA_BF16 ? 2 : 4, n, C, nchunks);
    if (!workspace || ((uintptr_t)workspace & 255u) != 0 || workspace_bytes < (size_t)L.total) return LOLA_EINVAL;
    lola::HolaArgs a;
    a.BH = (int)BH;
    a.heads = st->n_heads;
    a.n = (int)n;
    a.C = C;
    a.w = st->w;
    a.nchunks = (int)nchunks;
    a.nqt = nqt;
    a.nblk = (int)((n + lola::kHolaBT - 1) / lola::kHolaBT);
    a.q = q; a.k = k; a.v = v;
    a.alpha = alpha; a.beta = beta;
    a.gamma_q = gamma_q; a.gamma_k = gamma_k;
    a.sink = sink; a.gate = gate;
    a.y = y;
    a.S_out = st->S;
    a.cache_pos_out = nullptr;
    a.cache_score_out = nullptr;
    a.ws = reinterpret_cast<char*>(workspace);
    a.L = L;
    a.st_cache_pos = st->cache_pos;
    a.st_cache_score = st->cache_score;
    a.st_cache_k = st->cache_k;
    a.st_cache_v = st->cache_v;
    a.st_open_k = st->open_k;
    a.st_open_v = st->open_v;
    a.st_open_score = st->open_score;
    if (lola::launch_hola(a, dtype, d, (hipStream_t)stream) != hipSuccess) return LOLA_EDEVICE;
    if (getenv("LOLA_DEBUG_SYNC") && hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return LOLA_EDEVICE;
    st->t = n;
    return LOLA_OK;
}

lola_status hola_decode_step(hola_state* st, const void* q, const void* k, const void* v, const float* alpha,
                             const float* beta, const float* gamma_q, const float* gamma_k, const float* sink,
                             const float* gate, void* y, void* stream) {
    lola_status rc = hola_state_check(st);
    if (rc != LOLA_OK) return rc;
    if (!q || !k || !v || !y || !alpha || !beta || !gamma_q || !gamma_k || !sink || !gate) return LOLA_EINVAL;
    if (st->t >= (int64_t)INT_MAX) return LOLA_EUNSUPPORTED;   // positions are int32
    lola::HolaDecodeArgs a;
    a.BH = st->B * st->n_heads;
    a.heads = st->n_heads;
    a.C = st->C;
    a.w = st->w;
    a.nopen = (int)(st->t % st->C);
    a.t = st->t;
    a.q = q; a.k = k; a.v = v;
    a.alpha = alpha; a.beta = beta;
    a.gamma_q = gamma_q; a.gamma_k = gamma_k;
    a.sink = sink; a.gate = gate;
    a.y = y;
    a.S = st->S;
    a.cache_pos = st->cache_pos;
    a.cache_score = st->cache_score;
    a.cache_k = st->cache_k;
    a.cache_v = st->cache_v;
    a.open_k = st->open_k;
    a.open_v = st->open_v;
    a.open_score = st->open_score;
    if (lola::launch_hola_decode(a, st->dtype, st->d, (hipStream_t)stream) != hipSuccess) return LOLA_EDEVICE;
    if (getenv("LOLA_DEBUG_SYNC") && hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return LOLA_EDEVICE;
    st->t += 1;
    return LOLA_OK;
}

lola_status lola_sre_collisions(const lola_state* st, const void* v, const int32_t* fold_at, int64_t n,
                                int32_t C, const void* workspace, size_t workspace_bytes, int32_t relative,
                                float* out, void* stream) {
    lola_status rc = check_shape(st);
    if (rc != LOLA_OK) return rc;
    if (!st->H || !st->s || !aligned16(st->H) || !aligned16(st->s)) return LOLA_EINVAL;
    if (n < 0 || C < 1 || (relative != 0 && relative != 1)) return LOLA_EINVAL;
    if (st->dec_chunk != 0) return LOLA_EINVAL;
    if (C > kMaxChunk || n > INT_MAX / 2) return LOLA_EUNSUPPORTED;
    if (n == 0) return LOLA_OK;
    if (!v || !fold_at || !out || !aligned16(v) || !aligned16(fold_at) || !aligned16(out)) return LOLA_EINVAL;
    const WsLayout L = make_layout(st, n, C);
    const size_t need = (size_t)L.per_bh * (size_t)st->B * (size_t)st->n_heads;
    if (!workspace || ((uintptr_t)workspace & 255u) != 0 || workspace_bytes < need) return LOLA_EINVAL;

    lola::CollideArgs a;
    a.BH = st->B * st->n_heads;
    a.n = (int)n;
    a.C = C;
    a.eta = st->eta;
    a.nchunks = L.nchunks;
    a.tok_per_block = lola::kCollideTokensPerBlock;
    a.nblk = (int)((n + a.tok_per_block - 1) / a.tok_per_block);
    a.relative = relative;
    a.v = v;
    a.fold_at = fold_at;
    a.H = st->H;
    a.s = st->s;
    a.ws = reinterpret_cast<const char*>(workspace);
    a.L = L;
    a.out = out;
    if ((int64_t)a.BH * ((a.nchunks + lola::kCollideRows - 1) / lola::kCollideRows) * a.nblk > (int64_t)INT_MAX)
        return LOLA_EUNSUPPORTED;
    if (lola::launch_collide(a, st->dtype, st->d_k, (hipStream_t)stream) != hipSuccess) return LOLA_EDEVICE;
    if (getenv("LOLA_DEBUG_SYNC") && hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return LOLA_EDEVICE;
    return LOLA_OK;
}

}  // extern "C"
