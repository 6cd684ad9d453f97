// Building blocks of the bf16 read-out kernel (lola_readout_fast.hip):
// the query features of two 16-query tiles, the swizzles of staged key and value rows, and the
// transposing LDS read.
#pragma once

#include "lola_common.hpp"

namespace lola {
namespace rd {

constexpr unsigned kNoKey = 0x7FFFFFFFu;   // query-range start of a key that no query reads

// phi of two 16-query tiles (section 2.2), each W^T fragment from LDS serving both: the features as
// MFMA B operands pf[qq][ss] (reduction order over D) and phi(q).s in lden[qq] (this lane's part).
// The query fragments qf and the rows of W^T (16-byte aligned) are in the contiguous order over d_k.
template <int DK, int PHI>
__device__ __forceinline__ void phi_pair(const bf16* wt, int wt_ld, const Frag8<bf16> (&qf)[2][DK / 32],
                                         const float* s, Frag8<bf16> (&pf)[2][kFeat / 32], float (&lden)[2]) {
    constexpr int D = kFeat, DW = (PHI == kPhiSoftmaxPM) ? D / 2 : D;
    const int l = lane_id(), g = l >> 4, c = l & 15;
    f4 pre[DW / 16][2];
#pragma unroll
    for (int ft = 0; ft < DW / 16; ++ft) {
        pre[ft][0] = zero4();
        pre[ft][1] = zero4();
#pragma unroll
        for (int ss = 0; ss < DK / 32; ++ss) {
            const Frag8<bf16> a = load_frag_contig(wt + (16 * ft + c) * wt_ld, ss, g);
            mma32(pre[ft][0], a, qf[0][ss]);
            mma32(pre[ft][1], a, qf[1][ss]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
        float ph[D / 16][4];
        if constexpr (PHI == kPhiSoftmaxPM) {
            float mx = -INFINITY, mn = INFINITY;
#pragma unroll
            for (int ft = 0; ft < DW / 16; ++ft)
#pragma unroll
                for (int r = 0; r < 4; ++r) { mx = fmaxf(mx, pre[ft][qq][r]); mn = fminf(mn, pre[ft][qq][r]); }
            mx = max_groups(mx);
            mn = min_groups(mn);
            float sp = 0.f, sm = 0.f;
#pragma unroll
            for (int ft = 0; ft < DW / 16; ++ft)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float ep = fast_exp(pre[ft][qq][r] - mx);
                    const float em = fast_exp(mn - pre[ft][qq][r]);
                    ph[ft][r] = ep;
                    ph[ft + DW / 16][r] = em;
                    sp += ep;
                    sm += em;
                }
            const float ip = fast_rcp(sum_groups(sp)), im = fast_rcp(sum_groups(sm));
#pragma unroll
            for (int ft = 0; ft < DW / 16; ++ft)
#pragma unroll
                for (int r = 0; r < 4; ++r) { ph[ft][r] *= ip; ph[ft + DW / 16][r] *= im; }
        } else {
#pragma unroll
            for (int ft = 0; ft < DW / 16; ++ft)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float z = pre[ft][qq][r];
                    ph[ft][r] = z > 0.f ? z + 1.f : fast_exp(z);
                }
        }
        float ld = 0.f;
#pragma unroll
        for (int ft = 0; ft < D / 16; ++ft) {
            const f4 sv = *reinterpret_cast<const f4*>(s + 16 * ft + 4 * g);
#pragma unroll
            for (int r = 0; r < 4; ++r) ld += ph[ft][r] * sv[r];
        }
        asm volatile("" : "+v"(ld));      // formed here: the features are not kept live until it is used
        lden[qq] = ld;
#pragma unroll
        for (int ss = 0; ss < D / 32; ++ss)
            pf[qq][ss] = frag_from_acc<bf16>(f4{ph[2 * ss][0], ph[2 * ss][1], ph[2 * ss][2], ph[2 * ss][3]},
                                             f4{ph[2 * ss + 1][0], ph[2 * ss + 1][1], ph[2 * ss + 1][2], ph[2 * ss + 1][3]});
    }
}

// Staged rows are unpadded and swizzled so that fragment reads hit 64 distinct banks:
//   key row r, 16-byte chunk q  -> chunk q ^ ((r / RPB) mod CPK)
//     (a fragment read takes one chunk of 16 consecutive rows, or two halves of it);
//   value row r, 32-byte segment s -> segment s ^ ((r / RPB) mod SEG), chunk halves kept
//     (a transposed read takes one segment of 8 consecutive rows per half-wave).
template <int DK>
__device__ __forceinline__ int kswz(int row, int q) {
    constexpr int RPB = 256 / (2 * DK), CPK = DK / 8;
    return q ^ ((row / RPB) % CPK);
}
template <int DK>
__device__ __forceinline__ int vswz(int row, int q) {
    constexpr int RPB = 256 / (2 * DK), SEG = DK / 16;
    return (((q >> 1) ^ ((row / RPB) % SEG)) << 1) | (q & 1);
}

// Four bf16 of a transposed LDS read (gfx950): in each group of 16 lanes, lanes 4r .. 4r + 3 give
// the addresses of row r (four elements each, sixteen in all) and lane i receives element i of rows
// 0 .. 3.
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (v4s __attribute__((address_space(3)))*)((__attribute__((address_space(3))) char*)p));
    bf16x4 out;
    __builtin_memcpy(&out, &r, sizeof(out));
    return out;
}

}  // namespace rd
}  // namespace lola
