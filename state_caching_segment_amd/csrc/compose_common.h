// Device pieces shared by the sequential compose, the stand-alone seam advance
// and the tree-scan compose (internal to libhypic, gfx950 only).
//
// A wave owns a 32-column tile of a d x (columns) fp32 matrix -- the running
// state S, or one half of a [T | S] pair -- kept in MFMA accumulators in the
// C layout: X[rt][nt][jj] holds row 16*rt + 4*grp + jj, column 16*nt + r16 of
// the tile (lane = 16*grp + r16).
#pragma once
#include <type_traits>

#include "common.h"

namespace hy {

constexpr int SEAM_STAGE = 8;  // seam tokens staged in LDS at a time

// Up to SEAM_STAGE seam tokens of one chain, fp32; decays already exponentiated.
// a[t][i]: per-row decay (GLA, KDA); a[t][0]: scalar decay (other families).
template <int D, int FAM>
struct SeamSmem {
    float q[SEAM_STAGE][D];
    float k[SEAM_STAGE][D];
    float v[SEAM_STAGE][D];
    float a[SEAM_STAGE][fam_vgate(FAM) ? D : 1];
    float beta[SEAM_STAGE];
};

// The same stage with q, k, v kept as bf16 (bf16 inputs, scalar gates): half
// the LDS, and the rows are matrix-core operands as they stand.
template <int D>
struct SeamSmemB {
    bf16 q[SEAM_STAGE][D];
    bf16 k[SEAM_STAGE][D];
    bf16 v[SEAM_STAGE][D];
    float a[SEAM_STAGE][1];
    float beta[SEAM_STAGE];
};

// A stage of KDA seam tokens in the decayed forms the chunk seam uses: with
// E_t the window's cumulative per-channel decay through token t and E_c that
// of its last token, rows E_t o k_t and E_t o q_t, k_t / E_t, (E_c / E_t) o k_t,
// v_t, and E_c itself.  (Tokens past nt are zero tokens with decay 1.)  The
// decayed rows are matrix-core operands, stored once already split into hi
// and lo bf16 (so that no wave repeats the split): the row forms with the
// channels of each 32-block in the permuted k order (kda_seam_pos), E_t o k_t
// in rows 0-7 and E_t o q_t in rows 8-15 of lq; (E_c / E_t) o k_t transposed,
// one 16-byte row of eight tokens per channel.
template <int D>
struct __attribute__((aligned(16))) SeamSmemKda {
    bf16 lqh[2 * SEAM_STAGE][D], lql[2 * SEAM_STAGE][D];
    bf16 kbh[SEAM_STAGE][D], kbl[SEAM_STAGE][D];
    bf16 kth[D][SEAM_STAGE], ktl[D][SEAM_STAGE];
    float v[SEAM_STAGE][D];
    float ecl[D];
    float beta[SEAM_STAGE];
};

// Position of channel i in a permuted row: within each 32-block, lane group g
// reads positions 8g .. 8g+7, which hold channels 4g .. 4g+3 and
// 16+4g .. 16+4g+3 (the permuted k subset of the matrix-core convention).
__device__ __forceinline__ int kda_seam_pos(int i) {
    const int c = i & 31;
    return (i & ~31) + 8 * ((c & 15) >> 2) + 4 * (c >> 4) + (c & 3);
}

// Token t of channel i of a KDA seam stage, from its values (zero past nt),
// its cumulative decay et = E_t and the window's E_c = pr.
template <int D>
__device__ __forceinline__ void kda_stage_tok(SeamSmemKda<D> &sm, int i, int t, float qv, float kv, float vv, float et,
                                              float pr) {
    const int pi = kda_seam_pos(i);
    bf16 h, l;
    split1(et * kv, h, l);
    sm.lqh[t][pi] = h;
    sm.lql[t][pi] = l;
    split1(et * qv, h, l);
    sm.lqh[SEAM_STAGE + t][pi] = h;
    sm.lql[SEAM_STAGE + t][pi] = l;
    split1(kv / et, h, l);
    sm.kbh[t][pi] = h;
    sm.kbl[t][pi] = l;
    split1(kv * (pr / et), h, l);
    sm.kth[i][t] = h;
    sm.ktl[i][t] = l;
    sm.v[t][i] = vv;
}

// Cumulative decays of channel i over the window from its log-gates (e^g as
// 2^(g log2 e)); tokens past nt and padded channels decay by 1.  Returns E_c.
__device__ __forceinline__ float kda_window_decay(const float (&gv)[SEAM_STAGE], int i, int dk, int nt,
                                                  float (&e)[SEAM_STAGE]) {
    float p = 1.f;
#pragma unroll
    for (int t = 0; t < SEAM_STAGE; ++t) {
        p *= (t < nt && i < dk) ? __builtin_amdgcn_exp2f(gv[t] * 1.4426950408889634f) : 1.f;
        e[t] = p;
    }
    return p;
}

// e[t] for a token index known only at run time (no dynamic register index).
__device__ __forceinline__ float kda_pick(const float (&e)[SEAM_STAGE], int t) {
    float r = e[0];
#pragma unroll
    for (int s = 1; s < SEAM_STAGE; ++s) r = t == s ? e[s] : r;
    return r;
}

// Channel i's column of a KDA seam stage, from its window values (zeroed past
// nt), cumulative decays e[t] = E_t and E_c = pr.
template <int D>
__device__ __forceinline__ void kda_stage_write(SeamSmemKda<D> &sm, int i, const float (&qv)[SEAM_STAGE],
                                                const float (&kv)[SEAM_STAGE], const float (&vv)[SEAM_STAGE],
                                                const float (&e)[SEAM_STAGE], float pr) {
    const int pi = kda_seam_pos(i);
    bf16x8 th, tl;
#pragma unroll
    for (int t = 0; t < SEAM_STAGE; ++t) {
        bf16 h, l;
        split1(e[t] * kv[t], h, l);
        sm.lqh[t][pi] = h;
        sm.lql[t][pi] = l;
        split1(e[t] * qv[t], h, l);
        sm.lqh[SEAM_STAGE + t][pi] = h;
        sm.lql[SEAM_STAGE + t][pi] = l;
        split1(kv[t] / e[t], h, l);
        sm.kbh[t][pi] = h;
        sm.kbl[t][pi] = l;
        split1(kv[t] * (pr / e[t]), h, l);
        th[t] = h;
        tl[t] = l;
        sm.v[t][i] = vv[t];
    }
    *reinterpret_cast<bf16x8 *>(&sm.kth[i][0]) = th;
    *reinterpret_cast<bf16x8 *>(&sm.ktl[i][0]) = tl;
    sm.ecl[i] = pr;
}

template <int D, typename TIN>
__device__ void stage_seam_kda(SeamSmemKda<D> &sm, const Tok &x, int chain, int dk, int64_t tok0, int nt) {
    const int tid = threadIdx.x;
    const TIN *qp = reinterpret_cast<const TIN *>(x.q) + (int64_t)chain * x.cs;
    const TIN *kp = reinterpret_cast<const TIN *>(x.k) + (int64_t)chain * x.cs;
    const TIN *vp = reinterpret_cast<const TIN *>(x.v) + (int64_t)chain * x.cs;
    const TIN *gp = reinterpret_cast<const TIN *>(x.g) + (int64_t)chain * x.gcs;
    // one thread per channel (every launch has at least d threads): the
    // window's 4 x SEAM_STAGE loads are all issued before any is used
    if (tid < D) {
        const int i = tid, ic = i < dk ? i : dk - 1;
        float qv[SEAM_STAGE], kv[SEAM_STAGE], vv[SEAM_STAGE], gv[SEAM_STAGE];
#pragma unroll
        for (int t = 0; t < SEAM_STAGE; ++t) {
            const int64_t tc = tok0 + (t < nt ? t : nt - 1);
            qv[t] = ldf(qp + tc * x.ts + ic);
            kv[t] = ldf(kp + tc * x.ts + ic);
            vv[t] = ldf(vp + tc * x.ts + ic);
            gv[t] = ldf(gp + tc * x.gts + ic);
        }
        float e[SEAM_STAGE], p = 1.f;
#pragma unroll
        for (int t = 0; t < SEAM_STAGE; ++t) {
            const bool ok = t < nt && i < dk;
            p *= ok ? __builtin_amdgcn_exp2f(gv[t] * 1.4426950408889634f) : 1.f;  // e^g as 2^(g log2 e)
            e[t] = p;
            if (!ok) qv[t] = kv[t] = vv[t] = 0.f;
        }
        kda_stage_write<D>(sm, i, qv, kv, vv, e, p);
    }
    if (tid < SEAM_STAGE) {
        const int t = tid;
        const int64_t tc = tok0 + (t < nt ? t : nt - 1);
        const float bv = ldf(reinterpret_cast<const TIN *>(x.beta) + (int64_t)chain * x.bcs + tc * x.bts);
        sm.beta[t] = t < nt ? bv : 1.f;
    }
}

// Stage tokens tok0 .. tok0+nt-1 of `chain` into bf16 rows (scalar-gate
// families; rows past nt are zero tokens with a = beta = 1).
template <int D, int FAM>
__device__ void stage_seam_b(SeamSmemB<D> &sm, const Tok &x, int chain, int64_t tok0, int nt) {
    const int tid = threadIdx.x, nthr = blockDim.x;
    const bf16 *qp = reinterpret_cast<const bf16 *>(x.q) + (int64_t)chain * x.cs;
    const bf16 *kp = reinterpret_cast<const bf16 *>(x.k) + (int64_t)chain * x.cs;
    const bf16 *vp = reinterpret_cast<const bf16 *>(x.v) + (int64_t)chain * x.cs;
    for (int item = tid; item < SEAM_STAGE * D; item += nthr) {
        const int t = item / D, i = item % D;
        const bool ok = t < nt;
        const int64_t off = (tok0 + (ok ? t : nt - 1)) * x.ts + i;
        const bf16 qv = qp[off], kv = kp[off], vv = vp[off];
        sm.q[t][i] = ok ? qv : (bf16)0.f;
        sm.k[t][i] = ok ? kv : (bf16)0.f;
        sm.v[t][i] = ok ? vv : (bf16)0.f;
    }
    if (tid < SEAM_STAGE) {
        const int t = tid;
        const int64_t tc = tok0 + (t < nt ? t : nt - 1);
        float av = 1.f, bv = 1.f;
        if (fam_sgate(FAM)) av = expf(ldf(reinterpret_cast<const bf16 *>(x.g) + (int64_t)chain * x.gcs + tc * x.gts));
        if (fam_beta(FAM)) bv = ldf(reinterpret_cast<const bf16 *>(x.beta) + (int64_t)chain * x.bcs + tc * x.bts);
        sm.a[t][0] = t < nt ? av : 1.f;
        sm.beta[t] = t < nt ? bv : 1.f;
    }
}

// Stage tokens tok0 .. tok0+nt-1 of `chain` (rows past nt are zero tokens).
template <int D, int FAM, typename TIN>
__device__ void stage_seam(SeamSmem<D, FAM> &sm, const Tok &x, int chain, int dk, int64_t tok0, int nt) {
    const int tid = threadIdx.x, nthr = blockDim.x;
    const TIN *qp = reinterpret_cast<const TIN *>(x.q) + (int64_t)chain * x.cs;
    const TIN *kp = reinterpret_cast<const TIN *>(x.k) + (int64_t)chain * x.cs;
    const TIN *vp = reinterpret_cast<const TIN *>(x.v) + (int64_t)chain * x.cs;
    // loads are unconditional, from indices clamped into the valid range, and
    // masked afterwards: a load under a branch would make every one of them
    // wait for its data before the branch closes
    for (int item = tid; item < SEAM_STAGE * D; item += nthr) {
        const int t = item / D, i = item % D;
        const bool ok = t < nt && i < dk;
        const int64_t off = (tok0 + (t < nt ? t : nt - 1)) * x.ts + (i < dk ? i : dk - 1);
        const float qv = ldf(qp + off), kv = ldf(kp + off), vv = ldf(vp + off);
        sm.q[t][i] = ok ? qv : 0.f;
        sm.k[t][i] = ok ? kv : 0.f;
        sm.v[t][i] = ok ? vv : 0.f;
        if (fam_vgate(FAM)) {
            const float gv = ldf(reinterpret_cast<const TIN *>(x.g) + (int64_t)chain * x.gcs +
                                 (tok0 + (t < nt ? t : nt - 1)) * x.gts + (i < dk ? i : dk - 1));
            sm.a[t][i] = ok ? expf(gv) : 1.f;
        }
    }
    if (tid < SEAM_STAGE) {
        const int t = tid;
        const int64_t tc = tok0 + (t < nt ? t : nt - 1);
        float av = 1.f, bv = 1.f;
        if (fam_sgate(FAM)) av = expf(ldf(reinterpret_cast<const TIN *>(x.g) + (int64_t)chain * x.gcs + tc * x.gts));
        if (FAM == RETNET) av = x.gamma[chain];
        if (fam_beta(FAM)) bv = ldf(reinterpret_cast<const TIN *>(x.beta) + (int64_t)chain * x.bcs + tc * x.bts);
        if (!fam_vgate(FAM)) sm.a[t][0] = t < nt ? av : 1.f;
        sm.beta[t] = t < nt ? bv : 1.f;
    }
}

// The token recurrence S_t = A_t S_{t-1} + beta_t k_t v_t^T on this wave's
// tile, for nt staged tokens, writing o_t = S_t^T q_t for every token:
// o_first[t * o_tok_stride + ocol + c] for tile column c < ncols - ocol.
// vcol: the tile's first column in v; v_zero: the tile's v is zero (the T half
// of a [T | S] pair, which then yields T^T q, the pulled-back query).
template <int D, int FAM>
__device__ void seam_tokens(f32x4 (&X)[D / 16][2], const SeamSmem<D, FAM> &sm, int nt, float *o_first,
                            int64_t o_tok_stride, int ocol, int vcol, bool v_zero, int ncols) {
    constexpr int RT = D / 16;
    const int lane = lane_id(), r16 = lane & 15, grp = lane >> 4;
    for (int t = 0; t < nt; ++t) {
        if (fam_vgate(FAM)) {
            // per-row decay first: alone (GLA) or before the erase (KDA)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const f32x4 a4 = *reinterpret_cast<const f32x4 *>(&sm.a[t][16 * rt + 4 * grp]);
#pragma unroll
                for (int nt2 = 0; nt2 < 2; ++nt2)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) X[rt][nt2][jj] *= a4[jj];
            }
        }
        const float sa = fam_vgate(FAM) ? 1.f : sm.a[t][0];
        const float bt = sm.beta[t];
        float vc[2];
#pragma unroll
        for (int nt2 = 0; nt2 < 2; ++nt2) vc[nt2] = v_zero ? 0.f : sm.v[t][vcol + 16 * nt2 + r16];
        if (fam_dense(FAM)) {
            // p = k^T S per column, then S <- a (S - beta k p) + beta k v
            float p[2] = {0.f, 0.f};
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const f32x4 k4 = *reinterpret_cast<const f32x4 *>(&sm.k[t][16 * rt + 4 * grp]);
#pragma unroll
                for (int nt2 = 0; nt2 < 2; ++nt2)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) p[nt2] += k4[jj] * X[rt][nt2][jj];
            }
            float coef[2];
#pragma unroll
            for (int nt2 = 0; nt2 < 2; ++nt2) coef[nt2] = bt * (vc[nt2] - sa * wave_sum16x(p[nt2]));
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const f32x4 k4 = *reinterpret_cast<const f32x4 *>(&sm.k[t][16 * rt + 4 * grp]);
#pragma unroll
                for (int nt2 = 0; nt2 < 2; ++nt2)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) X[rt][nt2][jj] = sa * X[rt][nt2][jj] + k4[jj] * coef[nt2];
            }
        } else {
            // S <- a S + k v^T
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const f32x4 k4 = *reinterpret_cast<const f32x4 *>(&sm.k[t][16 * rt + 4 * grp]);
#pragma unroll
                for (int nt2 = 0; nt2 < 2; ++nt2)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) X[rt][nt2][jj] = sa * X[rt][nt2][jj] + k4[jj] * vc[nt2];
            }
        }
        float o[2] = {0.f, 0.f};
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const f32x4 q4 = *reinterpret_cast<const f32x4 *>(&sm.q[t][16 * rt + 4 * grp]);
#pragma unroll
            for (int nt2 = 0; nt2 < 2; ++nt2)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) o[nt2] += q4[jj] * X[rt][nt2][jj];
        }
#pragma unroll
        for (int nt2 = 0; nt2 < 2; ++nt2) {
            const float ov = wave_sum16x(o[nt2]);
            const int col = ocol + 16 * nt2 + r16;
            if (grp == 0 && col < ncols) o_first[t * o_tok_stride + col] = ov;
        }
    }
}

// Lane i of each quad of lanes holds row i of a 4 x 4 block (4 fp32); after
// the exchange it holds column i (DPP quad permutations: swap neighbours, then
// swap pairs).
template <int CTRL>
__device__ __forceinline__ float quad_move(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ f32x4 quad_transpose(f32x4 r, int lane) {
    const bool odd = lane & 1, hi = lane & 2;
    float t = quad_move<0xB1>(odd ? r[0] : r[1]);  // quad_perm [1,0,3,2]
    if (odd) r[0] = t; else r[1] = t;
    t = quad_move<0xB1>(odd ? r[2] : r[3]);
    if (odd) r[2] = t; else r[3] = t;
    const float t0 = quad_move<0x4E>(hi ? r[0] : r[2]);  // quad_perm [2,3,0,1]
    const float t1 = quad_move<0x4E>(hi ? r[1] : r[3]);
    if (hi) {
        r[0] = t0;
        r[1] = t1;
    } else {
        r[2] = t0;
        r[3] = t1;
    }
    return r;
}

// One seam stage's tokens, fetched into registers ahead of use: thread tid
// (tid < 2d) covers token tid / (D/4), features 4 (tid % (D/4)) .. +3 of q, k
// and v, and (for the first feature quad) the token's gate and beta.
template <int D, typename TIN>
struct SeamPrefetch {
    using V4 = typename std::conditional<std::is_same<TIN, float>::value, f32x4, bf16x4>::type;
    V4 q, k, v;
    V4 gv;  // per-channel log-gates (GLA)
    // gate and beta as raw bits in full registers (a bf16 sits in the low
    // half): 16-bit values packed into one register would be combined right
    // after the load, which waits for every load issued before them
    uint32_t g, b;
};

// A raw buffer view of nbytes from p (p wave-uniform); reads past nbytes return
// zero without touching memory, so a view of 0 bytes reads as all zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_view(const void *p, int nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, nbytes, 0x00020000);
}

template <typename TIN>
__device__ __forceinline__ uint32_t buffer_scalar_bits(__amdgpu_buffer_rsrc_t r, int off) {
    if constexpr (std::is_same<TIN, float>::value)
        return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    else
        return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

template <typename TIN>
__device__ __forceinline__ float scalar_from_bits(uint32_t u) {
    if constexpr (std::is_same<TIN, float>::value)
        return __builtin_bit_cast(float, u);
    else
        return __builtin_bit_cast(float, u << 16);
}

// Fetch the seam stage of tokens tok0 .. tok0 + nt - 1 of `chain`; when the
// entry has no seam (tok0 < 0) every view is empty and the registers read as
// zero.  The loads are the same on every path, so the compiler can count
// them and later waits cover only what they need.
template <int D, int FAM, typename TIN>
__device__ __forceinline__ void seam_fetch(SeamPrefetch<D, TIN> &p, const Tok &x, int chain, int dk, int64_t tok0, int nt) {
    using V4 = typename SeamPrefetch<D, TIN>::V4;
    // threads past the stage's 2d items (workgroups wider than d/32 waves)
    // repeat the first ones' loads and write nothing in seam_put
    const int tid = threadIdx.x, t = (tid / (D / 4)) % SEAM_STAGE, i = 4 * (tid % (D / 4));
    const bool on = tok0 >= 0;
    const int64_t tb = on ? tok0 : 0;
    const int row_bytes = (int)(((int64_t)(nt - 1) * x.ts + dk) * sizeof(TIN));
    const int off = (int)(((int64_t)t * x.ts + i) * sizeof(TIN));
    const int64_t base = (int64_t)chain * x.cs + tb * x.ts;
    auto ld4 = [&](const void *ptr) -> V4 {
        const auto r = buffer_view(reinterpret_cast<const TIN *>(ptr) + base, on ? row_bytes : 0);
        if constexpr (std::is_same<TIN, float>::value)
            return __builtin_bit_cast(V4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
        else
            return __builtin_bit_cast(V4, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    };
    p.q = ld4(x.q);
    p.k = ld4(x.k);
    p.v = ld4(x.v);
    if constexpr (fam_vgate(FAM)) {
        const auto r = buffer_view(reinterpret_cast<const TIN *>(x.g) + (int64_t)chain * x.gcs + tb * x.gts,
                                   on ? (int)(((int64_t)(nt - 1) * x.gts + dk) * sizeof(TIN)) : 0);
        const int goff = (int)(((int64_t)t * x.gts + i) * sizeof(TIN));
        if constexpr (std::is_same<TIN, float>::value)
            p.gv = __builtin_bit_cast(V4, __builtin_amdgcn_raw_buffer_load_b128(r, goff, 0, 0));
        else
            p.gv = __builtin_bit_cast(V4, __builtin_amdgcn_raw_buffer_load_b64(r, goff, 0, 0));
    }
    if (fam_sgate(FAM)) {
        const auto r = buffer_view(reinterpret_cast<const TIN *>(x.g) + (int64_t)chain * x.gcs + tb * x.gts,
                                   on ? (int)(((int64_t)(nt - 1) * x.gts + 1) * sizeof(TIN)) : 0);
        p.g = buffer_scalar_bits<TIN>(r, (int)((int64_t)t * x.gts * sizeof(TIN)));
    }
    if (fam_beta(FAM)) {
        const auto r = buffer_view(reinterpret_cast<const TIN *>(x.beta) + (int64_t)chain * x.bcs + tb * x.bts,
                                   on ? (int)(((int64_t)(nt - 1) * x.bts + 1) * sizeof(TIN)) : 0);
        p.b = buffer_scalar_bits<TIN>(r, (int)((int64_t)t * x.bts * sizeof(TIN)));
    }
}

// KDA seam stage fetched ahead into registers: thread i holds channel i % D of
// every token of the stage (the layout the staging's per-channel decay
// product needs), as raw bits; threads past d repeat loads and write nothing.
// When the entry has no seam (tok0 < 0) every view is empty and the values
// read as zero; so do tokens past nt.
// A KDA seam window fetched ahead into registers, spread over NG threads per
// channel (the launch has NG * d threads): thread (group gq, channel i) holds
// every gate of channel i and the q, k, v of tokens gq * SEAM_STAGE / NG
// onwards.
template <int D, typename TIN, int NG>
struct KdaSeamPrefetch {
    uint32_t g[SEAM_STAGE];
    uint32_t q[SEAM_STAGE / NG], k[SEAM_STAGE / NG], v[SEAM_STAGE / NG];
    uint32_t b;  // beta of token tid (threads tid < SEAM_STAGE)
};

template <int D, typename TIN, int NG>
__device__ __forceinline__ void seam_fetch_kda(KdaSeamPrefetch<D, TIN, NG> &p, const Tok &x, int chain, int dk,
                                               int64_t tok0, int nt) {
    constexpr int TPG = SEAM_STAGE / NG;
    const int tid = threadIdx.x, i = tid % D, t0 = NG == 1 ? 0 : tid / D * TPG, ic = i < dk ? i : dk - 1;
    const bool on = tok0 >= 0;
    const int64_t tb = on ? tok0 : 0;
    const int rb = on ? (int)(((int64_t)(nt - 1) * x.ts + dk) * sizeof(TIN)) : 0;
    const int gb = on ? (int)(((int64_t)(nt - 1) * x.gts + dk) * sizeof(TIN)) : 0;
    const int64_t base = (int64_t)chain * x.cs + tb * x.ts;
    const auto rq = buffer_view(reinterpret_cast<const TIN *>(x.q) + base, rb);
    const auto rk = buffer_view(reinterpret_cast<const TIN *>(x.k) + base, rb);
    const auto rv = buffer_view(reinterpret_cast<const TIN *>(x.v) + base, rb);
    const auto rg = buffer_view(reinterpret_cast<const TIN *>(x.g) + (int64_t)chain * x.gcs + tb * x.gts, gb);
#pragma unroll
    for (int t = 0; t < SEAM_STAGE; ++t)
        p.g[t] = buffer_scalar_bits<TIN>(rg, (int)(((int64_t)t * x.gts + ic) * sizeof(TIN)));
#pragma unroll
    for (int u = 0; u < TPG; ++u) {
        const int off = (int)(((int64_t)(t0 + u) * x.ts + ic) * sizeof(TIN));
        p.q[u] = buffer_scalar_bits<TIN>(rq, off);
        p.k[u] = buffer_scalar_bits<TIN>(rk, off);
        p.v[u] = buffer_scalar_bits<TIN>(rv, off);
    }
    const int tt = tid % SEAM_STAGE;
    const auto rbeta = buffer_view(reinterpret_cast<const TIN *>(x.beta) + (int64_t)chain * x.bcs + tb * x.bts,
                                   on ? (int)(((int64_t)(nt - 1) * x.bts + 1) * sizeof(TIN)) : 0);
    p.b = buffer_scalar_bits<TIN>(rbeta, (int)((int64_t)tt * x.bts * sizeof(TIN)));
}

// Stage a fetched KDA seam window in the decayed forms (the arithmetic of
// stage_seam_kda, from registers): each thread forms its channel's cumulative
// decays from all the gates and writes its group's tokens.
template <int D, typename TIN, int NG>
__device__ __forceinline__ void seam_put_kda(SeamSmemKda<D> &sm, const KdaSeamPrefetch<D, TIN, NG> &p, int dk,
                                             int nt) {
    constexpr int TPG = SEAM_STAGE / NG;
    const int tid = threadIdx.x;
    if (tid < NG * D) {
        const int i = tid % D, t0 = NG == 1 ? 0 : tid / D * TPG;
        float gv[SEAM_STAGE], e[SEAM_STAGE];
#pragma unroll
        for (int t = 0; t < SEAM_STAGE; ++t) gv[t] = scalar_from_bits<TIN>(p.g[t]);
        const float pr = kda_window_decay(gv, i, dk, nt, e);
#pragma unroll
        for (int u = 0; u < TPG; ++u) {
            const int t = t0 + u;
            const bool ok = t < nt && i < dk;
            kda_stage_tok<D>(sm, i, t, ok ? scalar_from_bits<TIN>(p.q[u]) : 0.f,
                             ok ? scalar_from_bits<TIN>(p.k[u]) : 0.f, ok ? scalar_from_bits<TIN>(p.v[u]) : 0.f,
                             kda_pick(e, t), pr);
        }
        if (t0 == 0) sm.ecl[i] = pr;
    }
    if (tid < SEAM_STAGE) sm.beta[tid] = tid < nt ? scalar_from_bits<TIN>(p.b) : 1.f;
}

// Write a fetched stage into the LDS staging area (zero tokens past nt); the
// scalar decay is e^g (Mamba2, GDN), retnet_gamma (RetNet) or 1.
template <int D, int FAM, typename TIN>
__device__ __forceinline__ void seam_put(SeamSmem<D, FAM> &sm, const SeamPrefetch<D, TIN> &p, int dk, int nt,
                                         float retnet_gamma = 1.f) {
    const int tid = threadIdx.x, t = tid / (D / 4), i = 4 * (tid % (D / 4));
    if (t >= SEAM_STAGE) return;  // (wave-uniform: whole waves past the stage's items)
    const bool ok = t < nt && i < dk;
    f32x4 q4, k4, v4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        q4[e] = ok ? (float)p.q[e] : 0.f;
        k4[e] = ok ? (float)p.k[e] : 0.f;
        v4[e] = ok ? (float)p.v[e] : 0.f;
    }
    *reinterpret_cast<f32x4 *>(&sm.q[t][i]) = q4;
    *reinterpret_cast<f32x4 *>(&sm.k[t][i]) = k4;
    *reinterpret_cast<f32x4 *>(&sm.v[t][i]) = v4;
    if constexpr (fam_vgate(FAM)) {
        f32x4 a4;
#pragma unroll
        for (int e = 0; e < 4; ++e) a4[e] = ok ? expf((float)p.gv[e]) : 1.f;
        *reinterpret_cast<f32x4 *>(&sm.a[t][i]) = a4;
    }
    if (i == 0) {
        if constexpr (!fam_vgate(FAM))
            sm.a[t][0] = t >= nt ? 1.f : fam_sgate(FAM) ? expf(scalar_from_bits<TIN>(p.g)) : retnet_gamma;
        sm.beta[t] = (fam_beta(FAM) && t < nt) ? scalar_from_bits<TIN>(p.b) : 1.f;
    }
}

// Write a fetched stage (bf16 inputs) into bf16 staging rows.
template <int D, int FAM>
__device__ __forceinline__ void seam_put_b(SeamSmemB<D> &sm, const SeamPrefetch<D, bf16> &p, int nt) {
    const int tid = threadIdx.x, t = tid / (D / 4), i = 4 * (tid % (D / 4));
    if (t >= SEAM_STAGE) return;  // (wave-uniform: whole waves past the stage's items)
    const bool ok = t < nt;
    const bf16x4 z = {(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
    *reinterpret_cast<bf16x4 *>(&sm.q[t][i]) = ok ? p.q : z;
    *reinterpret_cast<bf16x4 *>(&sm.k[t][i]) = ok ? p.k : z;
    *reinterpret_cast<bf16x4 *>(&sm.v[t][i]) = ok ? p.v : z;
    if (i == 0) {
        sm.a[t][0] = (fam_sgate(FAM) && ok) ? expf(scalar_from_bits<bf16>(p.g)) : 1.f;
        sm.beta[t] = (fam_beta(FAM) && ok) ? scalar_from_bits<bf16>(p.b) : 1.f;
    }
}

typedef short s4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s4v bf4(float a, float b, float c, float d) {
    return s4v{__builtin_bit_cast(short, (bf16)a), __builtin_bit_cast(short, (bf16)b), __builtin_bit_cast(short, (bf16)c),
               __builtin_bit_cast(short, (bf16)d)};
}

__device__ __forceinline__ void split4v(const f32x4 &x, s4v &h, s4v &l) {
    u32x2 hu, lu;
    uint32_t a, b;
    split2(x[0], x[1], a, b);
    hu[0] = a;
    lu[0] = b;
    split2(x[2], x[3], a, b);
    hu[1] = a;
    lu[1] = b;
    h = __builtin_bit_cast(s4v, hu);
    l = __builtin_bit_cast(s4v, lu);
}

__device__ __forceinline__ f32x4 mfma16(const s4v &a, const s4v &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Up to SEAM_STAGE seam tokens of a scalar-gate erasing family (DeltaNet,
// GDN) with bf16-exact staged q, k, v, as one chunk on the matrix cores
// (HYPIC, codernav.top article, section on seam windows: the window's state
// and outputs are computed on the fly).  With S0 the state entering the chunk,
// a_t = e^{g_t}, e_t = a_0 .. a_t, D_ti = a_{i+1} .. a_t (t >= i),
// lambda = e_{c-1}, ec_t = a_{t+1} .. a_{c-1}:
//     Y = V - diag(e) K S0,   R = (I + N)^-1 diag(beta) Y,
//     N_ti = beta_t (k_t . k_i) D_ti (t > i),
//     o_t = e_t q_t^T S0 + sum_{i<=t} (q_t . k_i) D_ti R_i,
//     S   = lambda S0 + K^T diag(ec) R,
// which is the token recurrence S_t = a_t (I - beta_t k_t k_t^T) S_{t-1} +
// beta_t k_t v_t^T, o_t = S_t^T q_t, regrouped.  Every decay factor is a
// product of a's, so none exceeds 1.  Tokens past nt are zero tokens with
// a = beta = 1.  sNw, sMw: this wave's 8 x 9 fp32 scratch.  v_zero: the
// tile's values are zero (the T half of a [T | S] pair), which makes the
// read-out T^T q, the pulled-back query.
template <int D, int FAM, typename SM, bool UPDATE_FIRST = false>
__device__ void seam_chunk_bf16(f32x4 (&X)[D / 16][2], const SM &sm, int nt, float *o_first,
                                int64_t o_tok_stride, int c0, int dk, float (*sNw)[9], float (*sMw)[9],
                                bool v_zero = false) {
    constexpr int RT = D / 16, KB = D / 32;
    const int lane = lane_fresh(), r16 = lane & 15, grp = lane >> 4;
    float a[SEAM_STAGE], eg[SEAM_STAGE], ec[SEAM_STAGE];
#pragma unroll
    for (int t = 0; t < SEAM_STAGE; ++t) a[t] = FAM == GDN ? sm.a[t][0] : 1.f;
    {
        float p = 1.f;
#pragma unroll
        for (int t = 0; t < SEAM_STAGE; ++t) eg[t] = p = p * a[t];
        p = 1.f;
#pragma unroll
        for (int t = SEAM_STAGE - 1; t >= 0; --t) {
            ec[t] = p;
            p *= a[t];
        }
    }
    const float lam = eg[SEAM_STAGE - 1];
    using E = typename std::remove_cv<typename std::remove_reference<decltype(sm.k[0][0])>::type>::type;
    constexpr bool B16 = std::is_same<E, bf16>::value;
    // The staged values the state update needs, read first (they do not
    // depend on the state, so their LDS latency overlaps the products below):
    // lane (r16, grp < 2) takes k rows 4 grp .. 4 grp + 3 of column 16 rt + r16
    // (the A operand of K^T) and v rows 4 grp .. of its two columns.  The reads
    // are unconditional (rows wrapped into the stage) and masked afterwards.
    s4v ktv[RT];
    float vv[2][4];
    {
        const int r0 = (4 * grp) & (SEAM_STAGE - 1);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            s4v k4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (B16)
                    k4[e] = __builtin_bit_cast(short, sm.k[r0 + e][16 * rt + r16]);
                else
                    k4[e] = __builtin_bit_cast(short, (bf16)sm.k[r0 + e][16 * rt + r16]);
            }
            ktv[rt] = grp < 2 ? k4 : s4v{0, 0, 0, 0};
        }
#pragma unroll
        for (int n2 = 0; n2 < 2; ++n2) {
            const int col = c0 + 16 * n2 + r16;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float v = (float)sm.v[r0 + jj][col < D ? col : D - 1];
                vv[n2][jj] = (grp < 2 && !v_zero) ? v : 0.f;
            }
        }
    }
    // P = [K; Q] S0 (rows 0-7: K S0, rows 8-15: Q S0) and the Gram [K;Q][K;Q]^T
    const E *qk = r16 < 8 ? &sm.k[r16][0] : &sm.q[r16 - 8][0];
    f32x4 P[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    f32x4 G = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        bf16x8 af;
        if constexpr (B16) {
            af = lds_perm(qk, 0, 0, 32 * kb, grp);
        } else {
            const f32x4 u = *reinterpret_cast<const f32x4 *>(qk + 32 * kb + 4 * grp);
            const f32x4 w = *reinterpret_cast<const f32x4 *>(qk + 32 * kb + 16 + 4 * grp);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                af[e] = (bf16)u[e];
                af[4 + e] = (bf16)w[e];
            }
        }
        G = mfma(af, af, G);
#pragma unroll
        for (int n2 = 0; n2 < 2; ++n2) {
            float xv[8];
            bf16x8 xh, xl;
            acc_to_perm(X[2 * kb][n2], X[2 * kb + 1][n2], xv);
            split8(xv, xh, xl);
            P[n2] = mfma(af, xh, P[n2]);
            P[n2] = mfma(af, xl, P[n2]);
        }
    }
    // G in C layout: lane (r16 = i, grp) holds row 4 grp + jj.  Rows 0-7 give
    // N (t > i), rows 8-15 give M (i <= t) for t = row - 8.
    if (r16 < 8) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int row = 4 * grp + jj, t = row & 7, i = r16;
            float dti = 1.f;
#pragma unroll
            for (int j = 1; j < SEAM_STAGE; ++j)
                if (i < j && j <= t) dti *= a[j];
            if (row < 8)
                sNw[t][i] = t > i ? sm.beta[t] * G[jj] * dti : 0.f;
            else
                sMw[t][i] = i <= t ? G[jj] * dti : 0.f;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // row r16 of (I + N)^-1 diag(beta): y (I + N) = e_r, swept from the last row up
    float y[SEAM_STAGE];
#pragma unroll
    for (int j = 0; j < SEAM_STAGE; ++j) y[j] = (j == r16) ? 1.f : 0.f;
#pragma unroll
    for (int i = SEAM_STAGE - 1; i > 0; --i)
#pragma unroll
        for (int j = 0; j < i; ++j) y[j] -= y[i] * sNw[i][j];
    // (register arrays are indexed only with unrolled constants: lane group
    // 0 takes entries 0-3, lane group 1 entries 4-7)
    f32x4 arow = {0.f, 0.f, 0.f, 0.f}, mrow = {0.f, 0.f, 0.f, 0.f};
    if (grp < 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = 4 * grp + e;
            arow[e] = r16 < 8 ? (grp == 0 ? y[e] : y[4 + e]) * sm.beta[j] : 0.f;
            mrow[e] = r16 >= 8 ? sMw[r16 - 8][j] : 0.f;
        }
    }
    f32x4 eg4 = {eg[0], eg[1], eg[2], eg[3]}, ec4 = {ec[0], ec[1], ec[2], ec[3]};
    if (grp & 1) {
        eg4 = f32x4{eg[4], eg[5], eg[6], eg[7]};
        ec4 = f32x4{ec[4], ec[5], ec[6], ec[7]};
    }
    s4v ah, al, mh, ml;
    split4v(arow, ah, al);
    split4v(mrow, mh, ml);
    // (the outputs are stored non-temporal: nothing here reads them again;
    // the lean compose over 960 GDN chains, d = 128, 48 entries, takes
    // 1.312-1.315 ms against 1.318-1.328 with plain stores in the same calls)
    if constexpr (UPDATE_FIRST) {
        // The state update first (the caller's next step waits for it), the
        // outputs after it.  The tree's block phase takes this order for GDN:
        // it spills fewer registers there (102 per lane instead of 115 at
        // d = 128; tree over 960 GDN chains 5.37-5.43 against 5.71-5.76 ms).
        // For DeltaNet's block phase it spills more (4.46-4.50 against
        // 4.31-4.33 ms) and the
        // lean compose runs as fast either way, so those keep the outputs
        // inside the loop.
        s4v rh[2], rl[2];
#pragma unroll
        for (int n2 = 0; n2 < 2; ++n2) {
            // Y rows 0-7 (lane groups 0, 1); zero in rows 8-15
            f32x4 yv;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) yv[jj] = grp < 2 ? vv[n2][jj] - eg4[jj] * P[n2][jj] : 0.f;
            s4v yh, yl;
            split4v(yv, yh, yl);
            f32x4 R = {0.f, 0.f, 0.f, 0.f};
            R = mfma16(ah, yh, R);
            R = mfma16(ah, yl, R);
            R = mfma16(al, yh, R);
            split4v(R, rh[n2], rl[n2]);
            // S = lambda S0 + K^T diag(ec) R  (R rows 8-15 are zero)
            f32x4 Rs = R;
            if (grp < 2) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) Rs[jj] *= ec4[jj];
            }
            s4v sh, sl;
            split4v(Rs, sh, sl);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                f32x4 acc = X[rt][n2] * lam;
                acc = mfma16(ktv[rt], sh, acc);
                X[rt][n2] = mfma16(ktv[rt], sl, acc);
            }
        }
#pragma unroll
        for (int n2 = 0; n2 < 2; ++n2) {
            const int col = c0 + 16 * n2 + r16;
            // outputs, rows 8-15: o_t = e_t (Q S0)_t + (M R)_t
            f32x4 O = {0.f, 0.f, 0.f, 0.f};
            O = mfma16(mh, rh[n2], O);
            O = mfma16(mh, rl[n2], O);
            O = mfma16(ml, rh[n2], O);
            if (grp >= 2 && col < dk) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int t = 4 * (grp - 2) + jj;
                    if (t < nt) __builtin_nontemporal_store(eg4[jj] * P[n2][jj] + O[jj], o_first + t * o_tok_stride + col);
                }
            }
        }
    } else {
#pragma unroll
        for (int n2 = 0; n2 < 2; ++n2) {
            const int col = c0 + 16 * n2 + r16;
            // Y rows 0-7 (lane groups 0, 1); zero in rows 8-15
            f32x4 yv;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) yv[jj] = grp < 2 ? vv[n2][jj] - eg4[jj] * P[n2][jj] : 0.f;
            s4v yh, yl;
            split4v(yv, yh, yl);
            f32x4 R = {0.f, 0.f, 0.f, 0.f};
            R = mfma16(ah, yh, R);
            R = mfma16(ah, yl, R);
            R = mfma16(al, yh, R);
            s4v rh, rl;
            split4v(R, rh, rl);
            // outputs, rows 8-15: o_t = e_t (Q S0)_t + (M R)_t
            f32x4 O = {0.f, 0.f, 0.f, 0.f};
            O = mfma16(mh, rh, O);
            O = mfma16(mh, rl, O);
            O = mfma16(ml, rh, O);
            if (grp >= 2 && col < dk) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int t = 4 * (grp - 2) + jj;
                    if (t < nt) __builtin_nontemporal_store(eg4[jj] * P[n2][jj] + O[jj], o_first + t * o_tok_stride + col);
                }
            }
            // S = lambda S0 + K^T diag(ec) R  (R rows 8-15 are zero)
            f32x4 Rs = R;
            if (grp < 2) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) Rs[jj] *= ec4[jj];
            }
            split4v(Rs, rh, rl);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                f32x4 acc = X[rt][n2] * lam;
                acc = mfma16(ktv[rt], rh, acc);
                X[rt][n2] = mfma16(ktv[rt], rl, acc);
            }
        }
    }
}

// Up to SEAM_STAGE seam tokens of KDA (per-channel decay before the delta
// erase) with bf16-exact staged q, k, v, as one chunk on the matrix cores
// (same article, section on seam windows).  With E_t the window's cumulative
// per-channel decay through token t (staged by stage_seam<..., true>) and
// S0 the state entering the window, the token recurrence
//     S_t = (I - beta_t k_t k_t^T) diag(a_t) S_{t-1} + beta_t k_t v_t^T,
//     o_t = S_t^T q_t
// regroups into
//     G_ti = sum_c k_tc k_ic E_tc / E_ic,   M_ti = sum_c q_tc k_ic E_tc / E_ic,
//     R    = (I + diag(beta) tril(G, -1))^-1 diag(beta) (V - (E o K) S0),
//     o_t  = ((E o Q) S0)_t + sum_{i<=t} M_ti R_i,
//     S    = diag(E_c) S0 + (E_c / E o K)^T R,
// where E o K scales row t of K by E_t channel-wise and E_c is the last
// token's E.  The ratios E_t / E_i (t >= i) are decays and at most 1; the
// factor 1 / E_i alone grows with the decay over at most SEAM_STAGE tokens,
// the same bounded range as the build's Gram.  The decayed operands are not
// bf16-exact: every product takes the three-pass split.  sNw, sMw: this
// wave's 8 x 9 fp32 scratch; v_zero as in seam_chunk_bf16.
template <int D>
__device__ void seam_chunk_kda(f32x4 (&X)[D / 16][2], const SeamSmemKda<D> &sm, int nt, float *o_first,
                               int64_t o_tok_stride, int c0, int dk, float (*sNw)[9], float (*sMw)[9],
                               bool v_zero = false) {
    constexpr int RT = D / 16, KB = D / 32;
    const int lane = lane_fresh(), r16 = lane & 15, grp = lane >> 4;
    const int tr = r16 & (SEAM_STAGE - 1);  // this lane's token row
    // [E o K; E o Q] rows (A operand of P and of the Gram) and (K / E) rows
    // (B operand of the Gram: columns 8-15 of the Gram repeat 0-7 and are
    // never read), staged split, per k block
    bf16x8 lh[KB], ll[KB], bh[KB], bl[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        lh[kb] = *reinterpret_cast<const bf16x8 *>(&sm.lqh[r16][32 * kb + 8 * grp]);
        ll[kb] = *reinterpret_cast<const bf16x8 *>(&sm.lql[r16][32 * kb + 8 * grp]);
        bh[kb] = *reinterpret_cast<const bf16x8 *>(&sm.kbh[tr][32 * kb + 8 * grp]);
        bl[kb] = *reinterpret_cast<const bf16x8 *>(&sm.kbl[tr][32 * kb + 8 * grp]);
    }
    // P = [E o K; E o Q] S0 and the Gram [E o K; E o Q] (K / E)^T
    f32x4 P[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    f32x4 G = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        G = mfma(lh[kb], bh[kb], G);
        G = mfma(lh[kb], bl[kb], G);
        G = mfma(ll[kb], bh[kb], G);
#pragma unroll
        for (int n2 = 0; n2 < 2; ++n2) {
            float xv[8];
            bf16x8 xh, xl;
            acc_to_perm(X[2 * kb][n2], X[2 * kb + 1][n2], xv);
            split8(xv, xh, xl);
            P[n2] = mfma(lh[kb], xh, P[n2]);
            P[n2] = mfma(lh[kb], xl, P[n2]);
            P[n2] = mfma(ll[kb], xh, P[n2]);
        }
    }
    // G in C layout: lane (r16 = i, grp) holds row 4 grp + jj.  Rows 0-7 give
    // N (t > i), rows 8-15 give M (i <= t) for t = row - 8.
    if (r16 < 8) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int row = 4 * grp + jj, t = row & 7, i = r16;
            if (row < 8)
                sNw[t][i] = t > i ? sm.beta[t] * G[jj] : 0.f;
            else
                sMw[t][i] = i <= t ? G[jj] : 0.f;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // row r16 of (I + N)^-1 diag(beta): y (I + N) = e_r, swept from the last row up
    float y[SEAM_STAGE];
#pragma unroll
    for (int j = 0; j < SEAM_STAGE; ++j) y[j] = (j == r16) ? 1.f : 0.f;
#pragma unroll
    for (int i = SEAM_STAGE - 1; i > 0; --i)
#pragma unroll
        for (int j = 0; j < i; ++j) y[j] -= y[i] * sNw[i][j];
    f32x4 arow = {0.f, 0.f, 0.f, 0.f}, mrow = {0.f, 0.f, 0.f, 0.f};
    if (grp < 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = 4 * grp + e;
            arow[e] = r16 < 8 ? (grp == 0 ? y[e] : y[4 + e]) * sm.beta[j] : 0.f;
            mrow[e] = r16 >= 8 ? sMw[r16 - 8][j] : 0.f;
        }
    }
    s4v ah, al, mh, ml;
    split4v(arow, ah, al);
    split4v(mrow, mh, ml);
    // state update operands: (E_c / E o K)^T tiles (rows = channels 16 rt + r16,
    // k = tokens 4 grp .. 4 grp + 3 for grp < 2) and E_c of this lane's rows
    const int r0 = (4 * grp) & (SEAM_STAGE - 1);
    s4v kth[RT], ktl[RT];
    f32x4 ecr[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int ch = 16 * rt + r16;
        const s4v h = *reinterpret_cast<const s4v *>(&sm.kth[ch][r0]);
        const s4v l = *reinterpret_cast<const s4v *>(&sm.ktl[ch][r0]);
        kth[rt] = grp < 2 ? h : s4v{0, 0, 0, 0};
        ktl[rt] = grp < 2 ? l : s4v{0, 0, 0, 0};
        ecr[rt] = *reinterpret_cast<const f32x4 *>(&sm.ecl[16 * rt + 4 * grp]);
    }
#pragma unroll
    for (int n2 = 0; n2 < 2; ++n2) {
        const int col = c0 + 16 * n2 + r16;
        // Y = V - (E o K) S0 in rows 0-7 (lane groups 0, 1); zero in rows 8-15
        f32x4 yv;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const float v = v_zero ? 0.f : sm.v[r0 + jj][col < D ? col : D - 1];
            yv[jj] = grp < 2 ? v - P[n2][jj] : 0.f;
        }
        s4v yh, yl;
        split4v(yv, yh, yl);
        f32x4 R = {0.f, 0.f, 0.f, 0.f};
        R = mfma16(ah, yh, R);
        R = mfma16(ah, yl, R);
        R = mfma16(al, yh, R);
        s4v rh, rl;
        split4v(R, rh, rl);
        // outputs, rows 8-15: o_t = ((E o Q) S0)_t + (M R)_t
        f32x4 O = {0.f, 0.f, 0.f, 0.f};
        O = mfma16(mh, rh, O);
        O = mfma16(mh, rl, O);
        O = mfma16(ml, rh, O);
        if (grp >= 2 && col < dk) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int t = 4 * (grp - 2) + jj;
                if (t < nt) o_first[t * o_tok_stride + col] = P[n2][jj] + O[jj];
            }
        }
        // S = diag(E_c) S0 + (E_c / E o K)^T R  (R rows 8-15 are zero)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            f32x4 acc = X[rt][n2] * ecr[rt];
            acc = mfma16(kth[rt], rh, acc);
            acc = mfma16(kth[rt], rl, acc);
            X[rt][n2] = mfma16(ktl[rt], rh, acc);
        }
    }
}

// Tile <- p[row * ld + c0 + c] (rows < nrows, columns c0 + c < ncols), zero
// elsewhere.  The loads are unconditional (clamped indices, masked values), so
// they are all in flight together.
template <int D>
__device__ __forceinline__ void load_tile(f32x4 (&X)[D / 16][2], const float *p, int ld, int nrows, int c0, int ncols) {
    const int lane = lane_id(), r16 = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < D / 16; ++rt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int row = 16 * rt + 4 * grp + jj, col = c0 + 16 * nt + r16;
                const float v = p[(row < nrows ? row : nrows - 1) * ld + (col < ncols ? col : ncols - 1)];
                X[rt][nt][jj] = (row < nrows && col < ncols) ? v : 0.f;
            }
}

// Tile <- identity columns c0 .. c0+31 of I (d x d)
template <int D>
__device__ __forceinline__ void identity_tile(f32x4 (&X)[D / 16][2], int c0) {
    const int lane = lane_id(), r16 = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < D / 16; ++rt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) X[rt][nt][jj] = (16 * rt + 4 * grp + jj == c0 + 16 * nt + r16) ? 1.f : 0.f;
}

template <int D>
__device__ __forceinline__ void store_tile(const f32x4 (&X)[D / 16][2], float *p, int ld, int nrows, int c0, int ncols) {
    const int lane = lane_id(), r16 = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < D / 16; ++rt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int row = 16 * rt + 4 * grp + jj, col = c0 + 16 * nt + r16;
                if (row < nrows && col < ncols) p[row * ld + col] = X[rt][nt][jj];
            }
}

// 8 fp32 of row `row` of a dk x dk row-major matrix at the permuted k subset of
// k block kb, zero outside dk.
__device__ __forceinline__ void glb_perm(const float *M, int dk, int row, int kb, int grp, float (&x)[8]) {
    const int c0 = 32 * kb + 4 * grp, c1 = c0 + 16;
    const int rc = row < dk ? row : dk - 1;
    f32x4 a = *reinterpret_cast<const f32x4 *>(M + rc * dk + (c0 < dk ? c0 : dk - 4));
    f32x4 b = *reinterpret_cast<const f32x4 *>(M + rc * dk + (c1 < dk ? c1 : dk - 4));
    if (!(row < dk && c0 < dk)) a = f32x4{0.f, 0.f, 0.f, 0.f};
    if (!(row < dk && c1 < dk)) b = f32x4{0.f, 0.f, 0.f, 0.f};
    x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
    x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}

// Tile <- T Tile (+ add[row * dk + c0 + c] when add != nullptr), T dense dk x dk
// streamed from memory into A operands; the old tile is the B operand.
template <int D, bool F32>
__device__ __forceinline__ void apply_dense_T(f32x4 (&X)[D / 16][2], const float *T, int dk, const float *add, int c0) {
    constexpr int RT = D / 16, KB = D / 32;
    const int lane = lane_id(), r16 = lane & 15, grp = lane >> 4;
    float xv[KB][2][8];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc_to_perm(X[2 * kb][nt], X[2 * kb + 1][nt], xv[kb][nt]);
    if (add)
        load_tile<D>(X, add, dk, dk, c0, dk);
    else
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) X[rt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            float tv[8];
            glb_perm(T, dk, 16 * rt + r16, kb, grp, tv);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) X[rt][nt] = mma_split<F32>(tv, xv[kb][nt], X[rt][nt]);
        }
}

// Tile I/O and the diagonal updates through buffer views of a dk x dk
// row-major matrix: one per-lane offset, each row's offset a scalar (the
// per-element 64-bit addresses of the plain helpers above would be held in
// registers).  Reads of rows past dk return zero; loads zero the columns past
// dk; the updates may leave values of no use there (every diagonal step keeps
// columns apart), and stores skip them.
template <int D>
__device__ __forceinline__ void load_tile_buf(f32x4 (&X)[D / 16][2], const float *p, int dk, int c0) {
    const int lane = lane_fresh(), r16 = lane & 15, grp = lane >> 4;
    const auto r = buffer_view(p, dk * dk * 4);
    const int v = (4 * grp * dk + c0 + r16) * 4;
#pragma unroll
    for (int rt = 0; rt < D / 16; ++rt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float x = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(r, v, ((16 * rt + jj) * dk + 16 * nt) * 4, 0));
                X[rt][nt][jj] = c0 + 16 * nt + r16 < dk ? x : 0.f;
            }
}

template <int D>
__device__ __forceinline__ void store_tile_buf(const f32x4 (&X)[D / 16][2], float *p, int dk, int c0) {
    const int lane = lane_fresh(), r16 = lane & 15, grp = lane >> 4;
    const auto r = buffer_view(p, dk * dk * 4);
    const int v = (4 * grp * dk + c0 + r16) * 4;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        if (c0 + 16 * nt + r16 >= dk) continue;
#pragma unroll
        for (int rt = 0; rt < D / 16; ++rt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float x = X[rt][nt][jj];  // (copied out: bit_cast of a vector element reads element 0)
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), r, v,
                                                      ((16 * rt + jj) * dk + 16 * nt) * 4, 0);
            }
    }
}

// X <- diag(T) X + A, T and A dense dk x dk, the diagonal of T at stride dk + 1
template <int D>
__device__ __forceinline__ void apply_diag_agg(f32x4 (&X)[D / 16][2], const float *T, const float *A, int dk, int c0) {
    const int lane = lane_fresh(), r16 = lane & 15, grp = lane >> 4;
    const auto rT = buffer_view(T, dk * dk * 4);
    const auto rA = buffer_view(A, dk * dk * 4);
    const int vT = 4 * grp * (dk + 1) * 4, vA = (4 * grp * dk + c0 + r16) * 4;
#pragma unroll
    for (int rt = 0; rt < D / 16; ++rt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int r0 = 16 * rt + jj;
            const float tv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rT, vT, r0 * (dk + 1) * 4, 0));
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const float av = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(rA, vA, (r0 * dk + 16 * nt) * 4, 0));
                X[rt][nt][jj] = tv * X[rt][nt][jj] + av;
            }
        }
}

// X <- diag(T) X + add for a cached diagonal T (t_elems 1: a scalar; dk: a
// vector) and add dense dk x dk or null (zero)
template <int D>
__device__ __forceinline__ void apply_diag_T_buf(f32x4 (&X)[D / 16][2], const float *T, int64_t t_elems, int dk,
                                                 const float *add, int c0) {
    const int lane = lane_fresh(), r16 = lane & 15, grp = lane >> 4;
    const bool vec = t_elems != 1;
    const auto rT = buffer_view(T, (int)t_elems * 4);
    const auto rA = buffer_view(add, add ? dk * dk * 4 : 0);
    const int vT = vec ? 4 * grp * 4 : 0, vA = (4 * grp * dk + c0 + r16) * 4;
#pragma unroll
    for (int rt = 0; rt < D / 16; ++rt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int r0 = 16 * rt + jj;
            const float tv =
                __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rT, vT, vec ? r0 * 4 : 0, 0));
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const float av = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(rA, vA, (r0 * dk + 16 * nt) * 4, 0));
                X[rt][nt][jj] = tv * X[rt][nt][jj] + av;
            }
        }
}

}  // namespace hy
