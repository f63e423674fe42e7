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
template <int D>
struct SeamSmem {
    float q[SEAM_STAGE][D];
    float k[SEAM_STAGE][D];
    float v[SEAM_STAGE][D];
    float a[SEAM_STAGE][D];  // per-row decay (GLA, KDA), or a[t][0] (scalar decay)
    float beta[SEAM_STAGE];
};

// Stage tokens tok0 .. tok0+nt-1 of `chain` (rows past nt are zero tokens).
template <int D, int FAM, typename TIN>
__device__ void stage_seam(SeamSmem<D> &sm, const Tok &x, int chain, int dk, int64_t tok0, int nt) {
    const int tid = threadIdx.x, nthr = blockDim.x;
    const TIN *qp = reinterpret_cast<const TIN *>(x.q) + (int64_t)chain * x.cs;
    const TIN *kp = reinterpret_cast<const TIN *>(x.k) + (int64_t)chain * x.cs;
    const TIN *vp = reinterpret_cast<const TIN *>(x.v) + (int64_t)chain * x.cs;
    for (int item = tid; item < SEAM_STAGE * D; item += nthr) {
        const int t = item / D, i = item % D;
        float qv = 0.f, kv = 0.f, vv = 0.f, av = 1.f;
        if (t < nt && i < dk) {
            const int64_t off = (tok0 + t) * x.ts + i;
            qv = ldf(qp + off);
            kv = ldf(kp + off);
            vv = ldf(vp + off);
            if (fam_vgate(FAM))
                av = expf(ldf(reinterpret_cast<const TIN *>(x.g) + (int64_t)chain * x.gcs + (tok0 + t) * x.gts + i));
        }
        sm.q[t][i] = qv;
        sm.k[t][i] = kv;
        sm.v[t][i] = vv;
        if (fam_vgate(FAM)) sm.a[t][i] = av;
    }
    if (tid < SEAM_STAGE) {
        const int t = tid;
        float av = 1.f, bv = 1.f;
        if (t < nt) {
            if (fam_sgate(FAM))
                av = expf(ldf(reinterpret_cast<const TIN *>(x.g) + (int64_t)chain * x.gcs + (tok0 + t) * x.gts));
            if (FAM == RETNET) av = x.gamma[chain];
            if (fam_beta(FAM)) bv = ldf(reinterpret_cast<const TIN *>(x.beta) + (int64_t)chain * x.bcs + (tok0 + t) * x.bts);
        }
        if (!fam_vgate(FAM)) sm.a[t][0] = av;
        sm.beta[t] = bv;
    }
}

// The token recurrence S_t = A_t S_{t-1} + beta_t k_t v_t^T on this wave's
// tile, for nt staged tokens, writing o_t = S_t^T q_t for every token:
// o_first[t * o_tok_stride + ocol + c] for tile column c < ncols - ocol.
// vcol: the tile's first column in v; v_zero: the tile's v is zero (the T half
// of a [T | S] pair, which then yields T^T q, the pulled-back query).
template <int D, int FAM>
__device__ void seam_tokens(f32x4 (&X)[D / 16][2], const SeamSmem<D> &sm, int nt, float *o_first,
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

// Tile <- p[row * ld + c0 + c] (rows < nrows, columns c0 + c < ncols), zero elsewhere.
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
                X[rt][nt][jj] = (row < nrows && col < ncols) ? p[row * ld + col] : 0.f;
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
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
    if (row < dk) {
        if (c0 < dk) a = *reinterpret_cast<const f32x4 *>(M + row * dk + c0);
        if (c1 < dk) b = *reinterpret_cast<const f32x4 *>(M + row * dk + c1);
    }
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

// Tile <- diag(T) Tile (+ add), T a scalar (t_elems == 1) or a dk-vector.
template <int D>
__device__ __forceinline__ void apply_diag_T(f32x4 (&X)[D / 16][2], const float *T, int64_t t_elems, int dk,
                                             const float *add, int c0) {
    const int lane = lane_id(), r16 = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < D / 16; ++rt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int row = 16 * rt + 4 * grp + jj, col = c0 + 16 * nt + r16;
                if (row < dk && col < dk) {
                    const float tv = t_elems == 1 ? T[0] : T[row];
                    X[rt][nt][jj] = tv * X[rt][nt][jj] + (add ? add[row * dk + col] : 0.f);
                }
            }
}

}  // namespace hy
