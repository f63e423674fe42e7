// Dense-transition pair build (DeltaNet, Gated DeltaNet) for gfx950.
//
// For every (segment, chain) this computes T_C = A_n ... A_1 and S(C|0)
// (HYPIC, codernav.top article, section on linear layers: the pair cached at
// a segment's first prefill).  With A_t = a_t (I - beta_t k_t k_t^T), a_t =
// exp(g_t) (GDN) or 1 (DeltaNet), a chunk of c = 64 tokens is applied at once
// in the UT / WY form (Gamma_t = chunk-local cumulative log-decay):
//     G_ti = (k_t . k_i) exp(Gamma_t - Gamma_i)            for t > i
//     A    = (I + diag(beta) tril(G, -1))^-1 diag(beta)     (unit lower solve)
//     W    = A diag(exp(Gamma)) K,   U = A V
//     X   <- exp(Gamma_c) X + K^T diag(exp(Gamma_c - Gamma)) ([0 | U] - W X)
// on X = [T | S] (d x 2d), starting from [I | 0].
//
// Mapping: one workgroup per (segment, chain), 2d/32 waves; wave w owns
// columns 32w .. 32w+31 of X for the whole segment and keeps them in MFMA
// accumulators (the columns of X evolve independently given the chunk's W,
// U and K).  Chunk factors (Gram, inverse, W, U) are shared through LDS.
//
// Precision: bf16 inputs use bf16 matrix cores; keys and values are exact in
// bf16, every other operand is split into hi + lo (two or three passes, fp32
// accumulation, fp32 state).  fp32 inputs use the fp32 matrix cores for every
// contraction.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace hy {

template <int D, typename TIN>
struct DenseCfg {
    static constexpr bool F32 = std::is_same<TIN, float>::value;
    static constexpr int ES = F32 ? 4 : 2;  // bytes per LDS operand element
    static constexpr int NW = 2 * D / 32;
    static constexpr int NT = NW * 64;
    static constexpr int RT = D / 16;
    static constexpr int KB = D / 32;
    static constexpr int LDK = F32 ? D + 4 : D + 8;    // row stride of [CH][D] operand arrays
    static constexpr int LDT = F32 ? CH + 4 : CH + 8;  // row stride of [D][CH] operand arrays
    static constexpr int LDL = CH + 1;                 // fp32 row stride of L
    static constexpr int LDI = CH + 4;                 // fp32 row stride of Inv and U^T
    // region A: K rows (load, Gram), inverse scratch, then U^T (W/U, carry)
    static constexpr int szK = CH * LDK * ES;
    static constexpr int szP = 4 * 16 * 17 * 4;
    static constexpr int szU = D * LDI * 4;
    static constexpr int offA = 0;
    static constexpr int szA = (((szK + szP) > szU ? (szK + szP) : szU) + 15) / 16 * 16;
    static constexpr int offP = offA + szK;
    // region B: L (Gram, inverse), then W (hi/lo bf16, or fp32) (W/U, carry)
    static constexpr int szL = CH * LDL * 4;
    static constexpr int szW = CH * LDK * 4;
    static constexpr int offB = offA + szA;
    static constexpr int szB = ((szL > szW ? szL : szW) + 15) / 16 * 16;
    static constexpr int offKT = offB + szB;
    static constexpr int szKT = D * LDT * ES;
    static constexpr int offVT = offKT + szKT;
    static constexpr int szVT = D * LDT * ES;
    static constexpr int offInv = offVT + szVT;
    static constexpr int szInv = CH * LDI * 4;
    static constexpr int offSc = offInv + szInv;  // Gamma, exp(Gamma), exp(Gamma_c - Gamma), beta, lam
    static constexpr int szSc = (4 * CH + 4) * 4;
    static constexpr int total = offSc + szSc;
    static_assert(total <= 160 * 1024, "LDS budget");
};

template <int D, int FAM, typename TIN>
__global__ void __launch_bounds__(2 * D / 32 * 64)
k_build_dense(BuildArgs a) {
    using Cfg = DenseCfg<D, TIN>;
    constexpr bool F32 = Cfg::F32;
    using OpT = typename std::conditional<F32, float, bf16>::type;
    constexpr int NW = Cfg::NW, NT = Cfg::NT, RT = Cfg::RT, KB = Cfg::KB;
    constexpr int LDK = Cfg::LDK, LDT = Cfg::LDT, LDL = Cfg::LDL, LDI = Cfg::LDI;
    __shared__ __attribute__((aligned(16))) char smem[Cfg::total];
    OpT *sK = reinterpret_cast<OpT *>(smem + Cfg::offA);
    float *sP = reinterpret_cast<float *>(smem + Cfg::offP);
    float *sU = reinterpret_cast<float *>(smem + Cfg::offA);
    float *sL = reinterpret_cast<float *>(smem + Cfg::offB);
    bf16 *sWh = reinterpret_cast<bf16 *>(smem + Cfg::offB);  // bf16 path: hi then lo
    bf16 *sWl = sWh + CH * LDK;
    float *sWf = reinterpret_cast<float *>(smem + Cfg::offB);  // fp32 path
    OpT *sKT = reinterpret_cast<OpT *>(smem + Cfg::offKT);
    OpT *sVT = reinterpret_cast<OpT *>(smem + Cfg::offVT);
    float *sInv = reinterpret_cast<float *>(smem + Cfg::offInv);
    float *sGam = reinterpret_cast<float *>(smem + Cfg::offSc);
    float *sEg = sGam + CH;
    float *sEc = sEg + CH;
    float *sBeta = sEc + CH;
    float *sLam = sBeta + CH;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    const int seg = blockIdx.x / a.n_chains, chain = blockIdx.x % a.n_chains;
    const int dk = a.dk;
    const int64_t b0 = a.seg_begin[seg], n = a.seg_end[seg] - b0;
    const TIN *kp = reinterpret_cast<const TIN *>(a.x.k) + (int64_t)chain * a.x.cs;
    const TIN *vp = reinterpret_cast<const TIN *>(a.x.v) + (int64_t)chain * a.x.cs;
    const TIN *gp = FAM == GDN ? reinterpret_cast<const TIN *>(a.x.g) + (int64_t)chain * a.x.gcs : nullptr;
    const TIN *bp = reinterpret_cast<const TIN *>(a.x.beta) + (int64_t)chain * a.x.bcs;

    const int cbase = wv * 32;
    const bool isS = cbase >= D;
    f32x4 X[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                X[rt][nt][jj] = (16 * rt + 4 * grp + jj == cbase + 16 * nt + r16) ? 1.f : 0.f;

    for (int64_t c0 = 0; c0 < n; c0 += CH) {
        const int L = (int)(n - c0 < CH ? n - c0 : CH);
        const int64_t t0 = b0 + c0;
        // ---- stage the chunk's keys and values (zero rows past the segment end)
        for (int item = tid; item < CH * D / 8; item += NT) {
            const int t = item / (D / 8), i8 = (item % (D / 8)) * 8;
            float kv[8], vv[8];
            if (t < L && i8 < dk) {
                load8(kp + (t0 + t) * a.x.ts + i8, kv);
                load8(vp + (t0 + t) * a.x.ts + i8, vv);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) kv[e] = vv[e] = 0.f;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sK[t * LDK + i8 + e] = (OpT)kv[e];
                sKT[(i8 + e) * LDT + t] = (OpT)kv[e];
                sVT[(i8 + e) * LDT + t] = (OpT)vv[e];
            }
        }
        if (wv == 0) {
            float gt = 0.f, bt = 0.f;
            if (lane < L) {
                if (FAM == GDN) gt = ldf(gp + (t0 + lane) * a.x.gts);
                bt = ldf(bp + (t0 + lane) * a.x.bts);
            }
            float s = gt;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                float y = __shfl_up(s, off);
                if (lane >= off) s += y;
            }
            const float gc = __shfl(s, 63);
            sGam[lane] = s;
            sBeta[lane] = bt;
            sEg[lane] = expf(s);
            sEc[lane] = expf(gc - s);
            if (lane == 0) sLam[0] = expf(gc);
        }
        __syncthreads();

        // ---- Gram of the chunk's keys, scaled into the strictly lower L
        for (int tile = wv; tile < 10; tile += NW) {
            int mt = 0, nt = tile;
            while (nt > mt) { nt -= mt + 1; ++mt; }  // lower-triangular tile (mt >= nt)
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                if constexpr (F32) {
                    float av[8], bv[8];
                    lds_cont_f(sK, LDK, 16 * mt + r16, 32 * kb, grp, av);
                    lds_cont_f(sK, LDK, 16 * nt + r16, 32 * kb, grp, bv);
                    acc = mma_f32(av, bv, acc);
                } else {
                    acc = mfma(lds_cont(sK, LDK, 16 * mt + r16, 32 * kb, grp),
                               lds_cont(sK, LDK, 16 * nt + r16, 32 * kb, grp), acc);
                }
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int t = 16 * mt + 4 * grp + jj, i = 16 * nt + r16;
                float val = 0.f;
                if (t > i) {
                    val = sBeta[t] * acc[jj];
                    if (FAM == GDN) val *= expf(sGam[t] - sGam[i]);
                }
                sL[t * LDL + i] = val;
            }
        }
        __syncthreads();

        // ---- (I + L)^-1 by 16 x 16 blocks: diagonal blocks by forward substitution
        if (wv == 0) {
            const int bk = grp, c = r16;
            float xr[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float s = (r == c) ? 1.f : 0.f;
#pragma unroll
                for (int j = 0; j < r; ++j) s -= sL[(16 * bk + r) * LDL + 16 * bk + j] * xr[j];
                xr[r] = s;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sInv[(16 * bk + r) * LDI + 16 * bk + c] = xr[r];
        } else {
            // blocks above the diagonal are zero
            for (int idx = tid - 64; idx < 6 * 256; idx += NT - 64) {
                const int blk = idx >> 8, e = idx & 255;
                const int bi = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
                const int bj = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
                sInv[(16 * bi + (e >> 4)) * LDI + 16 * bj + (e & 15)] = 0.f;
            }
        }
        __syncthreads();
        // off-diagonal blocks, by distance from the diagonal:
        //   Inv_ij = -Inv_ii * sum_{k=j}^{i-1} L_ik Inv_kj
        for (int d = 1; d < 4; ++d) {
            for (int blk = wv; blk < 4 - d; blk += NW) {
                const int bi = blk + d, bj = blk;
                float *sp = sP + blk * 16 * 17;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int r = 4 * grp + jj;
                    float acc = 0.f;
                    for (int kb = bj; kb < bi; ++kb)
#pragma unroll
                        for (int m = 0; m < 16; ++m)
                            acc += sL[(16 * bi + r) * LDL + 16 * kb + m] * sInv[(16 * kb + m) * LDI + 16 * bj + r16];
                    sp[r * 17 + r16] = acc;
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int r = 4 * grp + jj;
                    float acc = 0.f;
#pragma unroll
                    for (int m = 0; m < 16; ++m) acc += sInv[(16 * bi + r) * LDI + 16 * bi + m] * sp[m * 17 + r16];
                    sInv[(16 * bi + r) * LDI + 16 * bj + r16] = -acc;
                }
            }
            __syncthreads();
        }

        // ---- W = A diag(exp Gamma) K and U = A V on the matrix cores
        for (int tile = wv; tile < 8 * RT; tile += NW) {
            const bool isU = tile >= 4 * RT;
            const int rem = isU ? tile - 4 * RT : tile;
            const int mt = rem / RT, nt = rem % RT;
            const OpT *Bm = isU ? sVT : sKT;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int i0 = 32 * kb + 8 * grp;
                const float *ip = sInv + (16 * mt + r16) * LDI + i0;
                float av[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) av[e] = ip[e] * (isU ? sBeta[i0 + e] : sBeta[i0 + e] * sEg[i0 + e]);
                if constexpr (F32) {
                    float bv[8];
                    lds_cont_f(Bm, LDT, 16 * nt + r16, 32 * kb, grp, bv);
                    acc = mma_f32(av, bv, acc);
                } else {
                    bf16x8 ah, al;
                    split8(av, ah, al);
                    const bf16x8 bh = lds_cont(Bm, LDT, 16 * nt + r16, 32 * kb, grp);
                    acc = mfma(ah, bh, acc);
                    acc = mfma(al, bh, acc);
                }
            }
            if (isU) {
                *reinterpret_cast<f32x4 *>(sU + (16 * nt + r16) * LDI + 16 * mt + 4 * grp) = acc;
            } else {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int t = 16 * mt + 4 * grp + jj, i = 16 * nt + r16;
                    if constexpr (F32) {
                        sWf[t * LDK + i] = acc[jj];
                    } else {
                        bf16 h, l;
                        split1(acc[jj], h, l);
                        sWh[t * LDK + i] = h;
                        sWl[t * LDK + i] = l;
                    }
                }
            }
        }
        __syncthreads();

        // ---- carry this wave's 32 columns of X = [T | S] through the chunk
        {
            f32x4 M[4][2];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) M[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            // M = W X
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                float xv[2][8];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) acc_to_perm(X[2 * kb][nt], X[2 * kb + 1][nt], xv[nt]);
                if constexpr (F32) {
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {
                        float wf[8];
                        lds_perm_f(sWf, LDK, 16 * mt + r16, 32 * kb, grp, wf);
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt) M[mt][nt] = mma_f32(wf, xv[nt], M[mt][nt]);
                    }
                } else {
                    bf16x8 xh[2], xl[2];
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) split8(xv[nt], xh[nt], xl[nt]);
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {
                        const bf16x8 wh = lds_perm(sWh, LDK, 16 * mt + r16, 32 * kb, grp);
                        const bf16x8 wl = lds_perm(sWl, LDK, 16 * mt + r16, 32 * kb, grp);
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt) {
                            M[mt][nt] = mfma(wh, xh[nt], M[mt][nt]);
                            M[mt][nt] = mfma(wh, xl[nt], M[mt][nt]);
                            M[mt][nt] = mfma(wl, xh[nt], M[mt][nt]);
                        }
                    }
                }
            }
            // R' = diag(exp(Gamma_c - Gamma)) ([0 | U] - M)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const f32x4 ec = *reinterpret_cast<const f32x4 *>(sEc + 16 * mt + 4 * grp);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    f32x4 u = {0.f, 0.f, 0.f, 0.f};
                    if (isS) u = *reinterpret_cast<const f32x4 *>(sU + (cbase - D + 16 * nt + r16) * LDI + 16 * mt + 4 * grp);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) M[mt][nt][jj] = (u[jj] - M[mt][nt][jj]) * ec[jj];
                }
            }
            // X = exp(Gamma_c) X + K^T R'
            const float lam = sLam[0];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) X[rt][nt] *= lam;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float rv[2][8];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) acc_to_perm(M[2 * kb][nt], M[2 * kb + 1][nt], rv[nt]);
                if constexpr (F32) {
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        float kf[8];
                        lds_perm_f(sKT, LDT, 16 * rt + r16, 32 * kb, grp, kf);
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt) X[rt][nt] = mma_f32(kf, rv[nt], X[rt][nt]);
                    }
                } else {
                    bf16x8 rh[2], rl[2];
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) split8(rv[nt], rh[nt], rl[nt]);
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        const bf16x8 kh = lds_perm(sKT, LDT, 16 * rt + r16, 32 * kb, grp);
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt) {
                            X[rt][nt] = mfma(kh, rh[nt], X[rt][nt]);
                            X[rt][nt] = mfma(kh, rl[nt], X[rt][nt]);
                        }
                    }
                }
            }
        }
        __syncthreads();
    }

    // ---- write the pair: T = X[:, :d], S = X[:, d:]
    float *To = a.T + ((int64_t)seg * a.n_chains + chain) * dk * dk;
    float *So = a.S + ((int64_t)seg * a.n_chains + chain) * dk * dk;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int row = 16 * rt + 4 * grp + jj;
                const int col = cbase + 16 * nt + r16 - (isS ? D : 0);
                if (row < dk && col < dk) (isS ? So : To)[row * dk + col] = X[rt][nt][jj];
            }
}

template <int D, int FAM, typename TIN>
static hipError_t launch_dense(const BuildArgs &a, int n_seg, hipStream_t st) {
    const dim3 grid((unsigned)(n_seg * (int64_t)a.n_chains));
    hipLaunchKernelGGL((k_build_dense<D, FAM, TIN>), grid, dim3(DenseCfg<D, TIN>::NT), 0, st, a);
    return hipGetLastError();
}

template <int FAM, typename TIN>
static hipError_t launch_dense_d(const BuildArgs &a, int D, int n_seg, hipStream_t st) {
    switch (D) {
    case 32: return launch_dense<32, FAM, TIN>(a, n_seg, st);
    case 64: return launch_dense<64, FAM, TIN>(a, n_seg, st);
    case 128: return launch_dense<128, FAM, TIN>(a, n_seg, st);
    }
    return hipErrorInvalidValue;
}

hipError_t build_dense(const BuildArgs &a, int family, bool bf16_in, int D, int n_seg, hipStream_t st) {
    if (family == GDN)
        return bf16_in ? launch_dense_d<GDN, bf16>(a, D, n_seg, st) : launch_dense_d<GDN, float>(a, D, n_seg, st);
    if (family == DELTANET)
        return bf16_in ? launch_dense_d<DELTANET, bf16>(a, D, n_seg, st)
                       : launch_dense_d<DELTANET, float>(a, D, n_seg, st);
    return hipErrorInvalidValue;
}

}  // namespace hy
