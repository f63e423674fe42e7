// Scalar / diagonal-decay pair build (plain linear attention, RetNet, Mamba2,
// GLA) for gfx950.
//
// T stays diagonal: T = exp(sum_t g_t) (a scalar times I, or one value per
// key channel) and S(C|0) = sum_t (exp(Gamma_end - Gamma_t) * k_t) v_t^T
// (HYPIC, codernav.top article, section on linear layers: the segment's
// transition product and zero-initial state).  Tokens are streamed in chunks
// of 64; per chunk the state takes exp(Gamma_c) S + Kt^T V' on the matrix
// cores, where the chunk-local decay is folded into the values (scalar
// decays) or into the keys (per-channel decay, GLA).
//
// Mapping: one workgroup per (segment, chain), d/32 waves, wave w keeps
// columns 32w .. 32w+31 of S in MFMA accumulators across the segment.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace hy {

template <int D, int FAM, typename TIN>
struct DiagCfg {
    static constexpr bool F32 = std::is_same<TIN, float>::value;  // fp32 inputs: fp32 matrix cores
    // bf16 inputs: the operand that carries the chunk-local decay is not
    // bf16-exact and gets a lo part
    static constexpr bool KLO = !F32 && FAM == GLA;
    static constexpr bool VLO = !F32 && (FAM == RETNET || FAM == MAMBA2);
    static constexpr int ES = F32 ? 4 : 2;
    static constexpr int NW = D / 32;
    static constexpr int NT = NW * 64;
    static constexpr int RT = D / 16;
    static constexpr int LDT = F32 ? CH + 4 : CH + 8;
    static constexpr int offKT = 0;
    static constexpr int szKT = (KLO ? 2 : 1) * D * LDT * ES;
    static constexpr int offVT = offKT + szKT;
    static constexpr int szVT = (VLO ? 2 : 1) * D * LDT * ES;
    static constexpr int offG = offVT + szVT;  // chunk log-gates: [CH] or [CH][D] fp32
    static constexpr int szG = (FAM == GLA ? CH * D : CH) * 4;
    static constexpr int offLam = offG + szG;  // exp(Gamma_c): [1] or [D]
    static constexpr int szLam = D * 4;
    static constexpr int offTot = offLam + szLam;  // running segment log-decay (double)
    static constexpr int szTot = D * 8;
    static constexpr int total = offTot + szTot;
    static_assert(total <= 160 * 1024, "LDS budget");
};

template <int D, int FAM, typename TIN>
__global__ void __launch_bounds__(D / 32 * 64)
k_build_diag(BuildArgs a) {
    using Cfg = DiagCfg<D, FAM, TIN>;
    constexpr int NT = Cfg::NT, RT = Cfg::RT, LDT = Cfg::LDT;
    constexpr bool KLO = Cfg::KLO, VLO = Cfg::VLO, F32 = Cfg::F32;
    using OpT = typename std::conditional<F32, float, bf16>::type;
    __shared__ __attribute__((aligned(16))) char smem[Cfg::total];
    OpT *sKTh = reinterpret_cast<OpT *>(smem + Cfg::offKT);
    OpT *sKTl = sKTh + D * LDT;
    OpT *sVTh = reinterpret_cast<OpT *>(smem + Cfg::offVT);
    OpT *sVTl = sVTh + D * LDT;
    float *sG = reinterpret_cast<float *>(smem + Cfg::offG);
    float *sLam = reinterpret_cast<float *>(smem + Cfg::offLam);
    double *sTot = reinterpret_cast<double *>(smem + Cfg::offTot);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    const int seg = blockIdx.x / a.n_chains, chain = blockIdx.x % a.n_chains;
    const int dk = a.dk;
    const int64_t b0 = a.seg_begin[seg], n = a.seg_end[seg] - b0;
    const TIN *kp = reinterpret_cast<const TIN *>(a.x.k) + (int64_t)chain * a.x.cs;
    const TIN *vp = reinterpret_cast<const TIN *>(a.x.v) + (int64_t)chain * a.x.cs;
    const TIN *gp = (FAM == MAMBA2 || FAM == GLA) ? reinterpret_cast<const TIN *>(a.x.g) + (int64_t)chain * a.x.gcs
                                                  : nullptr;
    const float lgam = FAM == RETNET ? logf(a.x.gamma[chain]) : 0.f;
    const int cbase = wv * 32;

    f32x4 X[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) X[rt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (tid < D) sTot[tid] = 0.0;

    for (int64_t c0 = 0; c0 < n; c0 += CH) {
        const int L = (int)(n - c0 < CH ? n - c0 : CH);
        const int64_t t0 = b0 + c0;
        // ---- chunk-local cumulative log-decay
        if (FAM == GLA) {
            for (int i = tid; i < D; i += NT) {
                float s = 0.f;
                for (int t = 0; t < CH; ++t) {
                    if (t < L && i < dk) s += ldf(gp + (t0 + t) * a.x.gts + i);
                    sG[t * D + i] = s;
                }
                sLam[i] = expf(s);
                sTot[i] += (double)s;
            }
        } else if (wv == 0) {
            float gt = 0.f;
            if (lane < L) gt = FAM == MAMBA2 ? ldf(gp + (t0 + lane) * a.x.gts) : (FAM == RETNET ? lgam : 0.f);
            float s = gt;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                float y = __shfl_up(s, off);
                if (lane >= off) s += y;
            }
            sG[lane] = s;
            const float gc = __shfl(s, 63);
            if (lane == 0) {
                sLam[0] = expf(gc);
                sTot[0] += (double)gc;
            }
        }
        __syncthreads();
        // ---- stage K^T and V^T with the decay exp(Gamma_c - Gamma_t) folded in
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
            if (FAM == GLA) {
#pragma unroll
                for (int e = 0; e < 8; ++e) kv[e] *= expf(sG[(CH - 1) * D + i8 + e] - sG[t * D + i8 + e]);
            } else if (FAM != LINEAR) {
                const float f = expf(sG[CH - 1] - sG[t]);
#pragma unroll
                for (int e = 0; e < 8; ++e) vv[e] *= f;
            }
            if constexpr (F32) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sKTh[(i8 + e) * LDT + t] = kv[e];
                    sVTh[(i8 + e) * LDT + t] = vv[e];
                }
            } else {
                bf16x8 h, l;
                split8(kv, h, l);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sKTh[(i8 + e) * LDT + t] = h[e];
                    if (KLO) sKTl[(i8 + e) * LDT + t] = l[e];
                }
                split8(vv, h, l);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sVTh[(i8 + e) * LDT + t] = h[e];
                    if (VLO) sVTl[(i8 + e) * LDT + t] = l[e];
                }
            }
        }
        __syncthreads();
        // ---- S <- exp(Gamma_c) S + Kt^T V'
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            f32x4 lam;
            if (FAM == GLA) {
                lam = *reinterpret_cast<const f32x4 *>(sLam + 16 * rt + 4 * grp);
            } else {
                const float l0 = FAM == LINEAR ? 1.f : sLam[0];
                lam = f32x4{l0, l0, l0, l0};
            }
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) X[rt][nt][jj] *= lam[jj];
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if constexpr (F32) {
                float vf[2][8];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) lds_cont_f(sVTh, LDT, cbase + 16 * nt + r16, 32 * kb, grp, vf[nt]);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    float kf[8];
                    lds_cont_f(sKTh, LDT, 16 * rt + r16, 32 * kb, grp, kf);
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) X[rt][nt] = mma_f32(kf, vf[nt], X[rt][nt]);
                }
            } else {
                bf16x8 vh[2], vl[2];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    vh[nt] = lds_cont(sVTh, LDT, cbase + 16 * nt + r16, 32 * kb, grp);
                    if (VLO) vl[nt] = lds_cont(sVTl, LDT, cbase + 16 * nt + r16, 32 * kb, grp);
                }
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const bf16x8 kh = lds_cont(sKTh, LDT, 16 * rt + r16, 32 * kb, grp);
                    bf16x8 kl;
                    if (KLO) kl = lds_cont(sKTl, LDT, 16 * rt + r16, 32 * kb, grp);
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        X[rt][nt] = mfma(kh, vh[nt], X[rt][nt]);
                        if (VLO) X[rt][nt] = mfma(kh, vl[nt], X[rt][nt]);
                        if (KLO) X[rt][nt] = mfma(kl, vh[nt], X[rt][nt]);
                    }
                }
            }
        }
        __syncthreads();
    }

    float *So = a.S + ((int64_t)seg * a.n_chains + chain) * dk * dk;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int row = 16 * rt + 4 * grp + jj, col = cbase + 16 * nt + r16;
                if (row < dk && col < dk) So[row * dk + col] = X[rt][nt][jj];
            }
    if (FAM == GLA) {
        for (int i = tid; i < dk; i += NT) a.T[((int64_t)seg * a.n_chains + chain) * dk + i] = (float)exp(sTot[i]);
    } else if (tid == 0) {
        float tv = 1.f;
        if (FAM == RETNET) tv = (float)pow((double)a.x.gamma[chain], (double)n);
        if (FAM == MAMBA2) tv = (float)exp(sTot[0]);
        a.T[(int64_t)seg * a.n_chains + chain] = tv;
    }
}

template <int D, int FAM, typename TIN>
static hipError_t launch_diag(const BuildArgs &a, int n_seg, hipStream_t st) {
    const dim3 grid((unsigned)(n_seg * (int64_t)a.n_chains));
    hipLaunchKernelGGL((k_build_diag<D, FAM, TIN>), grid, dim3(DiagCfg<D, FAM, TIN>::NT), 0, st, a);
    return hipGetLastError();
}

template <int FAM, typename TIN>
static hipError_t launch_diag_d(const BuildArgs &a, int D, int n_seg, hipStream_t st) {
    switch (D) {
    case 32: return launch_diag<32, FAM, TIN>(a, n_seg, st);
    case 64: return launch_diag<64, FAM, TIN>(a, n_seg, st);
    case 128: return launch_diag<128, FAM, TIN>(a, n_seg, st);
    }
    return hipErrorInvalidValue;
}

template <typename TIN>
static hipError_t diag_by_family(const BuildArgs &a, int family, int D, int n_seg, hipStream_t st) {
    switch (family) {
    case LINEAR: return launch_diag_d<LINEAR, TIN>(a, D, n_seg, st);
    case RETNET: return launch_diag_d<RETNET, TIN>(a, D, n_seg, st);
    case MAMBA2: return launch_diag_d<MAMBA2, TIN>(a, D, n_seg, st);
    case GLA: return launch_diag_d<GLA, TIN>(a, D, n_seg, st);
    }
    return hipErrorInvalidValue;
}

hipError_t build_diag(const BuildArgs &a, int family, bool bf16_in, int D, int n_seg, hipStream_t st) {
    return bf16_in ? diag_by_family<bf16>(a, family, D, n_seg, st) : diag_by_family<float>(a, family, D, n_seg, st);
}

}  // namespace hy
