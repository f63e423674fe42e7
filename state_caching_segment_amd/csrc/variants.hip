// Variant patches around the cached pair, for gfx950 (HYPIC, codernav.top
// article, section on linear layers, last paragraph: conv-state warm-up and
// state re-rotation).
//
// Re-rotation.  With rotary position embeddings on the keys, channel pairs
// (i, i + d/2) are rotated by p * theta_i, theta_i = base^(-2i/d).  A pair
// cached with its keys at local positions and reused at offset P becomes
//     T' = R(P) T R(P)^T,   S' = R(P) S
// (exact when the decay commutes with R(P): scalar gates, no gates).  R(P) is
// block-diagonal in 2 x 2 rotations, so both are elementwise over quads of
// rows (i, i + d/2) and columns (j, j + d/2): a pass bound by HBM.  Angles are
// formed in fp64 and reduced modulo 2 pi before the fp32 rotation, so large
// offsets lose nothing.
//
// Conv warm-up.  A short causal depthwise convolution (K taps) feeds the
// recurrence; a seam window's first K - 1 tokens take taps from the previous
// segment.  The kernel writes the window's convolved q, k, v with those taps
// read from the raw inputs just before the window (tokens before index 0 read
// as zero), optionally through SiLU.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace hy {

constexpr int VAR_THREADS = 256;

// One (item, chain) per workgroup.
__global__ void __launch_bounds__(VAR_THREADS)
k_rerotate(RerotateArgs a) {
    __shared__ __attribute__((aligned(16))) float cs[64];
    __shared__ __attribute__((aligned(16))) float sn[64];
    const int item = blockIdx.x / a.n_chains, chain = blockIdx.x % a.n_chains;
    const int dk = a.dk, h = dk / 2, tid = threadIdx.x;
    if (tid < h) {
        const double th = pow(a.base, -2.0 * tid / dk);
        double ang = fmod((double)a.offset[item] * th, 6.283185307179586476925286766559);
        float s, c;
        sincosf((float)ang, &s, &c);
        cs[tid] = c;
        sn[tid] = s;
    }
    __syncthreads();
    const int64_t slot = a.slot[item];
    const float *T = a.T + (slot * a.n_chains + chain) * a.t_elems;
    const float *S = a.S + (slot * a.n_chains + chain) * (int64_t)dk * dk;
    float *To = a.T_out + ((int64_t)item * a.n_chains + chain) * a.t_elems;
    float *So = a.S_out + ((int64_t)item * a.n_chains + chain) * (int64_t)dk * dk;
    // S' = R S: row pairs (i, i + h), four columns per thread
    const int q4 = dk / 4;
    for (int it = tid; it < h * q4; it += VAR_THREADS) {
        const int i = it / q4, j = 4 * (it % q4);
        const f32x4 x = *reinterpret_cast<const f32x4 *>(S + i * dk + j);
        const f32x4 y = *reinterpret_cast<const f32x4 *>(S + (i + h) * dk + j);
        const float c = cs[i], s = sn[i];
        *reinterpret_cast<f32x4 *>(So + i * dk + j) = c * x - s * y;
        *reinterpret_cast<f32x4 *>(So + (i + h) * dk + j) = s * x + c * y;
    }
    if (a.t_elems == 1) {
        if (tid == 0) To[0] = T[0];  // a scalar transition commutes with R
        return;
    }
    // T' = R T R^T: rows (i, i + h) x columns (j .. j+3, j+h .. j+h+3)
    const int h4 = h / 4;  // (dk >= 16: h is a multiple of 4)
    for (int it = tid; it < h * h4; it += VAR_THREADS) {
        const int i = it / h4, j = 4 * (it % h4);
        const f32x4 t00 = *reinterpret_cast<const f32x4 *>(T + i * dk + j);
        const f32x4 t01 = *reinterpret_cast<const f32x4 *>(T + i * dk + j + h);
        const f32x4 t10 = *reinterpret_cast<const f32x4 *>(T + (i + h) * dk + j);
        const f32x4 t11 = *reinterpret_cast<const f32x4 *>(T + (i + h) * dk + j + h);
        const float ci = cs[i], si = sn[i];
        // rows
        const f32x4 a00 = ci * t00 - si * t10, a01 = ci * t01 - si * t11;
        const f32x4 a10 = si * t00 + ci * t10, a11 = si * t01 + ci * t11;
        // columns
        const f32x4 cj = *reinterpret_cast<const f32x4 *>(cs + j), sj = *reinterpret_cast<const f32x4 *>(sn + j);
        *reinterpret_cast<f32x4 *>(To + i * dk + j) = cj * a00 - sj * a01;
        *reinterpret_cast<f32x4 *>(To + i * dk + j + h) = sj * a00 + cj * a01;
        *reinterpret_cast<f32x4 *>(To + (i + h) * dk + j) = cj * a10 - sj * a11;
        *reinterpret_cast<f32x4 *>(To + (i + h) * dk + j + h) = sj * a10 + cj * a11;
    }
}

// A thread takes CPT adjacent channels of one of q, k, v of one (item,
// chain), so that each token row is one vector load and one vector store;
// consecutive threads take consecutive channel groups, then tensors, chains
// and items, and every thread of a workgroup has work.  The taps sit right-aligned in KMAX slots (zeros in front), so the
// output for window token t is sum_m taps2[m] * b[t + m] over a buffer b
// whose first KMAX - 1 entries are the tokens before the round: every index
// is a compile-time constant for any conv_k.  Each round requests its TB
// tokens before it uses any of them.
template <typename TIN>
__global__ void __launch_bounds__(VAR_THREADS)
k_conv_warmup(ConvArgs a) {
    constexpr int KMAX = 8, CPT = 4, TB = 8;
    using V = typename std::conditional<std::is_same<TIN, float>::value, f32x4, bf16x4>::type;
    const int K = a.K, nq = a.dk / CPT;
    const int64_t ts = a.x.ts, ots = (int64_t)a.n_chains * a.dk;
    const int64_t unit = (int64_t)blockIdx.x * VAR_THREADS + threadIdx.x;
    if (unit < (int64_t)a.n_items * a.n_chains * 3 * nq) {
        const int q4 = (int)(unit % nq), which = (int)(unit / nq % 3);  // 0: q, 1: k, 2: v
        const int chain = (int)(unit / (3 * nq) % a.n_chains), item = (int)(unit / (3 * nq * a.n_chains));
        const int c = q4 * CPT;
        const int64_t s0 = a.tok_begin[item];
        const TIN *x = reinterpret_cast<const TIN *>(which == 0 ? a.x.q : which == 1 ? a.x.k : a.x.v) +
                       (int64_t)chain * a.x.cs + c;
        TIN *y = reinterpret_cast<TIN *>(which == 0 ? a.q_out : which == 1 ? a.k_out : a.v_out) +
                 ((int64_t)item * a.w * a.n_chains + chain) * a.dk + c;
        const float *tp = a.taps + (((int64_t)which * a.n_chains + chain) * a.dk + c) * K;
        float taps2[CPT][KMAX];
#pragma unroll
        for (int e = 0; e < CPT; ++e)
#pragma unroll
            for (int m = 0; m < KMAX; ++m) taps2[e][m] = m >= KMAX - K ? tp[e * K + m - (KMAX - K)] : 0.f;
        float b[CPT][KMAX - 1 + TB];
        // b[.][KMAX - 2 - i] = token s0 - 1 - i: the K - 1 tokens before the
        // window (zero before token 0; older slots meet zero taps)
#pragma unroll
        for (int i = 0; i < KMAX - 1; ++i) {
            const int64_t u = s0 - 1 - i;
            V v{};
            if (i < K - 1 && u >= 0) v = *reinterpret_cast<const V *>(x + u * ts);
#pragma unroll
            for (int e = 0; e < CPT; ++e) b[e][KMAX - 2 - i] = (float)v[e];
        }
        for (int t0 = 0; t0 < a.w; t0 += TB) {
#pragma unroll
            for (int tt = 0; tt < TB; ++tt) {
                V v{};
                if (t0 + tt < a.w) v = *reinterpret_cast<const V *>(x + (s0 + t0 + tt) * ts);
#pragma unroll
                for (int e = 0; e < CPT; ++e) b[e][KMAX - 1 + tt] = (float)v[e];
            }
#pragma unroll
            for (int tt = 0; tt < TB; ++tt) {
                V out;
#pragma unroll
                for (int e = 0; e < CPT; ++e) {
                    float z = 0.f;
#pragma unroll
                    for (int m = 0; m < KMAX; ++m) z += taps2[e][m] * b[e][tt + m];
                    if (a.act == 1) z = z / (1.f + __expf(-z));
                    out[e] = (TIN)z;
                }
                if (t0 + tt < a.w) *reinterpret_cast<V *>(y + (t0 + tt) * ots) = out;
            }
#pragma unroll
            for (int e = 0; e < CPT; ++e)
#pragma unroll
                for (int i = 0; i < KMAX - 1; ++i) b[e][i] = b[e][TB + i];
        }
    }
}

// Compact pairs: one workgroup per (slot, chain) finds max |T| and writes
// T^ = T / sigma in bf16 with sigma = 2^e, max |T| = m 2^e, m in [0.5, 1), so
// that |T^| < 1 and the division is exact; T = 0 (or not finite) keeps
// sigma = 1.
__global__ void __launch_bounds__(VAR_THREADS)
k_pair_compact(const float *T, bf16 *Tc, float *scale, int dk) {
    __shared__ float wmax[VAR_THREADS / 64];
    const int64_t p = blockIdx.x;
    const float *t = T + p * dk * dk;
    bf16 *tc = Tc + p * dk * dk;
    const int n4 = dk * dk / 4, tid = threadIdx.x;
    // T is read once: each thread keeps its (at most 16) float4s for the
    // conversion after the maximum is known
    constexpr int MAXV = 128 * 128 / 4 / VAR_THREADS;
    f32x4 v[MAXV];
    float mx = 0.f;
#pragma unroll
    for (int r = 0; r < MAXV; ++r) {
        const int i = tid + r * VAR_THREADS;
        v[r] = i < n4 ? reinterpret_cast<const f32x4 *>(t)[i] : f32x4{0.f, 0.f, 0.f, 0.f};
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[r][0]), fabsf(v[r][1])), fmaxf(fabsf(v[r][2]), fabsf(v[r][3]))));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if ((tid & 63) == 0) wmax[tid >> 6] = mx;
    __syncthreads();
    mx = wmax[0];
#pragma unroll
    for (int w = 1; w < VAR_THREADS / 64; ++w) mx = fmaxf(mx, wmax[w]);
    int e = 0;
    if (mx > 0.f && isfinite(mx)) frexpf(mx, &e);
    if (tid == 0) scale[p] = ldexpf(1.f, e);
#pragma unroll
    for (int r = 0; r < MAXV; ++r) {
        const int i = tid + r * VAR_THREADS;
        bf16x4 h;
        // (ldexp, not a product with 2^-e: for a T in fp32's subnormal range
        // 2^-e itself overflows)
#pragma unroll
        for (int k = 0; k < 4; ++k) h[k] = (bf16)ldexpf(v[r][k], -e);
        if (i < n4) reinterpret_cast<bf16x4 *>(tc)[i] = h;
    }
}

hipError_t pair_compact(const float *T, bf16 *Tc, float *scale, int dk, int64_t n_pairs, hipStream_t st) {
    hipLaunchKernelGGL(k_pair_compact, dim3((unsigned)n_pairs), dim3(VAR_THREADS), 0, st, T, Tc, scale, dk);
    return hipGetLastError();
}

hipError_t rerotate(const RerotateArgs &a, int n_items, hipStream_t st) {
    hipLaunchKernelGGL(k_rerotate, dim3((unsigned)((int64_t)n_items * a.n_chains)), dim3(VAR_THREADS), 0, st, a);
    return hipGetLastError();
}

hipError_t conv_warmup(const ConvArgs &a, bool bf16_in, int n_items, hipStream_t st) {
    const int64_t units = (int64_t)n_items * a.n_chains * 3 * (a.dk / 4);
    const dim3 grid((unsigned)((units + VAR_THREADS - 1) / VAR_THREADS)), block(VAR_THREADS);
    if (bf16_in)
        hipLaunchKernelGGL(k_conv_warmup<bf16>, grid, block, 0, st, a);
    else
        hipLaunchKernelGGL(k_conv_warmup<float>, grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace hy
