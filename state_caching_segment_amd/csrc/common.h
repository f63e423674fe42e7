// Internal helpers shared by the libhypic kernels (gfx950 / CDNA4 only).
//
// Matrix-core convention used throughout: v_mfma_f32_16x16x32_bf16 computes a
// 16x16 fp32 tile D += A(16x32) B(32x16).  Lane l (r16 = l % 16, grp = l / 16)
// holds 8 bf16 of A's row r16 and 8 bf16 of B's column r16, and after the op
// holds D[4*grp + jj][r16] for jj = 0..3 (the "C layout").  The hardware pairs
// A element e with B element e of the same lane group, so the eight k values a
// lane group covers may be any fixed subset of the 32 as long as A and B use
// the same one.  Two subsets are used:
//   contiguous: k = 8*grp + e                 (both operands read from LDS)
//   permuted:   k = 4*grp + e        (e < 4)
//               k = 16 + 4*grp + e-4 (e >= 4) (one operand is a C-layout
//               accumulator pair: rows 4*grp+jj of two stacked 16-row tiles)
// The permuted subset lets a state kept in accumulators feed the next product
// directly, without a round trip through LDS.
//
// fp32 accuracy on bf16 matrix cores: x = hi + lo with hi = bf16(x) and
// lo = bf16(x - hi) (the residual is exact in fp32).  x*y is taken as
// hi*hi + hi*lo + lo*hi (three passes, relative error ~2^-17) or, when one
// operand is exactly a bf16 value, as two passes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hy {

constexpr int CH = 64;  // tokens per chunk of the chunked (UT/WY) build

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum Family { LINEAR = 0, RETNET = 1, MAMBA2 = 2, GLA = 3, DELTANET = 4, GDN = 5, KDA = 6 };

__host__ __device__ constexpr bool fam_dense(int f) { return f == DELTANET || f == GDN || f == KDA; }
__host__ __device__ constexpr bool fam_beta(int f) { return f == DELTANET || f == GDN || f == KDA; }
__host__ __device__ constexpr bool fam_vgate(int f) { return f == GLA || f == KDA; }
__host__ __device__ constexpr bool fam_sgate(int f) { return f == MAMBA2 || f == GDN; }

// Token tensors, strides in elements (innermost feature axis contiguous).
struct Tok {
    const void *q, *k, *v, *g, *beta;
    const float *gamma;
    int64_t ts, cs;    // q, k, v: token, chain
    int64_t gts, gcs;  // g
    int64_t bts, bcs;  // beta
};

__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// The lane index as a value the compiler cannot carry across calls: per-lane
// constants derived from it are recomputed where they are used instead of
// being hoisted out of a loop, where they would hold registers for its whole
// length (the empty asm emits no instruction).
__device__ __forceinline__ int lane_fresh() {
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    return lane;
}

__device__ __forceinline__ void split1(float x, bf16 &h, bf16 &l) {
    h = (bf16)x;
    l = (bf16)(x - (float)h);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Split two fp32 values into hi = bf16(x) and lo = bf16(x - hi) (both round to
// nearest even), as packed pairs: one packed conversion each, hi widened back
// with a shift and a mask rather than converted again.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t &h, uint32_t &l) {
    h = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, bf16x2));
    const float h0 = __builtin_bit_cast(float, h << 16), h1 = __builtin_bit_cast(float, h & 0xffff0000u);
    l = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0 - h0, x1 - h1}, bf16x2));
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Split eight fp32 values into hi / lo bf16 vectors.
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8 &h, bf16x8 &l) {
    u32x4 hu, lu;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        uint32_t a, b;
        split2(x[2 * e], x[2 * e + 1], a, b);
        hu[e] = a;
        lu[e] = b;
    }
    h = __builtin_bit_cast(bf16x8, hu);
    l = __builtin_bit_cast(bf16x8, lu);
}

// 8 bf16 of row `row` of a row-major LDS matrix, permuted k subset at kbase.
__device__ __forceinline__ bf16x8 lds_perm(const bf16 *M, int ld, int row, int kbase, int grp) {
    const bf16 *p = M + row * ld + kbase + 4 * grp;
    bf16x4 a = *reinterpret_cast<const bf16x4 *>(p);
    bf16x4 b = *reinterpret_cast<const bf16x4 *>(p + 16);
    bf16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
    r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
    return r;
}

// 8 bf16 of row `row`, contiguous k subset at kbase.
__device__ __forceinline__ bf16x8 lds_cont(const bf16 *M, int ld, int row, int kbase, int grp) {
    return *reinterpret_cast<const bf16x8 *>(M + row * ld + kbase + 8 * grp);
}

// Gather the permuted-k B operand of one 32-row k block from two stacked
typedef short s4 __attribute__((ext_vector_type(4)));

// 4 consecutive rows k0 .. k0+3 of column c0 + r16 of a row-major bf16 LDS
// matrix (all 16 lanes of a lane group pass the same k0 and c0): the gfx950
// transpose read, where source lane 4m + q supplies row k0 + m, columns
// c0 + 4q .. c0 + 4q + 3.
__device__ __forceinline__ bf16x4 lds_tr4(const bf16 *M, int ld, int k0, int c0, int r16) {
    const bf16 *p = M + (k0 + (r16 >> 2)) * ld + c0 + 4 * (r16 & 3);
    const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4 *)(p));
    return __builtin_bit_cast(bf16x4, v);
}

// permuted-k A fragment of row-major M transposed: rows = columns c0 + r16 of
// M, k = rows kbase + {4grp .. 4grp+3, 16+4grp .. 16+4grp+3}
__device__ __forceinline__ bf16x8 lds_tr_perm(const bf16 *M, int ld, int kbase, int c0, int r16, int grp) {
    const bf16x4 a = lds_tr4(M, ld, kbase + 4 * grp, c0, r16);
    const bf16x4 b = lds_tr4(M, ld, kbase + 16 + 4 * grp, c0, r16);
    bf16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
    r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
    return r;
}

// C-layout accumulator tiles (rows 0..15 in `top`, rows 16..31 in `bot`).
__device__ __forceinline__ void acc_to_perm(const f32x4 &top, const f32x4 &bot, float (&x)[8]) {
    x[0] = top[0]; x[1] = top[1]; x[2] = top[2]; x[3] = top[3];
    x[4] = bot[0]; x[5] = bot[1]; x[6] = bot[2]; x[7] = bot[3];
}

template <typename T>
__device__ __forceinline__ float ldf(const T *p) { return (float)(*p); }

// Load 8 consecutive elements as fp32 (16-byte aligned for bf16, 32 for fp32).
__device__ __forceinline__ void load8(const bf16 *p, float (&x)[8]) {
    bf16x8 v = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
}
__device__ __forceinline__ void load8(const float *p, float (&x)[8]) {
    f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
    x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
    x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}

__device__ __forceinline__ float wave_sum16x(float v) {
    // sum over the four lane groups that share r16 (lanes l, l^16, l^32, l^48)
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

}  // namespace hy

namespace hy {

// ---- fp32 matrix-core path (fp32 inputs): the same 8-element k subsets, each
// element position e taken by one v_mfma_f32_16x16x4_f32 (k = lane group).
__device__ __forceinline__ void lds_cont_f(const float *M, int ld, int row, int kbase, int grp, float (&x)[8]) {
    const float *p = M + row * ld + kbase + 8 * grp;
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
    x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
    x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}

__device__ __forceinline__ void lds_perm_f(const float *M, int ld, int row, int kbase, int grp, float (&x)[8]) {
    const float *p = M + row * ld + kbase + 4 * grp;
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 16);
    x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
    x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}

__device__ __forceinline__ f32x4 mma_f32(const float (&a)[8], const float (&b)[8], f32x4 c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    return c;
}

// D += A B with fp32 fragments: fp32 matrix cores (F32) or the three-pass
// bf16 split (hi*hi + hi*lo + lo*hi).
template <bool F32>
__device__ __forceinline__ f32x4 mma_split(const float (&a)[8], const float (&b)[8], f32x4 c) {
    if constexpr (F32) {
        return mma_f32(a, b, c);
    } else {
        bf16x8 ah, al, bh, bl;
        split8(a, ah, al);
        split8(b, bh, bl);
        c = mfma(ah, bh, c);
        c = mfma(ah, bl, c);
        c = mfma(al, bh, c);
        return c;
    }
}

}  // namespace hy
