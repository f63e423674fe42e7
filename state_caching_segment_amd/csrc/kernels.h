// Launchers of the libhypic kernels (internal; the C ABI is in include/hypic.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace hy {

struct BuildArgs {
    Tok x;
    int n_chains;
    int dk;
    const int64_t *seg_begin;
    const int64_t *seg_end;
    float *T;  // [seg][chain][t_elems]
    float *S;  // [seg][chain][dk][dk]
    void *o;   // fused prefill: per-token outputs o[t * ots + chain * ocs + j], in the input dtype; else null
    int64_t ots, ocs;
};

struct ComposeArgs {
    Tok x;  // seam tokens (q, k, v, g, beta, gamma)
    int n_chains;
    int dk;
    int w;
    int has_seam;
    const int32_t *list_off;
    const int32_t *pair_id;
    const float *T;
    const float *S;
    int64_t t_elems;
    const int64_t *seam_begin;
    float *state;   // [req][chain][dk][dk]
    float *o;       // [entry][w][chain][dk]
    float *prefix;  // [entry][chain][dk][dk]: state after each entry, or null
    const float *t_scale;  // compact pairs: T = t_scale[slot][chain] * T^ (bf16 at T); else null
};

struct SeamArgs {
    Tok x;
    int n_chains;
    int dk;
    int w;
    const int64_t *tok_begin;
    float *state;  // [item][chain][dk][dk]
    float *o;      // [item][w][chain][dk]
};

struct TreeArgs {
    ComposeArgs c;
    int B;         // entries per block
    int NB;        // blocks per request (upper bound)
    int max_list;  // entries per request (upper bound)
    float *aggT;   // [req][NB][chain][dk][dk] block aggregates
    float *aggS;
    float *sin;    // [req][NB][chain][dk][dk] state entering each block
    float *pvec;   // [req][max_list][w][chain][dk] pulled-back seam queries
    int32_t *blk_off;  // [req * NB + 1] entry offsets of every block (prefix states only)
};

// D is the padded state size (32, 64 or 128) the kernel is instantiated for.
hipError_t build_dense(const BuildArgs &a, int family, bool bf16_in, int D, int n_seg, hipStream_t st);
hipError_t build_dense_pipe(const BuildArgs &a, int family, int D, int n_seg, hipStream_t st);
hipError_t build_kda(const BuildArgs &a, bool bf16_in, int D, int n_seg, hipStream_t st);
hipError_t build_kda_pipe(const BuildArgs &a, int D, int n_seg, hipStream_t st);  // bf16 inputs
hipError_t build_diag(const BuildArgs &a, int family, bool bf16_in, int D, int n_seg, hipStream_t st);
hipError_t compose_seq(const ComposeArgs &a, int family, bool bf16_in, int D, int n_req, hipStream_t st);
hipError_t compose_tree(const TreeArgs &t, int family, bool bf16_in, int D, int n_req, hipStream_t st);
hipError_t seam_advance(const SeamArgs &a, int family, bool bf16_in, int D, int n_items, hipStream_t st);
// sequential compose of compact pairs (DeltaNet, GDN; bf16 inputs; D 64 or 128)
hipError_t compose_seq_compact(const ComposeArgs &a, int family, int D, int n_req, hipStream_t st);
// compact pairs: T^ (bf16) and the power-of-two scale of each (slot, chain) from fp32 T
hipError_t pair_compact(const float *T, bf16 *Tc, float *scale, int dk, int64_t n_pairs, hipStream_t st);

// Re-rotation of cached pairs to absolute offsets (rotary embeddings): item i
// reads slot slot[i] and writes (R T R^T, R S) at offset offset[i] to item i.
struct RerotateArgs {
    int n_chains;
    int dk;
    int64_t t_elems;      // 1 (scalar T) or dk * dk
    const int32_t *slot;  // [item]
    const int64_t *offset;
    double base;
    const float *T, *S;
    float *T_out, *S_out;
};

// Conv warm-up of seam windows: q, k, v of tokens tok_begin[i] .. + w - 1
// through the causal depthwise convolution, taps [3][chain][dk][K].
struct ConvArgs {
    Tok x;  // raw (pre-convolution) q, k, v
    int n_chains;
    int n_items;
    int dk;
    int w;
    int K;
    int act;  // 0: none, 1: SiLU
    const int64_t *tok_begin;
    const float *taps;
    void *q_out, *k_out, *v_out;  // [item][w][chain][dk], input dtype
};

hipError_t rerotate(const RerotateArgs &a, int n_items, hipStream_t st);
hipError_t conv_warmup(const ConvArgs &a, bool bf16_in, int n_items, hipStream_t st);

// The library's own tree-compose workspace: kStaticWorkspaceBytes of device
// memory per GPU (a file-scope device array), its address on the current
// device in *ptr.  Every call on one GPU shares it.
constexpr size_t kStaticWorkspaceBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
hipError_t static_workspace(void **ptr);

}  // namespace hy
