/*
 * hypic.h -- C ABI of libhypic: segment state caching for the linear-attention
 * layers of hybrid models, on AMD Instinct MI355X (gfx950).
 *
 * The method (HYPIC; codernav.top article, section "linear layers: caching
 * the segment-accumulated transition operator"; xix.ai article, paragraph on
 * linear layers):  a linear-attention layer keeps one state S (dk x dv) per
 * head and every token t updates it as
 *        S_t = A_t S_{t-1} + beta_t k_t v_t^T,      o_t = S_t^T q_t
 * with a family-specific transition A_t.  For each prompt segment C the
 * library caches the pair (T_C, S(C|0)): T_C is the ordered product of the
 * segment's transitions (later tokens on the left) and S(C|0) the segment's
 * final state read from a zero state.  Any request's state is then assembled
 * with the composition law  S(C1.C2) = T(C2) S(C1) + S(C2).  The first w
 * tokens of every internal segment (the seam window; codernav.top article,
 * section on full-attention layers and seam windows, w = 8 by default) are
 * kept out of the cache and advanced token by token at reuse, emitting their
 * outputs o_t.
 *
 * Transitions (state S is dk x dv; g is the log-gate, decay = exp(g)):
 *   HYPIC_LINEAR    A = I                                  beta = 1
 *   HYPIC_RETNET    A = gamma I   (gamma per chain)        beta = 1
 *   HYPIC_MAMBA2    A = exp(g_t) I   (scalar g)            beta = 1
 *   HYPIC_GLA       A = diag(exp(g_t))   (g_t in R^dk)     beta = 1
 *   HYPIC_DELTANET  A = I - beta_t k_t k_t^T
 *   HYPIC_GDN       A = exp(g_t) (I - beta_t k_t k_t^T)
 *   HYPIC_KDA       A = (I - beta_t k_t k_t^T) diag(exp(g_t))   (decay, then erase)
 *
 * Conventions shared by every call
 *   - A "chain" is one (layer, head) of one request; n_chains chains share
 *     every token index.  Token tensors are token-major:
 *       q, k: x[t*tok_stride + c*chain_stride + i], i < dk
 *       v:    x[t*tok_stride + c*chain_stride + j], j < dv
 *       g:    g[t*g_tok_stride + c*g_chain_stride (+ i for GLA/KDA)]
 *       beta: beta[t*b_tok_stride + c*b_chain_stride]
 *     Strides are in elements; the innermost (feature) axis is contiguous.
 *   - q, k, v, g, beta have the layout's in_dtype (fp32 or bf16).  gamma,
 *     T, S, states and outputs are fp32.
 *   - dk == dv, with dk in {16, 32, 64, 128}.
 *   - Every pointer argument named d_* is DEVICE memory the caller owns; the
 *     library never allocates, frees or keeps device memory (a workspace, when
 *     an op needs one, is passed in and sized by hypic_workspace_bytes).
 *     Structs and scalar arguments are host memory, read during the call.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) with no host synchronisation.  Calls on different streams are
 *     thread-safe.
 *   - Errors: arguments visible on the host are validated before any HIP
 *     call (null pointers, unknown family/dtype, dims, w, strides and 16-byte
 *     alignment of q/k/v rows, token strides up to 2^24 elements, workspace
 *     size).  A failing check returns a negative status and enqueues nothing.
 *     Launch failures return HYPIC_E_DEVICE.  Device-resident contents
 *     (offsets, slot ids) are trusted; out-of-range values there are
 *     undefined behaviour -- unless the environment variable HYPIC_VALIDATE
 *     is "1": then every call first reads them back (a synchronous copy on
 *     `stream`) and rejects, with HYPIC_E_INVALID, segment ranges that are
 *     negative, reversed or longer than max_seg_len; list offsets that are
 *     negative, decreasing or longer than max_list_len; slot ids outside
 *     [0, n_slots); seam starts below -1; negative seam-advance starts.  The
 *     token count is not an argument, so token indices are checked for sign
 *     only.  The detail of the last error on the calling thread is in
 *     hypic_last_error().  On error the outputs are unspecified.
 *   - HYPIC_FAULT_INJECT ("1" or "all"; or "build", "compose", "seam",
 *     "rerotate", "conv", "compact" for one call): after its arguments have been validated, the call returns
 *     HYPIC_E_DEVICE and enqueues nothing.  For testing callers' error paths.
 *   - HYPIC_DEBUG (any value but "0"): every call synchronizes `stream`
 *     after its launch, so that an error in the kernel's execution returns
 *     HYPIC_E_DEVICE from the call that launched it, naming the launch in
 *     hypic_last_error() (without it, such an error surfaces at the caller's
 *     next synchronization).  Calls become synchronous.
 *   - dv must equal dk (HYPIC_E_UNSUPPORTED otherwise): every kernel keeps the
 *     state and T in tiles of the same width, and every workload these
 *     kernels are sized for has dk == dv.
 */
#ifndef HYPIC_H
#define HYPIC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum hypic_status {
    HYPIC_OK = 0,
    HYPIC_E_INVALID = -1,     /* bad argument (null pointer, size, stride, alignment, w) */
    HYPIC_E_UNSUPPORTED = -2, /* valid request this build does not implement */
    HYPIC_E_WORKSPACE = -3,   /* workspace missing or too small */
    HYPIC_E_DEVICE = -4       /* HIP launch or runtime error */
};

enum hypic_family {
    HYPIC_LINEAR = 0,
    HYPIC_RETNET = 1,
    HYPIC_MAMBA2 = 2,
    HYPIC_GLA = 3,
    HYPIC_DELTANET = 4,
    HYPIC_GDN = 5,
    HYPIC_KDA = 6
};

enum hypic_dtype { HYPIC_F32 = 0, HYPIC_BF16 = 1 };

/* hypic_compose modes: left-to-right, or the associative tree scan with
 * (T_b, S_b) o (T_a, S_a) = (T_b T_a, T_b S_a + S_b). */
enum hypic_mode { HYPIC_SEQ = 0, HYPIC_TREE = 1 };

/* hypic_workspace_bytes ops */
enum hypic_op { HYPIC_OP_BUILD = 0, HYPIC_OP_COMPOSE_SEQ = 1, HYPIC_OP_COMPOSE_TREE = 2, HYPIC_OP_SEAM = 3 };

typedef struct hypic_layout {
    int32_t family;   /* enum hypic_family */
    int32_t in_dtype; /* enum hypic_dtype of q, k, v, g, beta */
    int32_t n_chains; /* chains per token index (e.g. layers x heads), >= 1 */
    int32_t dk;       /* key / state rows */
    int32_t dv;       /* value / state columns; must equal dk */
} hypic_layout;

typedef struct hypic_tokens {
    const void *q;       /* [tok][chain][dk]; read only by seam advance (may be NULL for build) */
    const void *k;       /* [tok][chain][dk] */
    const void *v;       /* [tok][chain][dv] */
    const void *g;       /* log-gates: [tok][chain] (MAMBA2, GDN) or [tok][chain][dk] (GLA, KDA); else NULL */
    const void *beta;    /* [tok][chain] (DELTANET, GDN, KDA); else NULL */
    const float *gamma;  /* [n_chains] fp32 (RETNET); else NULL */
    int64_t tok_stride, chain_stride;     /* q, k, v */
    int64_t g_tok_stride, g_chain_stride; /* g */
    int64_t b_tok_stride, b_chain_stride; /* beta */
} hypic_tokens;

/* Number of fp32 values one cached T occupies for a family: 1 (LINEAR,
 * RETNET, MAMBA2: a scalar times I), dk (GLA: a diagonal), dk*dk (DELTANET,
 * GDN, KDA: dense, row-major).  0 for an unknown family. */
int64_t hypic_t_elems(int32_t family, int32_t dk);

/* Device workspace, in bytes, that `op` needs for n_items (segments for
 * BUILD, requests for COMPOSE_*, items for SEAM) with max_len the longest
 * segment (BUILD) or list (COMPOSE_*) and seam width w (0: no seams).  0 means
 * no workspace is needed (every op but HYPIC_OP_COMPOSE_TREE), and also the
 * answer for invalid arguments.  The workspace holds no state between calls. */
size_t hypic_workspace_bytes(const hypic_layout *L, int32_t op, int32_t n_items, int64_t max_len, int32_t w);

/*
 * hypic_segment_build -- the cached pair of every segment on every chain.
 * (codernav.top, linear layers: at a segment's first prefill the system
 * caches (T_C, S(C|0)); both depend only on the segment's own tokens.)
 *
 * Segment s covers tokens [d_seg_begin[s], d_seg_end[s]) of x; an empty range
 * gives T = I, S = 0.  max_seg_len (host) bounds every segment's length.
 * Outputs, fully overwritten:
 *   d_T [n_seg][n_chains][hypic_t_elems(family, dk)]
 *   d_S [n_seg][n_chains][dk][dv]
 * d_T and d_S must not overlap the inputs.
 */
int hypic_segment_build(const hypic_layout *L, const hypic_tokens *x, int32_t n_seg,
                        const int64_t *d_seg_begin, const int64_t *d_seg_end, int64_t max_seg_len,
                        float *d_T, float *d_S, void *d_ws, size_t ws_bytes, void *stream);

/*
 * hypic_segment_prefill -- the fused cold prefill of segment bodies: in one
 * chunked pass, every token's output and the segment's cached pair
 * (codernav.top, linear layers: the pair is cached at the segment's first
 * prefill; results: building it costs a few percent of that forward).
 * Segment s covers tokens [d_seg_begin[s], d_seg_end[s]) and is read from a
 * zero state, so its outputs are those of the position-independent body:
 *   o_t = S_t^T q_t,  S_t the state after token t of the segment from S = 0,
 * written to d_out[t * out_tok_stride + c * out_chain_stride + j] (j < dv) in
 * the input dtype; d_T and d_S as hypic_segment_build writes them.  q is
 * required.  Implemented for DeltaNet and GDN with bf16 inputs
 * (HYPIC_E_UNSUPPORTED otherwise).  Every chunk of 64 tokens must keep its
 * total log-decay above about -80 (the chunk form scales the solved rows by
 * the chunk's decay).  d_out must not overlap the inputs or the pair; it is
 * 8-byte aligned with strides that are multiples of 4 elements
 * (HYPIC_E_INVALID otherwise).
 */
int hypic_segment_prefill(const hypic_layout *L, const hypic_tokens *x, int32_t n_seg,
                          const int64_t *d_seg_begin, const int64_t *d_seg_end, int64_t max_seg_len,
                          float *d_T, float *d_S, void *d_out, int64_t out_tok_stride,
                          int64_t out_chain_stride, void *stream);

/*
 * hypic_compose -- assemble request states from cached pairs
 * (codernav.top, linear layers: reuse left-multiplies T_C, then adds S(C|0);
 * seam windows: the linear layers advance the running state through each
 * seam window and pass every seam token's output up).
 *
 * Request r walks its entries e = d_list_off[r] .. d_list_off[r+1]-1 in
 * order.  For each entry: if seam != NULL and d_seam_begin[e] >= 0, advance
 * the state through tokens d_seam_begin[e] .. +w-1 of `seam`, writing
 * o_t = S_t^T q_t to d_o[((e*w + i)*n_chains + c)*dv + j]; then apply the
 * entry's pair:  S <- T[slot] S + S[slot],  slot = d_pair_id[e].
 *   d_T, d_S      pair cache laid out as hypic_segment_build writes it,
 *                 slots 0 .. n_slots-1 (read only)
 *   d_state       [n_req][n_chains][dk][dv]: in = initial state (zero for a
 *                 fresh request), out = final state
 *   d_o           [n_entries][w][n_chains][dv]; rows of entries without a seam
 *                 are left untouched.  May be NULL when seam == NULL.
 *   d_prefix_states  NULL, or [n_entries][n_chains][dk][dv]: the state after
 *                 entry e (its seam window and its pair), for every entry e
 *                 the lists name (the running states a combine step hands on;
 *                 codernav.top, segment parallelism).  Indexed like d_pair_id.
 *                 In HYPIC_TREE mode they come from a second, parallel pass
 *                 over each block from the state entering it (the scan's
 *                 down-sweep), which also writes the block's seam outputs.
 * mode HYPIC_TREE computes the same result (to rounding) through the
 * associative scan: blocks of about sqrt(max_list_len) entries (shorter ones
 * when the blocks cannot fill the GPU; fewer, longer ones, at most 64
 * entries, when n_req * n_chains alone fill it) are reduced in parallel,
 * their aggregates scanned, and seam outputs fixed up; it needs a
 * workspace of hypic_workspace_bytes(L, HYPIC_OP_COMPOSE_TREE, n_req,
 * max_list_len, w) bytes (HYPIC_E_WORKSPACE if missing or smaller).  HYPIC_SEQ
 * needs none.  max_list_len must bound every request's entry count.
 * Alignment: d_T and d_S 16-byte, d_state, d_o and d_prefix_states 4-byte
 * (HYPIC_E_INVALID otherwise).
 */
int hypic_compose(const hypic_layout *L, int32_t mode, int32_t n_req, int32_t max_list_len,
                  const int32_t *d_list_off, const int32_t *d_pair_id, int64_t n_slots,
                  const float *d_T, const float *d_S, const hypic_tokens *seam,
                  const int64_t *d_seam_begin, int32_t w, float *d_state, float *d_o,
                  float *d_prefix_states, void *d_ws, size_t ws_bytes, void *stream);

/*
 * hypic_compose_tree_noalloc -- hypic_compose in HYPIC_TREE mode for callers
 * that cannot allocate device memory (code under graph capture, tight serving
 * loops, harnesses that forbid allocation).  Arguments and results are those
 * of hypic_compose with mode HYPIC_TREE; the workspace is the library's own:
 * HYPIC_NOALLOC_WORKSPACE_BYTES of device memory per GPU, part of the loaded
 * code object and held until the process ends.  The call allocates nothing.
 * A call whose workspace (hypic_workspace_bytes with HYPIC_OP_COMPOSE_TREE)
 * would exceed it returns HYPIC_E_WORKSPACE before any HIP call.  Every call
 * on one GPU shares that GPU's workspace: calls that overlap on one GPU (on
 * different streams, or from different threads) race and give undefined
 * results; calls on one stream are ordered and safe.  Nothing in the
 * workspace needs to start at any value.
 */
#define HYPIC_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)
int hypic_compose_tree_noalloc(const hypic_layout *L, int32_t n_req, int32_t max_list_len,
                               const int32_t *d_list_off, const int32_t *d_pair_id, int64_t n_slots,
                               const float *d_T, const float *d_S, const hypic_tokens *seam,
                               const int64_t *d_seam_begin, int32_t w, float *d_state, float *d_o,
                               float *d_prefix_states, void *stream);

/*
 * hypic_seam_advance -- advance n_items independent states through w tokens
 * each (codernav.top, seam windows: the linear layers compute the window's
 * transition and state on the fly, advance the running state and emit each
 * seam token's output).
 *   d_tok_begin [n_items]: first token of each item's window in x
 *   d_state     [n_items][n_chains][dk][dv], updated in place
 *   d_o         [n_items][w][n_chains][dv], o_t = S_t^T q_t (post-update)
 */
int hypic_seam_advance(const hypic_layout *L, const hypic_tokens *x, int32_t n_items,
                       const int64_t *d_tok_begin, int32_t w, float *d_state, float *d_o,
                       void *stream);

/*
 * hypic_rerotate -- move cached pairs to the absolute offsets they are reused
 * at, for models with rotary position embeddings on the keys (codernav.top,
 * linear layers, last paragraph: state re-rotation; xix.ai, paragraph on
 * linear layers).  Rotation R(p): each channel pair (i, i + dk/2), i < dk/2,
 * turns by p * rope_base^(-2i/dk):
 *     (R x)_i = cos x_i - sin x_{i+dk/2},   (R x)_{i+dk/2} = sin x_i + cos x_{i+dk/2}
 * (angles formed in fp64).  A pair built with the segment's keys at local
 * positions 0, 1, ... and reused with its first token at position p is then
 *     T' = R(p) T R(p)^T  (a scalar T is unchanged),   S' = R(p) S.
 * Item i reads slot d_slot[i] of (d_T, d_S) and writes item i of
 *   d_T_out [n_items][n_chains][t_elems], d_S_out [n_items][n_chains][dk][dv]
 * at offset d_offset[i].  In place is allowed when d_T_out == d_T,
 * d_S_out == d_S and d_slot[i] == i; no other overlap.  The law holds when
 * the decay commutes with R(p): LINEAR, RETNET, MAMBA2, DELTANET, GDN.  GLA
 * and KDA (per-channel gates) return HYPIC_E_UNSUPPORTED.  All pointers 16-byte
 * aligned; rope_base > 1.
 */
int hypic_rerotate(const hypic_layout *L, int32_t n_items, const int32_t *d_slot, const int64_t *d_offset,
                   double rope_base, const float *d_T, const float *d_S, float *d_T_out, float *d_S_out,
                   void *stream);

/*
 * hypic_conv_warmup -- the seam windows' inputs for models with a short
 * causal depthwise convolution before the recurrence (codernav.top, linear
 * layers, last paragraph: conv-state warm-up).  A seam window's first
 * conv_k - 1 tokens take taps from the previous segment; this call feeds them
 * the raw inputs just before the window:
 *     y_t[c] = act( sum_{j<conv_k} taps[c][j] x_{t-conv_k+1+j}[c] )
 * for t = d_tok_begin[i] .. + w - 1 (raw tokens before index 0 read as zero),
 * for each of q, k, v.
 *   raw        raw (pre-convolution) q, k, v, strided as hypic_tokens
 *              (g, beta, gamma unused)
 *   d_taps     [3][n_chains][dk][conv_k] fp32 (q, k, v), 1 <= conv_k <= 8
 *   act        0: none, 1: SiLU  z / (1 + e^-z)
 *   d_q_out, d_k_out, d_v_out  [n_items][w][n_chains][dk] in the input dtype,
 *              ready to pass to hypic_compose / hypic_seam_advance as seam
 *              tokens (tok_stride n_chains * dk, window i at token i * w).
 * raw q, k, v and the outputs 16-byte aligned, raw strides multiples of 16
 * bytes (HYPIC_E_INVALID otherwise).
 */
int hypic_conv_warmup(const hypic_layout *L, const hypic_tokens *raw, const float *d_taps, int32_t conv_k,
                      int32_t act, int32_t n_items, const int64_t *d_tok_begin, int32_t w, void *d_q_out,
                      void *d_k_out, void *d_v_out, void *stream);

/*
 * Compact pairs (precision of the pair store; codernav.top, summary: tiered
 * caching of the pairs).  hypic_pair_compact converts the dense T of n_slots
 * slots to bf16 T^ with a power-of-two scale per (slot, chain):
 *     T = sigma T^,   sigma = 2^e where max|T| = m 2^e, m in [0.5, 1)
 * (|T^| < 1, the scaling exact; T = 0 keeps sigma = 1).  For GDN sigma
 * absorbs the segment's total decay.  Outputs d_Tc [n_slots][n_chains][dk][dk]
 * bf16 (8-byte aligned), d_Tscale [n_slots][n_chains] fp32; S is unchanged.
 * Dense families only.  hypic_compose_compact is the sequential
 * hypic_compose over compact pairs (T^ read in bf16: 64 + 32 KiB per pair and
 * chain at d = 128 instead of 128 KiB); DeltaNet and GDN with bf16 inputs,
 * dk >= 64.  T^'s rounding (relative 2^-8 at most per element) enters each step's
 * T S, so its error is that of bf16 T, not of the fp32 pair.  Alignment:
 * d_Tc 8-byte, d_S 16-byte, d_state, d_o and d_prefix_states 4-byte.
 */
int hypic_pair_compact(const hypic_layout *L, int32_t n_slots, const float *d_T, void *d_Tc, float *d_Tscale,
                       void *stream);
int hypic_compose_compact(const hypic_layout *L, int32_t n_req, int32_t max_list_len,
                          const int32_t *d_list_off, const int32_t *d_pair_id, int64_t n_slots,
                          const void *d_Tc, const float *d_Tscale, const float *d_S,
                          const hypic_tokens *seam, const int64_t *d_seam_begin, int32_t w,
                          float *d_state, float *d_o, float *d_prefix_states, void *stream);

/*
 * Pair store -- the host-side index of a pool of cached pairs (codernav.top,
 * segment parallelism: the router probes which segments hit the cache;
 * misses are inevitable as the corpus changes and rarely used documents are
 * evicted).  The pool is device memory the caller owns: slots
 * 0 .. n_slots-1 of the T and S arrays that hypic_segment_build writes and
 * hypic_compose reads.  The store maps a segment's content key (for example
 * hypic_content_key of its token ids) to its slot; it allocates host memory
 * only and is not thread-safe (one caller at a time per store).
 *
 * hypic_store_acquire gives every one of n keys a slot: a key already in the
 * store keeps its slot (a hit); a new key (a miss, miss_out = 1: the caller
 * builds its pair into that slot before composing) takes a free slot, else
 * evicts the entry acquired least often, ties broken by least recent
 * acquisition, never one named earlier in the same call.  Free slots are
 * handed out lowest first, then most recently freed first.  Returns the
 * number of misses, HYPIC_E_WORKSPACE (and changes nothing) if the call names
 * more distinct keys than the pool has slots, or HYPIC_E_INVALID.
 * hypic_store_evict drops a key (returns 1 if it was present, else 0);
 * hypic_store_stats fills out[4] = {entries, hits, misses, evictions}.
 */
typedef struct hypic_store hypic_store;
hypic_store *hypic_store_create(int64_t n_slots); /* NULL if n_slots is not in 1 .. 2^31-1 */
void hypic_store_destroy(hypic_store *store);
int hypic_store_acquire(hypic_store *store, int32_t n, const uint64_t *keys, int32_t *slots_out,
                        uint8_t *miss_out);
int hypic_store_evict(hypic_store *store, uint64_t key);
int hypic_store_stats(const hypic_store *store, int64_t *out);
/* 64-bit FNV-1a hash of nbytes of host memory: a content key. */
uint64_t hypic_content_key(const void *data, size_t nbytes);

/* Static text for a status code. */
const char *hypic_status_string(int status);
/* Detail of the last failing call on this thread ("" if none). */
const char *hypic_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* HYPIC_H */
