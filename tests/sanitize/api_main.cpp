// Host sanitizer driver for the C ABI's host code (test infrastructure):
// argument validation of every entry point, the workspace and status
// helpers, under AddressSanitizer and UndefinedBehaviorSanitizer, with the
// kernel launchers replaced by stand-ins.  Device pointers are never
// dereferenced on these paths, so placeholders stand for them.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/hypic.h"

#define CHECK(c) do { if (!(c)) { std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

static void *P(uintptr_t a) { return reinterpret_cast<void *>(a); }

int main() {
    // placeholders, 256-byte aligned
    const uintptr_t A = 0x100000;
    hypic_layout L{HYPIC_GDN, HYPIC_BF16, 4, 128, 128};
    hypic_tokens x{};
    x.q = P(A); x.k = P(A); x.v = P(A); x.g = P(A); x.beta = P(A);
    x.tok_stride = 4 * 128; x.chain_stride = 128;
    x.g_tok_stride = 4; x.g_chain_stride = 1;
    x.b_tok_stride = 4; x.b_chain_stride = 1;
    const int64_t *sb = static_cast<const int64_t *>(P(A)), *se = static_cast<const int64_t *>(P(A + 256));
    float *T = static_cast<float *>(P(A)), *S = static_cast<float *>(P(A + 512));

    CHECK(hypic_t_elems(HYPIC_GDN, 128) == 128 * 128 && hypic_t_elems(HYPIC_GLA, 64) == 64);
    CHECK(hypic_t_elems(HYPIC_RETNET, 32) == 1 && hypic_t_elems(42, 32) == 0);
    for (int s = 1; s >= -6; --s) CHECK(hypic_status_string(s) != nullptr);

    // build: each bad argument refused
    hypic_layout bad = L; bad.dk = bad.dv = 100;
    CHECK(hypic_segment_build(&bad, &x, 1, sb, se, 10, T, S, nullptr, 0, nullptr) == HYPIC_E_INVALID);
    bad = L; bad.dv = 64;
    CHECK(hypic_segment_build(&bad, &x, 1, sb, se, 10, T, S, nullptr, 0, nullptr) == HYPIC_E_UNSUPPORTED);
    bad = L; bad.n_chains = 0;
    CHECK(hypic_segment_build(&bad, &x, 1, sb, se, 10, T, S, nullptr, 0, nullptr) == HYPIC_E_INVALID);
    bad = L; bad.family = 9;
    CHECK(hypic_segment_build(&bad, &x, 1, sb, se, 10, T, S, nullptr, 0, nullptr) == HYPIC_E_INVALID);
    hypic_tokens xb = x; xb.k = P(A + 2);
    CHECK(hypic_segment_build(&L, &xb, 1, sb, se, 10, T, S, nullptr, 0, nullptr) == HYPIC_E_INVALID);
    xb = x; xb.g = nullptr;
    CHECK(hypic_segment_build(&L, &xb, 1, sb, se, 10, T, S, nullptr, 0, nullptr) == HYPIC_E_INVALID);
    xb = x; xb.tok_stride = (int64_t(1) << 24) + 8;  // 32-bit offsets in the kernels
    CHECK(hypic_segment_build(&L, &xb, 1, sb, se, 10, T, S, nullptr, 0, nullptr) == HYPIC_E_UNSUPPORTED);
    CHECK(hypic_segment_build(&L, &x, -1, sb, se, 10, T, S, nullptr, 0, nullptr) == HYPIC_E_INVALID);
    CHECK(hypic_segment_build(&L, &x, 2, nullptr, se, 10, T, S, nullptr, 0, nullptr) == HYPIC_E_INVALID);
    CHECK(hypic_segment_build(&L, &x, 0, nullptr, nullptr, 0, nullptr, nullptr, nullptr, 0, nullptr) == HYPIC_OK);
    // a call that passes validation reaches the (stand-in) launcher
    CHECK(hypic_segment_build(&L, &x, 2, sb, se, 10, T, S, nullptr, 0, nullptr) == HYPIC_E_DEVICE);
    CHECK(hypic_last_error() != nullptr && std::strlen(hypic_last_error()) > 0);

    // compose and seam advance
    hypic_layout L64{HYPIC_GDN, HYPIC_BF16, 4, 64, 64};
    hypic_tokens x64 = x; x64.tok_stride = 4 * 64; x64.chain_stride = 64;
    const int32_t *lo = static_cast<const int32_t *>(P(A)), *pid = static_cast<const int32_t *>(P(A + 256));
    float *st = static_cast<float *>(P(A + 1024)), *o = static_cast<float *>(P(A + 2048));
    CHECK(hypic_compose(&L64, 5, 1, 2, lo, pid, 2, T, S, nullptr, nullptr, 0, st, nullptr, nullptr, nullptr, 0,
                        nullptr) == HYPIC_E_INVALID);
    CHECK(hypic_compose(&L64, HYPIC_SEQ, 1, 2, lo, pid, 2, T, S, &x64, sb, -1, st, o, nullptr, nullptr, 0,
                        nullptr) == HYPIC_E_INVALID);
    CHECK(hypic_compose(&L64, HYPIC_SEQ, 1, 2, lo, pid, 2, T, S, &x64, nullptr, 8, st, o, nullptr, nullptr, 0,
                        nullptr) == HYPIC_E_INVALID);
    CHECK(hypic_compose(&L64, HYPIC_TREE, 1, 2, lo, pid, 2, T, S, nullptr, nullptr, 0, st, nullptr, nullptr,
                        nullptr, 0, nullptr) == HYPIC_E_WORKSPACE);
    CHECK(hypic_compose(&L64, HYPIC_SEQ, 0, 0, nullptr, nullptr, 0, nullptr, nullptr, nullptr, nullptr, 0, nullptr,
                        nullptr, nullptr, nullptr, 0, nullptr) == HYPIC_OK);
    CHECK(hypic_workspace_bytes(&L64, HYPIC_OP_COMPOSE_TREE, 3, 48, 8) > 0);
    CHECK(hypic_workspace_bytes(&L64, 99, 3, 48, 8) == 0);
    CHECK(hypic_seam_advance(&L64, &x64, 2, nullptr, 8, st, o, nullptr) == HYPIC_E_INVALID);

    // variant patches and compact pairs refuse bad arguments
    CHECK(hypic_rerotate(&L, -1, nullptr, nullptr, 10000.0, T, S, T, S, nullptr) == HYPIC_E_INVALID);
    CHECK(hypic_pair_compact(&L, -1, T, P(A), st, nullptr) == HYPIC_E_INVALID);
    hypic_layout Lk{HYPIC_KDA, HYPIC_BF16, 4, 128, 128};
    CHECK(hypic_rerotate(&Lk, 1, pid, sb, 10000.0, T, S, T, S, nullptr) == HYPIC_E_UNSUPPORTED);
    std::printf("api sanitizer driver: ok\n");
    return 0;
}
