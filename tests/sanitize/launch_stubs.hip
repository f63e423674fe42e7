// Host-only stand-ins for the kernel launchers (test infrastructure): the
// sanitizer build of the C ABI's host code links these instead of the device
// code and exercises argument validation only.  Every launch reports a
// device error, so a call that passes validation fails with HYPIC_E_DEVICE
// without touching a GPU.
#include "../../state_caching_segment_amd/csrc/kernels.h"

namespace hy {
hipError_t build_dense(const BuildArgs &, int, bool, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t build_dense_pipe(const BuildArgs &, int, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t build_kda(const BuildArgs &, bool, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t build_kda_pipe(const BuildArgs &, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t build_diag(const BuildArgs &, int, bool, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t compose_seq(const ComposeArgs &, int, bool, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t compose_tree(const TreeArgs &, int, bool, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t seam_advance(const SeamArgs &, int, bool, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t compose_seq_compact(const ComposeArgs &, int, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t pair_compact(const float *, bf16 *, float *, int, int64_t, hipStream_t) { return hipErrorInvalidValue; }
hipError_t rerotate(const RerotateArgs &, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t conv_warmup(const ConvArgs &, bool, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t static_workspace(void **ptr) {
    *ptr = nullptr;
    return hipErrorInvalidValue;
}
}  // namespace hy
