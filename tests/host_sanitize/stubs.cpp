// Kernel launchers replaced by stubs for the host-only sanitizer build: the
// driver exercises only paths that return before any launch, so none of
// these runs; they exist to resolve the library's references.
#include "../../sparse_kv_attention_sfi_amd/csrc/sfi_internal.hpp"

namespace sfi {
hipError_t launch_slow_partial(const SlowArgs&, int, int, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_slow_combine(const CombineArgs&, int, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_select(const SelectArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_score(const ScoreArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_fast_partial(const FastArgs&, int, int, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_fast_merge(const FastArgs&, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_support(const SupportArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_pack(const PackArgs&, int, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_append(const AppendArgs&, int, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_fill_zero(void*, size_t, hipStream_t) { return hipErrorInvalidValue; }
int fast_chunk_rows() { return 128; }
int32_t noalloc_scratch(hipStream_t, char**) { return SFI_ERR_HIP; }
}  // namespace sfi
