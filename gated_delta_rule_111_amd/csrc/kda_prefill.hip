// placeholder translation unit (replaced by the chunked prefill kernel)
#include "kda_common.h"
#include "kda_internal.h"
namespace kda {
size_t prefill_workspace_bytes(int, int, int, int, int64_t) { return 0; }
hipError_t launch_prefill(const PrefillArgs&) { return hipErrorNotSupported; }
}  // namespace kda
