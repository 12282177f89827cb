// gr_fast.hip -- MFMA fast path (placeholder until implemented).
#include "gr_device.h"
#include "gr_internal.h"

namespace grk {
bool fast_path_ok(const ReadArgs &) { return false; }
size_t fast_workspace_bytes(int64_t, int, int, int) { return 0; }
hipError_t launch_read_fast(const ReadArgs &, hipStream_t) { return hipErrorNotSupported; }
}  // namespace grk
