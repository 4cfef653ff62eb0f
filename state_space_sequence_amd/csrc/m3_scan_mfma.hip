// Matrix-core (bf16 MFMA) chunked-scan prefill: placeholder until the kernel lands.
#include "m3_internal.h"

namespace m3i {
bool mfma_kernel_available() { return false; }
int mfma_auto_segments(int64_t, int64_t) { return 1; }
size_t mfma_workspace_bytes(int64_t, int, int64_t, int64_t) { return 0; }
void mfma_workspace_carve(void *, int64_t, int, int64_t, int64_t, SplitPlan *) {}
hipError_t launch_scan_mfma(const ScanArgs &, const SplitPlan &, hipStream_t) { return hipErrorNotSupported; }
}  // namespace m3i
