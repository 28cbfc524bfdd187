// Launch stubs for the host-validation fuzz (tests/c/abi_fuzz.cpp): they
// stand in for the kernel launchers so that api.hip links without device
// kernels; a call that passes every host check reaches one of these and gets
// hipErrorNotSupported back.  Nothing here touches the (fake) pointers.
#include "pa_kernels.h"

namespace pa {
hipError_t launch_kv_append(const AppendArgs&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_copy_blocks(const CopyArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_row_partials(const RowAttnArgs&, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_row_merge(const RowAttnArgs&, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_prefill_mfma(const PrefillArgs&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_prefill_split_merge(const PrefillArgs&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_cascade_merge(const CascadeMergeArgs&, int, hipStream_t) { return hipErrorNotSupported; }
int prefill_rows_per_tile(int g) { return 128 / g; }
}  // namespace pa
