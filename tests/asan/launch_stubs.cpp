// Stand-ins for the decode kernels' launchers in the host-only
// AddressSanitizer build of the C ABI layer.  The ABI tests run there check
// argument validation on a machine without a GPU, so no call ever reaches a
// launch; every stub reports failure.  split_columns is host arithmetic the
// validation uses, so it keeps the decode source's definition.
#include "decode.h"
#include "prefill.h"

namespace pa {

hipError_t launch_decode(const DecodeArgs&, int, int, int, dim3, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_reduce(const ReduceArgs&, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_multi(const DecodeArgs&, int, int, int, dim3, bool, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_multi_balanced(const DecodeArgs&, int, int, int, int, bool,
                                 hipStream_t) {
  return hipErrorNotSupported;
}
int multi_balanced_grid(int, int, int, bool) { return 0; }
int split_columns(int head_size, int group) {
  return (head_size == 128 && group <= 4) ? 4 : 8;
}
hipError_t launch_multi_reduce(const ReduceArgs&, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_prefix_marks(const DecodeArgs&, int, int*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_prefix(const DecodeArgs&, int, int, int, dim3, bool, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_balanced(const DecodeArgs&, int, int, int, int, hipStream_t, int) {
  return hipErrorNotSupported;
}
int balanced_grid(int, int, int, int) { return 0; }
hipError_t launch_prefill(const PrefillArgs&, int, int, int, dim3, bool, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_prefill_fold(const PrefillArgs&, int, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace pa
