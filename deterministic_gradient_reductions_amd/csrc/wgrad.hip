// det_grouped_wgrad_acc (placeholder until the kernels land).
#include "common.hpp"
using namespace detgrad;
extern "C" int det_grouped_wgrad_acc_workspace_size(int64_t, int32_t, int64_t, int64_t, const det_wgrad_cfg*,
                                                    int atomic, size_t* bytes) {
  if (int s = check_atomic_flag(atomic)) return s;
  if (bytes) *bytes = 0;
  return set_error(DET_ERR_UNSUPPORTED, "wgrad: not implemented yet");
}
extern "C" int det_grouped_wgrad_acc(float*, int64_t, int64_t, const void*, int64_t, const void*, int64_t,
                                     const int32_t*, int32_t, int64_t, int64_t, int64_t, const det_wgrad_cfg*, void*,
                                     size_t, int atomic, void*) {
  if (int s = check_atomic_flag(atomic)) return s;
  return set_error(DET_ERR_UNSUPPORTED, "wgrad: not implemented yet");
}
