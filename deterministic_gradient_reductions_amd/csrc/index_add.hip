// det_index_add (placeholder until the kernels land).
#include "common.hpp"
using namespace detgrad;
extern "C" int det_index_add_workspace_size(int64_t, int64_t, int64_t, const det_index_add_cfg*, int atomic,
                                            size_t* bytes) {
  if (int s = check_atomic_flag(atomic)) return s;
  if (bytes) *bytes = 0;
  return set_error(DET_ERR_UNSUPPORTED, "index_add: not implemented yet");
}
extern "C" int det_index_add(float*, int64_t, int64_t, int64_t, const int32_t*, int64_t, const void*, int64_t, int,
                             const det_index_add_cfg*, void*, size_t, int atomic, void*) {
  if (int s = check_atomic_flag(atomic)) return s;
  return set_error(DET_ERR_UNSUPPORTED, "index_add: not implemented yet");
}
extern "C" int det_index_add_bad_ids(const void*, size_t, int64_t*, void*) {
  return set_error(DET_ERR_UNSUPPORTED, "index_add: not implemented yet");
}
