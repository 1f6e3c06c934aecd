// Library-wide entry points: version, error text, workspace header init.
#include "common.hpp"

namespace detgrad {

namespace {
thread_local char g_err[512] = "";
}

int set_error(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return DET_OK;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(DET_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

int check_atomic_flag(int atomic) {
  if (atomic != 0 && atomic != 1)
    return set_error(DET_ERR_INVALID_ARG, "atomic must be 0 (deterministic) or 1 (atomic arm), got %d", atomic);
  return DET_OK;
}

int check_workspace(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return DET_OK;
  if (!ws) return set_error(DET_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
  if (!aligned(ws, 256)) return set_error(DET_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < need) return set_error(DET_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  return DET_OK;
}

__global__ void ws_header_fill(uint32_t* hdr) { hdr[threadIdx.x] = 0u; }

}  // namespace detgrad

using namespace detgrad;

extern "C" int det_abi_version(void) { return DET_ABI_VERSION; }

extern "C" const char* det_last_error(void) { return g_err; }

extern "C" int det_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws) return set_error(DET_ERR_WORKSPACE, "det_workspace_init: NULL workspace");
  if (!aligned(ws, 256)) return set_error(DET_ERR_WORKSPACE, "det_workspace_init: workspace must be 256-byte aligned");
  if (ws_bytes < DET_WS_HEADER_BYTES)
    return set_error(DET_ERR_WORKSPACE, "det_workspace_init: need at least %d bytes", DET_WS_HEADER_BYTES);
  hipLaunchKernelGGL(ws_header_fill, dim3(1), dim3(DET_WS_HEADER_BYTES / 4), 0, as_stream(stream),
                     static_cast<uint32_t*>(ws));
  return check_launch("det_workspace_init");
}
