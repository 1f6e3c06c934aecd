// Diagnostic entry point: evaluates the device detmath functions elementwise,
// so tests can compare the GPU's bits with the CPU oracle's.
#include "common.hpp"
#include "detmath.hpp"

namespace detgrad {
namespace {
__global__ void detmath_eval_kernel(const float* __restrict__ x, float* __restrict__ y, int64_t n, int fn) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float v = x[i];
  float r;
  switch (fn) {
    case 0: r = dm::exp32(v); break;
    case 1: r = dm::log1p32(v); break;
    case 2: r = dm::softplus_e(v, dm::exp32(dm::neg_abs(v))); break;
    default: r = dm::sigmoid_e(v, dm::exp32(dm::neg_abs(v))); break;
  }
  y[i] = r;
}
}  // namespace
}  // namespace detgrad

using namespace detgrad;

extern "C" int det_detmath_eval(const float* x, float* y, int64_t n, int fn, void* stream) {
  if (n < 0 || fn < 0 || fn > 3) return set_error(DET_ERR_INVALID_ARG, "detmath_eval: bad n or fn");
  if (n == 0) return ok();
  if (!x || !y) return set_error(DET_ERR_INVALID_ARG, "detmath_eval: NULL pointer");
  if (overlaps(range1d(x, n * 4), range1d(y, n * 4)))
    return set_error(DET_ERR_OVERLAP, "detmath_eval: y overlaps x");
  const int64_t grid = ceil_div(n, 256);
  if (grid > 0x7FFFFFFF) return set_error(DET_ERR_UNSUPPORTED, "detmath_eval: n too large");
  hipLaunchKernelGGL(detmath_eval_kernel, dim3(grid), dim3(256), 0, as_stream(stream), x, y, n, fn);
  return check_launch("det_detmath_eval");
}
