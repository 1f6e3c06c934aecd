// Diagnostic entry points: the device detmath functions evaluated elementwise,
// and chains of the matrix-core instruction of the weight gradient on plain
// row-major operands, so tests can compare the GPU's bits with the CPU
// oracle's.
#include "common.hpp"
#include "detmath.hpp"

namespace detgrad {
namespace {
typedef __bf16 dbf16x8_t __attribute__((ext_vector_type(8)));
typedef float df32x16_t __attribute__((ext_vector_type(16)));

// One wave per chain. Lane l = 32 kg + r holds A[r][16 b + 8 kg + e] and
// B[16 b + 8 kg + e][r] (e = 0..7) of block b, and accumulator c holds
// D[8 (c / 4) + 4 kg + c % 4][r]: the operand layout of the weight-gradient
// kernel, where k = 8 kg + e is the token row inside a 16-row block.
__global__ __launch_bounds__(256) void mfma_eval_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                        const float* __restrict__ C, float* __restrict__ D, int64_t n,
                                                        int kblocks) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (q >= n) return;
  const int lane = threadIdx.x & 63;
  const int r = lane & 31, kg = lane >> 5;
  const int K = 16 * kblocks;
  const uint16_t* a = A + q * 32 * K;
  const uint16_t* b = B + q * K * 32;
  df32x16_t acc;
#pragma unroll
  for (int c = 0; c < 16; ++c) acc[c] = C[q * 1024 + (8 * (c / 4) + 4 * kg + c % 4) * 32 + r];
  for (int blk = 0; blk < kblocks; ++blk) {
    dbf16x8_t fa, fb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = 16 * blk + 8 * kg + e;
      fa[e] = __builtin_bit_cast(__bf16, a[r * K + k]);
      fb[e] = __builtin_bit_cast(__bf16, b[k * 32 + r]);
    }
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc, 0, 0, 0);
  }
#pragma unroll
  for (int c = 0; c < 16; ++c) D[q * 1024 + (8 * (c / 4) + 4 * kg + c % 4) * 32 + r] = acc[c];
}

// The weight gradient's accumulator pattern alone: every wave holds four A and
// four B fragments (lane layout as above) read once from `ops`, then runs
// `iters` rounds of the 4 x 4 MFMAs into sixteen accumulators, with no memory
// traffic in the loop. Lane l of wave w takes its 64 operand values from set
// (global wave index mod kRateSets). Each lane writes the sum of its
// accumulators once, so no MFMA can be dropped. A measurement aid: how fast
// the matrix cores run on the caller's operand values.
constexpr int kRateSets = 64;
constexpr int64_t kRateOps = static_cast<int64_t>(kRateSets) * 64 * 64;  // bf16 values the kernel reads

__global__ __launch_bounds__(256) void mfma_rate_kernel(const uint16_t* __restrict__ ops, float* __restrict__ out,
                                                        int iters) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const uint16_t* src = ops + ((gw % kRateSets) * 64 + lane) * 64;
  dbf16x8_t a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[i][e] = __builtin_bit_cast(__bf16, src[8 * i + e]);
      b[i][e] = __builtin_bit_cast(__bf16, src[32 + 8 * i + e]);
    }
  df32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int c = 0; c < 16; ++c) acc[i][j][c] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int c = 0; c < 16; ++c) s = s + acc[i][j][c];
  out[gw * 64 + lane] = s;
}

__global__ void detmath_eval_kernel(const float* __restrict__ x, float* __restrict__ y, int64_t n, int fn) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float v = x[i];
  float r, sp, sg;
  switch (fn) {
    case 0: r = dm::exp32(v); break;
    case 1: r = dm::log1p32(v); break;
    case 2: dm::softplus_sigmoid(v, sp, sg); r = sp; break;   // the gate's own evaluation
    default: dm::softplus_sigmoid(v, sp, sg); r = sg; break;
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

extern "C" int det_mfma_eval(const uint16_t* A, const uint16_t* B, const float* C, float* D, int64_t n, int kblocks,
                             void* stream) {
  if (n < 0 || kblocks < 1 || kblocks > 4096) return set_error(DET_ERR_INVALID_ARG, "mfma_eval: bad n or kblocks");
  if (n == 0) return ok();
  if (!A || !B || !C || !D) return set_error(DET_ERR_INVALID_ARG, "mfma_eval: NULL pointer");
  const size_t ab = static_cast<size_t>(n) * 32 * 16 * kblocks * 2;
  const Range d = range1d(D, static_cast<size_t>(n) * 4096);
  if (overlaps(d, range1d(A, ab)) || overlaps(d, range1d(B, ab)) || overlaps(d, range1d(C, static_cast<size_t>(n) * 4096)))
    return set_error(DET_ERR_OVERLAP, "mfma_eval: D overlaps an input");
  const int64_t grid = ceil_div(n, 4);
  if (grid > 0x7FFFFFFF) return set_error(DET_ERR_UNSUPPORTED, "mfma_eval: n too large");
  hipLaunchKernelGGL(mfma_eval_kernel, dim3(grid), dim3(256), 0, as_stream(stream), A, B, C, D, n, kblocks);
  return check_launch("det_mfma_eval");
}

extern "C" int det_mfma_rate(const uint16_t* ops, int64_t n_ops, float* out, int64_t n_out, int blocks, int iters,
                             void* stream) {
  if (blocks < 1 || blocks > (1 << 20) || iters < 0 || iters > (1 << 24))
    return set_error(DET_ERR_INVALID_ARG, "mfma_rate: blocks must be in [1, 2^20] and iters in [0, 2^24]");
  if (!ops || !out) return set_error(DET_ERR_INVALID_ARG, "mfma_rate: NULL pointer");
  if (n_ops < kRateOps)
    return set_error(DET_ERR_INVALID_ARG, "mfma_rate: ops must hold %lld bf16 values", static_cast<long long>(kRateOps));
  if (n_out < static_cast<int64_t>(blocks) * 256)
    return set_error(DET_ERR_INVALID_ARG, "mfma_rate: out must hold 256 floats per block");
  if (overlaps(range1d(out, static_cast<size_t>(n_out) * 4), range1d(ops, static_cast<size_t>(n_ops) * 2)))
    return set_error(DET_ERR_OVERLAP, "mfma_rate: out overlaps ops");
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(blocks), dim3(256), 0, as_stream(stream), ops, out, iters);
  return check_launch("det_mfma_rate");
}
