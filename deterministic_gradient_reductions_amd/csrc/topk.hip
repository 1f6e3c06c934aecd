// det_topk_canonicalize: canonical order of a compact indexer top-k.
//
// Megatron-LM PR #7441 (DSv4 deterministic mode), source 1: the compact
// indexer top-k returns a row's selected ids in a run-dependent slot order,
// and its compact softmax is accumulated in that order. The fix sorts each
// row's ids with the padding last, permutes the logits the same way,
// recomputes the softmax in that order, and gives all-padding rows zero
// probabilities instead of NaN.
//
// One wave per row. Each of the K slots becomes a 64-bit key (id << 32 | slot
// for a valid id, 2^31 << 32 | slot for padding, all ones for the positions
// that round K up to a power of two): the keys are distinct, so the sorted
// order is unique and equals the stable order with padding last. The keys are
// sorted with a bitonic network held in registers: element i = lane * EPL + r
// (EPL elements per lane), partners within a lane are swapped in registers,
// partners across lanes are exchanged with one shuffle per 32-bit half. The
// sorted keys give each output position its source slot, from which the id
// and the logit are gathered. The softmax: the exact maximum of the valid
// logits (a wave reduction), e = exp32(logit - max) (the gate's fixed
// sequence), the left-to-right sum of the e's in the sorted order (readlane
// feeds one dependent add per slot), and one correctly rounded division per
// slot. Padding slots get +0.0.
#include "common.hpp"
#include "detmath.hpp"

namespace detgrad {
namespace {

constexpr int kMaxK = 1024;

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
  const uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
  const uint32_t a = static_cast<uint32_t>(__shfl_xor(static_cast<int>(lo), m));
  const uint32_t b = static_cast<uint32_t>(__shfl_xor(static_cast<int>(hi), m));
  return static_cast<uint64_t>(b) << 32 | a;
}

template <int EPL>
__global__ __launch_bounds__(256) void topk_canon_kernel(const int32_t* __restrict__ ids, const float* __restrict__ logits,
                                                         int64_t Q, int K, int64_t ld, int32_t* __restrict__ ids_out,
                                                         float* __restrict__ logits_out, float* __restrict__ probs,
                                                         int64_t ld_out) {
  constexpr int N = 64 * EPL;  // padded row length, a power of two
  const int lane = threadIdx.x & 63;
  const int64_t q = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (q >= Q) return;  // wave-uniform
  const int32_t* const ir = ids + q * ld;
  const float* const lr = logits + q * ld;
  uint64_t key[EPL];
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    const int i = lane * EPL + r;
    if (i < K) {
      const int32_t id = ir[i];
      const uint32_t hi = id >= 0 ? static_cast<uint32_t>(id) : 0x80000000u;
      key[r] = static_cast<uint64_t>(hi) << 32 | static_cast<uint32_t>(i);
    } else {
      key[r] = ~0ull;
    }
  }
  // bitonic sort, ascending
#pragma unroll
  for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
    for (int d = k >> 1; d > 0; d >>= 1) {
      if (d < EPL) {
#pragma unroll
        for (int r = 0; r < EPL; ++r) {
          const int rp = r ^ d;
          if (rp > r) {
            const int i = lane * EPL + r;
            const bool up = (i & k) == 0;
            const uint64_t a = key[r], b = key[rp];
            const bool swap = up ? (a > b) : (a < b);
            key[r] = swap ? b : a;
            key[rp] = swap ? a : b;
          }
        }
      } else {
        const int m = d / EPL;  // partner lane = lane ^ m
#pragma unroll
        for (int r = 0; r < EPL; ++r) {
          const int i = lane * EPL + r;
          const uint64_t o = shfl_xor64(key[r], m);
          const bool up = (i & k) == 0;
          const bool lower = (i & d) == 0;  // this element is the lower index of the pair
          // ascending pair: the lower index keeps the smaller key
          const bool keep_min = (up == lower);
          const uint64_t mn = key[r] < o ? key[r] : o, mx = key[r] < o ? o : key[r];
          key[r] = keep_min ? mn : mx;
        }
      }
    }
  }
  // gather ids and logits by source slot; the valid slots come first
  int32_t idv[EPL];
  float lg[EPL];
  int nv_lane = 0;
  float mx = -__builtin_inff();
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    const int i = lane * EPL + r;
    const uint32_t slot = static_cast<uint32_t>(key[r]);
    const bool in = i < K;
    idv[r] = in ? ir[slot] : 0;
    lg[r] = in ? lr[slot] : 0.0f;
    const bool valid = in && (key[r] >> 32) < 0x80000000ull;
    nv_lane += valid ? 1 : 0;
    if (valid) mx = mx > lg[r] ? mx : lg[r];
  }
  // exact maximum over the wave
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) {
    const float o = __shfl_xor(mx, m);
    mx = mx > o ? mx : o;
  }
  int nv = nv_lane;
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) nv += __shfl_xor(nv, m);
  float e[EPL];
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    const int i = lane * EPL + r;
    e[r] = i < nv ? dm::exp32(lg[r] - mx) : 0.0f;
  }
  // left-to-right sum in the sorted order: element i = lane * EPL + r
  float S = -0.0f;
  for (int l = 0; l < 64; ++l) {
    if (l * EPL >= nv) break;  // uniform
#pragma unroll
    for (int r = 0; r < EPL; ++r)
      if (l * EPL + r < nv) S = S + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e[r]), l));
  }
  int32_t* const io = ids_out + q * ld_out;
  float* const lo = logits_out + q * ld_out;
  float* const po = probs + q * ld_out;
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    const int i = lane * EPL + r;
    if (i < K) {
      io[i] = idv[r];
      lo[i] = lg[r];
      po[i] = i < nv ? e[r] / S : 0.0f;
    }
  }
}

}  // namespace
}  // namespace detgrad

using namespace detgrad;

extern "C" int det_topk_canonicalize(const int32_t* ids, const float* logits, int64_t Q, int64_t K, int64_t ld,
                                     int32_t* ids_out, float* logits_out, float* probs, int64_t ld_out,
                                     void* stream) {
  if (Q < 0 || K < 0) return set_error(DET_ERR_INVALID_ARG, "topk: Q and K must be >= 0");
  if (K > kMaxK) return set_error(DET_ERR_UNSUPPORTED, "topk: K must be <= %d, got %lld", kMaxK, static_cast<long long>(K));
  if (Q == 0 || K == 0) return ok();
  if (!ids || !logits || !ids_out || !logits_out || !probs) return set_error(DET_ERR_INVALID_ARG, "topk: NULL pointer");
  if (ld < K || ld_out < K) return set_error(DET_ERR_INVALID_ARG, "topk: ld and ld_out must be >= K");
  if (ceil_div(Q, 4) > 0x7FFFFFFF) return set_error(DET_ERR_UNSUPPORTED, "topk: Q too large");
  const Range ins[] = {range2d(ids, Q, K, ld, 4), range2d(logits, Q, K, ld, 4)};
  const Range outs[] = {range2d(ids_out, Q, K, ld_out, 4), range2d(logits_out, Q, K, ld_out, 4),
                        range2d(probs, Q, K, ld_out, 4)};
  for (int a = 0; a < 3; ++a) {
    for (const Range& r : ins)
      if (overlaps(outs[a], r)) return set_error(DET_ERR_OVERLAP, "topk: an output overlaps an input");
    for (int b = a + 1; b < 3; ++b)
      if (overlaps(outs[a], outs[b])) return set_error(DET_ERR_OVERLAP, "topk: outputs overlap each other");
  }
  const hipStream_t st = as_stream(stream);
  const dim3 grid(static_cast<uint32_t>(ceil_div(Q, 4)));
  const int epl = K <= 64 ? 1 : (K <= 128 ? 2 : (K <= 256 ? 4 : (K <= 512 ? 8 : 16)));
#define DET_TOPK_LAUNCH(E)                                                                                       \
  if (epl == E)                                                                                                  \
    hipLaunchKernelGGL(topk_canon_kernel<E>, grid, dim3(256), 0, st, ids, logits, Q, static_cast<int>(K), ld,   \
                       ids_out, logits_out, probs, ld_out);
  DET_TOPK_LAUNCH(1) DET_TOPK_LAUNCH(2) DET_TOPK_LAUNCH(4) DET_TOPK_LAUNCH(8) DET_TOPK_LAUNCH(16)
#undef DET_TOPK_LAUNCH
  return check_launch("det_topk_canonicalize");
}
