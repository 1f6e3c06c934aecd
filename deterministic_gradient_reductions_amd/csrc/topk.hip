// det_topk_canonicalize: canonical order of a compact indexer top-k.
//
// Megatron-LM PR #7441 (DSv4 deterministic mode), source 1 and its fix: the
// slot order of a row's selected ids, and so the order of its softmax sum,
// changed between runs. Here every row is put in one canonical order (ids
// ascending, padding after them), its logits follow the same permutation, the
// softmax is summed again in that order, and a row without any valid id gets
// probabilities of zero.
//
// One wave per row. Each of the K slots becomes a 64-bit key (id << 32 | slot
// for a valid id, 2^31 << 32 | slot for padding, all ones for the positions
// that round K up to a power of two): the keys are distinct, so the sorted
// order is unique and equals the stable order with padding last. When every
// id of the row is below 2^21 - 1 the same order is carried by a 32-bit key
// (id << 10 | slot, padding as id 2^21 - 1), which halves the cross-lane
// traffic. The keys are sorted with a bitonic network held in registers:
// element i = r * 64 + lane (EPL elements per lane, so loads and stores are
// coalesced); partners at a distance below 64 are exchanged across lanes (DPP
// quad permutations for distances 1 and 2, ds_bpermute beyond, all exchanges
// of a step issued together), partners further apart are swapped between
// registers. The
// sorted keys give each output position its source slot, from which the id
// and the logit are gathered. The softmax: the exact maximum of the valid
// logits (a wave reduction), e = exp32(logit - max) (the gate's fixed
// sequence), the left-to-right sum of the e's in the sorted order, and one
// correctly rounded division per slot. For the sums the four waves of a
// workgroup leave their e's in LDS and lanes 0..3 of the first wave add one
// row each, so four dependent-add chains share one instruction stream.
// Padding slots get +0.0.
#include "common.hpp"
#include "detmath.hpp"

namespace detgrad {
namespace {

constexpr int kMaxK = 1024;

// The value of lane ^ m. m = 1 and m = 2 stay inside a group of four lanes
// and move by a DPP quad permutation (a VALU operand modifier, no LDS-pipe
// round trip); larger distances use ds_bpermute. Every lane of the wave is
// active here.
__device__ __forceinline__ uint32_t shfl_xor_k(uint32_t v, int m) {
  if (m == 1) return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, true));
  if (m == 2) return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, true));
  return static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), m));
}
__device__ __forceinline__ uint64_t shfl_xor_k(uint64_t v, int m) {
  const uint32_t lo = shfl_xor_k(static_cast<uint32_t>(v), m), hi = shfl_xor_k(static_cast<uint32_t>(v >> 32), m);
  return static_cast<uint64_t>(hi) << 32 | lo;
}

// Ascending bitonic sort of the wave's 64 * EPL keys, element i = r * 64 +
// lane: partners closer than 64 are in other lanes (shuffles), partners
// further apart in other registers.
template <int EPL, typename T>
__device__ __forceinline__ void bitonic(T (&key)[EPL], int lane) {
  constexpr int N = 64 * EPL;
#pragma unroll
  for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
    for (int d = k >> 1; d > 0; d >>= 1) {
      if (d >= 64) {
        const int dr = d / 64;
#pragma unroll
        for (int r = 0; r < EPL; ++r) {
          const int rp = r ^ dr;
          if (rp > r) {
            const int i = r * 64 + lane;
            const bool up = (i & k) == 0;
            const T a = key[r], b = key[rp];
            const bool swap = up ? (a > b) : (a < b);
            key[r] = swap ? b : a;
            key[rp] = swap ? a : b;
          }
        }
      } else {
        // all exchanges of the step first, so that they are in flight together
        T o[EPL];
#pragma unroll
        for (int r = 0; r < EPL; ++r) o[r] = shfl_xor_k(key[r], d);
#pragma unroll
        for (int r = 0; r < EPL; ++r) {
          const int i = r * 64 + lane;
          const bool up = (i & k) == 0;
          const bool lower = (i & d) == 0;  // this element is the lower index of the pair
          // an ascending pair keeps the smaller key at its lower index
          const bool keep_min = (up == lower);
          const T mn = key[r] < o[r] ? key[r] : o[r], mx = key[r] < o[r] ? o[r] : key[r];
          key[r] = keep_min ? mn : mx;
        }
      }
    }
  }
}

// True when every valid id of the row is below 2^21 - 1 (so id << 10 | slot
// is a 32-bit key).
template <int EPL>
__device__ __forceinline__ bool wave_ids_narrow(const uint64_t (&key)[EPL]) {
  bool wide = false;
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    const uint32_t hi = static_cast<uint32_t>(key[r] >> 32);
    wide = wide || (key[r] != ~0ull && hi != 0x80000000u && hi >= 0x1FFFFFu);
  }
  return __ballot(wide) == 0;
}

template <int EPL>
__global__ __launch_bounds__(256) void topk_canon_kernel(const int32_t* __restrict__ ids, const float* __restrict__ logits,
                                                         int64_t Q, int K, int64_t ld, int32_t* __restrict__ ids_out,
                                                         float* __restrict__ logits_out, float* __restrict__ probs,
                                                         int64_t ld_out) {
  constexpr int N = 64 * EPL;  // padded row length, a power of two
  __shared__ float es[4][N];   // each wave's e values, in sorted order, for the sums
  __shared__ float sums[4];
  __shared__ int nvs[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t q = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  const bool row = q < Q;  // wave-uniform; every wave reaches the barrier
  const int32_t* const ir = ids + (row ? q : 0) * ld;
  const float* const lr = logits + (row ? q : 0) * ld;
  // element i = r * 64 + lane: partners at distance d < 64 sit in another
  // lane (one shuffle per 32-bit half), at d >= 64 in another register
  uint64_t key[EPL];
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    const int i = r * 64 + lane;
    if (row && i < K) {
      const int32_t id = ir[i];
      const uint32_t hi = id >= 0 ? static_cast<uint32_t>(id) : 0x80000000u;
      key[r] = static_cast<uint64_t>(hi) << 32 | static_cast<uint32_t>(i);
    } else {
      key[r] = ~0ull;
    }
  }
  // keys of 32 bits (id << 10 | slot) when every id of the row is below
  // 2^21 - 1 (K <= 1024 slots), else of 64 bits: the same order, half the
  // cross-lane traffic
  const bool narrow = wave_ids_narrow<EPL>(key);
  if (narrow) {
    uint32_t k32[EPL];
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
      const uint32_t hi = static_cast<uint32_t>(key[r] >> 32), lo = static_cast<uint32_t>(key[r]);
      k32[r] = key[r] == ~0ull ? ~0u : ((hi == 0x80000000u ? 0x1FFFFFu : hi) << 10 | lo);
    }
    bitonic<EPL>(k32, lane);
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
      const uint32_t hi = k32[r] >> 10, lo = k32[r] & 0x3FFu;
      key[r] = k32[r] == ~0u ? ~0ull
                             : (static_cast<uint64_t>(hi == 0x1FFFFFu ? 0x80000000u : hi) << 32 | lo);
    }
  } else {
    bitonic<EPL>(key, lane);
  }
  // gather ids and logits by source slot; the valid slots come first
  int32_t idv[EPL];
  float lg[EPL];
  int nv_lane = 0;
  float mx = -__builtin_inff();
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    const int i = r * 64 + lane;
    const uint32_t slot = static_cast<uint32_t>(key[r]);
    const bool in = row && i < K;
    idv[r] = in ? ir[slot] : 0;
    lg[r] = in ? lr[slot] : 0.0f;
    const bool valid = in && (key[r] >> 32) < 0x80000000ull;
    nv_lane += valid ? 1 : 0;
    if (valid) mx = mx > lg[r] ? mx : lg[r];
  }
  // exact maximum and valid count over the wave
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
    const int i = r * 64 + lane;
    e[r] = i < nv ? dm::exp32(lg[r] - mx) : 0.0f;
    es[wave][i] = e[r];
  }
  if (lane == 0) nvs[wave] = row ? nv : 0;
  __syncthreads();
  // the left-to-right sums: lane w of wave 0 adds row w's values in order
  // (four independent dependent-add chains in one instruction stream)
  if (wave == 0 && lane < 4) {
    const int nvw = nvs[lane];  // valid values of row `lane` (0 past Q): the prefix of its es row
    const float* const ew = es[lane];
    float S = -0.0f;
    int i = 0;
    for (; i + 4 <= nvw; i += 4) {
      const float4 v = *reinterpret_cast<const float4*>(ew + i);
      S = S + v.x; S = S + v.y; S = S + v.z; S = S + v.w;
    }
    for (; i < nvw; ++i) S = S + ew[i];
    sums[lane] = S;
  }
  __syncthreads();
  if (!row) return;
  const float S = sums[wave];
  int32_t* const io = ids_out + q * ld_out;
  float* const lo = logits_out + q * ld_out;
  float* const po = probs + q * ld_out;
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    const int i = r * 64 + lane;
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
