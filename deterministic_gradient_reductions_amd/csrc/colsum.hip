// det_colsum: ordered A_log / dt_bias column sums of the Gated-DeltaNet gate
// backward (Megatron-LM PR #8244).
//
// One workgroup of 256 threads owns a tile of block_t rows x block_h heads.
// Each thread takes block_t*block_h/256 consecutive rows of one head, computes
// the two gradient terms per element (detmath, so the CPU oracle can match
// every bit) and reduces its rows with the adjacent pairwise tree in
// registers; the remaining tree levels run over LDS. The resulting tile slot
// (one per head and gradient) goes to the workspace; the last workgroup to
// finish (an integer ticket in the workspace header) folds the slots of every
// head in tile order and adds the totals into dA_log / ddt_bias. One launch,
// no float atomics, and the ticket resets itself for the next call.
//
// The atomic arm computes the same tile slots and adds them into the outputs
// with hardware float atomics, in whatever order the tiles finish.
//
// The per-element work is about 80 VALU operations (exp, log1p, two divisions),
// so at large T the kernel is bound by vector ALU throughput, not HBM.
#include "common.hpp"
#include "detmath.hpp"

namespace detgrad {
namespace {

constexpr int kWG = 256;

struct ColsumArgs {
  const uint16_t* a;
  int64_t a_st, a_sh;
  const uint16_t* dg;
  int64_t dg_st, dg_sh;
  const float* A_log;
  const float* dt_bias;
  int64_t T, H;
  float* dA_log;
  float* ddt_bias;
  uint32_t* ticket;  // workspace header word 0
  float* slot1;      // [S][H]
  float* slot2;      // [S][H]
};

// Adjacent pairwise tree over v[0..n-1] in place (n a power of two <= 32).
template <int N>
__device__ __forceinline__ float tree_regs(float (&v)[N]) {
#pragma unroll
  for (int w = 1; w < N; w *= 2) {
#pragma unroll
    for (int i = 0; i < N; i += 2 * w) v[i] = v[i] + v[i + w];
  }
  return v[0];
}

template <int R, int BH, bool ATOMIC>
__global__ __launch_bounds__(kWG) void colsum_kernel(ColsumArgs p) {
  constexpr int kBT = R * kWG / BH;   // rows per tile
  constexpr int kNB = kWG / BH;       // row blocks per tile (threads per head)
  __shared__ float red1[kWG];
  __shared__ float red2[kWG];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int hl = tid % BH;
  const int rb = tid / BH;
  const int64_t h = static_cast<int64_t>(blockIdx.y) * BH + hl;
  const int64_t tile = blockIdx.x;
  const int64_t r0 = tile * kBT + static_cast<int64_t>(rb) * R;

  float v1[R], v2[R];
  if (h < p.H) {
    const float nA = -dm::exp32(p.A_log[h]);
    const float bias = p.dt_bias[h];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int64_t t = r0 + i;
      if (t < p.T) {
        const float x = bf16_to_f32(p.a[t * p.a_st + h * p.a_sh]) + bias;
        const float d = bf16_to_f32(p.dg[t * p.dg_st + h * p.dg_sh]);
        const float e = dm::exp32(dm::neg_abs(x));
        const float sp = dm::softplus_e(x, e);
        const float sg = dm::sigmoid_e(x, e);
        v1[i] = d * (nA * sp);
        v2[i] = d * (nA * sg);
      } else {
        v1[i] = -0.0f;
        v2[i] = -0.0f;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      v1[i] = -0.0f;
      v2[i] = -0.0f;
    }
  }
  red1[rb * BH + hl] = tree_regs<R>(v1);
  red2[rb * BH + hl] = tree_regs<R>(v2);
  __syncthreads();

  if (tid < BH) {
    float w1[kNB], w2[kNB];
#pragma unroll
    for (int i = 0; i < kNB; ++i) {
      w1[i] = red1[i * BH + tid];
      w2[i] = red2[i * BH + tid];
    }
    const float s1 = tree_regs<kNB>(w1);
    const float s2 = tree_regs<kNB>(w2);
    if (h < p.H) {
      if (ATOMIC) {
        unsafeAtomicAdd(p.dA_log + h, s1);
        unsafeAtomicAdd(p.ddt_bias + h, s2);
      } else {
        p.slot1[tile * p.H + h] = s1;
        p.slot2[tile * p.H + h] = s2;
      }
    }
  }
  if (ATOMIC) return;

  // Publish the slots, then take a ticket; the last workgroup folds.
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t n_wg = gridDim.x * gridDim.y;
    const uint32_t t = atomicAdd(p.ticket, 1u);
    s_last = (t == n_wg - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const int64_t S = gridDim.x;
  constexpr int kBatch = 16;  // slot loads in flight before the dependent adds
  for (int64_t hh = tid; hh < p.H; hh += kWG) {
    float tot1 = -0.0f, tot2 = -0.0f;
    for (int64_t i0 = 0; i0 < S; i0 += kBatch) {
      float b1[kBatch], b2[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int64_t i = i0 + j < S ? i0 + j : S - 1;
        b1[j] = p.slot1[i * p.H + hh];
        b2[j] = p.slot2[i * p.H + hh];
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (i0 + j < S) {
          tot1 = tot1 + b1[j];
          tot2 = tot2 + b2[j];
        }
      }
    }
    p.dA_log[hh] = p.dA_log[hh] + tot1;
    p.ddt_bias[hh] = p.ddt_bias[hh] + tot2;
  }
  if (tid == 0) __hip_atomic_store(p.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

bool valid_cfg(const det_colsum_cfg& c) {
  return (c.block_t == 64 || c.block_t == 128 || c.block_t == 256) &&
         (c.block_h == 8 || c.block_h == 16 || c.block_h == 32);
}

int resolve_cfg(int64_t T, int64_t H, const det_colsum_cfg* cfg, det_colsum_cfg* out);

size_t ws_bytes_for(int64_t T, int64_t H, const det_colsum_cfg& c) {
  const int64_t S = ceil_div(T, c.block_t);
  return DET_WS_HEADER_BYTES + align_up(static_cast<size_t>(S * H) * 4, 256) * 2;
}

template <int BT, int BH>
void launch_one(const ColsumArgs& p, int atomic, dim3 grid, hipStream_t st) {
  constexpr int R = BT * BH / kWG;
  if (atomic)
    hipLaunchKernelGGL((colsum_kernel<R, BH, true>), grid, dim3(kWG), 0, st, p);
  else
    hipLaunchKernelGGL((colsum_kernel<R, BH, false>), grid, dim3(kWG), 0, st, p);
}

void launch(const ColsumArgs& p, const det_colsum_cfg& c, int atomic, hipStream_t st) {
  const dim3 grid(static_cast<uint32_t>(ceil_div(p.T, c.block_t)), static_cast<uint32_t>(ceil_div(p.H, c.block_h)));
#define DET_COLSUM_CASE(bt, bh) \
  if (c.block_t == bt && c.block_h == bh) return launch_one<bt, bh>(p, atomic, grid, st);
  DET_COLSUM_CASE(64, 8) DET_COLSUM_CASE(64, 16) DET_COLSUM_CASE(64, 32)
  DET_COLSUM_CASE(128, 8) DET_COLSUM_CASE(128, 16) DET_COLSUM_CASE(128, 32)
  DET_COLSUM_CASE(256, 8) DET_COLSUM_CASE(256, 16) DET_COLSUM_CASE(256, 32)
#undef DET_COLSUM_CASE
}

int resolve_cfg(int64_t T, int64_t H, const det_colsum_cfg* cfg, det_colsum_cfg* out) {
  if (cfg) {
    if (!valid_cfg(*cfg))
      return set_error(DET_ERR_INVALID_ARG, "colsum: block_t must be 64/128/256 and block_h 8/16/32, got %d x %d",
                       cfg->block_t, cfg->block_h);
    *out = *cfg;
    return DET_OK;
  }
  return det_colsum_select_cfg(T, H, out);
}

}  // namespace
}  // namespace detgrad

using namespace detgrad;

// Shape-only selector (the deterministic route never times kernels to pick a
// tile: the page replaces timing-based autotuning by a block-size rule).
// block_h: the smallest of {8,16,32} covering H (all heads in one tile when
// H <= 32). block_t: the largest of {256,128,64} that still yields at least one
// workgroup per compute unit (256 CUs) in total, else 64.
extern "C" int det_colsum_select_cfg(int64_t T, int64_t H, det_colsum_cfg* out) {
  if (!out) return set_error(DET_ERR_INVALID_ARG, "colsum: out is NULL");
  if (T < 0 || H < 0) return set_error(DET_ERR_INVALID_ARG, "colsum: T and H must be >= 0");
  det_colsum_cfg c;
  c.block_h = H <= 8 ? 8 : (H <= 16 ? 16 : 32);
  const int64_t hb = ceil_div(H > 0 ? H : 1, c.block_h);
  c.block_t = 64;
  for (int bt : {256, 128}) {
    if (ceil_div(T, bt) * hb >= 256) {
      c.block_t = bt;
      break;
    }
  }
  *out = c;
  return ok();
}

extern "C" int det_colsum_workspace_size(int64_t T, int64_t H, const det_colsum_cfg* cfg, int atomic, size_t* bytes) {
  if (int s = check_atomic_flag(atomic)) return s;
  if (T < 0 || H < 0) return set_error(DET_ERR_INVALID_ARG, "colsum: T and H must be >= 0");
  if (!bytes) return set_error(DET_ERR_INVALID_ARG, "colsum: bytes is NULL");
  det_colsum_cfg c;
  if (int s = resolve_cfg(T, H, cfg, &c)) return s;
  *bytes = (atomic || T == 0 || H == 0) ? 0 : ws_bytes_for(T, H, c);
  return ok();
}

extern "C" int det_colsum(const void* a, int64_t a_st, int64_t a_sh, const void* dg, int64_t dg_st, int64_t dg_sh,
                          int in_dtype, const float* A_log, const float* dt_bias, int64_t T, int64_t H, float* dA_log,
                          float* ddt_bias, const det_colsum_cfg* cfg, void* ws, size_t ws_bytes, int atomic,
                          void* stream) {
  if (int s = check_atomic_flag(atomic)) return s;
  if (T < 0 || H < 0) return set_error(DET_ERR_INVALID_ARG, "colsum: T and H must be >= 0");
  if (in_dtype != DET_BF16 && in_dtype != DET_F32)
    return set_error(DET_ERR_INVALID_ARG, "colsum: unknown dtype %d", in_dtype);
  if (in_dtype != DET_BF16) return set_error(DET_ERR_UNSUPPORTED, "colsum: only bf16 inputs are implemented");
  det_colsum_cfg c;
  if (int s = resolve_cfg(T, H, cfg, &c)) return s;
  if (T == 0 || H == 0) return ok();
  if (!a || !dg || !A_log || !dt_bias || !dA_log || !ddt_bias)
    return set_error(DET_ERR_INVALID_ARG, "colsum: NULL pointer");
  if (a_st < 1 || a_sh < 1 || dg_st < 1 || dg_sh < 1)
    return set_error(DET_ERR_INVALID_ARG, "colsum: element strides must be >= 1");
  if (ceil_div(T, c.block_t) > 0x7FFFFFFF || ceil_div(H, c.block_h) > 65535)
    return set_error(DET_ERR_UNSUPPORTED, "colsum: problem too large for the launch grid");
  const size_t need = atomic ? 0 : ws_bytes_for(T, H, c);
  if (int s = check_workspace(ws, ws_bytes, need)) return s;
  const Range o1 = range1d(dA_log, H * 4), o2 = range1d(ddt_bias, H * 4);
  const Range ins[] = {range_strided(a, T, H, a_st, a_sh, 2), range_strided(dg, T, H, dg_st, dg_sh, 2),
                       range1d(A_log, H * 4), range1d(dt_bias, H * 4), range1d(ws, ws_bytes)};
  if (overlaps(o1, o2)) return set_error(DET_ERR_OVERLAP, "colsum: dA_log overlaps ddt_bias");
  for (const Range& r : ins)
    if (overlaps(o1, r) || overlaps(o2, r))
      return set_error(DET_ERR_OVERLAP, "colsum: an output overlaps an input or the workspace");
  ColsumArgs p;
  p.a = static_cast<const uint16_t*>(a);
  p.a_st = a_st;
  p.a_sh = a_sh;
  p.dg = static_cast<const uint16_t*>(dg);
  p.dg_st = dg_st;
  p.dg_sh = dg_sh;
  p.A_log = A_log;
  p.dt_bias = dt_bias;
  p.T = T;
  p.H = H;
  p.dA_log = dA_log;
  p.ddt_bias = ddt_bias;
  char* w = static_cast<char*>(ws);
  const size_t slot_bytes = align_up(static_cast<size_t>(ceil_div(T, c.block_t) * H) * 4, 256);
  p.ticket = atomic ? nullptr : reinterpret_cast<uint32_t*>(w);
  p.slot1 = atomic ? nullptr : reinterpret_cast<float*>(w + DET_WS_HEADER_BYTES);
  p.slot2 = atomic ? nullptr : reinterpret_cast<float*>(w + DET_WS_HEADER_BYTES + slot_bytes);
  launch(p, c, atomic, as_stream(stream));
  return check_launch("det_colsum");
}
