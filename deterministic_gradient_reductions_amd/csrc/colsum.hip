// det_colsum: ordered A_log / dt_bias column sums of the Gated-DeltaNet gate
// backward (Megatron-LM PR #8244).
//
// One workgroup of 256 threads owns a tile of block_t rows x block_h heads.
// Each thread takes block_t*block_h/256 consecutive rows of one head, computes
// the two gradient terms per element (detmath, so the CPU oracle can match
// every bit) and reduces its rows with the adjacent pairwise tree in
// registers; the remaining tree levels run over LDS. The resulting tile slot
// (one per head and gradient) goes to the workspace. A second kernel on the
// same stream folds the slots of every head in tile order and adds the totals
// into dA_log / ddt_bias (the page has the caller reduce the partials on the
// same stream the backward runs on); the kernel boundary orders the slot writes before the fold without
// any device-wide fence inside a kernel.
//
// The atomic arm computes the same tile slots and adds them into the outputs
// with hardware float atomics, in whatever order the tiles finish.
//
// The per-element work is about 80 VALU lane-operations (exp, log1p, two
// divisions), so at large T the tile kernel is bound by vector ALU
// throughput; its workgroup order (below) keeps the HBM traffic at one read
// of each input line.
#include <mutex>

#include "common.hpp"
#include "detmath.hpp"

namespace detgrad {
namespace {

constexpr int kWG = 256;

struct ColsumArgs {
  const void* a;     // bf16 bits or float32 values (the kernel's input type)
  int64_t a_st, a_sh;
  const void* dg;
  int64_t dg_st, dg_sh;
  const float* A_log;
  const float* dt_bias;
  int64_t T, H;
  float* dA_log;
  float* ddt_bias;
  float* slot1;      // [S][H]
  float* slot2;      // [S][H]
  int64_t n_tiles;   // S
  int n_hg;          // head groups: ceil(H / block_h)
  void* da;          // [T, H] in the input type, or NULL
  int64_t da_st, da_sh;
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

// Gate inputs: bf16 (widened exactly) or float32.
__device__ __forceinline__ float gate_in(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float gate_in(const float* p, int64_t i) { return p[i]; }

// The elementwise da, stored in the input type: bf16 by round to nearest even
// on the bit pattern (NaN kept quiet), float32 as is.
__device__ __forceinline__ void gate_out(uint16_t* p, int64_t i, float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t r = (u & 0x7FFFFFFFu) > 0x7F800000u ? (u >> 16) | 0x40u : (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  p[i] = static_cast<uint16_t>(r);
}
__device__ __forceinline__ void gate_out(float* p, int64_t i, float v) { p[i] = v; }

template <int R, int BH, bool ATOMIC, typename TIn>
__global__ __launch_bounds__(kWG) void colsum_kernel(ColsumArgs p) {
  const TIn* const pa = static_cast<const TIn*>(p.a);
  const TIn* const pdg = static_cast<const TIn*>(p.dg);
  constexpr int kBT = R * kWG / BH;   // rows per tile
  constexpr int kNB = kWG / BH;       // row blocks per tile (threads per head)
  __shared__ float red1[kWG];
  __shared__ float red2[kWG];

  // XCD-aware order. Workgroups are dispatched to the 8 XCDs round-robin
  // (workgroup u runs on XCD u % 8) and each XCD has its own L2. Workgroup
  // u = 8 * n_hg * c + 8 * j + x takes tile 8c + x and head group j, so the
  // head groups of one tile run back to back on one XCD: a head group reads
  // block_h of a row's H elements, and the row's other head groups then find
  // its cache lines in that XCD's L2 instead of fetching them again.
  const uint32_t u = blockIdx.x;
  const uint32_t per = 8u * static_cast<uint32_t>(p.n_hg);
  const uint32_t r = u % per;
  const int64_t tile = static_cast<int64_t>(u / per) * 8 + (r & 7u);
  if (tile >= p.n_tiles) return;  // the last group of 8 tiles may be short
  const int tid = threadIdx.x;
  const int hl = tid % BH;
  const int rb = tid / BH;
  const int64_t h = static_cast<int64_t>(r >> 3) * BH + hl;
  const int64_t r0 = tile * kBT + static_cast<int64_t>(rb) * R;

  float v1[R], v2[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    v1[i] = -0.0f;
    v2[i] = -0.0f;
  }
  if (h < p.H) {
    const float nA = -dm::exp32(p.A_log[h]);
    const float bias = p.dt_bias[h];
    // row r0 of head h; row r0 + i is i row strides further (the strides are
    // uniform, so each row costs one 64-bit address add)
    const TIn* const ra = pa + r0 * p.a_st + h * p.a_sh;
    const TIn* const rd = pdg + r0 * p.dg_st + h * p.dg_sh;
    // All of the thread's loads are issued before any math, so their latencies
    // overlap (da, when it is written, overlaps no input: the host checks that).
    float xa[R], xd[R];
    auto term = [&](int i) {
      float sp, sg;
      dm::softplus_sigmoid(xa[i], sp, sg);
      v1[i] = xd[i] * (nA * sp);
      v2[i] = xd[i] * (nA * sg);
      if (p.da) gate_out(static_cast<TIn*>(p.da), (r0 + i) * p.da_st + h * p.da_sh, v2[i]);  // da = the ddt_bias term
    };
    if ((tile + 1) * kBT <= p.T) {  // every row of the tile exists (all tiles but a tail)
#pragma unroll
      for (int i = 0; i < R; ++i) {
        xa[i] = gate_in(ra, i * p.a_st) + bias;
        xd[i] = gate_in(rd, i * p.dg_st);
      }
#pragma unroll
      for (int i = 0; i < R; ++i) term(i);
    } else {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const bool in = r0 + i < p.T;
        xa[i] = in ? gate_in(ra, i * p.a_st) + bias : 0.0f;
        xd[i] = in ? gate_in(rd, i * p.dg_st) : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < R; ++i)
        if (r0 + i < p.T) term(i);
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
}

// Phase 2: fold the tile slots of every head left to right and add the totals.
// One wave per (head, gradient); the fold is one chain of dependent adds, so
// its time is the chain's length times the add's issue latency. Rounds of 1024
// tiles: lane j loads tiles 16j .. 16j + 15 of the round (the next round's
// loads are in flight while a round is added) and parks them in LDS; the chain
// then reads four consecutive tiles at a time with one LDS read that every
// lane makes at the same address, so each tile costs one add with a register
// operand. Tiles past S read as -0.0, which leaves the sum bitwise unchanged.
constexpr int kFoldRound = 1024;
constexpr int kFoldPerLane = kFoldRound / 64;
constexpr int kFoldAhead = 16;  // LDS reads in flight ahead of the chain

__global__ __launch_bounds__(64) void colsum_fold_kernel(const float* __restrict__ slot1,
                                                         const float* __restrict__ slot2, int64_t S, int64_t H,
                                                         float* __restrict__ dA_log, float* __restrict__ ddt_bias) {
  __shared__ float4 park[kFoldRound / 4];
  const int lane = threadIdx.x;
  const int64_t h = blockIdx.x;
  const bool second = blockIdx.y != 0;
  const float* const s = (second ? slot2 : slot1) + h;
  float v[kFoldPerLane];
  auto load = [&](int64_t i0) {
#pragma unroll
    for (int k = 0; k < kFoldPerLane; ++k) {
      const int64_t i = i0 + kFoldPerLane * lane + k;
      v[k] = i < S ? s[i * H] : -0.0f;
    }
  };
  float tot = -0.0f;
  load(0);
  for (int64_t i0 = 0; i0 < S; i0 += kFoldRound) {
    // the previous round's LDS reads precede these writes in the wave's order
#pragma unroll
    for (int q = 0; q < kFoldPerLane / 4; ++q)
      park[(kFoldPerLane / 4) * lane + q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    if (i0 + kFoldRound < S) load(i0 + kFoldRound);
    const int64_t left = S - i0;
    if (left >= kFoldRound) {
      // a whole round, unrolled, with each LDS read issued kFoldAhead steps
      // before the adds that use it (the scheduling barriers keep that order)
      float4 w[kFoldAhead];
#pragma unroll
      for (int q = 0; q < kFoldAhead; ++q) w[q] = park[q];
#pragma unroll
      for (int q = 0; q < kFoldRound / 4; ++q) {
        const float4 x = w[q % kFoldAhead];
        if (q + kFoldAhead < kFoldRound / 4) w[q % kFoldAhead] = park[q + kFoldAhead];
        tot = tot + x.x;
        tot = tot + x.y;
        tot = tot + x.z;
        tot = tot + x.w;
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      const int n16 = static_cast<int>((left + 15) / 16);
      for (int g = 0; g < n16; ++g) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 w = park[4 * g + q];
          tot = tot + w.x;
          tot = tot + w.y;
          tot = tot + w.z;
          tot = tot + w.w;
        }
      }
    }
  }
  if (lane == 0) {
    float* const o = (second ? ddt_bias : dA_log) + h;
    *o = *o + tot;
  }
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

template <int BT, int BH, typename TIn>
void launch_one(const ColsumArgs& p, int atomic, dim3 grid, hipStream_t st) {
  constexpr int R = BT * BH / kWG;
  if (atomic) {
    hipLaunchKernelGGL((colsum_kernel<R, BH, true, TIn>), grid, dim3(kWG), 0, st, p);
  } else {
    hipLaunchKernelGGL((colsum_kernel<R, BH, false, TIn>), grid, dim3(kWG), 0, st, p);
    hipLaunchKernelGGL(colsum_fold_kernel, dim3(static_cast<uint32_t>(p.H), 2), dim3(64), 0, st, p.slot1, p.slot2,
                       p.n_tiles, p.H, p.dA_log, p.ddt_bias);
  }
}

void launch(const ColsumArgs& p, const det_colsum_cfg& c, int atomic, bool f32_in, hipStream_t st) {
  // groups of 8 tiles times the head groups (see colsum_kernel's order)
  const dim3 grid(static_cast<uint32_t>(ceil_div(p.n_tiles, 8) * 8 * p.n_hg));
#define DET_COLSUM_CASE(bt, bh) \
  if (c.block_t == bt && c.block_h == bh)                                                                 \
    return f32_in ? launch_one<bt, bh, float>(p, atomic, grid, st) : launch_one<bt, bh, uint16_t>(p, atomic, grid, st);
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
// block_h never changes a bit, so it is the smallest, 8: more workgroups hide
// the latency of the per-element transcendental chains. block_t: the largest
// of {256, 128} that still yields at least four workgroups per compute unit
// (1024 on 256 CUs), else 64.
extern "C" int det_colsum_select_cfg(int64_t T, int64_t H, det_colsum_cfg* out) {
  if (!out) return set_error(DET_ERR_INVALID_ARG, "colsum: out is NULL");
  if (T < 0 || H < 0) return set_error(DET_ERR_INVALID_ARG, "colsum: T and H must be >= 0");
  det_colsum_cfg c;
  c.block_h = 8;
  const int64_t hb = ceil_div(H > 0 ? H : 1, c.block_h);
  c.block_t = 64;
  for (int bt : {256, 128}) {
    if (ceil_div(T, bt) * hb >= 1024) {
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

// ---------------------------------------------------------------------------
// Static scratch of det_colsum_noalloc, for callers that cannot allocate. Each
// GPU the library runs on holds its own copy of this array until the process
// ends. Host code never passes the array's name to a kernel (on the host that
// name is only a stand-in): the device address of each GPU's copy is looked up
// once per device with hipGetSymbolAddress and kept here.
namespace detgrad {
namespace {
constexpr size_t kNoAllocBytes = size_t(4) << 20;  // header + two slot arrays of up to 2 MiB - 128 B each
}  // namespace
}  // namespace detgrad

static __device__ __align__(256) char scratch[detgrad::kNoAllocBytes];

namespace detgrad {
namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The device address of this GPU's copy of `scratch` (the current device's).
int noalloc_scratch(void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(DET_ERR_HIP, "colsum_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return set_error(DET_ERR_UNSUPPORTED, "colsum_noalloc: device %d", dev);
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev])
    return set_error(DET_ERR_HIP, "colsum_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(g_scratch_err[dev]));
  *out = g_scratch_ptr[dev];
  return DET_OK;
}
}  // namespace
}  // namespace detgrad

namespace detgrad {
namespace {
int colsum_entry(const void* a, int64_t a_st, int64_t a_sh, const void* dg, int64_t dg_st, int64_t dg_sh, int in_dtype,
                 const float* A_log, const float* dt_bias, int64_t T, int64_t H, float* dA_log, float* ddt_bias,
                 void* da, int64_t da_st, int64_t da_sh, bool with_da, const det_colsum_cfg* cfg, void* ws,
                 size_t ws_bytes, int atomic, void* stream, bool noalloc = false) {
  if (int s = check_atomic_flag(atomic)) return s;
  if (T < 0 || H < 0) return set_error(DET_ERR_INVALID_ARG, "colsum: T and H must be >= 0");
  if (in_dtype != DET_BF16 && in_dtype != DET_F32)
    return set_error(DET_ERR_INVALID_ARG, "colsum: unknown dtype %d", in_dtype);
  det_colsum_cfg c;
  if (int s = resolve_cfg(T, H, cfg, &c)) return s;
  if (T == 0 || H == 0) return ok();
  if (!a || !dg || !A_log || !dt_bias || !dA_log || !ddt_bias || (with_da && !da))
    return set_error(DET_ERR_INVALID_ARG, "colsum: NULL pointer");
  if (a_st < 1 || a_sh < 1 || dg_st < 1 || dg_sh < 1)
    return set_error(DET_ERR_INVALID_ARG, "colsum: element strides must be >= 1");
  if (ceil_div(H, c.block_h) > 65535 || ceil_div(ceil_div(T, c.block_t), 8) * 8 * ceil_div(H, c.block_h) > 0x7FFFFFFF)
    return set_error(DET_ERR_UNSUPPORTED, "colsum: problem too large for the launch grid");
  const size_t need = atomic ? 0 : ws_bytes_for(T, H, c);
  if (noalloc) {
    if (need > kNoAllocBytes)
      return set_error(DET_ERR_WORKSPACE,
                       "colsum_noalloc: the slots need %zu bytes, more than the %zu of the library's static scratch "
                       "(use det_colsum with a workspace, or a larger block_t)",
                       need, static_cast<size_t>(kNoAllocBytes));
    if (need > 0) {
      if (int s = noalloc_scratch(&ws)) return s;
      ws_bytes = kNoAllocBytes;
    }
  } else if (int s = check_workspace(ws, ws_bytes, need)) {
    return s;
  }
  const Range o1 = range1d(dA_log, H * 4), o2 = range1d(ddt_bias, H * 4);
  const size_t esz = in_dtype == DET_F32 ? 4 : 2;
  const Range ins[] = {range_strided(a, T, H, a_st, a_sh, esz), range_strided(dg, T, H, dg_st, dg_sh, esz),
                       range1d(A_log, H * 4), range1d(dt_bias, H * 4), range1d(ws, ws_bytes)};
  if (overlaps(o1, o2)) return set_error(DET_ERR_OVERLAP, "colsum: dA_log overlaps ddt_bias");
  for (const Range& r : ins)
    if (overlaps(o1, r) || overlaps(o2, r))
      return set_error(DET_ERR_OVERLAP, "colsum: an output overlaps an input or the workspace");
  if (with_da) {
    if (da_st < 1 || da_sh < 1) return set_error(DET_ERR_INVALID_ARG, "colsum: da strides must be >= 1");
    // one of the two strides must step over the whole extent of the other, so
    // that no two elements of da share an address
    if (!(da_st >= H * da_sh || da_sh >= T * da_st))
      return set_error(DET_ERR_INVALID_ARG, "colsum: da strides map two elements to one address");
    const Range od = range_strided(da, T, H, da_st, da_sh, esz);
    if (overlaps(od, o1) || overlaps(od, o2)) return set_error(DET_ERR_OVERLAP, "colsum: da overlaps another output");
    for (const Range& r : ins)
      if (overlaps(od, r)) return set_error(DET_ERR_OVERLAP, "colsum: da overlaps an input or the workspace");
  }
  ColsumArgs p;
  p.a = a;
  p.a_st = a_st;
  p.a_sh = a_sh;
  p.dg = dg;
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
  p.slot1 = atomic ? nullptr : reinterpret_cast<float*>(w + DET_WS_HEADER_BYTES);
  p.slot2 = atomic ? nullptr : reinterpret_cast<float*>(w + DET_WS_HEADER_BYTES + slot_bytes);
  p.n_tiles = ceil_div(T, c.block_t);
  p.n_hg = static_cast<int>(ceil_div(H, c.block_h));
  p.da = with_da ? da : nullptr;
  p.da_st = da_st;
  p.da_sh = da_sh;
  launch(p, c, atomic, in_dtype == DET_F32, as_stream(stream));
  return check_launch(with_da ? "det_colsum_da" : "det_colsum");
}
}  // namespace
}  // namespace detgrad

extern "C" int det_colsum(const void* a, int64_t a_st, int64_t a_sh, const void* dg, int64_t dg_st, int64_t dg_sh,
                          int in_dtype, const float* A_log, const float* dt_bias, int64_t T, int64_t H, float* dA_log,
                          float* ddt_bias, const det_colsum_cfg* cfg, void* ws, size_t ws_bytes, int atomic,
                          void* stream) {
  return colsum_entry(a, a_st, a_sh, dg, dg_st, dg_sh, in_dtype, A_log, dt_bias, T, H, dA_log, ddt_bias, nullptr, 1, 1,
                      false, cfg, ws, ws_bytes, atomic, stream);
}

extern "C" int det_colsum_da(const void* a, int64_t a_st, int64_t a_sh, const void* dg, int64_t dg_st, int64_t dg_sh,
                             int in_dtype, const float* A_log, const float* dt_bias, int64_t T, int64_t H,
                             float* dA_log, float* ddt_bias, void* da, int64_t da_st, int64_t da_sh,
                             const det_colsum_cfg* cfg, void* ws, size_t ws_bytes, int atomic, void* stream) {
  return colsum_entry(a, a_st, a_sh, dg, dg_st, dg_sh, in_dtype, A_log, dt_bias, T, H, dA_log, ddt_bias, da, da_st,
                      da_sh, true, cfg, ws, ws_bytes, atomic, stream);
}

// For callers that cannot allocate: det_colsum with its slots in the library's
// static scratch (see noalloc_scratch). Every call on a GPU shares that GPU's
// scratch, so calls that can overlap on one GPU race.
extern "C" int det_colsum_noalloc(const void* a, int64_t a_st, int64_t a_sh, const void* dg, int64_t dg_st,
                                  int64_t dg_sh, int in_dtype, const float* A_log, const float* dt_bias, int64_t T,
                                  int64_t H, float* dA_log, float* ddt_bias, const det_colsum_cfg* cfg, int atomic,
                                  void* stream) {
  return colsum_entry(a, a_st, a_sh, dg, dg_st, dg_sh, in_dtype, A_log, dt_bias, T, H, dA_log, ddt_bias, nullptr, 1, 1,
                      false, cfg, nullptr, 0, atomic, stream, true);
}
