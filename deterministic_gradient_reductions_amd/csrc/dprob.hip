// det_grouped_dprob: dprob[m] += sum_n dY[m,n] * relu(C[m,n])^2 with one slot
// per 128-wide N tile, reduced in tile order.
//
// cudnn-frontend PR #521 (deterministic dprob in the grouped-GEMM dsReLU
// backward) fixes two sources of order variation: the running sum over N
// subtiles inside a CTA, and the cross-CTA atomics on dprob[token]. Here one
// wave owns a whole row, so both disappear by construction: the wave computes
// every 128-column tile partial itself (adjacent pairwise tree: 8 terms in
// each lane, then four DPP levels across 16 lanes) and folds the tile slots in
// tile order in registers before one add into dprob[m]. The slots never leave
// the chip, so the deterministic route needs no workspace at all.
//
// Memory layout and traffic: dY and C are read once, 16 bytes per lane per
// load (row-contiguous, fully coalesced), dprob is read and written once:
// 4 bytes per (m, n) plus 8 bytes per row. The kernel is HBM-bound.
//
// The atomic arm keeps the same tile partials but adds every one of them into
// dprob[m] with a hardware float atomic, as the page's default path does
// across CTAs. The four 512-column chunks of a row go to the four waves of one
// workgroup, which run side by side, so the order in which a row's sixteen
// adds land follows the scheduler and the memory system.
#include "common.hpp"

namespace detgrad {
namespace {

constexpr int kTileN = 128;
constexpr int kChunk = 512;  // columns one wave covers per step: 64 lanes x 8
constexpr int kWG = 256;
constexpr int kWaves = kWG / 64;
constexpr int kUnroll = 4;  // chunks whose loads are in flight together

__device__ __forceinline__ float term(float y, float c) {
  const float sq = c > 0.0f ? c * c : 0.0f;
  return y * sq;
}

__device__ __forceinline__ float tree8(const float (&t)[8]) {
  return ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
}

__device__ __forceinline__ float terms8_vec(const uint4& vy, const uint4& vc) {
  const uint32_t wy[4] = {vy.x, vy.y, vy.z, vy.w};
  const uint32_t wc[4] = {vc.x, vc.y, vc.z, vc.w};
  float t[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    t[2 * k] = term(bf16_lo(wy[k]), bf16_lo(wc[k]));
    t[2 * k + 1] = term(bf16_hi(wy[k]), bf16_hi(wc[k]));
  }
  return tree8(t);
}

__device__ __forceinline__ float terms8_scalar(const uint16_t* y, const uint16_t* c, int64_t col, int64_t N) {
  float t[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    t[i] = (col + i < N) ? term(bf16_to_f32(y[col + i]), bf16_to_f32(c[col + i])) : -0.0f;
  return tree8(t);
}

__device__ __forceinline__ void valid_rows(const int32_t* offs, int E, int64_t M, int64_t& lo, int64_t& hi) {
  int64_t a = offs[0], b = offs[E];
  lo = a < 0 ? 0 : (a > M ? M : a);
  hi = b < lo ? lo : (b > M ? M : b);
}

// Partial of this lane's 8 columns of chunk `ch`, reduced over the 16-lane row:
// afterwards lanes 16q..16q+15 hold the slot of tile 4*ch + q.
template <bool VEC>
__device__ __forceinline__ float chunk_slots(const uint16_t* y, const uint16_t* c, int64_t ch, int64_t N, int lane) {
  const int64_t col = ch * kChunk + 8 * lane;
  float s;
  if (VEC) {
    s = -0.0f;
    if (col < N) {
      const uint4 vy = *reinterpret_cast<const uint4*>(y + col);
      const uint4 vc = *reinterpret_cast<const uint4*>(c + col);
      s = terms8_vec(vy, vc);
    }
  } else {
    s = terms8_scalar(y, c, col, N);
  }
  return row16_tree(s);
}

template <bool VEC>
__global__ __launch_bounds__(kWG) void dprob_det_kernel(float* __restrict__ dprob, const uint16_t* __restrict__ dY,
                                                        int64_t ldy, const uint16_t* __restrict__ C, int64_t ldc,
                                                        int64_t M, int64_t N, const int32_t* __restrict__ offs, int E,
                                                        int rows_per_wg) {
  int64_t lo, hi;
  valid_rows(offs, E, M, lo, hi);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t first = lo + static_cast<int64_t>(blockIdx.x) * rows_per_wg;
  const int64_t end = first + rows_per_wg < hi ? first + rows_per_wg : hi;
  const int64_t n_chunks = (N + kChunk - 1) / kChunk;
  for (int64_t m = first + wave; m < end; m += kWaves) {
    const uint16_t* y = dY + m * ldy;
    const uint16_t* c = C + m * ldc;
    float total = -0.0f;
    for (int64_t ch0 = 0; ch0 < n_chunks; ch0 += kUnroll) {
      float s[kUnroll];
      if (VEC) {
        uint4 vy[kUnroll], vc[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
          const int64_t col = (ch0 + k) * kChunk + 8 * lane;
          if (col < N) {
            vy[k] = *reinterpret_cast<const uint4*>(y + col);
            vc[k] = *reinterpret_cast<const uint4*>(c + col);
          }
        }
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
          const int64_t col = (ch0 + k) * kChunk + 8 * lane;
          s[k] = row16_tree(col < N ? terms8_vec(vy[k], vc[k]) : -0.0f);
        }
      } else {
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) s[k] = chunk_slots<false>(y, c, ch0 + k, N, lane);
      }
#pragma unroll
      for (int k = 0; k < kUnroll; ++k) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if ((ch0 + k) * kChunk + q * kTileN < N) total = total + readlane(s[k], 16 * q);
        }
      }
    }
    if (lane == 0) dprob[m] = dprob[m] + total;
  }
}

template <bool VEC>
__global__ __launch_bounds__(kWG) void dprob_atomic_kernel(float* __restrict__ dprob, const uint16_t* __restrict__ dY,
                                                           int64_t ldy, const uint16_t* __restrict__ C, int64_t ldc,
                                                           int64_t M, int64_t N, const int32_t* __restrict__ offs,
                                                           int E) {
  int64_t lo, hi;
  valid_rows(offs, E, M, lo, hi);
  const int lane = threadIdx.x & 63;
  const int64_t rows = hi - lo;
  const int64_t n_chunks = (N + kChunk - 1) / kChunk;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (rows <= 0 || w >= rows * n_chunks) return;
  const int64_t m = lo + w / n_chunks;  // row-major: the chunks of one row run on neighbouring waves
  const int64_t ch = w % n_chunks;
  const float s = chunk_slots<VEC>(dY + m * ldy, C + m * ldc, ch, N, lane);
  // lanes 16q hold the slot of tile 4 ch + q
  if ((lane & 15) == 0 && ch * kChunk + (lane >> 4) * kTileN < N) unsafeAtomicAdd(dprob + m, s);
}

int check_cfg(const det_dprob_cfg* cfg, det_dprob_cfg* out) {
  det_dprob_cfg c{kTileN, 4};
  if (cfg) c = *cfg;
  if (c.tile_n != kTileN) return set_error(DET_ERR_INVALID_ARG, "dprob: tile_n must be %d, got %d", kTileN, c.tile_n);
  if (c.rows_per_wg < 1 || c.rows_per_wg > 1024)
    return set_error(DET_ERR_INVALID_ARG, "dprob: rows_per_wg must be in [1, 1024], got %d", c.rows_per_wg);
  *out = c;
  return DET_OK;
}

}  // namespace
}  // namespace detgrad

using namespace detgrad;

extern "C" int det_grouped_dprob_workspace_size(int64_t M, int64_t N, const det_dprob_cfg* cfg, int atomic,
                                                size_t* bytes) {
  if (int s = check_atomic_flag(atomic)) return s;
  if (M < 0 || N < 0) return set_error(DET_ERR_INVALID_ARG, "dprob: M and N must be >= 0");
  if (!bytes) return set_error(DET_ERR_INVALID_ARG, "dprob: bytes is NULL");
  det_dprob_cfg c;
  if (int s = check_cfg(cfg, &c)) return s;
  *bytes = 0;
  return ok();
}

extern "C" int det_grouped_dprob(float* dprob, const void* dY, int64_t ldy, const void* C, int64_t ldc, int64_t M,
                                 int64_t N, const int32_t* offs, int32_t E, const det_dprob_cfg* cfg, void* ws,
                                 size_t ws_bytes, int atomic, void* stream) {
  if (int s = check_atomic_flag(atomic)) return s;
  if (M < 0 || N < 0 || E < 0) return set_error(DET_ERR_INVALID_ARG, "dprob: M, N and E must be >= 0");
  det_dprob_cfg c;
  if (int s = check_cfg(cfg, &c)) return s;
  if (M == 0 || N == 0) return ok();  // every total is -0.0: outputs unchanged
  if (!dprob || !dY || !C || !offs) return set_error(DET_ERR_INVALID_ARG, "dprob: NULL pointer");
  if (ldy < N || ldc < N) return set_error(DET_ERR_INVALID_ARG, "dprob: ldy and ldc must be >= N");
  const Range out = range1d(dprob, static_cast<size_t>(M) * 4);
  if (overlaps(out, range2d(dY, M, N, ldy, 2)) || overlaps(out, range2d(C, M, N, ldc, 2)) ||
      overlaps(out, range1d(offs, (static_cast<size_t>(E) + 1) * 4)) || overlaps(out, range1d(ws, ws_bytes)))
    return set_error(DET_ERR_OVERLAP, "dprob: dprob overlaps an input or the workspace");
  const bool vec = aligned(dY, 16) && aligned(C, 16) && ldy % 8 == 0 && ldc % 8 == 0 && N % 8 == 0;
  const hipStream_t st = as_stream(stream);
  const auto* y = static_cast<const uint16_t*>(dY);
  const auto* cc = static_cast<const uint16_t*>(C);
  if (atomic == 0) {
    const int64_t grid = ceil_div(M, c.rows_per_wg);
    if (vec)
      hipLaunchKernelGGL(dprob_det_kernel<true>, dim3(grid), dim3(kWG), 0, st, dprob, y, ldy, cc, ldc, M, N, offs, E,
                         c.rows_per_wg);
    else
      hipLaunchKernelGGL(dprob_det_kernel<false>, dim3(grid), dim3(kWG), 0, st, dprob, y, ldy, cc, ldc, M, N, offs, E,
                         c.rows_per_wg);
  } else {
    const int64_t waves = M * ceil_div(N, kChunk);
    const int64_t grid = ceil_div(waves, kWaves);
    if (grid > 0x7FFFFFFF) return set_error(DET_ERR_UNSUPPORTED, "dprob: problem too large for the atomic arm");
    if (vec)
      hipLaunchKernelGGL(dprob_atomic_kernel<true>, dim3(grid), dim3(kWG), 0, st, dprob, y, ldy, cc, ldc, M, N, offs, E);
    else
      hipLaunchKernelGGL(dprob_atomic_kernel<false>, dim3(grid), dim3(kWG), 0, st, dprob, y, ldy, cc, ldc, M, N, offs,
                         E);
  }
  return check_launch("det_grouped_dprob");
}
