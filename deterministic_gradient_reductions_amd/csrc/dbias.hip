// det_grouped_dbias: dbias[e][n] += sum of dA[m][n] over the rows m of expert e,
// with one float32 slot per (M tile, column), folded per expert in tile order.
//
// cudnn-frontend PR #521 (deterministic dprob/dbias in the grouped-GEMM dsReLU
// backward), the commit that extends the determinism flag to dbias: dbias
// contends across M tiles, so each (M block, column) gets its own slot with a
// single writer, and a per-expert segment sum of the slots replaces the
// atomics; experts start on tile boundaries, so no tile holds two experts.
// Here tiles are counted from each expert's first row (with aligned experts
// these are the absolute M blocks), and the segment sum is a left-to-right fold
// of the expert's slots, added once into dbias.
//
// Tile kernel: a workgroup owns one tile (block_m rows of one expert) and 512
// columns. Lane l of each wave holds 8 consecutive columns (one 16-byte load
// per row, fully coalesced); wave w takes the w-th quarter of the tile's rows
// and reduces it with the adjacent pairwise tree in registers (rows past the
// expert's end are -0.0); the four quarter values meet in LDS as
// ((q0 + q1) + (q2 + q3)), the top two levels of the same tree. The slot (or,
// on the atomic arm, a float atomic add into dbias) is written once.
// Fold kernel: one thread per (expert, column) adds the expert's slots left to
// right and adds the total into dbias.
//
// Traffic: dA is read once (2 bytes per element); the slots are written and
// read once (4 bytes per tile and column, 1/64 of dA's bytes at block_m 128);
// dbias is read and written once. The tile kernel is HBM-bound.
#include "common.hpp"

namespace detgrad {
namespace {

constexpr int kCols = 512;  // columns per workgroup: 64 lanes x 8

// Expert tile table, computed by every workgroup from the device offsets:
// b_e = min(M, max(0, offs[0..e])) (clamped monotone), tiles_e =
// ceil((b_{e+1} - b_e) / block_m), tile_start_e = sum of tiles before e.
// Returns the expert of global tile t (or -1 past the last tile) and its rows.
__device__ bool tile_of(const int32_t* __restrict__ offs, int E, int64_t M, int bm, int64_t t, int& e_out,
                        int64_t& r0, int64_t& r1) {
  const int lane = threadIdx.x & 63;
  int64_t run_b = offs[0];  // b of the first expert of this chunk
  run_b = run_b < 0 ? 0 : (run_b < M ? run_b : M);
  int64_t run_t = 0;        // tiles before this chunk
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    // running max of the offsets inside the chunk (lanes past E repeat the last bound)
    int64_t v = e < E + 1 ? static_cast<int64_t>(offs[e < E ? e + 1 : E]) : 0;
    v = v < 0 ? 0 : v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int64_t u = __shfl_up(v, d);
      if (lane >= d) v = v > u ? v : u;
    }
    int64_t b1 = v > run_b ? v : run_b;   // b_{e+1}
    b1 = b1 < M ? b1 : M;
    int64_t b0 = __shfl_up(b1, 1);
    if (lane == 0) b0 = run_b;             // b_e
    const int64_t nt = (e < E && b1 > b0) ? (b1 - b0 + bm - 1) / bm : 0;
    int64_t incl = nt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int64_t u = __shfl_up(incl, d);
      if (lane >= d) incl += u;
    }
    const int64_t first = run_t + incl - nt;
    const uint64_t hit = __ballot(e < E && t >= first && t < first + nt);
    if (hit) {
      const int j = __builtin_ctzll(hit);
      e_out = e0 + j;
      const int64_t f = __shfl(first, j), lo = __shfl(b0, j), hi = __shfl(b1, j);
      r0 = lo + (t - f) * bm;
      r1 = r0 + bm < hi ? r0 + bm : hi;
      return true;
    }
    run_t += __shfl(incl, 63);
    run_b = __shfl(b1, 63);
    if (run_b < 0) run_b = 0;
  }
  return false;
}

// Pairwise tree over Q rows of 8 columns held as Q x 8 floats: in place, level by level.
template <int Q>
__device__ __forceinline__ void tree_rows(float (&x)[Q][8]) {
#pragma unroll
  for (int s = 1; s < Q; s <<= 1)
#pragma unroll
    for (int r = 0; r < Q; r += 2 * s)
#pragma unroll
      for (int c = 0; c < 8; ++c) x[r][c] = x[r][c] + x[r + s][c];
}

// Rows [a, a + Q) of the tile (absolute row index base + i), -0.0 at rows >= r1.
template <int Q>
__device__ __forceinline__ void load_rows(float (&x)[Q][8], const uint16_t* __restrict__ dA, int64_t lda,
                                          int64_t a, int64_t r1, int64_t col) {
  uint4 v[Q];
#pragma unroll
  for (int i = 0; i < Q; ++i) {
    const int64_t r = a + i < r1 ? a + i : a;  // a < r1 always: a valid row
    v[i] = *reinterpret_cast<const uint4*>(dA + r * lda + col);
  }
#pragma unroll
  for (int i = 0; i < Q; ++i) {
    const bool in = a + i < r1;  // wave-uniform
    x[i][0] = in ? bf16_lo(v[i].x) : -0.0f; x[i][1] = in ? bf16_hi(v[i].x) : -0.0f;
    x[i][2] = in ? bf16_lo(v[i].y) : -0.0f; x[i][3] = in ? bf16_hi(v[i].y) : -0.0f;
    x[i][4] = in ? bf16_lo(v[i].z) : -0.0f; x[i][5] = in ? bf16_hi(v[i].z) : -0.0f;
    x[i][6] = in ? bf16_lo(v[i].w) : -0.0f; x[i][7] = in ? bf16_hi(v[i].w) : -0.0f;
  }
}

// Q rows per wave (block_m / 4), loaded and reduced in pieces of at most 32 rows.
template <int Q, bool ATOMIC>
__global__ __launch_bounds__(256) void dbias_tile_kernel(const uint16_t* __restrict__ dA, int64_t lda, int64_t M,
                                                         int64_t N, const int32_t* __restrict__ offs, int E,
                                                         float* __restrict__ slots, int32_t* __restrict__ tstart,
                                                         float* __restrict__ dbias, int64_t ld_e) {
  constexpr int BM = 4 * Q;
  constexpr int P = Q < 32 ? Q : 32;  // rows per piece
  __shared__ float part[4][kCols + 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the tile table for the fold: tile starts per expert (and the total),
  // written by the first workgroup whether or not any expert has rows
  if (!ATOMIC && blockIdx.x == 0 && blockIdx.y == 0 && wave == 0) {
    int64_t run_b = 0, run_t = 0;
    for (int e0 = 0; e0 <= E; e0 += 64) {
      const int ee = e0 + lane;
      int64_t v = ee < E + 1 ? static_cast<int64_t>(offs[ee]) : 0;
      v = v < 0 ? 0 : v;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int64_t u = __shfl_up(v, d);
        if (lane >= d) v = v > u ? v : u;
      }
      int64_t b = v > run_b ? v : run_b;
      b = b < M ? b : M;                    // b_ee
      int64_t bp = __shfl_up(b, 1);
      if (lane == 0) bp = e0 == 0 ? b : run_b;  // b_{ee-1} (b_0 for ee = 0: no tiles before it)
      const int64_t nt = (ee >= 1 && ee <= E && b > bp) ? (b - bp + BM - 1) / BM : 0;  // tiles of expert ee-1
      int64_t incl = nt;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int64_t u = __shfl_up(incl, d);
        if (lane >= d) incl += u;
      }
      if (ee <= E) tstart[ee] = static_cast<int32_t>(run_t + incl);  // tiles of experts before ee
      run_t += __shfl(incl, 63);
      run_b = __shfl(b, 63);
    }
  }
  const int64_t t = blockIdx.x;
  int e;
  int64_t r0, r1;
  if (!tile_of(offs, E, M, BM, t, e, r0, r1)) return;  // past the last tile (the grid covers the worst case)
  const int64_t col = static_cast<int64_t>(blockIdx.y) * kCols + 8 * lane;
  const bool live = col < N;  // N % 8 == 0: a lane's 8 columns are all inside or all outside
  float q[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) q[c] = -0.0f;
  const int64_t a0 = r0 + static_cast<int64_t>(wave) * Q;
  if (live && a0 < r1) {
#pragma unroll
    for (int p = 0; p < Q / P; ++p) {
      const int64_t a = a0 + p * P;
      float x[P][8];
      if (a < r1) {
        load_rows<P>(x, dA, lda, a, r1, col);
        tree_rows<P>(x);
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) x[0][c] = -0.0f;
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) q[c] = p == 0 ? x[0][c] : q[c] + x[0][c];
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) part[wave][8 * lane + c] = q[c];
  __syncthreads();
  // the top two tree levels: thread i combines column i of the four quarters
  for (int i = threadIdx.x; i < kCols; i += 256) {
    const int64_t n = static_cast<int64_t>(blockIdx.y) * kCols + i;
    if (n >= N) break;
    const float s = (part[0][i] + part[1][i]) + (part[2][i] + part[3][i]);
    if (ATOMIC)
      unsafeAtomicAdd(dbias + static_cast<int64_t>(e) * ld_e + n, s);
    else
      slots[t * N + n] = s;
  }

}

// dbias[e][n] += ((slot[t0][n] + slot[t0+1][n]) + ...) over the expert's tiles.
__global__ __launch_bounds__(256) void dbias_fold_kernel(const float* __restrict__ slots,
                                                         const int32_t* __restrict__ tstart, int64_t N,
                                                         float* __restrict__ dbias, int64_t ld_e) {
  const int64_t n = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int e = blockIdx.y;
  if (n >= N) return;
  const int64_t t0 = tstart[e], t1 = tstart[e + 1];
  if (t1 <= t0) return;  // no rows: dbias[e] bitwise unchanged
  float tot = -0.0f;
  for (int64_t t = t0; t < t1; t += 8) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = t + i < t1 ? slots[(t + i) * N + n] : -0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) tot = tot + v[i];
  }
  float* const o = dbias + static_cast<int64_t>(e) * ld_e + n;
  *o = *o + tot;
}

int check_cfg(const det_dbias_cfg* cfg, det_dbias_cfg* out) {
  det_dbias_cfg c{128, 512};
  if (cfg) c = *cfg;
  if (c.block_m != 64 && c.block_m != 128 && c.block_m != 256)
    return set_error(DET_ERR_INVALID_ARG, "dbias: block_m must be 64, 128 or 256, got %d", c.block_m);
  if (c.block_n != 512) return set_error(DET_ERR_INVALID_ARG, "dbias: block_n must be 512, got %d", c.block_n);
  *out = c;
  return DET_OK;
}

int64_t max_tiles(int64_t M, int64_t E, int bm) { return ceil_div(M, bm) + E; }

size_t ws_bytes_for(int64_t M, int64_t N, int64_t E, int bm) {
  return DET_WS_HEADER_BYTES + align_up(static_cast<size_t>(E + 1) * 4, 256) +
         align_up(static_cast<size_t>(max_tiles(M, E, bm) * N) * 4, 256);
}

}  // namespace
}  // namespace detgrad

using namespace detgrad;

extern "C" int det_grouped_dbias_workspace_size(int64_t M, int64_t N, int32_t E, const det_dbias_cfg* cfg, int atomic,
                                                size_t* bytes) {
  if (int s = check_atomic_flag(atomic)) return s;
  if (!bytes) return set_error(DET_ERR_INVALID_ARG, "dbias: bytes is NULL");
  if (M < 0 || N < 0 || E < 0) return set_error(DET_ERR_INVALID_ARG, "dbias: M, N and E must be >= 0");
  det_dbias_cfg c;
  if (int s = check_cfg(cfg, &c)) return s;
  *bytes = (atomic || M == 0 || N == 0 || E == 0) ? 0 : ws_bytes_for(M, N, E, c.block_m);
  return ok();
}

extern "C" int det_grouped_dbias(float* dbias, int64_t ld_e, const void* dA, int64_t lda, int64_t M, int64_t N,
                                 const int32_t* offs, int32_t E, const det_dbias_cfg* cfg, void* ws, size_t ws_bytes,
                                 int atomic, void* stream) {
  if (int s = check_atomic_flag(atomic)) return s;
  if (M < 0 || N < 0 || E < 0) return set_error(DET_ERR_INVALID_ARG, "dbias: M, N and E must be >= 0");
  det_dbias_cfg c;
  if (int s = check_cfg(cfg, &c)) return s;
  if (M == 0 || N == 0 || E == 0) return ok();  // no rows or no columns: dbias unchanged
  if (!dbias || !dA || !offs) return set_error(DET_ERR_INVALID_ARG, "dbias: NULL pointer");
  if (lda < N || ld_e < N) return set_error(DET_ERR_INVALID_ARG, "dbias: lda and ld_e must be >= N");
  if (N % 8 || lda % 8 || !aligned(dA, 16))
    return set_error(DET_ERR_UNSUPPORTED, "dbias: N and lda must be multiples of 8 and dA 16-byte aligned");
  if (E > 65535) return set_error(DET_ERR_UNSUPPORTED, "dbias: E must be <= 65535");
  const int64_t nt = max_tiles(M, E, c.block_m);
  if (nt > 0x7FFFFFFF || ceil_div(N, kCols) > 65535 || nt * N > (int64_t(1) << 40))
    return set_error(DET_ERR_UNSUPPORTED, "dbias: problem too large");
  const size_t need = atomic ? 0 : ws_bytes_for(M, N, E, c.block_m);
  if (int s = check_workspace(ws, ws_bytes, need)) return s;
  const Range out = range2d(dbias, E, N, ld_e, 4);
  if (overlaps(out, range2d(dA, M, N, lda, 2)) || overlaps(out, range1d(offs, (static_cast<size_t>(E) + 1) * 4)) ||
      overlaps(out, range1d(ws, ws_bytes)))
    return set_error(DET_ERR_OVERLAP, "dbias: dbias overlaps an input or the workspace");
  const hipStream_t st = as_stream(stream);
  const auto* a = static_cast<const uint16_t*>(dA);
  char* w = static_cast<char*>(ws);
  auto* tstart = atomic ? nullptr : reinterpret_cast<int32_t*>(w + DET_WS_HEADER_BYTES);
  auto* slots = atomic ? nullptr
                       : reinterpret_cast<float*>(w + DET_WS_HEADER_BYTES + align_up(static_cast<size_t>(E + 1) * 4, 256));
  const dim3 grid(static_cast<uint32_t>(nt), static_cast<uint32_t>(ceil_div(N, kCols)));
#define DET_DBIAS_LAUNCH(Q)                                                                                       \
  if (c.block_m == 4 * Q) {                                                                                       \
    if (atomic)                                                                                                   \
      hipLaunchKernelGGL((dbias_tile_kernel<Q, true>), grid, dim3(256), 0, st, a, lda, M, N, offs, E, slots,      \
                         tstart, dbias, ld_e);                                                                    \
    else                                                                                                          \
      hipLaunchKernelGGL((dbias_tile_kernel<Q, false>), grid, dim3(256), 0, st, a, lda, M, N, offs, E, slots,     \
                         tstart, dbias, ld_e);                                                                    \
  }
  DET_DBIAS_LAUNCH(16) DET_DBIAS_LAUNCH(32) DET_DBIAS_LAUNCH(64)
#undef DET_DBIAS_LAUNCH
  if (!atomic)
    hipLaunchKernelGGL(dbias_fold_kernel, dim3(static_cast<uint32_t>(ceil_div(N, 256)), static_cast<uint32_t>(E)),
                       dim3(256), 0, st, slots, tstart, N, dbias, ld_e);
  return check_launch("det_grouped_dbias");
}
