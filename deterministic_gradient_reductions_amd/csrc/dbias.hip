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
// Tile kernel: a workgroup owns one tile (block_m rows of one expert) and
// block_n columns (512, 256 or 128: columns are independent, so the width
// never changes a bit; narrower blocks give more workgroups, which evens out
// the work per compute unit); consecutive workgroups take the column blocks of
// one tile. Lane l of each wave holds block_n / 64 consecutive columns (one
// 16-, 8- or 4-byte load per row, coalesced); wave w takes the w-th quarter of the tile's rows and reduces it
// with the adjacent pairwise tree, fed row by row into a stack of partial
// sums while the next 16 rows' loads are in flight (rows past the expert's
// end are -0.0); the four quarter values meet in LDS as
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

// Columns per workgroup: 64 lanes x CPL (8, 4 or 2 columns per lane, one
// 16-, 8- or 4-byte load per row), the configuration's block_n.

// Inclusive scans over the 64 lanes on DPP (row shifts by 1, 2, 4, 8, then
// the last lane of row 0 into rows 1 and 3 and of row 1 into rows 2 and 3);
// lanes without a source read 0, the identity of both (the values are >= 0).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_src(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROW_MASK, 0xF, false));
}
__device__ __forceinline__ uint32_t scan_add(uint32_t v) {
  v += dpp_src<0x111, 0xF>(v); v += dpp_src<0x112, 0xF>(v); v += dpp_src<0x114, 0xF>(v);
  v += dpp_src<0x118, 0xF>(v); v += dpp_src<0x142, 0xA>(v); v += dpp_src<0x143, 0xC>(v);
  return v;
}
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t scan_max(uint32_t v) {
  v = umax(v, dpp_src<0x111, 0xF>(v)); v = umax(v, dpp_src<0x112, 0xF>(v)); v = umax(v, dpp_src<0x114, 0xF>(v));
  v = umax(v, dpp_src<0x118, 0xF>(v)); v = umax(v, dpp_src<0x142, 0xA>(v)); v = umax(v, dpp_src<0x143, 0xC>(v));
  return v;
}
// the value of the lane below, `fill` in lane 0 (DPP wave_shr:1 with the fill
// as the old value; computed with every lane active, never under a branch)
__device__ __forceinline__ uint32_t from_lane_below(uint32_t v, uint32_t fill) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(fill), static_cast<int>(v), 0x138, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t lane_value(uint32_t v, int j) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), j));
}
__device__ __forceinline__ uint32_t clamp_off(int32_t o, uint32_t M) {
  const uint32_t v = o < 0 ? 0u : static_cast<uint32_t>(o);
  return v < M ? v : M;
}

// Expert tile table, computed by every workgroup from the device offsets:
// b_e = min(M, max(0, offs[0..e])) (clamped monotone), tiles_e =
// ceil((b_{e+1} - b_e) / block_m), tile_start_e = sum of tiles before e.
// Returns the expert of global tile t (false past the last tile) and its rows.
__device__ bool tile_of(const int32_t* __restrict__ offs, int E, uint32_t M, int log_bm, uint32_t t, int& e_out,
                        uint32_t& r0, uint32_t& r1) {
  const int lane = threadIdx.x & 63;
  const uint32_t bm = 1u << log_bm;
  uint32_t run_b = clamp_off(offs[0], M);  // b of the first expert of the chunk
  uint32_t run_t = 0;                      // tiles before the chunk
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    // b_{e+1}: running max of the offsets (lanes past E repeat offs[E])
    const uint32_t b1 = umax(scan_max(clamp_off(offs[e < E ? e + 1 : E], M)), run_b);
    const uint32_t b0 = from_lane_below(b1, run_b);
    const uint32_t nt = (e < E && b1 > b0) ? (b1 - b0 + bm - 1) >> log_bm : 0u;
    const uint32_t incl = scan_add(nt);
    const uint32_t first = run_t + incl - nt;
    const uint64_t hit = __ballot(e < E && t >= first && t < first + nt);
    if (hit) {
      const int j = __builtin_ctzll(hit);
      e_out = e0 + j;
      r0 = lane_value(b0, j) + ((t - lane_value(first, j)) << log_bm);
      const uint32_t hi = lane_value(b1, j);
      r1 = r0 + bm < hi ? r0 + bm : hi;
      return true;
    }
    run_t += lane_value(incl, 63);
    run_b = lane_value(b1, 63);
  }
  return false;
}

// One row of a lane's CPL columns as CPL / 2 words (two bf16 each).
template <int CPL>
__device__ __forceinline__ void load_row(uint32_t (&w)[CPL / 2], const uint16_t* p) {
  if constexpr (CPL == 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (CPL == 4) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  } else {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  }
}

// Rows of one piece: a row at or past the tile's end r1 loads row `safe`
// (< r1; a whole piece can lie past r1) and is replaced by -0.0 when it is
// added.
template <int P, int CPL>
__device__ __forceinline__ void load_piece(uint32_t (&v)[P][CPL / 2], const uint16_t* __restrict__ dA, int64_t lda,
                                           int64_t a, int64_t r1, int64_t safe, int64_t col) {
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int64_t r = a + i < r1 ? a + i : safe;
    load_row<CPL>(v[i], dA + r * lda + col);
  }
}

// Adds the rows of piece p (rows p P .. p P + P - 1 of the wave's quarter) to
// the adjacent pairwise tree kept as a stack of partial sums: row i goes in
// as the right operand of every completed level (i's trailing one bits), so
// the stack ends holding exactly the tree of all Q rows.
template <int P, int LQ, int CPL>
__device__ __forceinline__ void push_piece(float (&stk)[LQ + 1][CPL], const uint32_t (&v)[P][CPL / 2], int p,
                                           int64_t a, int64_t r1) {
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int idx = p * P + i;
    const bool in = a + i < r1;  // wave-uniform
    float c[CPL];
#pragma unroll
    for (int k = 0; k < CPL / 2; ++k) {
      c[2 * k] = in ? bf16_lo(v[i][k]) : -0.0f;
      c[2 * k + 1] = in ? bf16_hi(v[i][k]) : -0.0f;
    }
    int l = 0;
#pragma unroll
    for (; l < LQ && ((idx >> l) & 1); ++l)
#pragma unroll
      for (int k = 0; k < CPL; ++k) c[k] = stk[l][k] + c[k];
#pragma unroll
    for (int k = 0; k < CPL; ++k) stk[l][k] = c[k];
  }
}

// Q rows per wave (block_m / 4), loaded and reduced in pieces of at most 32 rows.
template <int Q, int CPL, bool ATOMIC>
__global__ __launch_bounds__(256) void dbias_tile_kernel(const uint16_t* __restrict__ dA, int64_t lda, int64_t M,
                                                         int64_t N, const int32_t* __restrict__ offs, int E,
                                                         float* __restrict__ slots, int32_t* __restrict__ tstart,
                                                         float* __restrict__ dbias, int64_t ld_e, int ncb) {
  constexpr int BM = 4 * Q;
  constexpr int LOG_BM = BM == 64 ? 6 : (BM == 128 ? 7 : 8);
  static_assert((1 << LOG_BM) == BM, "block_m is 64, 128 or 256");
  constexpr int P = 16;  // rows per piece: the next piece's loads are in flight while one is added
  constexpr int NP = Q / P;
  constexpr int LQ = Q == 16 ? 4 : (Q == 32 ? 5 : 6);
  static_assert((1 << LQ) == Q && Q % P == 0, "Q is 16, 32 or 64");
  constexpr int kCols = 64 * CPL;
  const uint32_t Mu = static_cast<uint32_t>(M);
  __shared__ float part[4][kCols + 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the tile table for the fold: tile starts per expert (and the total),
  // written by the first workgroup whether or not any expert has rows
  // workgroup w: tile w / ncb, column block w % ncb (the column blocks of a
  // tile run side by side, so the workgroups in flight read whole rows)
  const uint32_t cb = blockIdx.x % ncb;
  if (!ATOMIC && blockIdx.x == 0 && wave == 0) {
    uint32_t run_b = 0, run_t = 0;
    for (int e0 = 0; e0 <= E; e0 += 64) {
      const int ee = e0 + lane;
      const uint32_t b = umax(scan_max(clamp_off(ee <= E ? offs[ee] : 0, Mu)), run_b);  // b_ee
      const uint32_t bp = from_lane_below(b, e0 == 0 ? b : run_b);                     // b_{ee-1}
      const uint32_t nt = (ee >= 1 && ee <= E && b > bp) ? (b - bp + BM - 1) / BM : 0u;  // tiles of expert ee-1
      const uint32_t incl = scan_add(nt);
      if (ee <= E) tstart[ee] = static_cast<int32_t>(run_t + incl);  // tiles of experts before ee
      run_t += lane_value(incl, 63);
      run_b = lane_value(b, 63);
    }
  }
  const uint32_t t = blockIdx.x / ncb;
  int e;
  uint32_t r0, r1;
  if (!tile_of(offs, E, Mu, LOG_BM, t, e, r0, r1)) return;  // past the last tile (the grid covers the worst case)
  const int64_t col = static_cast<int64_t>(cb) * kCols + CPL * lane;
  const bool live = col < N;  // N % 8 == 0: a lane's CPL columns are all inside or all outside
  float q[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) q[c] = -0.0f;
  const int64_t a0 = r0 + static_cast<int64_t>(wave) * Q;
  if (live && a0 < r1) {
    float stk[LQ + 1][CPL];
    uint32_t va[P][CPL / 2], vb[P][CPL / 2];
    load_piece<P, CPL>(va, dA, lda, a0, r1, a0, col);
#pragma unroll
    for (int p = 0; p < NP; p += 2) {
      if (p + 1 < NP) load_piece<P, CPL>(vb, dA, lda, a0 + (p + 1) * P, r1, a0, col);
      push_piece<P, LQ, CPL>(stk, va, p, a0 + p * P, r1);
      if (p + 1 < NP) {
        if (p + 2 < NP) load_piece<P, CPL>(va, dA, lda, a0 + (p + 2) * P, r1, a0, col);
        push_piece<P, LQ, CPL>(stk, vb, p + 1, a0 + (p + 1) * P, r1);
      }
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) q[c] = stk[LQ][c];
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) part[wave][CPL * lane + c] = q[c];
  __syncthreads();
  // the top two tree levels: thread i combines column i of the four quarters
  for (int i = threadIdx.x; i < kCols; i += 256) {
    const int64_t n = static_cast<int64_t>(cb) * kCols + i;
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
  // 32 slots' loads in flight at a time (an expert of 4096 rows has 32 tiles of 128)
  for (int64_t t = t0; t < t1; t += 32) {
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = t + i < t1 ? slots[(t + i) * N + n] : -0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) tot = tot + v[i];
  }
  float* const o = dbias + static_cast<int64_t>(e) * ld_e + n;
  *o = *o + tot;
}

int64_t max_tiles(int64_t M, int64_t E, int bm);

// block_n of the default configuration: the widest of 512, 256, 128 columns
// per workgroup that still gives 2048 workgroups (eight per compute unit), so
// that no compute unit holds a third more work than the average; 128 below.
int default_block_n(int64_t M, int64_t N, int64_t E) {
  for (int bn : {512, 256})
    if (max_tiles(M, E, 128) * ceil_div(N, bn) >= 2048) return bn;
  return 128;
}

int check_cfg(const det_dbias_cfg* cfg, det_dbias_cfg* out, int64_t M = 0, int64_t N = 0, int64_t E = 0) {
  det_dbias_cfg c{128, default_block_n(M, N, E)};
  if (cfg) c = *cfg;
  if (c.block_m != 64 && c.block_m != 128 && c.block_m != 256)
    return set_error(DET_ERR_INVALID_ARG, "dbias: block_m must be 64, 128 or 256, got %d", c.block_m);
  if (c.block_n != 128 && c.block_n != 256 && c.block_n != 512)
    return set_error(DET_ERR_INVALID_ARG, "dbias: block_n must be 128, 256 or 512, got %d", c.block_n);
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
  if (int s = check_cfg(cfg, &c, M, N, E)) return s;
  *bytes = (atomic || M == 0 || N == 0 || E == 0) ? 0 : ws_bytes_for(M, N, E, c.block_m);
  return ok();
}

extern "C" int det_grouped_dbias(float* dbias, int64_t ld_e, const void* dA, int64_t lda, int64_t M, int64_t N,
                                 const int32_t* offs, int32_t E, const det_dbias_cfg* cfg, void* ws, size_t ws_bytes,
                                 int atomic, void* stream) {
  if (int s = check_atomic_flag(atomic)) return s;
  if (M < 0 || N < 0 || E < 0) return set_error(DET_ERR_INVALID_ARG, "dbias: M, N and E must be >= 0");
  det_dbias_cfg c;
  if (int s = check_cfg(cfg, &c, M, N, E)) return s;
  if (M == 0 || N == 0 || E == 0) return ok();  // no rows or no columns: dbias unchanged
  if (!dbias || !dA || !offs) return set_error(DET_ERR_INVALID_ARG, "dbias: NULL pointer");
  if (M > 0x7FFFFFFF) return set_error(DET_ERR_UNSUPPORTED, "dbias: M must be < 2^31");
  if (lda < N || ld_e < N) return set_error(DET_ERR_INVALID_ARG, "dbias: lda and ld_e must be >= N");
  if (N % 8 || lda % 8 || !aligned(dA, 16))
    return set_error(DET_ERR_UNSUPPORTED, "dbias: N and lda must be multiples of 8 and dA 16-byte aligned");
  if (E > 65535) return set_error(DET_ERR_UNSUPPORTED, "dbias: E must be <= 65535");
  const int64_t nt = max_tiles(M, E, c.block_m);
  if (nt * ceil_div(N, c.block_n) > 0x7FFFFFFF || nt * N > (int64_t(1) << 40))
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
  const int ncb = static_cast<int>(ceil_div(N, c.block_n));
  const dim3 grid(static_cast<uint32_t>(nt * ncb));
#define DET_DBIAS_LAUNCH(Q, CPL)                                                                                  \
  if (c.block_m == 4 * Q && c.block_n == 64 * CPL) {                                                              \
    if (atomic)                                                                                                   \
      hipLaunchKernelGGL((dbias_tile_kernel<Q, CPL, true>), grid, dim3(256), 0, st, a, lda, M, N, offs, E, slots, \
                         tstart, dbias, ld_e, ncb);                                                               \
    else                                                                                                          \
      hipLaunchKernelGGL((dbias_tile_kernel<Q, CPL, false>), grid, dim3(256), 0, st, a, lda, M, N, offs, E,       \
                         slots, tstart, dbias, ld_e, ncb);                                                        \
  }
  DET_DBIAS_LAUNCH(16, 8) DET_DBIAS_LAUNCH(32, 8) DET_DBIAS_LAUNCH(64, 8)
  DET_DBIAS_LAUNCH(16, 4) DET_DBIAS_LAUNCH(32, 4) DET_DBIAS_LAUNCH(64, 4)
  DET_DBIAS_LAUNCH(16, 2) DET_DBIAS_LAUNCH(32, 2) DET_DBIAS_LAUNCH(64, 2)
#undef DET_DBIAS_LAUNCH
  if (!atomic)
    hipLaunchKernelGGL(dbias_fold_kernel, dim3(static_cast<uint32_t>(ceil_div(N, 256)), static_cast<uint32_t>(E)),
                       dim3(256), 0, st, slots, tstart, N, dbias, ld_e);
  return check_launch("det_grouped_dbias");
}
