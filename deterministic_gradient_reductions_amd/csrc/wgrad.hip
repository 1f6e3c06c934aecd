// det_grouped_wgrad_acc: main_grad[e] += G_e^T X_e with a fixed-order split-K
// (FlashInfer PR #8602: fused fp32 weight-gradient accumulate into main_grad;
// #8924: deterministic accumulate, bitwise the AccumulateGrad of the
// deterministic dW, with expert offsets read on the device).
//
// Contraction on the matrix cores (v_mfma_f32_32x32x16_bf16). G_e [T_e x M]
// and X_e [T_e x N] both have the token index as their row index, so the
// reduction runs down the rows of both operands, while the instruction wants
// each lane to hold 8 consecutive k values of one output row (A) or column
// (B). Each lane therefore holds 8 token rows x 4 consecutive columns (8 bytes
// per row; 32 lanes cover 128 contiguous columns) and transposes the 8 x 4
// block in registers with v_perm_b32. Fragment i (i = 0..3) then holds output
// rows m0 + 4r + i for lane slot r: one MFMA computes a strided 32 x 32
// sub-tile, and 4 x 4 MFMAs cover a wave's 128 x 128 output tile.
//
// Operand paths. A workgroup of W waves owns a 128 (m) x 128W (n) tile; wave
// w owns the n columns n0 + 128w. The G block is shared by all waves, so it is
// staged in LDS: 16-byte loads into registers three 32-row stages ahead, one
// 16-byte LDS write per lane and stage, three LDS stages. The X block of a
// wave is private to it, so it goes from global memory straight into
// registers, six 16-row blocks ahead. This keeps LDS traffic to the G operand
// alone (the LDS of one CU moves about 128 bytes per clock, less than both
// operands need at the matrix-core rate). All loads are ordinary loads whose
// waits the compiler places.
//
// Canonical order (the oracle's): an expert's rows are cut into splits of
// k_tile * ktiles_per_split rows counted from the expert's first row (one split
// when ktiles_per_split = 0). A split's partial is the chain of MFMAs over its
// rows in ascending 16-row blocks starting from +0.0 (rows past the split end
// are zero). With one split the epilogue adds the partial into main_grad
// directly; with several, each partial goes to scratch and a second kernel adds
// (((Q0 + Q1) + Q2) + ...) into main_grad once. The tile shape and the order
// in which workgroups take splits never change a bit.
//
// Scheduling. Experts differ in size, so splits are handed out largest expert
// first (ties by expert index): the hardware dispatches workgroups in index
// order to whichever CU frees up, which makes this a longest-job-first list
// schedule.
//
// The atomic arm adds every split's partial into main_grad with float atomics.
#include "common.hpp"

namespace detgrad {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 128;      // m columns of G per workgroup tile
constexpr int kWaveN = 128;   // n columns of X per wave
constexpr int kBlk = 16;      // token rows per MFMA block
constexpr int kStage = 32;    // token rows per LDS stage of G (two blocks)
constexpr int kAStages = 3;   // LDS stages of G
constexpr int kBSlots = 6;    // 16-row X blocks held in registers per wave
constexpr int kKTile = 512;
constexpr int kTileM = kBM;
constexpr int kXcds = 8;
constexpr int kRankMaxE = 63;  // experts are ordered by size when E <= 63

// Raw buffer descriptor word 3 of the gfx9 family (32-bit data format, no
// swizzle); the range check returns zeros past num_records bytes.
constexpr uint32_t kRsrcWord3 = 0x00020000u;

// Per-stage G: 32 rows x 128 columns x 2 bytes = 8 pieces of 1 KiB (4 rows of
// 256 bytes each; one 16-byte load per lane), shared out over the waves.
constexpr int kDmaA = kStage * kBM * 2 / 1024;
constexpr int kBLoads = 8;  // 8-byte X loads per lane per 16-row block

template <int W>
struct Shape {
  static constexpr int kThreads = 64 * W;
  static constexpr int kBN = kWaveN * W;
  static constexpr int kALoads = kDmaA / W;  // 16-byte G loads per lane and stage
  static_assert(kDmaA % W == 0, "G transfers must divide over the waves");
};

struct WgradArgs {
  float* mg;
  int64_t ld_e, ld_m;
  const uint16_t* G;
  int64_t ldg;
  const uint16_t* X;
  int64_t ldx;
  const int32_t* offs;
  int E;
  int T_total;
  int M, N;
  int split_rows;  // 0: one split per expert
  int tiles_m, tiles_n;
  int xcd_m, xcd_n;  // XCD cut of a split's tiles (0: plain order)
  int64_t n_units;
  float* scratch;   // [max_splits][M][N]
  int64_t max_splits;
  uint16_t* mg16;   // bf16 main_grad (the route where every split's partial goes to scratch)
};

// One split of one expert. Expert boundaries come from device offsets and are
// clamped monotone: b_e = clamp(offs[e], b_{e-1}, T_total), b_{-1} = 0.
struct Split {
  int e;
  int64_t g;        // natural split index (expert order, then split order): scratch slot
  int64_t n_split;  // splits of this expert
  int r0, r1;       // token rows [r0, r1)
};

__device__ __forceinline__ int clamp_i(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

__device__ __forceinline__ int splits_of(int te, int split_rows) {
  return te <= 0 ? 0 : (split_rows == 0 ? 1 : (te + split_rows - 1) / split_rows);
}

// Split q in natural order (experts ascending, splits ascending).
__device__ bool split_natural(const WgradArgs& p, int64_t q, Split& out) {
  int prev = clamp_i(p.offs[0], 0, p.T_total);
  int64_t cum = 0;
  for (int e = 0; e < p.E; ++e) {
    const int nb = clamp_i(p.offs[e + 1], prev, p.T_total);
    const int se = splits_of(nb - prev, p.split_rows);
    if (q < cum + se) {
      const int s = static_cast<int>(q - cum);
      out.e = e;
      out.g = q;
      out.n_split = se;
      out.r0 = p.split_rows == 0 ? prev : prev + s * p.split_rows;
      out.r1 = p.split_rows == 0 ? nb : (out.r0 + p.split_rows < nb ? out.r0 + p.split_rows : nb);
      return true;
    }
    cum += se;
    prev = nb;
  }
  return false;
}

// Split q in size order: experts by decreasing row count (ties by index), each
// expert's splits in ascending order. Lane e of the wave handles expert e.
__device__ bool split_by_size(const WgradArgs& p, int64_t q, Split& out) {
  if (p.E > kRankMaxE) return split_natural(p, q, out);
  const int lane = threadIdx.x & 63;
  const int E = p.E;
  // b_j = min(T, max(0, offs[0..j])) for j = 0..E (lanes 0..E)
  int b = lane <= E ? p.offs[lane] : 0;
  b = b < 0 ? 0 : b;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(b, d);
    if (lane >= d) b = b > t ? b : t;
  }
  b = b < p.T_total ? b : p.T_total;
  const int end = __shfl_down(b, 1);
  const int te = lane < E ? end - b : 0;
  const int se = lane < E ? splits_of(te, p.split_rows) : 0;
  // natural exclusive prefix of split counts (scratch slots)
  int gs = se;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(gs, d);
    if (lane >= d) gs += t;
  }
  gs -= se;
  // position of this expert's first split in the size order
  int pos = 0;
  for (int j = 0; j < E; ++j) {
    const int tj = __builtin_amdgcn_readlane(te, j);
    const int sj = __builtin_amdgcn_readlane(se, j);
    const bool before = tj > te || (tj == te && j < lane);
    pos += before ? sj : 0;
  }
  const bool mine = lane < E && se > 0 && q >= pos && q < pos + se;
  const uint64_t m = __ballot(mine);
  if (m == 0) return false;
  const int e = __builtin_ctzll(m);
  const int e_pos = __builtin_amdgcn_readlane(pos, e);
  const int e_b = __builtin_amdgcn_readlane(b, e);
  const int e_end = __builtin_amdgcn_readlane(end, e);
  const int s = static_cast<int>(q) - e_pos;
  out.e = e;
  out.g = static_cast<int64_t>(__builtin_amdgcn_readlane(gs, e)) + s;
  out.n_split = __builtin_amdgcn_readlane(se, e);
  out.r0 = p.split_rows == 0 ? e_b : e_b + s * p.split_rows;
  out.r1 = p.split_rows == 0 ? e_end : (out.r0 + p.split_rows < e_end ? out.r0 + p.split_rows : e_end);
  return true;
}

// MFMA operand of column c (0..3) of a lane's 8-row x 4-column block: dword q
// packs rows 2q (low 16 bits) and 2q+1 (high 16 bits) of that column.
template <int C>
__device__ __forceinline__ bf16x8_t frag(const u32x2_t* v) {
  constexpr uint32_t sel = (C & 1) ? 0x07060302u : 0x05040100u;
  u32x4_t d;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t lo = (C >> 1) ? v[2 * q].y : v[2 * q].x;
    const uint32_t hi = (C >> 1) ? v[2 * q + 1].y : v[2 * q + 1].x;
    d[q] = __builtin_amdgcn_perm(hi, lo, sel);
  }
  return __builtin_bit_cast(bf16x8_t, d);
}

typedef uint16_t StageA[kStage][kBM];

// This wave's pieces of G stage `st` (token rows 32 st ..): piece i covers
// rows 4i .. 4i+3; lane l loads row 4i + l/16, columns 8 (l % 16) .. + 7.
template <int W>
__device__ __forceinline__ void load_a(u32x4_t* v, __amdgpu_buffer_rsrc_t rsrc, int32_t voff, int32_t krow, int32_t st,
                                       int wave) {
#pragma unroll
  for (int u = 0; u < Shape<W>::kALoads; ++u) {
    const int i = wave * Shape<W>::kALoads + u;
    v[u] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, (st * kStage + 4 * i) * krow, 0);
  }
}

template <int W>
__device__ __forceinline__ void write_a(StageA& la, const u32x4_t* v, int lane, int wave) {
#pragma unroll
  for (int u = 0; u < Shape<W>::kALoads; ++u) {
    const int i = wave * Shape<W>::kALoads + u;
    *reinterpret_cast<u32x4_t*>(&la[4 * i + lane / 16][8 * (lane % 16)]) = v[u];
  }
}

// The 8 X rows of 16-row block `blk` this lane needs: rows 16 blk + 8 kg + e.
__device__ __forceinline__ void issue_b(u32x2_t* slot, __amdgpu_buffer_rsrc_t rsrc, int32_t voff, int32_t krow,
                                        int32_t blk) {
#pragma unroll
  for (int e = 0; e < kBLoads; ++e) slot[e] = __builtin_amdgcn_raw_buffer_load_b64(rsrc, voff, (blk * kBlk + e) * krow, 0);
}

// The G rows of one LDS stage this lane needs: rows 8 kg + e (block 0, into
// v[0..7]) and 16 + 8 kg + e (block 1, into v[8..15]), columns 4r .. 4r+3.
__device__ __forceinline__ void read_a(const StageA& la, int r, int kg, u32x2_t* v) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    v[e] = *reinterpret_cast<const u32x2_t*>(&la[8 * kg + e][4 * r]);
    v[8 + e] = *reinterpret_cast<const u32x2_t*>(&la[16 + 8 * kg + e][4 * r]);
  }
}

// Pin the use of an X slot to this point of the program: volatile asm keeps
// its place among the pipeline's other volatile asm (the stage syncs), so the
// transposes and MFMAs that read the slot cannot be hoisted ahead of the stage
// they belong to, and the compiler's wait for the slot's loads lands here.
__device__ __forceinline__ void pin(u32x2_t* v) {
#pragma unroll
  for (int e = 0; e < kBLoads; ++e) asm volatile("" : "+v"(v[e]));
}

__device__ __forceinline__ void mma_block(const u32x2_t* a, const u32x2_t* b, f32x16_t (&acc)[4][4]) {
  const bf16x8_t fa[4] = {frag<0>(a), frag<1>(a), frag<2>(a), frag<3>(a)};
  const bf16x8_t fb[4] = {frag<0>(b), frag<1>(b), frag<2>(b), frag<3>(b)};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
}

// XCD-aware placement. Workgroups are dispatched to the 8 XCDs round-robin
// (workgroup u runs on XCD u % 8), and each XCD has its own L2. The tiles of
// every split are cut into 8 rectangles, xcd_m (m-parts) x xcd_n (n-parts),
// one per XCD; the host picks the cut that minimises the G and X bytes per
// token row one XCD reads (its m-range of G plus its n-range of X), since the
// workgroups of one rectangle share those rows through their XCD's L2. XCD x
// takes its rectangle's tiles split after split, so every XCD gets the same
// share of every split and the XCDs stay balanced.
__device__ __forceinline__ bool unit_of(const WgradArgs& p, uint32_t u, int64_t& q, int& mt, int& nt) {
  if (p.xcd_m > 0) {
    const int x = static_cast<int>(u % kXcds);
    const int64_t slot = u / kXcds;
    const int xm = x / p.xcd_n, xn = x % p.xcd_n;
    const int mlo = xm * p.tiles_m / p.xcd_m, mhi = (xm + 1) * p.tiles_m / p.xcd_m;
    const int nlo = xn * p.tiles_n / p.xcd_n, nhi = (xn + 1) * p.tiles_n / p.xcd_n;
    const int per = (mhi - mlo) * (nhi - nlo);
    if (per == 0) return false;
    q = slot / per;
    if (q >= p.max_splits) return false;
    const int t = static_cast<int>(slot % per);
    mt = mlo + t / (nhi - nlo);
    nt = nlo + t % (nhi - nlo);
    return true;
  }
  // fewer tiles than XCDs: plain split-major order
  const int64_t tiles = static_cast<int64_t>(p.tiles_m) * p.tiles_n;
  q = static_cast<int64_t>(u) / tiles;
  if (q >= p.max_splits) return false;
  const int t = static_cast<int>(static_cast<int64_t>(u) % tiles);
  mt = t / p.tiles_n;
  nt = t % p.tiles_n;
  return true;
}

// Host: choose the XCD cut and the grid size.
__host__ void plan_xcds(WgradArgs& p, int block_m, int block_n) {
  p.xcd_m = 0;
  p.xcd_n = 0;
  int64_t best = -1;
  for (int pm = 1; pm <= kXcds; pm *= 2) {
    const int pn = kXcds / pm;
    if (pm > p.tiles_m || pn > p.tiles_n) continue;
    const int64_t bytes = static_cast<int64_t>((p.tiles_m + pm - 1) / pm) * block_m * 2 +
                          static_cast<int64_t>((p.tiles_n + pn - 1) / pn) * block_n * 2;
    if (best < 0 || bytes < best) {
      best = bytes;
      p.xcd_m = pm;
      p.xcd_n = pn;
    }
  }
  if (p.xcd_m > 0) {
    int per_max = 0;
    for (int x = 0; x < kXcds; ++x) {
      const int xm = x / p.xcd_n, xn = x % p.xcd_n;
      const int per = ((xm + 1) * p.tiles_m / p.xcd_m - xm * p.tiles_m / p.xcd_m) *
                      ((xn + 1) * p.tiles_n / p.xcd_n - xn * p.tiles_n / p.xcd_n);
      per_max = per > per_max ? per : per_max;
    }
    p.n_units = static_cast<int64_t>(kXcds) * per_max * p.max_splits;
  } else {
    p.n_units = static_cast<int64_t>(p.tiles_m) * p.tiles_n * p.max_splits;
  }
}

// One workgroup = W waves = a 128 (m) x 128W (n) output tile; wave w owns the
// 128 x 128 columns n0 + 128w.
//
// Pipeline per stage s (blocks 2s and 2s+1):
//   block 2s:    MFMAs on G rows of stage s (registers) and X block 2s (slot),
//                then X block 2s+6 into the freed slot
//   G stage s+1: registers -> LDS stage (s+1) % 3; barrier
//   G stage s+4: global -> the registers that stage s+1 came through
//   G stage s+1: LDS -> registers
//   block 2s+1:  MFMAs, then X block 2s+7 into the freed slot
// The LDS stage written at stage s was last read at stage s-3, before two
// barriers, and every LDS read of a stage follows the barrier after its write.
// ALLS: every split's partial goes to scratch, also a lone split (the bf16
// main_grad route); a template flag, so the other instances are unchanged.
template <int W, bool ATOMIC, bool ALLS = false>
__global__ __launch_bounds__(64 * W) void wgrad_kernel(WgradArgs p) {
  __shared__ __attribute__((aligned(16))) StageA la[kAStages];
  int64_t uq;
  int mt, nt;
  if (!unit_of(p, blockIdx.x, uq, mt, nt)) return;
  Split sp;
  if (!split_by_size(p, uq, sp)) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int m0 = mt * kBM;
  const int n0 = nt * Shape<W>::kBN;
  const int r = lane & 31;
  const int kg = lane >> 5;

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int c = 0; c < 16; ++c) acc[i][j][c] = 0.0f;

  // Buffer resources cover the split's rows only: rows past its end read as
  // zero, which is the zero padding of the last block.
  const int32_t rows = sp.r1 - sp.r0;
  const int32_t krow_a = static_cast<int32_t>(p.ldg * 2);
  const int32_t krow_b = static_cast<int32_t>(p.ldx * 2);
  const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.G + static_cast<int64_t>(sp.r0) * p.ldg), 0, rows * krow_a, static_cast<int>(kRsrcWord3));
  const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.X + static_cast<int64_t>(sp.r0) * p.ldx), 0, rows * krow_b, static_cast<int>(kRsrcWord3));
  const int32_t voff_a = (lane / 16) * krow_a + (m0 + (lane % 16) * 8) * 2;
  const int32_t voff_b = 8 * kg * krow_b + (n0 + kWaveN * wave + 4 * r) * 2;

  u32x2_t bq[kBSlots][kBLoads];
  u32x4_t ga[kAStages][Shape<W>::kALoads];
  u32x2_t ra[16];

  // prologue: G stages 0..2 and X blocks 0..5 in flight; G stage 0 to LDS,
  // and its registers take G stage 3 (register set k holds the G stages
  // congruent to k mod 3)
  load_a<W>(ga[0], rsrc_a, voff_a, krow_a, 0, wave);
#pragma unroll
  for (int b = 0; b < kBSlots; ++b) {
    issue_b(bq[b], rsrc_b, voff_b, krow_b, b);
    if (b == 1) load_a<W>(ga[1], rsrc_a, voff_a, krow_a, 1, wave);
    if (b == 3) load_a<W>(ga[2], rsrc_a, voff_a, krow_a, 2, wave);
  }
  write_a<W>(la[0], ga[0], lane, wave);
  __syncthreads();
  load_a<W>(ga[0], rsrc_a, voff_a, krow_a, kAStages, wave);
  read_a(la[0], r, kg, ra);

  // Three stages per iteration, so that every LDS stage and register slot is
  // a compile-time index. Whole iterations (6 blocks inside the split) run
  // without any branch between their MFMA blocks; the last, partial iteration
  // runs the same stages with each MFMA block guarded. Every stage issues its
  // loads even past the split end (those read zeros), so all paths through the
  // loop issue the same loads and the compiler's waits stay loose.
#define DET_WGRAD_STAGE(SI, GUARD)                                                         \
  {                                                                                        \
    const int32_t s = s0 + (SI);                                                           \
    pin(bq[(2 * (SI)) % kBSlots]);                                                         \
    if (!(GUARD) || s * kStage < rows) mma_block(&ra[0], bq[(2 * (SI)) % kBSlots], acc);   \
    issue_b(bq[(2 * (SI)) % kBSlots], rsrc_b, voff_b, krow_b, 2 * s + 6);                  \
    write_a<W>(la[((SI) + 1) % kAStages], ga[((SI) + 1) % kAStages], lane, wave);          \
    __syncthreads();                                                                       \
    load_a<W>(ga[((SI) + 1) % kAStages], rsrc_a, voff_a, krow_a, s + 1 + kAStages, wave);  \
    u32x2_t rn[16];                                                                        \
    read_a(la[((SI) + 1) % kAStages], r, kg, rn);                                          \
    pin(bq[(2 * (SI) + 1) % kBSlots]);                                                     \
    if (!(GUARD) || s * kStage + kBlk < rows) mma_block(&ra[8], bq[(2 * (SI) + 1) % kBSlots], acc); \
    issue_b(bq[(2 * (SI) + 1) % kBSlots], rsrc_b, voff_b, krow_b, 2 * s + 7);              \
    _Pragma("unroll") for (int v = 0; v < 16; ++v) ra[v] = rn[v];                          \
  }
  int32_t s0 = 0;
  for (; (s0 + 3) * kStage <= rows; s0 += 3) {
    DET_WGRAD_STAGE(0, false)
    DET_WGRAD_STAGE(1, false)
    DET_WGRAD_STAGE(2, false)
  }
  if (s0 * kStage < rows) {
    DET_WGRAD_STAGE(0, true)
    DET_WGRAD_STAGE(1, true)
    DET_WGRAD_STAGE(2, true)
  }
#undef DET_WGRAD_STAGE

  // Epilogue: lane (r, kg), MFMA (i, j), accumulator q holds output
  // m = m0 + 4 * (8*(q/4) + 4*kg + q%4) + i,  n = n0 + 128*wave + 4*r + j.
  const bool direct = sp.n_split == 1 && !ALLS;
  float* dst_base;
  int64_t ld_m;
  if (ATOMIC || direct) {
    dst_base = p.mg + sp.e * p.ld_e;
    ld_m = p.ld_m;
  } else {
    dst_base = p.scratch + sp.g * static_cast<int64_t>(p.M) * p.N;
    ld_m = p.N;
  }
  const int nc = n0 + kWaveN * wave + 4 * r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int m = m0 + 4 * (8 * (q / 4) + 4 * kg + (q % 4)) + i;
      float* d = dst_base + static_cast<int64_t>(m) * ld_m + nc;
      const float v0 = acc[i][0][q], v1 = acc[i][1][q], v2 = acc[i][2][q], v3 = acc[i][3][q];
      if (ATOMIC) {
        unsafeAtomicAdd(d + 0, v0);
        unsafeAtomicAdd(d + 1, v1);
        unsafeAtomicAdd(d + 2, v2);
        unsafeAtomicAdd(d + 3, v3);
      } else if (direct) {
        float4 o = *reinterpret_cast<const float4*>(d);
        o.x = o.x + v0; o.y = o.y + v1; o.z = o.z + v2; o.w = o.w + v3;
        *reinterpret_cast<float4*>(d) = o;
      } else {
        *reinterpret_cast<float4*>(d) = make_float4(v0, v1, v2, v3);
      }
      // keep the scheduler from hoisting every read-modify-write of the
      // epilogue at once (that would need hundreds of registers)
      if (q % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ---------------------------------------------------------------------------
// 256 x 256 workgroup tile, operands transposed on their way into LDS.
//
// Four waves in a 2 x 2 arrangement each own a 128 x 128 quarter, so every G
// column block and every X column block feeds two waves. A stage is 64 token
// rows. Each of the 256 lanes loads an 8-row x 8-column block of G and one of
// X (eight 16-byte loads each), turns each block around in registers with
// v_perm_b32 into eight 16-byte vectors (8 consecutive token rows of one
// column: exactly what one MFMA operand lane holds), and stores the vectors to
// LDS with 16-byte writes. Every MFMA fragment is then a single 16-byte LDS
// read per lane. Plain 16-byte LDS reads are the fastest LDS access on gfx950
// (the transposing 8-byte read moves less than half as many bytes per clock),
// and a 128 x 128 wave tile needs 64 bytes per clock per CU of fragment reads
// at the matrix-core rate.
//
// LDS layout of one operand and stage: [k-group 8][column 256][8 rows] bf16,
// the vector of column c stored at slot c ^ (((c >> 4) ^ ((c >> 1) & 4)) & 7)
// (a permutation of the low three bits of c inside each group of 8). Every 8
// consecutive lanes of a store (columns 8 apart) and of a fragment read (32
// consecutive columns) then cover 8 distinct 16-byte bank groups, and every 16
// consecutive lanes 16 distinct ones, so neither access has bank conflicts
// whether the LDS serves a 16-byte access 8 or 16 lanes per pass.
//
// Pipeline: two LDS buffers per operand. While the MFMAs of stage s run from
// one buffer, the loads of stage s+1 (issued right after the previous
// barrier) land in registers, are transposed and written to the other buffer
// after the stage's second block; one barrier per stage.
constexpr int kTT = 256;                 // tile edge (m and n)
constexpr int kTRows = 64;               // token rows per stage
constexpr int kTGroups = kTRows / 8;     // 8-row k-groups per stage
constexpr int kTGroupBytes = kTT * 16;   // bytes of one k-group of one operand
typedef uint32_t TStage[kTGroups][kTT][4];  // 32 KiB

__device__ __forceinline__ int tslot(int c) { return c ^ (((c >> 4) ^ ((c >> 1) & 4)) & 7); }

// Stage s of one operand: lane rows 8 rg .. 8 rg + 7 (relative to the split
// start), columns 8 c8 .. 8 c8 + 7 of the tile (voff holds both).
__device__ __forceinline__ void t_load(u32x4_t (&v)[8], __amdgpu_buffer_rsrc_t rsrc, int32_t voff, int32_t krow,
                                       int32_t s) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    v[e] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, (s * kTRows + e) * krow, 0));
}

// v[e] holds row e, dword q = columns 2q (low half) and 2q + 1 (high half).
// Column i's vector: dword q = rows 2q (low half) and 2q + 1 (high half).
__device__ __forceinline__ void t_store(TStage& st, const u32x4_t (&v)[8], int rg, int c8) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
    u32x4_t o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = __builtin_amdgcn_perm(v[2 * q + 1][i >> 1], v[2 * q][i >> 1], sel);
    *reinterpret_cast<u32x4_t*>(&st[rg][tslot(8 * c8 + i)][0]) = o;
  }
}

struct TFrag {
  bf16x8_t a[4];
  bf16x8_t b[4];
};

// Fragments of 16-row block `blk` of the stage pair at `base` (A at base,
// B one stage further): lane (r, kg) reads k-group 2 blk + kg of columns
// 32 i + r of its quarter (offsets precomputed, B's include the stage size).
__device__ __forceinline__ void t_frag(const char* base, int blk, const int (&oa)[4], const int (&ob)[4], TFrag& f) {
  const char* pb = base + blk * 2 * kTGroupBytes;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.a[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(pb + oa[i]));
    f.b[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(pb + ob[i]));
  }
}

__device__ __forceinline__ void t_mma(const TFrag& f, f32x16_t (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// Epilogue of one wave: lane (r, kg), MFMA (i, j), accumulator c holds output
// row m = mw + 32 i + 8 (c/4) + 4 kg + c%4 and column n = nw + 32 j + r, so a
// wave instruction covers two 128-byte row segments. MODE 0 adds into the
// destination (one rounding per element), 1 stores, 2 adds with float
// atomics. Each quarter i moves 64 values per lane with all loads in flight.
template <int MODE>
__device__ __forceinline__ void t_epilogue(float* dst, int64_t ld, int mw, int nw, int r, int kg,
                                           const f32x16_t (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float* row0 = dst + static_cast<int64_t>(mw + 32 * i + 4 * kg) * ld + nw + r;
    if (MODE == 0) {
      float v[16][4];
#pragma unroll
      for (int c = 0; c < 16; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) v[c][j] = row0[static_cast<int64_t>(8 * (c / 4) + (c % 4)) * ld + 32 * j];
#pragma unroll
      for (int c = 0; c < 16; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          row0[static_cast<int64_t>(8 * (c / 4) + (c % 4)) * ld + 32 * j] = v[c][j] + acc[i][j][c];
    } else {
#pragma unroll
      for (int c = 0; c < 16; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float* d = row0 + static_cast<int64_t>(8 * (c / 4) + (c % 4)) * ld + 32 * j;
          if (MODE == 1)
            *d = acc[i][j][c];
          else
            unsafeAtomicAdd(d, acc[i][j][c]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Transpose and store column i (0..7) of a lane's 8 x 8 block into the stage
// at `st` (see t_store).
__device__ __forceinline__ void t_store_col(char* st, const u32x4_t (&v)[8], int rg, int c8, int i) {
  const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
  u32x4_t o;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = __builtin_amdgcn_perm(v[2 * q + 1][i >> 1], v[2 * q][i >> 1], sel);
  *reinterpret_cast<u32x4_t*>(st + (rg * kTT + tslot(8 * c8 + i)) * 16) = o;
}

// Fragment q of block `blk` (q < 4: A fragment q, else B fragment q - 4).
__device__ __forceinline__ void t_frag1(const char* base, int blk, const int (&oa)[4], const int (&ob)[4], int q,
                                        TFrag& f) {
  const char* pb = base + blk * 2 * kTGroupBytes;
  if (q < 4)
    f.a[q] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(pb + oa[q]));
  else
    f.b[q - 4] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(pb + ob[q - 4]));
}

__device__ __forceinline__ void t_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
}

template <bool ATOMIC, bool ALLS = false>
__global__ __launch_bounds__(256) void wgrad_tl_kernel(WgradArgs p) {
  // [stage buffer 2][operand 2]: A (G) of buffer b at 2b, B (X) at 2b + 1
  __shared__ __attribute__((aligned(16))) TStage lds[4];
  int64_t uq;
  int mt, nt;
  if (!unit_of(p, blockIdx.x, uq, mt, nt)) return;
  Split sp;
  if (!split_by_size(p, uq, sp)) return;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = mt * kTT, n0 = nt * kTT;
  // M is a multiple of 128, so a wave's 128 rows are all inside or all
  // outside M; a wave outside stores nothing.
  const bool live = m0 + 128 * wm < p.M;

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int c = 0; c < 16; ++c) acc[i][j][c] = 0.0f;

  // Buffer resources cover the split's rows only: rows past its end read as
  // zero (the zero padding of the last block). G columns past M (the last
  // m tile when M % 256 == 128) read the next row or zero and only feed the
  // waves that are not live.
  const int32_t rows = sp.r1 - sp.r0;
  const int32_t krow_a = static_cast<int32_t>(p.ldg * 2);
  const int32_t krow_b = static_cast<int32_t>(p.ldx * 2);
  const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.G + static_cast<int64_t>(sp.r0) * p.ldg), 0, rows * krow_a, static_cast<int>(kRsrcWord3));
  const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.X + static_cast<int64_t>(sp.r0) * p.ldx), 0, rows * krow_b, static_cast<int>(kRsrcWord3));
  const int c8 = t & 31, rg = t >> 5;
  const int32_t voff_a = rg * 8 * krow_a + (m0 + 8 * c8) * 2;
  const int32_t voff_b = rg * 8 * krow_b + (n0 + 8 * c8) * 2;
  const int r = lane & 31, kg = lane >> 5;
  int oa[4], ob[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    oa[i] = kg * kTGroupBytes + tslot(128 * wm + 32 * i + r) * 16;
    ob[i] = static_cast<int>(sizeof(TStage)) + kg * kTGroupBytes + tslot(128 * wn + 32 * i + r) * 16;
  }
  char* const lbase = reinterpret_cast<char*>(&lds[0][0][0][0]);
  constexpr int kPair = 2 * static_cast<int>(sizeof(TStage));
  constexpr int kOpB = static_cast<int>(sizeof(TStage));

  // Stage k's rows live in register set k & 1 from their loads until their
  // transposition, which happens during stage k - 1: loads are issued about
  // two stages ahead of their use.
  u32x4_t ra[2][8], rb[2][8];
  t_load(ra[0], rsrc_a, voff_a, krow_a, 0);
  t_load(rb[0], rsrc_b, voff_b, krow_b, 0);
  t_load(ra[1], rsrc_a, voff_a, krow_a, 1);
  t_load(rb[1], rsrc_b, voff_b, krow_b, 1);
  t_store(lds[0], ra[0], rg, c8);
  t_store(lds[1], rb[0], rg, c8);
  t_load(ra[0], rsrc_a, voff_a, krow_a, 2);
  t_load(rb[0], rsrc_b, voff_b, krow_b, 2);
  __syncthreads();

  TFrag fb[2];
  t_frag(lbase, 0, oa, ob, fb[0]);

  // Full stages (all four blocks inside the split). The 64 MFMAs of stage s
  // are issue slots k = 0..63 (block k / 16, MFMA (i, j) = (k % 16 / 4,
  // k % 4)); the other work of the stage is spread over them so that the
  // matrix pipe never waits for it:
  //   slots 16b .. 16b+7 (b < 3): the 8 fragments of block b + 1
  //   odd slots 1 .. 15: G columns of stage s + 1 (registers) -> the other
  //                      buffer (every wave finished reading it before the
  //                      previous barrier); odd slots 17 .. 31: X columns
  //   slots 16, 20, .. 44: G loads of stage s + 3 into the registers just
  //                        freed; slots 34, 38, .. 62: X loads (one load
  //                        per two slots, so the memory pipe never backs up
  //                        into the instruction stream)
  //   slot 51: barrier (every wave has written the other buffer and read
  //            the last fragments of this one)
  //   slots 52 .. 59: the fragments of block 0 of stage s + 1
  // Scheduling fences between slots keep this order.
#define DET_WGRAD_T_STAGE(P, MMA)                                                                               \
  {                                                                                                             \
    const int cur = (P) * kPair;                                                                                \
    const int nxt = kPair - cur;                                                                                \
    _Pragma("unroll") for (int k = 0; k < 64; ++k) {                                                            \
      const int b = k / 16, q = k % 16;                                                                         \
      if (MMA)                                                                                                  \
        acc[q / 4][q % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[b & 1].a[q / 4], fb[b & 1].b[q % 4],     \
                                                                    acc[q / 4][q % 4], 0, 0, 0);                \
      if (b < 3 && q < 8) t_frag1(lbase + cur, b + 1, oa, ob, q, fb[(b + 1) & 1]);                              \
      if (k < 16 && (k & 1)) t_store_col(lbase + nxt, ra[(P) ^ 1], rg, c8, k >> 1);                            \
      if (k >= 16 && k < 32 && (k & 1)) t_store_col(lbase + nxt + kOpB, rb[(P) ^ 1], rg, c8, (k - 16) >> 1);   \
      if (k >= 16 && k < 48 && (k % 4) == 0)                                                                    \
        ra[(P) ^ 1][(k - 16) / 4] = __builtin_bit_cast(                                                         \
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc_a, voff_a, ((s + 3) * kTRows + (k - 16) / 4) * krow_a, 0)); \
      if (k >= 34 && (k % 4) == 2)                                                                              \
        rb[(P) ^ 1][(k - 34) / 4] = __builtin_bit_cast(                                                         \
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc_b, voff_b, ((s + 3) * kTRows + (k - 34) / 4) * krow_b, 0)); \
      if (k == 51) t_sync();                                                                                    \
      if (k >= 52 && k < 60) t_frag1(lbase + nxt, 0, oa, ob, k - 52, fb[0]);                                    \
      __builtin_amdgcn_sched_barrier(0);                                                                        \
    }                                                                                                           \
    ++s;                                                                                                        \
  }
  // A wave past M (the second half of the last m tile when M % 256 == 128)
  // runs the same stages without MFMAs: it still moves its share of both
  // operands and meets every barrier.
  int s = 0;
  const int full = rows / kTRows;
  if (live) {
    while (s + 1 < full) {
      DET_WGRAD_T_STAGE(0, true)
      DET_WGRAD_T_STAGE(1, true)
    }
    if (s < full) DET_WGRAD_T_STAGE(0, true)
  } else {
    while (s + 1 < full) {
      DET_WGRAD_T_STAGE(0, false)
      DET_WGRAD_T_STAGE(1, false)
    }
    if (s < full) DET_WGRAD_T_STAGE(0, false)
  }
#undef DET_WGRAD_T_STAGE
  // Last, partial stage: blocks inside the split only.
  if (live && s * kTRows < rows) {
    const int cur = (s & 1) * kPair;
    const int nb = (rows - s * kTRows + kBlk - 1) / kBlk;
    t_mma(fb[0], acc);
    if (nb > 1) { t_frag(lbase + cur, 1, oa, ob, fb[1]); t_mma(fb[1], acc); }
    if (nb > 2) { t_frag(lbase + cur, 2, oa, ob, fb[0]); t_mma(fb[0], acc); }
    if (nb > 3) { t_frag(lbase + cur, 3, oa, ob, fb[1]); t_mma(fb[1], acc); }
  }
  if (!live) return;

  const int mw = m0 + 128 * wm, nw = n0 + 128 * wn;
  if (ATOMIC) {
    t_epilogue<2>(p.mg + sp.e * p.ld_e, p.ld_m, mw, nw, r, kg, acc);
  } else if (sp.n_split == 1 && !ALLS) {
    t_epilogue<0>(p.mg + sp.e * p.ld_e, p.ld_m, mw, nw, r, kg, acc);
  } else {
    t_epilogue<1>(p.scratch + sp.g * static_cast<int64_t>(p.M) * p.N, p.N, mw, nw, r, kg, acc);
  }
}

// Fold of multi-split experts: main_grad[e] += ((Q0 + Q1) + ...) elementwise.
__global__ __launch_bounds__(256) void wgrad_fold_kernel(WgradArgs p) {
  const int64_t per_e = static_cast<int64_t>(p.M) * p.N / 4;  // float4 per expert
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int e = static_cast<int>(blockIdx.y);
  if (idx >= per_e) return;
  // locate expert e's splits (same clamping as the matrix kernel)
  int64_t prev = p.offs[0];
  prev = prev < 0 ? 0 : (prev > p.T_total ? p.T_total : prev);
  int64_t g0 = 0, se = 0;
  for (int x = 0; x <= e; ++x) {
    int64_t nb = p.offs[x + 1];
    nb = nb < prev ? prev : (nb > p.T_total ? p.T_total : nb);
    const int64_t te = nb - prev;
    const int64_t s = te == 0 ? 0 : (te + p.split_rows - 1) / p.split_rows;
    if (x < e) g0 += s; else se = s;
    prev = nb;
  }
  if (se < 2) return;
  const int64_t m = (idx * 4) / p.N;
  const int64_t n = (idx * 4) % p.N;
  float4 tot = make_float4(-0.0f, -0.0f, -0.0f, -0.0f);
  for (int64_t s = 0; s < se; ++s) {
    const float4 q = *reinterpret_cast<const float4*>(p.scratch + (g0 + s) * static_cast<int64_t>(p.M) * p.N + m * p.N + n);
    tot.x = tot.x + q.x; tot.y = tot.y + q.y; tot.z = tot.z + q.z; tot.w = tot.w + q.w;
  }
  float* d = p.mg + e * p.ld_e + m * p.ld_m + n;
  float4 o = *reinterpret_cast<const float4*>(d);
  o.x = o.x + tot.x; o.y = o.y + tot.y; o.z = o.z + tot.z; o.w = o.w + tot.w;
  *reinterpret_cast<float4*>(d) = o;
}

// bf16 main_grad: dW = ((Q0 + Q1) + ...) in float32, rounded to bf16 (nearest
// even), added to main_grad in float32 and the sum rounded to bf16: the bf16
// tensor add of the bf16 dW. Experts with no rows are left untouched.
__device__ __forceinline__ uint32_t rne_bf16(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u & 0x7FFFFFFFu) > 0x7F800000u ? ((u >> 16) | 0x40u) & 0xFFFFu : ((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ uint32_t add_bf16(uint32_t m, float dw) {
  const float d16 = __uint_as_float(rne_bf16(dw) << 16);
  return rne_bf16(__uint_as_float(m << 16) + d16);
}

__global__ __launch_bounds__(256) void wgrad_fold_bf16_kernel(WgradArgs p) {
  const int64_t per_e = static_cast<int64_t>(p.M) * p.N / 4;  // 4 values per thread
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int e = static_cast<int>(blockIdx.y);
  if (idx >= per_e) return;
  int64_t prev = p.offs[0];
  prev = prev < 0 ? 0 : (prev > p.T_total ? p.T_total : prev);
  int64_t g0 = 0, se = 0;
  for (int x = 0; x <= e; ++x) {
    int64_t nb = p.offs[x + 1];
    nb = nb < prev ? prev : (nb > p.T_total ? p.T_total : nb);
    const int64_t te = nb - prev;
    const int64_t s = te == 0 ? 0 : (p.split_rows == 0 ? 1 : (te + p.split_rows - 1) / p.split_rows);
    if (x < e) g0 += s; else se = s;
    prev = nb;
  }
  if (se == 0) return;
  const int64_t m = (idx * 4) / p.N;
  const int64_t n = (idx * 4) % p.N;
  float4 tot = make_float4(-0.0f, -0.0f, -0.0f, -0.0f);
  for (int64_t s = 0; s < se; ++s) {
    const float4 q = *reinterpret_cast<const float4*>(p.scratch + (g0 + s) * static_cast<int64_t>(p.M) * p.N + m * p.N + n);
    tot.x = tot.x + q.x; tot.y = tot.y + q.y; tot.z = tot.z + q.z; tot.w = tot.w + q.w;
  }
  uint2* const d = reinterpret_cast<uint2*>(p.mg16 + e * p.ld_e + m * p.ld_m + n);
  const uint2 o = *d;
  uint2 r;
  r.x = add_bf16(o.x & 0xFFFFu, tot.x) | add_bf16(o.x >> 16, tot.y) << 16;
  r.y = add_bf16(o.y & 0xFFFFu, tot.z) | add_bf16(o.y >> 16, tot.w) << 16;
  *d = r;
}

int resolve(const det_wgrad_cfg* cfg, det_wgrad_cfg* out) {
  det_wgrad_cfg c{kTT, kTT, kKTile, 0};
  if (cfg) c = *cfg;
  const bool shape_ok = (c.block_m == 128 && (c.block_n == 256 || c.block_n == 512)) ||
                        (c.block_m == kTT && c.block_n == kTT);
  if (!shape_ok)
    return set_error(DET_ERR_UNSUPPORTED, "wgrad: block_m x block_n must be 128 x 256, 128 x 512 or 256 x 256, got %d x %d",
                     c.block_m, c.block_n);
  if (c.k_tile != kKTile) return set_error(DET_ERR_INVALID_ARG, "wgrad: k_tile must be %d, got %d", kKTile, c.k_tile);
  if (c.ktiles_per_split < 0 || c.ktiles_per_split > (1 << 20))
    return set_error(DET_ERR_INVALID_ARG, "wgrad: ktiles_per_split must be in [0, 2^20], got %d", c.ktiles_per_split);
  *out = c;
  return DET_OK;
}

int check_shape(int64_t T_total, int32_t E, int64_t M, int64_t N, const det_wgrad_cfg& c) {
  if (T_total < 0 || E < 0 || M < 0 || N < 0) return set_error(DET_ERR_INVALID_ARG, "wgrad: sizes must be >= 0");
  if (M % kTileM || N % c.block_n)
    return set_error(DET_ERR_UNSUPPORTED, "wgrad: M and N must be multiples of %d and %d, got %lld x %lld", kTileM,
                     c.block_n, static_cast<long long>(M), static_cast<long long>(N));
  if (M > (1 << 20) || N > (1 << 20) || E > 4096) return set_error(DET_ERR_UNSUPPORTED, "wgrad: problem too large");
  if (T_total >= (1LL << 30)) return set_error(DET_ERR_UNSUPPORTED, "wgrad: T_total too large");
  return DET_OK;
}

int64_t max_splits(int64_t T_total, int32_t E, const det_wgrad_cfg& c) {
  if (c.ktiles_per_split == 0) return E;
  const int64_t step = static_cast<int64_t>(c.k_tile) * c.ktiles_per_split;
  return ceil_div(T_total, step) + E;
}

size_t scratch_bytes(int64_t T_total, int32_t E, int64_t M, int64_t N, const det_wgrad_cfg& c) {
  if (c.ktiles_per_split == 0) return 0;  // one split per expert: partials stay in registers
  return static_cast<size_t>(max_splits(T_total, E, c)) * static_cast<size_t>(M * N) * 4;
}

// Every split's partial in scratch (the bf16 main_grad route), also with one split per expert.
size_t scratch_bytes_all(int64_t T_total, int32_t E, int64_t M, int64_t N, const det_wgrad_cfg& c) {
  if (T_total == 0 || E == 0 || M == 0 || N == 0) return 0;
  return static_cast<size_t>(max_splits(T_total, E, c)) * static_cast<size_t>(M * N) * 4;
}

}  // namespace
}  // namespace detgrad

using namespace detgrad;

extern "C" int det_grouped_wgrad_acc_workspace_size(int64_t T_total, int32_t E, int64_t M, int64_t N,
                                                    const det_wgrad_cfg* cfg, int atomic, size_t* bytes) {
  if (int s = check_atomic_flag(atomic)) return s;
  if (!bytes) return set_error(DET_ERR_INVALID_ARG, "wgrad: bytes is NULL");
  det_wgrad_cfg c;
  if (int s = resolve(cfg, &c)) return s;
  if (int s = check_shape(T_total, E, M, N, c)) return s;
  const size_t sb = scratch_bytes(T_total, E, M, N, c);
  *bytes = (atomic || sb == 0) ? 0 : DET_WS_HEADER_BYTES + align_up(sb, 256);
  return ok();
}

namespace {
// bf16: main_grad holds bf16 values; every split's partial goes to scratch and
// wgrad_fold_bf16_kernel adds the folded dW in bf16 (deterministic arm only).
int wgrad_entry(void* main_grad, bool bf16, int64_t ld_e, int64_t ld_m, const void* G, int64_t ldg, const void* X,
                int64_t ldx, const int32_t* offs, int32_t E, int64_t T_total, int64_t M, int64_t N,
                const det_wgrad_cfg* cfg, void* ws, size_t ws_bytes, int atomic, void* stream) {
  if (int s = check_atomic_flag(atomic)) return s;
  if (bf16 && atomic) return set_error(DET_ERR_UNSUPPORTED, "wgrad: a bf16 main_grad has no atomic arm");
  det_wgrad_cfg c;
  if (int s = resolve(cfg, &c)) return s;
  if (int s = check_shape(T_total, E, M, N, c)) return s;
  if (E == 0 || M == 0 || N == 0 || T_total == 0) return ok();
  if (!main_grad || !G || !X || !offs) return set_error(DET_ERR_INVALID_ARG, "wgrad: NULL pointer");
  if (ld_m < N || ld_e < M * ld_m)
    return set_error(DET_ERR_INVALID_ARG, "wgrad: need ld_m >= N and ld_e >= M*ld_m (an expanded main_grad is rejected)");
  if (ldg < M || ldx < N) return set_error(DET_ERR_INVALID_ARG, "wgrad: need ldg >= M and ldx >= N");
  if (ldg % 8 || ldx % 8 || !aligned(G, 16) || !aligned(X, 16) || ld_m % 4 || ld_e % 4 ||
      !aligned(main_grad, bf16 ? 8 : 16))
    return set_error(DET_ERR_UNSUPPORTED, "wgrad: rows of G, X and main_grad must be 16-byte (bf16 main_grad: 8-byte) aligned");
  // buffer loads use 32-bit byte offsets inside one split, including the rows
  // read ahead past its end (fewer than 512)
  if ((T_total + 512) * (ldg > ldx ? ldg : ldx) * 2 >= (1LL << 31))
    return set_error(DET_ERR_UNSUPPORTED, "wgrad: T_total x max(ldg, ldx) too large for 32-bit offsets");
  const size_t sb = bf16 ? scratch_bytes_all(T_total, E, M, N, c) : scratch_bytes(T_total, E, M, N, c);
  const size_t need = (atomic || sb == 0) ? 0 : DET_WS_HEADER_BYTES + align_up(sb, 256);
  if (int s = check_workspace(ws, ws_bytes, need)) return s;
  Range out_full;
  out_full.lo = reinterpret_cast<uintptr_t>(main_grad);
  out_full.hi = out_full.lo + static_cast<uintptr_t>(((E - 1) * ld_e + (M - 1) * ld_m + N) * (bf16 ? 2 : 4));
  if (overlaps(out_full, range2d(G, T_total, M, ldg, 2)) || overlaps(out_full, range2d(X, T_total, N, ldx, 2)) ||
      overlaps(out_full, range1d(offs, (static_cast<size_t>(E) + 1) * 4)) || overlaps(out_full, range1d(ws, ws_bytes)))
    return set_error(DET_ERR_OVERLAP, "wgrad: main_grad overlaps an input or the workspace");
  WgradArgs p;
  p.mg = bf16 ? nullptr : static_cast<float*>(main_grad);
  p.mg16 = bf16 ? static_cast<uint16_t*>(main_grad) : nullptr;
  p.ld_e = ld_e;
  p.ld_m = ld_m;
  p.G = static_cast<const uint16_t*>(G);
  p.ldg = ldg;
  p.X = static_cast<const uint16_t*>(X);
  p.ldx = ldx;
  p.offs = offs;
  p.E = E;
  p.T_total = static_cast<int>(T_total);
  p.M = static_cast<int>(M);
  p.N = static_cast<int>(N);
  p.split_rows = c.ktiles_per_split == 0 ? 0 : c.k_tile * c.ktiles_per_split;
  p.tiles_m = static_cast<int>((M + c.block_m - 1) / c.block_m);
  p.tiles_n = static_cast<int>(N / c.block_n);
  p.max_splits = max_splits(T_total, E, c);
  plan_xcds(p, c.block_m, c.block_n);
  p.scratch = (atomic || sb == 0) ? nullptr : reinterpret_cast<float*>(static_cast<char*>(ws) + DET_WS_HEADER_BYTES);
  if (p.n_units > 0x7FFFFFFF) return set_error(DET_ERR_UNSUPPORTED, "wgrad: too many work units");
  const hipStream_t st = as_stream(stream);
  const dim3 grid(static_cast<uint32_t>(p.n_units));
  if (c.block_m == kTT) {
    if (atomic)
      hipLaunchKernelGGL((wgrad_tl_kernel<true>), grid, dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL((bf16 ? wgrad_tl_kernel<false, true> : wgrad_tl_kernel<false>), grid, dim3(256), 0, st, p);
  } else if (c.block_n == 512) {
    if (atomic)
      hipLaunchKernelGGL((wgrad_kernel<4, true>), grid, dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL((bf16 ? wgrad_kernel<4, false, true> : wgrad_kernel<4, false>), grid, dim3(256), 0, st, p);
  } else {
    if (atomic)
      hipLaunchKernelGGL((wgrad_kernel<2, true>), grid, dim3(128), 0, st, p);
    else
      hipLaunchKernelGGL((bf16 ? wgrad_kernel<2, false, true> : wgrad_kernel<2, false>), grid, dim3(128), 0, st, p);
  }
  if (!atomic) {
    const int64_t per_e = M * N / 4;
    const dim3 fgrid(static_cast<uint32_t>(ceil_div(per_e, 256)), static_cast<uint32_t>(E));
    if (bf16)
      hipLaunchKernelGGL(wgrad_fold_bf16_kernel, fgrid, dim3(256), 0, st, p);
    else if (p.split_rows != 0)
      hipLaunchKernelGGL(wgrad_fold_kernel, fgrid, dim3(256), 0, st, p);
  }
  return check_launch(bf16 ? "det_grouped_wgrad_acc_bf16" : "det_grouped_wgrad_acc");
}
}  // namespace

extern "C" int det_grouped_wgrad_acc(float* main_grad, int64_t ld_e, int64_t ld_m, const void* G, int64_t ldg,
                                     const void* X, int64_t ldx, const int32_t* offs, int32_t E, int64_t T_total,
                                     int64_t M, int64_t N, const det_wgrad_cfg* cfg, void* ws, size_t ws_bytes,
                                     int atomic, void* stream) {
  return wgrad_entry(main_grad, false, ld_e, ld_m, G, ldg, X, ldx, offs, E, T_total, M, N, cfg, ws, ws_bytes, atomic,
                     stream);
}

extern "C" int det_grouped_wgrad_acc_bf16_workspace_size(int64_t T_total, int32_t E, int64_t M, int64_t N,
                                                         const det_wgrad_cfg* cfg, size_t* bytes) {
  if (!bytes) return set_error(DET_ERR_INVALID_ARG, "wgrad: bytes is NULL");
  det_wgrad_cfg c;
  if (int s = resolve(cfg, &c)) return s;
  if (int s = check_shape(T_total, E, M, N, c)) return s;
  const size_t sb = scratch_bytes_all(T_total, E, M, N, c);
  *bytes = sb == 0 ? 0 : DET_WS_HEADER_BYTES + align_up(sb, 256);
  return ok();
}

extern "C" int det_grouped_wgrad_acc_bf16(uint16_t* main_grad, int64_t ld_e, int64_t ld_m, const void* G, int64_t ldg,
                                          const void* X, int64_t ldx, const int32_t* offs, int32_t E, int64_t T_total,
                                          int64_t M, int64_t N, const det_wgrad_cfg* cfg, void* ws, size_t ws_bytes,
                                          void* stream) {
  return wgrad_entry(main_grad, true, ld_e, ld_m, G, ldg, X, ldx, offs, E, T_total, M, N, cfg, ws, ws_bytes, 0,
                     stream);
}
