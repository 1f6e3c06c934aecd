// det_grouped_wgrad_acc: main_grad[e] += G_e^T X_e with a fixed-order split-K
// (FlashInfer PR #8602: fused fp32 weight-gradient accumulate into main_grad;
// #8924: deterministic accumulate, bitwise the AccumulateGrad of the
// deterministic dW, with expert offsets read on the device).
//
// Contraction on the matrix cores. G_e [T_e x M] and X_e [T_e x N] both have
// the token index as their row index, so the reduction runs down the rows of
// both operands, while v_mfma_f32_32x32x16_bf16 wants each lane to hold 8
// consecutive k values of one output row (A) or column (B). Each lane therefore
// reads 8 token rows x 4 consecutive columns (8 bytes per row, 32 lanes cover
// 128 contiguous columns) from LDS and transposes the 8x4 block in registers
// with v_perm_b32. Fragment i (i = 0..3) then holds output rows m0 + 4r + i
// for lane slot r: one MFMA computes a strided 32x32 sub-tile, and 4 x 4 MFMAs
// cover the wave's 128 x 128 output tile. G and X reach LDS in their memory
// layout through 16-byte buffer loads that write LDS directly (no register
// round trip), over three LDS stages of 32 token rows, so two stages of loads
// are in flight while the matrix cores work on the third.
//
// Canonical order (the oracle's): an expert's rows are cut into splits of
// k_tile * ktiles_per_split rows counted from the expert's first row (one split
// when ktiles_per_split = 0). A split's partial is the chain of MFMAs over its
// rows in ascending 16-row blocks starting from +0.0 (rows past the split end
// are zero). With one split the epilogue adds the partial into main_grad
// directly; with several, each partial goes to scratch and a second kernel adds
// (((Q0 + Q1) + Q2) + ...) into main_grad once.
//
// The atomic arm adds every split's partial into main_grad with float atomics.
#include "common.hpp"

namespace detgrad {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 128;     // workgroup tile: 128 (m) x 512 (n), 4 waves of 128 x 128
constexpr int kBN = 512;
constexpr int kBK = 32;      // token rows per LDS stage
constexpr int kWaveN = 128;
constexpr int kThreads = 256;
constexpr int kTileM = kBM;
constexpr int kTileN = kBN;
constexpr int kKTile = 512;

struct WgradArgs {
  float* mg;
  int64_t ld_e, ld_m;
  const uint16_t* G;
  int64_t ldg;
  const uint16_t* X;
  int64_t ldx;
  const int32_t* offs;
  int E;
  int64_t T_total;
  int M, N;
  int64_t split_rows;  // 0: one split per expert
  int tiles_m, tiles_n;
  int64_t n_units;  // tiles * max_splits
  float* scratch;   // [max_splits][M][N]
  int64_t max_splits;
};

// Expert row range with clamping (offsets are device data and cannot be
// validated on the host): b_e = clamp(offs[e], b_{e-1}, T_total).
struct Split {
  int e;
  int64_t g;       // global split index (scratch slot)
  int64_t n_split;  // splits of this expert
  int64_t r0, r1;
};

__device__ __forceinline__ bool find_split(const WgradArgs& p, int64_t g, Split& out) {
  int64_t prev = 0, cum = 0;
  int64_t b = p.offs[0];
  b = b < 0 ? 0 : (b > p.T_total ? p.T_total : b);
  prev = b;
  for (int e = 0; e < p.E; ++e) {
    int64_t nb = p.offs[e + 1];
    nb = nb < prev ? prev : (nb > p.T_total ? p.T_total : nb);
    const int64_t te = nb - prev;
    const int64_t se = te == 0 ? 0 : (p.split_rows == 0 ? 1 : (te + p.split_rows - 1) / p.split_rows);
    if (g < cum + se) {
      const int64_t s = g - cum;
      out.e = e;
      out.g = g;
      out.n_split = se;
      if (p.split_rows == 0) {
        out.r0 = prev;
        out.r1 = nb;
      } else {
        out.r0 = prev + s * p.split_rows;
        out.r1 = out.r0 + p.split_rows < nb ? out.r0 + p.split_rows : nb;
      }
      return true;
    }
    cum += se;
    prev = nb;
  }
  return false;
}

// MFMA operand of column c (0..3) of a lane's 8-row x 4-column block: dword q
// packs rows 2q (low 16 bits) and 2q+1 (high 16 bits) of that column.
template <int C>
__device__ __forceinline__ bf16x8_t frag(const uint2 (&v)[8]) {
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

// One K step of kBK token rows lands in LDS as row-major [k][m] and [k][n]
// slabs (the layout of G and X in memory) through direct buffer-to-LDS loads:
// each instruction moves 64 lanes x 16 bytes into 1 KiB of LDS in lane order,
// so no registers hold the data in flight. The buffer resources cover the
// split's rows only; rows past the split end read as zero. G: 8 instructions
// per step (4 rows of 256 B each), X: 32 (one 1 KiB row each), 10 per wave.
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // gfx9-family raw buffer descriptor
constexpr int kDmaA = kBK * kBM * 2 / 1024;     // 1 KiB transfers of G per step
constexpr int kDmaB = kBK * kBN * 2 / 1024;     // 1 KiB transfers of X per step
constexpr int kDmaPerWave = (kDmaA + kDmaB) / (kThreads / 64);

typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor: base address, stride 0, num_records bytes.
__device__ __forceinline__ i32x4_t make_rsrc(const void* base, uint32_t num_records) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r[0] = static_cast<int32_t>(a & 0xFFFFFFFFu);
  r[1] = static_cast<int32_t>((a >> 32) & 0xFFFFu);
  r[2] = static_cast<int32_t>(num_records);
  r[3] = static_cast<int32_t>(kRsrcWord3);
  return r;
}

// LDS byte address of a __shared__ object (wave-uniform here).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  typedef __attribute__((address_space(3))) const char* lds_ptr_t;
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)(p)));  // generic -> LDS address space
}

// One 1 KiB transfer: every lane's 16 bytes at rsrc + voff + soff land at
// LDS[m0 + 16 * lane]. Issued as inline assembly (as the composable-kernel
// library does for its asynchronous copies) so that the compiler does not
// insert conservative waits on these loads before unrelated LDS reads; the
// kernel waits for them explicitly with s_waitcnt vmcnt.
__device__ __forceinline__ void dma16(uint32_t lds, i32x4_t rsrc, int32_t voff, int32_t soff) {
  asm volatile("s_mov_b32 m0, %0" : : "s"(lds) : "memory");
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" : : "v"(voff), "s"(rsrc), "s"(soff) : "memory");
}

struct Src {
  i32x4_t ra, rb;           // G and X rows [r0, r1), rebased at r0
  int32_t voff_a, voff_b;   // this lane's byte offset inside one transfer
  int32_t krow_a, krow_b;   // bytes per token row
};

// Issue this wave's share of the transfers of the step starting at split row krel.
__device__ __forceinline__ void stage_issue(const Src& src, int32_t krel, uint16_t (*la)[kBM], uint16_t (*lb)[kBN],
                                            int wave) {
#pragma unroll
  for (int u = 0; u < kDmaA / 4; ++u) {
    const int i = wave * (kDmaA / 4) + u;  // transfer i covers rows 4i .. 4i+3
    dma16(lds_addr(&la[4 * i][0]), src.ra, src.voff_a, (krel + 4 * i) * src.krow_a);
  }
#pragma unroll
  for (int u = 0; u < kDmaB / 4; ++u) {
    const int i = wave * (kDmaB / 4) + u;  // transfer i covers row i
    dma16(lds_addr(&lb[i][0]), src.rb, src.voff_b, (krel + i) * src.krow_b);
  }
}

// Wait until this wave's transfers of the oldest in-flight step have landed
// (the younger step's kDmaPerWave may still be pending), then meet the other
// waves so that every wave's transfers of that step are visible.
template <bool YOUNGER_PENDING>
__device__ __forceinline__ void stage_wait() {
  static_assert(kDmaPerWave == 10, "vmcnt literal below");
  if (YOUNGER_PENDING)
    asm volatile("s_waitcnt vmcnt(10)" : : : "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
  __builtin_amdgcn_s_barrier();
}

// One 16-row MFMA block from LDS rows [row0, row0 + 16): lane (r, kg) reads
// rows row0 + 8*kg + e of its 4 G columns (4r..4r+3) and its 4 X columns
// (128*wave + 4r ..), transposes, and issues 4 x 4 MFMAs.
__device__ __forceinline__ void mma_block(const uint16_t (*la)[kBM], const uint16_t (*lb)[kBN], int row0, int r,
                                          int kg, int wave, f32x16_t (&acc)[4][4]) {
  uint2 ra[8], rb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ra[e] = *reinterpret_cast<const uint2*>(&la[row0 + 8 * kg + e][4 * r]);
    rb[e] = *reinterpret_cast<const uint2*>(&lb[row0 + 8 * kg + e][kWaveN * wave + 4 * r]);
  }
  const bf16x8_t fa[4] = {frag<0>(ra), frag<1>(ra), frag<2>(ra), frag<3>(ra)};
  const bf16x8_t fb[4] = {frag<0>(rb), frag<1>(rb), frag<2>(rb), frag<3>(rb)};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
}

// XCD-aware placement. Workgroups are dispatched to the 8 XCDs round-robin
// (workgroup u runs on XCD u % 8), and each XCD has its own L2. XCD x takes,
// for every split, the tiles of n-tile column x % tiles_n and of its share of
// the m-tiles; consecutive workgroups on one XCD are tiles of the same split
// and column, so their X rows come from that XCD's L2 after the first read.
// Every XCD gets a share of every expert, which keeps the XCDs balanced.
constexpr int kXcds = 8;

__device__ __forceinline__ bool unit_of(const WgradArgs& p, uint32_t u, int64_t& g, int& mt, int& nt) {
  const int x = static_cast<int>(u % kXcds);
  const int64_t slot = u / kXcds;
  const int NT = p.tiles_n, MT = p.tiles_m;
  if (kXcds % NT == 0) {
    const int parts = kXcds / NT;           // m-tile parts per column
    const int part = x / NT;
    const int mlo = part * MT / parts, mhi = (part + 1) * MT / parts;
    const int per = mhi - mlo;
    if (per == 0) return false;
    g = slot / per;
    if (g >= p.max_splits) return false;
    mt = mlo + static_cast<int>(slot % per);
    nt = x % NT;
    return true;
  }
  // any other column count: plain split-major order
  const int64_t t = static_cast<int64_t>(u) % (static_cast<int64_t>(MT) * NT);
  g = static_cast<int64_t>(u) / (static_cast<int64_t>(MT) * NT);
  if (g >= p.max_splits) return false;
  mt = static_cast<int>(t / NT);
  nt = static_cast<int>(t % NT);
  return true;
}

__host__ int64_t wgrad_grid(int tiles_m, int tiles_n, int64_t max_splits) {
  if (kXcds % tiles_n == 0) {
    const int parts = kXcds / tiles_n;
    int per_max = 0;
    for (int part = 0; part < parts; ++part) {
      const int per = (part + 1) * tiles_m / parts - part * tiles_m / parts;
      per_max = per > per_max ? per : per_max;
    }
    return static_cast<int64_t>(kXcds) * per_max * max_splits;
  }
  return static_cast<int64_t>(tiles_m) * tiles_n * max_splits;
}

// One workgroup = 4 waves = a 128 (m) x 512 (n) output tile; wave w owns the
// 128 x 128 columns n0 + 128w. K runs in steps of kBK rows through two LDS
// buffers: while the matrix cores work on one, the next step's global loads
// are in flight in registers and then written to the other.
template <bool ATOMIC>
__global__ __launch_bounds__(kThreads) void wgrad_kernel(WgradArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t la0[kBK][kBM];
  __shared__ __attribute__((aligned(16))) uint16_t la1[kBK][kBM];
  __shared__ __attribute__((aligned(16))) uint16_t la2[kBK][kBM];
  __shared__ __attribute__((aligned(16))) uint16_t lb0[kBK][kBN];
  __shared__ __attribute__((aligned(16))) uint16_t lb1[kBK][kBN];
  __shared__ __attribute__((aligned(16))) uint16_t lb2[kBK][kBN];
  int64_t g;
  int mt, nt;
  if (!unit_of(p, blockIdx.x, g, mt, nt)) return;
  Split sp;
  if (!find_split(p, g, sp)) return;
  // wave-uniform by construction; readfirstlane lets the compiler keep it (and
  // every LDS transfer base derived from it) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int m0 = mt * kBM;
  const int n0 = nt * kBN;
  const int r = lane & 31;
  const int kg = lane >> 5;

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  const int64_t r0 = sp.r0, r1 = sp.r1;
  const int32_t rows = static_cast<int32_t>(r1 - r0);
  Src src;
  src.ra = make_rsrc(p.G + r0 * p.ldg, static_cast<uint32_t>(rows * p.ldg * 2));
  src.rb = make_rsrc(p.X + r0 * p.ldx, static_cast<uint32_t>(rows * p.ldx * 2));
  src.krow_a = static_cast<int32_t>(p.ldg * 2);
  src.krow_b = static_cast<int32_t>(p.ldx * 2);
  src.voff_a = (lane / (kBM / 8)) * src.krow_a + (m0 + (lane % (kBM / 8)) * 8) * 2;
  src.voff_b = (n0 + lane * 8) * 2;

  // Three LDS buffers: while the matrix cores work on step s, the transfers of
  // steps s+1 and s+2 are in flight. The loop is unrolled over the buffers so
  // that each buffer is its own LDS object (exact wait counts) and every LDS
  // address is a per-lane base plus a constant.
  stage_issue(src, 0, la0, lb0, wave);
  if (kBK < rows) stage_issue(src, kBK, la1, lb1, wave);
#define DET_WGRAD_STEP(LA, LB, LA_NEXT2, LB_NEXT2, OFF)                              \
  {                                                                                 \
    const int32_t k = k0 + (OFF);                                                   \
    if (k >= rows) break;                                                           \
    if (k + kBK < rows) stage_wait<true>(); else stage_wait<false>();               \
    if (k + 2 * kBK < rows) stage_issue(src, k + 2 * kBK, LA_NEXT2, LB_NEXT2, wave); \
    mma_block(LA, LB, 0, r, kg, wave, acc);                                         \
    if (k + 16 < rows) mma_block(LA, LB, 16, r, kg, wave, acc);                     \
  }
  for (int32_t k0 = 0; k0 < rows; k0 += 3 * kBK) {
    DET_WGRAD_STEP(la0, lb0, la2, lb2, 0)
    DET_WGRAD_STEP(la1, lb1, la0, lb0, kBK)
    DET_WGRAD_STEP(la2, lb2, la1, lb1, 2 * kBK)
  }
#undef DET_WGRAD_STEP

  // Epilogue: lane (r, kg), MFMA (i, j), accumulator q holds output
  // m = m0 + 4 * (8*(q/4) + 4*kg + q%4) + i,  n = n0 + 128*wave + 4*r + j.
  const bool direct = sp.n_split == 1;
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

int resolve(const det_wgrad_cfg* cfg, det_wgrad_cfg* out) {
  det_wgrad_cfg c{kTileM, kTileN, kKTile, 0};
  if (cfg) c = *cfg;
  if (c.block_m != kTileM || c.block_n != kTileN)
    return set_error(DET_ERR_UNSUPPORTED, "wgrad: block_m x block_n must be %d x %d, got %d x %d", kTileM, kTileN,
                     c.block_m, c.block_n);
  if (c.k_tile != kKTile) return set_error(DET_ERR_INVALID_ARG, "wgrad: k_tile must be %d, got %d", kKTile, c.k_tile);
  if (c.ktiles_per_split < 0 || c.ktiles_per_split > (1 << 20))
    return set_error(DET_ERR_INVALID_ARG, "wgrad: ktiles_per_split must be in [0, 2^20], got %d", c.ktiles_per_split);
  *out = c;
  return DET_OK;
}

int check_shape(int64_t T_total, int32_t E, int64_t M, int64_t N) {
  if (T_total < 0 || E < 0 || M < 0 || N < 0) return set_error(DET_ERR_INVALID_ARG, "wgrad: sizes must be >= 0");
  if (M % kTileM || N % kTileN)
    return set_error(DET_ERR_UNSUPPORTED, "wgrad: M and N must be multiples of %d and %d, got %lld x %lld", kTileM,
                     kTileN, static_cast<long long>(M), static_cast<long long>(N));
  if (M > (1 << 20) || N > (1 << 20) || E > 4096) return set_error(DET_ERR_UNSUPPORTED, "wgrad: problem too large");
  // buffer loads use 32-bit byte offsets inside one split's rows
  if (T_total * (M > N ? M : N) * 2 >= (1LL << 31))
    return set_error(DET_ERR_UNSUPPORTED, "wgrad: T_total x max(M, N) too large for 32-bit offsets");
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

}  // namespace
}  // namespace detgrad

using namespace detgrad;

extern "C" int det_grouped_wgrad_acc_workspace_size(int64_t T_total, int32_t E, int64_t M, int64_t N,
                                                    const det_wgrad_cfg* cfg, int atomic, size_t* bytes) {
  if (int s = check_atomic_flag(atomic)) return s;
  if (!bytes) return set_error(DET_ERR_INVALID_ARG, "wgrad: bytes is NULL");
  if (int s = check_shape(T_total, E, M, N)) return s;
  det_wgrad_cfg c;
  if (int s = resolve(cfg, &c)) return s;
  const size_t sb = scratch_bytes(T_total, E, M, N, c);
  *bytes = (atomic || sb == 0) ? 0 : DET_WS_HEADER_BYTES + align_up(sb, 256);
  return ok();
}

extern "C" int det_grouped_wgrad_acc(float* main_grad, int64_t ld_e, int64_t ld_m, const void* G, int64_t ldg,
                                     const void* X, int64_t ldx, const int32_t* offs, int32_t E, int64_t T_total,
                                     int64_t M, int64_t N, const det_wgrad_cfg* cfg, void* ws, size_t ws_bytes,
                                     int atomic, void* stream) {
  if (int s = check_atomic_flag(atomic)) return s;
  if (int s = check_shape(T_total, E, M, N)) return s;
  det_wgrad_cfg c;
  if (int s = resolve(cfg, &c)) return s;
  if (E == 0 || M == 0 || N == 0 || T_total == 0) return ok();
  if (!main_grad || !G || !X || !offs) return set_error(DET_ERR_INVALID_ARG, "wgrad: NULL pointer");
  if (ld_m < N || ld_e < M * ld_m)
    return set_error(DET_ERR_INVALID_ARG, "wgrad: need ld_m >= N and ld_e >= M*ld_m (an expanded main_grad is rejected)");
  if (ldg < M || ldx < N) return set_error(DET_ERR_INVALID_ARG, "wgrad: need ldg >= M and ldx >= N");
  if (ldg % 8 || ldx % 8 || !aligned(G, 16) || !aligned(X, 16) || ld_m % 4 || ld_e % 4 || !aligned(main_grad, 16))
    return set_error(DET_ERR_UNSUPPORTED, "wgrad: rows of G, X and main_grad must be 16-byte aligned");
  const size_t sb = scratch_bytes(T_total, E, M, N, c);
  const size_t need = (atomic || sb == 0) ? 0 : DET_WS_HEADER_BYTES + align_up(sb, 256);
  if (int s = check_workspace(ws, ws_bytes, need)) return s;
  Range out_full;
  out_full.lo = reinterpret_cast<uintptr_t>(main_grad);
  out_full.hi = out_full.lo + static_cast<uintptr_t>(((E - 1) * ld_e + (M - 1) * ld_m + N) * 4);
  if (overlaps(out_full, range2d(G, T_total, M, ldg, 2)) || overlaps(out_full, range2d(X, T_total, N, ldx, 2)) ||
      overlaps(out_full, range1d(offs, (static_cast<size_t>(E) + 1) * 4)) || overlaps(out_full, range1d(ws, ws_bytes)))
    return set_error(DET_ERR_OVERLAP, "wgrad: main_grad overlaps an input or the workspace");
  WgradArgs p;
  p.mg = main_grad;
  p.ld_e = ld_e;
  p.ld_m = ld_m;
  p.G = static_cast<const uint16_t*>(G);
  p.ldg = ldg;
  p.X = static_cast<const uint16_t*>(X);
  p.ldx = ldx;
  p.offs = offs;
  p.E = E;
  p.T_total = T_total;
  p.M = static_cast<int>(M);
  p.N = static_cast<int>(N);
  p.split_rows = c.ktiles_per_split == 0 ? 0 : static_cast<int64_t>(c.k_tile) * c.ktiles_per_split;
  p.tiles_m = static_cast<int>(M / kTileM);
  p.tiles_n = static_cast<int>(N / kTileN);
  p.max_splits = max_splits(T_total, E, c);
  p.n_units = wgrad_grid(p.tiles_m, p.tiles_n, p.max_splits);
  p.scratch = (atomic || sb == 0) ? nullptr : reinterpret_cast<float*>(static_cast<char*>(ws) + DET_WS_HEADER_BYTES);
  if (p.n_units > 0x7FFFFFFF) return set_error(DET_ERR_UNSUPPORTED, "wgrad: too many work units");
  const hipStream_t st = as_stream(stream);
  if (atomic) {
    hipLaunchKernelGGL(wgrad_kernel<true>, dim3(static_cast<uint32_t>(p.n_units)), dim3(kThreads), 0, st, p);
  } else {
    hipLaunchKernelGGL(wgrad_kernel<false>, dim3(static_cast<uint32_t>(p.n_units)), dim3(kThreads), 0, st, p);
    if (p.split_rows != 0) {
      const int64_t per_e = M * N / 4;
      hipLaunchKernelGGL(wgrad_fold_kernel, dim3(static_cast<uint32_t>(ceil_div(per_e, 256)), static_cast<uint32_t>(E)),
                         dim3(256), 0, st, p);
    }
  }
  return check_launch("det_grouped_wgrad_acc");
}
