// det_index_add: out[ids[p]] += src[p] without float atomics (sparse-indexer dK,
// Megatron-LM PR #7441, source 3: a stable sort of the ids and a prefix sum of
// their counts replace the atomic accumulation).
//
// Pipeline (all on `stream`, integer-only until step 5):
//  1. count    per block of 4096 source positions, an LDS histogram of the ids
//              (integer LDS atomics: the counts are exact in any order); the
//              block's row hist[b][*] is written densely. Out-of-range ids other
//              than -1 are counted as bad.
//  2. prefix   per id, exclusive prefix of hist[*][id] over blocks (in place)
//              and the id's total count.
//  3. scan     per-workgroup totals of the counts, then exclusive scans of the
//              counts (segment offsets of the sorted order) and of
//              ceil(count / L) (chunk offsets), and the chunk descriptors.
//  4. scatter  per block, the lanes holding the same id in a batch of 64
//              positions find each other with one ballot per id bit, so each
//              lane's rank among equal ids is its position order inside the
//              batch plus the id's running LDS count, walked batch by batch: a
//              stable counting sort. perm[seg_off[id] + prefix + rank] = p (the
//              fused indexer dK stores the pair (p, coefficient of p) there).
//  5. gather   one wave (or lane group) per chunk of L sorted rows of one id:
//              each lane owns consecutive dims of the row and folds the
//              chunk's rows left to right. Stored bf16 rows below 2^31 bytes
//              are read through a buffer resource with a rolling window of
//              row loads in flight; the fused indexer dK at dim 128 takes four
//              chunks per wave with 16-byte loads of its query rows. A
//              single-chunk id is added into out directly; otherwise the
//              partial goes to scratch.
//  6. fold     ids with several chunks fold their chunk partials left to right
//              and add the total into out once.
// Traffic: the src rows of valid ids (256 B per row at dim 128) dominate;
// ids, perm, the histograms and out are small next to them.
//
// The atomic arm adds each src row into out[id] with per-element hardware float
// atomics and no sort, as a non-deterministic index_add does.
#include <type_traits>

#include "common.hpp"

namespace detgrad {
namespace {

constexpr int kBlockPos = 4096;  // source positions per count/scatter block
constexpr int kMaxRows = 16384;  // LDS histogram capacity (64 KiB)
constexpr int kMaxDim = 512;

constexpr int kSegBlocks = 16;   // blocks per prefix segment
// block counts and their prefix inside a segment are stored as 16-bit words
static_assert((kSegBlocks - 1) * kBlockPos <= 0xFFFF, "a segment prefix must fit in 16 bits");

// Row stride of the block histograms (16-bit entries): rows start 16-byte aligned.
inline __host__ __device__ int hist_stride(int64_t n_rows) { return static_cast<int>((n_rows + 7) / 8 * 8); }
constexpr int kMaxGroups = kMaxRows / 256;  // workgroups of the offsets kernel (one thread per id)

struct Layout {
  size_t hist, segtot, wg_tot, seg_off, chunk_off, full_off, chunk_desc, perm, scratch, coef, pairs, total;
  int64_t nblk, nseg, max_chunks;
};

// coef: the fused indexer dK's per-slot coefficients [n_src] float32 follow,
// then its sorted order as (slot, coefficient) pairs [n_src] (in place of perm).
Layout layout(int64_t n_src, int64_t dim, int64_t n_rows, int64_t L, bool coef = false) {
  Layout l;
  l.nblk = ceil_div(n_src, kBlockPos);
  l.nseg = ceil_div(l.nblk, kSegBlocks);
  l.max_chunks = n_src / L + (n_rows < n_src ? n_rows : n_src) + 1;
  size_t o = DET_WS_HEADER_BYTES;
  l.hist = o;      o = align_up(o + static_cast<size_t>(l.nblk * hist_stride(n_rows)) * 2, 256);
  l.segtot = o;    o = align_up(o + static_cast<size_t>(l.nseg * n_rows) * 4, 256);
  l.wg_tot = o;   o = align_up(o + static_cast<size_t>(3 * kMaxGroups) * 4, 256);
  l.seg_off = o;   o = align_up(o + static_cast<size_t>(n_rows + 1) * 4, 256);
  l.chunk_off = o; o = align_up(o + static_cast<size_t>(n_rows + 1) * 4, 256);
  l.full_off = o;  o = align_up(o + static_cast<size_t>(n_rows + 1) * 4, 256);
  l.chunk_desc = o; o = align_up(o + static_cast<size_t>(l.max_chunks) * 16, 256);
  l.perm = o;      o = align_up(o + static_cast<size_t>(n_src) * 4, 256);
  l.scratch = o;   o = align_up(o + static_cast<size_t>(l.max_chunks * dim) * 4, 256);
  l.coef = o;      o = coef ? align_up(o + static_cast<size_t>(n_src) * 4, 256) : o;
  l.pairs = o;     o = coef ? align_up(o + static_cast<size_t>(n_src) * 8, 256) : o;
  l.total = o;
  return l;
}

// Lanes of one wave holding the same id find each other with one ballot per
// id bit (ids are below 2^14); returns the mask of those lanes (0 for invalid
// lanes). Invalid lanes are never in a mask: the first ballot drops them.
constexpr int kIdBits = 14;
static_assert((1 << kIdBits) >= kMaxRows, "ids must fit in kIdBits bits");

__device__ __forceinline__ uint64_t match_peers(int32_t id, bool valid) {
  uint64_t peers = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < kIdBits; ++bit) {
    const bool set = (id >> bit) & 1;
    const uint64_t m = __ballot(set);
    peers &= set ? m : ~m;
  }
  return valid ? peers : 0ull;
}

// ---- 1. count. Integer LDS atomics: the counts are exact in any order (the
// hot Zipf key makes a few lanes of an instruction share an address, which
// the LDS serialises; that is far cheaper than matching lanes first). A block
// of positions is one workgroup of kSortThreads threads (16 waves, so that
// the two blocks a compute unit holds keep its SIMDs busy).
constexpr int kSortThreads = 1024;

// (launch bounds: 16 waves per block and two blocks per compute unit, so at
// most 64 registers per lane)
__global__ __launch_bounds__(kSortThreads, 8) void ia_count(const int32_t* __restrict__ ids, int64_t n_src,
                                                            int n_rows, int hist_ld, uint16_t* __restrict__ hist,
                                                            uint32_t* __restrict__ hdr) {
  extern __shared__ uint32_t lds_hist[];
  for (int k = threadIdx.x; k < hist_ld; k += kSortThreads) lds_hist[k] = 0u;
  const int64_t b = blockIdx.x;
  const int64_t p0 = b * kBlockPos;
  const int64_t p1 = p0 + kBlockPos < n_src ? p0 + kBlockPos : n_src;
  constexpr int kPer = kBlockPos / kSortThreads;
  int32_t idv[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int64_t p = p0 + threadIdx.x + u * kSortThreads;
    idv[u] = p < p1 ? ids[p] : -1;
  }
  __syncthreads();
  uint32_t bad = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int32_t id = idv[u];
    if (id >= 0 && id < n_rows)
      atomicAdd(&lds_hist[id], 1u);
    else if (id != -1)
      ++bad;
  }
  __syncthreads();
  // counts are at most kBlockPos: eight 16-bit entries per 16-byte store
  uint4* row = reinterpret_cast<uint4*>(hist + b * hist_ld);
  for (int k8 = threadIdx.x; k8 < hist_ld / 8; k8 += kSortThreads) {
    const uint32_t* c = lds_hist + 8 * k8;
    row[k8] = make_uint4(c[0] | c[1] << 16, c[2] | c[3] << 16, c[4] | c[5] << 16, c[6] | c[7] << 16);
  }
  if (bad) atomicAdd(hdr, bad);
}

// ---- 2a. per id and segment of kSegBlocks blocks: exclusive prefix over the
// segment's blocks (in place) and the segment total.
__global__ __launch_bounds__(256) void ia_prefix_seg(uint16_t* __restrict__ hist, int hist_ld, int64_t nblk,
                                                     int n_rows, uint32_t* __restrict__ segtot) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  const int64_t seg = blockIdx.y;
  if (k >= n_rows) return;
  const int64_t b0 = seg * kSegBlocks;
  uint32_t c[kSegBlocks];
#pragma unroll
  for (int j = 0; j < kSegBlocks; ++j) c[j] = (b0 + j < nblk) ? hist[(b0 + j) * hist_ld + k] : 0u;
  uint32_t run = 0;
#pragma unroll
  for (int j = 0; j < kSegBlocks; ++j) {
    if (b0 + j < nblk) hist[(b0 + j) * hist_ld + k] = static_cast<uint16_t>(run);
    run += c[j];
  }
  segtot[seg * n_rows + k] = run;
}

// ceil(n / L) for n < 2^31 + L with a reciprocal computed on the host,
// rcp = floor((2^32 - 1) / L): the quotient estimate is low by at most 2 and
// is corrected exactly with two compare-and-subtract steps (no branches; a
// hardware integer division does not exist).
__device__ __forceinline__ uint32_t ceil_div_rcp(uint32_t n, uint32_t L, uint32_t rcp) {
  const uint32_t m = n + L - 1;
  uint32_t q = __umulhi(m, rcp);
  uint32_t r = m - q * L;
  const uint32_t c1 = r >= L ? 1u : 0u;
  q += c1;
  r -= c1 * L;
  q += r >= L ? 1u : 0u;
  return q;
}

// floor(n / K) for n < 2^31, with rcp = floor((2^32 - 1) / K) as above.
__device__ __forceinline__ uint32_t floor_div_rcp(uint32_t n, uint32_t K, uint32_t rcp) {
  uint32_t q = __umulhi(n, rcp);
  uint32_t r = n - q * K;
  const uint32_t c1 = r >= K ? 1u : 0u;
  q += c1;
  r -= c1 * K;
  q += r >= K ? 1u : 0u;
  return q;
}

// ---- 3. offsets and chunk descriptors, one thread per id and 256 ids per
// workgroup, in two kernels. ia_totals: thread k adds up id k's segment totals
// (leaving their exclusive prefix in place) to its count c, parks c in its
// seg_off entry, and with n = ceil(c / L) chunks of which f = floor(c / L) are
// full, every workgroup stores its totals of c, n and f in the workspace.
// ia_offsets: the exclusive scans over ids of c (segment offsets), n (chunk
// offsets) and f (full chunks): a workgroup scans its own ids and adds the
// totals of the workgroups before it, and takes the grand totals from all of
// them. The kernel boundary orders every workgroup's totals before any read of
// them, so no workgroup ever waits for another. Integer sums only: exact in
// any order.
//
// Then the 16-byte descriptors {id, first sorted row, rows, scratch slot} of
// every chunk, so a gather wave starts from one load. The gather takes them
// in list order, so the list puts the chunks of L rows first and the shorter
// last chunks of the ids after them: the waves that start last are the short
// ones. The scratch slot is the chunk's canonical index (chunk offset + j,
// where the fold reads it), or -1 for the only chunk of an id (added into out
// directly).

// Inclusive scan over the 16 lanes of row 0 (the other rows are ignored).
__device__ __forceinline__ uint32_t row_incl_scan(uint32_t v) {
  v = dpp_add<0x111, 0xF>(v);
  v = dpp_add<0x112, 0xF>(v);
  v = dpp_add<0x114, 0xF>(v);
  v = dpp_add<0x118, 0xF>(v);
  return v;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wave_incl_scan(v)), 63));
}

// Count c of id k (its segment totals turned into their exclusive prefix in
// place), its chunks n and its full chunks f.
__device__ __forceinline__ void id_counts(uint32_t c, int L, uint32_t rcp, uint32_t& nc, uint32_t& fc) {
  nc = ceil_div_rcp(c, L, rcp);
  fc = nc - (nc * static_cast<uint32_t>(L) != c ? 1u : 0u);
}

__global__ __launch_bounds__(256) void ia_totals(uint32_t* __restrict__ segtot, int64_t nseg, int n_rows, int L,
                                                 uint32_t rcp, uint32_t* __restrict__ wg_tot,
                                                 uint32_t* __restrict__ counts) {
  __shared__ uint32_t w_tot[3][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x;
  const int k = b * 256 + tid;
  uint32_t c = 0;
  if (k < n_rows) {
    for (int64_t s0 = 0; s0 < nseg; s0 += 16) {
      uint32_t v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = (s0 + j < nseg) ? segtot[(s0 + j) * n_rows + k] : 0u;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (s0 + j < nseg) segtot[(s0 + j) * n_rows + k] = c;
        c += v[j];
      }
    }
    counts[k] = c;
  }
  uint32_t nc, fc;
  id_counts(c, L, rcp, nc, fc);
  const uint32_t t0 = wave_sum(c), t1 = wave_sum(nc), t2 = wave_sum(fc);
  if (lane == 0) {
    w_tot[0][wave] = t0;
    w_tot[1][wave] = t1;
    w_tot[2][wave] = t2;
  }
  __syncthreads();
  if (tid < 3) wg_tot[tid * kMaxGroups + b] = w_tot[tid][0] + w_tot[tid][1] + w_tot[tid][2] + w_tot[tid][3];
}

__global__ __launch_bounds__(256) void ia_offsets(int n_rows, int L, uint32_t rcp, int64_t n_src,
                                                  const uint32_t* __restrict__ wg_tot,
                                                  uint32_t* __restrict__ seg_off, uint32_t* __restrict__ chunk_off,
                                                  uint32_t* __restrict__ full_off, int4* __restrict__ desc,
                                                  uint32_t* __restrict__ hdr) {
  __shared__ uint32_t w_tot[3][4];
  __shared__ uint32_t g_tot[2][3];  // [0]: workgroups before this one, [1]: all
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x, ng = gridDim.x;
  const int k = b * 256 + tid;
  const uint32_t c = k < n_rows ? seg_off[k] : 0u;  // the count ia_totals parked there
  uint32_t nc, fc;
  id_counts(c, L, rcp, nc, fc);
  const uint32_t i0 = wave_incl_scan(c), i1 = wave_incl_scan(nc), i2 = wave_incl_scan(fc);
  if (lane == 63) {
    w_tot[0][wave] = i0;
    w_tot[1][wave] = i1;
    w_tot[2][wave] = i2;
  }
  if (wave == 0) {
    // lane j holds workgroup j's totals (written by ia_totals, a finished kernel)
    const uint32_t v0 = lane < ng ? wg_tot[lane] : 0u, v1 = lane < ng ? wg_tot[kMaxGroups + lane] : 0u,
                   v2 = lane < ng ? wg_tot[2 * kMaxGroups + lane] : 0u;
    const uint32_t p0 = wave_sum(lane < b ? v0 : 0u), p1 = wave_sum(lane < b ? v1 : 0u),
                   p2 = wave_sum(lane < b ? v2 : 0u);
    const uint32_t a0 = wave_sum(v0), a1 = wave_sum(v1), a2 = wave_sum(v2);
    if (lane == 0) {
      g_tot[0][0] = p0; g_tot[0][1] = p1; g_tot[0][2] = p2;
      g_tot[1][0] = a0; g_tot[1][1] = a1; g_tot[1][2] = a2;
    }
  }
  __syncthreads();
  uint32_t e0 = i0 - c, e1 = i1 - nc, e2 = i2 - fc;  // exclusive prefix inside the workgroup
#pragma unroll
  for (int w = 0; w < 3; ++w)
    if (w < wave) {
      e0 += w_tot[0][w];
      e1 += w_tot[1][w];
      e2 += w_tot[2][w];
    }
  const uint32_t seg = g_tot[0][0] + e0, chk = g_tot[0][1] + e1, ful = g_tot[0][2] + e2;
  const uint32_t n_full = g_tot[1][2];
  if (k < n_rows) {
    seg_off[k] = seg;
    chunk_off[k] = chk;
    full_off[k] = ful;
  }
  if (b == 0 && tid == 0) {
    seg_off[n_rows] = g_tot[1][0];
    chunk_off[n_rows] = g_tot[1][1];
    full_off[n_rows] = n_full;
    hdr[1] = hdr[0];  // bad ids of this call
    hdr[0] = 0u;      // reset the accumulator for the next call
  }
  // descriptors: a thread writes those of its own id when it has at most
  // kDescSerial chunks (most ids have one); the wave writes those of its ids
  // with more, 64 chunks at a time (a hot id owns thousands)
  constexpr uint32_t kDescSerial = 4;
  const uint32_t s1 = static_cast<uint64_t>(seg) + c > static_cast<uint64_t>(n_src) ? static_cast<uint32_t>(n_src)
                                                                                     : seg + c;
  auto put = [&](int id, uint32_t s0, uint32_t s1, uint32_t c0, uint32_t nj, uint32_t f0, uint32_t i) {
    const uint32_t r0 = s0 + i * static_cast<uint32_t>(L);
    const uint32_t len = r0 + static_cast<uint32_t>(L) < s1 ? static_cast<uint32_t>(L) : (s1 > r0 ? s1 - r0 : 0u);
    // full chunks keep their order among full chunks; an id's partial chunk
    // is its last, numbered among the partial chunks (c0 - f0 before it)
    const uint32_t at = len == static_cast<uint32_t>(L) ? f0 + i : n_full + (c0 - f0);
    desc[at] = make_int4(id, static_cast<int>(r0), static_cast<int>(len), nj == 1 ? -1 : static_cast<int>(c0 + i));
  };
  if (k < n_rows && nc <= kDescSerial)
    for (uint32_t i = 0; i < nc; ++i) put(k, seg, s1, chk, nc, ful, i);
  uint64_t big = __ballot(k < n_rows && nc > kDescSerial);
  while (big) {
    const int j = __builtin_ctzll(big);
    big &= big - 1;
    const int kj = __builtin_amdgcn_readlane(k, j);
    const uint32_t s0j = __builtin_amdgcn_readlane(seg, j), s1j = __builtin_amdgcn_readlane(s1, j);
    const uint32_t c0j = __builtin_amdgcn_readlane(chk, j), nj = __builtin_amdgcn_readlane(nc, j);
    const uint32_t f0j = __builtin_amdgcn_readlane(ful, j);
    for (uint32_t i = lane; i < nj; i += 64) put(kj, s0j, s1j, c0j, nj, f0j, i);
  }
}

// ---- 4. stable scatter. One workgroup of 16 waves per block of 4096
// positions, cut into NW sub-blocks (one walking wave each).
//   match:  wave w takes the block's 64-position batches w, w + 16, ...; the
//           lanes holding the same id find each other with one ballot per id
//           bit, which gives each lane its rank among equal ids of the batch
//           and the group size. The group's lowest lane adds the size into
//           the count table of the batch's sub-block (one LDS add per
//           distinct id and batch: exact in any order), and (id, rank, group
//           size at the lowest lane) is packed into the block's LDS list.
//   bases:  for every id present in the block, the first destination of each
//           sub-block = segment offset + earlier segments + earlier blocks +
//           the counts of the earlier sub-blocks (global loads for present
//           ids, issued without branches).
//   chain:  each walking wave walks its sub-block in order, batch by batch:
//           destination = the id's running count + rank, written over the
//           packed entry, then the group's lowest lane advances the running
//           count: a stable counting sort. Within one wave the LDS read of an
//           id's running count precedes its leader's update in program order,
//           so no barrier is needed, and the chain touches only LDS.
//   store:  all waves write perm[destination] = p for the block's positions
//           (for the fused indexer dK the pair (p, coefficient of slot p)
//           instead: one 8-byte store, and the gather then reads every
//           coefficient in the sorted order instead of one random 4-byte
//           read per row).
// Packed match result: id (14 bits) | rank << 14 (6 bits) | size << 20 (7
// bits, 0 except at the group's lowest lane); -1 for ids out of range.
constexpr uint32_t kPackRank = 14, kPackSize = 20;

template <int NW>
__global__ __launch_bounds__(kSortThreads, 8) void ia_scatter(const int32_t* __restrict__ ids, int64_t n_src,
                                                              int n_rows, int tab_ld, int hist_ld,
                                                              const uint16_t* __restrict__ prefix,
                                                              const uint32_t* __restrict__ segbase,
                                                              const uint32_t* __restrict__ seg_off,
                                                              int32_t* __restrict__ perm,
                                                              const float* __restrict__ coef_in,
                                                              int2* __restrict__ pairs) {
  extern __shared__ uint32_t lds[];
  uint32_t* tab = lds;                                           // [NW][tab_ld], tab_ld = n_rows rounded up to 4
  int32_t* lid = reinterpret_cast<int32_t*>(lds + NW * tab_ld);  // [kBlockPos]
  constexpr int kWaves = kSortThreads / 64;
  constexpr int kSub = kBlockPos / NW;
  constexpr int kBatches = kBlockPos / 64;
  constexpr int kBpS = kBatches / NW;       // batches per sub-block
  constexpr int kMine = kBatches / kWaves;  // batches per wave
  static_assert(kMine * kWaves == kBatches && kBpS * NW == kBatches, "whole batches per wave and sub-block");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t b = blockIdx.x;
  const int64_t p0 = b * kBlockPos;
  const int64_t p1 = p0 + kBlockPos < n_src ? p0 + kBlockPos : n_src;
  int32_t x[kMine];
#pragma unroll
  for (int q = 0; q < kMine; ++q) {
    const int64_t p = p0 + 64 * (wave + kWaves * q) + lane;
    x[q] = p < p1 ? ids[p] : -1;
  }
  // The global part of every id's base (segment offset + earlier segments +
  // earlier blocks of the segment), loaded now for all ids k = tid + 1024 u
  // (one round covers every n_rows the LDS tables allow), so that the loads'
  // latency hides behind the match; absent ids' values are never used.
  constexpr int kU = 16 / NW;
  const uint16_t* pre = prefix + b * hist_ld;
  const uint32_t* sb = segbase + (b / kSegBlocks) * n_rows;
  uint32_t gbase[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int k = tid + kSortThreads * u;
    gbase[u] = k < n_rows ? seg_off[k] + sb[k] + pre[k] : 0u;
  }
  {
    uint4* t4 = reinterpret_cast<uint4*>(tab);
    for (int k = tid; k < NW * tab_ld / 4; k += kSortThreads) t4[k] = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  {
    const uint64_t lt = __lanemask_lt();
#pragma unroll
    for (int q = 0; q < kMine; ++q) {
      const int32_t id = x[q];
      const bool valid = id >= 0 && id < n_rows;
      const uint64_t peers = match_peers(id, valid);
      const uint32_t rank = static_cast<uint32_t>(__popcll(peers & lt));
      const uint32_t size = (valid && rank == 0) ? static_cast<uint32_t>(__popcll(peers)) : 0u;
      const int batch = wave + kWaves * q;
      if (size != 0) atomicAdd(&tab[(batch / kBpS) * tab_ld + id], size);
      lid[64 * batch + lane] =
          valid ? static_cast<int32_t>(static_cast<uint32_t>(id) | (rank << kPackRank) | (size << kPackSize)) : -1;
    }
  }
  __syncthreads();
  // bases: only ids present in the block need one (absent ids are never read
  // in the walk); each present id's sub-blocks start at its global base plus
  // the counts of the earlier sub-blocks
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int k = tid + kSortThreads * u;
    uint32_t c[NW];
    uint32_t any = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      c[w] = k < n_rows ? tab[w * tab_ld + k] : 0u;
      any |= c[w];
    }
    if (any != 0) {
      uint32_t run = gbase[u];
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        tab[w * tab_ld + k] = run;
        run += c[w];
      }
    }
  }
  __syncthreads();
  if (wave < NW) {
    uint32_t* t = tab + wave * tab_ld;
    int32_t* mine = lid + wave * kSub;
    constexpr int kSteps = kSub / 64;
#pragma unroll 8
    for (int q = 0; q < kSteps; ++q) {
      const int32_t xv = mine[64 * q + lane];
      if (xv >= 0) {
        const int32_t id = xv & 0x3FFF;
        const uint32_t rank = (static_cast<uint32_t>(xv) >> kPackRank) & 0x3Fu;
        const uint32_t size = (static_cast<uint32_t>(xv) >> kPackSize) & 0x7Fu;
        const uint32_t old = t[id];
        const uint64_t dest = static_cast<uint64_t>(old) + rank;
        mine[64 * q + lane] = dest < static_cast<uint64_t>(n_src) ? static_cast<int32_t>(dest) : -1;
        __builtin_amdgcn_wave_barrier();
        if (size != 0) t[id] = old + size;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();
  constexpr int kPerT = kBlockPos / kSortThreads;
  float cv[kPerT];
  if (coef_in) {
#pragma unroll
    for (int u = 0; u < kPerT; ++u) {
      const int64_t p = p0 + tid + kSortThreads * u;
      cv[u] = p < p1 ? coef_in[p] : 0.0f;
    }
  }
#pragma unroll
  for (int u = 0; u < kPerT; ++u) {
    const int pos = tid + kSortThreads * u;
    const int32_t d = lid[pos];
    if (d >= 0) {
      if (coef_in)
        pairs[d] = make_int2(static_cast<int32_t>(p0 + pos), __float_as_int(cv[u]));
      else
        perm[d] = static_cast<int32_t>(p0 + pos);
    }
  }
}

// Walking waves of the scatter: as many as fit while two workgroups still
// share a CU's 160 KiB of LDS (one count table per walking wave plus the
// block's ids), so that all blocks of the workload run in one round.
int scatter_waves(int64_t n_rows) {
  const int64_t pad_rows = (n_rows + 3) / 4 * 4;
  for (int nw = 4; nw > 1; nw /= 2)
    if (static_cast<int64_t>(nw) * pad_rows * 4 + kBlockPos * 4 <= 80 * 1024) return nw;
  return 1;
}
// The scatter loads every id's global base in one round, ids tid + 1024 u for
// u < 16 / NW: the LDS rule above leaves at most that many ids for each NW.
static_assert(kSortThreads * 16 >= kMaxRows && (80 * 1024 - kBlockPos * 4) / (2 * 4) <= kSortThreads * 8 &&
                  (80 * 1024 - kBlockPos * 4) / (4 * 4) <= kSortThreads * 4,
              "one round of bases per scatter workgroup");

template <int NW>
void launch_scatter(int64_t nblk, int n_rows, hipStream_t st, const int32_t* ids, int64_t n_src,
                    const uint16_t* hist, const uint32_t* segtot, const uint32_t* seg_off, int32_t* perm,
                    const float* coef_in, int2* pairs) {
  const int pad_rows = (n_rows + 3) / 4 * 4;  // table rows padded for 16-byte zeroing
  const size_t lds = static_cast<size_t>(NW) * pad_rows * 4 + kBlockPos * 4;
  if (lds > 64 * 1024) {
    static bool raised = false;  // allow up to the 160 KiB of a gfx950 workgroup, once per process
    if (!raised) {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(ia_scatter<NW>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      raised = true;
    }
  }
  hipLaunchKernelGGL(ia_scatter<NW>, dim3(static_cast<uint32_t>(nblk)), dim3(kSortThreads), lds, st, ids, n_src, n_rows,
                     pad_rows, hist_stride(n_rows), hist, segtot, seg_off, perm, coef_in, pairs);
}

// Binary search: the id whose chunk range [chunk_off[k], chunk_off[k+1]) holds c.
__device__ __forceinline__ int chunk_owner(const uint32_t* chunk_off, int n_rows, uint32_t c) {
  int lo = 0, hi = n_rows;  // invariant: chunk_off[lo] <= c < chunk_off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (chunk_off[mid] <= c) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ void add8_bf16(float (&acc)[8], const uint4& v) {
  acc[0] = acc[0] + bf16_lo(v.x); acc[1] = acc[1] + bf16_hi(v.x);
  acc[2] = acc[2] + bf16_lo(v.y); acc[3] = acc[3] + bf16_hi(v.y);
  acc[4] = acc[4] + bf16_lo(v.z); acc[5] = acc[5] + bf16_hi(v.z);
  acc[6] = acc[6] + bf16_lo(v.w); acc[7] = acc[7] + bf16_hi(v.w);
}

__device__ __forceinline__ void store_add8(float* dst, const float (&acc)[8]) {
  float4 a = *reinterpret_cast<const float4*>(dst);
  float4 b = *reinterpret_cast<const float4*>(dst + 4);
  a.x = a.x + acc[0]; a.y = a.y + acc[1]; a.z = a.z + acc[2]; a.w = a.w + acc[3];
  b.x = b.x + acc[4]; b.y = b.y + acc[5]; b.z = b.z + acc[6]; b.w = b.w + acc[7];
  *reinterpret_cast<float4*>(dst) = a;
  *reinterpret_cast<float4*>(dst + 4) = b;
}

// Eight consecutive source elements of one row: bf16 (one 16-byte load,
// widened exactly) or float32 (two 16-byte loads).
template <typename E>
struct Row8;
template <>
struct Row8<uint16_t> {
  uint4 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void clear() { v = make_uint4(0u, 0u, 0u, 0u); }
  __device__ __forceinline__ void add_to(float (&acc)[8]) const { add8_bf16(acc, v); }
  __device__ __forceinline__ float get(int i) const {
    const uint32_t w = i < 2 ? v.x : (i < 4 ? v.y : (i < 6 ? v.z : v.w));
    return (i & 1) ? bf16_hi(w) : bf16_lo(w);
  }
};
template <>
struct Row8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void clear() { a = b = make_float4(0.0f, 0.0f, 0.0f, 0.0f); }
  __device__ __forceinline__ void add_to(float (&acc)[8]) const {
    acc[0] = acc[0] + a.x; acc[1] = acc[1] + a.y; acc[2] = acc[2] + a.z; acc[3] = acc[3] + a.w;
    acc[4] = acc[4] + b.x; acc[5] = acc[5] + b.y; acc[6] = acc[6] + b.z; acc[7] = acc[7] + b.w;
  }
  __device__ __forceinline__ float get(int i) const {
    const float4& q = i < 4 ? a : b;
    const int r = i & 3;
    return r == 0 ? q.x : (r == 1 ? q.y : (r == 2 ? q.z : q.w));
  }
};

// ---- 5. chunk gather-sum. GS lanes per chunk, 8 dims per lane. The chunk's
// source positions (at most 16 per lane, GS * 16 rows) are loaded once,
// handed out by lane shuffles; the rows are then read up to 16 at a time (all
// their loads in flight) and folded in order.
constexpr int kPosPerLane = 16;  // chunk capacity of ia_gather: GS * 16 rows (longer chunks: ia_gather_long)

template <int GS, typename E>
__global__ __launch_bounds__(256) void ia_gather(const E* __restrict__ src, int64_t src_ld, int dim,
                                                 const int32_t* __restrict__ perm,
                                                 const uint32_t* __restrict__ seg_off,
                                                 const uint32_t* __restrict__ chunk_off, int n_rows, int L,
                                                 float* __restrict__ out, int64_t out_ld,
                                                 float* __restrict__ scratch, int64_t n_src, int64_t max_chunks) {
  const int g = threadIdx.x / GS;
  const int lg = threadIdx.x % GS;
  const uint32_t c = static_cast<uint32_t>(blockIdx.x) * (256 / GS) + g;
  const uint32_t n_chunks = chunk_off[n_rows];
  const bool live = c < n_chunks && c < max_chunks;
  int k = 0;
  uint32_t r0 = 0, len = 0;
  if (live) {
    k = chunk_owner(chunk_off, n_rows, c);
    const uint32_t j = c - chunk_off[k];
    r0 = seg_off[k] + j * static_cast<uint32_t>(L);
    const uint32_t r_end = seg_off[k + 1] < static_cast<uint64_t>(n_src) ? seg_off[k + 1] : static_cast<uint32_t>(n_src);
    len = r0 + static_cast<uint32_t>(L) < r_end ? static_cast<uint32_t>(L) : (r_end > r0 ? r_end - r0 : 0u);
  }
  const bool active = live && 8 * lg < dim;
  const int d0 = 8 * lg;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = -0.0f;
  // positions: lane lg of the group holds rows lg, lg + GS, lg + 2 GS, ...
  int32_t pos[kPosPerLane];
#pragma unroll
  for (int i = 0; i < kPosPerLane; ++i) {
    const uint32_t t = lg + GS * i;
    pos[i] = (live && t < len) ? perm[r0 + t] : 0;
  }
  constexpr int kBatch = GS < 16 ? GS : 16;  // rows whose loads are in flight together
#pragma unroll
  for (int i = 0; i < kPosPerLane; ++i) {
#pragma unroll
    for (int h = 0; h < GS; h += kBatch) {
      if (GS * i + h >= static_cast<int>(len)) continue;  // skipped when no lane of the wave needs it
      // rows GS*i + h .. GS*i + h + kBatch - 1 of the chunk
      Row8<E> v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int64_t p = __shfl(pos[i], h + u, GS);
        const bool ok = active && GS * i + h + u < static_cast<int>(len) && p >= 0 && p < n_src;
        if (ok)
          v[u].load(src + p * src_ld + d0);
        else
          v[u].clear();
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (active && GS * i + h + u < static_cast<int>(len)) v[u].add_to(acc);
    }
  }
  if (!active) return;
  const uint32_t nk = chunk_off[k + 1] - chunk_off[k];
  if (nk == 1) {
    store_add8(out + static_cast<int64_t>(k) * out_ld + d0, acc);
  } else {
    float* sp = scratch + static_cast<int64_t>(c) * dim + d0;
    *reinterpret_cast<float4*>(sp) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *reinterpret_cast<float4*>(sp + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

// One wave per chunk (dim = 64 * DPL, DPL in {2, 4, 8}): every lane owns DPL
// consecutive dims, so a row is one coalesced 64-lane load and a wave's time is
// its own chunk's length (several chunks of different lengths in one wave would
// leave lanes idle until the longest finishes). Up to 64 * 16 rows per chunk.
template <int DPL>
struct RowVec;
template <>
struct RowVec<2> { typedef uint32_t T; };
template <>
struct RowVec<4> { typedef uint2 T; };
template <>
struct RowVec<8> { typedef uint4 T; };

__device__ __forceinline__ void add_bf16(float (&acc)[2], uint32_t v) {
  acc[0] = acc[0] + bf16_lo(v); acc[1] = acc[1] + bf16_hi(v);
}
__device__ __forceinline__ void add_bf16(float (&acc)[4], uint2 v) {
  acc[0] = acc[0] + bf16_lo(v.x); acc[1] = acc[1] + bf16_hi(v.x);
  acc[2] = acc[2] + bf16_lo(v.y); acc[3] = acc[3] + bf16_hi(v.y);
}
__device__ __forceinline__ void add_bf16(float (&acc)[8], uint4 v) { add8_bf16(acc, v); }
// bf16 -0.0 in every element: adding it leaves an fp32 accumulator unchanged bit for bit
__device__ __forceinline__ uint32_t neg_zero_vec(uint32_t) { return 0x80008000u; }
__device__ __forceinline__ uint2 neg_zero_vec(uint2) { return make_uint2(0x80008000u, 0x80008000u); }
__device__ __forceinline__ uint4 neg_zero_vec(uint4) { return make_uint4(0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u); }
__device__ __forceinline__ uint32_t zero_vec(uint32_t) { return 0u; }
__device__ __forceinline__ uint2 zero_vec(uint2) { return make_uint2(0u, 0u); }
__device__ __forceinline__ uint4 zero_vec(uint4) { return make_uint4(0u, 0u, 0u, 0u); }

// Source rows made on the fly (the fused indexer dK): source row p is
// RN32(coef[p] * q[p / K]), q being the bf16 query rows (row stride q_ld).
struct FusedSrc {
  const float* coef;         // by slot p (the atomic arm)
  const int2* pairs;         // by sorted row r: (slot, coefficient bits) (the gather)
  uint32_t K, krcp;
};

__device__ __forceinline__ void add_scaled_bf16(float (&acc)[2], uint32_t v, float c) {
  acc[0] = acc[0] + c * bf16_lo(v); acc[1] = acc[1] + c * bf16_hi(v);
}
__device__ __forceinline__ void add_scaled_bf16(float (&acc)[4], uint2 v, float c) {
  acc[0] = acc[0] + c * bf16_lo(v.x); acc[1] = acc[1] + c * bf16_hi(v.x);
  acc[2] = acc[2] + c * bf16_lo(v.y); acc[3] = acc[3] + c * bf16_hi(v.y);
}
__device__ __forceinline__ void add_scaled_bf16(float (&acc)[8], uint4 v, float c) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    acc[2 * k] = acc[2 * k] + c * bf16_lo(w[k]);
    acc[2 * k + 1] = acc[2 * k + 1] + c * bf16_hi(w[k]);
  }
}

template <int DPL, int NPOS, bool FUSED = false>
__global__ __launch_bounds__(256) void ia_gather_wave(const uint16_t* __restrict__ src, int64_t src_ld, int dim,
                                                      const int32_t* __restrict__ perm,
                                                      const uint32_t* __restrict__ chunk_off,
                                                      const int4* __restrict__ desc, int n_rows,
                                                      float* __restrict__ out, int64_t out_ld,
                                                      float* __restrict__ scratch, int64_t n_src,
                                                      int64_t max_chunks, FusedSrc fz) {
  typedef typename RowVec<DPL>::T V;
  const int lane = threadIdx.x & 63;
  const uint32_t w = static_cast<uint32_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (w >= max_chunks) return;  // wave-uniform
  // the descriptor load does not wait for the chunk count: entries past the
  // count are read but never used
  const uint32_t n_chunks = chunk_off[n_rows];
  const int4 dsc = desc[w];
  if (w >= n_chunks) return;  // wave-uniform
  const int k = dsc.x;
  const uint32_t r0 = static_cast<uint32_t>(dsc.y);
  const int len = dsc.z;
  const int slot = dsc.w;  // canonical chunk index, or -1: the id's only chunk
  const int d0 = DPL * lane;
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = -0.0f;
  // NPOS * 64 >= the chunk length: positions beyond len are never read
  int32_t pos[NPOS];
  // fused source: the sorted (slot, coefficient) pairs; each lane turns its
  // slots into query rows once (rows past the chunk end take 1.0, see below)
  int32_t qrow[NPOS];
  float cf[NPOS];
#pragma unroll
  for (int i = 0; i < NPOS; ++i) {
    const bool in = 64 * i + lane < len;
    if (FUSED) {
      const int2 pr = fz.pairs[in ? r0 + 64 * i + lane : r0];
      pos[i] = in ? pr.x : 0;
      cf[i] = in ? __int_as_float(pr.y) : 1.0f;
    } else {
      const int32_t x = perm[in ? r0 + 64 * i + lane : r0];
      pos[i] = in ? x : 0;
    }
  }
  if (FUSED) {
#pragma unroll
    for (int i = 0; i < NPOS; ++i) {
      const bool ok = 64 * i + lane < len && pos[i] >= 0 && pos[i] < n_src;
      const uint32_t pp = ok ? static_cast<uint32_t>(pos[i]) : 0u;
      qrow[i] = static_cast<int32_t>(floor_div_rcp(pp, fz.K, fz.krcp));
      if (!ok) cf[i] = 1.0f;
    }
  }
  // a single-chunk id adds into out directly: its out row is fetched now,
  // while the row loads are in flight
  float* const dst = slot < 0 ? out + static_cast<int64_t>(k) * out_ld + d0 : scratch + static_cast<int64_t>(slot) * dim + d0;
  float o[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) o[i] = slot < 0 ? dst[i] : 0.0f;
  // rows whose loads are in flight together: 32 / 16 / 8 for 4 / 8 / 16-byte rows
  // (few registers, so eight waves fit on a SIMD).
  // A row's position is read from its lane with readlane (wave-uniform, so
  // the row address is scalar); rows past the chunk end load a valid row and
  // add -0.0 instead, which leaves every value bitwise unchanged, so the
  // adds need no branches.
  constexpr int kB = 64 / DPL;
#pragma unroll
  for (int i = 0; i < NPOS; ++i) {
#pragma unroll
    for (int h = 0; h < 64; h += kB) {
      if (64 * i + h >= len) continue;  // wave-uniform skip
      V v[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        int64_t p;
        if (FUSED) {
          p = __builtin_amdgcn_readlane(qrow[i], h + u);  // a query row below Q
        } else {
          p = __builtin_amdgcn_readlane(pos[i], h + u);
          p = (p >= 0 && p < n_src) ? p : 0;  // always a valid row
        }
        v[u] = *reinterpret_cast<const V*>(src + p * src_ld + d0);
      }
      if (FUSED) {
        // past the chunk end: bf16 -0.0 times 1.0 is -0.0, which leaves every sum unchanged
#pragma unroll
        for (int u = 0; u < kB; ++u)
          add_scaled_bf16(acc, 64 * i + h + u < len ? v[u] : neg_zero_vec(v[u]),
                          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cf[i]), h + u)));
      } else {
#pragma unroll
        for (int u = 0; u < kB; ++u) add_bf16(acc, 64 * i + h + u < len ? v[u] : neg_zero_vec(v[u]));
      }
    }
  }
#pragma unroll
  for (int i = 0; i < DPL; ++i) dst[i] = (slot < 0 ? o[i] + acc[i] : acc[i]);
}

// The same gather with the rows loaded through a buffer resource (source
// tensors below 2^31 bytes): every lane holds the 32-bit byte offsets of its
// positions' rows, computed once, so a row costs one readlane and one load,
// and a rolling window keeps kB row loads in flight across the chunk (the row
// that leaves the window is added, the next one is issued into its place).
// Rows past the chunk end are not loaded: their offset is out of the resource
// range (the load returns zeros without a memory access) and -0.0 is added in
// their place, which leaves every sum bitwise unchanged. Same fold order as
// ia_gather_wave: rows left to right from -0.0.
template <typename V>
__device__ __forceinline__ V buf_load(__amdgpu_buffer_rsrc_t r, int32_t voff, int32_t soff);
template <>
__device__ __forceinline__ uint32_t buf_load<uint32_t>(__amdgpu_buffer_rsrc_t r, int32_t voff, int32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
template <>
__device__ __forceinline__ uint2 buf_load<uint2>(__amdgpu_buffer_rsrc_t r, int32_t voff, int32_t soff) {
  typedef uint32_t u2 __attribute__((ext_vector_type(2)));
  const u2 v = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
  return make_uint2(v[0], v[1]);
}
template <>
__device__ __forceinline__ uint4 buf_load<uint4>(__amdgpu_buffer_rsrc_t r, int32_t voff, int32_t soff) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  const u4 v = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int DPL, int NPOS>
__global__ __launch_bounds__(256) void ia_gather_buf(const uint16_t* __restrict__ src, int64_t src_ld, int dim,
                                                     uint32_t src_bytes, const int32_t* __restrict__ perm,
                                                     const uint32_t* __restrict__ chunk_off,
                                                     const int4* __restrict__ desc, int n_rows,
                                                     float* __restrict__ out, int64_t out_ld,
                                                     float* __restrict__ scratch, int64_t n_src,
                                                     int64_t max_chunks) {
  typedef typename RowVec<DPL>::T V;
  const int lane = threadIdx.x & 63;
  const uint32_t w = static_cast<uint32_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (w >= max_chunks) return;  // wave-uniform
  const uint32_t n_chunks = chunk_off[n_rows];
  const int4 dsc = desc[w];
  if (w >= n_chunks) return;  // wave-uniform
  // the descriptor is the same in every lane: keep it in scalar registers
  const int k = __builtin_amdgcn_readfirstlane(dsc.x);
  const uint32_t r0 = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(dsc.y));
  const int len = __builtin_amdgcn_readfirstlane(dsc.z);
  const int slot = __builtin_amdgcn_readfirstlane(dsc.w);
  const int d0 = DPL * lane;
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = -0.0f;
  const uint32_t row_bytes = static_cast<uint32_t>(src_ld) * 2u;
  uint32_t off[NPOS];
#pragma unroll
  for (int i = 0; i < NPOS; ++i) {
    const bool in = 64 * i + lane < len;
    const int32_t x = perm[in ? r0 + 64 * i + lane : r0];
    const bool ok = in && x >= 0 && x < n_src;  // always a valid row
    off[i] = (ok ? static_cast<uint32_t>(x) : 0u) * row_bytes;
  }
  float* const dst = slot < 0 ? out + static_cast<int64_t>(k) * out_ld + d0 : scratch + static_cast<int64_t>(slot) * dim + d0;
  float o[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) o[i] = slot < 0 ? dst[i] : 0.0f;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(src), 0,
                                                                      static_cast<int>(src_bytes), 0x00020000);
  const int32_t voff = d0 * 2;
  constexpr int kB = 64 / DPL;           // loads in flight
  constexpr int kRows = 64 * NPOS;
  // soffset of row r: its byte offset, or past the resource (no load) beyond the chunk
#define DET_IA_SOFF(r) ((r) < len ? static_cast<int32_t>(__builtin_amdgcn_readlane(off[(r) / 64], (r) % 64)) \
                                  : static_cast<int32_t>(0x80000000u))
  V buf[kB];
#pragma unroll
  for (int u = 0; u < kB; ++u) buf[u] = buf_load<V>(rs, voff, DET_IA_SOFF(u));
#pragma unroll
  for (int b = 0; b < kRows / kB; ++b) {
    if (b * kB >= len) break;  // wave-uniform
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int r = b * kB + u;
      const V x = buf[u];
      if (r + kB < kRows) buf[u] = buf_load<V>(rs, voff, DET_IA_SOFF(r + kB));
      add_bf16(acc, r < len ? x : neg_zero_vec(x));
    }
  }
#undef DET_IA_SOFF
#pragma unroll
  for (int i = 0; i < DPL; ++i) dst[i] = (slot < 0 ? o[i] + acc[i] : acc[i]);
}

// The fused gather at dim 128: four chunks per wave, a 16-lane group per chunk
// and 8 dims per lane, so a query row is one 16-byte load per lane and a wave
// instruction reads four rows (a quarter of the load instructions of the
// one-wave-per-chunk form, whose 4-byte loads of L2-resident query rows are
// limited by the address units). Lane lg of a group holds the (slot,
// coefficient) pairs of rows lg, lg + 16, ...; row r's query-row offset and
// coefficient reach the group by a DPP row broadcast from lane r % 16. Each
// group folds its own chunk left to right from -0.0; rows past a group's
// chunk end load nothing (offset outside the resource) and add -0.0 times
// 1.0, which leaves its sum bitwise unchanged. A wave runs as many rows as
// its longest chunk (the descriptor list gives the full chunks first, so most
// waves hold four chunks of equal length).
constexpr int kQuadInFlight = 4;  // rows of each group in flight (fewer registers, more waves per SIMD)

template <int R>
__device__ __forceinline__ uint32_t row_bcast16(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x150 + R, 0xF, 0xF, false));
}

// Steps U.. of block B (rows B * KB + U): add the row that leaves the window,
// load the row KB ahead into its place.
template <bool UNI, int KB, int B, int U>
__device__ __forceinline__ void quad_steps(__amdgpu_buffer_rsrc_t rs, int32_t lgoff, const uint32_t (&off)[16],
                                           const uint32_t (&cf)[16], int len, float (&acc)[8], uint4 (&buf)[KB]) {
  if constexpr (U < KB) {
    constexpr int r = B * KB + U;
    const uint4 x = buf[U];
    if constexpr (r + KB < 256)
      buf[U] = buf_load<uint4>(rs, static_cast<int32_t>(row_bcast16<(r + KB) % 16>(off[(r + KB) / 16])) + lgoff, 0);
    const uint4 v = (UNI || r < len) ? x : make_uint4(0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u);
    add_scaled_bf16(acc, v, __uint_as_float(row_bcast16<r % 16>(cf[r / 16])));
    quad_steps<UNI, KB, B, U + 1>(rs, lgoff, off, cf, len, acc, buf);
  }
}

template <bool UNI, int KB, int B>
__device__ __forceinline__ void quad_blocks(__amdgpu_buffer_rsrc_t rs, int32_t lgoff, const uint32_t (&off)[16],
                                            const uint32_t (&cf)[16], int len, int lmax, float (&acc)[8],
                                            uint4 (&buf)[KB]) {
  if constexpr (B * KB < 256) {
    if (B * KB >= lmax) return;  // wave-uniform
    quad_steps<UNI, KB, B, 0>(rs, lgoff, off, cf, len, acc, buf);
    quad_blocks<UNI, KB, B + 1>(rs, lgoff, off, cf, len, lmax, acc, buf);
  }
}

template <int KB, int U>
__device__ __forceinline__ void quad_prologue(__amdgpu_buffer_rsrc_t rs, int32_t lgoff, const uint32_t (&off)[16],
                                              uint4 (&buf)[KB]) {
  if constexpr (U < KB) {
    buf[U] = buf_load<uint4>(rs, static_cast<int32_t>(row_bcast16<U % 16>(off[U / 16])) + lgoff, 0);
    quad_prologue<KB, U + 1>(rs, lgoff, off, buf);
  }
}

// UNI: all four chunks have the wave's length (a multiple of KB): no per-row select.
template <bool UNI, int KB>
__device__ __forceinline__ void quad_run(std::integral_constant<bool, UNI>, __amdgpu_buffer_rsrc_t rs, int32_t lgoff,
                                         const uint32_t (&off)[16], const uint32_t (&cf)[16], int len, int lmax,
                                         float (&acc)[8]) {
  uint4 buf[KB];
  quad_prologue<KB, 0>(rs, lgoff, off, buf);
  quad_blocks<UNI, KB, 0>(rs, lgoff, off, cf, len, lmax, acc, buf);
}

__global__ __launch_bounds__(256) void ia_gather_quad(const uint16_t* __restrict__ q, int64_t q_ld, uint32_t q_bytes,
                                                      const uint32_t* __restrict__ chunk_off,
                                                      const int4* __restrict__ desc, int n_rows,
                                                      float* __restrict__ out, int64_t out_ld,
                                                      float* __restrict__ scratch, int64_t n_src, int64_t max_chunks,
                                                      FusedSrc fz) {
  constexpr int KB = kQuadInFlight;
  const int lane = threadIdx.x & 63, lg = lane & 15;
  const uint32_t c0 = 4 * (static_cast<uint32_t>(blockIdx.x) * 4 + (threadIdx.x >> 6));
  if (c0 >= max_chunks) return;  // wave-uniform
  const uint32_t n_chunks = chunk_off[n_rows];
  if (c0 >= n_chunks) return;  // wave-uniform
  const uint32_t c = c0 + (lane >> 4);
  const bool live = c < n_chunks && c < max_chunks;
  const int4 dsc = desc[live ? c : c0];
  const int k = dsc.x;
  const uint32_t r0 = static_cast<uint32_t>(dsc.y);
  const int len = live ? dsc.z : 0;
  const int slot = dsc.w;
  const int l0 = __builtin_amdgcn_readlane(len, 0), l1 = __builtin_amdgcn_readlane(len, 16);
  const int l2 = __builtin_amdgcn_readlane(len, 32), l3 = __builtin_amdgcn_readlane(len, 48);
  const int lmax = max(max(l0, l1), max(l2, l3));
  const bool uni = l0 == lmax && l1 == lmax && l2 == lmax && l3 == lmax && lmax % KB == 0;
  const uint32_t row_bytes = static_cast<uint32_t>(q_ld) * 2u;
  uint32_t off[16], cf[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = lg + 16 * i;
    const bool in = t < len;
    const int2 pr = fz.pairs[in ? r0 + t : r0];
    const bool ok = in && pr.x >= 0 && pr.x < n_src;  // always a valid slot
    const uint32_t pp = ok ? static_cast<uint32_t>(pr.x) : 0u;
    off[i] = in ? floor_div_rcp(pp, fz.K, fz.krcp) * row_bytes : 0x80000000u;
    cf[i] = in ? static_cast<uint32_t>(pr.y) : __float_as_uint(1.0f);
  }
  const int d0 = 8 * lg;
  float* const dst = slot < 0 ? out + static_cast<int64_t>(k) * out_ld + d0 : scratch + static_cast<int64_t>(slot) * 128 + d0;
  float4 oa = make_float4(0.0f, 0.0f, 0.0f, 0.0f), ob = oa;
  if (live && slot < 0) {
    oa = *reinterpret_cast<const float4*>(dst);
    ob = *reinterpret_cast<const float4*>(dst + 4);
  }
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = -0.0f;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(q), 0,
                                                                      static_cast<int>(q_bytes), 0x00020000);
  if (uni)
    quad_run<true, KB>(std::integral_constant<bool, true>(), rs, d0 * 2, off, cf, len, lmax, acc);
  else
    quad_run<false, KB>(std::integral_constant<bool, false>(), rs, d0 * 2, off, cf, len, lmax, acc);
  if (!live) return;
  if (slot < 0) {
    oa.x = oa.x + acc[0]; oa.y = oa.y + acc[1]; oa.z = oa.z + acc[2]; oa.w = oa.w + acc[3];
    ob.x = ob.x + acc[4]; ob.y = ob.y + acc[5]; ob.z = ob.z + acc[6]; ob.w = ob.w + acc[7];
  } else {
    oa = make_float4(acc[0], acc[1], acc[2], acc[3]);
    ob = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
  *reinterpret_cast<float4*>(dst) = oa;
  *reinterpret_cast<float4*>(dst + 4) = ob;
}

// Chunks longer than GS * 16 rows (a large chunk_rows setting): one lane group
// walks the rows with the permutation read as it goes.
template <int GS, typename E>
__global__ __launch_bounds__(256) void ia_gather_long(const E* __restrict__ src, int64_t src_ld, int dim,
                                                      const int32_t* __restrict__ perm,
                                                      const uint32_t* __restrict__ seg_off,
                                                      const uint32_t* __restrict__ chunk_off, int n_rows, int L,
                                                      float* __restrict__ out, int64_t out_ld,
                                                      float* __restrict__ scratch, int64_t n_src,
                                                      int64_t max_chunks) {
  const int g = threadIdx.x / GS;
  const int lg = threadIdx.x % GS;
  const uint32_t c = static_cast<uint32_t>(blockIdx.x) * (256 / GS) + g;
  const uint32_t n_chunks = chunk_off[n_rows];
  if (c >= n_chunks || c >= max_chunks) return;
  const int k = chunk_owner(chunk_off, n_rows, c);
  const uint32_t j = c - chunk_off[k];
  const uint32_t r0 = seg_off[k] + j * static_cast<uint32_t>(L);
  const uint32_t r_end = seg_off[k + 1];
  uint32_t r1 = r0 + static_cast<uint32_t>(L) < r_end ? r0 + static_cast<uint32_t>(L) : r_end;
  if (r1 > static_cast<uint64_t>(n_src)) r1 = static_cast<uint32_t>(n_src);
  const bool active = 8 * lg < dim;
  const int d0 = 8 * lg;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = -0.0f;
  constexpr int kU = 8;
  for (uint32_t r = r0; r < r1; r += kU) {
    Row8<E> v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (active && r + u < r1) {
        const int64_t p = perm[r + u];
        if (p >= 0 && p < n_src)
          v[u].load(src + p * src_ld + d0);
        else
          v[u].clear();
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (active && r + u < r1) v[u].add_to(acc);
  }
  if (!active) return;
  const uint32_t nk = chunk_off[k + 1] - chunk_off[k];
  if (nk == 1) {
    store_add8(out + static_cast<int64_t>(k) * out_ld + d0, acc);
  } else {
    float* sp = scratch + static_cast<int64_t>(c) * dim + d0;
    *reinterpret_cast<float4*>(sp) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *reinterpret_cast<float4*>(sp + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

// ---- 6. fold of multi-chunk ids. The dimensions are cut into slices of DS
// (8, 16 or 32) and a workgroup owns one slice of the ids k = gi + groups j
// (at most 64 ids per group: n_rows <= 64 groups); lane j of each wave reads
// that id's chunk range in one go, and the workgroup folds the ids with
// several chunks one after another. The slices of one id run on different
// compute units, so the longest run (the hottest key) is spread over
// dim / DS of them.
//
// Lane d of wave 0 adds dimension d of the slice, left to right over the id's
// chunk partials: one dependent add chain per dimension, fed from LDS. The
// partials (contiguous in scratch from slot chunk_off[k]) pass through LDS in
// rounds of R = 8192 / DS chunks, transposed to [DS][R] so that one 16-byte
// LDS read gives a lane four consecutive chunks of its dimension. Every
// thread loads two 4 x 4 blocks per round (4 chunks x 4 dims, four 16-byte
// loads each), turns them around in registers and stores four 16-byte
// vectors; chunks past the id's last one are stored as -0.0, which leaves a
// chain bitwise unchanged, so every round is added in whole groups of 64
// chunks. The 16-byte column blocks of row d are XOR-swizzled (fold_swz), so
// that neither the reads nor the stores have bank conflicts. The loads of the
// next two rounds are in flight in registers while a round is added; the two
// LDS buffers alternate.
constexpr int kFoldGroups = 256;  // id groups
static_assert(kFoldGroups * 64 >= kMaxRows, "a fold group owns at most 64 ids");
constexpr int kFoldFloats = 8192;  // floats per LDS round buffer (32 KiB): DS * R
constexpr int kFoldDirect = 32;    // ids with at most this many chunks are folded by one wave

inline int fold_slice(int64_t dim) { return dim % 32 == 0 ? 32 : (dim % 16 == 0 ? 16 : 8); }

// Column-block swizzle of dimension row d (a value below 16, XORed into the
// low four bits of the block index). With D4 = DS / 4 dim groups per chunk,
// 16 consecutive store lanes are 16 / D4 consecutive column blocks times the
// D4 groups: the group g = d / 4 fills the block bits above those the lanes'
// own blocks vary in. The 16 rows a read covers differ in g % 4 and d % 4,
// which fill the remaining bits.
template <int DS>
__device__ __forceinline__ int fold_swz(int d) {
  constexpr int s = DS == 32 ? 1 : (DS == 16 ? 2 : 3);
  const int e = d & 3;
  const int ee = DS == 32 ? ((e & 1) | ((e >> 1) << 3)) : e;
  return ((d >> 2) << s) ^ ee;
}

template <int DS>
__global__ __launch_bounds__(256) void ia_fold(const uint32_t* __restrict__ chunk_off, int n_rows, int dim,
                                               const float* __restrict__ scratch, float* __restrict__ out,
                                               int64_t out_ld) {
  constexpr int R = kFoldFloats / DS;  // chunks per round
  constexpr int NG = R / 64;           // groups of 64 chunks per round
  constexpr int D4 = DS / 4;           // 4-dim groups per chunk of the slice
  static_assert((R / 4) * D4 == 512, "512 4 x 4 blocks per round");
  __shared__ __attribute__((aligned(16))) float buf[2][kFoldFloats];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int parts = dim / DS;
  const int groups = static_cast<int>(gridDim.x) / parts;
  const int gi = static_cast<int>(blockIdx.x) / parts;
  const int d0 = DS * (static_cast<int>(blockIdx.x) % parts);
  const int kj = gi + groups * lane;
  const uint32_t lo_j = kj < n_rows ? chunk_off[kj] : 0u, hi_j = kj < n_rows ? chunk_off[kj + 1] : 0u;
  const uint32_t nj = hi_j - lo_j;
  // the same masks in every wave
  uint64_t small = __ballot(nj >= 2 && nj <= kFoldDirect);
  uint64_t big = __ballot(nj > kFoldDirect);

  // ids with at most kFoldDirect chunks: one wave each, in turn; lane d loads
  // dimension d of every chunk partial at once and adds them left to right
  // (chunks past the last add -0.0, which changes no bit)
  for (int i = 0; small; small &= small - 1, ++i) {
    if ((i & 3) != wave) continue;
    const int j = __builtin_ctzll(small);
    const int k = gi + groups * j;
    const uint32_t c0 = __builtin_amdgcn_readlane(lo_j, j);
    const int n = static_cast<int>(__builtin_amdgcn_readlane(nj, j));
    if (lane < DS) {
      const float* p = scratch + static_cast<int64_t>(c0) * dim + d0 + lane;
      float x[kFoldDirect];
#pragma unroll
      for (int c = 0; c < kFoldDirect; ++c) x[c] = c < n ? p[static_cast<int64_t>(c) * dim] : -0.0f;
      float a = -0.0f;
#pragma unroll
      for (int c = 0; c < kFoldDirect; ++c) a = a + x[c];
      float* const o = out + static_cast<int64_t>(k) * out_ld + d0 + lane;
      *o = *o + a;
    }
  }

  // longer runs: the whole workgroup; waves 1..3 stage the rounds through LDS,
  // wave 0 runs the add chains
  const int u = tid - 64;  // staging thread (waves 1..3): blocks u, u + 192 and (u < 128) u + 384
  while (big) {
    const int j = __builtin_ctzll(big);
    big &= big - 1;
    const int k = gi + groups * j;
    const uint32_t c0 = __builtin_amdgcn_readlane(lo_j, j);
    const int n = static_cast<int>(__builtin_amdgcn_readlane(nj, j));
    const int rounds = (n + R - 1) / R;
    // block b = cb * D4 + g: chunks 4 cb .. 4 cb + 3 of the round, dims 4 g .. 4 g + 3 of the slice
    float4 va[3][4], vb[3][4];
    auto load = [&](float4 (&v)[3][4], int r) {
      // one buffer resource per round (offsets stay below R * dim * 4 <= 2 MiB);
      // partials past the id's last chunk read as zero (stored as -0.0)
      const int left = n - r * R;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(scratch + (static_cast<int64_t>(c0) + static_cast<int64_t>(r) * R) * dim + d0), 0,
          ((left < R ? left : R) * dim - d0) * 4, 0x00020000);
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        if (q == 2 && wave == 3) break;
        const int b = u + 192 * q;
        const int cb = b / D4, g = b % D4;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[q][e] = __builtin_bit_cast(
              float4, __builtin_amdgcn_raw_buffer_load_b128(rs, ((4 * cb + e) * dim + 4 * g) * 4, 0, 0));
      }
    };
    auto store = [&](const float4 (&v)[3][4], int r) {
      float* const bb = buf[r & 1];
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        if (q == 2 && wave == 3) break;
        const int b = u + 192 * q;
        const int cb = b / D4, g = b % D4;
        float4 w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = r * R + 4 * cb + e < n ? v[q][e] : make_float4(-0.0f, -0.0f, -0.0f, -0.0f);
        const int d = 4 * g;
        *reinterpret_cast<float4*>(bb + (d + 0) * R + 4 * (cb ^ fold_swz<DS>(d + 0))) = make_float4(w[0].x, w[1].x, w[2].x, w[3].x);
        *reinterpret_cast<float4*>(bb + (d + 1) * R + 4 * (cb ^ fold_swz<DS>(d + 1))) = make_float4(w[0].y, w[1].y, w[2].y, w[3].y);
        *reinterpret_cast<float4*>(bb + (d + 2) * R + 4 * (cb ^ fold_swz<DS>(d + 2))) = make_float4(w[0].z, w[1].z, w[2].z, w[3].z);
        *reinterpret_cast<float4*>(bb + (d + 3) * R + 4 * (cb ^ fold_swz<DS>(d + 3))) = make_float4(w[0].w, w[1].w, w[2].w, w[3].w);
      }
    };
    // 64-chunk group h of dimension row `row`: 16 16-byte reads
    const int f = fold_swz<DS>(lane & (DS - 1));
    auto rd = [&](float4 (&x)[16], const float* row, int h) {
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = *reinterpret_cast<const float4*>(row + 4 * (16 * h + (i ^ f)));
    };
    auto add = [&](const float4 (&x)[16], float a) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        a = a + x[i].x;
        a = a + x[i].y;
        a = a + x[i].z;
        a = a + x[i].w;
      }
      return a;
    };
    __syncthreads();  // the previous id's reads of both buffers are done
    if (wave != 0) {
      load(va, 0);
      if (rounds > 1) load(vb, 1);
      store(va, 0);
      if (rounds > 2) load(va, 2);
    }
    __syncthreads();
    float a = -0.0f;
    // round r: wave 0 adds buffer r & 1, 64 chunks per group with the next
    // group's reads in flight; meanwhile round r + 1 (registers of parity
    // (r + 1) & 1) goes to the other buffer and those registers take the
    // loads of round r + 3
#define DET_IA_FOLD_ROUND(r, vnext)                                                     \
  {                                                                                      \
    if (wave == 0) {                                                                     \
      if (lane < DS) {                                                                   \
        const float* const row = buf[(r) & 1] + lane * R;                                \
        const int m = n - (r) * R < R ? n - (r) * R : R;                                 \
        const int ng = (m + 63) / 64;                                                    \
        float4 xa[16], xb[16];                                                           \
        rd(xa, row, 0);                                                                  \
        _Pragma("unroll") for (int h = 0; h < NG; h += 2) {                              \
          if (h < ng) {                                                                  \
            if (h + 1 < ng) rd(xb, row, h + 1);                                          \
            __builtin_amdgcn_sched_barrier(0);                                           \
            a = add(xa, a);                                                              \
          }                                                                              \
          if (h + 1 < ng) {                                                              \
            if (h + 2 < ng) rd(xa, row, h + 2);                                          \
            __builtin_amdgcn_sched_barrier(0);                                           \
            a = add(xb, a);                                                              \
          }                                                                              \
        }                                                                                \
      }                                                                                  \
    } else if ((r) + 1 < rounds) {                                                       \
      store(vnext, (r) + 1);                                                             \
      if ((r) + 3 < rounds) load(vnext, (r) + 3);                                        \
    }                                                                                    \
    __syncthreads();                                                                     \
  }
    for (int r = 0; r < rounds; r += 2) {
      DET_IA_FOLD_ROUND(r, vb)
      if (r + 1 >= rounds) break;
      DET_IA_FOLD_ROUND(r + 1, va)
    }
#undef DET_IA_FOLD_ROUND
    if (wave == 0 && lane < DS) {
      float* const o = out + static_cast<int64_t>(k) * out_ld + d0 + lane;
      *o = *o + a;
    }
  }
}

// ---- atomic arm: per-element float atomics, no sort
template <int GS, typename E>
__global__ __launch_bounds__(256) void ia_atomic(const int32_t* __restrict__ ids, int64_t n_src,
                                                 const E* __restrict__ src, int64_t src_ld, int dim, int n_rows,
                                                 float* __restrict__ out, int64_t out_ld) {
  const int g = threadIdx.x / GS;
  const int lg = threadIdx.x % GS;
  const int64_t p = static_cast<int64_t>(blockIdx.x) * (256 / GS) + g;
  if (p >= n_src || 8 * lg >= dim) return;
  const int32_t id = ids[p];
  if (id < 0 || id >= n_rows) return;
  const int d0 = 8 * lg;
  Row8<E> v;
  v.load(src + p * src_ld + d0);
  float* o = out + static_cast<int64_t>(id) * out_ld + d0;
#pragma unroll
  for (int i = 0; i < 8; ++i) unsafeAtomicAdd(o + i, v.get(i));
}

// ---- fused indexer dK: per-slot coefficients of the clipped-KL score gradient
// (DSv4 page, source 3 fix). One wave per query row, four rows per workgroup.
// Lane l holds slots 8 l .. 8 l + 7 of each 512-slot piece of the row (16-byte
// loads of ids, target and predict, all issued at once) and turns its targets
// into kept targets (max(target, e^-100) on a slot whose id lies in
// [0, n_rows), +0 elsewhere and past K). The row sum S is then the ordered
// chain over the slots, each value fetched from its lane with readlane (an
// appended +0 never changes a non-empty sum); finally every slot gets
// c = RN32(RN32(RN32(predict * S) - kept) * scale), and 0 on a dropped slot.
constexpr uint32_t kEps100Bits = 0x0000001Bu;  // the float32 nearest e^-100 (27 * 2^-149)
constexpr int kCoefPiece = 512;                // slots per piece: 64 lanes x 8
constexpr int kCoefMaxPieces = 2;              // K <= 1024
constexpr int kCoefAhead = 16;                 // LDS loads in flight ahead of the S chain

__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8(const int32_t* p, int32_t (&v)[8]) {
  const int4 a = *reinterpret_cast<const int4*>(p), b = *reinterpret_cast<const int4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <int PIECES, bool VEC>
__global__ __launch_bounds__(256) void ia_coef(const int32_t* __restrict__ ids, const float* __restrict__ predict,
                                               const float* __restrict__ target, int64_t Q, int K, int n_rows,
                                               float scale, float* __restrict__ coef) {
  const int lane = threadIdx.x & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= Q) return;  // wave-uniform
  const int64_t base = r * K;
  const float eps = __uint_as_float(kEps100Bits);
  int32_t id[PIECES][8];
  float tg[PIECES][8], pr[PIECES][8];
#pragma unroll
  for (int c = 0; c < PIECES; ++c) {
    const int j0 = c * kCoefPiece + 8 * lane;
    if (VEC && j0 + 8 <= K) {  // K % 8 == 0 here, so a piece's lane is all in or all out
      load8(ids + base + j0, id[c]);
      load8(target + base + j0, tg[c]);
      load8(predict + base + j0, pr[c]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool in = j0 + e < K;
        id[c][e] = in ? ids[base + j0 + e] : -1;
        tg[c][e] = in ? target[base + j0 + e] : 0.0f;
        pr[c][e] = in ? predict[base + j0 + e] : 0.0f;
      }
    }
  }
  float kept[PIECES][8];
#pragma unroll
  for (int c = 0; c < PIECES; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool valid = id[c][e] >= 0 && id[c][e] < n_rows;  // slots past K carry id -1
      // max(target, eps) that keeps a NaN target, as numpy's maximum does
      kept[c][e] = valid ? (!(tg[c][e] <= eps) ? tg[c][e] : eps) : 0.0f;
    }
  // S = ((-0 + kept_0) + kept_1) + ... in slot order. Slot 512 c + 8 l + e sits
  // in lane l, register (c, e); the wave parks the row's kept values in LDS in
  // slot order and the chain reads four consecutive slots with one LDS load
  // that every lane makes at the same address, each load issued kCoefAhead
  // steps before its adds (so each slot costs one dependent add with a
  // register operand). The wave reads only what it wrote itself, and a wave's
  // LDS accesses complete in order.
  __shared__ float4 park[4][PIECES * kCoefPiece / 4];
  float4* const kw = park[threadIdx.x >> 6];
#pragma unroll
  for (int c = 0; c < PIECES; ++c) {
    kw[c * (kCoefPiece / 4) + 2 * lane] = make_float4(kept[c][0], kept[c][1], kept[c][2], kept[c][3]);
    kw[c * (kCoefPiece / 4) + 2 * lane + 1] = make_float4(kept[c][4], kept[c][5], kept[c][6], kept[c][7]);
  }
  constexpr int kN4 = PIECES * kCoefPiece / 4;
  float S = -0.0f;
  float4 w[kCoefAhead];
#pragma unroll
  for (int q = 0; q < kCoefAhead; ++q) w[q] = kw[q];
#pragma unroll
  for (int q = 0; q < kN4; ++q) {
    const float4 x = w[q % kCoefAhead];
    if (q + kCoefAhead < kN4) w[q % kCoefAhead] = kw[q + kCoefAhead];
    S = S + x.x;
    S = S + x.y;
    S = S + x.z;
    S = S + x.w;
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int c = 0; c < PIECES; ++c) {
    const int j0 = c * kCoefPiece + 8 * lane;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool valid = id[c][e] >= 0 && id[c][e] < n_rows;
      const float g = pr[c][e] * S - kept[c][e];
      o[e] = valid ? g * scale : 0.0f;
    }
    if (VEC && j0 + 8 <= K) {
      *reinterpret_cast<float4*>(coef + base + j0) = make_float4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<float4*>(coef + base + j0 + 4) = make_float4(o[4], o[5], o[6], o[7]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (j0 + e < K) coef[base + j0 + e] = o[e];
    }
  }
}

// Comparison arm of the fused indexer dK: every element of every valid slot's
// source row RN32(c * q) added into dk with a hardware float atomic, no sort.
template <int GS>
__global__ __launch_bounds__(256) void ia_atomic_fused(const int32_t* __restrict__ ids, int64_t n_src,
                                                       const uint16_t* __restrict__ q, int64_t q_ld, int dim,
                                                       int n_rows, float* __restrict__ out, int64_t out_ld,
                                                       FusedSrc fz) {
  const int g = threadIdx.x / GS;
  const int lg = threadIdx.x % GS;
  const int64_t p = static_cast<int64_t>(blockIdx.x) * (256 / GS) + g;
  if (p >= n_src || 8 * lg >= dim) return;
  const int32_t id = ids[p];
  if (id < 0 || id >= n_rows) return;
  const int d0 = 8 * lg;
  const uint32_t row = floor_div_rcp(static_cast<uint32_t>(p), fz.K, fz.krcp);
  const float c = fz.coef[p];
  Row8<uint16_t> v;
  v.load(q + static_cast<int64_t>(row) * q_ld + d0);
  float* o = out + static_cast<int64_t>(id) * out_ld + d0;
#pragma unroll
  for (int i = 0; i < 8; ++i) unsafeAtomicAdd(o + i, c * v.get(i));
}

int group_size(int64_t dim) {
  const int64_t d8 = dim / 8;
  int gs = 1;
  while (gs < d8) gs *= 2;
  return gs;
}

int resolve(const det_index_add_cfg* cfg, int* L) {
  const int v = cfg ? cfg->chunk_rows : 256;
  if (v < 1 || v > 65536) return set_error(DET_ERR_INVALID_ARG, "index_add: chunk_rows must be in [1, 65536], got %d", v);
  *L = v;
  return DET_OK;
}

int check_shape(int64_t n_src, int64_t dim, int64_t n_rows) {
  if (n_src < 0 || dim < 0 || n_rows < 0) return set_error(DET_ERR_INVALID_ARG, "index_add: sizes must be >= 0");
  if (dim % 8 != 0 || dim > kMaxDim)
    return set_error(DET_ERR_UNSUPPORTED, "index_add: dim must be a multiple of 8 and <= %d, got %lld", kMaxDim,
                     static_cast<long long>(dim));
  if (n_rows > kMaxRows)
    return set_error(DET_ERR_UNSUPPORTED, "index_add: n_rows must be <= %d, got %lld", kMaxRows,
                     static_cast<long long>(n_rows));
  if (n_src > 0x7FFFFFFFLL) return set_error(DET_ERR_UNSUPPORTED, "index_add: n_src must be < 2^31");
  return DET_OK;
}

// Stages 1-6 on `stream` (the caller has validated every argument). With fz,
// source row p is RN32(fz->coef[p] * src[p / fz->K]) (bf16 query rows, the
// one-wave-per-chunk gather only: dim in {128, 256, 512}, L <= 1024).
int pipeline(const Layout& l, void* ws, float* out, int64_t n_rows, int64_t dim, int64_t out_ld,
             const int32_t* ids, int64_t n_src, const void* src, int64_t src_ld, bool f32, int L, hipStream_t st,
             const FusedSrc* fz, const char* what) {
  const auto* s16 = static_cast<const uint16_t*>(src);
  const auto* s32 = static_cast<const float*>(src);
  const int gs = group_size(dim);
  const int nr = static_cast<int>(n_rows);
  char* w = static_cast<char*>(ws);
  auto* hdr = reinterpret_cast<uint32_t*>(w);
  auto* hist = reinterpret_cast<uint16_t*>(w + l.hist);
  const int hist_ld = hist_stride(n_rows);
  auto* wg_tot = reinterpret_cast<uint32_t*>(w + l.wg_tot);
  auto* seg_off = reinterpret_cast<uint32_t*>(w + l.seg_off);
  auto* chunk_off = reinterpret_cast<uint32_t*>(w + l.chunk_off);
  auto* full_off = reinterpret_cast<uint32_t*>(w + l.full_off);
  auto* chunk_desc = reinterpret_cast<int4*>(w + l.chunk_desc);
  auto* perm = reinterpret_cast<int32_t*>(w + l.perm);
  auto* scratch = reinterpret_cast<float*>(w + l.scratch);
  const size_t lds_count = static_cast<size_t>(hist_ld) * 4;
  auto* segtot = reinterpret_cast<uint32_t*>(w + l.segtot);
  hipLaunchKernelGGL(ia_count, dim3(l.nblk), dim3(kSortThreads), lds_count, st, ids, n_src, nr, hist_ld, hist, hdr);
  hipLaunchKernelGGL(ia_prefix_seg, dim3(ceil_div(n_rows, 256), l.nseg), dim3(256), 0, st, hist, hist_ld, l.nblk, nr,
                     segtot);
  const uint32_t rcp = static_cast<uint32_t>(0xFFFFFFFFull / static_cast<uint64_t>(L));
  const dim3 off_grid(static_cast<uint32_t>(ceil_div(n_rows, 256)));
  hipLaunchKernelGGL(ia_totals, off_grid, dim3(256), 0, st, segtot, l.nseg, nr, L, rcp, wg_tot, seg_off);
  hipLaunchKernelGGL(ia_offsets, off_grid, dim3(256), 0, st, nr, L, rcp, n_src, wg_tot, seg_off, chunk_off, full_off,
                     chunk_desc, hdr);
  // the fused indexer dK's coefficients follow the positions into the sorted order
  const float* coef_in = fz ? fz->coef : nullptr;
  int2* pairs = fz ? reinterpret_cast<int2*>(w + l.pairs) : nullptr;
  switch (scatter_waves(n_rows)) {
    case 4: launch_scatter<4>(l.nblk, nr, st, ids, n_src, hist, segtot, seg_off, perm, coef_in, pairs); break;
    case 2: launch_scatter<2>(l.nblk, nr, st, ids, n_src, hist, segtot, seg_off, perm, coef_in, pairs); break;
    default: launch_scatter<1>(l.nblk, nr, st, ids, n_src, hist, segtot, seg_off, perm, coef_in, pairs); break;
  }
  const int64_t grid_g = ceil_div(l.max_chunks, 256 / gs);
#define DET_IA_TAIL_T(G, E, S)                                                                                  \
  if (gs == G) {                                                                                                 \
    if (L <= G * kPosPerLane)                                                                                    \
      hipLaunchKernelGGL((ia_gather<G, E>), dim3(grid_g), dim3(256), 0, st, S, src_ld, (int)dim, perm, seg_off,  \
                         chunk_off, nr, L, out, out_ld, scratch, n_src, l.max_chunks);                           \
    else                                                                                                         \
      hipLaunchKernelGGL((ia_gather_long<G, E>), dim3(grid_g), dim3(256), 0, st, S, src_ld, (int)dim, perm,      \
                         seg_off, chunk_off, nr, L, out, out_ld, scratch, n_src, l.max_chunks);                  \
  }
#define DET_IA_TAIL(G)                   \
  if (f32) {                             \
    DET_IA_TAIL_T(G, float, s32)         \
  } else {                               \
    DET_IA_TAIL_T(G, uint16_t, s16)      \
  }
  const int dpl = (dim % 64 == 0) ? static_cast<int>(dim / 64) : 0;
  // the one-wave-per-chunk gather is for bf16 rows; float32 rows take the lane-group gather
  if (fz || (!f32 && (dpl == 2 || dpl == 4 || dpl == 8) && L <= 64 * kPosPerLane)) {
    const int64_t grid_w = ceil_div(l.max_chunks, 4);
    // position registers per lane sized to the chunk length (fewer registers, more waves per SIMD)
    // stored source rows below 2^31 bytes: the buffer-resource gather
    const bool bufok = !fz && n_src * src_ld * 2 < (static_cast<int64_t>(1) << 31);
    const uint32_t src_bytes = bufok ? static_cast<uint32_t>(n_src * src_ld * 2) : 0u;
    // fused at dim 128 with chunks of at most 256 rows and query rows below 2^31 bytes: four chunks per wave
    const int64_t q_bytes = fz ? n_src / fz->K * src_ld * 2 : 0;
    const bool quad = fz && dim == 128 && L <= 256 && q_bytes < (static_cast<int64_t>(1) << 31);
    if (quad)
      hipLaunchKernelGGL(ia_gather_quad, dim3(ceil_div(l.max_chunks, 16)), dim3(256), 0, st, s16, src_ld,
                         static_cast<uint32_t>(q_bytes), chunk_off, chunk_desc, nr, out, out_ld, scratch, n_src,
                         l.max_chunks, *fz);
#define DET_IA_WAVE(D, NP)                                                                                      \
  if (!fz && dpl == D && L <= 64 * NP && (NP == 4 || L > 64 * (NP / 2))) {                                      \
    if (bufok)                                                                                                  \
      hipLaunchKernelGGL((ia_gather_buf<D, NP>), dim3(grid_w), dim3(256), 0, st, s16, src_ld, (int)dim,         \
                         src_bytes, perm, chunk_off, chunk_desc, nr, out, out_ld, scratch, n_src, l.max_chunks);  \
    else                                                                                                        \
      hipLaunchKernelGGL((ia_gather_wave<D, NP>), dim3(grid_w), dim3(256), 0, st, s16, src_ld, (int)dim, perm,   \
                         chunk_off, chunk_desc, nr, out, out_ld, scratch, n_src, l.max_chunks, FusedSrc{});   \
  }                                                                                                             \
  if (!quad && fz && dpl == D && L <= 64 * NP && (NP == 4 || L > 64 * (NP / 2)))                                \
    hipLaunchKernelGGL((ia_gather_wave<D, NP, true>), dim3(grid_w), dim3(256), 0, st, s16, src_ld, (int)dim,      \
                       perm, chunk_off, chunk_desc, nr, out, out_ld, scratch, n_src, l.max_chunks, *fz);
    DET_IA_WAVE(2, 4) DET_IA_WAVE(2, 8) DET_IA_WAVE(2, 16)
    DET_IA_WAVE(4, 4) DET_IA_WAVE(4, 8) DET_IA_WAVE(4, 16)
    DET_IA_WAVE(8, 4) DET_IA_WAVE(8, 8) DET_IA_WAVE(8, 16)
#undef DET_IA_WAVE
  } else {
    DET_IA_TAIL(1) DET_IA_TAIL(2) DET_IA_TAIL(4) DET_IA_TAIL(8) DET_IA_TAIL(16) DET_IA_TAIL(32) DET_IA_TAIL(64)
  }
#undef DET_IA_TAIL
#undef DET_IA_TAIL_T
  const int ds = fold_slice(dim);
  const dim3 fold_grid(static_cast<uint32_t>((n_rows < kFoldGroups ? n_rows : kFoldGroups) * (dim / ds)));
  if (ds == 32)
    hipLaunchKernelGGL(ia_fold<32>, fold_grid, dim3(256), 0, st, chunk_off, nr, (int)dim, scratch, out, out_ld);
  else if (ds == 16)
    hipLaunchKernelGGL(ia_fold<16>, fold_grid, dim3(256), 0, st, chunk_off, nr, (int)dim, scratch, out, out_ld);
  else
    hipLaunchKernelGGL(ia_fold<8>, fold_grid, dim3(256), 0, st, chunk_off, nr, (int)dim, scratch, out, out_ld);
  return check_launch(what);
}

}  // namespace
}  // namespace detgrad

using namespace detgrad;

extern "C" int det_index_add_workspace_size(int64_t n_src, int64_t dim, int64_t n_rows, const det_index_add_cfg* cfg,
                                            int atomic, size_t* bytes) {
  if (int s = check_atomic_flag(atomic)) return s;
  if (!bytes) return set_error(DET_ERR_INVALID_ARG, "index_add: bytes is NULL");
  if (int s = check_shape(n_src, dim, n_rows)) return s;
  int L;
  if (int s = resolve(cfg, &L)) return s;
  *bytes = (atomic || n_src == 0 || n_rows == 0 || dim == 0) ? 0 : layout(n_src, dim, n_rows, L).total;
  return ok();
}

extern "C" int det_index_add(float* out, int64_t n_rows, int64_t dim, int64_t out_ld, const int32_t* ids, int64_t n_src,
                             const void* src, int64_t src_ld, int src_dtype, const det_index_add_cfg* cfg, void* ws,
                             size_t ws_bytes, int atomic, void* stream) {
  if (int s = check_atomic_flag(atomic)) return s;
  if (int s = check_shape(n_src, dim, n_rows)) return s;
  int L;
  if (int s = resolve(cfg, &L)) return s;
  if (src_dtype != DET_BF16 && src_dtype != DET_F32)
    return set_error(DET_ERR_INVALID_ARG, "index_add: unknown dtype %d", src_dtype);
  if (n_src == 0 || n_rows == 0 || dim == 0) return ok();
  if (!out || !ids || !src) return set_error(DET_ERR_INVALID_ARG, "index_add: NULL pointer");
  if (out_ld < dim || src_ld < dim) return set_error(DET_ERR_INVALID_ARG, "index_add: out_ld and src_ld must be >= dim");
  if (out_ld % 4 || src_ld % 8 || !aligned(out, 16) || !aligned(src, 16))
    return set_error(DET_ERR_UNSUPPORTED, "index_add: out/src rows must be 16-byte aligned");
  const Layout l = layout(n_src, dim, n_rows, L);
  const size_t need = atomic ? 0 : l.total;
  if (int s = check_workspace(ws, ws_bytes, need)) return s;
  const Range o = range2d(out, n_rows, dim, out_ld, 4);
  if (overlaps(o, range1d(ids, n_src * 4)) || overlaps(o, range2d(src, n_src, dim, src_ld, src_dtype == DET_F32 ? 4 : 2)) ||
      overlaps(o, range1d(ws, ws_bytes)))
    return set_error(DET_ERR_OVERLAP, "index_add: out overlaps an input or the workspace");
  const hipStream_t st = as_stream(stream);
  const auto* s16 = static_cast<const uint16_t*>(src);
  const auto* s32 = static_cast<const float*>(src);
  const bool f32 = src_dtype == DET_F32;
  const int gs = group_size(dim);
  const int nr = static_cast<int>(n_rows);
  if (atomic) {
    const int64_t grid = ceil_div(n_src, 256 / gs);
#define DET_IA_ATOMIC(G) \
  if (gs == G && f32)                                                                                           \
    hipLaunchKernelGGL((ia_atomic<G, float>), dim3(grid), dim3(256), 0, st, ids, n_src, s32, src_ld, (int)dim, nr, out, \
                       out_ld);                                                                                  \
  if (gs == G && !f32)                                                                                          \
    hipLaunchKernelGGL((ia_atomic<G, uint16_t>), dim3(grid), dim3(256), 0, st, ids, n_src, s16, src_ld, (int)dim, nr, \
                       out, out_ld);
    DET_IA_ATOMIC(1) DET_IA_ATOMIC(2) DET_IA_ATOMIC(4) DET_IA_ATOMIC(8) DET_IA_ATOMIC(16) DET_IA_ATOMIC(32)
    DET_IA_ATOMIC(64)
#undef DET_IA_ATOMIC
    return check_launch("det_index_add (atomic)");
  }
  return pipeline(l, ws, out, n_rows, dim, out_ld, ids, n_src, src, src_ld, f32, L, st, nullptr, "det_index_add");
}

extern "C" int det_index_add_bad_ids(const void* ws, size_t ws_bytes, int64_t* count, void* stream) {
  if (!count) return set_error(DET_ERR_INVALID_ARG, "index_add_bad_ids: count is NULL");
  if (int s = check_workspace(ws, ws_bytes, DET_WS_HEADER_BYTES)) return s;
  uint32_t v = 0u;  // header word 1: bad ids of the last call
  const hipStream_t st = as_stream(stream);
  hipError_t e = hipMemcpyAsync(&v, static_cast<const char*>(ws) + 4, 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return set_error(DET_ERR_HIP, "index_add_bad_ids: %s", hipGetErrorString(e));
  *count = v;
  return ok();
}

// ---------------------------------------------------------------------------
// det_indexer_dk: the fused sparse-indexer dK (DSv4 page, source 3 fix). The
// coefficient kernel turns (ids, predict, target) into one float32 per slot;
// the index_add pipeline then gathers RN32(c * q[row]) instead of stored
// source rows. The comparison arm adds the same products with float atomics.
namespace {
int indexer_dk_check(int64_t Q, int64_t K, int64_t dim, int64_t n_rows, const det_index_add_cfg* cfg, int* L) {
  if (Q < 0 || K < 0) return set_error(DET_ERR_INVALID_ARG, "indexer_dk: Q and K must be >= 0");
  if (K > kCoefMaxPieces * kCoefPiece)
    return set_error(DET_ERR_UNSUPPORTED, "indexer_dk: K must be <= %d, got %lld", kCoefMaxPieces * kCoefPiece,
                     static_cast<long long>(K));
  if (Q * K > 0x7FFFFFFFLL) return set_error(DET_ERR_UNSUPPORTED, "indexer_dk: Q * K must be < 2^31");
  if (int s = check_shape(Q * K, dim, n_rows)) return s;
  if (int s = resolve(cfg, L)) return s;
  if (dim != 0 && dim != 128 && dim != 256 && dim != 512)
    return set_error(DET_ERR_UNSUPPORTED, "indexer_dk: dim must be 128, 256 or 512, got %lld", static_cast<long long>(dim));
  if (*L > 1024) return set_error(DET_ERR_UNSUPPORTED, "indexer_dk: chunk_rows must be <= 1024, got %d", *L);
  return DET_OK;
}

size_t indexer_dk_ws(int64_t Q, int64_t K, int64_t dim, int64_t n_rows, int L, int atomic) {
  const int64_t n_src = Q * K;
  if (n_src == 0 || n_rows == 0 || dim == 0) return 0;
  if (atomic) return DET_WS_HEADER_BYTES + align_up(static_cast<size_t>(n_src) * 4, 256);
  return layout(n_src, dim, n_rows, L, true).total;
}
}  // namespace

extern "C" int det_indexer_dk_workspace_size(int64_t Q, int64_t K, int64_t dim, int64_t n_rows,
                                            const det_index_add_cfg* cfg, int atomic, size_t* bytes) {
  if (int s = check_atomic_flag(atomic)) return s;
  if (!bytes) return set_error(DET_ERR_INVALID_ARG, "indexer_dk: bytes is NULL");
  int L;
  if (int s = indexer_dk_check(Q, K, dim, n_rows, cfg, &L)) return s;
  *bytes = indexer_dk_ws(Q, K, dim, n_rows, L, atomic);
  return ok();
}

extern "C" int det_indexer_dk(float* dk, int64_t n_rows, int64_t dim, int64_t dk_ld, const int32_t* ids,
                              const float* predict, const float* target, int64_t Q, int64_t K, const void* q,
                              int64_t q_ld, int q_dtype, float scale, const det_index_add_cfg* cfg, void* ws,
                              size_t ws_bytes, int atomic, void* stream) {
  if (int s = check_atomic_flag(atomic)) return s;
  int L;
  if (int s = indexer_dk_check(Q, K, dim, n_rows, cfg, &L)) return s;
  if (q_dtype != DET_BF16)
    return set_error(q_dtype == DET_F32 ? DET_ERR_UNSUPPORTED : DET_ERR_INVALID_ARG,
                     "indexer_dk: q must be bf16 (dtype %d)", q_dtype);
  const int64_t n_src = Q * K;
  if (n_src == 0 || n_rows == 0 || dim == 0) return ok();
  if (!dk || !ids || !predict || !target || !q) return set_error(DET_ERR_INVALID_ARG, "indexer_dk: NULL pointer");
  if (dk_ld < dim || q_ld < dim) return set_error(DET_ERR_INVALID_ARG, "indexer_dk: dk_ld and q_ld must be >= dim");
  if (dk_ld % 4 || q_ld % 8 || !aligned(dk, 16) || !aligned(q, 16))
    return set_error(DET_ERR_UNSUPPORTED, "indexer_dk: dk and q rows must be 16-byte aligned");
  const size_t need = indexer_dk_ws(Q, K, dim, n_rows, L, atomic);
  if (int s = check_workspace(ws, ws_bytes, need)) return s;
  const Range o = range2d(dk, n_rows, dim, dk_ld, 4);
  const size_t slot_bytes = static_cast<size_t>(n_src) * 4;
  if (overlaps(o, range1d(ids, slot_bytes)) || overlaps(o, range1d(predict, slot_bytes)) ||
      overlaps(o, range1d(target, slot_bytes)) || overlaps(o, range2d(q, Q, dim, q_ld, 2)) ||
      overlaps(o, range1d(ws, ws_bytes)))
    return set_error(DET_ERR_OVERLAP, "indexer_dk: dk overlaps an input or the workspace");
  const hipStream_t st = as_stream(stream);
  char* w = static_cast<char*>(ws);
  const Layout l = layout(n_src, dim, n_rows, L, true);
  float* coef = reinterpret_cast<float*>(w + (atomic ? DET_WS_HEADER_BYTES : l.coef));
  // one wave per query row; 16-byte loads when every row starts 32-byte aligned
  const dim3 coef_grid(static_cast<uint32_t>(ceil_div(Q, 4)));
  const bool vec = K % 8 == 0 && aligned(ids, 32) && aligned(predict, 32) && aligned(target, 32) && aligned(ws, 32);
  const int Ki = static_cast<int>(K), nr = static_cast<int>(n_rows);
#define DET_IA_COEF(P, V)                                                                                         \
  hipLaunchKernelGGL((ia_coef<P, V>), coef_grid, dim3(256), 0, st, ids, predict, target, Q, Ki, nr, scale, coef);
  if (K <= kCoefPiece) {
    if (vec) { DET_IA_COEF(1, true) } else { DET_IA_COEF(1, false) }
  } else {
    if (vec) { DET_IA_COEF(2, true) } else { DET_IA_COEF(2, false) }
  }
#undef DET_IA_COEF
  FusedSrc fz;
  fz.coef = coef;
  fz.pairs = atomic ? nullptr : reinterpret_cast<const int2*>(w + l.pairs);
  fz.K = static_cast<uint32_t>(K);
  fz.krcp = static_cast<uint32_t>(0xFFFFFFFFull / static_cast<uint64_t>(K));
  const auto* q16 = static_cast<const uint16_t*>(q);
  if (atomic) {
    const int gs = group_size(dim);
    const int64_t grid = ceil_div(n_src, 256 / gs);
    const int nr = static_cast<int>(n_rows);
    if (gs == 16)
      hipLaunchKernelGGL(ia_atomic_fused<16>, dim3(grid), dim3(256), 0, st, ids, n_src, q16, q_ld, (int)dim, nr, dk,
                         dk_ld, fz);
    else if (gs == 32)
      hipLaunchKernelGGL(ia_atomic_fused<32>, dim3(grid), dim3(256), 0, st, ids, n_src, q16, q_ld, (int)dim, nr, dk,
                         dk_ld, fz);
    else
      hipLaunchKernelGGL(ia_atomic_fused<64>, dim3(grid), dim3(256), 0, st, ids, n_src, q16, q_ld, (int)dim, nr, dk,
                         dk_ld, fz);
    return check_launch("det_indexer_dk (atomic)");
  }
  return pipeline(l, ws, dk, n_rows, dim, dk_ld, ids, n_src, q, q_ld, false, L, st, &fz, "det_indexer_dk");
}
