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
//  3. scan     one workgroup: exclusive scans of the counts (segment offsets of
//              the sorted order) and of ceil(count / L) (chunk offsets).
//  4. scatter  one wave per block walks its positions in order, 64 at a time;
//              the lanes holding the same id find each other with one ballot
//              per id bit, so each lane's rank among equal ids is its position
//              order inside the batch plus the id's running LDS count: a stable
//              counting sort. perm[seg_off[id] + prefix + rank] = p.
//  5. gather   one lane group per chunk of L sorted rows of one id: each lane
//              owns 8 consecutive dims (one 16-byte bf16 load per row) and
//              folds the chunk's rows left to right. A single-chunk id is added
//              into out directly; otherwise the partial goes to scratch.
//  6. fold     ids with several chunks fold their chunk partials left to right
//              and add the total into out once.
// Traffic: the src rows of valid ids (256 B per row at dim 128) dominate;
// ids, perm, the histograms and out are small next to them.
//
// The atomic arm adds each src row into out[id] with per-element hardware float
// atomics and no sort, as a non-deterministic index_add does.
#include "common.hpp"

namespace detgrad {
namespace {

constexpr int kBlockPos = 4096;  // source positions per count/scatter block
constexpr int kMaxRows = 16384;  // LDS histogram capacity (64 KiB)
constexpr int kMaxDim = 512;

constexpr int kSegBlocks = 32;   // blocks per prefix segment

struct Layout {
  size_t hist, segtot, count, seg_off, chunk_off, perm, scratch, total;
  int64_t nblk, nseg, max_chunks;
};

Layout layout(int64_t n_src, int64_t dim, int64_t n_rows, int64_t L) {
  Layout l;
  l.nblk = ceil_div(n_src, kBlockPos);
  l.nseg = ceil_div(l.nblk, kSegBlocks);
  l.max_chunks = n_src / L + (n_rows < n_src ? n_rows : n_src) + 1;
  size_t o = DET_WS_HEADER_BYTES;
  l.hist = o;      o = align_up(o + static_cast<size_t>(l.nblk * n_rows) * 4, 256);
  l.segtot = o;    o = align_up(o + static_cast<size_t>(l.nseg * n_rows) * 4, 256);
  l.count = o;     o = align_up(o + static_cast<size_t>(n_rows) * 4, 256);
  l.seg_off = o;   o = align_up(o + static_cast<size_t>(n_rows + 1) * 4, 256);
  l.chunk_off = o; o = align_up(o + static_cast<size_t>(n_rows + 1) * 4, 256);
  l.perm = o;      o = align_up(o + static_cast<size_t>(n_src) * 4, 256);
  l.scratch = o;   o = align_up(o + static_cast<size_t>(l.max_chunks * dim) * 4, 256);
  l.total = o;
  return l;
}

// Lanes of one wave holding the same id find each other with one ballot per
// id bit; returns the mask of those lanes (0 for invalid lanes).
__device__ __forceinline__ uint64_t match_peers(int32_t id, bool valid, int id_bits) {
  uint64_t peers = __ballot(valid);
  for (int bit = 0; bit < id_bits; ++bit) {
    const bool set = valid && ((id >> bit) & 1);
    const uint64_t m = __ballot(set);
    peers &= set ? m : ~m;
  }
  return valid ? peers : 0ull;
}

// ---- 1. count. One LDS increment per distinct id per wave (the hot Zipf
// key would otherwise serialise dozens of LDS atomics per instruction).
__global__ __launch_bounds__(256) void ia_count(const int32_t* __restrict__ ids, int64_t n_src, int n_rows,
                                                int id_bits, uint32_t* __restrict__ hist,
                                                uint32_t* __restrict__ bad_accum) {
  extern __shared__ uint32_t lds_hist[];
  for (int k = threadIdx.x; k < n_rows; k += 256) lds_hist[k] = 0u;
  __syncthreads();
  const int64_t b = blockIdx.x;
  const int64_t p0 = b * kBlockPos;
  const int64_t p1 = p0 + kBlockPos < n_src ? p0 + kBlockPos : n_src;
  const uint64_t lt = __lanemask_lt();
  uint32_t bad = 0;
  constexpr int kPer = kBlockPos / 256;
  int32_t idv[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int64_t p = p0 + threadIdx.x + u * 256;
    idv[u] = p < p1 ? ids[p] : -1;
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int32_t id = idv[u];
    const bool valid = id >= 0 && id < n_rows;
    if (!valid && id != -1) ++bad;
    const uint64_t peers = match_peers(id, valid, id_bits);
    if (valid && (peers & lt) == 0) atomicAdd(&lds_hist[id], static_cast<uint32_t>(__popcll(peers)));
  }
  __syncthreads();
  uint32_t* row = hist + b * n_rows;
  for (int k = threadIdx.x; k < n_rows; k += 256) row[k] = lds_hist[k];
  if (bad) atomicAdd(bad_accum, bad);
}

// ---- 2a. per id and segment of kSegBlocks blocks: exclusive prefix over the
// segment's blocks (in place) and the segment total.
__global__ __launch_bounds__(256) void ia_prefix_seg(uint32_t* __restrict__ hist, int64_t nblk, int n_rows,
                                                     uint32_t* __restrict__ segtot) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  const int64_t seg = blockIdx.y;
  if (k >= n_rows) return;
  const int64_t b0 = seg * kSegBlocks;
  uint32_t c[kSegBlocks];
#pragma unroll
  for (int j = 0; j < kSegBlocks; ++j) c[j] = (b0 + j < nblk) ? hist[(b0 + j) * n_rows + k] : 0u;
  uint32_t run = 0;
#pragma unroll
  for (int j = 0; j < kSegBlocks; ++j) {
    if (b0 + j < nblk) hist[(b0 + j) * n_rows + k] = run;
    run += c[j];
  }
  segtot[seg * n_rows + k] = run;
}

// ---- 2b. per id: exclusive prefix over segments (in place) and the total.
__global__ __launch_bounds__(256) void ia_prefix_tot(uint32_t* __restrict__ segtot, int64_t nseg, int n_rows,
                                                     uint32_t* __restrict__ count) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= n_rows) return;
  uint32_t run = 0;
  for (int64_t s0 = 0; s0 < nseg; s0 += 16) {
    uint32_t c[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) c[j] = (s0 + j < nseg) ? segtot[(s0 + j) * n_rows + k] : 0u;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (s0 + j < nseg) segtot[(s0 + j) * n_rows + k] = run;
      run += c[j];
    }
  }
  count[k] = run;
}

// ---- 3. scan over ids (single workgroup of 1024 threads)
__global__ __launch_bounds__(1024) void ia_scan(const uint32_t* __restrict__ count, int n_rows, int L,
                                                uint32_t* __restrict__ seg_off, uint32_t* __restrict__ chunk_off,
                                                uint32_t* __restrict__ hdr) {
  __shared__ uint32_t s_seg[1024];
  __shared__ uint32_t s_chk[1024];
  const int per = (n_rows + 1023) / 1024;
  const int k0 = threadIdx.x * per;
  uint32_t seg = 0, chk = 0;
  for (int i = 0; i < per; ++i) {
    const int k = k0 + i;
    if (k < n_rows) {
      const uint32_t c = count[k];
      seg += c;
      chk += (c + L - 1) / L;
    }
  }
  s_seg[threadIdx.x] = seg;
  s_chk[threadIdx.x] = chk;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 1024 per-thread totals (integers: exact)
  for (int off = 1; off < 1024; off *= 2) {
    const uint32_t a = threadIdx.x >= off ? s_seg[threadIdx.x - off] : 0u;
    const uint32_t c = threadIdx.x >= off ? s_chk[threadIdx.x - off] : 0u;
    __syncthreads();
    s_seg[threadIdx.x] += a;
    s_chk[threadIdx.x] += c;
    __syncthreads();
  }
  uint32_t run_seg = threadIdx.x ? s_seg[threadIdx.x - 1] : 0u;
  uint32_t run_chk = threadIdx.x ? s_chk[threadIdx.x - 1] : 0u;
  for (int i = 0; i < per; ++i) {
    const int k = k0 + i;
    if (k < n_rows) {
      seg_off[k] = run_seg;
      chunk_off[k] = run_chk;
      const uint32_t c = count[k];
      run_seg += c;
      run_chk += (c + L - 1) / L;
    }
  }
  if (threadIdx.x == 1023) {
    seg_off[n_rows] = s_seg[1023];
    chunk_off[n_rows] = s_chk[1023];
    hdr[1] = hdr[0];  // bad ids of this call
    hdr[0] = 0u;      // reset the accumulator for the next call
  }
}

// ---- 4. stable scatter. All 256 threads stage the block's ids and, for every
// id, its first destination (segment offset + prefix of earlier segments +
// prefix of earlier blocks of this segment) in LDS; then wave 0 alone walks
// the block in order, 64 positions at a time, so the walk touches global
// memory only to write perm. Within one wave the LDS read of an id's base
// precedes its leader's update in program order, so no barrier is needed.
__global__ __launch_bounds__(256) void ia_scatter(const int32_t* __restrict__ ids, int64_t n_src, int n_rows,
                                                  int id_bits, const uint32_t* __restrict__ prefix,
                                                  const uint32_t* __restrict__ segbase,
                                                  const uint32_t* __restrict__ seg_off, int32_t* __restrict__ perm) {
  extern __shared__ uint32_t lds[];
  uint32_t* base = lds;                                     // [n_rows]
  int32_t* lid = reinterpret_cast<int32_t*>(lds + n_rows);  // [kBlockPos]
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  const uint32_t* pre = prefix + b * n_rows;
  const uint32_t* sb = segbase + (b / kSegBlocks) * n_rows;
  for (int k0 = 0; k0 < n_rows; k0 += 256 * 8) {
    uint32_t v0[8], v1[8], v2[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = k0 + tid + 256 * u;
      v0[u] = k < n_rows ? seg_off[k] : 0u;
      v1[u] = k < n_rows ? sb[k] : 0u;
      v2[u] = k < n_rows ? pre[k] : 0u;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = k0 + tid + 256 * u;
      if (k < n_rows) base[k] = v0[u] + v1[u] + v2[u];
    }
  }
  const int64_t p0 = b * kBlockPos;
  const int64_t p1 = p0 + kBlockPos < n_src ? p0 + kBlockPos : n_src;
  {
    constexpr int kPer = kBlockPos / 256;
    int32_t v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int64_t p = p0 + tid + 256 * u;
      v[u] = p < p1 ? ids[p] : -1;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) lid[tid + 256 * u] = v[u];
  }
  __syncthreads();
  if (tid >= 64) return;
  const int lane = tid;
  const uint64_t lt = __lanemask_lt();
  for (int64_t off = 0; p0 + off < p1; off += 64) {
    const int32_t id = lid[off + lane];
    const bool valid = id >= 0 && id < n_rows;
    const uint64_t peers = match_peers(id, valid, id_bits);
    if (valid) {
      const uint32_t old = base[id];
      const uint64_t dest = static_cast<uint64_t>(old) + static_cast<uint32_t>(__popcll(peers & lt));
      if (dest < static_cast<uint64_t>(n_src)) perm[dest] = static_cast<int32_t>(p0 + off + lane);
      __builtin_amdgcn_wave_barrier();
      if ((peers & lt) == 0) base[id] = old + static_cast<uint32_t>(__popcll(peers));
    }
    __builtin_amdgcn_wave_barrier();
  }
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

// ---- 5. chunk gather-sum. GS lanes per chunk, 8 dims per lane. The chunk's
// source positions (at most 16 per lane, GS * 16 rows) are loaded once,
// handed out by lane shuffles; the rows are then read up to 16 at a time (all
// their loads in flight) and folded in order.
constexpr int kPosPerLane = 16;  // chunk capacity of ia_gather: GS * 16 rows (longer chunks: ia_gather_long)

template <int GS>
__global__ __launch_bounds__(256) void ia_gather(const uint16_t* __restrict__ src, int64_t src_ld, int dim,
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
      uint4 v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int64_t p = __shfl(pos[i], h + u, GS);
        const bool ok = active && GS * i + h + u < static_cast<int>(len) && p >= 0 && p < n_src;
        v[u] = ok ? *reinterpret_cast<const uint4*>(src + p * src_ld + d0) : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (active && GS * i + h + u < static_cast<int>(len)) add8_bf16(acc, v[u]);
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
__device__ __forceinline__ uint32_t zero_vec(uint32_t) { return 0u; }
__device__ __forceinline__ uint2 zero_vec(uint2) { return make_uint2(0u, 0u); }
__device__ __forceinline__ uint4 zero_vec(uint4) { return make_uint4(0u, 0u, 0u, 0u); }

template <int DPL>
__global__ __launch_bounds__(256) void ia_gather_wave(const uint16_t* __restrict__ src, int64_t src_ld, int dim,
                                                      const int32_t* __restrict__ perm,
                                                      const uint32_t* __restrict__ seg_off,
                                                      const uint32_t* __restrict__ chunk_off, int n_rows, int L,
                                                      float* __restrict__ out, int64_t out_ld,
                                                      float* __restrict__ scratch, int64_t n_src,
                                                      int64_t max_chunks) {
  typedef typename RowVec<DPL>::T V;
  const int lane = threadIdx.x & 63;
  const uint32_t c = static_cast<uint32_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const uint32_t n_chunks = chunk_off[n_rows];
  if (c >= n_chunks || c >= max_chunks) return;  // wave-uniform
  const int k = chunk_owner(chunk_off, n_rows, c);
  const uint32_t j = c - chunk_off[k];
  const uint32_t r0 = seg_off[k] + j * static_cast<uint32_t>(L);
  uint32_t r_end = seg_off[k + 1];
  if (r_end > static_cast<uint64_t>(n_src)) r_end = static_cast<uint32_t>(n_src);
  const int len = static_cast<int>(r0 + static_cast<uint32_t>(L) < r_end ? static_cast<uint32_t>(L)
                                                                          : (r_end > r0 ? r_end - r0 : 0u));
  const int d0 = DPL * lane;
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = -0.0f;
  int32_t pos[kPosPerLane];
#pragma unroll
  for (int i = 0; i < kPosPerLane; ++i) {
    const bool ok = 64 * i + lane < len;
    const int32_t x = perm[ok ? r0 + 64 * i + lane : r0];
    pos[i] = ok ? x : 0;
  }
  // rows whose loads are in flight together: 64 / 32 / 16 for 4 / 8 / 16-byte rows
  constexpr int kB = 128 / DPL;
#pragma unroll
  for (int i = 0; i < kPosPerLane; ++i) {
#pragma unroll
    for (int h = 0; h < 64; h += kB) {
      if (64 * i + h >= len) continue;  // wave-uniform skip
      V v[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        int64_t p = __shfl(pos[i], h + u, 64);
        p = (p >= 0 && p < n_src) ? p : 0;  // always a valid row; masked below
        v[u] = *reinterpret_cast<const V*>(src + p * src_ld + d0);
      }
#pragma unroll
      for (int u = 0; u < kB; ++u)
        if (64 * i + h + u < len) add_bf16(acc, v[u]);
    }
  }
  const uint32_t nk = chunk_off[k + 1] - chunk_off[k];
  float* dst = nk == 1 ? out + static_cast<int64_t>(k) * out_ld + d0 : scratch + static_cast<int64_t>(c) * dim + d0;
#pragma unroll
  for (int i = 0; i < DPL; ++i) dst[i] = (nk == 1 ? dst[i] + acc[i] : acc[i]);
}

// Chunks longer than GS * 16 rows (a large chunk_rows setting): one lane group
// walks the rows with the permutation read as it goes.
template <int GS>
__global__ __launch_bounds__(256) void ia_gather_long(const uint16_t* __restrict__ src, int64_t src_ld, int dim,
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
    uint4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (active && r + u < r1) {
        const int64_t p = perm[r + u];
        v[u] = (p >= 0 && p < n_src) ? *reinterpret_cast<const uint4*>(src + p * src_ld + d0) : make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (active && r + u < r1) add8_bf16(acc, v[u]);
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

// ---- 6. fold of multi-chunk ids: one workgroup per id. A round is a block
// of R = floor(1024 / (dim/4)) chunk partials (at most 16 KiB); every thread
// loads up to 4 float4 of a round, kAhead rounds are in flight in registers, each round is staged in
// LDS, and one thread per group of 4 dims folds it left to right.
constexpr int kAhead = 4;
constexpr int kRoundF4 = 1024;  // float4 per round

__global__ __launch_bounds__(256) void ia_fold(const uint32_t* __restrict__ chunk_off, int n_rows, int dim,
                                               const float* __restrict__ scratch, float* __restrict__ out,
                                               int64_t out_ld) {
  const int k = blockIdx.x;
  if (k >= n_rows) return;
  const uint32_t c0 = chunk_off[k], c1 = chunk_off[k + 1];
  if (c1 - c0 < 2) return;
  __shared__ float4 stage[kRoundF4];
  const int quads = dim / 4;
  const int R = kRoundF4 / quads;  // chunks per round
  const int tid = threadIdx.x;
  const uint32_t n = c1 - c0;
  const uint32_t rounds = (n + R - 1) / R;
  const float4* base = reinterpret_cast<const float4*>(scratch + static_cast<int64_t>(c0) * dim);
  float4 acc = make_float4(-0.0f, -0.0f, -0.0f, -0.0f);
  // four named register buffers (rounds r, r+1, r+2, r+3 in flight)
  float4 b0[4], b1[4], b2[4], b3[4];
  const uint32_t round_f4 = static_cast<uint32_t>(R * quads);  // <= kRoundF4
  const uint32_t total_f4 = n * static_cast<uint32_t>(quads);
  // unconditional loads from a clamped (always valid) index, then a select:
  // no branches, so the loads of several rounds stay in flight together
  auto load = [&](uint32_t rd, float4 (&v)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t j = tid + 256 * s;      // float4 index inside the round
      const uint32_t e = rd * round_f4 + j;  // float4 index from c0
      const bool ok = rd < rounds && j < round_f4 && e < total_f4;
      const float4 x = base[ok ? e : 0u];
      v[s] = ok ? x : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
  };
  auto consume = [&](uint32_t rd, float4 (&v)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) stage[tid + 256 * s] = v[s];
    __syncthreads();
    load(rd + kAhead, v);
    if (tid < quads) {
      const uint32_t m = n - rd * R < static_cast<uint32_t>(R) ? n - rd * R : static_cast<uint32_t>(R);
      uint32_t i = 0;
      for (; i + 8 <= m; i += 8) {  // 8 LDS reads in flight ahead of the dependent adds
        float4 q[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) q[u] = stage[(i + u) * quads + tid];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          acc.x = acc.x + q[u].x; acc.y = acc.y + q[u].y; acc.z = acc.z + q[u].z; acc.w = acc.w + q[u].w;
        }
      }
      for (; i < m; ++i) {
        const float4 q = stage[i * quads + tid];
        acc.x = acc.x + q.x; acc.y = acc.y + q.y; acc.z = acc.z + q.z; acc.w = acc.w + q.w;
      }
    }
    __syncthreads();
  };
  load(0, b0); load(1, b1); load(2, b2); load(3, b3);
  for (uint32_t rd = 0; rd < rounds; rd += kAhead) {
    consume(rd, b0);
    if (rd + 1 < rounds) consume(rd + 1, b1);
    if (rd + 2 < rounds) consume(rd + 2, b2);
    if (rd + 3 < rounds) consume(rd + 3, b3);
  }
  if (tid < quads) {
    float* d = out + static_cast<int64_t>(k) * out_ld + 4 * tid;
    float4 o = *reinterpret_cast<const float4*>(d);
    o.x = o.x + acc.x; o.y = o.y + acc.y; o.z = o.z + acc.z; o.w = o.w + acc.w;
    *reinterpret_cast<float4*>(d) = o;
  }
}

// ---- atomic arm: per-element float atomics, no sort
template <int GS>
__global__ __launch_bounds__(256) void ia_atomic(const int32_t* __restrict__ ids, int64_t n_src,
                                                 const uint16_t* __restrict__ src, int64_t src_ld, int dim, int n_rows,
                                                 float* __restrict__ out, int64_t out_ld) {
  const int g = threadIdx.x / GS;
  const int lg = threadIdx.x % GS;
  const int64_t p = static_cast<int64_t>(blockIdx.x) * (256 / GS) + g;
  if (p >= n_src || 8 * lg >= dim) return;
  const int32_t id = ids[p];
  if (id < 0 || id >= n_rows) return;
  const int d0 = 8 * lg;
  const uint4 v = *reinterpret_cast<const uint4*>(src + p * src_ld + d0);
  float* o = out + static_cast<int64_t>(id) * out_ld + d0;
  unsafeAtomicAdd(o + 0, bf16_lo(v.x)); unsafeAtomicAdd(o + 1, bf16_hi(v.x));
  unsafeAtomicAdd(o + 2, bf16_lo(v.y)); unsafeAtomicAdd(o + 3, bf16_hi(v.y));
  unsafeAtomicAdd(o + 4, bf16_lo(v.z)); unsafeAtomicAdd(o + 5, bf16_hi(v.z));
  unsafeAtomicAdd(o + 6, bf16_lo(v.w)); unsafeAtomicAdd(o + 7, bf16_hi(v.w));
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
  if (src_dtype != DET_BF16) return set_error(DET_ERR_UNSUPPORTED, "index_add: only bf16 src is implemented");
  if (n_src == 0 || n_rows == 0 || dim == 0) return ok();
  if (!out || !ids || !src) return set_error(DET_ERR_INVALID_ARG, "index_add: NULL pointer");
  if (out_ld < dim || src_ld < dim) return set_error(DET_ERR_INVALID_ARG, "index_add: out_ld and src_ld must be >= dim");
  if (out_ld % 4 || src_ld % 8 || !aligned(out, 16) || !aligned(src, 16))
    return set_error(DET_ERR_UNSUPPORTED, "index_add: out/src rows must be 16-byte aligned");
  const Layout l = layout(n_src, dim, n_rows, L);
  const size_t need = atomic ? 0 : l.total;
  if (int s = check_workspace(ws, ws_bytes, need)) return s;
  const Range o = range2d(out, n_rows, dim, out_ld, 4);
  if (overlaps(o, range1d(ids, n_src * 4)) || overlaps(o, range2d(src, n_src, dim, src_ld, 2)) ||
      overlaps(o, range1d(ws, ws_bytes)))
    return set_error(DET_ERR_OVERLAP, "index_add: out overlaps an input or the workspace");
  const hipStream_t st = as_stream(stream);
  const auto* s16 = static_cast<const uint16_t*>(src);
  const int gs = group_size(dim);
  const int nr = static_cast<int>(n_rows);
  if (atomic) {
    const int64_t grid = ceil_div(n_src, 256 / gs);
#define DET_IA_ATOMIC(G) \
  if (gs == G) hipLaunchKernelGGL(ia_atomic<G>, dim3(grid), dim3(256), 0, st, ids, n_src, s16, src_ld, (int)dim, nr, out, out_ld);
    DET_IA_ATOMIC(1) DET_IA_ATOMIC(2) DET_IA_ATOMIC(4) DET_IA_ATOMIC(8) DET_IA_ATOMIC(16) DET_IA_ATOMIC(32)
    DET_IA_ATOMIC(64)
#undef DET_IA_ATOMIC
    return check_launch("det_index_add (atomic)");
  }
  char* w = static_cast<char*>(ws);
  auto* hdr = reinterpret_cast<uint32_t*>(w);
  auto* hist = reinterpret_cast<uint32_t*>(w + l.hist);
  auto* count = reinterpret_cast<uint32_t*>(w + l.count);
  auto* seg_off = reinterpret_cast<uint32_t*>(w + l.seg_off);
  auto* chunk_off = reinterpret_cast<uint32_t*>(w + l.chunk_off);
  auto* perm = reinterpret_cast<int32_t*>(w + l.perm);
  auto* scratch = reinterpret_cast<float*>(w + l.scratch);
  int id_bits = 0;
  while ((1LL << id_bits) < n_rows) ++id_bits;
  const size_t lds_count = static_cast<size_t>(n_rows) * 4;
  const size_t lds_scatter = lds_count + kBlockPos * 4;
  if (lds_scatter > 64 * 1024) {
    static bool raised = false;  // allow up to the 160 KiB of a gfx950 workgroup once per process
    if (!raised) {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(ia_scatter),
                                hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      raised = true;
    }
  }
  auto* segtot = reinterpret_cast<uint32_t*>(w + l.segtot);
  hipLaunchKernelGGL(ia_count, dim3(l.nblk), dim3(256), lds_count, st, ids, n_src, nr, id_bits, hist, hdr);
  hipLaunchKernelGGL(ia_prefix_seg, dim3(ceil_div(n_rows, 256), l.nseg), dim3(256), 0, st, hist, l.nblk, nr, segtot);
  hipLaunchKernelGGL(ia_prefix_tot, dim3(ceil_div(n_rows, 256)), dim3(256), 0, st, segtot, l.nseg, nr, count);
  hipLaunchKernelGGL(ia_scan, dim3(1), dim3(1024), 0, st, count, nr, L, seg_off, chunk_off, hdr);
  hipLaunchKernelGGL(ia_scatter, dim3(l.nblk), dim3(256), lds_scatter, st, ids, n_src, nr, id_bits, hist, segtot,
                     seg_off, perm);
  const int64_t grid_g = ceil_div(l.max_chunks, 256 / gs);
#define DET_IA_TAIL(G)                                                                                           \
  if (gs == G) {                                                                                                 \
    if (L <= G * kPosPerLane)                                                                                    \
      hipLaunchKernelGGL(ia_gather<G>, dim3(grid_g), dim3(256), 0, st, s16, src_ld, (int)dim, perm, seg_off,   \
                         chunk_off, nr, L, out, out_ld, scratch, n_src, l.max_chunks);                           \
    else                                                                                                         \
      hipLaunchKernelGGL(ia_gather_long<G>, dim3(grid_g), dim3(256), 0, st, s16, src_ld, (int)dim, perm,       \
                         seg_off, chunk_off, nr, L, out, out_ld, scratch, n_src, l.max_chunks);                  \
  }
  const int dpl = (dim % 64 == 0) ? static_cast<int>(dim / 64) : 0;
  if ((dpl == 2 || dpl == 4 || dpl == 8) && L <= 64 * kPosPerLane) {
    const int64_t grid_w = ceil_div(l.max_chunks, 4);
#define DET_IA_WAVE(D)                                                                                          \
  if (dpl == D)                                                                                                 \
    hipLaunchKernelGGL(ia_gather_wave<D>, dim3(grid_w), dim3(256), 0, st, s16, src_ld, (int)dim, perm, seg_off, \
                       chunk_off, nr, L, out, out_ld, scratch, n_src, l.max_chunks);
    DET_IA_WAVE(2) DET_IA_WAVE(4) DET_IA_WAVE(8)
#undef DET_IA_WAVE
  } else {
    DET_IA_TAIL(1) DET_IA_TAIL(2) DET_IA_TAIL(4) DET_IA_TAIL(8) DET_IA_TAIL(16) DET_IA_TAIL(32) DET_IA_TAIL(64)
  }
#undef DET_IA_TAIL
  hipLaunchKernelGGL(ia_fold, dim3(static_cast<uint32_t>(n_rows)), dim3(256), 0, st, chunk_off, nr, (int)dim, scratch,
                     out, out_ld);
  return check_launch("det_index_add");
}

extern "C" int det_index_add_bad_ids(const void* ws, size_t ws_bytes, int64_t* count, void* stream) {
  if (!count) return set_error(DET_ERR_INVALID_ARG, "index_add_bad_ids: count is NULL");
  if (int s = check_workspace(ws, ws_bytes, DET_WS_HEADER_BYTES)) return s;
  uint32_t v = 0;
  const hipStream_t st = as_stream(stream);
  hipError_t e = hipMemcpyAsync(&v, static_cast<const char*>(ws) + 4, 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return set_error(DET_ERR_HIP, "index_add_bad_ids: %s", hipGetErrorString(e));
  *count = v;
  return ok();
}
