// det_index_add: out[ids[p]] += src[p] without float atomics (sparse-indexer dK,
// Megatron-LM PR #7441, source 3: "stable sort + prefix sum" in place of the
// atomic accumulation).
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

struct Layout {
  size_t hist, count, seg_off, chunk_off, perm, scratch, total;
  int64_t nblk, max_chunks;
};

Layout layout(int64_t n_src, int64_t dim, int64_t n_rows, int64_t L) {
  Layout l;
  l.nblk = ceil_div(n_src, kBlockPos);
  l.max_chunks = n_src / L + (n_rows < n_src ? n_rows : n_src) + 1;
  size_t o = DET_WS_HEADER_BYTES;
  l.hist = o;      o = align_up(o + static_cast<size_t>(l.nblk * n_rows) * 4, 256);
  l.count = o;     o = align_up(o + static_cast<size_t>(n_rows) * 4, 256);
  l.seg_off = o;   o = align_up(o + static_cast<size_t>(n_rows + 1) * 4, 256);
  l.chunk_off = o; o = align_up(o + static_cast<size_t>(n_rows + 1) * 4, 256);
  l.perm = o;      o = align_up(o + static_cast<size_t>(n_src) * 4, 256);
  l.scratch = o;   o = align_up(o + static_cast<size_t>(l.max_chunks * dim) * 4, 256);
  l.total = o;
  return l;
}

// ---- 1. count
__global__ __launch_bounds__(256) void ia_count(const int32_t* __restrict__ ids, int64_t n_src, int n_rows,
                                                uint32_t* __restrict__ hist, uint32_t* __restrict__ bad_accum) {
  extern __shared__ uint32_t lds_hist[];
  for (int k = threadIdx.x; k < n_rows; k += 256) lds_hist[k] = 0u;
  __syncthreads();
  const int64_t b = blockIdx.x;
  const int64_t p0 = b * kBlockPos;
  const int64_t p1 = p0 + kBlockPos < n_src ? p0 + kBlockPos : n_src;
  uint32_t bad = 0;
  for (int64_t p = p0 + threadIdx.x; p < p1; p += 256) {
    const int32_t id = ids[p];
    if (id >= 0 && id < n_rows)
      atomicAdd(&lds_hist[id], 1u);
    else if (id != -1)
      ++bad;
  }
  __syncthreads();
  uint32_t* row = hist + b * n_rows;
  for (int k = threadIdx.x; k < n_rows; k += 256) row[k] = lds_hist[k];
  if (bad) atomicAdd(bad_accum, bad);
}

// ---- 2. per-id prefix over blocks
__global__ __launch_bounds__(256) void ia_prefix(uint32_t* __restrict__ hist, int64_t nblk, int n_rows,
                                                 uint32_t* __restrict__ count) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= n_rows) return;
  constexpr int kU = 8;
  uint32_t run = 0;
  for (int64_t b0 = 0; b0 < nblk; b0 += kU) {
    uint32_t c[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j) c[j] = (b0 + j < nblk) ? hist[(b0 + j) * n_rows + k] : 0u;
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      if (b0 + j < nblk) {
        hist[(b0 + j) * n_rows + k] = run;
        run += c[j];
      }
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

// ---- 4. stable scatter (one wave per block)
__global__ __launch_bounds__(64) void ia_scatter(const int32_t* __restrict__ ids, int64_t n_src, int n_rows,
                                                 int id_bits, const uint32_t* __restrict__ prefix,
                                                 const uint32_t* __restrict__ seg_off, int32_t* __restrict__ perm) {
  extern __shared__ uint32_t lds_cnt[];
  const int lane = threadIdx.x;
  for (int k = lane; k < n_rows; k += 64) lds_cnt[k] = 0u;
  __syncthreads();
  const int64_t b = blockIdx.x;
  const uint32_t* pre = prefix + b * n_rows;
  const int64_t p0 = b * kBlockPos;
  const int64_t p1 = p0 + kBlockPos < n_src ? p0 + kBlockPos : n_src;
  const uint64_t lt = __lanemask_lt();
  for (int64_t base = p0; base < p1; base += 64) {
    const int64_t p = base + lane;
    const int32_t id = p < p1 ? ids[p] : -1;
    const bool valid = id >= 0 && id < n_rows;
    uint64_t peers = __ballot(valid);
    for (int bit = 0; bit < id_bits; ++bit) {
      const bool set = valid && ((id >> bit) & 1);
      const uint64_t m = __ballot(set);
      peers &= set ? m : ~m;
    }
    uint32_t old = 0;
    if (valid) {
      old = lds_cnt[id];
      const uint32_t rank = __popcll(peers & lt);
      const uint64_t dest = static_cast<uint64_t>(seg_off[id]) + pre[id] + old + rank;
      if (dest < static_cast<uint64_t>(n_src)) perm[dest] = static_cast<int32_t>(p);
    }
    __syncthreads();  // every lane has read its id's count before any leader updates it
    if (valid && (peers & lt) == 0) lds_cnt[id] = old + static_cast<uint32_t>(__popcll(peers));
    __syncthreads();
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

// ---- 5. chunk gather-sum. GS lanes per chunk, 8 dims per lane.
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
        // perm holds a permutation of valid source rows; the check only keeps a
        // corrupted workspace from turning into an out-of-bounds read
        v[u] = (p >= 0 && p < n_src) ? *reinterpret_cast<const uint4*>(src + p * src_ld + d0) : make_uint4(0, 0, 0, 0);
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
    float* s = scratch + static_cast<int64_t>(c) * dim + d0;
    *reinterpret_cast<float4*>(s) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *reinterpret_cast<float4*>(s + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

// ---- 6. fold of multi-chunk ids
template <int GS>
__global__ __launch_bounds__(256) void ia_fold(const uint32_t* __restrict__ chunk_off, int n_rows, int dim,
                                               const float* __restrict__ scratch, float* __restrict__ out,
                                               int64_t out_ld) {
  const int g = threadIdx.x / GS;
  const int lg = threadIdx.x % GS;
  const int k = blockIdx.x * (256 / GS) + g;
  if (k >= n_rows) return;
  const uint32_t c0 = chunk_off[k], c1 = chunk_off[k + 1];
  if (c1 - c0 < 2 || 8 * lg >= dim) return;
  const int d0 = 8 * lg;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = -0.0f;
  constexpr int kU = 8;
  for (uint32_t c = c0; c < c1; c += kU) {
    float4 a[kU], b[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (c + u < c1) {
        const float* s = scratch + static_cast<int64_t>(c + u) * dim + d0;
        a[u] = *reinterpret_cast<const float4*>(s);
        b[u] = *reinterpret_cast<const float4*>(s + 4);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (c + u < c1) {
        acc[0] = acc[0] + a[u].x; acc[1] = acc[1] + a[u].y; acc[2] = acc[2] + a[u].z; acc[3] = acc[3] + a[u].w;
        acc[4] = acc[4] + b[u].x; acc[5] = acc[5] + b[u].y; acc[6] = acc[6] + b[u].z; acc[7] = acc[7] + b[u].w;
      }
    }
  }
  store_add8(out + static_cast<int64_t>(k) * out_ld + d0, acc);
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
  const size_t lds = static_cast<size_t>(n_rows) * 4;
  hipLaunchKernelGGL(ia_count, dim3(l.nblk), dim3(256), lds, st, ids, n_src, nr, hist, hdr);
  hipLaunchKernelGGL(ia_prefix, dim3(ceil_div(n_rows, 256)), dim3(256), 0, st, hist, l.nblk, nr, count);
  hipLaunchKernelGGL(ia_scan, dim3(1), dim3(1024), 0, st, count, nr, L, seg_off, chunk_off, hdr);
  hipLaunchKernelGGL(ia_scatter, dim3(l.nblk), dim3(64), lds, st, ids, n_src, nr, id_bits, hist, seg_off, perm);
  const int64_t grid_g = ceil_div(l.max_chunks, 256 / gs);
  const int64_t grid_f = ceil_div(n_rows, 256 / gs);
#define DET_IA_TAIL(G)                                                                                         \
  if (gs == G) {                                                                                               \
    hipLaunchKernelGGL(ia_gather<G>, dim3(grid_g), dim3(256), 0, st, s16, src_ld, (int)dim, perm, seg_off,   \
                       chunk_off, nr, L, out, out_ld, scratch, n_src, l.max_chunks);                                                \
    hipLaunchKernelGGL(ia_fold<G>, dim3(grid_f), dim3(256), 0, st, chunk_off, nr, (int)dim, scratch, out,    \
                       out_ld);                                                                                \
  }
  DET_IA_TAIL(1) DET_IA_TAIL(2) DET_IA_TAIL(4) DET_IA_TAIL(8) DET_IA_TAIL(16) DET_IA_TAIL(32) DET_IA_TAIL(64)
#undef DET_IA_TAIL
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
