// det_topk_canonicalize: canonical order of a compact indexer top-k.
//
// Megatron-LM PR #7441 (DSv4 deterministic mode), source 1 and its fix: the
// slot order of a row's selected ids, and so the order of its softmax sum,
// changed between runs. Here every row is put in one canonical order (ids
// ascending, padding after them), its logits follow the same permutation, the
// softmax is summed again in that order, and a row without any valid id gets
// probabilities of zero.
//
// One wave per row. A row whose valid ids are distinct and span at most
// kRankBits values is placed by counting from a bitmap of its id window
// (topk_count); any other row is sorted. For the sort, each of the K slots
// becomes a 64-bit key (id << 32 | slot for a valid id, 2^31 << 32 | slot
// for padding, all ones for the positions that round K up to a power of
// two): the keys are distinct, so the sorted
// order is unique and equals the stable order with padding last. When every
// id of the row is below 2^21 - 1 the same order is carried by a 32-bit key
// (id << 10 | slot, padding as id 2^21 - 1), which halves the cross-lane
// traffic. The keys are sorted with a bitonic network held in registers:
// element i = r * 64 + lane (EPL elements per lane, so loads and stores are
// coalesced); partners at a distance below 64 are exchanged across lanes on
// the VALU (DPP for distances 1 to 8, the gfx950 lane swaps for 16 and 32),
// partners further apart are swapped between registers. The
// sorted keys give each output position its source slot, from which the id
// and the logit are gathered. The softmax: the exact maximum of the valid
// logits (a wave reduction), e = exp32(logit - max) (the gate's fixed
// sequence), the left-to-right sum of the e's in the sorted order, and one
// correctly rounded division per slot. For the sum each wave leaves its e's
// in LDS and runs the chain from uniform LDS reads issued ahead of the adds,
// one dependent add per value. Padding slots get +0.0.
#include "common.hpp"
#include "detmath.hpp"

namespace detgrad {
namespace {

constexpr int kMaxK = 1024;
constexpr int kSumAhead = 16;  // LDS reads in flight ahead of the softmax sum chain
constexpr int kRankBits = 16384;             // id window of the counting path
constexpr int kRankWords = kRankBits / 32;   // its bitmap words per row

// The value of lane ^ m, on the VALU (no LDS round trip): m = 1 and m = 2 by
// a DPP quad permutation; m = 4 and m = 8 stay inside a row of 16 lanes, so
// the partner is lane + m (row_shl) or lane - m (row_shr), whichever the
// lane's bit m selects; m = 16 and m = 32 cross rows, and the gfx950 lane
// swaps (v_permlane16_swap, v_permlane32_swap) of the value with itself give
// each lane the other half's copy in one of their two results. Every lane of
// the wave is active here (the DPP shifts' missing sources are never
// selected).
template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v, int lane) {
  const int x = static_cast<int>(v);
  if constexpr (M == 1) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true));
  } else if constexpr (M == 2) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true));
  } else if constexpr (M == 4 || M == 8) {
    const uint32_t dn = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, x, 0x110 + M, 0xF, 0xF, false));  // row_shr
    const uint32_t up = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, x, 0x100 + M, 0xF, 0xF, false));  // row_shl
    return (lane & M) ? dn : up;
  } else if constexpr (M == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane & 16) ? p[0] : p[1];
  } else {
    static_assert(M == 32, "lane distances 1 .. 32");
    const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane & 32) ? p[0] : p[1];
  }
}
template <int M>
__device__ __forceinline__ uint64_t xor_lane(uint64_t v, int lane) {
  const uint32_t lo = xor_lane<M>(static_cast<uint32_t>(v), lane), hi = xor_lane<M>(static_cast<uint32_t>(v >> 32), lane);
  return static_cast<uint64_t>(hi) << 32 | lo;
}

// Ascending bitonic sort of the wave's 64 * EPL keys, element i = r * 64 +
// lane: partners closer than 64 are in other lanes (shuffles), partners
// further apart in other registers.
// One step of phase K at distance D, then the phase's remaining steps. The
// phase and distance are template arguments, so every exchange is a fixed
// instruction sequence.
template <int EPL, int K, int D, typename T>
__device__ __forceinline__ void bitonic_step(T (&key)[EPL], int lane) {
  if constexpr (D >= 64) {
    constexpr int dr = D / 64;
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
      const int rp = r ^ dr;
      if (rp > r) {
        const int i = r * 64 + lane;
        const bool up = (i & K) == 0;
        const T a = key[r], b = key[rp];
        const bool swap = up ? (a > b) : (a < b);
        key[r] = swap ? b : a;
        key[rp] = swap ? a : b;
      }
    }
  } else {
    // all exchanges of the step first, so that they are in flight together
    T o[EPL];
#pragma unroll
    for (int r = 0; r < EPL; ++r) o[r] = xor_lane<D>(key[r], lane);
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
      const int i = r * 64 + lane;
      const bool up = (i & K) == 0;
      const bool lower = (i & D) == 0;  // this element is the lower index of the pair
      // an ascending pair keeps the smaller key at its lower index. The
      // element takes its partner's key when that one belongs here: the
      // smaller one where the minimum stays, the larger one where the maximum
      // does. Keys are distinct except the all-ones padding, and for equal
      // keys either choice keeps the same value, so one compare decides.
      const bool keep_min = (up == lower);
      key[r] = ((o[r] > key[r]) != keep_min) ? o[r] : key[r];
    }
  }
  if constexpr (D > 1) bitonic_step<EPL, K, D / 2>(key, lane);
}

template <int EPL, int K, typename T>
__device__ __forceinline__ void bitonic_phase(T (&key)[EPL], int lane) {
  bitonic_step<EPL, K, K / 2>(key, lane);
  if constexpr (K < 64 * EPL) bitonic_phase<EPL, 2 * K>(key, lane);
}

template <int EPL, typename T>
__device__ __forceinline__ void bitonic(T (&key)[EPL], int lane) {
  bitonic_phase<EPL, 2>(key, lane);
}

// True when every valid id of the row is below 2^21 - 1 (so id << 10 | slot
// is a 32-bit key).
template <int EPL>
__device__ __forceinline__ bool wave_ids_narrow(const uint64_t (&key)[EPL]) {
  bool wide = false;
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    const uint32_t hi = static_cast<uint32_t>(key[r] >> 32);
    wide = wide || (key[r] != ~0ull && hi != 0x80000000u && hi >= 0x1FFFFFu);
  }
  return __ballot(wide) == 0;
}

// A row's ids and logits in slot order (position i = r * 64 + lane; past K
// or past Q: id 0, logit 0, never used).
template <int EPL>
struct TopkRow {
  int32_t id[EPL];
  float lg[EPL];
};

template <int EPL>
__device__ __forceinline__ void topk_load(TopkRow<EPL>& in, const int32_t* __restrict__ ids,
                                          const float* __restrict__ logits, int64_t q, bool row, int K, int64_t ld,
                                          int lane) {
  const int32_t* const ir = ids + (row ? q : 0) * ld;
  const float* const lr = logits + (row ? q : 0) * ld;
  // Every id load before the logit loads, none under a branch (a position past
  // K reads slot K - 1 of the row and is then replaced): the placement needs
  // only the ids, so it starts while the logits are still in flight.
  int32_t iv[EPL];
  float lv[EPL];
#pragma unroll
  for (int r = 0; r < EPL; ++r) iv[r] = ir[r * 64 + lane < K ? r * 64 + lane : K - 1];
#pragma unroll
  for (int r = 0; r < EPL; ++r) lv[r] = lr[r * 64 + lane < K ? r * 64 + lane : K - 1];
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    const bool in_row = row && r * 64 + lane < K;
    in.id[r] = in_row ? iv[r] : 0;
    in.lg[r] = in_row ? lv[r] : 0.0f;
  }
}

// Compiler barrier between the LDS phases of one wave (a wave's LDS accesses
// execute in program order; this keeps the compiler from moving them).
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

// The row's canonical positions by counting, for a row whose valid ids are
// distinct and span fewer than kRankBits values (lo .. hi): each valid id sets
// bit id - lo of the wave's LDS bitmap, a valid slot's position is the number
// of set bits below its own (the words' exclusive prefix counts from one wave
// scan, plus a popcount inside the word), and a padding slot's position is nv
// plus the padding slots before it. Every slot's id and logit are written at
// that position of is and es. A repeated id shows as a bit that the LDS atomic
// OR finds already set. Returns false, placing nothing, for a wider span or a
// repeated id (the row is then sorted); both ways give every slot the same
// position, so the choice never changes a bit.
template <int EPL>
__device__ __forceinline__ bool topk_count(const TopkRow<EPL>& in, bool row, int K, int lane, float* es, int32_t* is,
                                           uint32_t* bm, uint32_t* pre, int& nv_out) {
  int lo = 0x7FFFFFFF, hi = -1;
  int nv = 0;
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    const bool valid = row && r * 64 + lane < K && in.id[r] >= 0;
    if (valid) {
      lo = in.id[r] < lo ? in.id[r] : lo;
      hi = in.id[r] > hi ? in.id[r] : hi;
    }
    nv += __builtin_popcountll(__ballot(valid));
  }
  auto mm = [&](int olo, int ohi) {
    lo = olo < lo ? olo : lo;
    hi = ohi > hi ? ohi : hi;
  };
  mm(static_cast<int>(xor_lane<32>(static_cast<uint32_t>(lo), lane)), static_cast<int>(xor_lane<32>(static_cast<uint32_t>(hi), lane)));
  mm(static_cast<int>(xor_lane<16>(static_cast<uint32_t>(lo), lane)), static_cast<int>(xor_lane<16>(static_cast<uint32_t>(hi), lane)));
  mm(static_cast<int>(xor_lane<8>(static_cast<uint32_t>(lo), lane)), static_cast<int>(xor_lane<8>(static_cast<uint32_t>(hi), lane)));
  mm(static_cast<int>(xor_lane<4>(static_cast<uint32_t>(lo), lane)), static_cast<int>(xor_lane<4>(static_cast<uint32_t>(hi), lane)));
  mm(static_cast<int>(xor_lane<2>(static_cast<uint32_t>(lo), lane)), static_cast<int>(xor_lane<2>(static_cast<uint32_t>(hi), lane)));
  mm(static_cast<int>(xor_lane<1>(static_cast<uint32_t>(lo), lane)), static_cast<int>(xor_lane<1>(static_cast<uint32_t>(hi), lane)));
  if (nv > 0 && hi - lo >= kRankBits) return false;  // (wave-uniform; hi >= lo >= 0 here)
  uint4* const b4 = reinterpret_cast<uint4*>(bm);
  static_assert(kRankWords == 64 * 8, "a lane owns eight bitmap words");
  b4[2 * lane] = make_uint4(0u, 0u, 0u, 0u);
  b4[2 * lane + 1] = make_uint4(0u, 0u, 0u, 0u);
  lds_order();
  bool dup = false;
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    if (row && r * 64 + lane < K && in.id[r] >= 0) {
      const uint32_t b = static_cast<uint32_t>(in.id[r] - lo), bit = 1u << (b & 31u);
      dup = dup || (atomicOr(&bm[b >> 5], bit) & bit) != 0u;
    }
  }
  if (__ballot(dup) != 0ull) return false;
  lds_order();
  // lane l owns words 8 l .. 8 l + 7
  const uint4 wa = b4[2 * lane], wb = b4[2 * lane + 1];
  const uint32_t c[8] = {static_cast<uint32_t>(__builtin_popcount(wa.x)), static_cast<uint32_t>(__builtin_popcount(wa.y)),
                         static_cast<uint32_t>(__builtin_popcount(wa.z)), static_cast<uint32_t>(__builtin_popcount(wa.w)),
                         static_cast<uint32_t>(__builtin_popcount(wb.x)), static_cast<uint32_t>(__builtin_popcount(wb.y)),
                         static_cast<uint32_t>(__builtin_popcount(wb.z)), static_cast<uint32_t>(__builtin_popcount(wb.w))};
  const uint32_t tot = ((c[0] + c[1]) + (c[2] + c[3])) + ((c[4] + c[5]) + (c[6] + c[7]));
  uint32_t run = wave_incl_scan(tot) - tot;
  uint32_t pr[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    pr[j] = run;
    run += c[j];
  }
  uint4* const p4 = reinterpret_cast<uint4*>(pre);
  p4[2 * lane] = make_uint4(pr[0], pr[1], pr[2], pr[3]);
  p4[2 * lane + 1] = make_uint4(pr[4], pr[5], pr[6], pr[7]);
  lds_order();
  int pads = 0;  // padding slots in the registers before r (wave-uniform)
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    const bool in_row = row && r * 64 + lane < K;
    const bool valid = in_row && in.id[r] >= 0, pad = in_row && in.id[r] < 0;
    const uint64_t pm = __ballot(pad);
    int pos = 0;
    if (valid) {
      const uint32_t b = static_cast<uint32_t>(in.id[r] - lo), w = b >> 5;
      pos = static_cast<int>(pre[w] + static_cast<uint32_t>(__builtin_popcount(bm[w] & ((1u << (b & 31u)) - 1u))));
    } else {
      pos = nv + pads +
            static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(pm >> 32),
                                                       __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(pm), 0u)));
    }
    if (valid || pad) {
      is[pos] = in.id[r];
      es[pos] = in.lg[r];
    }
    pads += __builtin_popcountll(pm);
  }
  lds_order();
  nv_out = nv;
  return true;
}

// One row, by one wave, from its loaded ids and logits; es and is are the
// wave's LDS rows.
template <int EPL>
__device__ __forceinline__ void topk_row(const TopkRow<EPL>& in, int64_t q, bool row, int K, int lane, float* es,
                                         int32_t* is, uint32_t* bm, uint32_t* pre, int32_t* __restrict__ ids_out,
                                         float* __restrict__ logits_out, float* __restrict__ probs,
                                         int64_t ld_out) {
  constexpr int N = 64 * EPL;  // padded row length, a power of two
  int32_t idv[EPL];
  float lg[EPL];
  int nv = 0;
  if (topk_count<EPL>(in, row, K, lane, es, is, bm, pre, nv)) {
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
      const int i = r * 64 + lane;
      const bool in_row = row && i < K;
      idv[r] = in_row ? is[i] : 0;
      lg[r] = in_row ? es[i] : 0.0f;
    }
  } else {
    // element i = r * 64 + lane: partners at distance d < 64 sit in another
    // lane, at d >= 64 in another register
    uint64_t key[EPL];
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
      const int i = r * 64 + lane;
      if (row && i < K) {
        const int32_t id = in.id[r];
        const uint32_t hi = id >= 0 ? static_cast<uint32_t>(id) : 0x80000000u;
        key[r] = static_cast<uint64_t>(hi) << 32 | static_cast<uint32_t>(i);
      } else {
        key[r] = ~0ull;
      }
    }
    // keys of 32 bits (id << 10 | slot) when every id of the row is below
    // 2^21 - 1 (K <= 1024 slots), else of 64 bits: the same order, half the
    // cross-lane traffic
    const bool narrow = wave_ids_narrow<EPL>(key);
    if (narrow) {
      uint32_t k32[EPL];
#pragma unroll
      for (int r = 0; r < EPL; ++r) {
        const uint32_t hi = static_cast<uint32_t>(key[r] >> 32), lo = static_cast<uint32_t>(key[r]);
        k32[r] = key[r] == ~0ull ? ~0u : ((hi == 0x80000000u ? 0x1FFFFFu : hi) << 10 | lo);
      }
      bitonic<EPL>(k32, lane);
#pragma unroll
      for (int r = 0; r < EPL; ++r) {
        const uint32_t hi = k32[r] >> 10, lo = k32[r] & 0x3FFu;
        key[r] = k32[r] == ~0u ? ~0ull
                               : (static_cast<uint64_t>(hi == 0x1FFFFFu ? 0x80000000u : hi) << 32 | lo);
      }
    } else {
      bitonic<EPL>(key, lane);
    }
    // ids and logits by source slot from the wave's LDS rows (parked there in
    // slot order; padding keeps its own negative id); the valid slots come
    // first.
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
      es[r * 64 + lane] = in.lg[r];
      is[r * 64 + lane] = in.id[r];
    }
    int nv_lane = 0;
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
      const int i = r * 64 + lane;
      const uint32_t slot = static_cast<uint32_t>(key[r]);
      const bool in_row = row && i < K;
      idv[r] = in_row ? is[slot] : 0;
      lg[r] = in_row ? es[slot] : 0.0f;
      nv_lane += (in_row && (key[r] >> 32) < 0x80000000ull) ? 1 : 0;
    }
    uint32_t nvu = static_cast<uint32_t>(nv_lane);
    nvu += xor_lane<32>(nvu, lane);
    nvu += xor_lane<16>(nvu, lane);
    nvu += xor_lane<8>(nvu, lane);
    nvu += xor_lane<4>(nvu, lane);
    nvu += xor_lane<2>(nvu, lane);
    nvu += xor_lane<1>(nvu, lane);
    nv = static_cast<int>(nvu);
  }
  // exact maximum of the valid logits (positions below nv) over the wave
  // (butterflies over lane distances 32, 16, .., 1, the same in every lane)
  float mx = -__builtin_inff();
#pragma unroll
  for (int r = 0; r < EPL; ++r)
    if (r * 64 + lane < nv) mx = mx > lg[r] ? mx : lg[r];
  auto max_step = [&](float o) { mx = mx > o ? mx : o; };
  max_step(__uint_as_float(xor_lane<32>(__float_as_uint(mx), lane)));
  max_step(__uint_as_float(xor_lane<16>(__float_as_uint(mx), lane)));
  max_step(__uint_as_float(xor_lane<8>(__float_as_uint(mx), lane)));
  max_step(__uint_as_float(xor_lane<4>(__float_as_uint(mx), lane)));
  max_step(__uint_as_float(xor_lane<2>(__float_as_uint(mx), lane)));
  max_step(__uint_as_float(xor_lane<1>(__float_as_uint(mx), lane)));
  // e values in sorted order: each wave parks its row in LDS, then every lane
  // runs the row's left-to-right sum from the same uniform-address LDS reads
  // (four values per read, the reads issued ahead of their adds), so the wave
  // needs no barrier and every lane ends with the sum. Positions past nv hold
  // +0.0: once a valid value has been added the sum is not -0.0, so adding
  // +0.0 leaves its bits unchanged, and the chain can run over the whole
  // padded row; a row without valid values uses no sum.
  float e[EPL];
  const float4* const ew = reinterpret_cast<const float4*>(es);
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    const int i = r * 64 + lane;
    e[r] = i < nv ? dm::exp32(lg[r] - mx) : 0.0f;
    es[i] = e[r];
  }
  constexpr int kN4 = N / 4;
  float S = -0.0f;
  float4 w[kSumAhead];
#pragma unroll
  for (int t = 0; t < kSumAhead; ++t) w[t] = ew[t];
  // (no scheduling barriers here: the compiler keeps the reads ahead by
  // itself, and barriers in this fully unrolled loop made it spill)
#pragma unroll
  for (int t = 0; t < kN4; ++t) {
    const float4 x = w[t % kSumAhead];
    if (t + kSumAhead < kN4) w[t % kSumAhead] = ew[t + kSumAhead];
    S = S + x.x;
    S = S + x.y;
    S = S + x.z;
    S = S + x.w;
  }
  if (!row) return;  // (wave-uniform)
  int32_t* const io = ids_out + q * ld_out;
  float* const lo = logits_out + q * ld_out;
  float* const po = probs + q * ld_out;
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
    const int i = r * 64 + lane;
    if (i < K) {
      io[i] = idv[r];
      lo[i] = lg[r];
      po[i] = i < nv ? e[r] / S : 0.0f;
    }
  }
}

// One wave per row, four rows per workgroup. (Two rows per wave, the second
// row's loads in flight during the first row's sort, was slower: half as
// many waves hide less latency.)
template <int EPL>
__global__ __launch_bounds__(256) void topk_canon_kernel(const int32_t* __restrict__ ids, const float* __restrict__ logits,
                                                         int64_t Q, int K, int64_t ld, int32_t* __restrict__ ids_out,
                                                         float* __restrict__ logits_out, float* __restrict__ probs,
                                                         int64_t ld_out) {
  constexpr int N = 64 * EPL;
  __shared__ __attribute__((aligned(16))) float es[4][N];  // each wave's logits by slot, then its e values in sorted order
  __shared__ int32_t is[4][N];                             // each wave's ids by slot
  __shared__ __attribute__((aligned(16))) uint32_t bm[4][kRankWords];   // each wave's id bitmap (counting path)
  __shared__ __attribute__((aligned(16))) uint32_t pre[4][kRankWords];  // its words' exclusive prefix counts
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t q = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  TopkRow<EPL> in;
  topk_load<EPL>(in, ids, logits, q, q < Q, K, ld, lane);
  topk_row<EPL>(in, q, q < Q, K, lane, es[wave], is[wave], bm[wave], pre[wave], ids_out, logits_out, probs,
                 ld_out);
}

}  // namespace
}  // namespace detgrad

using namespace detgrad;

extern "C" int det_topk_canonicalize(const int32_t* ids, const float* logits, int64_t Q, int64_t K, int64_t ld,
                                     int32_t* ids_out, float* logits_out, float* probs, int64_t ld_out,
                                     void* stream) {
  if (Q < 0 || K < 0) return set_error(DET_ERR_INVALID_ARG, "topk: Q and K must be >= 0");
  if (K > kMaxK) return set_error(DET_ERR_UNSUPPORTED, "topk: K must be <= %d, got %lld", kMaxK, static_cast<long long>(K));
  if (Q == 0 || K == 0) return ok();
  if (!ids || !logits || !ids_out || !logits_out || !probs) return set_error(DET_ERR_INVALID_ARG, "topk: NULL pointer");
  if (ld < K || ld_out < K) return set_error(DET_ERR_INVALID_ARG, "topk: ld and ld_out must be >= K");
  if (ceil_div(Q, 4) > 0x7FFFFFFF) return set_error(DET_ERR_UNSUPPORTED, "topk: Q too large");
  const Range ins[] = {range2d(ids, Q, K, ld, 4), range2d(logits, Q, K, ld, 4)};
  const Range outs[] = {range2d(ids_out, Q, K, ld_out, 4), range2d(logits_out, Q, K, ld_out, 4),
                        range2d(probs, Q, K, ld_out, 4)};
  for (int a = 0; a < 3; ++a) {
    for (const Range& r : ins)
      if (overlaps(outs[a], r)) return set_error(DET_ERR_OVERLAP, "topk: an output overlaps an input");
    for (int b = a + 1; b < 3; ++b)
      if (overlaps(outs[a], outs[b])) return set_error(DET_ERR_OVERLAP, "topk: outputs overlap each other");
  }
  const hipStream_t st = as_stream(stream);
  const dim3 grid(static_cast<uint32_t>(ceil_div(Q, 4)));
  const int epl = K <= 64 ? 1 : (K <= 128 ? 2 : (K <= 256 ? 4 : (K <= 512 ? 8 : 16)));
#define DET_TOPK_LAUNCH(E)                                                                                       \
  if (epl == E)                                                                                                  \
    hipLaunchKernelGGL(topk_canon_kernel<E>, grid, dim3(256), 0, st, ids, logits, Q, static_cast<int>(K), ld,   \
                       ids_out, logits_out, probs, ld_out);
  DET_TOPK_LAUNCH(1) DET_TOPK_LAUNCH(2) DET_TOPK_LAUNCH(4) DET_TOPK_LAUNCH(8) DET_TOPK_LAUNCH(16)
#undef DET_TOPK_LAUNCH
  return check_launch("det_topk_canonicalize");
}
