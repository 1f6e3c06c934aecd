// Shared host and device helpers of libdetgrad (gfx950).
//
// Arithmetic rule for every deterministic kernel: IEEE binary32 with
// round-to-nearest-even, one rounding per + - * /, no contraction (the library
// is compiled with -ffp-contract=off), no flush of subnormals. bf16 inputs are
// widened exactly by a 16-bit shift.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstddef>
#include <cstdint>
#include <cstdio>

#include "../../include/detgrad.h"

namespace detgrad {

// ------------------------------------------------------------------ host side
int set_error(int status, const char* fmt, ...);
int ok();  // clears the thread's error text, returns DET_OK
int check_launch(const char* what);  // hipGetLastError after a launch

struct Range {
  uintptr_t lo = 0, hi = 0;  // [lo, hi) bytes; empty when lo == hi
};

// Bytes covered by a strided 2-D tensor of rows x cols elements.
inline Range range2d(const void* p, int64_t rows, int64_t cols, int64_t ld, size_t elem) {
  Range r;
  if (!p || rows <= 0 || cols <= 0) return r;
  r.lo = reinterpret_cast<uintptr_t>(p);
  r.hi = r.lo + static_cast<uintptr_t>(((rows - 1) * ld + cols) * static_cast<int64_t>(elem));
  return r;
}

// Bytes covered by a strided 2-D view with arbitrary positive element strides.
inline Range range_strided(const void* p, int64_t d0, int64_t d1, int64_t s0, int64_t s1, size_t elem) {
  Range r;
  if (!p || d0 <= 0 || d1 <= 0) return r;
  r.lo = reinterpret_cast<uintptr_t>(p);
  r.hi = r.lo + static_cast<uintptr_t>(((d0 - 1) * s0 + (d1 - 1) * s1 + 1) * static_cast<int64_t>(elem));
  return r;
}

inline Range range1d(const void* p, size_t bytes) {
  Range r;
  if (!p || bytes == 0) return r;
  r.lo = reinterpret_cast<uintptr_t>(p);
  r.hi = r.lo + bytes;
  return r;
}

inline bool overlaps(const Range& a, const Range& b) {
  return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

// Common checks of the `atomic` flag and the workspace.
int check_atomic_flag(int atomic);
int check_workspace(const void* ws, size_t ws_bytes, size_t need);

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// ---------------------------------------------------------------- device side
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// Cross-lane moves inside a 16-lane DPP row. After k levels of an adjacent
// pairwise tree, every lane of an aligned block of 2^k lanes holds that block's
// value; these controls fetch the value of the neighbouring block, so adding it
// performs the next tree level in every lane (binary32 addition is
// commutative bit for bit, so both blocks obtain the same sum).
//   level over lane pairs (i, i^1):  quad_perm [1,0,3,2]
//   level over pairs of 2-blocks:     quad_perm [2,3,0,1]
//   level over pairs of 4-blocks:     row_half_mirror (lane i <- 7-i in each 8)
//   level over pairs of 8-blocks:     row_mirror      (lane i <- 15-i)
enum : int { DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140 };

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Adjacent pairwise tree across the 16 lanes of a DPP row; every lane of the
// row ends with the row's total.
__device__ __forceinline__ float row16_tree(float v) {
  v = v + dpp_mov<DPP_XOR1>(v);
  v = v + dpp_mov<DPP_XOR2>(v);
  v = v + dpp_mov<DPP_HALF_MIRROR>(v);
  v = v + dpp_mov<DPP_MIRROR>(v);
  return v;
}

__device__ __forceinline__ float readlane(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Integer scans on DPP row shifts and row broadcasts in registers.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_add(uint32_t v) {
  // lanes without a source lane read 0 (the `old` operand)
  return v + static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROW_MASK, 0xF, false));
}

// Inclusive scan over the 64 lanes: shifts by 1, 2, 4, 8 inside each row of
// 16, then the last lane of row 0 into row 1 and 3 (row_bcast:15) and of row
// 1 into rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v = dpp_add<0x111, 0xF>(v);  // row_shr:1
  v = dpp_add<0x112, 0xF>(v);  // row_shr:2
  v = dpp_add<0x114, 0xF>(v);  // row_shr:4
  v = dpp_add<0x118, 0xF>(v);  // row_shr:8
  v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  return v;
}

}  // namespace detgrad
