// Shared device and host helpers of libdiagattn (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/diagattn.h"

namespace da {

// ---------------------------------------------------------------- host side

// Records `msg` as the calling thread's last error and returns `code`.
int fail(int code, const char* fmt, ...);
// Clears the thread's last error.
void clear_error();
// Checks hipGetLastError() after a launch; returns DA_OK or DA_EHIP.
int check_launch(const char* what);
// Validates a mask; DA_OK or DA_EINVAL with the reason recorded.
int check_mask(const da_mask* m);

inline bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
inline int ilog2(int64_t x) {
  int r = 0;
  while ((int64_t(1) << r) < x) ++r;
  return r;
}

// Window-part keep test shared by the host count and the device builder:
// d = i - j for a key j >= P inside the window range.  Future keys (d < 0,
// matrix form only) are kept within B; past keys within B of the main
// diagonal (BAND) or of any raster-row diagonal k*G (ROWDIAG).
// d is 64-bit so that d = i - j stays exact for any int32 i, j; a past
// key's d (0 <= d <= i) fits 32 bits, so the residue is a 32-bit modulo.
__host__ __device__ inline bool window_keep(int mode, int64_t d, int B, int G) {
  if (d < 0) return -d <= (int64_t)B;
  if (mode == DA_MODE_BAND) return d <= B;
  const int r = (int)((uint32_t)d % (uint32_t)G);
  return r <= B || G - r <= B;
}

// ---------------------------------------------------------------- device side

__device__ inline int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// 16-byte vector of raw bits (8 bf16 or 4 fp32).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN -> quiet NaN).
__device__ inline uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Unpacks one 16-byte chunk into EPL floats.
template <int EPL>
__device__ inline void unpack(const u32x4 w, float (&x)[EPL]) {
  if constexpr (EPL == 8) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf16_lo(w[e]);
      x[2 * e + 1] = bf16_hi(w[e]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(w[e]);
  }
}

// Matrix-core operand and result types.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef short v4i16 __attribute__((ext_vector_type(4)));

// Max across the lanes l, l ^ 16, l ^ 32 and l ^ 48 (VALU lane swaps): the
// four lanes that hold one column of a 16x16 matrix-core result.
__device__ inline float max_over_row_groups(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Sum across the lanes l, l ^ 16, l ^ 32 and l ^ 48.
__device__ inline float sum_over_row_groups(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// LDS position of 16-byte chunk p of row r is p ^ swz(r) in row-major tiles
// of CPR chunks a row.  The tiles are read two ways: as matrix-core A
// operands (ds_read_b128: lane l reads row l % 16, chunk 4c + l / 16) and
// transposed (ds_read_b64_tr_b16: rows 4(l / 16) + (l % 16) / 4, chunks
// 2m + (l % 4) / 2).  Both patterns read with no bank conflict under these
// swizzles, as measured with the LDS bank-conflict counter on this part
// (the earlier choice for 16 chunks, ((r & 7) << 1) | ((r >> 3) & 1), left
// four conflict cycles on every operand read).  The 16-chunk swizzle is an
// XOR-linear map of r mod 16, so rows 16 apart share it and their LDS
// addresses differ by a constant.
template <int CPR>
__device__ inline int swz(int r) {
  if constexpr (CPR == 16) return (r & 3) ^ ((r & 1) << 2) ^ ((r & 4) << 1) ^ (((r >> 3) & 1) * 9);
  else return r % CPR;
}

// DPP lane moves within 16-lane rows.
template <int CTRL>
__device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int DPP_XOR1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;
constexpr int DPP_MIRROR = 0x140;

// Sum over aligned groups of N consecutive lanes (N = 8, 16 or 32); every
// lane of the group receives the group sum.
template <int N>
__device__ inline float group_sum(float x) {
  static_assert(N == 8 || N == 16 || N == 32, "group size");
  x += dpp<DPP_XOR1>(x);
  x += dpp<DPP_XOR2>(x);
  x += dpp<DPP_HALF_MIRROR>(x);
  if constexpr (N >= 16) x += dpp<DPP_MIRROR>(x);
  if constexpr (N == 32) x += __shfl_xor(x, 16);
  return x;
}

}  // namespace da
