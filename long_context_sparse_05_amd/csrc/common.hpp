// common.hpp -- device helpers shared by the gfx950 indexer kernels.
//
// Data formats: keys and queries are bf16 (stored as uint16 bits), weights
// and scores fp32.  MFMA lane layouts used below (v_mfma_f32_16x16x32_bf16,
// wave64): lane l supplies A[row = l%16][k = 8*(l/16) + e] and
// B[k = 8*(l/16) + e][col = l%16] for e = 0..7, and receives
// D[row = 4*(l/16) + r][col = l%16] for r = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace misa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;          // key dimension
#define MISA_MAX_HEADS_DEV 128   // largest H the kernels are built for
constexpr int kWave = 64;        // wavefront width on CDNA
constexpr int kHistBits = 12;    // first radix digit: top 12 bits of the key
constexpr int kHistBins = 1 << kHistBits;
constexpr int kHistShift = 32 - kHistBits;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// 16-byte load marked non-temporal: streamed data that is read once should
// not displace reused lines from the caches.
__device__ __forceinline__ uint4 load_nt16(const void *p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4 *)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// An LDS address, for the buffer loads that write LDS directly.
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float(((uint32_t)u) << 16);
}

// Order-preserving map of a non-NaN fp32 to uint32 (larger float -> larger
// key).  -0.0 is first folded to +0.0 so the two rank as equal.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// fp32 -> three bf16 terms whose sum is exactly x (hi, mid: truncations;
// lo: the exact remainder, at most 8 significant bits).
__device__ __forceinline__ void split3(float x, uint16_t &hi, uint16_t &mid, uint16_t &lo) {
  uint32_t ux = __float_as_uint(x);
  uint32_t uh = ux & 0xFFFF0000u;
  float r1 = x - __uint_as_float(uh);
  uint32_t um = __float_as_uint(r1) & 0xFFFF0000u;
  float r2 = r1 - __uint_as_float(um);
  hi = (uint16_t)(uh >> 16);
  mid = (uint16_t)(um >> 16);
  lo = (uint16_t)(__float_as_uint(r2) >> 16);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Sum over the 16 lanes of each DPP row (lanes 16r .. 16r+15), on the vector
// ALU with row rotations (no LDS round trip); every lane gets its row's sum.
__device__ __forceinline__ float row_sum16(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false));
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave on the DPP network:
// shifts right by 1, 2, 4 and 8 lanes within each row of 16 (lanes whose
// source falls outside the row add 0), then lane 15 of rows 0 and 2 is
// added to rows 1 and 3 (row_bcast:15) and lane 31 to rows 2 and 3
// (row_bcast:31).  No LDS traffic, unlike a ds_bpermute shuffle.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);
  return v;
}

// Wave-wide maximum of unsigned values (the same DPP pattern; lane 63 ends
// with the maximum of all lanes), returned in every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

}  // namespace misa
