// Device helpers shared by the libtq kernels (internal, not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "tq.h"

namespace tq {

constexpr int kWave = 64;

__device__ inline float load_in(const void *x, int dtype, size_t i) {
  if (dtype == TQ_BF16) {
    uint32_t u = static_cast<uint32_t>(static_cast<const uint16_t *>(x)[i]) << 16;
    return __uint_as_float(u);
  }
  return static_cast<const float *>(x)[i];
}

// The value of lane l ^ s (s = 32, 16, 8, 4, 2, 1).  Below 16 the exchange stays
// inside a 16-lane row, so it is a DPP move (no LDS round trip): a rotation by
// 8, quad permutations for 2 and 1, and for 4 a shift up or down by 4 chosen
// by the lane's own bit 2 (DPP controls as measured on gfx950: row_shl:n reads
// lane l + n, row_shr:n lane l - n, row_ror:8 lane l ^ 8).
__device__ inline uint32_t lane_xor(uint32_t a, int s, int lane) {
  const int v = static_cast<int>(a);
  switch (s) {
    case 8: return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false));
    case 4: {
      const int up = __builtin_amdgcn_update_dpp(0, v, 0x104, 0xF, 0xF, false);
      const int dn = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);
      return static_cast<uint32_t>((lane & 4) ? dn : up);
    }
    case 2: return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));
    case 1: return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));
    default: return static_cast<uint32_t>(__shfl_xor(v, s, kWave));
  }
}

__device__ inline float lane_xor_f(float v, int s, int lane) {
  return __uint_as_float(lane_xor(__float_as_uint(v), s, lane));
}

__device__ inline double wave_sum_d(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ inline float wave_sum_f(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ inline float wave_max_f(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// IEEE binary16 bits of v >= 0, rounded to nearest even directly from float64.
// v > 65504 saturates to 65504 and sets *over.
__device__ inline uint32_t f16_bits(double v, bool *over) {
  if (!(v == v)) return 0x7E00u;
  if (v > 65504.0) {
    *over = true;
    return 0x7BFFu;
  }
  if (v < 6.103515625e-05) return static_cast<uint32_t>(rint(v * 16777216.0));  // subnormal grid 2^-24
  int e;
  double f = frexp(v, &e);                         // v = f 2^e, f in [0.5, 1)
  double mant = rint((f * 2.0 - 1.0) * 1024.0);    // exact scaling, then RNE
  int ex = e - 1;
  if (mant >= 1024.0) {
    mant = 0.0;
    ex += 1;
  }
  return (static_cast<uint32_t>(ex + 15) << 10) | static_cast<uint32_t>(mant);
}

__device__ inline float f16_val(uint32_t bits) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

}  // namespace tq
