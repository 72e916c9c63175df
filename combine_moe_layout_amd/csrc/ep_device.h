// ep_device.h -- device helpers shared by the gfx950 kernels of libep.so: the
// wave64 width, 16-byte vector types with non-temporal accesses, and bf16 and
// OCP FP8 E4M3 conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kFp8Block = 128;     // channels per FP8 scale
constexpr float kFp8Max = 448.0f;  // largest finite E4M3 value
constexpr float kScaleFloor = 1e-4f;

struct alignas(16) u32x4 {
  uint32_t x, y, z, w;
};
typedef uint32_t u32x4_vec __attribute__((ext_vector_type(4)));

// 16-byte (and 8-byte) loads and stores with the non-temporal hint, for
// streams touched once.  Each wave instruction using them must cover whole
// cache lines (64 lanes x 16 or 8 contiguous bytes: 1 KiB or 512 B): a
// non-temporal access does not keep the line, so a second instruction reading
// the other half of a line would fetch it again.
// Inclusive sum over the 64 lanes of a wave with DPP moves (no LDS): four
// shifts inside each row of 16 lanes, then row 0's and row 2's last lanes
// into rows 1 and 3, then lane 31 into rows 2 and 3.  Every lane of the wave
// must be active.
__device__ __forceinline__ int32_t wave_inclusive_sum(int32_t x) {
  const int row_lane = threadIdx.x & 15;
  const int row = (threadIdx.x & 63) >> 4;
  int32_t t;
  t = __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  if (row_lane >= 1) x += t;
  t = __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  if (row_lane >= 2) x += t;
  t = __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  if (row_lane >= 4) x += t;
  t = __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  if (row_lane >= 8) x += t;
  t = __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  if (row & 1) x += t;
  t = __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  if (row >= 2) x += t;
  return x;
}

__device__ __forceinline__ u32x4 load_nt(const u32x4* p) {
  const u32x4_vec v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_vec*>(p));
  return u32x4{v.x, v.y, v.z, v.w};
}
typedef uint32_t u32x2_vec __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2_vec load_nt8(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2_vec*>(p));
}
__device__ __forceinline__ void store_nt(u32x4* p, const u32x4& a) {
  const u32x4_vec v = {a.x, a.y, a.z, a.w};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_vec*>(p));
}

__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) {
  return __uint_as_float(packed & 0xFFFF0000u);
}

// fp32 -> bf16 bit pattern, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

// Rounds the exact value p + err to bf16 (nearest, ties to even), where p is an
// fp32 value and err the exact remainder of the product that produced it
// (|err| <= half an fp32 ulp of p).  Only a p that sits exactly on a bf16
// midpoint needs err: then err's sign decides the direction.
__device__ __forceinline__ uint32_t bf16_round_exact(float p, float err) {
  uint32_t u = __float_as_uint(p);
  if ((u & 0xFFFFu) == 0x8000u && err != 0.0f) {
    bool away = (err > 0.0f) == (p > 0.0f);  // exact value lies beyond the midpoint
    return away ? (u >> 16) + 1u : (u >> 16);
  }
  return bf16_rne(p);
}

// ---------------------------------------------------------------------------
// OCP FP8 E4M3 (bias 7, 3 mantissa bits, subnormals, largest finite 448).
// ---------------------------------------------------------------------------

// Software encoder of v already clamped to [-448, 448]: nearest code, ties to
// even, sign kept (a negative value that rounds to zero gives 0x80).
__device__ __forceinline__ uint32_t e4m3_encode_sw(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t mag = u & 0x7FFFFFFFu;
  uint32_t code;
  if (mag >= 0x3C800000u) {  // |v| >= 2^-6: normal E4M3 range
    uint32_t e8 = (mag >> 23) - 120u;  // unbiased exponent + 7
    uint32_t m = mag & 0x7FFFFFu;
    code = (e8 << 3) | (m >> 20);
    uint32_t rem = m & 0xFFFFFu;
    code += (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) ? 1u : 0u;
    code = code > 0x7Eu ? 0x7Eu : code;  // a guard: |v| <= 448 never rounds past 0x7E
  } else {
    // subnormal codes are multiples of 2^-9: round |v| * 2^9 to an integer, ties to even
    code = (uint32_t)__builtin_rintf(__uint_as_float(mag) * 512.0f);
  }
  return sign | code;
}

// Hardware conversion of two clamped values to two E4M3 bytes (low 16 bits).
__device__ __forceinline__ uint32_t e4m3_encode2_hw(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Encode four clamped values into one 32-bit word, byte i = value i.
template <bool kHw>
__device__ __forceinline__ uint32_t e4m3_encode4(float a, float b, float c, float d) {
  if constexpr (kHw) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
  } else {
    return e4m3_encode_sw(a) | (e4m3_encode_sw(b) << 8) | (e4m3_encode_sw(c) << 16) |
           (e4m3_encode_sw(d) << 24);
  }
}

// Clamp to [-448, 448] (one v_med3_f32).  A NaN comes out as -448, so
// callers that can meet NaN test for it themselves.
__device__ __forceinline__ float clamp_fp8(float v) { return fminf(fmaxf(v, -kFp8Max), kFp8Max); }

// E4M3 code -> fp32 (exact).  0x7F / 0xFF decode to NaN.
__device__ __forceinline__ float e4m3_decode(uint32_t code) {
  uint32_t s = (code & 0x80u) << 24;
  uint32_t e = (code >> 3) & 0xFu;
  uint32_t m = code & 7u;
  float mag;
  if (e == 0u) {
    mag = (float)m * 0.001953125f;  // m * 2^-9
  } else if (e == 15u && m == 7u) {
    mag = __uint_as_float(0x7FC00000u);
  } else {
    mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
  }
  return __uint_as_float(__float_as_uint(mag) | s);
}

}  // namespace ep
