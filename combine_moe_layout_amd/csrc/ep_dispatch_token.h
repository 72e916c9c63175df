// ep_dispatch_token.h -- the per-token work of dispatch, shared by the
// dispatch kernels and the fused low-latency layout+dispatch kernel.
//
// A token's lanes are lt = 0 .. lanes-1; each lane walks the row in steps of
// `lanes` vectors.  `slots` holds the token's k receive rows (-1 = none) and
// may live in global memory or LDS.
#pragma once

#include "ep.h"
#include "ep_device.h"

namespace ep {

// Scales of one token fit in LDS: hidden <= EP_MAX_HIDDEN gives at most 512.
constexpr int kMaxScalesPerBlock = EP_MAX_HIDDEN / kFp8Block;

// bf16: 8 channels (one 16-byte vector) per lane and step, copied to every
// valid row with non-temporal stores (the rows are written once).
__device__ __forceinline__ void bf16_token_copy(const u32x4* __restrict__ src, int32_t hidden,
                                                int32_t lt, int32_t lanes, const int32_t* slots,
                                                int32_t k, u32x4* __restrict__ recv) {
  const int32_t vec_per_row = hidden / 8;
  for (int32_t v = lt; v < vec_per_row; v += lanes) {
    const u32x4 d = src[v];
    for (int32_t j = 0; j < k; ++j) {
      const int32_t s = slots[j];
      if (s >= 0) store_nt(recv + (int64_t)s * vec_per_row + v, d);
    }
  }
}

// FP8 codes of one 16-channel slice (vector v of the code row: bf16 vectors
// 2v and 2v+1 given in lo / hi), stored to every valid row; the 8 lanes of a
// 128-channel block must call it together (their maximum is reduced with lane
// swizzles).  The block scale goes to my_scales[v / 8].
// The block scale and its reciprocal.  kPow2 = false: scale = a / 448 and
// inv = 448 / a, single correctly rounded fp32 divisions.  kPow2 = true: the
// smallest power of two s with 448 * s >= a: with a = (1 + m) * 2^ea and
// 448 = 1.75 * 2^8, s = 2^(ea - 8) when 1 + m <= 1.75 (mantissa bits <=
// 0x600000), else 2^(ea - 7); inv = 1 / s exactly.  a >= 1e-4 is normal, so
// both powers of two are normal fp32 values.
template <bool kPow2>
__device__ __forceinline__ void fp8_block_scale(float a, float& scale, float& inv) {
  if constexpr (kPow2) {
    const uint32_t bits = __float_as_uint(a);
    const int32_t e = (int32_t)(bits >> 23) - 127 - 8 + ((bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    scale = __uint_as_float((uint32_t)(127 + e) << 23);
    inv = __uint_as_float((uint32_t)(127 - e) << 23);
  } else {
    scale = a / kFp8Max;  // correctly rounded fp32 divisions
    inv = kFp8Max / a;
  }
}

template <bool kHw, bool kPow2 = false>
__device__ __forceinline__ void fp8_vector_codes(const u32x4& lo, const u32x4& hi, int32_t v,
                                                 const int32_t* slots, int32_t k,
                                                 u32x4* __restrict__ recv,
                                                 int32_t out_vec_per_row, float* my_scales) {
  float f[16] = {bf16_lo(lo.x), bf16_hi(lo.x), bf16_lo(lo.y), bf16_hi(lo.y),
                 bf16_lo(lo.z), bf16_hi(lo.z), bf16_lo(lo.w), bf16_hi(lo.w),
                 bf16_lo(hi.x), bf16_hi(hi.x), bf16_lo(hi.y), bf16_hi(hi.y),
                 bf16_lo(hi.z), bf16_hi(hi.z), bf16_lo(hi.w), bf16_hi(hi.w)};
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  amax = fmaxf(amax, __shfl_xor(amax, 4));
  float scale, inv;
  fp8_block_scale<kPow2>(fmaxf(amax, kScaleFloor), scale, inv);
  u32x4 q;
  q.x = e4m3_encode4<kHw>(clamp_fp8(f[0] * inv), clamp_fp8(f[1] * inv), clamp_fp8(f[2] * inv),
                          clamp_fp8(f[3] * inv));
  q.y = e4m3_encode4<kHw>(clamp_fp8(f[4] * inv), clamp_fp8(f[5] * inv), clamp_fp8(f[6] * inv),
                          clamp_fp8(f[7] * inv));
  q.z = e4m3_encode4<kHw>(clamp_fp8(f[8] * inv), clamp_fp8(f[9] * inv),
                          clamp_fp8(f[10] * inv), clamp_fp8(f[11] * inv));
  q.w = e4m3_encode4<kHw>(clamp_fp8(f[12] * inv), clamp_fp8(f[13] * inv),
                          clamp_fp8(f[14] * inv), clamp_fp8(f[15] * inv));
  if ((v & 7) == 0) my_scales[v / 8] = scale;
  for (int32_t j = 0; j < k; ++j) {
    const int32_t s = slots[j];
    if (s >= 0) store_nt(recv + (int64_t)s * out_vec_per_row + v, q);
  }
}

// FP8: 16 channels per lane and step (two 16-byte loads of bf16, one 16-byte
// store of codes per valid row); 8 lanes make one 128-channel block.  `lanes`
// must be a multiple of 8 so that the 8 lanes of a block step together.  The
// block scales are left in my_scales for fp8_token_scales.
template <bool kHw, bool kPow2 = false>
__device__ __forceinline__ void fp8_token_codes(const u32x4* __restrict__ src, int32_t hidden,
                                                int32_t lt, int32_t lanes, const int32_t* slots,
                                                int32_t k, u32x4* __restrict__ recv,
                                                float* my_scales) {
  const int32_t out_vec_per_row = hidden / 16;  // 16-byte vectors of codes
  for (int32_t v = lt; v < out_vec_per_row; v += lanes)
    fp8_vector_codes<kHw, kPow2>(src[2 * v], src[2 * v + 1], v, slots, k, recv, out_vec_per_row,
                                 my_scales);
}

// After a block barrier: the token's lanes write its staged scales to each
// valid row, consecutive lanes on consecutive blocks, so every row's scales
// leave as one contiguous run.  Ordinary stores, so that partial cache lines
// shared with neighbouring rows can merge in the caches.
__device__ __forceinline__ void fp8_token_scales(int32_t hidden, int32_t lt, int32_t lanes,
                                                 const int32_t* slots, int32_t k,
                                                 const float* my_scales,
                                                 float* __restrict__ scales) {
  const int32_t blocks_per_row = hidden / kFp8Block;
  const int32_t n = k * blocks_per_row;
  for (int32_t i = lt; i < n; i += lanes) {
    const int32_t j = i / blocks_per_row;
    const int32_t b = i - j * blocks_per_row;
    const int32_t s = slots[j];
    if (s >= 0) scales[(int64_t)s * blocks_per_row + b] = my_scales[b];
  }
}

}  // namespace ep
