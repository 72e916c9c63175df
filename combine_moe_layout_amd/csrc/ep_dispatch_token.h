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

// Scales of one token fit in LDS: hidden <= EP_MAX_HIDDEN gives at most 512
// scale words (one 4-byte word per 128 channels in every scale format).
constexpr int kMaxScalesPerBlock = EP_MAX_HIDDEN / kFp8Block;

// Scale formats of FP8 dispatch.  kScaleF32 / kScalePow2: one fp32 scale per
// 128 channels.  kScaleMx: MXFP8, one E8M0 byte per 32 channels, i.e. four
// bytes (one word) per 128 channels, so the scale rows have the same size and
// the same word-wise store pattern in every format.
enum ScaleMode : int { kScaleF32 = 0, kScalePow2 = 1, kScaleMx = 2 };

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

// MXFP8 shared exponent of a 32-channel block (the OCP Microscaling
// conversion): se = floor(log2(amax)) - 8, where 8 is the exponent of E4M3's
// largest normal (448 = 1.75 * 2^8), clamped to [-127, 127].  For amax >= 0
// floor(log2(amax)) is the biased exponent field minus 127; a zero or fp32
// subnormal maximum (field 0) lies below 2^-126 and clamps to -127, and the
// largest finite amax gives 119, so only the lower clamp can act.  Returns the
// E8M0 byte se + 127 and sets inv = 2^-se (a normal fp32 power of two).
__device__ __forceinline__ uint32_t mx_block_scale(float amax, float& inv) {
  const int32_t field = (int32_t)(__float_as_uint(amax) >> 23);
  const int32_t se = field == 0 ? -127 : (field - 135 < -127 ? -127 : field - 135);
  inv = __uint_as_float((uint32_t)(127 - se) << 23);
  return (uint32_t)(se + 127);
}

// FP8 codes of one 16-channel slice (vector v of the code row: bf16 vectors
// 2v and 2v+1 given in lo / hi), stored to every valid row; the lanes of one
// scale block must call it together (their maximum is reduced with lane
// swizzles: 8 lanes per 128-channel block, 2 lanes per 32-channel MX block).
// The block's scale word goes to word v / 8 of my_scales (MX: the block's
// E8M0 byte to byte v / 2).
// E4M3 codes of 16 values scaled by inv and clamped to +-448, four bytes per word.
template <bool kHw>
__device__ __forceinline__ void fp8_encode16(const float (&f)[16], float inv, u32x4& q) {
  q.x = e4m3_encode4<kHw>(clamp_fp8(f[0] * inv), clamp_fp8(f[1] * inv), clamp_fp8(f[2] * inv),
                          clamp_fp8(f[3] * inv));
  q.y = e4m3_encode4<kHw>(clamp_fp8(f[4] * inv), clamp_fp8(f[5] * inv), clamp_fp8(f[6] * inv),
                          clamp_fp8(f[7] * inv));
  q.z = e4m3_encode4<kHw>(clamp_fp8(f[8] * inv), clamp_fp8(f[9] * inv),
                          clamp_fp8(f[10] * inv), clamp_fp8(f[11] * inv));
  q.w = e4m3_encode4<kHw>(clamp_fp8(f[12] * inv), clamp_fp8(f[13] * inv),
                          clamp_fp8(f[14] * inv), clamp_fp8(f[15] * inv));
}

// Codes of a 128-channel block that holds a NaN or an infinity (fp32 scales):
// the block maximum ignores NaN, as in the scale's definition, so a block with
// an infinity gets scale = inf and inv = 0; finite values then encode as +-0
// and every product that is NaN (a NaN input, or inf * 0) encodes as 0x7F.
// Rare, so it is kept apart from the common path.
template <bool kHw>
__device__ __forceinline__ void fp8_nonfinite_block(const float (&f)[16], int32_t v, u32x4& q,
                                                 uint32_t* my_scales) {
  // Comparisons, not fmaxf: IEEE maxNum turns a signalling NaN (bf16 0x7F81,
  // say) into a quiet NaN result instead of skipping it, while a comparison
  // with any NaN is false, so NaN of either kind is skipped.
  const auto larger = [](float a, float b) { return b > a ? b : a; };
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = larger(amax, fabsf(f[i]));
  amax = larger(amax, __shfl_xor(amax, 1));
  amax = larger(amax, __shfl_xor(amax, 2));
  amax = larger(amax, __shfl_xor(amax, 4));
  float scale, inv;
  fp8_block_scale<false>(fmaxf(amax, kScaleFloor), scale, inv);
  if ((v & 7) == 0) my_scales[v / 8] = __float_as_uint(scale);
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float p[4];
    uint32_t nan_bytes = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      p[b] = f[4 * i + b] * inv;
      if (p[b] != p[b]) nan_bytes |= 0xFFu << (8 * b);
    }
    const uint32_t c = e4m3_encode4<kHw>(clamp_fp8(p[0]), clamp_fp8(p[1]), clamp_fp8(p[2]),
                                         clamp_fp8(p[3]));
    w[i] = (c & ~nan_bytes) | (0x7F7F7F7Fu & nan_bytes);
  }
  q = u32x4{w[0], w[1], w[2], w[3]};
}

// FP8 codes of one 16-channel slice (vector v of the code row: bf16 vectors
// 2v and 2v+1 given in lo / hi), stored to every valid row; the lanes of one
// scale block must call it together (their maximum is reduced with lane
// swizzles: 8 lanes per 128-channel block, 2 lanes per 32-channel MX block).
// The block's scale word goes to word v / 8 of my_scales (MX: the block's
// E8M0 byte to byte v / 2).
//
// fp32 scales: the block maximum is taken with the NaN-propagating maximum
// (v_maximum3_f32, as cheap as the ordinary one), so one comparison of the
// finished maximum tells whether the block holds a NaN or an infinity; such
// a block takes fp8_nonfinite_block.  In the common path every product lies
// within +-448 * (1 + 2^-23) and the clamp only trims rounding.  (Non-finite
// inputs are outside the power-of-two and MXFP8 formats' definitions.)
template <bool kHw, int kMode = kScaleF32>
__device__ __forceinline__ void fp8_vector_codes(const u32x4& lo, const u32x4& hi, int32_t v,
                                                 const int32_t* slots, int32_t k,
                                                 u32x4* __restrict__ recv,
                                                 int32_t out_vec_per_row, uint32_t* my_scales) {
  float f[16] = {bf16_lo(lo.x), bf16_hi(lo.x), bf16_lo(lo.y), bf16_hi(lo.y),
                 bf16_lo(lo.z), bf16_hi(lo.z), bf16_lo(lo.w), bf16_hi(lo.w),
                 bf16_lo(hi.x), bf16_hi(hi.x), bf16_lo(hi.y), bf16_hi(hi.y),
                 bf16_lo(hi.z), bf16_hi(hi.z), bf16_lo(hi.w), bf16_hi(hi.w)};
  u32x4 q;
  if constexpr (kMode == kScaleF32) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = __builtin_elementwise_maximum(amax, fabsf(f[i]));
    amax = __builtin_elementwise_maximum(amax, __shfl_xor(amax, 1));
    amax = __builtin_elementwise_maximum(amax, __shfl_xor(amax, 2));
    amax = __builtin_elementwise_maximum(amax, __shfl_xor(amax, 4));
    if (!(amax <= 3.40282347e38f)) {  // NaN or infinity somewhere in the block
      fp8_nonfinite_block<kHw>(f, v, q, my_scales);
    } else {
      float scale, inv;
      fp8_block_scale<false>(fmaxf(amax, kScaleFloor), scale, inv);
      if ((v & 7) == 0) my_scales[v / 8] = __float_as_uint(scale);
      fp8_encode16<kHw>(f, inv, q);
    }
  } else {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    float inv;
    if constexpr (kMode == kScaleMx) {
      const uint32_t byte = mx_block_scale(amax, inv);
      if ((v & 1) == 0) reinterpret_cast<uint8_t*>(my_scales)[v / 2] = (uint8_t)byte;
    } else {
      amax = fmaxf(amax, __shfl_xor(amax, 2));
      amax = fmaxf(amax, __shfl_xor(amax, 4));
      float scale;
      fp8_block_scale<true>(fmaxf(amax, kScaleFloor), scale, inv);
      if ((v & 7) == 0) my_scales[v / 8] = __float_as_uint(scale);
    }
    fp8_encode16<kHw>(f, inv, q);
  }
  for (int32_t j = 0; j < k; ++j) {
    const int32_t s = slots[j];
    if (s >= 0) store_nt(recv + (int64_t)s * out_vec_per_row + v, q);
  }
}

// FP8: 16 channels per lane and step (two 16-byte loads of bf16, one 16-byte
// store of codes per valid row); 8 lanes make one 128-channel block.  `lanes`
// must be a multiple of 8 so that the 8 lanes of a block step together.  The
// block scales are left in my_scales for fp8_token_scales.
template <bool kHw, int kMode = kScaleF32>
__device__ __forceinline__ void fp8_token_codes(const u32x4* __restrict__ src, int32_t hidden,
                                                int32_t lt, int32_t lanes, const int32_t* slots,
                                                int32_t k, u32x4* __restrict__ recv,
                                                uint32_t* my_scales) {
  const int32_t out_vec_per_row = hidden / 16;  // 16-byte vectors of codes
  for (int32_t v = lt; v < out_vec_per_row; v += lanes)
    fp8_vector_codes<kHw, kMode>(src[2 * v], src[2 * v + 1], v, slots, k, recv, out_vec_per_row,
                                 my_scales);
}

// After a block barrier: the token's lanes write its staged scale words to
// each valid row, consecutive lanes on consecutive words, so every row's
// scales leave as one contiguous run.  Ordinary stores, so that partial cache
// lines shared with neighbouring rows can merge in the caches.  The words are
// copied as integers (a word of E8M0 bytes may look like a NaN as an fp32).
__device__ __forceinline__ void fp8_token_scales(int32_t hidden, int32_t lt, int32_t lanes,
                                                 const int32_t* slots, int32_t k,
                                                 const uint32_t* my_scales,
                                                 uint32_t* __restrict__ scales) {
  const int32_t blocks_per_row = hidden / kFp8Block;
  const int32_t n = k * blocks_per_row;
  for (int32_t i = lt; i < n; i += lanes) {
    const int32_t j = i / blocks_per_row;
    const int32_t b = i - j * blocks_per_row;
    const int32_t s = slots[j];
    if (s >= 0) scales[(int64_t)s * blocks_per_row + b] = my_scales[b];
  }
}

// The MN-major (transposed) scale layout: entry c of receive row s goes to
// c * rows + s, so one block column's entries for consecutive rows are
// contiguous.  Entries are the 4-byte scale words (one per 128 channels) or,
// with kBytes, the MXFP8 E8M0 bytes (one per 32 channels).  Ordinary stores:
// the entries of neighbouring rows share cache lines and merge in the caches.
template <bool kBytes>
__device__ __forceinline__ void fp8_token_scales_mn(int32_t hidden, int32_t lt, int32_t lanes,
                                                    const int32_t* slots, int32_t k,
                                                    const uint32_t* my_scales, int64_t rows,
                                                    void* __restrict__ scales) {
  const int32_t per_row = kBytes ? hidden / 32 : hidden / kFp8Block;
  const int32_t n = k * per_row;
  for (int32_t i = lt; i < n; i += lanes) {
    const int32_t j = i / per_row;
    const int32_t c = i - j * per_row;
    const int32_t s = slots[j];
    if (s < 0) continue;
    const int64_t at = (int64_t)c * rows + s;
    if constexpr (kBytes)
      static_cast<uint8_t*>(scales)[at] = reinterpret_cast<const uint8_t*>(my_scales)[c];
    else
      static_cast<uint32_t*>(scales)[at] = my_scales[c];
  }
}

// Writes the staged scales of one token in the layout the caller chose:
// row-major when mn_rows == 0, else MN-major over mn_rows receive rows.
template <int kMode>
__device__ __forceinline__ void fp8_token_scales_any(int32_t hidden, int32_t lt, int32_t lanes,
                                                     const int32_t* slots, int32_t k,
                                                     const uint32_t* my_scales, int64_t mn_rows,
                                                     uint32_t* __restrict__ scales) {
  if (mn_rows > 0)
    fp8_token_scales_mn<kMode == kScaleMx>(hidden, lt, lanes, slots, k, my_scales, mn_rows, scales);
  else
    fp8_token_scales(hidden, lt, lanes, slots, k, my_scales, scales);
}

}  // namespace ep
