// ep_dispatch.hip -- MoE dispatch on gfx950: token rows -> expert-ordered
// receive rows, as a bf16 bit copy or as OCP FP8 E4M3 codes with one fp32
// scale per 128 channels.
//
// What it computes: every (token, k) pair with a receive row gets a copy of
// the token's hidden state ("DeepEP是什麼？…" (yololab.net), section
// "MoE為什麼需要All-to-all？", stage table, dispatch row), one row per pair
// ("DeepEP 编址服务深度对抗分析", section 五.2), optionally in FP8 with
// per-block scales (section "FP8與低精度通訊" of the first page).
//
// How: the work is HBM-bound (one read of x, k row writes per token), so the
// kernel is shaped for bandwidth, not arithmetic.  Lanes own contiguous
// 16-channel slices of one token.  The token is read once; for FP8 the block
// maximum is reduced over the 8 lanes of each 128-channel block with lane
// swizzles, the token is quantised once, and the same 16 code bytes are
// stored to every one of its k receive rows with one 16-byte non-temporal
// store per lane and row; the scales are gathered in LDS and written per row.
// Stores go straight to the final buffer: the pages note that skipping a
// staging copy saves HBM bandwidth ("DeepEP 编址服务深度对抗分析", section 五.1).
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

// Encoder used by dispatch: the gfx950 conversion instruction (OCP E4M3,
// round to nearest even); verified against the software encoder over every
// fp32 input of magnitude <= 448.
const bool kDispatchUsesHwCast = true;

struct TokenMap {
  int32_t lanes_per_token;   // lanes sharing one token (multiple of 8)
  int32_t tokens_per_block;  // tokens handled by one workgroup
};

__device__ __forceinline__ void token_of_thread(const TokenMap& m, int64_t& t, int32_t& lt) {
  if (m.tokens_per_block == 1) {
    t = blockIdx.x;
    lt = threadIdx.x;
  } else {
    t = (int64_t)blockIdx.x * m.tokens_per_block + threadIdx.x / m.lanes_per_token;
    lt = threadIdx.x % m.lanes_per_token;
  }
}

// bf16: every lane copies 8 channels (16 bytes) per step; receive rows are
// written once and never read back by this kernel, so they are stored with
// the non-temporal hint.
__global__ __launch_bounds__(1024) void dispatch_bf16_kernel(
    const u32x4* __restrict__ x, int64_t num_tokens, int32_t k, int32_t hidden, TokenMap m,
    const int32_t* __restrict__ slot_idx, u32x4* __restrict__ recv) {
  int64_t t;
  int32_t lt;
  token_of_thread(m, t, lt);
  if (t >= num_tokens) return;
  const int32_t vec_per_row = hidden / 8;
  const u32x4* src = x + t * vec_per_row;
  const int32_t* slots = slot_idx + t * k;
  for (int32_t v = lt; v < vec_per_row; v += m.lanes_per_token) {
    const u32x4 d = src[v];
    for (int32_t j = 0; j < k; ++j) {
      const int32_t s = slots[j];
      if (s >= 0) store_nt(recv + (int64_t)s * vec_per_row + v, d);
    }
  }
}

// Scales of one token fit in LDS: hidden <= EP_MAX_HIDDEN gives at most 512.
constexpr int kMaxScalesPerBlock = EP_MAX_HIDDEN / kFp8Block;

// FP8: every lane quantises 16 channels (two 16-byte loads of bf16, one
// 16-byte store of codes per receive row); 8 lanes make one 128-channel block.
// Codes go to the receive rows with non-temporal stores.  The block scales are
// staged in LDS and written afterwards row by row by consecutive lanes, so each
// receive row's scales leave as one contiguous run instead of 4-byte pieces
// from separate waves; they use ordinary stores so that partial cache lines
// shared by neighbouring rows can merge in the caches.
template <bool kHw>
__global__ __launch_bounds__(1024) void dispatch_fp8_kernel(
    const u32x4* __restrict__ x, int64_t num_tokens, int32_t k, int32_t hidden, TokenMap m,
    const int32_t* __restrict__ slot_idx, u32x4* __restrict__ recv, float* __restrict__ scales) {
  __shared__ float s_scale[kMaxScalesPerBlock];
  int64_t t;
  int32_t lt;
  token_of_thread(m, t, lt);
  const int32_t tok_in_block = m.tokens_per_block == 1 ? 0 : threadIdx.x / m.lanes_per_token;
  const int32_t in_vec_per_row = hidden / 8;    // 16-byte vectors of bf16
  const int32_t out_vec_per_row = hidden / 16;  // 16-byte vectors of codes
  const int32_t blocks_per_row = hidden / kFp8Block;
  float* my_scales = s_scale + tok_in_block * blocks_per_row;
  if (t < num_tokens) {  // whole 8-lane groups share t
    const u32x4* src = x + t * in_vec_per_row;
    const int32_t* slots = slot_idx + t * k;
    for (int32_t v = lt; v < out_vec_per_row; v += m.lanes_per_token) {
      const u32x4 lo = src[2 * v];
      const u32x4 hi = src[2 * v + 1];
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
      const float a = fmaxf(amax, kScaleFloor);
      const float scale = a / kFp8Max;  // correctly rounded fp32 divisions
      const float inv = kFp8Max / a;
      u32x4 q;
      q.x = e4m3_encode4<kHw>(clamp_fp8(f[0] * inv), clamp_fp8(f[1] * inv),
                              clamp_fp8(f[2] * inv), clamp_fp8(f[3] * inv));
      q.y = e4m3_encode4<kHw>(clamp_fp8(f[4] * inv), clamp_fp8(f[5] * inv),
                              clamp_fp8(f[6] * inv), clamp_fp8(f[7] * inv));
      q.z = e4m3_encode4<kHw>(clamp_fp8(f[8] * inv), clamp_fp8(f[9] * inv),
                              clamp_fp8(f[10] * inv), clamp_fp8(f[11] * inv));
      q.w = e4m3_encode4<kHw>(clamp_fp8(f[12] * inv), clamp_fp8(f[13] * inv),
                              clamp_fp8(f[14] * inv), clamp_fp8(f[15] * inv));
      if ((lt & 7) == 0) my_scales[v / 8] = scale;
      for (int32_t j = 0; j < k; ++j) {
        const int32_t s = slots[j];
        if (s >= 0) store_nt(recv + (int64_t)s * out_vec_per_row + v, q);
      }
    }
  }
  __syncthreads();
  // scales: the token's lanes walk its k rows, consecutive lanes on consecutive blocks
  if (t < num_tokens) {
    const int32_t* slots = slot_idx + t * k;
    const int32_t n = k * blocks_per_row;
    for (int32_t i = lt; i < n; i += m.lanes_per_token) {
      const int32_t j = i / blocks_per_row;
      const int32_t b = i - j * blocks_per_row;
      const int32_t s = slots[j];
      if (s >= 0) scales[(int64_t)s * blocks_per_row + b] = my_scales[b];
    }
  }
}

// Lanes per token: one lane per vector when that fits a workgroup (rounded up
// to whole waves), else a full 1024-lane workgroup looping over the row; rows
// shorter than a wave share a 256-lane workgroup with other tokens (at most 32
// tokens of fewer than 8 scale blocks each, so their scales fit the LDS array).
static TokenMap token_map(int32_t vecs_per_row) {
  TokenMap m;
  if (vecs_per_row >= 64) {
    m.lanes_per_token = vecs_per_row <= 1024 ? ((vecs_per_row + 63) / 64) * 64 : 1024;
    m.tokens_per_block = 1;
  } else {
    int32_t l = 8;
    while (l < vecs_per_row) l *= 2;
    m.lanes_per_token = l;
    m.tokens_per_block = 256 / l;
  }
  return m;
}

hipError_t launch_dispatch(const void* x, const ep_layout_t& L, int32_t hidden, bool fp8,
                           void* recv_x, float* recv_scales, hipStream_t stream) {
  const int64_t T = L.num_tokens;
  if (T == 0) return hipSuccess;
  const TokenMap m = token_map(fp8 ? hidden / 16 : hidden / 8);
  const int64_t blocks = (T + m.tokens_per_block - 1) / m.tokens_per_block;
  const int32_t threads = m.lanes_per_token * m.tokens_per_block;
  if (fp8) {
    if (kDispatchUsesHwCast)
      hipLaunchKernelGGL(dispatch_fp8_kernel<true>, dim3((unsigned)blocks), dim3(threads), 0,
                         stream, static_cast<const u32x4*>(x), T, L.num_topk, hidden, m,
                         L.slot_idx, static_cast<u32x4*>(recv_x), recv_scales);
    else
      hipLaunchKernelGGL(dispatch_fp8_kernel<false>, dim3((unsigned)blocks), dim3(threads), 0,
                         stream, static_cast<const u32x4*>(x), T, L.num_topk, hidden, m,
                         L.slot_idx, static_cast<u32x4*>(recv_x), recv_scales);
  } else {
    hipLaunchKernelGGL(dispatch_bf16_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       static_cast<const u32x4*>(x), T, L.num_topk, hidden, m, L.slot_idx,
                       static_cast<u32x4*>(recv_x));
  }
  return hipGetLastError();
}

}  // namespace ep
