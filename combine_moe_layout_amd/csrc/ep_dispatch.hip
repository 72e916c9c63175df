// ep_dispatch.hip -- MoE dispatch on gfx950: token rows -> expert-ordered
// receive rows, as a bf16 / fp16 bit copy, or as OCP FP8 E4M3 codes with one
// fp32 scale per 128 channels or one E8M0 scale per 32 channels (MXFP8).
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
#include "ep_dispatch_token.h"
#include "ep_internal.h"

namespace ep {

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
  bf16_token_copy(x + t * (hidden / 8), hidden, lt, m.lanes_per_token, slot_idx + t * k, k, recv);
}

// FP8: every lane quantises 16 channels (two 16-byte loads of bf16, one
// 16-byte store of codes per receive row); 8 lanes make one 128-channel block.
// Codes go to the receive rows with non-temporal stores.  The block scales are
// staged in LDS and written afterwards row by row by consecutive lanes, so each
// receive row's scales leave as one contiguous run instead of 4-byte pieces
// from separate waves; mn_rows > 0 selects the MN-major scale layout instead.
template <bool kHw, int kMode>
__global__ __launch_bounds__(1024) void dispatch_fp8_kernel(
    const u32x4* __restrict__ x, int64_t num_tokens, int32_t k, int32_t hidden, TokenMap m,
    const int32_t* __restrict__ slot_idx, u32x4* __restrict__ recv, uint32_t* __restrict__ scales,
    int64_t mn_rows) {
  __shared__ uint32_t s_scale[kMaxScalesPerBlock];
  int64_t t;
  int32_t lt;
  token_of_thread(m, t, lt);
  const int32_t tok_in_block = m.tokens_per_block == 1 ? 0 : threadIdx.x / m.lanes_per_token;
  uint32_t* my_scales = s_scale + tok_in_block * (hidden / kFp8Block);
  if (t < num_tokens)  // whole 8-lane groups share t
    fp8_token_codes<kHw, kMode>(x + t * (hidden / 8), hidden, lt, m.lanes_per_token,
                                slot_idx + t * k, k, recv, my_scales);
  __syncthreads();
  if (t < num_tokens)
    fp8_token_scales_any<kMode>(hidden, lt, m.lanes_per_token, slot_idx + t * k, k, my_scales,
                                mn_rows, scales);
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

hipError_t launch_dispatch(const void* x, const ep_layout_t& L, int32_t hidden, int32_t dtype,
                           void* recv_x, void* recv_scales, hipStream_t stream) {
  const int64_t T = L.num_tokens;
  if (T == 0) return hipSuccess;
  const int64_t mn_rows = dtype_scales_mn(dtype) ? L.num_recv_rows : 0;
  dtype = dtype_base(dtype);
  const bool fp8 = dtype_is_fp8(dtype);
  uint32_t* sw = static_cast<uint32_t*>(recv_scales);
  const TokenMap m = token_map(fp8 ? hidden / 16 : hidden / 8);
  const dim3 grid((unsigned)((T + m.tokens_per_block - 1) / m.tokens_per_block));
  const dim3 block(m.lanes_per_token * m.tokens_per_block);
  const u32x4* xv = static_cast<const u32x4*>(x);
  u32x4* rv = static_cast<u32x4*>(recv_x);
  if (dtype == EP_FP8_E4M3)
    hipLaunchKernelGGL((dispatch_fp8_kernel<kDispatchUsesHwCast, kScaleF32>), grid, block, 0,
                       stream, xv, T, L.num_topk, hidden, m, L.slot_idx, rv, sw, mn_rows);
  else if (dtype == EP_FP8_E4M3_POW2)
    hipLaunchKernelGGL((dispatch_fp8_kernel<kDispatchUsesHwCast, kScalePow2>), grid, block, 0,
                       stream, xv, T, L.num_topk, hidden, m, L.slot_idx, rv, sw, mn_rows);
  else if (dtype == EP_MXFP8_E4M3)
    hipLaunchKernelGGL((dispatch_fp8_kernel<kDispatchUsesHwCast, kScaleMx>), grid, block, 0,
                       stream, xv, T, L.num_topk, hidden, m, L.slot_idx, rv, sw, mn_rows);
  else  // EP_BF16 and EP_F16: a bit copy of 2-byte elements
    hipLaunchKernelGGL(dispatch_bf16_kernel, grid, block, 0, stream, xv, T, L.num_topk, hidden, m,
                       L.slot_idx, rv);
  return hipGetLastError();
}

}  // namespace ep
