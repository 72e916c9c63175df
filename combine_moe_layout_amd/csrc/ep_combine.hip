// ep_combine.hip -- MoE combine on gfx950: expert outputs back to token order,
// reduced with the top-k routing weights.
//
// What it computes: out[t] = bf16(sum_j w[t,j] * y[slot[t,j]]) over the pairs
// that have a receive row, summed in fp32 in j order, rounded to nearest-even
// ("DeepEP是什麼？…" (yololab.net), section "MoE為什麼需要All-to-all？",
// stage table, combine row: back to the original token order, with a
// reduction; BF16 combine as in the DeepEP v2 release notes (donniechu.com),
// section "Số liệu kỹ thuật").
//
// How: HBM-bound (k row reads and one row write per token).  Lanes own
// contiguous 16-channel slices of one token; the k rows of a slice are loaded
// before any arithmetic (the top-k is a template parameter for the common
// sizes, so all 2k 16-byte loads are in flight together), then accumulated
// with fp32 fma.  A pair without a receive row is loaded from row 0 and
// discarded with a select, never multiplied, so unwritten rows (padded mode)
// cannot leak NaNs into the sum.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

struct CombineMap {
  int32_t lanes_per_token;
  int32_t tokens_per_block;
};

__device__ __forceinline__ void unpack16(const u32x4& a, const u32x4& b, float* f) {
  f[0] = bf16_lo(a.x); f[1] = bf16_hi(a.x); f[2] = bf16_lo(a.y); f[3] = bf16_hi(a.y);
  f[4] = bf16_lo(a.z); f[5] = bf16_hi(a.z); f[6] = bf16_lo(a.w); f[7] = bf16_hi(a.w);
  f[8] = bf16_lo(b.x); f[9] = bf16_hi(b.x); f[10] = bf16_lo(b.y); f[11] = bf16_hi(b.y);
  f[12] = bf16_lo(b.z); f[13] = bf16_hi(b.z); f[14] = bf16_lo(b.w); f[15] = bf16_hi(b.w);
}

// K > 0: compile-time top-k.  K == 0: any top-k, one row at a time.
template <int K>
__global__ __launch_bounds__(1024) void combine_kernel(
    const u32x4* __restrict__ y, const float* __restrict__ w,
    const int32_t* __restrict__ slot_idx, int64_t num_tokens, int32_t k, int32_t hidden,
    CombineMap m, u32x4* __restrict__ out) {
  int64_t t;
  int32_t lt;
  if (m.tokens_per_block == 1) {
    t = blockIdx.x;
    lt = threadIdx.x;
  } else {
    t = (int64_t)blockIdx.x * m.tokens_per_block + threadIdx.x / m.lanes_per_token;
    lt = threadIdx.x % m.lanes_per_token;
  }
  if (t >= num_tokens) return;
  const int32_t vec_per_row = hidden / 8;   // 16-byte vectors per bf16 row
  const int32_t pairs_per_row = hidden / 16;  // 16-channel slices per row
  const int32_t kk = K > 0 ? K : k;
  const int32_t* slots = slot_idx + t * kk;
  const float* wt = w + t * kk;
  u32x4* dst = out + t * vec_per_row;

  if constexpr (K > 0) {
    int32_t s[K];
    float ww[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      s[j] = slots[j];
      ww[j] = wt[j];
    }
    for (int32_t v = lt; v < pairs_per_row; v += m.lanes_per_token) {
      u32x4 a[K], b[K];
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const int64_t row = s[j] >= 0 ? s[j] : 0;
        const u32x4* src = y + row * vec_per_row + 2 * v;
        a[j] = src[0];
        b[j] = src[1];
      }
      float acc[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
#pragma unroll
      for (int j = 0; j < K; ++j) {
        float f[16];
        unpack16(a[j], b[j], f);
        const bool valid = s[j] >= 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = valid ? fmaf(ww[j], f[i], acc[i]) : acc[i];
      }
      u32x4 o0, o1;
      o0.x = pack_bf16x2(acc[0], acc[1]);
      o0.y = pack_bf16x2(acc[2], acc[3]);
      o0.z = pack_bf16x2(acc[4], acc[5]);
      o0.w = pack_bf16x2(acc[6], acc[7]);
      o1.x = pack_bf16x2(acc[8], acc[9]);
      o1.y = pack_bf16x2(acc[10], acc[11]);
      o1.z = pack_bf16x2(acc[12], acc[13]);
      o1.w = pack_bf16x2(acc[14], acc[15]);
      dst[2 * v] = o0;
      dst[2 * v + 1] = o1;
    }
  } else {
    for (int32_t v = lt; v < pairs_per_row; v += m.lanes_per_token) {
      float acc[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
      for (int32_t j = 0; j < k; ++j) {
        const int32_t sj = slots[j];
        if (sj < 0) continue;
        const u32x4* src = y + (int64_t)sj * vec_per_row + 2 * v;
        float f[16];
        unpack16(src[0], src[1], f);
        const float wj = wt[j];
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = fmaf(wj, f[i], acc[i]);
      }
      u32x4 o0, o1;
      o0.x = pack_bf16x2(acc[0], acc[1]);
      o0.y = pack_bf16x2(acc[2], acc[3]);
      o0.z = pack_bf16x2(acc[4], acc[5]);
      o0.w = pack_bf16x2(acc[6], acc[7]);
      o1.x = pack_bf16x2(acc[8], acc[9]);
      o1.y = pack_bf16x2(acc[10], acc[11]);
      o1.z = pack_bf16x2(acc[12], acc[13]);
      o1.w = pack_bf16x2(acc[14], acc[15]);
      dst[2 * v] = o0;
      dst[2 * v + 1] = o1;
    }
  }
}

// Rows of 8 channels that are not a multiple of 16: the same sum, 8 channels
// (one 16-byte vector) per lane and step.
__global__ __launch_bounds__(1024) void combine_vec8_kernel(
    const u32x4* __restrict__ y, const float* __restrict__ w,
    const int32_t* __restrict__ slot_idx, int64_t num_tokens, int32_t k, int32_t hidden,
    CombineMap m, u32x4* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * m.tokens_per_block + threadIdx.x / m.lanes_per_token;
  const int32_t lt = threadIdx.x % m.lanes_per_token;
  if (t >= num_tokens) return;
  const int32_t vec_per_row = hidden / 8;
  for (int32_t v = lt; v < vec_per_row; v += m.lanes_per_token) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int32_t j = 0; j < k; ++j) {
      const int32_t sj = slot_idx[t * k + j];
      if (sj < 0) continue;
      const u32x4 d = y[(int64_t)sj * vec_per_row + v];
      const float wj = w[t * k + j];
      acc[0] = fmaf(wj, bf16_lo(d.x), acc[0]);
      acc[1] = fmaf(wj, bf16_hi(d.x), acc[1]);
      acc[2] = fmaf(wj, bf16_lo(d.y), acc[2]);
      acc[3] = fmaf(wj, bf16_hi(d.y), acc[3]);
      acc[4] = fmaf(wj, bf16_lo(d.z), acc[4]);
      acc[5] = fmaf(wj, bf16_hi(d.z), acc[5]);
      acc[6] = fmaf(wj, bf16_lo(d.w), acc[6]);
      acc[7] = fmaf(wj, bf16_hi(d.w), acc[7]);
    }
    u32x4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    out[t * vec_per_row + v] = o;
  }
}

static CombineMap combine_map(int32_t lanes_needed) {
  CombineMap m;
  if (lanes_needed >= 64) {
    m.lanes_per_token = lanes_needed <= 1024 ? ((lanes_needed + 63) / 64) * 64 : 1024;
    m.tokens_per_block = 1;
  } else {
    int32_t l = 1;
    while (l < lanes_needed) l *= 2;
    m.lanes_per_token = l;
    m.tokens_per_block = 256 / l;
  }
  return m;
}

template <int K>
static void launch_k(dim3 grid, dim3 block, hipStream_t stream, const void* y, const float* w,
                     const ep_layout_t& L, int32_t hidden, CombineMap m, void* out) {
  hipLaunchKernelGGL(combine_kernel<K>, grid, block, 0, stream, static_cast<const u32x4*>(y), w,
                     L.slot_idx, L.num_tokens, L.num_topk, hidden, m, static_cast<u32x4*>(out));
}

hipError_t launch_combine(const void* y, const float* w, const ep_layout_t& L, int32_t hidden,
                          void* out, hipStream_t stream) {
  const int64_t T = L.num_tokens;
  if (T == 0) return hipSuccess;
  if (hidden % 16 != 0) {
    const CombineMap m = combine_map(hidden / 8);
    const int64_t blocks = (T + m.tokens_per_block - 1) / m.tokens_per_block;
    hipLaunchKernelGGL(combine_vec8_kernel, dim3((unsigned)blocks),
                       dim3(m.lanes_per_token * m.tokens_per_block), 0, stream,
                       static_cast<const u32x4*>(y), w, L.slot_idx, T, L.num_topk, hidden, m,
                       static_cast<u32x4*>(out));
    return hipGetLastError();
  }
  const CombineMap m = combine_map(hidden / 16);
  const dim3 grid((unsigned)((T + m.tokens_per_block - 1) / m.tokens_per_block));
  const dim3 block(m.lanes_per_token * m.tokens_per_block);
  switch (L.num_topk) {
    case 1: launch_k<1>(grid, block, stream, y, w, L, hidden, m, out); break;
    case 2: launch_k<2>(grid, block, stream, y, w, L, hidden, m, out); break;
    case 3: launch_k<3>(grid, block, stream, y, w, L, hidden, m, out); break;
    case 4: launch_k<4>(grid, block, stream, y, w, L, hidden, m, out); break;
    case 5: launch_k<5>(grid, block, stream, y, w, L, hidden, m, out); break;
    case 6: launch_k<6>(grid, block, stream, y, w, L, hidden, m, out); break;
    case 7: launch_k<7>(grid, block, stream, y, w, L, hidden, m, out); break;
    case 8: launch_k<8>(grid, block, stream, y, w, L, hidden, m, out); break;
    default: launch_k<0>(grid, block, stream, y, w, L, hidden, m, out); break;
  }
  return hipGetLastError();
}

}  // namespace ep
