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
// The same kernel, by template flags, also serves fp16 rows and output
// (ep_combine_f16) and the unit-weight group combine of the per-group dedup
// variant (ep_combine_groups); the second half of this file is the combine of
// FP8 expert outputs (ep_combine_fp8).
//
// How: HBM-bound (k row reads and one row write per token, each read once).
// One workgroup per token by default, one lane per 16-byte vector (8
// channels) of the row, so every wave instruction covers 1 KiB of one row and
// the rows can be read with the non-temporal hint.  Short rows share a
// workgroup (rows shorter than a wave; at prefill size, rows of 128 to 512
// lanes), and a token's row is split over several workgroups in decode-sized
// batches and, for FP8 rows wider than four waves, at prefill size.
// The k rows of a lane are loaded before any arithmetic (the top-k is a
// template parameter for the common sizes, so all k loads are in flight
// together), then accumulated with fp32 fma.  A pair without a receive row is
// loaded from row 0 and discarded with a select, never multiplied, so
// unwritten rows (padded mode) cannot leak NaNs; the group combine skips such
// loads instead.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

struct CombineMap {
  int32_t lanes_per_token;   // lanes of one workgroup given to a token
  int32_t tokens_per_block;
  int32_t slices;            // workgroups per token (1 unless one token per workgroup)
};


// Rows hold 2-byte elements: bf16, or IEEE fp16 when kF16 (decoded exactly
// by the conversion instruction; results rounded to nearest-even by it, with
// fp16 subnormals kept and overflow to infinity).
template <bool kF16>
__device__ __forceinline__ float elem_lo(uint32_t w) {
  if constexpr (kF16) return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
  else return bf16_lo(w);
}

template <bool kF16>
__device__ __forceinline__ float elem_hi(uint32_t w) {
  if constexpr (kF16) return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  else return bf16_hi(w);
}

template <bool kF16>
__device__ __forceinline__ uint32_t pack_elem2(float a, float b) {
  if constexpr (kF16)
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
  else
    return pack_bf16x2(a, b);
}

template <bool kF16 = false>
__device__ __forceinline__ void accumulate8(float* acc, const u32x4& d, float w, bool valid) {
  const float f[8] = {elem_lo<kF16>(d.x), elem_hi<kF16>(d.x), elem_lo<kF16>(d.y),
                      elem_hi<kF16>(d.y), elem_lo<kF16>(d.z), elem_hi<kF16>(d.z),
                      elem_lo<kF16>(d.w), elem_hi<kF16>(d.w)};
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = valid ? fmaf(w, f[i], acc[i]) : acc[i];
}

template <bool kF16 = false>
__device__ __forceinline__ u32x4 pack8(const float* acc) {
  return u32x4{pack_elem2<kF16>(acc[0], acc[1]), pack_elem2<kF16>(acc[2], acc[3]),
               pack_elem2<kF16>(acc[4], acc[5]), pack_elem2<kF16>(acc[6], acc[7])};
}

// Token and lane of this thread.  kWhole: one token per workgroup (or per
// m.slices consecutive workgroups, each taking every slices-th run of
// lanes_per_token vectors), so the token index is uniform and its slots and
// weights come in through scalar loads.
template <bool kWhole>
__device__ __forceinline__ bool combine_token(const CombineMap& m, int64_t num_tokens, int64_t& t,
                                              int32_t& lt) {
  if constexpr (kWhole) {
    t = blockIdx.x / m.slices;
    lt = (int32_t)(blockIdx.x % m.slices) * m.lanes_per_token + threadIdx.x;
  } else {
    t = (int64_t)blockIdx.x * m.tokens_per_block + threadIdx.x / m.lanes_per_token;
    lt = threadIdx.x % m.lanes_per_token;
  }
  return t < num_tokens;
}

// K > 0: compile-time top-k.  K == 0: any top-k, one row at a time.
// kUnit: every weight is 1 and w is not read (the group combine of the dedup
// variant, whose rows arrive already weighted).  kF16: fp16 rows and output.
// kWhole: one token per workgroup, its slots and weights through scalar loads.
template <int K, bool kUnit, bool kF16 = false, bool kWhole = false>
__global__ __launch_bounds__(1024) void combine_kernel(
    const u32x4* __restrict__ y, const float* __restrict__ w,
    const int32_t* __restrict__ slot_idx, int64_t num_tokens, int32_t k, int32_t hidden,
    CombineMap m, u32x4* __restrict__ out) {
  int64_t t;
  int32_t lt;
  if (!combine_token<kWhole>(m, num_tokens, t, lt)) return;
  const int32_t vec_per_row = hidden / 8;
  const int32_t stride = m.lanes_per_token * m.slices;
  const int32_t kk = K > 0 ? K : k;
  const int32_t* slots = slot_idx + t * kk;
  const float* wt = kUnit ? nullptr : w + t * kk;
  u32x4* dst = out + t * vec_per_row;

  if constexpr (K > 0) {
    int32_t s[K];
    float ww[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      s[j] = slots[j];
      ww[j] = kUnit ? 1.0f : wt[j];
    }
    for (int32_t v = lt; v < vec_per_row; v += stride) {
      u32x4 d[K];
#pragma unroll
      for (int j = 0; j < K; ++j) {
        if constexpr (kUnit) {
          // group rows: a token's entries are its rows, then padding; with
          // many padded entries (skewed routing) loading only the real rows
          // saves most of the row-0 loads
          d[j] = u32x4{0u, 0u, 0u, 0u};
          if (s[j] >= 0) d[j] = load_nt(y + (int64_t)s[j] * vec_per_row + v);
        } else {
          const int64_t row = s[j] >= 0 ? s[j] : 0;
          d[j] = load_nt(y + row * vec_per_row + v);
        }
      }
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < K; ++j) accumulate8<kF16>(acc, d[j], ww[j], s[j] >= 0);
      store_nt(dst + v, pack8<kF16>(acc));
    }
  } else {
    for (int32_t v = lt; v < vec_per_row; v += stride) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int32_t j = 0; j < k; ++j) {
        const int32_t sj = slots[j];
        if (sj < 0) continue;
        accumulate8<kF16>(acc, load_nt(y + (int64_t)sj * vec_per_row + v), kUnit ? 1.0f : wt[j],
                          true);
      }
      store_nt(dst + v, pack8<kF16>(acc));
    }
  }
}

// One lane per 16-byte vector when the row fits a workgroup (rounded up to
// whole waves), else 1024 lanes looping over the row; rows shorter than a wave
// share a 256-lane workgroup with other tokens.
static CombineMap combine_map(int32_t vecs_per_row) {
  CombineMap m;
  m.slices = 1;
  if (vecs_per_row >= 64) {
    m.lanes_per_token = vecs_per_row <= 1024 ? ((vecs_per_row + 63) / 64) * 64 : 1024;
    m.tokens_per_block = 1;
  } else {
    int32_t l = 1;
    while (l < vecs_per_row) l *= 2;
    m.lanes_per_token = l;
    m.tokens_per_block = 256 / l;
  }
  return m;
}

// Decode-sized batches (one token per workgroup, at most kDecodeCombinePairs pairs)
// leave most of the chip idle: each token is spread over up to 8 workgroups,
// each taking at least one wave of vectors, so that about one workgroup runs
// per CU and all CUs share the row traffic.  Measured at hidden 7168, top-8,
// with the calls replayed from a HIP graph: bf16 5.0 -> 4.2 us at 128 tokens
// and 4.1 -> 3.0 us at 32; FP8 4.6 -> 3.8 and 3.9 -> 3.0 us.  At 256 tokens
// (already one per CU) splitting gains nothing.
static void split_tokens(int32_t vecs, int64_t T, CombineMap& m, dim3& grid, dim3& block) {
  int64_t S = kChipCUs / T;
  if (S > 8) S = 8;
  if (S > vecs / 64) S = vecs / 64;
  if (S <= 1) return;
  int32_t lanes = (((vecs + S - 1) / S + 63) / 64) * 64;
  if (lanes > 1024) lanes = 1024;
  m.lanes_per_token = lanes;
  m.slices = (int32_t)S;
  grid = dim3((unsigned)(T * S));
  block = dim3((unsigned)lanes);
}

// Large batches take the general token mapping (which also covers one token
// per workgroup): slots and weights then arrive as per-lane vector loads,
// about 3% faster there than the scalar loads of the uniform-token form (179
// vs 185 us at 8192 tokens x 7168, top-8).  Decode-sized batches (at most
// kDecodeCombinePairs pairs, one token per workgroup) are latency-bound, and there
// the scalar loads win (6.7 vs 7.2 us per call at 128 tokens, top-8).
template <int K, bool kUnit, bool kF16>
static void launch_k(dim3 grid, dim3 block, hipStream_t stream, const void* y, const float* w,
                     const ep_layout_t& L, int32_t hidden, CombineMap m, void* out) {
  const bool whole = m.tokens_per_block == 1 &&
                     L.num_tokens * (int64_t)L.num_topk <= (int64_t)kDecodeCombinePairs;
  if (whole) {
    split_tokens(hidden / 8, L.num_tokens, m, grid, block);
    hipLaunchKernelGGL((combine_kernel<K, kUnit, kF16, true>), grid, block, 0, stream,
                       static_cast<const u32x4*>(y), w, L.slot_idx, L.num_tokens, L.num_topk,
                       hidden, m, static_cast<u32x4*>(out));
  } else
    hipLaunchKernelGGL((combine_kernel<K, kUnit, kF16>), grid, block, 0, stream,
                       static_cast<const u32x4*>(y), w, L.slot_idx, L.num_tokens, L.num_topk,
                       hidden, m, static_cast<u32x4*>(out));
}

// Prefill-sized batches whose rows take a power-of-two number of lanes up to
// 512 fill 1024-lane workgroups with 1024 / lanes tokens: fewer, larger
// workgroups for the same lanes.  Measured on MI355X (bf16 rows, random
// routing, one combine per event pair): hidden 4096, top-6, 65,536 tokens
// 647-649 -> 624-631 us (654 -> 623 us inside the layout/dispatch/combine
// step); hidden 4096, top-8, 16,384 tokens 206-208 -> 204 us; hidden 2048,
// 131,072 tokens 851 -> 831 us; hidden 1024, 262,144 tokens 832-844 -> 829-831
// us.  Partly filled workgroups (2 tokens of 256 lanes, 2 or 4 of 128)
// measured slower than one token.  The FP8 combine keeps a uniform token per
// workgroup (its scalar slot and weight loads need one) and splits wide rows
// over several workgroups instead (split_prefill_rows).
static void pack_prefill_tokens(const ep_layout_t& L, CombineMap& m) {
  if (m.tokens_per_block == 1 && m.slices == 1 &&
      L.num_tokens * (int64_t)L.num_topk > (int64_t)kDecodeCombinePairs &&
      m.lanes_per_token <= 512 && 1024 % m.lanes_per_token == 0)
    m.tokens_per_block = 1024 / m.lanes_per_token;
}

template <bool kUnit, bool kF16 = false>
static hipError_t launch_combine_weights(const void* y, const float* w, const ep_layout_t& L,
                                         int32_t hidden, void* out, hipStream_t stream) {
  const int64_t T = L.num_tokens;
  if (T == 0) return hipSuccess;
  CombineMap m = combine_map(hidden / 8);
  pack_prefill_tokens(L, m);
  const dim3 grid((unsigned)((T + m.tokens_per_block - 1) / m.tokens_per_block));
  const dim3 block(m.lanes_per_token * m.tokens_per_block);
  switch (L.num_topk) {
    case 1: launch_k<1, kUnit, kF16>(grid, block, stream, y, w, L, hidden, m, out); break;
    case 2: launch_k<2, kUnit, kF16>(grid, block, stream, y, w, L, hidden, m, out); break;
    case 3: launch_k<3, kUnit, kF16>(grid, block, stream, y, w, L, hidden, m, out); break;
    case 4: launch_k<4, kUnit, kF16>(grid, block, stream, y, w, L, hidden, m, out); break;
    case 5: launch_k<5, kUnit, kF16>(grid, block, stream, y, w, L, hidden, m, out); break;
    case 6: launch_k<6, kUnit, kF16>(grid, block, stream, y, w, L, hidden, m, out); break;
    case 7: launch_k<7, kUnit, kF16>(grid, block, stream, y, w, L, hidden, m, out); break;
    case 8: launch_k<8, kUnit, kF16>(grid, block, stream, y, w, L, hidden, m, out); break;
    default: launch_k<0, kUnit, kF16>(grid, block, stream, y, w, L, hidden, m, out); break;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const void* y, const float* w, const ep_layout_t& L, int32_t hidden,
                          void* out, hipStream_t stream) {
  return launch_combine_weights<false>(y, w, L, hidden, out, stream);
}

hipError_t launch_combine_groups(const void* z, const ep_layout_t& GL, int32_t hidden, void* out,
                                 hipStream_t stream) {
  return launch_combine_weights<true>(z, nullptr, GL, hidden, out, stream);
}

hipError_t launch_combine_f16(const void* y, const float* w, const ep_layout_t& L,
                              int32_t hidden, void* out, hipStream_t stream) {
  return launch_combine_weights<false, true>(y, w, L, hidden, out, stream);
}

// ---------------------------------------------------------------------------
// Combine of FP8 expert outputs: every lane owns 8 channels of the token, reads
// their 8 code bytes from each row (one non-temporal 8-byte load; a wave
// covers 512 contiguous bytes of the row) and the row's scale for its
// 128-channel block, decodes with the gfx950 conversion instruction (exact),
// and accumulates w * scale * value in fp32; the 8 bf16 results leave as one
// 16-byte non-temporal store (a wave writes 1 KiB of the output row).  Eight
// channels per lane measured about 9% faster than sixteen, whose two 16-byte
// output stores per lane each cover only half of every cache line.  When a
// workgroup holds one token (or one slice of one token's row), the token index
// is uniform and its slots and weights come in through scalar loads before the
// row loads: about 10% faster than per-lane loads for this kernel (112 vs 124
// us at 8192 x 7168, top-8, one workgroup per token).

typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void accumulate8_fp8(float* acc, const u32x2_vec& c, float ws,
                                                bool valid) {
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.x, false);
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.x, true);
  const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.y, false);
  const f32x2 e = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.y, true);
  const float f[8] = {a.x, a.y, b.x, b.y, d.x, d.y, e.x, e.y};
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = valid ? fmaf(ws, f[i], acc[i]) : acc[i];
}

// E8M0 byte -> fp32 2^(b - 127): the exponent field itself for b >= 1, the
// subnormal 2^-127 for b = 0; 255 is NaN.
__device__ __forceinline__ float e8m0_to_float(uint32_t b) {
  if (b == 255u) return __uint_as_float(0x7FC00000u);
  return __uint_as_float(b == 0u ? 0x00400000u : (b << 23));
}

// Scale of row `row` for 8-channel slice v: kMx = E8M0 bytes, one per 32
// channels ([R, hidden/32]); else fp32, one per 128 channels ([R, hidden/128]).
template <bool kMx>
__device__ __forceinline__ float fp8_row_scale(const void* __restrict__ scales, int64_t row,
                                               int32_t hidden, int32_t v) {
  if constexpr (kMx)
    return e8m0_to_float(static_cast<const uint8_t*>(scales)[row * (hidden / 32) + v / 4]);
  else
    return static_cast<const float*>(scales)[row * (hidden / kFp8Block) + v / 16];
}

// One 8-channel slice v of token t: all K code and scale loads first, then the sum.
template <int K, bool kMx>
__device__ __forceinline__ void combine_fp8_slice(const uint8_t* __restrict__ q,
                                                  const void* __restrict__ scales,
                                                  const int32_t* s, const float* wt, int32_t k,
                                                  int32_t hidden, int32_t v,
                                                  u32x4* __restrict__ dst) {
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if constexpr (K > 0) {
    u32x2_vec c[K];
    float sc[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int64_t row = s[j] >= 0 ? s[j] : 0;
      c[j] = load_nt8(q + row * hidden + 8 * v);
      sc[j] = fp8_row_scale<kMx>(scales, row, hidden, v);
    }
#pragma unroll
    for (int j = 0; j < K; ++j) accumulate8_fp8(acc, c[j], wt[j] * sc[j], s[j] >= 0);
  } else {
    for (int32_t j = 0; j < k; ++j) {
      const int32_t sj = s[j];
      if (sj < 0) continue;
      accumulate8_fp8(acc, load_nt8(q + (int64_t)sj * hidden + 8 * v),
                      wt[j] * fp8_row_scale<kMx>(scales, sj, hidden, v), true);
    }
  }
  store_nt(dst + v, pack8(acc));
}

template <int K, bool kWhole, bool kMx>
__global__ __launch_bounds__(1024) void combine_fp8_kernel(
    const uint8_t* __restrict__ q, const void* __restrict__ scales, const float* __restrict__ w,
    const int32_t* __restrict__ slot_idx, int64_t num_tokens, int32_t k, int32_t hidden,
    CombineMap m, u32x4* __restrict__ out) {
  int64_t t;
  int32_t lt;
  if (!combine_token<kWhole>(m, num_tokens, t, lt)) return;
  const int32_t vecs = hidden / 8;  // 8-channel slices per row
  const int32_t stride = m.lanes_per_token * m.slices;
  const int32_t kk = K > 0 ? K : k;
  u32x4* dst = out + t * vecs;
  int32_t s[K > 0 ? K : 1];
  float ww[K > 0 ? K : 1];
  if constexpr (K > 0) {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      s[j] = slot_idx[t * K + j];
      ww[j] = w[t * K + j];
    }
  }
  const int32_t* sp = K > 0 ? s : slot_idx + t * kk;
  const float* wp = K > 0 ? ww : w + t * kk;
  if (vecs <= stride) {
    // one pass covers the row: straight-line code, every load issued up front
    if (lt < vecs) combine_fp8_slice<K, kMx>(q, scales, sp, wp, k, hidden, lt, dst);
  } else {
    for (int32_t v = lt; v < vecs; v += stride)
      combine_fp8_slice<K, kMx>(q, scales, sp, wp, k, hidden, v, dst);
  }
}

// FP8 rows of prefill-sized batches wider than four waves are split into
// slices of whole waves, one workgroup each: slices of 4, 3 or 2 waves when
// one of these divides the row's waves (the widest that does), else 2-wave
// slices with a last slice of one wave.  Measured on MI355X (top-8, random
// routing, 8192 tokens unless noted; one token per workgroup -> split, both
// on one box): hidden 7168 (14 waves, 7 x 2) 116-121 -> 101-102 us, MXFP8
// 115-121 -> 103-104 us, top-6 90-92 -> 80-82 us, 600 tokens 13.6 -> 12.0
// us; 6656 (13 waves, 2 x 6 + 1) 109-114 -> 93-94 us; 8192 (4 x 4) 125-130
// -> 111-112 us; 8704 (17 waves) 141-156 -> 119-121 us; 16384 at 4096 tokens
// (8 x 4) 119-125 -> 111-112 us; 6144 (3 x 4) 90-93 -> 87-88 us; 5120
// (5 x 2) 81-84 -> 73-74 us; 4608 (3 x 3) 74-77 -> 67-68 us; ragged 7296
// (912 vectors, 5 x 3) 124 -> 106 us; 2560 (2 + 2 + 1) 40.4-41.2 -> 39.3-39.5
// us; 3200 (7 waves) 51-53 us either way; 4096 at 65,536 tokens, top-6
// (2 x 4) 337-346 us either way.  Every split gave output identical to the
// unsplit launch.  Slices of 4 waves over a 5-wave row (one full, one a
// quarter full) measured slower (46.8 us), as did a 256-lane target that
// leaves a partly filled last slice at 7168 (104 us).  The bf16 combine reads
// twice the bytes per vector and measured slower split (182 -> 187-194 us at
// hidden 7168), so it keeps whole rows.
static void split_prefill_rows(int32_t vecs, int64_t T, CombineMap& m, dim3& grid, dim3& block) {
  const int32_t waves = (vecs + 63) / 64;
  if (waves <= 4) return;
  const int32_t w = waves % 4 == 0 ? 4 : (waves % 3 == 0 ? 3 : 2);
  const int64_t S = (waves + w - 1) / w;
  if (T * S * 64 * w > (int64_t)INT32_MAX) return;  // work items must fit the 32-bit grid size
  m.lanes_per_token = 64 * w;
  m.slices = (int32_t)S;
  grid = dim3((unsigned)(T * S));
  block = dim3((unsigned)(64 * w));
}

template <int K, bool kMx>
static void launch_fp8_k(dim3 grid, dim3 block, hipStream_t stream, const uint8_t* q,
                         const void* scales, const float* w, const ep_layout_t& L,
                         int32_t hidden, CombineMap m, void* out) {
  if (m.tokens_per_block == 1) {
    if (L.num_tokens * (int64_t)L.num_topk <= (int64_t)kDecodeCombinePairs)
      split_tokens(hidden / 8, L.num_tokens, m, grid, block);
    else
      split_prefill_rows(hidden / 8, L.num_tokens, m, grid, block);
  }
  if (m.tokens_per_block == 1)
    hipLaunchKernelGGL((combine_fp8_kernel<K, true, kMx>), grid, block, 0, stream, q, scales, w,
                       L.slot_idx, L.num_tokens, L.num_topk, hidden, m, static_cast<u32x4*>(out));
  else
    hipLaunchKernelGGL((combine_fp8_kernel<K, false, kMx>), grid, block, 0, stream, q, scales, w,
                       L.slot_idx, L.num_tokens, L.num_topk, hidden, m, static_cast<u32x4*>(out));
}

template <bool kMx>
static hipError_t launch_combine_codes(const uint8_t* q, const void* scales, const float* w,
                                       const ep_layout_t& L, int32_t hidden, void* out,
                                       hipStream_t stream) {
  const int64_t T = L.num_tokens;
  if (T == 0) return hipSuccess;
  const CombineMap m = combine_map(hidden / 8);
  const dim3 grid((unsigned)((T + m.tokens_per_block - 1) / m.tokens_per_block));
  const dim3 block(m.lanes_per_token * m.tokens_per_block);
  switch (L.num_topk) {
    case 1: launch_fp8_k<1, kMx>(grid, block, stream, q, scales, w, L, hidden, m, out); break;
    case 2: launch_fp8_k<2, kMx>(grid, block, stream, q, scales, w, L, hidden, m, out); break;
    case 4: launch_fp8_k<4, kMx>(grid, block, stream, q, scales, w, L, hidden, m, out); break;
    case 6: launch_fp8_k<6, kMx>(grid, block, stream, q, scales, w, L, hidden, m, out); break;
    case 8: launch_fp8_k<8, kMx>(grid, block, stream, q, scales, w, L, hidden, m, out); break;
    default: launch_fp8_k<0, kMx>(grid, block, stream, q, scales, w, L, hidden, m, out); break;
  }
  return hipGetLastError();
}

hipError_t launch_combine_fp8(const uint8_t* q, const float* scales, const float* w,
                              const ep_layout_t& L, int32_t hidden, void* out,
                              hipStream_t stream) {
  return launch_combine_codes<false>(q, scales, w, L, hidden, out, stream);
}

hipError_t launch_combine_mxfp8(const uint8_t* q, const uint8_t* scales, const float* w,
                                const ep_layout_t& L, int32_t hidden, void* out,
                                hipStream_t stream) {
  return launch_combine_codes<true>(q, scales, w, L, hidden, out, stream);
}

}  // namespace ep
