// ep_aux.hip -- helpers around the path: the identity-expert stand-ins for
// FP8 and MXFP8 receive buffers, the FP8 encoder exposed for verification, and
// a streaming copy kernel that serves as the bandwidth reference.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

// y = bf16 of decode(q) * scale, rounded once from the exact product: the
// product of a 4-significant-bit code and an fp32 scale has at most 28 bits,
// so fma recovers the rounding error of the fp32 product exactly.
__global__ __launch_bounds__(256) void dequant_fp8_kernel(const u32x4* __restrict__ q,
                                                          const float* __restrict__ scales,
                                                          int64_t units, int32_t units_per_row,
                                                          int32_t blocks_per_row,
                                                          u32x4* __restrict__ y) {
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < units;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = u / units_per_row;
    const int32_t c16 = (int32_t)(u % units_per_row);
    const float s = scales[r * blocks_per_row + c16 / 8];
    const u32x4 codes = q[u];
    const uint32_t words[4] = {codes.x, codes.y, codes.z, codes.w};
    uint32_t outw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t word = words[i / 2];
      const int sh = (i % 2) * 16;
      const float d0 = e4m3_decode((word >> sh) & 0xFFu);
      const float d1 = e4m3_decode((word >> (sh + 8)) & 0xFFu);
      const float p0 = d0 * s, p1 = d1 * s;
      const float e0 = fmaf(d0, s, -p0), e1 = fmaf(d1, s, -p1);
      outw[i] = bf16_round_exact(p0, e0) | (bf16_round_exact(p1, e1) << 16);
    }
    y[2 * u] = u32x4{outw[0], outw[1], outw[2], outw[3]};
    y[2 * u + 1] = u32x4{outw[4], outw[5], outw[6], outw[7]};
  }
}

template <int kMethod>
__global__ __launch_bounds__(256) void cast_bits_kernel(uint32_t first, int64_t n,
                                                        uint8_t* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float v = clamp_fp8(__uint_as_float(first + (uint32_t)i));
    uint32_t code;
    if constexpr (kMethod == 2) {
      code = e4m3_encode2_hw(v, 0.0f) & 0xFFu;
    } else {
      code = e4m3_encode_sw(v);
    }
    out[i] = (uint8_t)code;
  }
}

// Streaming copy: each workgroup moves 16 KiB, every lane four 16-byte vectors
// 4 KiB apart (so each wave instruction covers 1 KiB), all four loads issued
// before the stores, non-temporal both ways like the dispatch and combine rows.
constexpr int kCopyThreads = 256;
constexpr int kCopyVecs = 4;

__global__ __launch_bounds__(kCopyThreads) void copy_kernel(const u32x4* __restrict__ src,
                                                            u32x4* __restrict__ dst, int64_t n) {
  const int64_t base = (int64_t)blockIdx.x * (kCopyThreads * kCopyVecs) + threadIdx.x;
  u32x4 v[kCopyVecs];
#pragma unroll
  for (int u = 0; u < kCopyVecs; ++u)
    if (base + u * kCopyThreads < n) v[u] = load_nt(src + base + u * kCopyThreads);
#pragma unroll
  for (int u = 0; u < kCopyVecs; ++u)
    if (base + u * kCopyThreads < n) store_nt(dst + base + u * kCopyThreads, v[u]);
}

static unsigned grid_for(int64_t work, int per_block) {
  int64_t g = (work + per_block - 1) / per_block;
  const int64_t cap = 256 * 32;  // 32 workgroups per CU on 256 CUs, then grid-stride
  return (unsigned)(g < 1 ? 1 : (g > cap ? cap : g));
}

hipError_t launch_dequant_fp8(const uint8_t* q, const float* scales, int64_t rows, int32_t hidden,
                              void* y, hipStream_t stream) {
  const int64_t units = rows * (int64_t)(hidden / 16);
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_fp8_kernel, dim3(grid_for(units, 256)), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4*>(q), scales, units, hidden / 16,
                     hidden / kFp8Block, static_cast<u32x4*>(y));
  return hipGetLastError();
}

// y = bf16 of decode(q) * 2^(byte - 127) for MXFP8 rows (one E8M0 byte per
// 32 channels): the product of a 4-significant-bit code and a power of two
// between 2^-127 and 2^119 is exact in fp32 (subnormal results included), so
// one rounding to bf16 gives the nearest value.
__global__ __launch_bounds__(256) void dequant_mxfp8_kernel(const u32x4* __restrict__ q,
                                                            const uint8_t* __restrict__ scales,
                                                            int64_t units, int32_t units_per_row,
                                                            int32_t blocks_per_row,
                                                            u32x4* __restrict__ y) {
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < units;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = u / units_per_row;
    const int32_t c16 = (int32_t)(u % units_per_row);
    const uint32_t byte = scales[r * blocks_per_row + c16 / 2];
    const int32_t e = (int32_t)byte - 127;
    const u32x4 codes = q[u];
    const uint32_t words[4] = {codes.x, codes.y, codes.z, codes.w};
    uint32_t outw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t word = words[i / 2];
      const int sh = (i % 2) * 16;
      const float a = ldexpf(e4m3_decode((word >> sh) & 0xFFu), e);
      const float b = ldexpf(e4m3_decode((word >> (sh + 8)) & 0xFFu), e);
      // E8M0 byte 255 is NaN: the whole block becomes the quiet NaN 0x7FC0
      outw[i] = byte == 255u ? 0x7FC07FC0u : (bf16_rne(a) | (bf16_rne(b) << 16));
    }
    y[2 * u] = u32x4{outw[0], outw[1], outw[2], outw[3]};
    y[2 * u + 1] = u32x4{outw[4], outw[5], outw[6], outw[7]};
  }
}

hipError_t launch_dequant_mxfp8(const uint8_t* q, const uint8_t* scales, int64_t rows,
                                int32_t hidden, void* y, hipStream_t stream) {
  const int64_t units = rows * (int64_t)(hidden / 16);
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_mxfp8_kernel, dim3(grid_for(units, 256)), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4*>(q), scales, units, hidden / 16, hidden / 32,
                     static_cast<u32x4*>(y));
  return hipGetLastError();
}

hipError_t launch_cast_e4m3_bits(uint32_t first, int64_t n, int32_t method, uint8_t* out,
                                 hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const bool hw = method == 2 || (method == 0 && kDispatchUsesHwCast);
  if (hw)
    hipLaunchKernelGGL(cast_bits_kernel<2>, dim3(grid_for(n, 256)), dim3(256), 0, stream, first,
                       n, out);
  else
    hipLaunchKernelGGL(cast_bits_kernel<1>, dim3(grid_for(n, 256)), dim3(256), 0, stream, first,
                       n, out);
  return hipGetLastError();
}

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  const int64_t n = (int64_t)(bytes / 16);
  if (n == 0) return hipSuccess;
  const int64_t per_block = kCopyThreads * kCopyVecs;
  const int64_t blocks = (n + per_block - 1) / per_block;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, stream,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n);
  return hipGetLastError();
}

}  // namespace ep
