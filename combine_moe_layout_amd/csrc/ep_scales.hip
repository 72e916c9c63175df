// ep_scales.hip -- scale-layout conversion on gfx950: the row-major scales an
// FP8 dispatch writes (fp32 [rows, hidden/128], or MXFP8 E8M0 bytes
// [rows, hidden/32]) to the MN-major layout, where entry c of row r sits at
// c * rows + r.  Section "FP8與低精度通訊" of "DeepEP是什麼？…" (yololab.net)
// lists the scale format and the layout conversion among the checks of
// low-precision dispatch; MN-major keeps one block column's scales for
// consecutive rows together, as a GEMM over an expert's rows reads them.
//
// How: a workgroup owns a tile of consecutive rows and up to kColWords scale
// words of each.  Rows are contiguous, so consecutive lanes load consecutive
// words of the tile's rows into LDS, whose rows are padded to an odd word
// stride (reading one column across lanes then touches distinct banks).  The
// tile leaves column by column, consecutive lanes on consecutive rows, so each
// column of the tile is one contiguous run: 64 fp32 words or 128 E8M0 bytes,
// 256 or 128 bytes, stored 16 bytes per lane where alignment allows (for E8M0
// bytes a lane transposes 16 rows x 4 columns in registers).  Each byte is read
// once and written once.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

constexpr int kScaleThreads = 256;
constexpr int kColWords = 64;  // scale words per row in one tile

// kVec: 16-byte loads (four words of a row) and 16-byte stores (one column's
// entries of 16 / kEntryBytes consecutive rows, i.e. 4 fp32 words or 16 E8M0
// bytes); the host picks it when the row count, the row length and both
// pointers allow those accesses to be aligned.  Otherwise 4-byte loads and
// one store per entry.
template <int kEntryBytes, bool kVec>
__global__ __launch_bounds__(kScaleThreads) void scales_mn_kernel(
    const uint32_t* __restrict__ src, int64_t rows, int32_t row_words, uint8_t* __restrict__ dst) {
  constexpr int kTileRows = kEntryBytes == 4 ? 64 : 128;
  constexpr int kPerWord = 4 / kEntryBytes;  // entries per 4-byte word
  constexpr int kStride = kColWords + 1;     // odd: a column read across lanes hits distinct banks
  constexpr int kRowsPerStore = kVec ? 16 / kEntryBytes : 1;
  __shared__ uint32_t tile[kTileRows * kStride];
  const int64_t r0 = (int64_t)blockIdx.x * kTileRows;
  const int32_t w0 = (int32_t)blockIdx.y * kColWords;
  const int32_t nrows = rows - r0 < kTileRows ? (int32_t)(rows - r0) : kTileRows;
  const int32_t ncols = row_words - w0 < kColWords ? row_words - w0 : kColWords;

  if constexpr (kVec) {
    const int32_t quads = ncols / 4;
    for (int32_t i = threadIdx.x; i < nrows * quads; i += kScaleThreads) {
      const int32_t r = i / quads;
      const int32_t u = (i - r * quads) * 4;
      const u32x4 v = *reinterpret_cast<const u32x4*>(src + (r0 + r) * row_words + w0 + u);
      uint32_t* t = tile + r * kStride + u;
      t[0] = v.x;
      t[1] = v.y;
      t[2] = v.z;
      t[3] = v.w;
    }
  } else {
    for (int32_t i = threadIdx.x; i < nrows * ncols; i += kScaleThreads) {
      const int32_t r = i / ncols;
      const int32_t u = i - r * ncols;
      tile[r * kStride + u] = src[(r0 + r) * row_words + w0 + u];
    }
  }
  __syncthreads();

  // entry (row r, column c) of the tile; c counts entries, not words
  auto entry = [&](int32_t r, int32_t c) -> uint32_t {
    const uint32_t word = tile[r * kStride + c / kPerWord];
    return kEntryBytes == 4 ? word : (word >> (8 * (c % kPerWord))) & 0xFFu;
  };
  constexpr int kGroups = kTileRows / kRowsPerStore;  // stores per column of a tile
  if constexpr (kVec && kEntryBytes == 1) {
    // E8M0 bytes: a lane takes one tile word (4 columns) of 16 consecutive
    // rows, reads those 16 words once, transposes the 16 x 4 bytes in
    // registers and stores the 4 columns' 16-byte runs
    for (int32_t i = threadIdx.x; i < ncols * kGroups; i += kScaleThreads) {
      const int32_t u = i / kGroups;                        // tile word
      const int32_t r = (i - u * kGroups) * kRowsPerStore;  // first of 16 rows
      if (r >= nrows) continue;
      uint32_t rw[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) rw[q] = tile[(r + q) * kStride + u];
#pragma unroll
      for (int b = 0; b < 4; ++b) {  // column 4u + b
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w[q] = ((rw[4 * q] >> (8 * b)) & 0xFFu) | (((rw[4 * q + 1] >> (8 * b)) & 0xFFu) << 8) |
                 (((rw[4 * q + 2] >> (8 * b)) & 0xFFu) << 16) |
                 (((rw[4 * q + 3] >> (8 * b)) & 0xFFu) << 24);
        const int64_t at = (int64_t)(4 * (w0 + u) + b) * rows + r0 + r;
        *reinterpret_cast<u32x4*>(dst + at) = u32x4{w[0], w[1], w[2], w[3]};
      }
    }
    return;
  }
  const int32_t entries = ncols * kPerWord;
  for (int32_t i = threadIdx.x; i < entries * kGroups; i += kScaleThreads) {
    const int32_t c = i / kGroups;
    const int32_t r = (i - c * kGroups) * kRowsPerStore;
    if (r >= nrows) continue;  // with kVec, nrows is a multiple of kRowsPerStore
    const int64_t at = (int64_t)(w0 * kPerWord + c) * rows + r0 + r;  // in entries
    if constexpr (kVec) {
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (kEntryBytes == 4) {
          w[q] = entry(r + q, c);
        } else {
          w[q] = entry(r + 4 * q, c) | (entry(r + 4 * q + 1, c) << 8) |
                 (entry(r + 4 * q + 2, c) << 16) | (entry(r + 4 * q + 3, c) << 24);
        }
      }
      *reinterpret_cast<u32x4*>(dst + at * kEntryBytes) = u32x4{w[0], w[1], w[2], w[3]};
    } else if constexpr (kEntryBytes == 4) {
      reinterpret_cast<uint32_t*>(dst)[at] = entry(r, c);
    } else {
      dst[at] = (uint8_t)entry(r, c);
    }
  }
}

template <int kEntryBytes>
static void launch_scales_mn_as(const uint32_t* src, int64_t rows, int32_t row_words, uint8_t* dst,
                                bool vec, hipStream_t stream) {
  constexpr int kTileRows = kEntryBytes == 4 ? 64 : 128;
  const dim3 grid((unsigned)((rows + kTileRows - 1) / kTileRows),
                  (unsigned)((row_words + kColWords - 1) / kColWords));
  if (vec)
    hipLaunchKernelGGL((scales_mn_kernel<kEntryBytes, true>), grid, dim3(kScaleThreads), 0, stream,
                       src, rows, row_words, dst);
  else
    hipLaunchKernelGGL((scales_mn_kernel<kEntryBytes, false>), grid, dim3(kScaleThreads), 0, stream,
                       src, rows, row_words, dst);
}

hipError_t launch_scales_mn(const void* scales, int64_t rows, int32_t hidden, int32_t dtype,
                            void* scales_mn, hipStream_t stream) {
  const int32_t row_words = hidden / kFp8Block;  // 4-byte words per row in every scale format
  const bool mx = dtype == EP_MXFP8_E4M3;
  const int64_t rows_per_store = mx ? 16 : 4;
  // 16-byte accesses stay aligned when every row starts on a 16-byte boundary
  // (row_words % 4 == 0), every column run does (rows % rows_per_store == 0)
  // and both buffers do
  const bool vec = row_words % 4 == 0 && rows % rows_per_store == 0 &&
                   (reinterpret_cast<uintptr_t>(scales) & 15u) == 0 &&
                   (reinterpret_cast<uintptr_t>(scales_mn) & 15u) == 0;
  const uint32_t* src = static_cast<const uint32_t*>(scales);
  uint8_t* dst = static_cast<uint8_t*>(scales_mn);
  if (mx)
    launch_scales_mn_as<1>(src, rows, row_words, dst, vec, stream);
  else
    launch_scales_mn_as<4>(src, rows, row_words, dst, vec, stream);
  return hipGetLastError();
}

}  // namespace ep
