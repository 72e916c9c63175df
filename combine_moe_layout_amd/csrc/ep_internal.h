// ep_internal.h -- launchers shared between the kernel sources and the C ABI
// (ep_api.hip).  Arguments are validated by the caller before these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ep.h"

namespace ep {

// Layout: chunks of kChunkPairs (t, k) pairs; each chunk is one workgroup of
// the counting kernel.  The packed intermediate in slot_idx keeps the expert
// id in the low kExpertBits bits and the rank inside the chunk above them.
// The layout is latency-bound (a few dozen workgroups), so a chunk's
// workgroup is as wide as possible and each lane walks few pairs: 16 waves
// of 2 items (measured on MI355X: 13.7 us for the two launches at 65,536
// pairs, against 17.0 us with 4 waves of 8 items).
constexpr int kLayoutThreads = 1024;
constexpr int kLayoutWaves = kLayoutThreads / 64;
constexpr int kLayoutItems = 2;
constexpr int kWavePairs = kLayoutItems * 64;
constexpr int kChunkPairs = kWavePairs * kLayoutWaves;
constexpr int kExpertBits = 11;
static_assert((1 << kExpertBits) >= EP_MAX_EXPERTS, "expert id must fit the packed field");

inline int64_t layout_num_chunks(int64_t pairs) { return (pairs + kChunkPairs - 1) / kChunkPairs; }

// Bytes of layout workspace: per-chunk counts and flags, plus extra_flags
// flag entries for a kernel that prepares the ids (the group layout's table).
size_t layout_workspace_bytes(int64_t pairs, int32_t num_experts, int64_t extra_flags = 0);

hipError_t launch_layout(const int64_t* topk_idx, const ep_layout_t& L, void* workspace,
                         hipStream_t stream);

// The layout over an id table that another kernel wrote, which also left
// extra_flags bad-id flag entries at layout_extra_flags(L, workspace).  With
// warm != null, the two layout launches also read the first
// min(warm_bytes, kWarmMaxBytes) of `warm` into the last-level cache from
// kWarmBlocks extra workgroups each (kWarmCountShare percent during the count
// launch, the rest during the finish launch).
hipError_t launch_layout_ids(const int64_t* ids, const ep_layout_t& L, void* workspace,
                             int32_t extra_flags, hipStream_t stream,
                             const void* warm = nullptr, size_t warm_bytes = 0);
int32_t* layout_extra_flags(const ep_layout_t& L, void* workspace);

// The layout of a large batch whose dispatch source x (warm_bytes) follows:
// x is read into the last-level cache while the latency-bound layout runs.
#ifndef EP_WARM_COUNT_SHARE
#define EP_WARM_COUNT_SHARE 40
#endif
constexpr int kWarmCountShare = EP_WARM_COUNT_SHARE;
constexpr int kWarmBlocks = 256;
// At most half the MI355X MALL (256 MB) is read ahead: more would evict
// itself before dispatch reads it.  Of a larger source only the first part
// is read ahead; dispatch reads tokens in order, so it meets that part first.
constexpr size_t kWarmMaxBytes = (size_t)128 << 20;
hipError_t launch_layout_warm(const int64_t* topk_idx, const ep_layout_t& L, void* workspace,
                              const void* warm, size_t warm_bytes, hipStream_t stream);
// Receive dtypes whose rows are E4M3 codes with a scale row (the others are a
// bit copy of 2-byte elements).
inline bool dtype_is_fp8(int32_t dtype) {
  return dtype == EP_FP8_E4M3 || dtype == EP_FP8_E4M3_POW2 || dtype == EP_MXFP8_E4M3;
}

// A dispatch dtype splits into its element type and the option flags.
inline int32_t dtype_base(int32_t dtype) {
  return dtype & ~(EP_SCALES_MN_MAJOR | EP_READ_X_AHEAD);
}
inline bool dtype_scales_mn(int32_t dtype) { return (dtype & EP_SCALES_MN_MAJOR) != 0; }
inline bool dtype_read_x_ahead(int32_t dtype) { return (dtype & EP_READ_X_AHEAD) != 0; }

// recv_scales: fp32 [R, hidden/128] or, for EP_MXFP8_E4M3, E8M0 bytes
// [R, hidden/32]: hidden/128 4-byte words per row either way.  With
// EP_SCALES_MN_MAJOR in dtype the same entries are stored transposed.
hipError_t launch_dispatch(const void* x, const ep_layout_t& L, int32_t hidden, int32_t dtype,
                           void* recv_x, void* recv_scales, hipStream_t stream);

// Row-major scales of `rows` rows (the layout an FP8 dispatch of dtype writes
// without EP_SCALES_MN_MAJOR) -> the MN-major layout, every row.
hipError_t launch_scales_mn(const void* scales, int64_t rows, int32_t hidden, int32_t dtype,
                            void* scales_mn, hipStream_t stream);

hipError_t launch_combine(const void* y, const float* w, const ep_layout_t& L, int32_t hidden,
                          void* out, hipStream_t stream);

// Combine with fp16 expert outputs and fp16 output.
hipError_t launch_combine_f16(const void* y, const float* w, const ep_layout_t& L,
                              int32_t hidden, void* out, hipStream_t stream);

hipError_t launch_dequant_fp8(const uint8_t* q, const float* scales, int64_t rows, int32_t hidden,
                              void* y, hipStream_t stream);

hipError_t launch_dequant_mxfp8(const uint8_t* q, const uint8_t* scales, int64_t rows,
                                int32_t hidden, void* y, hipStream_t stream);

hipError_t launch_cast_e4m3_bits(uint32_t first, int64_t n, int32_t method, uint8_t* out,
                                 hipStream_t stream);

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

// The encoder ep_dispatch uses: the gfx950 conversion instruction (OCP E4M3,
// round to nearest even), checked against the software encoder and the
// oracle over every fp32 input of magnitude <= 448.
constexpr bool kDispatchUsesHwCast = true;

// Batches of at most this many (token, k) pairs, with top-k at most
// kFusedMaxTopk, take the one-launch layout (+ dispatch) kernels.
constexpr int kFusedMaxPairs = 2 * kChunkPairs;
// Combines of at most this many pairs are decode-sized: one token per
// workgroup, slots and weights through scalar loads, tokens split over
// several workgroups when there are fewer tokens than CUs.  (At 512 tokens,
// top-8, the scalar-load form measured 11.5 against 11.9 us for the bf16
// combine; at 8192 tokens the per-lane loads win.)
constexpr int kDecodeCombinePairs = kFusedMaxPairs;
constexpr int kFusedMaxTopk = 8;
// Compute units of the MI355X (gfx950) this library is built for.
constexpr int kChipCUs = 256;

bool fused_layout_dispatch_fits(const ep_layout_t& L);
hipError_t launch_layout_small(const int64_t* topk_idx, const ep_layout_t& L,
                               const int32_t* extra_flags, int32_t num_extra,
                               hipStream_t stream);

hipError_t launch_layout_dispatch_small(const int64_t* topk_idx, const ep_layout_t& L,
                                        const void* x, int32_t hidden, int32_t dtype,
                                        void* recv_x, void* recv_scales, hipStream_t stream);

hipError_t launch_combine_fp8(const uint8_t* q, const float* scales, const float* w,
                              const ep_layout_t& L, int32_t hidden, void* out, hipStream_t stream);

// Combine of MXFP8 expert outputs: E4M3 codes [R, hidden] with one E8M0 byte
// per 32 channels [R, hidden/32].
hipError_t launch_combine_mxfp8(const uint8_t* q, const uint8_t* scales, const float* w,
                                const ep_layout_t& L, int32_t hidden, void* out,
                                hipStream_t stream);

// Per-group dedup variant: the group layout (a layout whose experts are the
// G groups, with kg = min(k, G) entries per token) and its unit-weight combine.
size_t group_layout_workspace_bytes(int64_t T, int32_t k, int32_t G);

hipError_t launch_group_layout(const int64_t* topk_idx, const float* topk_weights, int32_t k,
                               int32_t E, const ep_layout_t& GL, int64_t* recv_idx,
                               float* recv_w, uint8_t* member, void* workspace,
                               hipStream_t stream);

hipError_t launch_combine_groups(const void* z, const ep_layout_t& GL, int32_t hidden, void* out,
                                 hipStream_t stream);

}  // namespace ep
