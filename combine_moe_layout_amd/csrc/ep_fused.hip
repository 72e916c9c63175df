// ep_fused.hip -- layout and dispatch in one launch for decode-sized batches.
//
// The pages' low-latency mode serves decode and small batches, where launch
// latency rather than bandwidth sets the time ("DeepEP是什麼？…" (yololab.net),
// section "高吞吐與低延遲工作負載"; v1's low-latency kernels dispatch in
// tens of microseconds: erai.pro DeepEP article, section "Chi tiết").  For a
// batch of at most kFusedMaxPairs (token, k) pairs this kernel computes the
// same layout as ep_get_layout and the same receive rows as ep_dispatch, with
// one launch and no barrier between workgroups:
//   - every workgroup reads the whole (small) top-k table; a token's
//     workgroup first issues the loads of its token's row, so that their
//     latency overlaps the table's;
//   - workgroup t < T finds its own token's receive rows directly: an LDS
//     histogram of the pairs before its token gives each of its k pairs the
//     rank within its expert (padded mode keeps rank < capacity), and in
//     contiguous mode an exclusive scan of the whole table's histogram gives
//     the expert's first row -- exactly the stable counting-sort position
//     ep_get_layout assigns;
//     it writes those slot_idx / recv_src entries and then dispatches the
//     token like ep_dispatch;
//   - workgroup T writes the per-expert counts, offsets, group totals and
//     error flags from an LDS histogram of the table.
#include "ep_device.h"
#include "ep_dispatch_token.h"
#include "ep_internal.h"
#include "ep_scan.h"

namespace ep {

struct FusedArgs {
  const int64_t* topk_idx;
  int64_t num_tokens;
  int32_t k, num_experts, num_groups, capacity, hidden;
  const u32x4* x;
  u32x4* recv;
  uint32_t* scales;
  int64_t scales_mn_rows;  // 0: row-major scales; else MN-major over this many rows
  int32_t* slot_idx;
  int32_t* recv_src;
  int32_t* num_tokens_per_expert;
  int32_t* expert_offsets;
  int32_t* num_tokens_per_group;
  int32_t* error_flags;
  const int32_t* extra_flags;  // flag entries a kernel that prepared the ids wrote (or null)
  int32_t num_extra_flags;
};

// Workgroups have at least kFusedMinLanes lanes, so a lane loads at most
// kTableTrips entries of the top-k table.
constexpr int kFusedMinLanes = 512;
constexpr int kTableTrips = kFusedMaxPairs / kFusedMinLanes;

// kDispatch = false: the layout alone (ep_get_layout for batches of one
// layout chunk); x, recv and scales are not touched.
template <bool kFp8, bool kHw, int kMode, bool kDispatch = true>
__global__ __launch_bounds__(1024) void layout_dispatch_small_kernel(FusedArgs a) {
  __shared__ int32_t s_tok[kFusedMaxTopk];  // this token's experts, -1 if none
  __shared__ int32_t s_slot[kFusedMaxTopk];
  __shared__ int32_t s_hist[EP_MAX_EXPERTS];
  __shared__ int32_t s_pre[EP_MAX_EXPERTS];
  __shared__ int32_t s_off[EP_MAX_EXPERTS];
  __shared__ int32_t s_wave[1024 / kWave];
  __shared__ int32_t s_flags;  // the metadata workgroup's error flags
  __shared__ uint32_t s_scale[kMaxScalesPerBlock];
  const int tid = threadIdx.x;
  const int E = a.num_experts, k = a.k;
  const int32_t P = (int32_t)(a.num_tokens * k);

  // A token's workgroup loads its slice of the token first (when one pass of
  // the lanes covers the row), so that this latency overlaps the table load
  // and the histograms below.
  const bool token_block = blockIdx.x < a.num_tokens;
  const int32_t vecs = kFp8 ? a.hidden / 16 : a.hidden / 8;
  const bool one_pass = vecs <= (int32_t)blockDim.x;
  const u32x4* src = a.x + (int64_t)blockIdx.x * (a.hidden / 8);
  u32x4 pre_lo = {0u, 0u, 0u, 0u}, pre_hi = {0u, 0u, 0u, 0u};
  if (kDispatch && token_block && one_pass && tid < vecs) {
    if constexpr (kFp8) {
      pre_lo = src[2 * tid];
      pre_hi = src[2 * tid + 1];
    } else {
      pre_lo = src[tid];
    }
  }

  // The table in at most kTableTrips loads per lane, all issued before the
  // first is used: a loop that handled each entry before loading the next
  // would wait one memory latency per trip.
  int64_t tv[kTableTrips];
#pragma unroll
  for (int i = 0; i < kTableTrips; ++i) {
    const int32_t p = tid + i * (int32_t)blockDim.x;
    tv[i] = p < P ? a.topk_idx[p] : -1;
  }
  // the metadata workgroup ORs in the flag entries of a prepared table
  int32_t extra_bits = 0;
  if (!token_block && a.extra_flags != nullptr)
    for (int32_t i = tid; i < a.num_extra_flags; i += blockDim.x) extra_bits |= a.extra_flags[i];

  // Histograms of the valid pairs: of the whole table (s_hist; the
  // metadata workgroup's counts, and each expert's first row in contiguous
  // mode after a scan) and of the pairs before this token (s_pre; the rank of
  // the token's pairs within their experts).  Padded mode places rows at
  // e * capacity, so its token workgroups need only s_pre.
  const bool need_hist = !token_block || a.capacity == 0;
  const int32_t p0 = token_block ? (int32_t)blockIdx.x * k : 0;
  for (int e = tid; e < E; e += blockDim.x) {
    s_hist[e] = 0;
    s_pre[e] = 0;
  }
  if (tid == 0) s_flags = 0;
  __syncthreads();
  bool bad = false;
#pragma unroll
  for (int i = 0; i < kTableTrips; ++i) {
    const int32_t p = tid + i * (int32_t)blockDim.x;
    if (p < P) {
      const bool ok = tv[i] >= 0 && tv[i] < E;
      bad |= !ok && tv[i] != -1;
      const int32_t e = ok ? (int32_t)tv[i] : -1;
      if (e >= 0) {
        if (need_hist) atomicAdd(&s_hist[e], 1);
        if (p < p0) atomicAdd(&s_pre[e], 1);
      }
      if (token_block && p >= p0 && p < p0 + k) s_tok[p - p0] = e;
    }
  }
  __syncthreads();

  if (!token_block) {
    // metadata: counts, offsets, group totals (differences of the exclusive
    // prefix), flags (one LDS OR per wave, ordered by the scan's barriers)
    bool over = false;
    for (int e = tid; e < E; e += blockDim.x) over |= a.capacity > 0 && s_hist[e] > a.capacity;
    bad |= (extra_bits & EP_FLAG_BAD_EXPERT) != 0;
    over |= (extra_bits & EP_FLAG_OVERFLOW) != 0;
    const bool wave_bad = __ballot(bad) != 0;
    const bool wave_over = __ballot(over) != 0;
    if (tid % kWave == 0 && (wave_bad || wave_over))
      atomicOr(&s_flags, (wave_bad ? EP_FLAG_BAD_EXPERT : 0) | (wave_over ? EP_FLAG_OVERFLOW : 0));
    const int32_t total = block_exclusive_scan(s_hist, s_off, E, s_wave);
    for (int e = tid; e < E; e += blockDim.x) {
      a.num_tokens_per_expert[e] = s_hist[e];
      a.expert_offsets[e] = a.capacity > 0 ? e * a.capacity : s_off[e];
    }
    if (tid == 0) {
      a.expert_offsets[E] = a.capacity > 0 ? E * a.capacity : total;
      a.error_flags[0] = s_flags;
    }
    const int per_group = E / a.num_groups;
    for (int g = tid; g < a.num_groups; g += blockDim.x) {
      const int32_t end = g + 1 == a.num_groups ? total : s_off[(g + 1) * per_group];
      a.num_tokens_per_group[g] = end - s_off[g * per_group];
    }
    return;
  }

  // this token's receive rows: pair j of expert e takes rank s_pre[e] plus
  // the token's earlier pairs of e -- its stable counting-sort position, as
  // ep_get_layout assigns it
  if (a.capacity == 0) block_exclusive_scan(s_hist, s_off, E, s_wave);
  if (tid < k) {
    const int j = tid;
    const int32_t e = s_tok[j];
    int32_t s = -1;
    if (e >= 0) {
      int32_t rank = s_pre[e];
      for (int i = 0; i < j; ++i) rank += s_tok[i] == e ? 1 : 0;
      if (a.capacity == 0) s = s_off[e] + rank;
      else if (rank < a.capacity) s = e * a.capacity + rank;
    }
    s_slot[j] = s;
    a.slot_idx[p0 + j] = s;
    if (a.recv_src != nullptr && s >= 0) a.recv_src[s] = p0 + j;
  }
  __syncthreads();

  if constexpr (!kDispatch) return;

  // dispatch the token (one token per workgroup, all lanes on its row)
  if (one_pass) {
    if (tid < vecs) {
      if constexpr (kFp8)
        fp8_vector_codes<kHw, kMode>(pre_lo, pre_hi, tid, s_slot, k, a.recv, vecs, s_scale);
      else
        for (int32_t j = 0; j < k; ++j)
          if (s_slot[j] >= 0) store_nt(a.recv + (int64_t)s_slot[j] * vecs + tid, pre_lo);
    }
  } else if constexpr (kFp8) {
    fp8_token_codes<kHw, kMode>(src, a.hidden, tid, blockDim.x, s_slot, k, a.recv, s_scale);
  } else {
    bf16_token_copy(src, a.hidden, tid, blockDim.x, s_slot, k, a.recv);
  }
  if constexpr (kFp8) {
    __syncthreads();
    fp8_token_scales_any<kMode>(a.hidden, tid, blockDim.x, s_slot, k, s_scale, a.scales_mn_rows,
                                a.scales);
  }
}

bool fused_layout_dispatch_fits(const ep_layout_t& L) {
  return L.num_tokens > 0 && L.num_tokens * (int64_t)L.num_topk <= kFusedMaxPairs &&
         L.num_topk <= kFusedMaxTopk;
}

hipError_t launch_layout_dispatch_small(const int64_t* topk_idx, const ep_layout_t& L,
                                        const void* x, int32_t hidden, int32_t dtype,
                                        void* recv_x, void* recv_scales, hipStream_t stream) {
  const int64_t mn_rows = dtype_scales_mn(dtype) ? L.num_recv_rows : 0;
  dtype = dtype_base(dtype);
  const bool fp8 = dtype_is_fp8(dtype);
  FusedArgs a = {};
  a.extra_flags = nullptr;  // the top-k table comes from the caller: no prepared flags
  a.num_extra_flags = 0;
  a.topk_idx = topk_idx;
  a.num_tokens = L.num_tokens;
  a.k = L.num_topk;
  a.num_experts = L.num_experts;
  a.num_groups = L.num_groups;
  a.capacity = L.capacity;
  a.hidden = hidden;
  a.x = static_cast<const u32x4*>(x);
  a.recv = static_cast<u32x4*>(recv_x);
  a.scales = static_cast<uint32_t*>(recv_scales);
  a.scales_mn_rows = mn_rows;
  a.slot_idx = L.slot_idx;
  a.recv_src = L.recv_src;
  a.num_tokens_per_expert = L.num_tokens_per_expert;
  a.expert_offsets = L.expert_offsets;
  a.num_tokens_per_group = L.num_tokens_per_group;
  a.error_flags = L.error_flags;
  // one token per workgroup: one lane per 16-byte output vector, whole waves,
  // at least kFusedMinLanes lanes for the table, at most 1024 (longer rows loop)
  const int32_t vecs = fp8 ? hidden / 16 : hidden / 8;
  int32_t lanes = ((vecs + 63) / 64) * 64;
  lanes = lanes < kFusedMinLanes ? kFusedMinLanes : (lanes > 1024 ? 1024 : lanes);
  const dim3 grid((unsigned)(L.num_tokens + 1));
  if (dtype == EP_FP8_E4M3)
    hipLaunchKernelGGL((layout_dispatch_small_kernel<true, kDispatchUsesHwCast, kScaleF32>), grid,
                       dim3(lanes), 0, stream, a);
  else if (dtype == EP_FP8_E4M3_POW2)
    hipLaunchKernelGGL((layout_dispatch_small_kernel<true, kDispatchUsesHwCast, kScalePow2>), grid,
                       dim3(lanes), 0, stream, a);
  else if (dtype == EP_MXFP8_E4M3)
    hipLaunchKernelGGL((layout_dispatch_small_kernel<true, kDispatchUsesHwCast, kScaleMx>), grid,
                       dim3(lanes), 0, stream, a);
  else  // EP_BF16 and EP_F16: a bit copy
    hipLaunchKernelGGL((layout_dispatch_small_kernel<false, kDispatchUsesHwCast, kScaleF32>), grid,
                       dim3(lanes), 0, stream, a);
  return hipGetLastError();
}

// The layout alone for a batch that fits the fused kernel: one workgroup of
// kFusedMinLanes lanes per token plus the metadata workgroup, one launch.
// extra_flags: num_extra flag entries written by the kernel that prepared the
// ids (the group layout's table), ORed into error_flags.
hipError_t launch_layout_small(const int64_t* topk_idx, const ep_layout_t& L,
                               const int32_t* extra_flags, int32_t num_extra,
                               hipStream_t stream) {
  FusedArgs a = {};
  a.extra_flags = extra_flags;
  a.num_extra_flags = num_extra;
  a.topk_idx = topk_idx;
  a.num_tokens = L.num_tokens;
  a.k = L.num_topk;
  a.num_experts = L.num_experts;
  a.num_groups = L.num_groups;
  a.capacity = L.capacity;
  a.slot_idx = L.slot_idx;
  a.recv_src = L.recv_src;
  a.num_tokens_per_expert = L.num_tokens_per_expert;
  a.expert_offsets = L.expert_offsets;
  a.num_tokens_per_group = L.num_tokens_per_group;
  a.error_flags = L.error_flags;
  hipLaunchKernelGGL((layout_dispatch_small_kernel<false, kDispatchUsesHwCast, kScaleF32, false>),
                     dim3((unsigned)(L.num_tokens + 1)), dim3(kFusedMinLanes), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ep
