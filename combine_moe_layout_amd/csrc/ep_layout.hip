// ep_layout.hip -- routing layout for MoE dispatch on gfx950.
//
// Computes, from the router's top-k expert ids, the per-expert and per-group
// counts, the expert offsets of the receive buffer and the receive row of
// every (token, k) pair -- the sort by expert that the dispatch stage needs
// ("DeepEP是什麼？…" (yololab.net), section "MoE為什麼需要All-to-all？",
// stage table, dispatch row; section "Load Imbalance" for the per-expert and
// per-rank counts).  The pages use remote atomics to claim receive space
// ("DeepEP 编址服务深度对抗分析", section 二.2), which gives a valid but
// run-dependent order; here the order inside an expert is stable in the pair
// index p = t*k + j, so the layout is deterministic.
//
// Two launches:
//   1. count: one workgroup per chunk of kChunkPairs pairs.  Each wave walks
//      its 512 pairs in order, 64 at a time; lanes that name the same expert
//      find each other with one ballot per expert-id bit, the lowest such
//      lane bumps the wave's private LDS histogram, and every lane's rank is
//      the histogram value plus the number of lower peer lanes.  No atomics,
//      so the ranks are deterministic.  The chunk's per-expert totals go to
//      the workspace; every pair's (rank in chunk, expert) goes, packed, into
//      slot_idx.
//   2. finish: one workgroup per chunk again.  Each sums the chunk totals of
//      earlier chunks (its base inside each expert) and of all chunks (the
//      expert totals) -- staging the whole count matrix in LDS with every load
//      in flight at once when it fits -- scans the totals into expert offsets,
//      and turns the packed values of its chunk into receive rows.  Workgroup
//      0 also writes the counts, offsets, group totals and error flags.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

size_t layout_workspace_bytes(int64_t pairs, int32_t num_experts) {
  int64_t chunks = layout_num_chunks(pairs);
  size_t bytes = (size_t)(chunks * num_experts + chunks) * sizeof(int32_t);
  return ((bytes + 255) / 256) * 256 + 256;
}

__global__ __launch_bounds__(kLayoutThreads) void layout_count_kernel(
    const int64_t* __restrict__ topk_idx, int64_t num_pairs, int32_t num_experts,
    int32_t expert_bits, int32_t* __restrict__ chunk_count, int32_t* __restrict__ chunk_flags,
    int32_t* __restrict__ packed) {
  __shared__ int32_t hist[kLayoutWaves][EP_MAX_EXPERTS];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int64_t wave_base = (int64_t)blockIdx.x * kChunkPairs + (int64_t)wave * kWavePairs;

  // Each wave owns one histogram row; LDS operations of one wave complete in
  // order, so the row needs no block barrier until other waves read it.
  for (int e = lane; e < num_experts; e += kWave) hist[wave][e] = 0;

  int32_t eid[kLayoutItems];
  bool bad = false;
#pragma unroll
  for (int i = 0; i < kLayoutItems; ++i) {
    const int64_t p = wave_base + i * kWave + lane;
    const int64_t v = p < num_pairs ? topk_idx[p] : -1;
    const bool ok = v >= 0 && v < num_experts;
    bad |= !ok && v != -1;
    eid[i] = ok ? (int32_t)v : -1;
  }

  const uint64_t below_me = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t rank[kLayoutItems];
#pragma unroll
  for (int i = 0; i < kLayoutItems; ++i) {
    const int e = eid[i];
    const bool valid = e >= 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < expert_bits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int lower = __popcll(peers & below_me);
    int32_t base = 0;
    if (valid) base = hist[wave][e];
    if (valid && lower == 0) hist[wave][e] = base + __popcll(peers);
    rank[i] = base + lower;
  }
  __syncthreads();

  // Chunk totals per expert; each wave's row becomes its exclusive prefix.
  for (int e = threadIdx.x; e < num_experts; e += kLayoutThreads) {
    int32_t run = 0;
#pragma unroll
    for (int w = 0; w < kLayoutWaves; ++w) {
      const int32_t h = hist[w][e];
      hist[w][e] = run;
      run += h;
    }
    chunk_count[(int64_t)blockIdx.x * num_experts + e] = run;
  }
  const int any_bad = __syncthreads_or(bad ? 1 : 0);
  if (threadIdx.x == 0) chunk_flags[blockIdx.x] = any_bad ? EP_FLAG_BAD_EXPERT : 0;

#pragma unroll
  for (int i = 0; i < kLayoutItems; ++i) {
    const int64_t p = wave_base + i * kWave + lane;
    if (p < num_pairs) {
      const int e = eid[i];
      packed[p] = e >= 0 ? (((hist[wave][e] + rank[i]) << kExpertBits) | e) : -1;
    }
  }
}

// Per-chunk counts up to this many ints are staged whole in LDS by the finish
// kernel (all loads in flight at once); larger matrices are summed from memory.
constexpr int kStageInts = 12288;
static_assert(kStageInts % (4 * kLayoutThreads) == 0, "staging is done in whole 16-byte batches");

__global__ __launch_bounds__(kLayoutThreads) void layout_finish_kernel(
    int64_t num_pairs, int32_t num_experts, int32_t num_groups, int32_t capacity,
    int32_t num_chunks, const int32_t* __restrict__ chunk_count,
    const int32_t* __restrict__ chunk_flags, int32_t* __restrict__ slot_idx,
    int32_t* __restrict__ recv_src, int32_t* __restrict__ num_tokens_per_expert,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ num_tokens_per_group,
    int32_t* __restrict__ error_flags) {
  __shared__ int32_t s_counts[kStageInts];
  __shared__ int32_t s_tot[EP_MAX_EXPERTS];
  __shared__ int32_t s_pre[EP_MAX_EXPERTS];
  __shared__ int32_t s_off[EP_MAX_EXPERTS];
  __shared__ int32_t s_wave[kLayoutWaves];
  const int E = num_experts;
  const int c = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int64_t chunk_base = (int64_t)c * kChunkPairs;

  // This chunk's packed (rank, expert) values, fetched now so that their
  // latency overlaps the count loads below.
  int32_t packed[kLayoutItems];
#pragma unroll
  for (int i = 0; i < kLayoutItems; ++i) {
    const int64_t p = chunk_base + i * kLayoutThreads + tid;
    packed[i] = p < num_pairs ? slot_idx[p] : -1;
  }

  // 1. expert totals over all chunks, and over the chunks before this one
  for (int e = tid; e < E; e += kLayoutThreads) {
    s_tot[e] = 0;
    s_pre[e] = 0;
  }
  const int64_t matrix = (int64_t)num_chunks * E;
  if (matrix <= kStageInts) {
    // 16-byte loads, a fixed number per thread, all issued before the first
    // is waited for (the workspace is 256-byte aligned)
    constexpr int kBatch = kStageInts / 4 / kLayoutThreads;
    const int n4 = (int)(matrix / 4);
    const int4* src4 = reinterpret_cast<const int4*>(chunk_count);
    int4* dst4 = reinterpret_cast<int4*>(s_counts);
    if (n4 > 0) {
      int4 r[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int i = tid + b * kLayoutThreads;
        r[b] = src4[i < n4 ? i : n4 - 1];  // unconditional, so r stays in registers
      }
      // unconditional as well: entries past the matrix land in the unused
      // tail of s_counts and are never read
#pragma unroll
      for (int b = 0; b < kBatch; ++b) dst4[tid + b * kLayoutThreads] = r[b];
    }
    for (int i = 4 * n4 + tid; i < matrix; i += kLayoutThreads) s_counts[i] = chunk_count[i];
    __syncthreads();
    const int lanes_per_expert = E >= kLayoutThreads ? 1 : kLayoutThreads / E;
    const int span = E >= kLayoutThreads ? E : E * lanes_per_expert;
    for (int idx = tid; idx < span; idx += kLayoutThreads) {
      const int e = idx % E;
      const int sub = idx / E;
      int32_t tot = 0, pre = 0;
      for (int cc = sub; cc < num_chunks; cc += lanes_per_expert) {
        const int32_t v = s_counts[cc * E + e];
        tot += v;
        pre += cc < c ? v : 0;
      }
      atomicAdd(&s_tot[e], tot);
      atomicAdd(&s_pre[e], pre);
    }
  } else {
    __syncthreads();
    const int lanes_per_expert = E >= kLayoutThreads ? 1 : kLayoutThreads / E;
    const int span = E >= kLayoutThreads ? E : E * lanes_per_expert;
    for (int idx = tid; idx < span; idx += kLayoutThreads) {
      const int e = idx % E;
      const int sub = idx / E;
      int32_t tot = 0, pre = 0;
#pragma unroll 16
      for (int cc = sub; cc < num_chunks; cc += lanes_per_expert) {
        const int32_t v = chunk_count[(int64_t)cc * E + e];
        tot += v;
        pre += cc < c ? v : 0;
      }
      atomicAdd(&s_tot[e], tot);
      atomicAdd(&s_pre[e], pre);
    }
  }
  __syncthreads();

  // 2. exclusive scan of the totals (contiguous mode) -> expert offsets
  const int per = (E + kLayoutThreads - 1) / kLayoutThreads;
  const int first = tid * per;
  int32_t mine = 0;
  for (int i = 0; i < per; ++i)
    if (first + i < E) mine += s_tot[first + i];
  int32_t incl = mine;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int32_t n = __shfl_up(incl, d);
    if (lane >= d) incl += n;
  }
  if (lane == kWave - 1) s_wave[wave] = incl;
  __syncthreads();
  int32_t before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kLayoutWaves; ++w) {
    before += w < wave ? s_wave[w] : 0;
    total += s_wave[w];
  }
  int32_t run = before + incl - mine;
  for (int i = 0; i < per; ++i) {
    if (first + i < E) {
      s_off[first + i] = capacity > 0 ? (first + i) * capacity : run;
      run += s_tot[first + i];
    }
  }
  __syncthreads();

  // 3. receive rows of this chunk's pairs
#pragma unroll
  for (int i = 0; i < kLayoutItems; ++i) {
    const int64_t p = chunk_base + i * kLayoutThreads + tid;
    if (p >= num_pairs) break;
    const int32_t v = packed[i];
    int32_t s = -1;
    if (v >= 0) {
      const int e = v & ((1 << kExpertBits) - 1);
      const int32_t r = s_pre[e] + (v >> kExpertBits);  // rank inside expert e
      if (capacity == 0 || r < capacity) s = s_off[e] + r;
    }
    slot_idx[p] = s;
    if (recv_src != nullptr && s >= 0) recv_src[s] = (int32_t)p;
  }

  // 4. metadata, once
  if (c == 0) {
    bool over = false;
    for (int e = tid; e < E; e += kLayoutThreads) {
      num_tokens_per_expert[e] = s_tot[e];
      expert_offsets[e] = s_off[e];
      over |= capacity > 0 && s_tot[e] > capacity;
    }
    if (tid == 0) expert_offsets[E] = capacity > 0 ? E * capacity : total;
    const int per_group = E / num_groups;
    for (int g = tid; g < num_groups; g += kLayoutThreads) {
      int32_t s = 0;
      for (int e = g * per_group; e < (g + 1) * per_group; ++e) s += s_tot[e];
      num_tokens_per_group[g] = s;
    }
    int32_t bad = 0;
    for (int cc = tid; cc < num_chunks; cc += kLayoutThreads) bad |= chunk_flags[cc];
    const int any_bad = __syncthreads_or(bad);
    const int any_over = __syncthreads_or(over ? 1 : 0);
    if (tid == 0)
      error_flags[0] = (any_bad ? EP_FLAG_BAD_EXPERT : 0) | (any_over ? EP_FLAG_OVERFLOW : 0);
  }
}

hipError_t launch_layout(const int64_t* topk_idx, const ep_layout_t& L, void* workspace,
                         hipStream_t stream) {
  const int64_t pairs = L.num_tokens * (int64_t)L.num_topk;
  const int64_t chunks = layout_num_chunks(pairs);
  const int32_t E = L.num_experts;
  int32_t* chunk_count = static_cast<int32_t*>(workspace);
  int32_t* chunk_flags = chunk_count + chunks * E;
  int bits = 0;
  while ((1 << bits) < E) ++bits;
  if (chunks > 0) {
    hipLaunchKernelGGL(layout_count_kernel, dim3((unsigned)chunks), dim3(kLayoutThreads), 0,
                       stream, topk_idx, pairs, E, bits, chunk_count, chunk_flags, L.slot_idx);
  }
  hipLaunchKernelGGL(layout_finish_kernel, dim3((unsigned)(chunks > 0 ? chunks : 1)),
                     dim3(kLayoutThreads), 0, stream, pairs, E, L.num_groups, L.capacity,
                     (int32_t)chunks, chunk_count, chunk_flags, L.slot_idx, L.recv_src,
                     L.num_tokens_per_expert, L.expert_offsets, L.num_tokens_per_group,
                     L.error_flags);
  return hipGetLastError();
}

}  // namespace ep
