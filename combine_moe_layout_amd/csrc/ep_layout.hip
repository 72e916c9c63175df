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
// The pairs are cut into chunks of kChunkPairs; one workgroup owns a chunk.
//   phase 1 (count): each wave walks its kWavePairs pairs in order, 64 at a time;
//      lanes that name the same expert find each other with one ballot per
//      expert-id bit, the lowest such lane bumps the wave's private LDS
//      histogram, and every lane's rank is the histogram value plus the
//      number of lower peer lanes.  No atomics, so the ranks are
//      deterministic.  The chunk's per-expert totals go to the workspace.
//   phase 2 (finish): each workgroup sums the chunk totals of earlier chunks
//      (its base inside each expert) and of all chunks (the expert totals),
//      staging the whole count matrix in LDS with every load in flight at once
//      when it fits, scans the totals into expert offsets and writes the
//      receive rows of its chunk.  Workgroup 0 also writes the counts,
//      offsets, group totals and error flags.
// Two launches run the phases; the ranks travel from one to the other through
// slot_idx, packed as (rank in chunk) << kExpertBits | expert.  An input of
// one chunk (up to kChunkPairs pairs: decode batches) runs both phases in a
// single workgroup and launch.  (A single cooperative launch with a grid
// barrier was measured slower on MI355X than the two ordinary launches.)
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

// Per-chunk counts up to this many ints are staged whole in LDS (all loads in
// flight at once); larger matrices are summed from memory.
constexpr int kStageInts = 16384;
static_assert(kStageInts % (4 * kLayoutThreads) == 0, "staging is done in whole 16-byte batches");
static_assert(kStageInts >= kLayoutWaves * EP_MAX_EXPERTS,
              "phase-1 histograms alias the staging area");

struct LayoutShared {
  int32_t counts[kStageInts];  // phase 2; phase 1 uses the front as kLayoutWaves histograms
  int32_t tot[EP_MAX_EXPERTS];
  int32_t pre[EP_MAX_EXPERTS];
  int32_t off[EP_MAX_EXPERTS];
  int32_t wave[kLayoutWaves];
};

size_t layout_workspace_bytes(int64_t pairs, int32_t num_experts, int64_t extra_flags) {
  int64_t chunks = layout_num_chunks(pairs);
  size_t bytes = (size_t)(chunks * num_experts + chunks + extra_flags) * sizeof(int32_t);
  return ((bytes + 255) / 256) * 256 + 256;
}

// Pair handled by item i of the calling lane in chunk c.
__device__ __forceinline__ int64_t pair_of(int64_t c, int i) {
  return c * kChunkPairs + (int64_t)(threadIdx.x / kWave) * kWavePairs + i * kWave +
         threadIdx.x % kWave;
}

// Phase 1 for chunk c: eid[i] = expert of item i (-1 if none), local[i] = its
// rank among the chunk's pairs of that expert.  Writes the chunk's totals and
// its bad-id flag (and, if tot_out is not null, the totals to that LDS array
// too); returns the flag.  Ends with the histograms no longer needed.
__device__ __forceinline__ int count_chunk(const int64_t* __restrict__ topk_idx,
                                           int64_t num_pairs, int32_t E, int32_t expert_bits,
                                           int64_t c, int32_t* hist,
                                           int32_t* __restrict__ chunk_count,
                                           int32_t* __restrict__ chunk_flags, int32_t* tot_out,
                                           int32_t (&eid)[kLayoutItems],
                                           int32_t (&local)[kLayoutItems]) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  int32_t* my_hist = hist + wave * EP_MAX_EXPERTS;

  // Each wave owns one histogram row; LDS operations of one wave complete in
  // order, so the row needs no block barrier until other waves read it.
  for (int e = lane; e < E; e += kWave) my_hist[e] = 0;

  bool bad = false;
#pragma unroll
  for (int i = 0; i < kLayoutItems; ++i) {
    const int64_t p = pair_of(c, i);
    const int64_t v = p < num_pairs ? topk_idx[p] : -1;
    const bool ok = v >= 0 && v < E;
    bad |= !ok && v != -1;
    eid[i] = ok ? (int32_t)v : -1;
  }

  const uint64_t below_me = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
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
    if (valid) base = my_hist[e];
    if (valid && lower == 0) my_hist[e] = base + __popcll(peers);
    local[i] = base + lower;
  }
  __syncthreads();

  // Chunk totals per expert; each wave's row becomes its exclusive prefix.
  for (int e = threadIdx.x; e < E; e += kLayoutThreads) {
    int32_t run = 0;
#pragma unroll
    for (int w = 0; w < kLayoutWaves; ++w) {
      const int32_t h = hist[w * EP_MAX_EXPERTS + e];
      hist[w * EP_MAX_EXPERTS + e] = run;
      run += h;
    }
    chunk_count[c * E + e] = run;
    if (tot_out != nullptr) tot_out[e] = run;
  }
  const int any_bad = __syncthreads_or(bad ? 1 : 0);
  if (threadIdx.x == 0) chunk_flags[c] = any_bad ? EP_FLAG_BAD_EXPERT : 0;
#pragma unroll
  for (int i = 0; i < kLayoutItems; ++i)
    if (eid[i] >= 0) local[i] += my_hist[eid[i]];
  __syncthreads();
  return any_bad ? EP_FLAG_BAD_EXPERT : 0;
}

// Expert totals over all chunks (sh.tot) and over the chunks before chunk c
// (sh.pre), from the per-chunk totals in memory.
__device__ __forceinline__ void chunk_totals(int32_t E, int32_t num_chunks, int64_t c,
                                             const int32_t* __restrict__ chunk_count,
                                             LayoutShared& sh) {
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kLayoutThreads) {
    sh.tot[e] = 0;
    sh.pre[e] = 0;
  }
  const int64_t matrix = (int64_t)num_chunks * E;
  const int lanes_per_expert = E >= kLayoutThreads ? 1 : kLayoutThreads / E;
  const int span = E >= kLayoutThreads ? E : E * lanes_per_expert;
  if (matrix <= kStageInts) {
    // 16-byte loads, a fixed number per thread, all issued before the first
    // is waited for (the workspace is 256-byte aligned)
    constexpr int kBatch = kStageInts / 4 / kLayoutThreads;
    const int n4 = (int)(matrix / 4);
    const int4* src4 = reinterpret_cast<const int4*>(chunk_count);
    int4* dst4 = reinterpret_cast<int4*>(sh.counts);
    if (n4 > 0) {
      int4 r[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int i = tid + b * kLayoutThreads;
        r[b] = src4[i < n4 ? i : n4 - 1];  // unconditional, so r stays in registers
      }
      // Only whole quads of the matrix are stored here.  Quad n4 holds the
      // last matrix % 4 entries, which the loop below fills from other
      // lanes; a store of the clamped copy to that quad from another wave
      // would race with it.
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int i = tid + b * kLayoutThreads;
        if (i < n4) dst4[i] = r[b];
      }
    }
    for (int i = 4 * n4 + tid; i < matrix; i += kLayoutThreads) sh.counts[i] = chunk_count[i];
    __syncthreads();
    for (int idx = tid; idx < span; idx += kLayoutThreads) {
      const int e = idx % E;
      const int sub = idx / E;
      int32_t tot = 0, pre = 0;
      for (int cc = sub; cc < num_chunks; cc += lanes_per_expert) {
        const int32_t v = sh.counts[cc * E + e];
        tot += v;
        pre += cc < c ? v : 0;
      }
      atomicAdd(&sh.tot[e], tot);
      atomicAdd(&sh.pre[e], pre);
    }
  } else {
    __syncthreads();
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
      atomicAdd(&sh.tot[e], tot);
      atomicAdd(&sh.pre[e], pre);
    }
  }
  __syncthreads();
}

// Phase 2 for chunk c, given every chunk's totals in memory.  kSingleChunk:
// there is only this chunk, and sh.tot and sh.pre are already set by the
// caller.  For c == 0, flag_bits is the OR of this thread's share of the flag
// entries (one per chunk, then any written by a kernel that prepared the ids),
// which the caller loads at its start so that their latency is hidden.
template <bool kSingleChunk>
__device__ __forceinline__ void finish_chunk(
    int64_t num_pairs, int32_t E, int32_t num_groups, int32_t capacity, int32_t num_chunks,
    int64_t c, const int32_t* __restrict__ chunk_count, LayoutShared& sh,
    const int32_t (&eid)[kLayoutItems], const int32_t (&local)[kLayoutItems],
    int32_t* __restrict__ slot_idx, int32_t* __restrict__ recv_src,
    int32_t* __restrict__ num_tokens_per_expert, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ num_tokens_per_group, int32_t* __restrict__ error_flags,
    int32_t flag_bits) {
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;

  // 1. expert totals over all chunks, and over the chunks before this one
  if constexpr (!kSingleChunk) chunk_totals(E, num_chunks, c, chunk_count, sh);

  // 2. exclusive scan of the totals (contiguous mode) -> expert offsets
  const int per = (E + kLayoutThreads - 1) / kLayoutThreads;
  const int first = tid * per;
  int32_t mine = 0;
  for (int i = 0; i < per; ++i)
    if (first + i < E) mine += sh.tot[first + i];
  int32_t incl = mine;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int32_t n = __shfl_up(incl, d);
    if (lane >= d) incl += n;
  }
  if (lane == kWave - 1) sh.wave[wave] = incl;
  __syncthreads();
  int32_t before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kLayoutWaves; ++w) {
    before += w < wave ? sh.wave[w] : 0;
    total += sh.wave[w];
  }
  int32_t run = before + incl - mine;
  for (int i = 0; i < per; ++i) {
    if (first + i < E) {
      sh.off[first + i] = capacity > 0 ? (first + i) * capacity : run;
      run += sh.tot[first + i];
    }
  }
  __syncthreads();

  // 3. receive rows of this chunk's pairs
#pragma unroll
  for (int i = 0; i < kLayoutItems; ++i) {
    const int64_t p = pair_of(c, i);
    if (p < num_pairs) {
      int32_t s = -1;
      const int e = eid[i];
      if (e >= 0) {
        const int32_t r = sh.pre[e] + local[i];  // rank inside expert e
        if (capacity == 0 || r < capacity) s = sh.off[e] + r;
      }
      slot_idx[p] = s;
      if (recv_src != nullptr && s >= 0) recv_src[s] = (int32_t)p;
    }
  }

  // 4. metadata, once
  if (c == 0) {
    bool over = false;
    for (int e = tid; e < E; e += kLayoutThreads) {
      num_tokens_per_expert[e] = sh.tot[e];
      expert_offsets[e] = sh.off[e];
      over |= capacity > 0 && sh.tot[e] > capacity;
    }
    if (tid == 0) expert_offsets[E] = capacity > 0 ? E * capacity : total;
    const int per_group = E / num_groups;
    for (int g = tid; g < num_groups; g += kLayoutThreads) {
      int32_t s = 0;
      for (int e = g * per_group; e < (g + 1) * per_group; ++e) s += sh.tot[e];
      num_tokens_per_group[g] = s;
    }
    const int any_bad = __syncthreads_or(flag_bits);
    const int any_over = __syncthreads_or(over ? 1 : 0);
    if (tid == 0)
      error_flags[0] = (any_bad ? EP_FLAG_BAD_EXPERT : 0) | (any_over ? EP_FLAG_OVERFLOW : 0);
  }
}

struct LayoutArgs {
  const int64_t* topk_idx;
  int64_t num_pairs;
  int32_t num_experts, expert_bits, num_groups, capacity, num_chunks, num_flags;
  int32_t* chunk_count;
  int32_t* chunk_flags;
  int32_t* slot_idx;
  int32_t* recv_src;
  int32_t* num_tokens_per_expert;
  int32_t* expert_offsets;
  int32_t* num_tokens_per_group;
  int32_t* error_flags;
  // Reading the dispatch source ahead (null when not asked for): workgroups
  // past the layout's own read 16-byte vectors [0, warm_split) of `warm`
  // during the count launch and [warm_split, warm_vecs) during the finish
  // launch, warm_blocks workgroups per launch.
  const u32x4* warm;
  int64_t warm_vecs, warm_split;
  int32_t warm_blocks;
};

// Workgroup `worker` of `workers` reads its share of vectors [begin, end) of
// src with ordinary loads and discards them.  Ordinary loads allocate in the
// last-level cache (the MALL, 256 MB on MI355X), so a kernel that reads the
// same rows next finds them there; the layout's few dozen latency-bound
// workgroups leave HBM idle, and this fills that time.  Each wave instruction
// covers 1 KiB of consecutive vectors; kWarmDepth loads per lane are in flight
// at once.
constexpr int kWarmDepth = 8;

// Not inlined: inlined into the finish kernel it took that kernel from 44 to 84
// VGPRs (5 waves per SIMD instead of 8); as a call it costs no registers there.
__device__ __noinline__ void warm_slab(const u32x4* __restrict__ src, int64_t begin, int64_t end,
                                       int32_t worker, int32_t workers) {
  const int64_t per = (end - begin + workers - 1) / workers;
  const int64_t lo = begin + (int64_t)worker * per;
  const int64_t hi = lo + per < end ? lo + per : end;
  uint32_t acc = 0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += (int64_t)kLayoutThreads * kWarmDepth) {
    u32x4 v[kWarmDepth];
#pragma unroll
    for (int u = 0; u < kWarmDepth; ++u) {
      const int64_t j = i + (int64_t)u * kLayoutThreads;
      v[u] = j < hi ? src[j] : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kWarmDepth; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // The loaded values are used by nothing; an empty asm statement that takes
  // their combination as a register input keeps the loads from being dropped.
  __asm__ volatile("" : : "v"(acc));
}

// Phase 1: ranks leave packed through slot_idx.
__global__ __launch_bounds__(kLayoutThreads) void layout_count_kernel(LayoutArgs a) {
  __shared__ int32_t hist[kLayoutWaves * EP_MAX_EXPERTS];
  if ((int32_t)blockIdx.x >= a.num_chunks) {
    warm_slab(a.warm, 0, a.warm_split, (int32_t)blockIdx.x - a.num_chunks, a.warm_blocks);
    return;
  }
  int32_t eid[kLayoutItems], local[kLayoutItems];
  count_chunk(a.topk_idx, a.num_pairs, a.num_experts, a.expert_bits, blockIdx.x, hist,
              a.chunk_count, a.chunk_flags, nullptr, eid, local);
#pragma unroll
  for (int i = 0; i < kLayoutItems; ++i) {
    const int64_t p = pair_of(blockIdx.x, i);
    if (p < a.num_pairs) a.slot_idx[p] = eid[i] >= 0 ? ((local[i] << kExpertBits) | eid[i]) : -1;
  }
}

// OR of this thread's share of flag entries [first, num_flags).
__device__ __forceinline__ int32_t load_flag_bits(const int32_t* __restrict__ chunk_flags,
                                                  int32_t first, int32_t num_flags) {
  int32_t bits = 0;
  for (int32_t cc = first + threadIdx.x; cc < num_flags; cc += kLayoutThreads)
    bits |= chunk_flags[cc];
  return bits;
}

// Phase 2 (also the whole layout when there are no pairs).
__global__ __launch_bounds__(kLayoutThreads) void layout_finish_kernel(LayoutArgs a) {
  __shared__ LayoutShared sh;
  const int32_t own = a.num_chunks > 0 ? a.num_chunks : 1;
  if ((int32_t)blockIdx.x >= own) {
    warm_slab(a.warm, a.warm_split, a.warm_vecs, (int32_t)blockIdx.x - own, a.warm_blocks);
    return;
  }
  int32_t eid[kLayoutItems], local[kLayoutItems];
  // workgroup 0 reports the flags; their loads are issued first and used last
  const int32_t flag_bits = blockIdx.x == 0 ? load_flag_bits(a.chunk_flags, 0, a.num_flags) : 0;
#pragma unroll
  for (int i = 0; i < kLayoutItems; ++i) {
    const int64_t p = pair_of(blockIdx.x, i);
    const int32_t v = p < a.num_pairs ? a.slot_idx[p] : -1;
    eid[i] = v >= 0 ? (v & ((1 << kExpertBits) - 1)) : -1;
    local[i] = v >= 0 ? (v >> kExpertBits) : 0;
  }
  finish_chunk<false>(a.num_pairs, a.num_experts, a.num_groups, a.capacity, a.num_chunks,
                      blockIdx.x, a.chunk_count, sh, eid, local, a.slot_idx, a.recv_src,
                      a.num_tokens_per_expert, a.expert_offsets, a.num_tokens_per_group,
                      a.error_flags, flag_bits);
}

// Inputs of at most one chunk (decode-sized batches): both phases in one
// workgroup and one launch; the totals stay in LDS.
__global__ __launch_bounds__(kLayoutThreads) void layout_single_kernel(LayoutArgs a) {
  __shared__ LayoutShared sh;
  int32_t eid[kLayoutItems], local[kLayoutItems];
  // entries after the chunk's own (written by a kernel that prepared the ids)
  const int32_t extra_bits = load_flag_bits(a.chunk_flags, 1, a.num_flags);
  const int bad = count_chunk(a.topk_idx, a.num_pairs, a.num_experts, a.expert_bits, 0,
                              sh.counts, a.chunk_count, a.chunk_flags, sh.tot, eid, local);
  for (int e = threadIdx.x; e < a.num_experts; e += kLayoutThreads) sh.pre[e] = 0;
  __syncthreads();
  finish_chunk<true>(a.num_pairs, a.num_experts, a.num_groups, a.capacity, 1, 0, a.chunk_count,
                     sh, eid, local, a.slot_idx, a.recv_src, a.num_tokens_per_expert,
                     a.expert_offsets, a.num_tokens_per_group, a.error_flags, bad | extra_bits);
}

hipError_t launch_layout(const int64_t* topk_idx, const ep_layout_t& L, void* workspace,
                         hipStream_t stream) {
  return launch_layout_ids(topk_idx, L, workspace, 0, stream);
}

hipError_t launch_layout_warm(const int64_t* topk_idx, const ep_layout_t& L, void* workspace,
                              const void* warm, size_t warm_bytes, hipStream_t stream) {
  return launch_layout_ids(topk_idx, L, workspace, 0, stream, warm, warm_bytes);
}

int32_t* layout_extra_flags(const ep_layout_t& L, void* workspace) {
  const int64_t chunks = layout_num_chunks(L.num_tokens * (int64_t)L.num_topk);
  return static_cast<int32_t*>(workspace) + chunks * L.num_experts + chunks;
}

hipError_t launch_layout_ids(const int64_t* topk_idx, const ep_layout_t& L, void* workspace,
                             int32_t extra_flags, hipStream_t stream, const void* warm,
                             size_t warm_bytes) {
  LayoutArgs a;
  a.topk_idx = topk_idx;
  a.num_pairs = L.num_tokens * (int64_t)L.num_topk;
  const int64_t chunks = layout_num_chunks(a.num_pairs);
  a.num_experts = L.num_experts;
  int bits = 0;
  while ((1 << bits) < L.num_experts) ++bits;
  a.expert_bits = bits;
  a.num_groups = L.num_groups;
  a.capacity = L.capacity;
  a.num_chunks = (int32_t)chunks;
  a.num_flags = (int32_t)chunks + extra_flags;
  a.chunk_count = static_cast<int32_t*>(workspace);
  a.chunk_flags = a.chunk_count + chunks * L.num_experts;
  a.slot_idx = L.slot_idx;
  a.recv_src = L.recv_src;
  a.num_tokens_per_expert = L.num_tokens_per_expert;
  a.expert_offsets = L.expert_offsets;
  a.num_tokens_per_group = L.num_tokens_per_group;
  a.error_flags = L.error_flags;
  // a larger source: its first kWarmMaxBytes, which dispatch reads first
  const size_t warm_span = warm_bytes < kWarmMaxBytes ? warm_bytes : kWarmMaxBytes;
  const bool warming = warm != nullptr && warm_span >= 16;
  a.warm = static_cast<const u32x4*>(warm);
  a.warm_vecs = warming ? (int64_t)(warm_span / 16) : 0;
  a.warm_split = a.warm_vecs * kWarmCountShare / 100;
  a.warm_blocks = warming ? kWarmBlocks : 0;

  // Batches the fused decode kernel takes: its layout-only form, one workgroup
  // per token.
  if (fused_layout_dispatch_fits(L))
    return launch_layout_small(topk_idx, L, a.chunk_flags + chunks, extra_flags, stream);
  if (chunks == 1) {
    hipLaunchKernelGGL(layout_single_kernel, dim3(1), dim3(kLayoutThreads), 0, stream, a);
    return hipGetLastError();
  }
  if (chunks > 0)
    hipLaunchKernelGGL(layout_count_kernel, dim3((unsigned)(chunks + a.warm_blocks)),
                       dim3(kLayoutThreads), 0, stream, a);
  hipLaunchKernelGGL(layout_finish_kernel, dim3((unsigned)((chunks > 0 ? chunks : 1) + a.warm_blocks)),
                     dim3(kLayoutThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ep
