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
//      up to kScanParts lanes per expert with each wave's loads on whole rows
//      of the counts, scans the totals into expert offsets with one DPP sum
//      per wave and writes the receive rows of its chunk.  Workgroup 0 also
//      writes the counts, offsets, group totals and error flags, before its
//      receive rows.
// Two launches run the phases (three for inputs with many chunks, whose bases
// one launch in between computes once, layout_bases_kernel); the ranks travel
// from phase 1 to phase 2 through slot_idx, packed as (rank in chunk) <<
// kExpertBits | expert.  An input of
// one chunk (up to kChunkPairs pairs: decode batches) runs both phases in a
// single workgroup and launch.  (A single cooperative launch with a grid
// barrier was measured slower on MI355X than the two ordinary launches.)
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

static_assert(EP_MAX_EXPERTS <= kLayoutThreads, "phase 2 gives every expert a lane");

// Phase 2 splits the chunks among up to kScanParts lanes per expert, and each
// such lane reads its counts kScanLoads at a time, all of a batch in flight at
// once (one batch covers 16 chunks per part: 64 of them at 256 experts).
constexpr int kScanParts = 64;
constexpr int kScanLoads = 16;

// Where phase 2 finds each expert's totals: already in LDS (an input of one
// chunk), summed from the per-chunk counts by every workgroup, or read from
// the bases one extra launch computed once (inputs whose count matrix every
// workgroup would otherwise re-read at great length).
enum ScanSource { kTotalsInLds = 0, kSumCounts = 1, kReadBases = 2 };

// The extra launch is taken when chunks * chunks * E, the per-chunk counts
// all the finish workgroups would read, exceeds this.
#ifndef EP_LAYOUT_BASES_MIN
#define EP_LAYOUT_BASES_MIN (8 << 20)
#endif
constexpr int64_t kBasesMinWork = EP_LAYOUT_BASES_MIN;

// Phase 2's LDS: per-expert totals, bases inside the expert (chunks before
// this one), offsets and the exclusive prefix of the totals; per-wave sums
// and flags; the parts' partial sums, [part][expert].
struct ScanShared {
  int32_t tot[EP_MAX_EXPERTS];
  int32_t pre[EP_MAX_EXPERTS];
  int32_t off[EP_MAX_EXPERTS];
  int32_t pfx[EP_MAX_EXPERTS + 1];  // exclusive prefix of tot, then the grand total
  int32_t wave[kLayoutWaves];
  int32_t wflag[kLayoutWaves];
  int32_t part_tot[kLayoutThreads];
  int32_t part_pre[kLayoutThreads];
};

size_t layout_workspace_bytes(int64_t pairs, int32_t num_experts, int64_t extra_flags) {
  int64_t chunks = layout_num_chunks(pairs);
  // per-chunk counts, per-chunk flags, extra flags, expert totals
  size_t bytes = (size_t)(chunks * num_experts + chunks + extra_flags + num_experts) *
                 sizeof(int32_t);
  return ((bytes + 255) / 256) * 256 + 256;
}

// Pair handled by item i of the calling lane in chunk c.
__device__ __forceinline__ int64_t pair_of(int64_t c, int i) {
  return c * kChunkPairs + (int64_t)(threadIdx.x / kWave) * kWavePairs + i * kWave +
         threadIdx.x % kWave;
}

// Phase 1 for chunk c: eid[i] = expert of item i (-1 if none), local[i] = its
// rank among the chunk's pairs of that expert.  Writes the chunk's totals (to
// chunk_count[c * E + e]) and its bad-id flag (and, if tot_out is not null,
// the totals to that LDS array too); returns the flag.  wave_flags is
// kLayoutWaves ints of LDS.  On return other waves may still read the
// histograms and wave_flags: a caller that reuses that LDS passes a barrier
// first.
__device__ __forceinline__ int count_chunk(const int64_t* __restrict__ topk_idx,
                                           int64_t num_pairs, int32_t E, int32_t expert_bits,
                                           int64_t c, int32_t* hist, int32_t* wave_flags,
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
  // the wave's bad-id flag, read by every thread after the barrier below
  const bool wave_bad = __ballot(bad) != 0;
  if (lane == 0) wave_flags[wave] = wave_bad ? 1 : 0;

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
  int any_bad = 0;
#pragma unroll
  for (int w = 0; w < kLayoutWaves; ++w) any_bad |= wave_flags[w];
  if (threadIdx.x == 0) chunk_flags[c] = any_bad ? EP_FLAG_BAD_EXPERT : 0;
  __syncthreads();  // the rows now hold each wave's exclusive prefix
#pragma unroll
  for (int i = 0; i < kLayoutItems; ++i)
    if (eid[i] >= 0) local[i] += my_hist[eid[i]];
  return any_bad ? EP_FLAG_BAD_EXPERT : 0;
}

// Expert totals over all chunks (sh.tot), over the chunks before chunk c
// (sh.pre), their exclusive prefix (sh.pfx, with the grand total at [E]) and
// the expert offsets (sh.off).  Lane (part, e) with e fastest sums every
// parts-th chunk's count of expert e straight from memory (so a wave's loads
// cover whole rows of the chunk-major counts) into LDS; lane e then adds its
// expert's parts, and one inclusive DPP sum per wave over those totals gives
// each expert the totals of the wave's earlier experts.  The waves' sums and
// flag bits meet in LDS across one barrier.  kSrc == kTotalsInLds: the totals
// are already in sh.tot (visible to every thread) and no chunk comes before;
// kReadBases: chunk_count holds each chunk's base inside every expert (its
// column prefix) and totals every expert's total.
// Returns the workgroup's flag bits (EP_FLAG_BAD_EXPERT if any thread's
// flag_bits is set, EP_FLAG_OVERFLOW if a padded expert overflows) and sets
// total to the number of routed pairs.
template <int kSrc>
__device__ __forceinline__ int32_t expert_scan(int32_t E, int32_t capacity, int32_t num_chunks,
                                               int64_t c, const int32_t* __restrict__ chunk_count,
                                               const int32_t* __restrict__ totals, ScanShared& sh,
                                               int32_t flag_bits, int32_t& total) {
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const bool serves = tid < E;  // lane e = tid of the scan
  int32_t tot = 0, pre = 0;
  if constexpr (kSrc == kTotalsInLds) {
    if (serves) tot = sh.tot[tid];
  } else if constexpr (kSrc == kReadBases) {
    if (serves) {
      tot = totals[tid];
      pre = chunk_count[c * E + tid];
    }
  } else {
    int parts = kLayoutThreads / E;
    if (parts > kScanParts) parts = kScanParts;
    const int part = tid / E;
    const int e = tid - part * E;
    if (part < parts) {
      // the part's chunks in batches of kScanLoads, every load of a batch in
      // flight at once (a fixed trip count; a plain loop would wait for each).
      // The first batch is straight-line code: most inputs need no other, and
      // a loop around it measured slower for them.
      int32_t pt = 0, pp = 0;
      auto batch = [&](int first) {
        int32_t v[kScanLoads];
#pragma unroll
        for (int i = 0; i < kScanLoads; ++i) {
          const int cc = first + i * parts;
          v[i] = cc < num_chunks ? chunk_count[(int64_t)cc * E + e] : 0;
        }
#pragma unroll
        for (int i = 0; i < kScanLoads; ++i) {
          pt += v[i];
          pp += first + i * parts < c ? v[i] : 0;
        }
      };
      batch(part);
      for (int first = part + kScanLoads * parts; first < num_chunks; first += kScanLoads * parts)
        batch(first);
      sh.part_tot[part * E + e] = pt;
      sh.part_pre[part * E + e] = pp;
    }
    __syncthreads();
    if (serves) {
      for (int q = 0; q < parts; ++q) {
        tot += sh.part_tot[q * E + tid];
        pre += sh.part_pre[q * E + tid];
      }
    }
  }
  const int32_t incl = wave_inclusive_sum(tot);
  const int32_t excl = incl - tot;  // the wave's experts before this one
  const bool over = serves && capacity > 0 && tot > capacity;
  const bool wave_bad = __ballot(flag_bits != 0) != 0;
  const bool wave_over = __ballot(over) != 0;
  const int32_t wave_sum = __builtin_amdgcn_readlane(incl, kWave - 1);
  if (lane == 0) {
    sh.wave[wave] = wave_sum;
    sh.wflag[wave] = (wave_bad ? EP_FLAG_BAD_EXPERT : 0) | (wave_over ? EP_FLAG_OVERFLOW : 0);
  }
  __syncthreads();
  int32_t before = 0, flags = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kLayoutWaves; ++w) {
    before += w < wave ? sh.wave[w] : 0;
    total += sh.wave[w];
    flags |= sh.wflag[w];
  }
  if (serves) {
    const int32_t run = before + excl;
    sh.tot[tid] = tot;
    sh.pre[tid] = pre;
    sh.pfx[tid] = run;
    sh.off[tid] = capacity > 0 ? tid * capacity : run;
  }
  if (tid == 0) sh.pfx[E] = total;
  __syncthreads();
  return flags;
}

// Phase 2 for chunk c, given every chunk's totals in memory (or, for kSrc ==
// kReadBases, every chunk's bases and the experts' totals; for kTotalsInLds
// there is only this chunk, and sh.tot is already set by the caller).  For
// c == 0, flag_bits is the OR of this thread's share of the flag entries (one
// per chunk, then any written by a kernel that prepared the ids), which the
// caller loads at its start so that their latency is hidden.
// Workgroup 0 writes the counts, offsets, group totals and flags as soon as
// the scan is done, before the receive rows, so that no store waits on
// another: the group totals are differences of the exclusive prefix, and the
// flags travel through one word per wave across the scan's own barrier.
template <int kSrc>
__device__ __forceinline__ void finish_chunk(
    int64_t num_pairs, int32_t E, int32_t num_groups, int32_t capacity, int32_t num_chunks,
    int64_t c, const int32_t* __restrict__ chunk_count, const int32_t* __restrict__ totals,
    ScanShared& sh,
    const int32_t (&eid)[kLayoutItems], const int32_t (&local)[kLayoutItems],
    int32_t* __restrict__ slot_idx, int32_t* __restrict__ recv_src,
    int32_t* __restrict__ num_tokens_per_expert, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ num_tokens_per_group, int32_t* __restrict__ error_flags,
    int32_t flag_bits) {
  const int tid = threadIdx.x;

  // 1-2. expert totals, bases inside each expert, offsets, flags
  int32_t total;
  const int32_t flags = expert_scan<kSrc>(E, capacity, num_chunks, c, chunk_count, totals, sh,
                                          flag_bits, total);

  // 3. metadata, once
  if (c == 0) {
    for (int e = tid; e < E; e += kLayoutThreads) {
      num_tokens_per_expert[e] = sh.tot[e];
      expert_offsets[e] = sh.off[e];
    }
    if (tid == 0) {
      expert_offsets[E] = capacity > 0 ? E * capacity : total;
      error_flags[0] = flags;
    }
    const int per_group = E / num_groups;
    for (int g = tid; g < num_groups; g += kLayoutThreads)
      num_tokens_per_group[g] = sh.pfx[(g + 1) * per_group] - sh.pfx[g * per_group];
  }

  // 4. receive rows of this chunk's pairs: every row first, then the stores
  int32_t slot[kLayoutItems];
#pragma unroll
  for (int i = 0; i < kLayoutItems; ++i) {
    slot[i] = -1;
    const int e = eid[i];
    if (e >= 0) {
      const int32_t r = sh.pre[e] + local[i];  // rank inside expert e
      if (capacity == 0 || r < capacity) slot[i] = sh.off[e] + r;
    }
  }
#pragma unroll
  for (int i = 0; i < kLayoutItems; ++i) {
    const int64_t p = pair_of(c, i);
    if (p < num_pairs) {
      slot_idx[p] = slot[i];
      if (recv_src != nullptr && slot[i] >= 0) recv_src[slot[i]] = (int32_t)p;
    }
  }
}

struct LayoutArgs {
  const int64_t* topk_idx;
  int64_t num_pairs;
  int32_t num_experts, expert_bits, num_groups, capacity, num_chunks, num_flags;
  int32_t* chunk_count;
  int32_t* chunk_flags;
  int32_t* totals;  // every expert's total, when the bases launch runs
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
  __shared__ int32_t wave_flags[kLayoutWaves];
  if ((int32_t)blockIdx.x >= a.num_chunks) {
    warm_slab(a.warm, 0, a.warm_split, (int32_t)blockIdx.x - a.num_chunks, a.warm_blocks);
    return;
  }
  int32_t eid[kLayoutItems], local[kLayoutItems];
  count_chunk(a.topk_idx, a.num_pairs, a.num_experts, a.expert_bits, blockIdx.x, hist,
              wave_flags, a.chunk_count, a.chunk_flags, nullptr, eid, local);
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
template <int kSrc>
__global__ __launch_bounds__(kLayoutThreads) void layout_finish_kernel(LayoutArgs a) {
  __shared__ ScanShared sh;
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
  finish_chunk<kSrc>(a.num_pairs, a.num_experts, a.num_groups, a.capacity, a.num_chunks,
                     blockIdx.x, a.chunk_count, a.totals, sh, eid, local, a.slot_idx,
                     a.recv_src, a.num_tokens_per_expert, a.expert_offsets,
                     a.num_tokens_per_group, a.error_flags, flag_bits);
}

// Between the two phases, for inputs with many chunks: each expert's total and
// each chunk's base inside it (the exclusive prefix of the expert's counts
// over the chunks), computed once instead of by every finish workgroup.  One
// workgroup per kWave experts, one lane per expert; wave w takes a contiguous
// block of chunks, sums it (each load instruction reads a run of a row of the
// chunk-major counts), the block sums meet in LDS, and the wave then writes
// its chunks' bases over their counts (no other wave reads those rows).
__global__ __launch_bounds__(kLayoutThreads) void layout_bases_kernel(LayoutArgs a) {
  __shared__ int32_t s_sum[kLayoutWaves][kWave];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int32_t E = a.num_experts;
  const int32_t C = a.num_chunks;
  const int e = (int)blockIdx.x * kWave + lane;
  const bool serves = e < E;
  const int32_t per = (C + kLayoutWaves - 1) / kLayoutWaves;
  const int32_t lo = wave * per;
  const int32_t hi = lo + per < C ? lo + per : C;
  int32_t* col = a.chunk_count + e;
  int32_t sum = 0;
  if (serves) {
    for (int32_t first = lo; first < hi; first += kScanLoads) {
      int32_t v[kScanLoads];
#pragma unroll
      for (int i = 0; i < kScanLoads; ++i)
        v[i] = first + i < hi ? col[(int64_t)(first + i) * E] : 0;
#pragma unroll
      for (int i = 0; i < kScanLoads; ++i) sum += v[i];
    }
  }
  s_sum[wave][lane] = sum;
  __syncthreads();
  int32_t run = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kLayoutWaves; ++w) {
    run += w < wave ? s_sum[w][lane] : 0;
    total += s_sum[w][lane];
  }
  if (!serves) return;
  if (wave == 0) a.totals[e] = total;
  for (int32_t first = lo; first < hi; first += kScanLoads) {
    int32_t v[kScanLoads];
#pragma unroll
    for (int i = 0; i < kScanLoads; ++i)
      v[i] = first + i < hi ? col[(int64_t)(first + i) * E] : 0;
#pragma unroll
    for (int i = 0; i < kScanLoads; ++i) {
      if (first + i < hi) col[(int64_t)(first + i) * E] = run;
      run += v[i];
    }
  }
}

// Inputs of at most one chunk (decode-sized batches): both phases in one
// workgroup and one launch; the totals stay in LDS.
__global__ __launch_bounds__(kLayoutThreads) void layout_single_kernel(LayoutArgs a) {
  __shared__ int32_t hist[kLayoutWaves * EP_MAX_EXPERTS];
  __shared__ int32_t wave_flags[kLayoutWaves];
  __shared__ ScanShared sh;
  int32_t eid[kLayoutItems], local[kLayoutItems];
  // entries after the chunk's own (written by a kernel that prepared the ids)
  const int32_t extra_bits = load_flag_bits(a.chunk_flags, 1, a.num_flags);
  const int bad = count_chunk(a.topk_idx, a.num_pairs, a.num_experts, a.expert_bits, 0, hist,
                              wave_flags, a.chunk_count, a.chunk_flags, sh.tot, eid, local);
  __syncthreads();  // the totals in sh.tot, for every thread
  finish_chunk<kTotalsInLds>(a.num_pairs, a.num_experts, a.num_groups, a.capacity, 1, 0,
                             a.chunk_count, a.totals,
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
  a.totals = a.chunk_flags + a.num_flags;
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
  const unsigned finish_blocks = (unsigned)((chunks > 0 ? chunks : 1) + a.warm_blocks);
  if (chunks * chunks * L.num_experts > kBasesMinWork) {
    hipLaunchKernelGGL(layout_bases_kernel, dim3((unsigned)((L.num_experts + kWave - 1) / kWave)),
                       dim3(kLayoutThreads), 0, stream, a);
    hipLaunchKernelGGL(layout_finish_kernel<kReadBases>, dim3(finish_blocks), dim3(kLayoutThreads),
                       0, stream, a);
  } else {
    hipLaunchKernelGGL(layout_finish_kernel<kSumCounts>, dim3(finish_blocks), dim3(kLayoutThreads),
                       0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace ep
