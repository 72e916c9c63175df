// ep_group.hip -- per-group dedup layout on gfx950.
//
// A variant of the routing layout in which a token is sent once to every group
// of experts (a rank, in a multi-GPU deployment) that holds at least one of its
// top-k experts, instead of once per expert.  The pages count the bytes each
// rank sends and receives ("DeepEP是什麼？…" (yololab.net), section "Load
// Imbalance") and give the per-expert volume batch x top_k x hidden
// ("DeepEP 编址服务深度对抗分析", section 五.2); sending per group cuts that
// volume whenever several of a token's experts share a group.
//
// What it computes (expert e belongs to group e / (E/G)):
//   - a token's entries are the groups it reaches, ascending, padded with -1
//     to kg = min(k, G) entries;
//   - receive rows are group-major and ascending in token inside a group: the
//     ordinary counting-sort layout over the entries, with the G groups in the
//     role of the experts;
//   - each used row carries the token's top-k list masked to the row's group
//     (other entries -1, weight 0), which is what the receiving side needs to
//     run its own experts.
//
// How: three steps on the caller's stream.
//   1. group_table_kernel: one lane per (token, k) pair, tokens in segments
//      of lanes (top-k rounded up to a power of two).  Each lane finds, with
//      shuffles inside its segment, whether its group is the first occurrence
//      in the token and how many distinct groups of the token are smaller:
//      that is the entry's position in the ascending list.  The int64 table
//      lands in the workspace; each workgroup writes one bad-id flag entry
//      (plain stores, no atomics, no memset).
//   2. the layout kernels over that table (E := G, k := kg); they OR the
//      table's flag entries into error_flags.
//   3. group_meta_kernel: lane (t, j) writes column j of every row of token t.
//   4. (optional) group_member_kernel: lane (t, g) writes is_token_in_group
//      [t, g], 1 when g is one of the token's entries in the table.
// Decode-sized batches take all four in one launch (group_layout_small_kernel
// below).
#include "ep_device.h"
#include "ep_internal.h"
#include "ep_scan.h"

namespace ep {

constexpr int kGroupThreads = 256;

struct GroupSeg {
  int32_t seg;               // lanes per token: top-k rounded up to a power of two (<= 64)
  int32_t tokens_per_block;  // kGroupThreads / seg
};

static GroupSeg group_seg(int32_t k) {
  int32_t s = 1;
  while (s < k) s *= 2;
  return GroupSeg{s, kGroupThreads / s};
}

static int64_t group_table_blocks(int64_t T, int32_t k) {
  const GroupSeg g = group_seg(k);
  return (T + g.tokens_per_block - 1) / g.tokens_per_block;
}

static size_t group_table_bytes(int64_t T, int32_t kg) {
  return (((size_t)(T * kg) * sizeof(int64_t) + 255) / 256) * 256;
}

size_t group_layout_workspace_bytes(int64_t T, int32_t k, int32_t G) {
  const int32_t kg = k < G ? k : G;
  return group_table_bytes(T, kg) + layout_workspace_bytes(T * kg, G, group_table_blocks(T, k));
}

__global__ __launch_bounds__(kGroupThreads) void group_table_kernel(
    const int64_t* __restrict__ topk_idx, int64_t T, int32_t k, int32_t E, int32_t per_group,
    int32_t kg, GroupSeg sg, int64_t* __restrict__ table, int32_t* __restrict__ block_flags) {
  const int64_t t = (int64_t)blockIdx.x * sg.tokens_per_block + threadIdx.x / sg.seg;
  const int32_t j = threadIdx.x % sg.seg;
  const bool live = t < T && j < k;
  const int64_t e = live ? topk_idx[t * k + j] : -1;
  const bool valid = e >= 0 && e < E;
  const bool bad = live && !valid && e != -1;
  const int32_t g = valid ? (int32_t)(e / per_group) : -1;

  // Every lane takes part in the shuffles; a segment never straddles a wave.
  const int32_t base = (int32_t)(threadIdx.x % kWave) - j;
  bool first = g >= 0;
  for (int32_t d = 0; d < sg.seg; ++d) {
    const int32_t gd = __shfl(g, base + d);
    if (d < j && gd == g) first = false;
  }
  int32_t rank = 0, ndist = 0;
  for (int32_t d = 0; d < sg.seg; ++d) {
    const int32_t gd = __shfl(g, base + d);
    const int32_t fd = __shfl(first ? 1 : 0, base + d);
    rank += (fd && gd < g) ? 1 : 0;
    ndist += fd;
  }
  // rank < ndist <= kg for a first occurrence; the padding positions
  // [ndist, kg) each have exactly one lane with that j
  if (t < T) {
    if (first) table[t * kg + rank] = g;
    if (j >= ndist && j < kg) table[t * kg + j] = -1;
  }
  const int any_bad = __syncthreads_or(bad ? 1 : 0);
  if (threadIdx.x == 0) block_flags[blockIdx.x] = any_bad ? EP_FLAG_BAD_EXPERT : 0;
}

__global__ __launch_bounds__(kGroupThreads) void group_meta_kernel(
    const int64_t* __restrict__ topk_idx, const float* __restrict__ topk_weights, int64_t T,
    int32_t k, int32_t E, int32_t per_group, int32_t kg, GroupSeg sg,
    const int64_t* __restrict__ table, const int32_t* __restrict__ group_slot,
    int64_t* __restrict__ recv_idx, float* __restrict__ recv_w) {
  const int64_t t = (int64_t)blockIdx.x * sg.tokens_per_block + threadIdx.x / sg.seg;
  const int32_t j = threadIdx.x % sg.seg;
  if (t >= T || j >= k) return;
  const int64_t e = topk_idx[t * k + j];
  const bool valid = e >= 0 && e < E;
  const int32_t g = valid ? (int32_t)(e / per_group) : -1;
  const float w = recv_w != nullptr ? topk_weights[t * k + j] : 0.0f;
  for (int32_t i = 0; i < kg; ++i) {
    const int32_t r = group_slot[t * kg + i];
    if (r < 0) break;  // the entries after the token's groups are all padding
    const bool mine = g >= 0 && (int64_t)g == table[t * kg + i];
    if (recv_idx != nullptr) recv_idx[(int64_t)r * k + j] = mine ? e : -1;
    if (recv_w != nullptr) recv_w[(int64_t)r * k + j] = mine ? w : 0.0f;
  }
}

// is_token_in_group[t, g] for the n = T * G (token, group) cells: a scan of
// the token's kg table entries (its groups ascending, then -1).
__global__ __launch_bounds__(kGroupThreads) void group_member_kernel(
    const int64_t* __restrict__ table, int64_t n, int32_t kg, int32_t G,
    uint8_t* __restrict__ member) {
  for (int64_t c = (int64_t)blockIdx.x * kGroupThreads + threadIdx.x; c < n;
       c += (int64_t)gridDim.x * kGroupThreads) {
    const int64_t t = c / G;
    const int64_t g = c - t * G;
    const int64_t* row = table + t * kg;
    uint8_t hit = 0;
    for (int32_t i = 0; i < kg; ++i) {
      const int64_t v = row[i];
      if (v < 0) break;
      hit |= v == g ? 1 : 0;
    }
    member[c] = hit;
  }
}

// Decode-sized batches (at most kFusedMaxPairs pairs, top-k at most
// kFusedMaxTopk): the whole group layout in one launch, one workgroup per token
// plus a metadata workgroup, the way the fused decode kernel computes the
// expert layout.  Every workgroup reads the whole top-k table and marks, for
// each pair, whether its group is the first occurrence in its token; the LDS
// histogram of those marks over all tokens gives the groups' totals (scanned
// into offsets), and over the tokens before this one the token's row inside
// each of its groups.  The token's workgroup then writes its entries (groups
// ascending, then -1), the receiving side's masked ids and weights for its
// rows, and its is_token_in_group row; the metadata workgroup writes the
// counts, offsets and flags.  Same results as the table, layout and metadata
// kernels.
constexpr int kGroupSmallLanes = 512;
constexpr int kGroupSmallTrips = kFusedMaxPairs / kGroupSmallLanes;

struct GroupSmallArgs {
  const int64_t* topk_idx;
  const float* topk_weights;
  int32_t T, k, E, per_group, G, kg;
  int32_t* slot_idx;
  int32_t* recv_src;
  int32_t* num_tokens_per_expert;
  int32_t* expert_offsets;
  int32_t* num_tokens_per_group;
  int32_t* error_flags;
  int64_t* recv_idx;
  float* recv_w;
  uint8_t* member;
};

__global__ __launch_bounds__(kGroupSmallLanes) void group_layout_small_kernel(GroupSmallArgs a) {
  __shared__ int32_t s_g[kFusedMaxPairs];  // group of every pair, -1 if none
  __shared__ int32_t s_hist[EP_MAX_EXPERTS];
  __shared__ int32_t s_pre[EP_MAX_EXPERTS];
  __shared__ int32_t s_off[EP_MAX_EXPERTS];
  __shared__ int32_t s_wave[kGroupSmallLanes / kWave];
  __shared__ int32_t s_bad;  // the metadata workgroup's bad-id flag
  __shared__ int32_t s_ent[kFusedMaxTopk];   // this token's entries: groups ascending, then -1
  __shared__ int32_t s_row[kFusedMaxTopk];   // their receive rows
  const int tid = threadIdx.x;
  const int32_t k = a.k, G = a.G, kg = a.kg;
  const int32_t P = a.T * k;
  const bool token_block = (int32_t)blockIdx.x < a.T;
  const int32_t t = blockIdx.x;
  const int32_t p0 = token_block ? t * k : 0;

  int64_t tv[kGroupSmallTrips];
#pragma unroll
  for (int i = 0; i < kGroupSmallTrips; ++i) {
    const int32_t p = tid + i * kGroupSmallLanes;
    tv[i] = p < P ? a.topk_idx[p] : -1;
  }
  for (int g = tid; g < G; g += kGroupSmallLanes) {
    s_hist[g] = 0;
    s_pre[g] = 0;
  }
  if (tid == 0) s_bad = 0;
  bool bad = false;
#pragma unroll
  for (int i = 0; i < kGroupSmallTrips; ++i) {
    const int32_t p = tid + i * kGroupSmallLanes;
    if (p < P) {
      const bool ok = tv[i] >= 0 && tv[i] < a.E;
      bad |= !ok && tv[i] != -1;
      s_g[p] = ok ? (int32_t)(tv[i] / a.per_group) : -1;
    }
  }
  __syncthreads();

  // a pair counts once for its group if no earlier pair of its token names it
  // (a fixed trip count over the at most kFusedMaxTopk - 1 earlier pairs, so
  // their LDS reads are all in flight together)
#pragma unroll
  for (int i = 0; i < kGroupSmallTrips; ++i) {
    const int32_t p = tid + i * kGroupSmallLanes;
    if (p < P) {
      const int32_t g = s_g[p];
      const int32_t j = p % k;
      bool first = g >= 0;
#pragma unroll
      for (int d = 1; d < kFusedMaxTopk; ++d)
        if (d <= j) first = first && s_g[p - d] != g;
      if (first) {
        atomicAdd(&s_hist[g], 1);
        if (p < p0) atomicAdd(&s_pre[g], 1);
      }
    }
  }
  // the bad-id flag: one LDS write per wave (the ballot with every lane
  // active), ordered by the scan's barriers
  const bool wave_bad = __ballot(bad) != 0;
  if (!token_block && tid % kWave == 0 && wave_bad) s_bad = 1;
  __syncthreads();
  const int32_t total = block_exclusive_scan(s_hist, s_off, G, s_wave);

  if (!token_block) {
    for (int g = tid; g < G; g += kGroupSmallLanes) {
      a.num_tokens_per_expert[g] = s_hist[g];
      a.expert_offsets[g] = s_off[g];
      a.num_tokens_per_group[g] = s_hist[g];  // the group layout's groups are its experts
    }
    if (tid == 0) {
      a.expert_offsets[G] = total;
      a.error_flags[0] = s_bad ? EP_FLAG_BAD_EXPERT : 0;
    }
    return;
  }

  // this token's entries: pair j's group, if first in the token, goes to entry
  // (number of the token's distinct groups below it); the rest are -1
  if (tid < k) {
    const int32_t j = tid;
    // the token's groups in registers (fixed trip counts, all reads in flight)
    int32_t gt[kFusedMaxTopk];
    bool fq[kFusedMaxTopk];
#pragma unroll
    for (int q = 0; q < kFusedMaxTopk; ++q) gt[q] = q < k ? s_g[p0 + q] : -1;
    int32_t g = -1, rank = 0, ndist = 0;
    bool first = false;
#pragma unroll
    for (int q = 0; q < kFusedMaxTopk; ++q) {
      fq[q] = gt[q] >= 0;
#pragma unroll
      for (int r = 0; r < q; ++r) fq[q] = fq[q] && gt[r] != gt[q];
      g = q == j ? gt[q] : g;
      first = q == j ? fq[q] : first;
    }
#pragma unroll
    for (int q = 0; q < kFusedMaxTopk; ++q) {
      ndist += fq[q] ? 1 : 0;
      rank += (fq[q] && gt[q] < g) ? 1 : 0;
    }
    if (first) {
      const int32_t row = s_off[g] + s_pre[g];
      s_ent[rank] = g;
      s_row[rank] = row;
      a.slot_idx[t * kg + rank] = row;
      if (a.recv_src != nullptr) a.recv_src[row] = t * kg + rank;
    }
    if (j >= ndist && j < kg) {
      s_ent[j] = -1;
      s_row[j] = -1;
      a.slot_idx[t * kg + j] = -1;
    }
  }
  __syncthreads();

  // the receiving side's metadata: column j of each of the token's rows
  if (a.recv_idx != nullptr || a.recv_w != nullptr) {
    for (int32_t l = tid; l < kg * k; l += kGroupSmallLanes) {
      const int32_t i = l / k, j = l - i * k;
      const int32_t row = s_row[i];
      if (row < 0) continue;
      const int32_t g = s_g[p0 + j];
      const bool mine = g >= 0 && g == s_ent[i];
      if (a.recv_idx != nullptr) a.recv_idx[(int64_t)row * k + j] = mine ? a.topk_idx[p0 + j] : -1;
      if (a.recv_w != nullptr)
        a.recv_w[(int64_t)row * k + j] = mine ? a.topk_weights[p0 + j] : 0.0f;
    }
  }
  if (a.member != nullptr) {
    int32_t ent[kFusedMaxTopk];
#pragma unroll
    for (int i = 0; i < kFusedMaxTopk; ++i) ent[i] = i < kg ? s_ent[i] : -1;
    for (int32_t g = tid; g < G; g += kGroupSmallLanes) {
      uint8_t hit = 0;
#pragma unroll
      for (int i = 0; i < kFusedMaxTopk; ++i) hit |= ent[i] == g ? 1 : 0;
      a.member[(int64_t)t * G + g] = hit;
    }
  }
}

hipError_t launch_group_layout(const int64_t* topk_idx, const float* topk_weights, int32_t k,
                               int32_t E, const ep_layout_t& GL, int64_t* recv_idx,
                               float* recv_w, uint8_t* member, void* workspace,
                               hipStream_t stream) {
  const int64_t T = GL.num_tokens;
  const int32_t G = GL.num_experts;
  const int32_t kg = GL.num_topk;
  if (T > 0 && T * k <= kFusedMaxPairs && k <= kFusedMaxTopk) {
    GroupSmallArgs a;
    a.topk_idx = topk_idx;
    a.topk_weights = topk_weights;
    a.T = (int32_t)T;
    a.k = k;
    a.E = E;
    a.per_group = E / G;
    a.G = G;
    a.kg = kg;
    a.slot_idx = GL.slot_idx;
    a.recv_src = GL.recv_src;
    a.num_tokens_per_expert = GL.num_tokens_per_expert;
    a.expert_offsets = GL.expert_offsets;
    a.num_tokens_per_group = GL.num_tokens_per_group;
    a.error_flags = GL.error_flags;
    a.recv_idx = recv_idx;
    a.recv_w = recv_w;
    a.member = member;
    hipLaunchKernelGGL(group_layout_small_kernel, dim3((unsigned)(T + 1)), dim3(kGroupSmallLanes),
                       0, stream, a);
    return hipGetLastError();
  }
  const GroupSeg sg = group_seg(k);
  const int64_t blocks = group_table_blocks(T, k);
  int64_t* table = static_cast<int64_t*>(workspace);
  void* layout_ws = static_cast<char*>(workspace) + group_table_bytes(T, kg);
  if (blocks > 0)
    hipLaunchKernelGGL(group_table_kernel, dim3((unsigned)blocks), dim3(kGroupThreads), 0, stream,
                       topk_idx, T, k, E, E / G, kg, sg, table,
                       layout_extra_flags(GL, layout_ws));
  hipError_t err = launch_layout_ids(table, GL, layout_ws, (int32_t)blocks, stream);
  if (err != hipSuccess) return err;
  if (blocks > 0 && (recv_idx != nullptr || recv_w != nullptr))
    hipLaunchKernelGGL(group_meta_kernel, dim3((unsigned)blocks), dim3(kGroupThreads), 0, stream,
                       topk_idx, topk_weights, T, k, E, E / G, kg, sg, table, GL.slot_idx,
                       recv_idx, recv_w);
  if (blocks > 0 && member != nullptr) {
    const int64_t n = T * G;
    const int64_t want = (n + kGroupThreads - 1) / kGroupThreads;
    const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
    hipLaunchKernelGGL(group_member_kernel, dim3(grid), dim3(kGroupThreads), 0, stream, table, n,
                       kg, G, member);
  }
  return hipGetLastError();
}

}  // namespace ep
