/*
 * ep.h -- C ABI of libep.so: MoE token dispatch and combine on one MI355X
 * (gfx950), as hand-written HIP kernels.
 *
 * The method (sources are web pages, cited by title and section):
 *   - "DeepEP是什麼？MoE Dispatch、Combine、All-to-all與V2架構" (yololab.net),
 *     section "MoE為什麼需要All-to-all？", stage table: dispatch takes the
 *     tokens, their top-k expert index and weights and produces hidden states
 *     arranged by expert; combine takes the expert outputs and the routing
 *     weights and produces results in the original token order, with a
 *     reduction.  Section "Load Imbalance": per-expert token counts and per-rank
 *     send/receive volume are the quantities to track.  Section "ElasticBuffer":
 *     buffers are sized from max tokens, top-k, hidden and EP degree, and an
 *     overflow needs a drop policy.  Section "FP8與低精度通訊": FP8 dispatch
 *     carries scales whose granularity and format must be checked.
 *   - "DeepEP 编址服务深度对抗分析" (backyes.github.io), section 五.2: each of
 *     dispatch and combine moves batch x top_k x hidden x sizeof(dtype), i.e.
 *     one receive row per (token, k) pair.
 *   - DeepEP v2 release notes (donniechu.com), section "Số liệu kỹ thuật": the
 *     DeepSeek-V3-style test case uses FP8 dispatch and BF16 combine; section
 *     "Có gì mới trong v2": an EPHandle carries orchestration state between
 *     calls (ep_layout_t plays that role here).
 *
 * One GPU holds every expert.  The G logical groups are the expert blocks a
 * real EP rank would own (experts [g*E/G, (g+1)*E/G)), laid out as partitions
 * of one receive buffer.
 *
 * Conventions for every call:
 *   - Ownership: the caller allocates and frees all device memory (inputs,
 *     outputs, layout arrays, workspace).  The library allocates nothing and
 *     keeps no mutable global state; calls on different buffers may run
 *     concurrently.  The one exception is ep_get_layout_noalloc, whose
 *     workspace is a fixed array the library holds on each GPU.
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the default
 *     stream).  Calls only enqueue work and never synchronise; outputs and
 *     error flags are valid once the stream has been synchronised.
 *   - Layout: every array is dense row-major.  Token rows have stride
 *     `hidden` elements; pointers to row data must be 16-byte aligned.
 *   - Errors checked on the host return a negative status before anything is
 *     enqueued.  Errors found on the device are reported in
 *     layout->error_flags (EP_FLAG_*); the offending pairs are skipped and no
 *     memory outside the caller's buffers is touched.
 */
#ifndef EP_H
#define EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum ep_status {
    EP_OK = 0,
    EP_ERR_NULL = -1,      /* a required pointer is NULL */
    EP_ERR_SHAPE = -2,     /* a size is out of range or sizes disagree */
    EP_ERR_ALIGN = -3,     /* a buffer is not aligned as its call requires */
    EP_ERR_WORKSPACE = -4, /* workspace smaller than its size query reports */
    EP_ERR_LAUNCH = -5,    /* the HIP runtime reported an error when launching */
    EP_ERR_DTYPE = -6      /* unknown receive dtype */
};

/* Receive-buffer element types for ep_dispatch. */
enum ep_dtype {
    EP_BF16 = 0,          /* bf16 rows, a bit copy of x */
    EP_FP8_E4M3 = 1,      /* OCP FP8 E4M3 codes + one fp32 scale per 128 channels */
    EP_FP8_E4M3_POW2 = 2, /* as EP_FP8_E4M3, with each scale a power of two (see ep_dispatch) */
    EP_MXFP8_E4M3 = 3,    /* OCP MXFP8: E4M3 codes + one E8M0 scale byte per 32 channels */
    EP_F16 = 4            /* fp16 rows: x is fp16 and the rows are a bit copy of it */
};

/* Flags OR-ed into the receive dtype.
 * EP_SCALES_MN_MAJOR: with an FP8 dtype (EP_FP8_E4M3, EP_FP8_E4M3_POW2 or
 *   EP_MXFP8_E4M3) of ep_dispatch / ep_layout_dispatch, the scales are stored
 *   transposed (MN-major), see ep_dispatch.
 * EP_READ_X_AHEAD: ep_layout_dispatch only, any dtype; see that call. */
enum ep_dtype_flag {
    EP_SCALES_MN_MAJOR = 0x100,
    EP_READ_X_AHEAD = 0x200
};

/* Bits of layout->error_flags, written by ep_get_layout. */
enum ep_flag {
    EP_FLAG_BAD_EXPERT = 1, /* some topk_idx entry is outside [-1, num_experts) */
    EP_FLAG_OVERFLOW = 2    /* padded mode: some expert received more than capacity pairs */
};

/* Limits checked by the host-side validation. */
#define EP_MAX_EXPERTS 1024
#define EP_MAX_TOPK 64
#define EP_MAX_HIDDEN 65536

/*
 * The routing layout: the handle that ep_get_layout fills and ep_dispatch /
 * ep_combine consume.  Size fields are set by ep_layout_init; the caller then
 * points the array fields at device memory it owns:
 *   num_tokens_per_expert [E]   pairs routed to each expert (unclamped demand)
 *   expert_offsets        [E+1] first receive row of each expert; [E] = rows used
 *                               (contiguous) or E*capacity (padded)
 *   num_tokens_per_group  [G]   pairs routed to each group of E/G experts
 *   slot_idx              [T*k] receive row of pair p = t*k + j, or -1 if the
 *                               pair is unrouted, names a bad expert, or was
 *                               dropped for capacity
 *   recv_src              [R]   optional (NULL to skip): pair index p stored in
 *                               each used receive row; unused rows untouched
 *   error_flags           [1]   EP_FLAG_* bits of the latest ep_get_layout call
 * Receive rows: R = T*k (contiguous, capacity == 0) or E*capacity (padded).
 */
typedef struct ep_layout {
    int64_t num_tokens;    /* T */
    int64_t num_recv_rows; /* R */
    int32_t num_topk;      /* k */
    int32_t num_experts;   /* E */
    int32_t num_groups;    /* G, divides E */
    int32_t capacity;      /* 0: contiguous; > 0: rows per expert (padded) */
    int32_t* num_tokens_per_expert;
    int32_t* expert_offsets;
    int32_t* num_tokens_per_group;
    int32_t* slot_idx;
    int32_t* recv_src;
    int32_t* error_flags;
} ep_layout_t;

/*
 * Fill the size fields of *layout (and set every array pointer to NULL).
 * Requires 0 <= num_tokens, 1 <= num_topk <= EP_MAX_TOPK,
 * 1 <= num_experts <= EP_MAX_EXPERTS, 1 <= num_groups, num_experts %
 * num_groups == 0, 0 <= capacity, num_tokens*num_topk and R below 2^31.
 * Returns EP_OK, EP_ERR_NULL or EP_ERR_SHAPE.  Host only.
 */
int ep_layout_init(ep_layout_t* layout, int64_t num_tokens, int32_t num_topk,
                   int32_t num_experts, int32_t num_groups, int32_t capacity);

/* R for these sizes (T*k, or E*capacity when capacity > 0); -1 if invalid.  Host only. */
int64_t ep_num_recv_rows(int64_t num_tokens, int32_t num_topk, int32_t num_experts,
                         int32_t capacity);

/* Bytes of device workspace ep_get_layout needs for these sizes: per-chunk
 * expert counts and flags and the experts' totals, sized from the batch's
 * tokens, top-k and experts as
 * the pages size their buffers ([yololab] "ElasticBuffer": buffer capacity
 * follows max tokens, top-k, hidden and EP degree).  Host only. */
size_t ep_layout_workspace_bytes(int64_t num_tokens, int32_t num_topk, int32_t num_experts);

/*
 * Routing layout ([yololab] stage table, dispatch row: the sort by expert;
 * section "Load Imbalance": per-expert and per-rank counts).
 * topk_idx: device int64 [T, k], the router's top-k expert ids; -1 = unrouted.
 * Writes every array of *layout.  Order inside an expert's segment is stable
 * in p = t*k + j, so the result is deterministic.  Padded mode keeps the
 * first `capacity` pairs of each expert (in p order) and drops the rest.
 * workspace: device memory of at least ep_layout_workspace_bytes(T, k, E)
 * bytes, 256-byte aligned; contents need no initialisation and are scratch.
 * Returns EP_OK, EP_ERR_NULL, EP_ERR_SHAPE, EP_ERR_WORKSPACE or EP_ERR_LAUNCH.
 */
int ep_get_layout(const int64_t* topk_idx, const ep_layout_t* layout, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * ep_get_layout for callers that cannot allocate device memory at call time
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same results, with the workspace taken from a fixed array
 * of EP_NOALLOC_SCRATCH_BYTES bytes that the library keeps in device memory,
 * one copy per GPU, held until the process ends.  It runs on the current
 * device (the one `stream` belongs to).  It allocates nothing: the first call
 * on a device only looks up that device's copy of the array.  Sizes whose
 * workspace (ep_layout_workspace_bytes) exceeds the array are rejected with
 * EP_ERR_WORKSPACE before anything is enqueued.  Every call on a GPU uses
 * that GPU's one array, which keeps the last call's contents (nothing in it
 * needs to start at zero): calls that overlap on one GPU -- on two streams,
 * or from two threads -- race and must be ordered by the caller.
 * Returns EP_OK, EP_ERR_NULL, EP_ERR_SHAPE, EP_ERR_WORKSPACE or EP_ERR_LAUNCH
 * (also when the device's array cannot be looked up).
 */
#define EP_NOALLOC_SCRATCH_BYTES (4u << 20)
int ep_get_layout_noalloc(const int64_t* topk_idx, const ep_layout_t* layout, void* stream);

/*
 * Dispatch ([yololab] stage table, dispatch row; [backyes] 五.2: one row
 * per pair).  x: device bf16 [T, hidden].  For every pair p with
 * slot_idx[p] >= 0, receive row slot_idx[p] gets token p/k:
 *   EP_BF16:     recv_x bf16 [R, hidden], a bit copy; recv_scales unused (may be NULL).
 *   EP_FP8_E4M3: recv_x uint8 [R, hidden] E4M3 codes and recv_scales fp32
 *                [R, hidden/128] ([yololab] "FP8與低精度通訊"): per block of
 *                128 channels a = max(max|x|, 1e-4), scale = a/448,
 *                code = nearest E4M3 (ties to even, sign kept) of
 *                clamp(x * (448/a), -448, 448); requires hidden % 128 == 0.
 *   EP_FP8_E4M3_POW2: the same layout, but each block's scale is the smallest
 *                power of two s with 448 * s >= a, and each code the nearest
 *                E4M3 of clamp(x / s, -448, 448) (an exact rescale).
 *   EP_MXFP8_E4M3: recv_x uint8 [R, hidden] E4M3 codes and recv_scales uint8
 *                [R, hidden/32] E8M0 bytes (the OCP Microscaling MXFP8 format
 *                that gfx950's scaled matrix instructions consume; the same
 *                bytes per row as the fp32 scales): per block of 32 channels
 *                se = floor(log2(max|x|)) - 8 clamped to [-127, 127] (-127 for
 *                an all-zero block), byte = se + 127, code = nearest E4M3 (ties
 *                to even) of clamp(x / 2^se, -448, 448); requires hidden % 128 == 0.
 *   EP_F16:      x is fp16 [T, hidden] and recv_x fp16 [R, hidden], a bit copy.
 * FP8 dtype | EP_SCALES_MN_MAJOR: the same codes and scale values, with the
 *                scales stored transposed: fp32 [hidden/128, R] (E8M0 bytes
 *                [hidden/32, R] for MXFP8), entry c of receive row r at
 *                c * R + r, so the scales of one block column over an expert's
 *                consecutive rows are contiguous (the scale-layout conversion
 *                that section "FP8與低精度通訊" of [yololab] lists among the
 *                checks, for GEMMs that read a tile's row scales together).
 *                R is layout->num_recv_rows.  The flag with a non-FP8 dtype,
 *                EP_READ_X_AHEAD, or any other extra bit, is EP_ERR_DTYPE.
 * recv_scales (fp32 or E8M0 rows) must be 4-byte aligned.
 * Rows that no slot names are left untouched.  hidden % 8 == 0.
 * Returns EP_OK, EP_ERR_NULL, EP_ERR_SHAPE, EP_ERR_ALIGN, EP_ERR_DTYPE or EP_ERR_LAUNCH.
 */
int ep_dispatch(const void* x, const ep_layout_t* layout, int32_t hidden, int32_t recv_dtype,
                void* recv_x, void* recv_scales, void* stream);

/*
 * Scale-layout conversion (the layout conversion [yololab] "FP8與低精度通訊"
 * lists among the checks of low-precision dispatch): copies the row-major
 * scales an ep_dispatch with FP8 recv_dtype wrote -- fp32 [rows, hidden/128]
 * for EP_FP8_E4M3 and EP_FP8_E4M3_POW2, E8M0 bytes [rows, hidden/32] for
 * EP_MXFP8_E4M3 -- into the MN-major layout that EP_SCALES_MN_MAJOR writes:
 * entry c of row r to scales_mn[c * rows + r].  Every row is converted,
 * including rows that no slot named (they carry whatever the source held).
 * For large batches this pass (each scale byte read once and written once) is
 * cheaper than dispatch's own MN-major stores, which scatter one store per
 * entry; for decode-sized batches the flag avoids a launch.
 * scales and scales_mn: device memory, 4-byte aligned, not overlapping.
 * Returns EP_OK, EP_ERR_NULL, EP_ERR_SHAPE (hidden not a multiple of 128, or
 * the buffers overlap), EP_ERR_ALIGN, EP_ERR_DTYPE or EP_ERR_LAUNCH.
 */
int ep_scales_to_mn_major(const void* scales, int64_t rows, int32_t hidden, int32_t recv_dtype,
                          void* scales_mn, void* stream);

/*
 * Layout and dispatch in one call: the same results as ep_get_layout followed
 * by ep_dispatch with the same arguments.  For decode-sized batches -- at most
 * 4096 (token, k) pairs and top-k at most 8 -- both run in a single launch
 * (the pages' low-latency mode: "DeepEP是什麼？…" (yololab.net), section
 * "高吞吐與低延遲工作負載"); larger batches run the two calls' kernels in turn.
 * Arguments, layouts and status codes are those of ep_get_layout and
 * ep_dispatch; the workspace is required in both cases.
 * recv_dtype | EP_READ_X_AHEAD (batches larger than the one-launch size;
 * ignored by decode-sized ones): the two layout launches also read x -- its
 * first 128 MiB when it is larger -- with cached loads from extra workgroups,
 * so that it sits in the last-level cache (the 256 MB MALL) when dispatch
 * reads it.  The layout alone leaves HBM idle, and x read from HBM during
 * dispatch competes with its row writes.  Results are unchanged.  It pays
 * when x is not already cached (measured on MI355X at 8192 tokens x 7168:
 * the layout + dispatch kernels 130 -> 123 us and the step 310 -> 303 us
 * after the caches were emptied; 65,536 tokens x 4096, whose x never fits:
 * step 1042 -> 1039 us) and costs about 12 us when it is (step 280 -> 292
 * us when the router has just read x).
 * ep_dispatch and ep_get_layout reject the flag (EP_ERR_DTYPE).
 */
int ep_layout_dispatch(const int64_t* topk_idx, const ep_layout_t* layout, void* workspace,
                       size_t workspace_bytes, const void* x, int32_t hidden, int32_t recv_dtype,
                       void* recv_x, void* recv_scales, void* stream);

/*
 * Combine ([yololab] stage table, combine row: back to token order with a
 * weighted reduction).  expert_out: device bf16 [R, hidden]; topk_weights:
 * device fp32 [T, k].  out[t] = bf16(sum over j with slot_idx[t*k+j] >= 0 of
 * topk_weights[t,j] * expert_out[slot]), accumulated in fp32, rounded to
 * nearest-even; a token with no valid pair gets +0.  No renormalisation.
 * out: device bf16 [T, hidden], must not alias the inputs.  hidden % 8 == 0.
 * Returns EP_OK, EP_ERR_NULL, EP_ERR_SHAPE, EP_ERR_ALIGN or EP_ERR_LAUNCH.
 */
int ep_combine(const void* expert_out, const float* topk_weights, const ep_layout_t* layout,
               int32_t hidden, void* out, void* stream);

/*
 * Combine with fp16 expert outputs and fp16 output (the pages' benchmark
 * matrix lists BF16, FP16 and FP8 as the precisions to cover: [yololab]
 * "Benchmark矩陣").  As ep_combine, with expert_out fp16 [R, hidden] and
 * out fp16 [T, hidden]: out[t] = fp16(sum over valid j of topk_weights[t,j] *
 * expert_out[slot]) accumulated in fp32, rounded to nearest-even with fp16
 * subnormals kept and overflow to infinity; +0 for a token with no valid pair.
 * Returns EP_OK, EP_ERR_NULL, EP_ERR_SHAPE, EP_ERR_ALIGN or EP_ERR_LAUNCH.
 */
int ep_combine_f16(const void* expert_out, const float* topk_weights, const ep_layout_t* layout,
                   int32_t hidden, void* out, void* stream);

/*
 * Combine of FP8 expert outputs ([yololab] stage table, combine row;
 * "FP8與低精度通訊": low precision cuts combine volume too).  expert_q: device
 * uint8 [R, hidden] E4M3 codes; expert_scales: device fp32 [R, hidden/128], one
 * scale per row and 128-channel block.  out[t] = bf16(sum over valid j of
 * topk_weights[t,j] * decode(code) * scale), accumulated in fp32, rounded to
 * nearest-even; +0 for a token with no valid pair.  hidden % 128 == 0.
 * Returns EP_OK, EP_ERR_NULL, EP_ERR_SHAPE, EP_ERR_ALIGN or EP_ERR_LAUNCH.
 */
int ep_combine_fp8(const uint8_t* expert_q, const float* expert_scales,
                   const float* topk_weights, const ep_layout_t* layout, int32_t hidden, void* out,
                   void* stream);

/*
 * Combine of MXFP8 expert outputs (the FP8 combine of [yololab] "FP8與低精度
 * 通訊" in the format EP_MXFP8_E4M3 dispatch produces).  expert_q: device uint8
 * [R, hidden] E4M3 codes; expert_scales: device uint8 [R, hidden/32], one E8M0
 * byte per row and 32-channel block, value 2^(byte - 127) (255 is NaN).
 * out[t] = bf16(sum over valid j of topk_weights[t,j] * decode(code) *
 * 2^(byte - 127)), accumulated in fp32, rounded to nearest-even; +0 for a token
 * with no valid pair.  hidden % 128 == 0.
 * Returns EP_OK, EP_ERR_NULL, EP_ERR_SHAPE, EP_ERR_ALIGN or EP_ERR_LAUNCH.
 */
int ep_combine_mxfp8(const uint8_t* expert_q, const uint8_t* expert_scales,
                     const float* topk_weights, const ep_layout_t* layout, int32_t hidden,
                     void* out, void* stream);

/*
 * Per-group dedup variant.  A token goes once to every group of experts that
 * holds at least one of its top-k experts (a group is what one EP rank would
 * own), instead of once per expert: the pages count each rank's send and
 * receive bytes ([yololab] "Load Imbalance") and give the per-expert volume
 * ([backyes] 五.2), which this variant cuts whenever several of a token's
 * experts share a group.
 *
 * The group layout is an ep_layout_t whose "experts" are the G groups:
 *   num_tokens = T, num_topk = kg = min(k, G), num_experts = num_groups = G,
 *   capacity = 0, num_recv_rows = T * kg.
 * Its arrays, written by ep_get_group_layout:
 *   num_tokens_per_expert [G]   tokens that reach each group (so do
 *   num_tokens_per_group  [G]   both arrays)
 *   expert_offsets        [G+1] first receive row of each group; [G] = rows used
 *   slot_idx              [T*kg] receive row of entry i of token t: the token's
 *                               groups in ascending order, then -1; rows are
 *                               group-major and ascending in t inside a group
 *   recv_src              [T*kg] optional: entry index t*kg + i of each used row
 *   error_flags           [1]   EP_FLAG_BAD_EXPERT if some topk_idx entry is
 *                               outside [-1, num_experts) (that entry is skipped)
 * Dispatching to the groups is ep_dispatch(x, group_layout, ...), every dtype.
 */

/* Fill the size fields of a group layout (arrays NULL).  Requires
 * 0 <= num_tokens, 1 <= num_topk <= EP_MAX_TOPK, 1 <= num_groups <=
 * EP_MAX_EXPERTS, num_tokens * num_topk below 2^31.  Host only. */
int ep_group_layout_init(ep_layout_t* group_layout, int64_t num_tokens, int32_t num_topk,
                         int32_t num_groups);

/* Bytes of device workspace ep_get_group_layout needs; 0 if the sizes are invalid.  Host only. */
size_t ep_group_layout_workspace_bytes(int64_t num_tokens, int32_t num_topk, int32_t num_groups);

/*
 * Group layout and the receiving side's routing metadata.
 * topk_idx: device int64 [T, num_topk]; topk_weights: device fp32
 * [T, num_topk] (needed only for recv_topk_weights).  num_experts must be a
 * multiple of the group layout's G; expert e belongs to group e / (E/G).
 * Writes every array of *group_layout and, for each used row r of token t and
 * group g (both optional, NULL to skip):
 *   recv_topk_idx     int64 [T*kg, num_topk]: topk_idx[t, j] if that expert is
 *                     valid and in group g, else -1
 *   recv_topk_weights fp32  [T*kg, num_topk]: topk_weights[t, j] for the same
 *                     entries, else 0
 * Rows past the used ones are left untouched.  Optional (NULL to skip):
 *   is_token_in_group uint8 [T, G]: 1 if token t has a valid expert in group g,
 *                     else 0 (per-rank membership, [yololab] "Load
 *                     Imbalance": what each rank receives).  workspace: at least
 * ep_group_layout_workspace_bytes(T, num_topk, G) bytes, 256-byte aligned,
 * scratch.  Returns EP_OK, EP_ERR_NULL, EP_ERR_SHAPE, EP_ERR_ALIGN,
 * EP_ERR_WORKSPACE or EP_ERR_LAUNCH.
 */
int ep_get_group_layout(const int64_t* topk_idx, const float* topk_weights, int32_t num_topk,
                        int32_t num_experts, const ep_layout_t* group_layout,
                        int64_t* recv_topk_idx, float* recv_topk_weights,
                        uint8_t* is_token_in_group, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Group combine: the sending side's reduction of the rows that come back.
 * The receiving side has already weighted and summed its experts' outputs
 * into one row per (token, group), so the weights here are all 1:
 * out[t] = bf16(sum over i with slot_idx[t*kg+i] >= 0 of z[slot]) in ascending
 * group order, accumulated in fp32, rounded to nearest-even; +0 for a token
 * with no group.  z: device bf16 [T*kg, hidden]; out: device bf16 [T, hidden],
 * not aliasing z.  hidden % 8 == 0.
 * Returns EP_OK, EP_ERR_NULL, EP_ERR_SHAPE, EP_ERR_ALIGN or EP_ERR_LAUNCH.
 */
int ep_combine_groups(const void* z, const ep_layout_t* group_layout, int32_t hidden, void* out,
                      void* stream);

/*
 * Identity-expert stand-in for FP8 receive buffers (not part of the path;
 * used to feed combine in checks and benchmarks): y[r, c] = the bf16 nearest
 * (ties to even) to decode(q[r, c]) * scales[r, c/128], rounded once from the
 * exact product.  q uint8 [rows, hidden], scales fp32 [rows, hidden/128],
 * y bf16 [rows, hidden]; hidden % 128 == 0.
 */
int ep_dequant_fp8(const uint8_t* q, const float* scales, int64_t rows, int32_t hidden, void* y,
                   void* stream);

/* Identity-expert stand-in for MXFP8 receive buffers (not part of the path):
 * y[r, c] = the bf16 nearest (ties to even) to decode(q[r, c]) *
 * 2^(scales[r, c/32] - 127), an exact product rounded once; a scale byte of
 * 255 (NaN in E8M0; dispatch never writes it) makes its 32 outputs the quiet
 * NaN 0x7FC0.  q uint8 [rows, hidden], scales uint8 [rows, hidden/32], y bf16
 * [rows, hidden]; hidden % 128 == 0. */
int ep_dequant_mxfp8(const uint8_t* q, const uint8_t* scales, int64_t rows, int32_t hidden,
                     void* y, void* stream);

/*
 * The FP8 encoder that ep_dispatch applies to x * inv, exposed for
 * verification: out[i] = E4M3 code of clamp(f, -448, 448) for the n fp32
 * values f whose bit patterns are first, first+1, ... (the sequence wraps
 * modulo 2^32).  method 0 = the encoder ep_dispatch uses; 1 = the software
 * encoder; 2 = the hardware conversion instruction.  out: device uint8 [n].
 */
int ep_cast_e4m3_bits(uint32_t first, int64_t n, int32_t method, uint8_t* out, void* stream);

/* Plain device copy of `bytes` bytes (both 16-byte aligned, bytes % 16 == 0);
 * the bandwidth reference that measurements are compared against. */
int ep_copy(const void* src, void* dst, size_t bytes, void* stream);

/* Human-readable text of a status code (static storage). */
const char* ep_status_string(int status);

/* Library version string (static storage). */
const char* ep_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EP_H */
