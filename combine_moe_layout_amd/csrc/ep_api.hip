// ep_api.hip -- the extern "C" entry points of libep.so (declared in ep.h):
// host-side argument checks, then the call's HIP kernels enqueued on the
// caller's stream.  Nothing here allocates or synchronises.
#include <stdint.h>

#include <mutex>

#include "ep_internal.h"

namespace {

constexpr int64_t kInt32Limit = INT32_MAX;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Sizes of a layout are valid on their own.
int check_sizes(int64_t T, int32_t k, int32_t E, int32_t G, int32_t cap) {
  if (T < 0 || k < 1 || k > EP_MAX_TOPK || E < 1 || E > EP_MAX_EXPERTS || G < 1 || E % G != 0 ||
      cap < 0)
    return EP_ERR_SHAPE;
  if (T > kInt32Limit / k) return EP_ERR_SHAPE;                      // pairs index int32 slots
  if (cap > 0 && (int64_t)E * cap > kInt32Limit) return EP_ERR_SHAPE;  // rows fit int32
  // the packed layout intermediate holds a rank below the chunk size
  return EP_OK;
}

int check_layout(const ep_layout_t* L) {
  if (L == nullptr) return EP_ERR_NULL;
  int rc = check_sizes(L->num_tokens, L->num_topk, L->num_experts, L->num_groups, L->capacity);
  if (rc != EP_OK) return rc;
  const int64_t R = L->capacity > 0 ? (int64_t)L->num_experts * L->capacity
                                    : L->num_tokens * L->num_topk;
  if (L->num_recv_rows != R) return EP_ERR_SHAPE;
  if (L->num_tokens > 0 && L->slot_idx == nullptr) return EP_ERR_NULL;
  return EP_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? EP_OK : EP_ERR_LAUNCH; }

// The layout's own arguments (everything but the workspace).
int check_layout_args(const int64_t* topk_idx, const ep_layout_t* layout) {
  int rc = check_layout(layout);
  if (rc != EP_OK) return rc;
  const ep_layout_t& L = *layout;
  if ((L.num_tokens > 0 && topk_idx == nullptr) || L.num_tokens_per_expert == nullptr ||
      L.expert_offsets == nullptr || L.num_tokens_per_group == nullptr ||
      L.error_flags == nullptr)
    return EP_ERR_NULL;
  return EP_OK;
}

size_t layout_workspace_need(const ep_layout_t& L) {
  return ep::layout_workspace_bytes(L.num_tokens * (int64_t)L.num_topk, L.num_experts);
}

// Checks shared by ep_get_layout and ep_layout_dispatch.
int check_get_layout(const int64_t* topk_idx, const ep_layout_t* layout, void* workspace,
                     size_t workspace_bytes) {
  int rc = check_layout_args(topk_idx, layout);
  if (rc != EP_OK) return rc;
  if (workspace == nullptr) return EP_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return EP_ERR_ALIGN;
  if (workspace_bytes < layout_workspace_need(*layout)) return EP_ERR_WORKSPACE;
  return EP_OK;
}

// ---------------------------------------------------------------------------
// Layout workspace for ep_get_layout_noalloc: a fixed array in device memory,
// one copy on every GPU the library runs on, held until the process ends.
// Host code never uses the array's name as an address (on the host it is a
// stand-in, not a device pointer): the first call on each device resolves
// that device's copy with hipGetSymbolAddress and keeps the pointer.
constexpr size_t kNoAllocScratchBytes = EP_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, or nullptr if it cannot be resolved.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

// Checks shared by ep_dispatch and ep_layout_dispatch (after the layout's);
// only the latter takes EP_READ_X_AHEAD.
int check_dispatch(const void* x, const ep_layout_t* layout, int32_t hidden, int32_t recv_dtype,
                   void* recv_x, void* recv_scales, bool read_ahead_ok) {
  const int32_t base = ep::dtype_base(recv_dtype);
  const bool fp8 = ep::dtype_is_fp8(base);
  if (base != EP_BF16 && base != EP_F16 && !fp8) return EP_ERR_DTYPE;
  if (ep::dtype_scales_mn(recv_dtype) && !fp8) return EP_ERR_DTYPE;
  if (ep::dtype_read_x_ahead(recv_dtype) && !read_ahead_ok) return EP_ERR_DTYPE;
  if (hidden < 8 || hidden > EP_MAX_HIDDEN || hidden % 8 != 0 || (fp8 && hidden % 128 != 0))
    return EP_ERR_SHAPE;
  if (layout->num_tokens == 0) return EP_OK;
  if (x == nullptr || recv_x == nullptr || (fp8 && recv_scales == nullptr)) return EP_ERR_NULL;
  if (!aligned16(x) || !aligned16(recv_x) ||
      (fp8 && (reinterpret_cast<uintptr_t>(recv_scales) & 3u) != 0))
    return EP_ERR_ALIGN;
  return EP_OK;
}

}  // namespace

extern "C" {

int ep_layout_init(ep_layout_t* layout, int64_t num_tokens, int32_t num_topk,
                   int32_t num_experts, int32_t num_groups, int32_t capacity) {
  if (layout == nullptr) return EP_ERR_NULL;
  const int rc = check_sizes(num_tokens, num_topk, num_experts, num_groups, capacity);
  if (rc != EP_OK) return rc;
  *layout = ep_layout_t{};
  layout->num_tokens = num_tokens;
  layout->num_topk = num_topk;
  layout->num_experts = num_experts;
  layout->num_groups = num_groups;
  layout->capacity = capacity;
  layout->num_recv_rows =
      capacity > 0 ? (int64_t)num_experts * capacity : num_tokens * (int64_t)num_topk;
  return EP_OK;
}

int64_t ep_num_recv_rows(int64_t num_tokens, int32_t num_topk, int32_t num_experts,
                         int32_t capacity) {
  if (check_sizes(num_tokens, num_topk, num_experts, 1, capacity) != EP_OK) return -1;
  return capacity > 0 ? (int64_t)num_experts * capacity : num_tokens * (int64_t)num_topk;
}

size_t ep_layout_workspace_bytes(int64_t num_tokens, int32_t num_topk, int32_t num_experts) {
  if (check_sizes(num_tokens, num_topk, num_experts, 1, 0) != EP_OK) return 0;
  return ep::layout_workspace_bytes(num_tokens * (int64_t)num_topk, num_experts);
}

int ep_get_layout(const int64_t* topk_idx, const ep_layout_t* layout, void* workspace,
                  size_t workspace_bytes, void* stream) {
  const int rc = check_get_layout(topk_idx, layout, workspace, workspace_bytes);
  if (rc != EP_OK) return rc;
  return launch_status(
      ep::launch_layout(topk_idx, *layout, workspace, static_cast<hipStream_t>(stream)));
}

int ep_get_layout_noalloc(const int64_t* topk_idx, const ep_layout_t* layout, void* stream) {
  int rc = check_layout_args(topk_idx, layout);
  if (rc != EP_OK) return rc;
  if (layout_workspace_need(*layout) > kNoAllocScratchBytes) return EP_ERR_WORKSPACE;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return EP_ERR_LAUNCH;
  return launch_status(
      ep::launch_layout(topk_idx, *layout, ws, static_cast<hipStream_t>(stream)));
}

int ep_dispatch(const void* x, const ep_layout_t* layout, int32_t hidden, int32_t recv_dtype,
                void* recv_x, void* recv_scales, void* stream) {
  int rc = check_layout(layout);
  if (rc != EP_OK) return rc;
  rc = check_dispatch(x, layout, hidden, recv_dtype, recv_x, recv_scales, false);
  if (rc != EP_OK || layout->num_tokens == 0) return rc;
  return launch_status(ep::launch_dispatch(x, *layout, hidden, recv_dtype, recv_x, recv_scales,
                                           static_cast<hipStream_t>(stream)));
}

int ep_layout_dispatch(const int64_t* topk_idx, const ep_layout_t* layout, void* workspace,
                       size_t workspace_bytes, const void* x, int32_t hidden, int32_t recv_dtype,
                       void* recv_x, void* recv_scales, void* stream) {
  int rc = check_get_layout(topk_idx, layout, workspace, workspace_bytes);
  if (rc != EP_OK) return rc;
  rc = check_dispatch(x, layout, hidden, recv_dtype, recv_x, recv_scales, true);
  if (rc != EP_OK) return rc;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool read_ahead = ep::dtype_read_x_ahead(recv_dtype);
  recv_dtype &= ~EP_READ_X_AHEAD;
  if (ep::fused_layout_dispatch_fits(*layout))
    return launch_status(ep::launch_layout_dispatch_small(topk_idx, *layout, x, hidden, recv_dtype,
                                                          recv_x, recv_scales, s));
  // With EP_READ_X_AHEAD the layout's launches also read x (2-byte elements)
  // into the last-level cache.
  const size_t x_bytes = read_ahead ? (size_t)layout->num_tokens * (size_t)hidden * 2 : 0;
  rc = launch_status(ep::launch_layout_warm(topk_idx, *layout, workspace, x, x_bytes, s));
  if (rc != EP_OK || layout->num_tokens == 0) return rc;
  return launch_status(ep::launch_dispatch(x, *layout, hidden, recv_dtype, recv_x, recv_scales, s));
}

int ep_combine(const void* expert_out, const float* topk_weights, const ep_layout_t* layout,
               int32_t hidden, void* out, void* stream) {
  int rc = check_layout(layout);
  if (rc != EP_OK) return rc;
  if (hidden < 8 || hidden > EP_MAX_HIDDEN || hidden % 8 != 0) return EP_ERR_SHAPE;
  if (layout->num_tokens == 0) return EP_OK;
  if (expert_out == nullptr || topk_weights == nullptr || out == nullptr) return EP_ERR_NULL;
  if (!aligned16(expert_out) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(topk_weights) & 3u) != 0)
    return EP_ERR_ALIGN;
  return launch_status(ep::launch_combine(expert_out, topk_weights, *layout, hidden, out,
                                          static_cast<hipStream_t>(stream)));
}

int ep_combine_f16(const void* expert_out, const float* topk_weights, const ep_layout_t* layout,
                   int32_t hidden, void* out, void* stream) {
  int rc = check_layout(layout);
  if (rc != EP_OK) return rc;
  if (hidden < 8 || hidden > EP_MAX_HIDDEN || hidden % 8 != 0) return EP_ERR_SHAPE;
  if (layout->num_tokens == 0) return EP_OK;
  if (expert_out == nullptr || topk_weights == nullptr || out == nullptr) return EP_ERR_NULL;
  if (!aligned16(expert_out) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(topk_weights) & 3u) != 0)
    return EP_ERR_ALIGN;
  return launch_status(ep::launch_combine_f16(expert_out, topk_weights, *layout, hidden, out,
                                              static_cast<hipStream_t>(stream)));
}

int ep_combine_fp8(const uint8_t* expert_q, const float* expert_scales,
                   const float* topk_weights, const ep_layout_t* layout, int32_t hidden, void* out,
                   void* stream) {
  int rc = check_layout(layout);
  if (rc != EP_OK) return rc;
  if (hidden < 128 || hidden > EP_MAX_HIDDEN || hidden % 128 != 0) return EP_ERR_SHAPE;
  if (layout->num_tokens == 0) return EP_OK;
  if (expert_q == nullptr || expert_scales == nullptr || topk_weights == nullptr || out == nullptr)
    return EP_ERR_NULL;
  if (!aligned16(expert_q) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(expert_scales) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(topk_weights) & 3u) != 0)
    return EP_ERR_ALIGN;
  return launch_status(ep::launch_combine_fp8(expert_q, expert_scales, topk_weights, *layout,
                                              hidden, out, static_cast<hipStream_t>(stream)));
}

int ep_combine_mxfp8(const uint8_t* expert_q, const uint8_t* expert_scales,
                     const float* topk_weights, const ep_layout_t* layout, int32_t hidden,
                     void* out, void* stream) {
  int rc = check_layout(layout);
  if (rc != EP_OK) return rc;
  if (hidden < 128 || hidden > EP_MAX_HIDDEN || hidden % 128 != 0) return EP_ERR_SHAPE;
  if (layout->num_tokens == 0) return EP_OK;
  if (expert_q == nullptr || expert_scales == nullptr || topk_weights == nullptr || out == nullptr)
    return EP_ERR_NULL;
  if (!aligned16(expert_q) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(topk_weights) & 3u) != 0)
    return EP_ERR_ALIGN;
  return launch_status(ep::launch_combine_mxfp8(expert_q, expert_scales, topk_weights, *layout,
                                                hidden, out, static_cast<hipStream_t>(stream)));
}

int ep_group_layout_init(ep_layout_t* group_layout, int64_t num_tokens, int32_t num_topk,
                         int32_t num_groups) {
  if (group_layout == nullptr) return EP_ERR_NULL;
  if (num_tokens < 0 || num_topk < 1 || num_topk > EP_MAX_TOPK || num_groups < 1 ||
      num_groups > EP_MAX_EXPERTS || num_tokens > kInt32Limit / num_topk)
    return EP_ERR_SHAPE;
  const int32_t kg = num_topk < num_groups ? num_topk : num_groups;
  return ep_layout_init(group_layout, num_tokens, kg, num_groups, num_groups, 0);
}

size_t ep_group_layout_workspace_bytes(int64_t num_tokens, int32_t num_topk, int32_t num_groups) {
  ep_layout_t tmp;
  if (ep_group_layout_init(&tmp, num_tokens, num_topk, num_groups) != EP_OK) return 0;
  return ep::group_layout_workspace_bytes(num_tokens, num_topk, num_groups);
}

int ep_get_group_layout(const int64_t* topk_idx, const float* topk_weights, int32_t num_topk,
                        int32_t num_experts, const ep_layout_t* group_layout,
                        int64_t* recv_topk_idx, float* recv_topk_weights,
                        uint8_t* is_token_in_group, void* workspace, size_t workspace_bytes,
                        void* stream) {
  int rc = check_layout(group_layout);
  if (rc != EP_OK) return rc;
  const ep_layout_t& GL = *group_layout;
  const int32_t G = GL.num_experts;
  if (num_topk < 1 || num_topk > EP_MAX_TOPK || num_experts < 1 ||
      num_experts > EP_MAX_EXPERTS || num_experts % G != 0 || GL.num_groups != G ||
      GL.capacity != 0 || GL.num_topk != (num_topk < G ? num_topk : G) ||
      GL.num_tokens > kInt32Limit / num_topk)
    return EP_ERR_SHAPE;
  const bool any = GL.num_tokens > 0;
  if ((any && topk_idx == nullptr) || GL.num_tokens_per_expert == nullptr ||
      GL.expert_offsets == nullptr || GL.num_tokens_per_group == nullptr ||
      GL.error_flags == nullptr || workspace == nullptr ||
      (any && recv_topk_weights != nullptr && topk_weights == nullptr))
    return EP_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
      (reinterpret_cast<uintptr_t>(topk_weights) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(recv_topk_idx) & 7u) != 0 ||
      (reinterpret_cast<uintptr_t>(recv_topk_weights) & 3u) != 0)
    return EP_ERR_ALIGN;
  if (workspace_bytes < ep::group_layout_workspace_bytes(GL.num_tokens, num_topk, G))
    return EP_ERR_WORKSPACE;
  return launch_status(ep::launch_group_layout(topk_idx, topk_weights, num_topk, num_experts, GL,
                                               recv_topk_idx, recv_topk_weights,
                                               is_token_in_group, workspace,
                                               static_cast<hipStream_t>(stream)));
}

int ep_combine_groups(const void* z, const ep_layout_t* group_layout, int32_t hidden, void* out,
                      void* stream) {
  int rc = check_layout(group_layout);
  if (rc != EP_OK) return rc;
  if (group_layout->capacity != 0 || group_layout->num_experts != group_layout->num_groups)
    return EP_ERR_SHAPE;
  if (hidden < 8 || hidden > EP_MAX_HIDDEN || hidden % 8 != 0) return EP_ERR_SHAPE;
  if (group_layout->num_tokens == 0) return EP_OK;
  if (z == nullptr || out == nullptr) return EP_ERR_NULL;
  if (!aligned16(z) || !aligned16(out)) return EP_ERR_ALIGN;
  return launch_status(ep::launch_combine_groups(z, *group_layout, hidden, out,
                                                 static_cast<hipStream_t>(stream)));
}

int ep_dequant_fp8(const uint8_t* q, const float* scales, int64_t rows, int32_t hidden, void* y,
                   void* stream) {
  if (rows < 0 || hidden < 128 || hidden > EP_MAX_HIDDEN || hidden % 128 != 0)
    return EP_ERR_SHAPE;
  if (rows == 0) return EP_OK;
  if (q == nullptr || scales == nullptr || y == nullptr) return EP_ERR_NULL;
  if (!aligned16(q) || !aligned16(y) || (reinterpret_cast<uintptr_t>(scales) & 3u) != 0)
    return EP_ERR_ALIGN;
  return launch_status(
      ep::launch_dequant_fp8(q, scales, rows, hidden, y, static_cast<hipStream_t>(stream)));
}

int ep_dequant_mxfp8(const uint8_t* q, const uint8_t* scales, int64_t rows, int32_t hidden,
                     void* y, void* stream) {
  if (rows < 0 || hidden < 128 || hidden > EP_MAX_HIDDEN || hidden % 128 != 0)
    return EP_ERR_SHAPE;
  if (rows == 0) return EP_OK;
  if (q == nullptr || scales == nullptr || y == nullptr) return EP_ERR_NULL;
  if (!aligned16(q) || !aligned16(y)) return EP_ERR_ALIGN;
  return launch_status(
      ep::launch_dequant_mxfp8(q, scales, rows, hidden, y, static_cast<hipStream_t>(stream)));
}

int ep_scales_to_mn_major(const void* scales, int64_t rows, int32_t hidden, int32_t recv_dtype,
                          void* scales_mn, void* stream) {
  if (!ep::dtype_is_fp8(recv_dtype)) return EP_ERR_DTYPE;
  if (rows < 0 || hidden < 128 || hidden > EP_MAX_HIDDEN || hidden % 128 != 0)
    return EP_ERR_SHAPE;
  if (rows == 0) return EP_OK;
  if (scales == nullptr || scales_mn == nullptr) return EP_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(scales) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(scales_mn) & 3u) != 0)
    return EP_ERR_ALIGN;
  const uintptr_t a = reinterpret_cast<uintptr_t>(scales);
  const uintptr_t b = reinterpret_cast<uintptr_t>(scales_mn);
  const uintptr_t bytes = (uintptr_t)rows * (uintptr_t)(hidden / 32);
  if (a < b + bytes && b < a + bytes) return EP_ERR_SHAPE;  // the buffers overlap
  return launch_status(ep::launch_scales_mn(scales, rows, hidden, recv_dtype, scales_mn,
                                            static_cast<hipStream_t>(stream)));
}

int ep_cast_e4m3_bits(uint32_t first, int64_t n, int32_t method, uint8_t* out, void* stream) {
  if (n < 0 || method < 0 || method > 2) return EP_ERR_SHAPE;
  if (n == 0) return EP_OK;
  if (out == nullptr) return EP_ERR_NULL;
  return launch_status(
      ep::launch_cast_e4m3_bits(first, n, method, out, static_cast<hipStream_t>(stream)));
}

int ep_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes % 16 != 0) return EP_ERR_SHAPE;
  if (bytes == 0) return EP_OK;
  if (src == nullptr || dst == nullptr) return EP_ERR_NULL;
  if (!aligned16(src) || !aligned16(dst)) return EP_ERR_ALIGN;
  return launch_status(ep::launch_copy(src, dst, bytes, static_cast<hipStream_t>(stream)));
}

const char* ep_status_string(int status) {
  switch (status) {
    case EP_OK: return "ok";
    case EP_ERR_NULL: return "a required pointer is NULL";
    case EP_ERR_SHAPE: return "a size is out of range or sizes disagree";
    case EP_ERR_ALIGN: return "a buffer is not aligned as required";
    case EP_ERR_WORKSPACE: return "workspace smaller than its size query reports";
    case EP_ERR_LAUNCH: return "the HIP runtime reported a launch error";
    case EP_ERR_DTYPE: return "unknown receive dtype";
    default: return "unknown status";
  }
}

const char* ep_version(void) { return "combine_moe_layout_amd 0.1.0 (gfx950)"; }

}  // extern "C"
