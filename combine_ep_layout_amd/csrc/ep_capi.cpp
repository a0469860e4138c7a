// C ABI of the library (declared in include/ep_mi355x.h).
//
// Every entry point validates its scalars and pointers on the host before
// anything is enqueued, reports errors by return code plus a per-thread
// message, never throws and never allocates, copies or synchronises
// ("MORI JIT v2", section 3.5: invalid configurations are rejected before any
// work; section 4: nothing but launches on the call path; section 6: C entry
// points catch everything and report through a last-error string).
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <exception>
#include <mutex>
#include <utility>
#include <vector>

#include "ep_launch.hpp"
#include "ep_mi355x.h"

namespace {

thread_local char g_last_error[512] = "";
thread_local hipError_t g_hip_error = hipSuccess;

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return code;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Byte offset of the dispatch plan inside ep_layout_dispatch's workspace: after
// the layout's own workspace, on a 256-byte boundary.
size_t plan_offset(size_t layout_bytes) { return (layout_bytes + 255) & ~(size_t)255; }

// A HIP error left on this thread by an earlier, unrelated call (another
// library's, say) would otherwise be read back after our launch and reported
// as its failure: each entry point drops it before launching anything.
void discard_stale_error() { (void)hipGetLastError(); }

int from_launch(int rc, const char *what) {
  if (rc == 0) {
    g_last_error[0] = '\0';
    return EP_OK;
  }
  if (rc == -2) return fail(EP_EUNSUPPORTED, "%s: no compiled kernel for this shape", what);
  return fail(EP_EHIP, "%s: kernel launch failed: %s", what, hipGetErrorString(g_hip_error));
}

int check_topk(const char *what, int32_t T, int32_t K) {
  if (T < 0) return fail(EP_EINVAL, "%s: num_tokens must be >= 0 (got %d)", what, T);
  if (K < 1 || K > EP_MAX_TOPK)
    return fail(EP_EINVAL, "%s: topk must be in 1..%d (got %d)", what, EP_MAX_TOPK, K);
  if ((int64_t)T * K > INT32_MAX)
    return fail(EP_EINVAL, "%s: num_tokens*topk overflows int32", what);
  return EP_OK;
}

}  // namespace

hipError_t &ep::last_hip_error() { return g_hip_error; }

// Workgroup caps per stream handle. Launchers look them up on every launch;
// while no cap is registered the lookup is one relaxed atomic load.
namespace {
std::mutex g_caps_mu;
std::vector<std::pair<hipStream_t, int>> g_caps;
std::atomic<int> g_caps_n{0};
}  // namespace

int ep::stream_workgroup_limit(hipStream_t stream) {
  if (g_caps_n.load(std::memory_order_acquire) == 0) return 0;
  std::lock_guard<std::mutex> lock(g_caps_mu);
  for (const auto &c : g_caps)
    if (c.first == stream) return c.second;
  return 0;
}

extern "C" {

const char *ep_last_error(void) { return g_last_error; }

int ep_set_workgroup_limit(void *stream, int32_t max_workgroups) {
  try {
    if (max_workgroups < 0)
      return fail(EP_EINVAL, "ep_set_workgroup_limit: max_workgroups must be >= 0 (got %d)",
                  max_workgroups);
    int cap = max_workgroups;
    if (cap > 0) {  // never more workgroups than compute units
      int dev = 0, cus = 0;
      hipError_t e = hipGetDevice(&dev);
      if (e == hipSuccess)
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      if (e != hipSuccess)
        return fail(EP_EHIP, "ep_set_workgroup_limit: cannot read the compute-unit count: %s",
                    hipGetErrorString(e));
      if (cus > 0 && cap > cus) cap = cus;
    }
    const hipStream_t s = (hipStream_t)stream;
    std::lock_guard<std::mutex> lock(g_caps_mu);
    size_t i = 0;
    while (i < g_caps.size() && g_caps[i].first != s) ++i;
    if (cap == 0) {
      if (i < g_caps.size()) g_caps.erase(g_caps.begin() + (ptrdiff_t)i);
    } else if (i < g_caps.size()) {
      g_caps[i].second = cap;
    } else {
      g_caps.emplace_back(s, cap);
    }
    g_caps_n.store((int)g_caps.size(), std::memory_order_release);
    g_last_error[0] = '\0';
    return EP_OK;
  } catch (const std::exception &e) {
    return fail(EP_EHIP, "ep_set_workgroup_limit: %s", e.what());
  } catch (...) {
    return fail(EP_EHIP, "ep_set_workgroup_limit: unknown exception");
  }
}

int ep_get_workgroup_limit(void *stream) {
  try {
    return ep::stream_workgroup_limit((hipStream_t)stream);
  } catch (...) {
    return fail(EP_EHIP, "ep_get_workgroup_limit: unknown exception");
  }
}

int ep_supported(int32_t pass, int32_t hidden, int32_t topk, int32_t dtype) {
  try {
    if (pass == 0) return ep::has_layout(topk) ? 1 : 0;
    if (pass == 1) return ep::has_dispatch(hidden, topk, dtype) ? 1 : 0;
    if (pass == 2) return ep::has_combine(hidden, topk, dtype) ? 1 : 0;
  } catch (...) {
  }
  return 0;
}

size_t ep_layout_dispatch_workspace_bytes(int32_t num_tokens, int32_t topk, int32_t num_experts) {
  try {
    if (num_tokens < 0 || topk < 1 || topk > EP_MAX_TOPK || num_experts < 1 ||
        num_experts > EP_MAX_EXPERTS || (int64_t)num_tokens * topk > INT32_MAX)
      return 0;
    return plan_offset(ep::layout_workspace(num_tokens, topk, num_experts)) +
           (size_t)num_tokens * topk * 8;
  } catch (...) {
    return 0;
  }
}

size_t ep_layout_workspace_bytes(int32_t num_tokens, int32_t topk, int32_t num_experts) {
  try {
    if (num_tokens < 0 || topk < 1 || topk > EP_MAX_TOPK || num_experts < 1 ||
        num_experts > EP_MAX_EXPERTS)
      return 0;
    return ep::layout_workspace(num_tokens, topk, num_experts);
  } catch (...) {
    return 0;
  }
}

}  // extern "C"

namespace {

// The optional read-ahead region of ep_layout: NULL with 0 bytes, or a
// 4-byte aligned pointer (the layout reads 4-byte words of it).
int check_prefetch(const char *what, const void *prefetch, size_t prefetch_bytes) {
  if (prefetch == nullptr && prefetch_bytes != 0)
    return fail(EP_EINVAL, "%s: prefetch is NULL but prefetch_bytes is %zu", what, prefetch_bytes);
  if (!aligned(prefetch, 4)) return fail(EP_EINVAL, "%s: prefetch must be 4-byte aligned", what);
  return EP_OK;
}

// Checks of ep_layout's arguments (shared with ep_layout_dispatch).
int check_layout(const char *what, const int32_t *topk_idx, int32_t num_tokens, int32_t topk,
                 int32_t num_experts, int32_t expert_alignment, int64_t capacity_rows,
                 const int32_t *counts, const int32_t *offsets, const int32_t *dst_slot,
                 const int32_t *recv_src_metadata, const int32_t *num_recv, const void *workspace,
                 size_t workspace_bytes) {
  if (int rc = check_topk(what, num_tokens, topk)) return rc;
  if (num_experts < 1 || num_experts > EP_MAX_EXPERTS)
    return fail(EP_EINVAL, "%s: num_experts must be in 1..%d (got %d)", what, EP_MAX_EXPERTS,
                num_experts);
  if (expert_alignment < 1)
    return fail(EP_EINVAL, "%s: expert_alignment must be >= 1 (got %d)", what, expert_alignment);
  const int64_t worst =
      (int64_t)num_tokens * topk + (int64_t)num_experts * (expert_alignment - 1);
  if (worst > INT32_MAX)
    return fail(EP_EINVAL, "%s: worst-case expand rows %lld overflow int32", what,
                (long long)worst);
  if (capacity_rows < worst)
    return fail(EP_ECAPACITY, "%s: capacity_rows %lld < worst case T*K + E*(A-1) = %lld", what,
                (long long)capacity_rows, (long long)worst);
  if (!counts || !offsets || !num_recv ||
      (num_tokens > 0 && (!topk_idx || !dst_slot || !recv_src_metadata)))
    return fail(EP_EINVAL, "%s: a required pointer is NULL", what);
  if (!ep::has_layout(topk))
    return fail(EP_EUNSUPPORTED, "%s: topk %d has no compiled layout kernel", what, topk);
  const size_t need = ep::layout_workspace(num_tokens, topk, num_experts);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(EP_EINVAL, "%s: workspace of %zu bytes needed (got %zu)", what, need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (need > 0 && !aligned(workspace, 16))
    return fail(EP_EINVAL, "%s: workspace must be 16-byte aligned", what);
  return EP_OK;
}

// Checks of ep_dispatch's arguments (shared with ep_layout_dispatch); on
// success *row_bytes receives the bytes of one token row.
int check_dispatch(const char *what, const void *x, const float *x_scales,
                   const float *topk_weights, const int32_t *dst_slot, int32_t num_tokens,
                   int32_t hidden, int32_t topk, int32_t dtype, int64_t capacity_rows,
                   const void *expand_x, const float *expand_scales, const float *expand_weights,
                   int64_t *row_bytes) {
  if (int rc = check_topk(what, num_tokens, topk)) return rc;
  if (hidden < 1) return fail(EP_EINVAL, "%s: hidden must be >= 1 (got %d)", what, hidden);
  if (capacity_rows < 0) return fail(EP_EINVAL, "%s: capacity_rows must be >= 0", what);
  // Bytes per hidden unit: hidden counts elements, except for fp4x2 where it
  // counts bytes (two e2m1 values per byte, as the caller packs them).
  int elt;
  if (dtype == EP_BF16) elt = 2;
  else if (dtype == EP_FP32) elt = 4;
  else if (dtype == EP_FP8_E4M3 || dtype == EP_FP4X2) elt = 1;
  else return fail(EP_EINVAL, "%s: unknown dtype %d", what, dtype);
  if (((int64_t)hidden * elt) % 16 != 0)
    return fail(EP_EINVAL, "%s: token bytes (%lld) must be a multiple of 16", what,
                (long long)hidden * elt);
  const bool byte_dtype = dtype == EP_FP8_E4M3 || dtype == EP_FP4X2;
  if ((x_scales == nullptr) != (expand_scales == nullptr))
    return fail(EP_EINVAL, "%s: x_scales and expand_scales go together", what);
  if (x_scales != nullptr) {
    if (!byte_dtype)
      return fail(EP_EINVAL, "%s: scale rows travel only with fp8 / fp4x2 rows", what);
    const int64_t elems = dtype == EP_FP4X2 ? 2 * (int64_t)hidden : hidden;
    if (elems % 128 != 0)
      return fail(EP_EINVAL, "%s: scales need a multiple of 128 elements per row (got %lld)",
                  what, (long long)elems);
  }
  if (num_tokens > 0 && (!x || !dst_slot || !expand_x))
    return fail(EP_EINVAL, "%s: a required pointer is NULL", what);
  if (!aligned(x, 16) || !aligned(expand_x, 16) || !aligned(x_scales, 16) ||
      !aligned(expand_scales, 16) || !aligned(dst_slot, 4) || !aligned(topk_weights, 4) ||
      !aligned(expand_weights, 4))
    return fail(EP_EINVAL, "%s: misaligned pointer (rows need 16 bytes)", what);
  if (!ep::has_dispatch(hidden, topk, dtype))
    return fail(EP_EUNSUPPORTED, "%s: (hidden %d, topk %d, dtype %d) has no compiled kernel",
                what, hidden, topk, dtype);
  *row_bytes = (int64_t)hidden * elt;
  return EP_OK;
}

// The checks of the non-expand dispatch's own arguments (the layout's outputs
// it reads are checked by the caller). Sets the row bytes and scale columns.
int check_dispatch_compact(const char *what, const void *x, const float *x_scales,
                           const int32_t *topk_idx, const float *topk_weights, int32_t num_tokens,
                           int32_t hidden, int32_t topk, int32_t dtype, const void *recv_x,
                           const float *recv_scales, const int32_t *recv_topk_idx,
                           const float *recv_topk_weights, int64_t *row_bytes,
                           int64_t *scale_cols) {
  if (int rc = check_topk(what, num_tokens, topk)) return rc;
  int elt;
  if (dtype == EP_BF16) elt = 2;
  else if (dtype == EP_FP32) elt = 4;
  else if (dtype == EP_FP8_E4M3 || dtype == EP_FP4X2) elt = 1;
  else return fail(EP_EINVAL, "%s: unknown dtype %d", what, dtype);
  const int64_t rb = (int64_t)hidden * elt;
  if (hidden < 1 || rb % 16 != 0 || rb > INT32_MAX)
    return fail(EP_EINVAL,
                "%s: token bytes must be a positive multiple of 16 below 2^31 (got %lld)", what,
                (long long)rb);
  if ((x_scales == nullptr) != (recv_scales == nullptr))
    return fail(EP_EINVAL, "%s: x_scales and recv_scales go together", what);
  int64_t sc = 0;
  if (x_scales != nullptr) {
    if (dtype != EP_FP8_E4M3 && dtype != EP_FP4X2)
      return fail(EP_EINVAL, "%s: scale rows travel only with fp8 / fp4x2 rows", what);
    const int64_t values = dtype == EP_FP4X2 ? 2 * (int64_t)hidden : hidden;
    if (values % 128 != 0)
      return fail(EP_EINVAL, "%s: scales need a multiple of 128 values per row", what);
    sc = values / 128;
  }
  if (num_tokens > 0 && (!x || !topk_idx || !recv_x || !recv_topk_idx))
    return fail(EP_EINVAL, "%s: a required pointer is NULL", what);
  if (topk_weights != nullptr && recv_topk_weights == nullptr)
    return fail(EP_EINVAL, "%s: topk_weights given without recv_topk_weights", what);
  if (!aligned(x, 16) || !aligned(recv_x, 16) || !aligned(x_scales, 4) ||
      !aligned(recv_scales, 4) || !aligned(topk_weights, 4) || !aligned(recv_topk_weights, 4))
    return fail(EP_EINVAL, "%s: misaligned pointer (rows need 16 bytes)", what);
  *row_bytes = rb;
  *scale_cols = sc;
  return EP_OK;
}

}  // namespace

extern "C" {

int ep_layout(const int32_t *topk_idx, int32_t num_tokens, int32_t topk, int32_t num_experts,
              int32_t expert_alignment, int64_t capacity_rows, int32_t *counts,
              int32_t *offsets, int32_t *dst_slot, int32_t *recv_src_metadata,
              int32_t *num_recv, void *workspace, size_t workspace_bytes, int32_t *dispatch_plan,
              const void *prefetch, size_t prefetch_bytes, void *stream) {
  try {
    const char *what = "ep_layout";
    discard_stale_error();
    if (int rc = check_layout(what, topk_idx, num_tokens, topk, num_experts, expert_alignment,
                              capacity_rows, counts, offsets, dst_slot, recv_src_metadata,
                              num_recv, workspace, workspace_bytes))
      return rc;
    if (!aligned(dispatch_plan, 8))
      return fail(EP_EINVAL, "%s: dispatch_plan must be 8-byte aligned", what);
    if (int rc = check_prefetch(what, prefetch, prefetch_bytes)) return rc;
    ep::LayoutArgs a{topk_idx, num_tokens, topk, num_experts, expert_alignment, counts, offsets,
                     dst_slot, recv_src_metadata, num_recv, workspace, dispatch_plan,
                     (hipStream_t)stream, prefetch, (int64_t)prefetch_bytes};
    return from_launch(ep::launch_layout(a), what);
  } catch (const std::exception &e) {
    return fail(EP_EHIP, "ep_layout: %s", e.what());
  } catch (...) {
    return fail(EP_EHIP, "ep_layout: unknown exception");
  }
}

int ep_layout_noalloc(const int32_t *topk_idx, int32_t num_tokens, int32_t topk,
                      int32_t num_experts, int32_t expert_alignment, int64_t capacity_rows,
                      int32_t *counts, int32_t *offsets, int32_t *dst_slot,
                      int32_t *recv_src_metadata, int32_t *num_recv, int32_t *dispatch_plan,
                      const void *prefetch, size_t prefetch_bytes, void *stream) {
  try {
    const char *what = "ep_layout_noalloc";
    discard_stale_error();
    if (int rc = check_topk(what, num_tokens, topk)) return rc;
    if (num_experts < 1 || num_experts > EP_MAX_EXPERTS)
      return fail(EP_EINVAL, "%s: num_experts must be in 1..%d (got %d)", what, EP_MAX_EXPERTS,
                  num_experts);
    const size_t need = ep::layout_workspace(num_tokens, topk, num_experts);
    if (need > (size_t)EP_LAYOUT_SCRATCH_BYTES)
      return fail(EP_EINVAL,
                  "%s: %d tokens x top-%d over %d experts need %zu bytes of layout scratch, "
                  "above the fixed %zu (use ep_layout with a workspace)",
                  what, num_tokens, topk, num_experts, need, (size_t)EP_LAYOUT_SCRATCH_BYTES);
    void *scratch = nullptr;
    if (need > 0) {  // the arguments are checked in full below, before any launch
      int dev = -1, stream_dev = -1;
      hipError_t e = hipGetDevice(&dev);
      if (e == hipSuccess) e = hipStreamGetDevice((hipStream_t)stream, &stream_dev);
      if (e != hipSuccess)
        return fail(EP_EHIP, "%s: cannot read the current device: %s", what, hipGetErrorString(e));
      if (stream_dev != dev)
        return fail(EP_EINVAL, "%s: the stream belongs to device %d, the current device is %d",
                    what, stream_dev, dev);
      e = ep::layout_scratch(dev, &scratch);
      if (e != hipSuccess)
        return fail(EP_EHIP, "%s: cannot resolve device %d's layout scratch: %s", what, dev,
                    hipGetErrorString(e));
    }
    if (int rc = check_layout(what, topk_idx, num_tokens, topk, num_experts, expert_alignment,
                              capacity_rows, counts, offsets, dst_slot, recv_src_metadata,
                              num_recv, scratch, need))
      return rc;
    if (!aligned(dispatch_plan, 8))
      return fail(EP_EINVAL, "%s: dispatch_plan must be 8-byte aligned", what);
    if (int rc = check_prefetch(what, prefetch, prefetch_bytes)) return rc;
    ep::LayoutArgs a{topk_idx, num_tokens, topk, num_experts, expert_alignment, counts, offsets,
                     dst_slot, recv_src_metadata, num_recv, scratch, dispatch_plan,
                     (hipStream_t)stream, prefetch, (int64_t)prefetch_bytes};
    return from_launch(ep::launch_layout(a), what);
  } catch (const std::exception &e) {
    return fail(EP_EHIP, "ep_layout_noalloc: %s", e.what());
  } catch (...) {
    return fail(EP_EHIP, "ep_layout_noalloc: unknown exception");
  }
}

int ep_dispatch(const void *x, const float *x_scales, const float *topk_weights,
                const int32_t *dst_slot, int32_t num_tokens, int32_t hidden, int32_t topk,
                int32_t dtype, int64_t capacity_rows, void *expand_x, float *expand_scales,
                float *expand_weights, const int32_t *dispatch_plan, void *stream) {
  try {
    const char *what = "ep_dispatch";
    discard_stale_error();
    int64_t row_bytes = 0;
    if (int rc = check_dispatch(what, x, x_scales, topk_weights, dst_slot, num_tokens, hidden,
                                topk, dtype, capacity_rows, expand_x, expand_scales,
                                expand_weights, &row_bytes))
      return rc;
    if (!aligned(dispatch_plan, 8))
      return fail(EP_EINVAL, "%s: misaligned pointer (rows need 16 bytes, the plan 8)", what);
    ep::DispatchArgs a{x, x_scales, topk_weights, dst_slot, num_tokens, hidden, topk, dtype,
                       capacity_rows, expand_x, expand_scales, expand_weights, dispatch_plan,
                       (hipStream_t)stream};
    return from_launch(ep::launch_dispatch(a), what);
  } catch (const std::exception &e) {
    return fail(EP_EHIP, "ep_dispatch: %s", e.what());
  } catch (...) {
    return fail(EP_EHIP, "ep_dispatch: unknown exception");
  }
}

int ep_layout_dispatch(const int32_t *topk_idx, int32_t num_tokens, int32_t topk,
                       int32_t num_experts, int32_t expert_alignment, int64_t capacity_rows,
                       int32_t *counts, int32_t *offsets, int32_t *dst_slot,
                       int32_t *recv_src_metadata, int32_t *num_recv, void *workspace,
                       size_t workspace_bytes, const void *x, const float *x_scales,
                       const float *topk_weights, int32_t hidden, int32_t dtype, void *expand_x,
                       float *expand_scales, float *expand_weights, void *stream) {
  try {
    const char *what = "ep_layout_dispatch";
    discard_stale_error();
    if (int rc = check_layout(what, topk_idx, num_tokens, topk, num_experts, expert_alignment,
                              capacity_rows, counts, offsets, dst_slot, recv_src_metadata,
                              num_recv, workspace, workspace_bytes))
      return rc;
    int64_t row_bytes = 0;
    if (int rc = check_dispatch(what, x, x_scales, topk_weights, dst_slot, num_tokens, hidden,
                                topk, dtype, capacity_rows, expand_x, expand_scales,
                                expand_weights, &row_bytes))
      return rc;
    ep::LayoutArgs l{topk_idx, num_tokens, topk, num_experts, expert_alignment, counts, offsets,
                     dst_slot, recv_src_metadata, num_recv, workspace, nullptr,
                     (hipStream_t)stream};
    ep::DispatchArgs d{x, x_scales, topk_weights, dst_slot, num_tokens, hidden, topk, dtype,
                       capacity_rows, expand_x, expand_scales, expand_weights, nullptr,
                       (hipStream_t)stream};
    if (num_tokens > 0) {
      const int64_t elems = dtype == EP_FP4X2 ? 2 * (int64_t)hidden : hidden;
      // whole 16-byte chunks: every compiled byte-row width is a multiple of 512 elements
      const int scale_chunks = x_scales != nullptr ? (int)(elems / 128 * 4 / 16) : 0;
      const int rc = ep::launch_layout_dispatch(l, d, (int)(row_bytes / 16), scale_chunks);
      if (rc != -3) return from_launch(rc, what);
    }
    // more than one tile (or nothing to copy): the two launches of ep_layout and ep_dispatch,
    // walking a dispatch plan kept in the workspace when it has room for one
    const size_t base = ep::layout_workspace(num_tokens, topk, num_experts);
    const size_t plan_bytes = (size_t)num_tokens * topk * 8;
    if (aligned(workspace, 16) && workspace != nullptr &&
        workspace_bytes >= plan_offset(base) + plan_bytes) {
      int32_t *plan = (int32_t *)((char *)workspace + plan_offset(base));
      l.plan = plan;
      d.plan = plan;
    }
    if (int rc = from_launch(ep::launch_layout(l), what)) return rc;
    return from_launch(ep::launch_dispatch(d), what);
  } catch (const std::exception &e) {
    return fail(EP_EHIP, "ep_layout_dispatch: %s", e.what());
  } catch (...) {
    return fail(EP_EHIP, "ep_layout_dispatch: unknown exception");
  }
}

int ep_combine(const void *expert_out, const float *topk_weights, const void *bias,
               const int32_t *dst_slot, int32_t num_tokens, int32_t hidden, int32_t topk,
               int32_t dtype, int64_t capacity_rows, void *out, void *stream) {
  try {
    const char *what = "ep_combine";
    discard_stale_error();
    if (int rc = check_topk(what, num_tokens, topk)) return rc;
    if (dtype == EP_FP8_E4M3 || dtype == EP_FP4X2)
      return fail(EP_EINVAL, "%s: combine sums its input; byte dtype %d is rejected", what, dtype);
    if (dtype != EP_BF16 && dtype != EP_FP32)
      return fail(EP_EINVAL, "%s: unknown dtype %d", what, dtype);
    const int elt = dtype == EP_BF16 ? 2 : 4;
    if (hidden < 1 || ((int64_t)hidden * elt) % 16 != 0)
      return fail(EP_EINVAL, "%s: token bytes must be a positive multiple of 16 (hidden %d)", what,
                  hidden);
    if (capacity_rows < 0) return fail(EP_EINVAL, "%s: capacity_rows must be >= 0", what);
    if (num_tokens > 0 && (!expert_out || !dst_slot || !out))
      return fail(EP_EINVAL, "%s: a required pointer is NULL", what);
    if (!aligned(expert_out, 16) || !aligned(out, 16) || !aligned(bias, 16) ||
        !aligned(dst_slot, 4) || !aligned(topk_weights, 4))
      return fail(EP_EINVAL, "%s: misaligned pointer (rows need 16 bytes)", what);
    if (!ep::has_combine(hidden, topk, dtype))
      return fail(EP_EUNSUPPORTED, "%s: (hidden %d, topk %d, dtype %d) has no compiled kernel",
                  what, hidden, topk, dtype);
    ep::CombineArgs a{expert_out, topk_weights, bias, dst_slot, num_tokens, hidden, topk, dtype,
                      capacity_rows, out, (hipStream_t)stream};
    return from_launch(ep::launch_combine(a), what);
  } catch (const std::exception &e) {
    return fail(EP_EHIP, "ep_combine: %s", e.what());
  } catch (...) {
    return fail(EP_EHIP, "ep_combine: unknown exception");
  }
}

int ep_zero_padding(void *expand_x, int64_t row_bytes, float *expand_scales, int64_t scale_cols,
                    float *expand_weights, const int32_t *counts, const int32_t *offsets,
                    int32_t num_experts, int32_t expert_alignment, int64_t capacity_rows,
                    void *stream) {
  try {
    const char *what = "ep_zero_padding";
    discard_stale_error();
    if (num_experts < 1 || num_experts > EP_MAX_EXPERTS)
      return fail(EP_EINVAL, "%s: num_experts must be in 1..%d (got %d)", what, EP_MAX_EXPERTS,
                  num_experts);
    if (expert_alignment < 1)
      return fail(EP_EINVAL, "%s: expert_alignment must be >= 1 (got %d)", what, expert_alignment);
    if (row_bytes < 16 || row_bytes % 16 != 0 || row_bytes > INT32_MAX)
      return fail(EP_EINVAL,
                  "%s: row_bytes must be a positive multiple of 16 below 2^31 (got %lld)", what,
                  (long long)row_bytes);
    if (capacity_rows < 0 || scale_cols < 0)
      return fail(EP_EINVAL, "%s: capacity_rows and scale_cols must be >= 0", what);
    if (!expand_x || !counts || !offsets || (scale_cols > 0 && !expand_scales))
      return fail(EP_EINVAL, "%s: a required pointer is NULL", what);
    if (!aligned(expand_x, 16) || !aligned(expand_scales, 4) || !aligned(expand_weights, 4) ||
        !aligned(counts, 4) || !aligned(offsets, 4))
      return fail(EP_EINVAL, "%s: misaligned pointer (rows need 16 bytes)", what);
    ep::ZeroPaddingArgs a{expand_x, row_bytes, scale_cols > 0 ? expand_scales : nullptr,
                          scale_cols, expand_weights, counts, offsets, num_experts,
                          expert_alignment, capacity_rows, (hipStream_t)stream};
    return from_launch(ep::launch_zero_padding(a), what);
  } catch (const std::exception &e) {
    return fail(EP_EHIP, "ep_zero_padding: %s", e.what());
  } catch (...) {
    return fail(EP_EHIP, "ep_zero_padding: unknown exception");
  }
}

int ep_dispatch_compact(const void *x, const float *x_scales, const int32_t *topk_idx,
                        const float *topk_weights, const int32_t *dst_slot,
                        const int32_t *recv_src_metadata, const int32_t *num_recv,
                        int32_t num_tokens, int32_t hidden, int32_t topk, int32_t dtype,
                        void *recv_x, float *recv_scales, int32_t *recv_topk_idx,
                        float *recv_topk_weights, void *stream) {
  try {
    const char *what = "ep_dispatch_compact";
    discard_stale_error();
    int64_t row_bytes = 0, scale_cols = 0;
    if (int rc = check_dispatch_compact(what, x, x_scales, topk_idx, topk_weights, num_tokens,
                                        hidden, topk, dtype, recv_x, recv_scales, recv_topk_idx,
                                        recv_topk_weights, &row_bytes, &scale_cols))
      return rc;
    if (num_tokens > 0 && (!dst_slot || !recv_src_metadata || !num_recv))
      return fail(EP_EINVAL, "%s: a required pointer is NULL", what);
    ep::CompactDispatchArgs a{x, row_bytes, x_scales, scale_cols, topk_idx,
                              recv_topk_weights ? topk_weights : nullptr, dst_slot,
                              recv_src_metadata, num_recv, num_tokens, topk, recv_x,
                              recv_scales, recv_topk_idx,
                              topk_weights ? recv_topk_weights : nullptr, (hipStream_t)stream};
    return from_launch(ep::launch_dispatch_compact(a), what);
  } catch (const std::exception &e) {
    return fail(EP_EHIP, "ep_dispatch_compact: %s", e.what());
  } catch (...) {
    return fail(EP_EHIP, "ep_dispatch_compact: unknown exception");
  }
}

int ep_layout_dispatch_compact(const int32_t *topk_idx, int32_t num_tokens, int32_t topk,
                               int32_t num_experts, int32_t expert_alignment,
                               int64_t capacity_rows, int32_t *counts, int32_t *offsets,
                               int32_t *dst_slot, int32_t *recv_src_metadata, int32_t *num_recv,
                               void *workspace, size_t workspace_bytes, const void *x,
                               const float *x_scales, const float *topk_weights, int32_t hidden,
                               int32_t dtype, void *recv_x, float *recv_scales,
                               int32_t *recv_topk_idx, float *recv_topk_weights, void *stream) {
  try {
    const char *what = "ep_layout_dispatch_compact";
    discard_stale_error();
    if (int rc = check_layout(what, topk_idx, num_tokens, topk, num_experts, expert_alignment,
                              capacity_rows, counts, offsets, dst_slot, recv_src_metadata,
                              num_recv, workspace, workspace_bytes))
      return rc;
    int64_t row_bytes = 0, scale_cols = 0;
    if (int rc = check_dispatch_compact(what, x, x_scales, topk_idx, topk_weights, num_tokens,
                                        hidden, topk, dtype, recv_x, recv_scales, recv_topk_idx,
                                        recv_topk_weights, &row_bytes, &scale_cols))
      return rc;
    ep::LayoutArgs l{topk_idx, num_tokens, topk, num_experts, expert_alignment, counts, offsets,
                     dst_slot, recv_src_metadata, num_recv, workspace, nullptr,
                     (hipStream_t)stream};
    ep::CompactDispatchArgs d{x, row_bytes, x_scales, scale_cols, topk_idx,
                              recv_topk_weights ? topk_weights : nullptr, dst_slot,
                              recv_src_metadata, num_recv, num_tokens, topk, recv_x,
                              recv_scales, recv_topk_idx,
                              topk_weights ? recv_topk_weights : nullptr, (hipStream_t)stream};
    if (num_tokens > 0) {
      const int rc = ep::launch_layout_dispatch_compact(l, d);
      if (rc != -3) return from_launch(rc, what);
    }
    // more than one tile (or no tokens): the launches of ep_layout and ep_dispatch_compact
    if (int rc = from_launch(ep::launch_layout(l), what)) return rc;
    return from_launch(ep::launch_dispatch_compact(d), what);
  } catch (const std::exception &e) {
    return fail(EP_EHIP, "ep_layout_dispatch_compact: %s", e.what());
  } catch (...) {
    return fail(EP_EHIP, "ep_layout_dispatch_compact: unknown exception");
  }
}

int ep_combine_compact(const void *expert_out, const void *bias, const int32_t *dst_slot,
                       const int32_t *recv_src_metadata, const int32_t *num_recv,
                       int32_t num_tokens, int32_t hidden, int32_t topk, int32_t dtype, void *out,
                       void *stream) {
  try {
    const char *what = "ep_combine_compact";
    discard_stale_error();
    if (int rc = check_topk(what, num_tokens, topk)) return rc;
    if (dtype == EP_FP8_E4M3 || dtype == EP_FP4X2)
      return fail(EP_EINVAL, "%s: combine adds its input; byte dtype %d is rejected", what, dtype);
    if (dtype != EP_BF16 && dtype != EP_FP32)
      return fail(EP_EINVAL, "%s: unknown dtype %d", what, dtype);
    const int64_t elt = dtype == EP_FP32 ? 4 : 2;
    if (hidden < 1 || ((int64_t)hidden * elt) % 16 != 0 || (int64_t)hidden * elt > INT32_MAX)
      return fail(EP_EINVAL,
                  "%s: token bytes must be a positive multiple of 16 below 2^31 (hidden %d)", what,
                  hidden);
    if (num_tokens > 0 && (!expert_out || !dst_slot || !recv_src_metadata || !num_recv || !out))
      return fail(EP_EINVAL, "%s: a required pointer is NULL", what);
    if (!aligned(expert_out, 16) || !aligned(out, 16) || !aligned(bias, 16))
      return fail(EP_EINVAL, "%s: misaligned pointer (rows need 16 bytes)", what);
    ep::CompactCombineArgs a{expert_out, (int64_t)hidden * elt, bias, dst_slot,
                             recv_src_metadata, num_recv, num_tokens, topk, out,
                             (hipStream_t)stream, dtype == EP_FP32};
    return from_launch(ep::launch_combine_compact(a), what);
  } catch (const std::exception &e) {
    return fail(EP_EHIP, "ep_combine_compact: %s", e.what());
  } catch (...) {
    return fail(EP_EHIP, "ep_combine_compact: unknown exception");
  }
}

}  // extern "C"
