// C ABI (include/tree_gdn.h): argument checks, the device plan, launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/tree_gdn.h"
#include "launch.hpp"
#include "plan.hpp"

struct tree_plan {
  tg::Plan p;
  // Device buffers this plan was uploaded into (tree_plan_upload) and their
  // sizes.  The entry points accept a device plan only from this list, so a
  // stale, short or foreign buffer is rejected on the host before any launch.
  // The plan is otherwise immutable; the list has its own lock so that the
  // plan can be shared across threads.
  mutable std::mutex mu;
  mutable std::vector<std::pair<const void*, size_t>> uploads;
};

namespace {

thread_local std::string g_err;

int fail(int code, const char* f, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, f);
  std::vsnprintf(buf, sizeof(buf), f, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(const char* what, hipError_t e) {
  return fail(TREE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool dtype_ok(int32_t d) { return d == TREE_DTYPE_F32 || d == TREE_DTYPE_BF16; }

// The device plan passed to an entry point must be one tree_plan_upload made
// from this plan, of at least the plan's device size.
int check_dplan(const tree_plan_t* plan, const void* dplan, size_t dplan_bytes, const char* fn) {
  const size_t need = plan->p.device_bytes();
  if (dplan_bytes < need)
    return fail(TREE_ERR_WORKSPACE, "%s: dplan has %zu bytes, the plan needs %zu", fn, dplan_bytes, need);
  std::lock_guard<std::mutex> lock(plan->mu);
  for (const auto& u : plan->uploads)
    if (u.first == dplan) {
      if (dplan_bytes > u.second)
        return fail(TREE_ERR_INVALID_ARG, "%s: dplan_bytes %zu exceeds the %zu bytes it was uploaded with", fn,
                    dplan_bytes, u.second);
      return TREE_OK;
    }
  return fail(TREE_ERR_INVALID_ARG, "%s: dplan %p is not an upload of this plan (tree_plan_upload)", fn, dplan);
}

// Blocks along the tokens of the conv backward (each walks every n-th tile).
int32_t conv_bwd_parts(const tg::Plan& p) {
  const int64_t tiles = (p.n_tokens + 63) / 64;
  return static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(tiles, 512)));
}

}  // namespace

extern "C" {

int tree_plan(const int32_t* parents, const int32_t* seg_lens, int32_t n_seg, int32_t conv_width,
              tree_plan_t** out) {
  if (!out) return fail(TREE_ERR_INVALID_ARG, "tree_plan: out is null");
  *out = nullptr;
  tree_plan_t* plan = new (std::nothrow) tree_plan_t;
  if (!plan) return fail(TREE_ERR_INVALID_ARG, "tree_plan: out of host memory");
  std::string err;
  const int rc = tg::build_plan(parents, seg_lens, n_seg, conv_width, &plan->p, &err);
  if (rc != TREE_OK) {
    delete plan;
    g_err = err;
    return rc;
  }
  *out = plan;
  return TREE_OK;
}

void tree_plan_free(tree_plan_t* plan) { delete plan; }

int tree_plan_query(const tree_plan_t* plan, tree_plan_stats_t* out) {
  if (!plan || !out) return fail(TREE_ERR_INVALID_ARG, "tree_plan_query: null argument");
  const tg::Plan& p = plan->p;
  out->n_tokens = p.n_tokens;
  out->path_tokens = p.path_tokens;
  out->max_path_tokens = p.max_path_tokens;
  out->por = p.path_tokens > 0 ? 1.0 - static_cast<double>(p.n_tokens) / p.path_tokens : 0.0;
  out->n_seg = p.n_seg;
  out->n_roots = p.n_roots;
  out->n_leaves = p.n_leaves;
  out->n_parents = p.n_parents;
  out->n_levels = p.n_levels;
  out->conv_width = p.width;
  out->path_entries = p.paths_ok ? p.path_entries : -1;
  return TREE_OK;
}

int tree_plan_paths(const tree_plan_t* plan, int32_t* path_off, int32_t* path_seg) {
  if (!plan || !path_off || !path_seg) return fail(TREE_ERR_INVALID_ARG, "tree_plan_paths: null argument");
  if (!plan->p.paths_ok)
    return fail(TREE_ERR_UNSUPPORTED, "tree_plan_paths: walk table of %lld entries not built",
                static_cast<long long>(plan->p.path_entries));
  std::copy(plan->p.path_off.begin(), plan->p.path_off.end(), path_off);
  std::copy(plan->p.path_seg.begin(), plan->p.path_seg.end(), path_seg);
  return TREE_OK;
}

int tree_plan_choose_schedule(const tree_plan_t* plan, int64_t fork_min_saved_tokens, int32_t* sched) {
  if (!plan || !sched) return fail(TREE_ERR_INVALID_ARG, "tree_plan_choose_schedule: null argument");
  if (fork_min_saved_tokens < 0)
    return fail(TREE_ERR_INVALID_ARG, "tree_plan_choose_schedule: fork_min_saved_tokens %lld < 0",
                static_cast<long long>(fork_min_saved_tokens));
  *sched = tg::choose_schedule(plan->p, fork_min_saved_tokens);
  return TREE_OK;
}

int tree_plan_conv_history(const tree_plan_t* plan, int32_t* hist) {
  if (!plan || !hist) return fail(TREE_ERR_INVALID_ARG, "tree_plan_conv_history: null argument");
  std::copy(plan->p.hist.begin(), plan->p.hist.end(), hist);
  return TREE_OK;
}

int tree_plan_levels(const tree_plan_t* plan, int32_t* level_start, int32_t* order) {
  if (!plan || !level_start || !order)
    return fail(TREE_ERR_INVALID_ARG, "tree_plan_levels: null argument");
  std::copy(plan->p.level_start.begin(), plan->p.level_start.end(), level_start);
  std::copy(plan->p.order.begin(), plan->p.order.end(), order);
  return TREE_OK;
}

size_t tree_plan_device_bytes(const tree_plan_t* plan) { return plan ? plan->p.device_bytes() : 0; }

int tree_plan_upload(const tree_plan_t* plan, void* dplan, size_t dplan_bytes, void* stream) {
  if (!plan || !dplan) return fail(TREE_ERR_INVALID_ARG, "tree_plan_upload: null argument");
  if (dplan_bytes < plan->p.device_bytes())
    return fail(TREE_ERR_WORKSPACE, "tree_plan_upload: dplan has %zu bytes, needs %zu", dplan_bytes,
                plan->p.device_bytes());
  const hipError_t e = hipMemcpyAsync(dplan, plan->p.mirror.data(), plan->p.device_bytes(),
                                      hipMemcpyHostToDevice, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("tree_plan_upload: hipMemcpyAsync", e);
  std::lock_guard<std::mutex> lock(plan->mu);
  for (auto& u : plan->uploads)
    if (u.first == dplan) {
      u.second = dplan_bytes;
      return TREE_OK;
    }
  plan->uploads.emplace_back(dplan, dplan_bytes);
  return TREE_OK;
}

int tree_conv(const void* x, const void* w, const void* bias, void* y, const void* init_ctx,
              void* ctx_out, int64_t n_tokens, int32_t channels, int32_t dtype, int32_t act,
              const tree_plan_t* plan, const void* dplan, size_t dplan_bytes, void* stream) {
  if (!plan || !x || !w || !y || !dplan) return fail(TREE_ERR_INVALID_ARG, "tree_conv: null argument");
  const tg::Plan& p = plan->p;
  if (n_tokens != p.n_tokens)
    return fail(TREE_ERR_SIZE, "tree_conv: n_tokens %lld != plan tokens %lld",
                static_cast<long long>(n_tokens), static_cast<long long>(p.n_tokens));
  if (channels <= 0) return fail(TREE_ERR_INVALID_ARG, "tree_conv: channels must be > 0");
  if (!dtype_ok(dtype)) return fail(TREE_ERR_INVALID_ARG, "tree_conv: bad dtype %d", dtype);
  if (act != TREE_ACT_NONE && act != TREE_ACT_SILU)
    return fail(TREE_ERR_INVALID_ARG, "tree_conv: bad activation %d", act);
  if (p.width > 4) return fail(TREE_ERR_UNSUPPORTED, "tree_conv: conv width %d > 4", p.width);
  if (x == y) return fail(TREE_ERR_INVALID_ARG, "tree_conv: y must not alias x");
  if (ctx_out != nullptr && (ctx_out == x || ctx_out == y || ctx_out == init_ctx))
    return fail(TREE_ERR_INVALID_ARG, "tree_conv: ctx_out must not alias x, y or init_ctx");
  if (const int rc = check_dplan(plan, dplan, dplan_bytes, "tree_conv")) return rc;
  const int32_t* base = static_cast<const int32_t*>(dplan);
  tg::ConvArgs a{x, w, bias, y, static_cast<int32_t>(n_tokens), channels, p.width, dtype, act,
                 base + p.m_seg_off, base + p.m_hist, p.n_seg, init_ctx, ctx_out, base + p.m_ctx};
  const hipError_t e = tg::launch_conv(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("tree_conv: launch", e);
  return TREE_OK;
}

size_t tree_conv_backward_workspace_bytes(const tree_plan_t* plan, int32_t channels) {
  if (!plan || channels <= 0) return 0;
  const tg::Plan& p = plan->p;
  const size_t heads = static_cast<size_t>(p.n_seg) * std::max(p.width - 1, 0) * channels;
  const size_t part = static_cast<size_t>(conv_bwd_parts(p)) * channels * (p.width + 1);
  return (heads + part) * sizeof(float);
}

int tree_conv_backward(const void* x, const void* w, const void* bias, const void* dy, const void* init_ctx,
                       void* dx, float* dw, float* dbias, float* dinit_ctx, int64_t n_tokens, int32_t channels,
                       int32_t dtype, int32_t act, const tree_plan_t* plan, const void* dplan,
                       size_t dplan_bytes, void* ws, size_t ws_bytes, void* stream) {
  if (!plan || !x || !w || !dy || !dx || !dw || !dplan)
    return fail(TREE_ERR_INVALID_ARG, "tree_conv_backward: null argument");
  const tg::Plan& p = plan->p;
  if (n_tokens != p.n_tokens)
    return fail(TREE_ERR_SIZE, "tree_conv_backward: n_tokens %lld != plan tokens %lld",
                static_cast<long long>(n_tokens), static_cast<long long>(p.n_tokens));
  if (channels <= 0) return fail(TREE_ERR_INVALID_ARG, "tree_conv_backward: channels must be > 0");
  if (!dtype_ok(dtype)) return fail(TREE_ERR_INVALID_ARG, "tree_conv_backward: bad dtype %d", dtype);
  if (act != TREE_ACT_NONE && act != TREE_ACT_SILU)
    return fail(TREE_ERR_INVALID_ARG, "tree_conv_backward: bad activation %d", act);
  if (p.width > 4) return fail(TREE_ERR_UNSUPPORTED, "tree_conv_backward: conv width %d > 4", p.width);
  if (dx == x || dx == dy) return fail(TREE_ERR_INVALID_ARG, "tree_conv_backward: dx must not alias x or dy");
  const size_t need = tree_conv_backward_workspace_bytes(plan, channels);
  if (!ws || ws_bytes < need)
    return fail(TREE_ERR_WORKSPACE, "tree_conv_backward: workspace has %zu bytes, needs %zu", ws ? ws_bytes : 0,
                need);
  if (const int rc = check_dplan(plan, dplan, dplan_bytes, "tree_conv_backward")) return rc;
  const int32_t* base = static_cast<const int32_t*>(dplan);
  tg::ConvBwdArgs a{};
  a.x = x;
  a.w = w;
  a.bias = bias;
  a.dy = dy;
  a.init_ctx = init_ctx;
  a.dx = dx;
  a.dw = dw;
  a.dbias = bias ? dbias : nullptr;
  a.dinit_ctx = p.width > 1 ? dinit_ctx : nullptr;
  a.heads = static_cast<float*>(ws);
  a.part = a.heads + static_cast<size_t>(p.n_seg) * std::max(p.width - 1, 0) * channels;
  a.n_part = conv_bwd_parts(p);
  a.n_tok = static_cast<int32_t>(n_tokens);
  a.channels = channels;
  a.width = p.width;
  a.dtype = dtype;
  a.act = act;
  a.n_seg = p.n_seg;
  a.n_roots = p.n_roots;
  a.seg_off = base + p.m_seg_off;
  a.hist = base + p.m_hist;
  a.fut_off = base + p.m_fut_off;
  a.fut = base + p.m_fut;
  a.ent_off = base + p.m_ent_off;
  a.ent = base + p.m_ent;
  a.roots = base + p.m_roots;
  const hipError_t e = tg::launch_conv_backward(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("tree_conv_backward: launch", e);
  return TREE_OK;
}

size_t tree_scan_workspace_bytes(const tree_plan_t* plan, int32_t h_v, int32_t d_k, int32_t d_v,
                                 int32_t with_states) {
  if (!plan || h_v <= 0 || d_k <= 0 || d_v <= 0 || with_states) return 0;
  return static_cast<size_t>(plan->p.n_parents) * h_v * d_k * d_v * sizeof(float);
}

size_t tree_workspace_bytes(const tree_plan_t* plan, int32_t h_v, int32_t d_k, int32_t d_v, int32_t sched) {
  if (!plan) return 0;
  if (sched == TREE_SCHED_AUTO) sched = tg::choose_schedule(plan->p, TREE_FORK_MIN_SAVED_TOKENS);
  if (sched != TREE_SCHED_LEVEL) return 0;
  return tree_scan_workspace_bytes(plan, h_v, d_k, d_v, 0);
}

}  // extern "C"

namespace {

// Argument checks shared by tree_gdn_scan and tree_gdn_scan_noalloc (all but
// the device plan and the workspace).  Resolves AUTO into *sched and returns
// in *need the parent-slot bytes the level schedule needs.
int check_scan(const char* fn, const void* q, const void* k, const void* v, const float* g, const float* beta,
               void* o, const float* states, int64_t n_tokens, int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v,
               int32_t dtype, int32_t* sched, const tree_plan_t* plan, size_t* need) {
  if (!plan || !q || !k || !v || !g || !beta || !o) return fail(TREE_ERR_INVALID_ARG, "%s: null argument", fn);
  const tg::Plan& p = plan->p;
  if (n_tokens != p.n_tokens)
    return fail(TREE_ERR_SIZE, "%s: n_tokens %lld != plan tokens %lld", fn, static_cast<long long>(n_tokens),
                static_cast<long long>(p.n_tokens));
  if (h_qk <= 0 || h_v <= 0 || d_k <= 0 || d_v <= 0)
    return fail(TREE_ERR_INVALID_ARG, "%s: head counts and sizes must be > 0", fn);
  if (h_v % h_qk != 0)
    return fail(TREE_ERR_UNSUPPORTED, "%s: h_v %d is not a multiple of h_qk %d", fn, h_v, h_qk);
  if (!dtype_ok(dtype)) return fail(TREE_ERR_INVALID_ARG, "%s: bad dtype %d", fn, dtype);
  if (*sched == TREE_SCHED_AUTO) *sched = tg::choose_schedule(p, TREE_FORK_MIN_SAVED_TOKENS);
  if (*sched != TREE_SCHED_LEVEL && *sched != TREE_SCHED_RESCAN)
    return fail(TREE_ERR_INVALID_ARG, "%s: bad schedule %d", fn, *sched);
  if (*sched == TREE_SCHED_RESCAN && !p.paths_ok)
    return fail(TREE_ERR_UNSUPPORTED, "%s: rescan walk table of %lld entries not built", fn,
                static_cast<long long>(p.path_entries));
  if (!tg::scan_supported(d_k, d_v, dtype))
    return fail(TREE_ERR_UNSUPPORTED, "%s: d_k=%d d_v=%d dtype=%d not compiled in", fn, d_k, d_v, dtype);
  *need = *sched == TREE_SCHED_LEVEL ? tree_scan_workspace_bytes(plan, h_v, d_k, d_v, states != nullptr) : 0;
  return TREE_OK;
}

// The scan's launches on a device plan `base` and parent-state slots `slots`.
int launch_scan_levels(const char* fn, const void* q, const void* k, const void* v, const float* g,
                       const float* beta, void* o, const float* init_states, float* states, int32_t h_qk,
                       int32_t h_v, int32_t d_k, int32_t d_v, float scale, int32_t dtype, int32_t sched,
                       const tg::Plan& p, const int32_t* base, float* slots, hipStream_t st) {
  tg::ScanArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.o = o;
  a.init = init_states;
  a.root_idx = base + p.m_root;
  a.states = states;
  a.slots = slots;
  a.seg_off = base + p.m_seg_off;
  a.parent = base + p.m_parent;
  a.slot = base + p.m_slot;
  a.h_qk = h_qk;
  a.h_v = h_v;
  a.scale = scale;
  if (sched == TREE_SCHED_RESCAN) {
    a.walk_off = base + p.m_path_off;
    a.walk = base + p.m_path_seg;
    a.n_items = p.n_leaves;
    const hipError_t e = tg::launch_scan(a, d_k, d_v, dtype, true, st);
    if (e != hipSuccess) return hip_fail(fn, e);
    return TREE_OK;
  }
  for (int32_t l = 0; l < p.n_levels; ++l) {
    a.items = base + p.m_order + p.level_start[l];
    a.n_items = p.level_start[l + 1] - p.level_start[l];
    const hipError_t e = tg::launch_scan(a, d_k, d_v, dtype, false, st);
    if (e != hipSuccess) return hip_fail(fn, e);
  }
  return TREE_OK;
}

// Device scratch of tree_gdn_scan_noalloc: the device plan at offset 0, the
// parent-state slots from the next 256-byte boundary.  Each GPU holds its own
// copy for the life of the process.  In host code `scratch` names a host-side
// stand-in, never the device memory: the device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) unsigned char scratch[TREE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_on_current_device(const char* fn, unsigned char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(fn, e);
  if (dev < 0 || dev >= kMaxDevices) return fail(TREE_ERR_UNSUPPORTED, "%s: device %d out of range", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(fn, e);
    if (!ptr) return fail(TREE_ERR_HIP, "%s: no device address for the scratch array", fn);
    g_scratch_ptr[dev] = ptr;
  }
  *out = static_cast<unsigned char*>(g_scratch_ptr[dev]);
  return TREE_OK;
}

}  // namespace

extern "C" {

int tree_gdn_scan(const void* q, const void* k, const void* v, const float* g, const float* beta,
                  void* o, const float* init_states, float* states, int64_t n_tokens, int32_t h_qk,
                  int32_t h_v, int32_t d_k, int32_t d_v, float scale, int32_t dtype, int32_t sched,
                  const tree_plan_t* plan, const void* dplan, size_t dplan_bytes, void* ws, size_t ws_bytes,
                  void* stream) {
  size_t need = 0;
  if (const int rc = check_scan("tree_gdn_scan", q, k, v, g, beta, o, states, n_tokens, h_qk, h_v, d_k, d_v, dtype,
                                &sched, plan, &need))
    return rc;
  if (!dplan) return fail(TREE_ERR_INVALID_ARG, "tree_gdn_scan: null argument");
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(TREE_ERR_WORKSPACE, "tree_gdn_scan: workspace has %zu bytes, needs %zu", ws ? ws_bytes : 0,
                need);
  if (const int rc = check_dplan(plan, dplan, dplan_bytes, "tree_gdn_scan")) return rc;
  return launch_scan_levels("tree_gdn_scan: launch", q, k, v, g, beta, o, init_states, states, h_qk, h_v, d_k, d_v,
                            scale, dtype, sched, plan->p, static_cast<const int32_t*>(dplan),
                            static_cast<float*>(ws), static_cast<hipStream_t>(stream));
}

int tree_gdn_scan_noalloc(const void* q, const void* k, const void* v, const float* g, const float* beta, void* o,
                          const float* init_states, float* states, int64_t n_tokens, int32_t h_qk, int32_t h_v,
                          int32_t d_k, int32_t d_v, float scale, int32_t dtype, int32_t sched,
                          const tree_plan_t* plan, void* stream) {
  const char* fn = "tree_gdn_scan_noalloc";
  size_t need = 0;
  if (const int rc = check_scan(fn, q, k, v, g, beta, o, states, n_tokens, h_qk, h_v, d_k, d_v, dtype, &sched,
                                plan, &need))
    return rc;
  const size_t plan_bytes = plan->p.device_bytes();
  const size_t slot_off = (plan_bytes + 255) / 256 * 256;
  if (slot_off + need > TREE_NOALLOC_SCRATCH_BYTES)
    return fail(TREE_ERR_WORKSPACE,
                "%s: needs %zu bytes of scratch (device plan %zu + parent states %zu), the static maximum is %zu; "
                "pass `states` (then no parent slots are needed) or use tree_gdn_scan with a workspace",
                fn, slot_off + need, plan_bytes, need, static_cast<size_t>(TREE_NOALLOC_SCRATCH_BYTES));
  unsigned char* ptr = nullptr;
  if (const int rc = scratch_on_current_device(fn, &ptr)) return rc;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // The device plan goes into the scratch on the caller's stream, ahead of
  // the launches that read it.  Nothing in the scratch needs clearing: every
  // parent slot is written by its parent before a child reads it.
  const hipError_t e = hipMemcpyAsync(ptr, plan->p.mirror.data(), plan_bytes, hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return hip_fail("tree_gdn_scan_noalloc: hipMemcpyAsync", e);
  return launch_scan_levels("tree_gdn_scan_noalloc: launch", q, k, v, g, beta, o, init_states, states, h_qk, h_v,
                            d_k, d_v, scale, dtype, sched, plan->p, reinterpret_cast<const int32_t*>(ptr),
                            reinterpret_cast<float*>(ptr + slot_off), st);
}

}  // extern "C"

namespace {

static_assert(tg::kBwdCkpt == tg::Plan::kBwdCkpt, "one checkpoint interval for the plan and the kernels");

// Scan backward workspace, in floats, in this order: checkpoint states (slot
// gck[s] + j for segment s's j-th),
// one start-state gradient per segment, every chunk's T, KK and QK, the
// level work-groups' re-run scratch (kBwdCkpt - 1 states each, for the
// largest level), and per-value-head dq, dk when h_v > 2 h_qk.
struct BwdLayout {
  size_t ck, dsseg, tws, scr, per_head, total;
};

BwdLayout bwd_layout(const tg::Plan& p, int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v) {
  const size_t dd = static_cast<size_t>(d_k) * d_v;
  int32_t max_level = 0;
  for (int32_t l = 0; l < p.n_levels; ++l) max_level = std::max(max_level, p.level_start[l + 1] - p.level_start[l]);
  BwdLayout b{};
  b.ck = 0;
  b.dsseg = b.ck + static_cast<size_t>(p.total_ckpts) * h_v * dd;
  b.tws = b.dsseg + static_cast<size_t>(p.n_seg) * h_v * dd;
  b.scr = b.tws + static_cast<size_t>(p.total_chunks) * h_v * 3 * tg::Plan::kBwdChunk * tg::Plan::kBwdChunk;
  b.per_head = b.scr + static_cast<size_t>(max_level) * h_v * (tg::kBwdCkpt - 1) * dd;
  b.total = b.per_head + (h_v > 2 * h_qk ? 2 * static_cast<size_t>(p.n_tokens) * h_v * d_k : 0);
  return b;
}

}  // namespace

extern "C" {

size_t tree_gdn_scan_backward_workspace_bytes(const tree_plan_t* plan, int32_t h_qk, int32_t h_v, int32_t d_k,
                                              int32_t d_v) {
  if (!plan || h_qk <= 0 || h_v <= 0 || d_k <= 0 || d_v <= 0) return 0;
  return bwd_layout(plan->p, h_qk, h_v, d_k, d_v).total * sizeof(float);
}

int tree_gdn_scan_backward(const void* q, const void* k, const void* v, const float* g, const float* beta,
                           const void* dout, const float* dstates, const float* init_states,
                           const float* states, float* dq, float* dk, float* dv, float* dg, float* dbeta,
                           float* dinit_states, int64_t n_tokens, int32_t h_qk, int32_t h_v, int32_t d_k,
                           int32_t d_v, float scale, int32_t dtype, const tree_plan_t* plan, const void* dplan,
                           size_t dplan_bytes, void* ws, size_t ws_bytes, void* stream) {
  if (!plan || !q || !k || !v || !g || !beta || !dout || !states || !dq || !dk || !dv || !dg || !dbeta || !dplan)
    return fail(TREE_ERR_INVALID_ARG, "tree_gdn_scan_backward: null argument");
  const tg::Plan& p = plan->p;
  if (n_tokens != p.n_tokens)
    return fail(TREE_ERR_SIZE, "tree_gdn_scan_backward: n_tokens %lld != plan tokens %lld",
                static_cast<long long>(n_tokens), static_cast<long long>(p.n_tokens));
  if (h_qk <= 0 || h_v <= 0 || d_k <= 0 || d_v <= 0)
    return fail(TREE_ERR_INVALID_ARG, "tree_gdn_scan_backward: head counts and sizes must be > 0");
  if (h_v % h_qk != 0)
    return fail(TREE_ERR_UNSUPPORTED, "tree_gdn_scan_backward: h_v %d is not a multiple of h_qk %d", h_v, h_qk);
  if (!dtype_ok(dtype)) return fail(TREE_ERR_INVALID_ARG, "tree_gdn_scan_backward: bad dtype %d", dtype);
  if (!tg::scan_backward_supported(d_k, d_v, dtype))
    return fail(TREE_ERR_UNSUPPORTED, "tree_gdn_scan_backward: d_k=%d d_v=%d dtype=%d not compiled in", d_k, d_v,
                dtype);
  const size_t need = tree_gdn_scan_backward_workspace_bytes(plan, h_qk, h_v, d_k, d_v);
  if (!ws || ws_bytes < need)
    return fail(TREE_ERR_WORKSPACE, "tree_gdn_scan_backward: workspace has %zu bytes, needs %zu",
                ws ? ws_bytes : 0, need);
  if (const int rc = check_dplan(plan, dplan, dplan_bytes, "tree_gdn_scan_backward")) return rc;
  const int32_t* base = static_cast<const int32_t*>(dplan);
  const size_t dd = static_cast<size_t>(d_k) * d_v;
  tg::ScanBwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.dout = dout;
  a.dstates = dstates;
  a.init = init_states;
  a.states = states;
  a.dv = dv;
  a.dg = dg;
  a.dbeta = dbeta;
  a.dinit = dinit_states;
  const BwdLayout lay = bwd_layout(p, h_qk, h_v, d_k, d_v);
  float* const wsf = static_cast<float*>(ws);
  a.hws = wsf + lay.ck;
  a.dsseg = wsf + lay.dsseg;
  a.tws = wsf + lay.tws;
  a.scr = wsf + lay.scr;
  float* per_head = wsf + lay.per_head;
  // One value head per q/k head: dq, dk written directly.  Two: the prep
  // launch clears dq, dk and both heads add into them.  More: per-value-head
  // parts, summed in head order.
  const bool pairwise = h_v == 2 * h_qk;
  const bool grouped = h_v > 2 * h_qk;
  a.dq = grouped ? per_head : dq;
  a.dk = grouped ? per_head + static_cast<size_t>(n_tokens) * h_v * d_k : dk;
  a.dq_heads = grouped ? h_v : h_qk;
  // Pairwise: the first value head of every pair stores its part of dq, dk
  // and the second, in a later launch, adds to it (a + b either way round),
  // so nothing needs clearing.  Level l's first heads run in the launch
  // after level l + 1's first heads, together with level l + 1's second.
  a.dq_accum = 0;
  a.dq_accum2 = 0;
  a.head_step = 1;
  a.head_off = 0;
  a.head_off2 = 0;
  a.items2 = nullptr;
  a.n_items2 = 0;
  a.seg_off = base + p.m_seg_off;
  a.parent = base + p.m_parent;
  a.root_idx = base + p.m_root;
  a.kid_off = base + p.m_kid_off;
  a.kid = base + p.m_kid;
  a.gchunk = base + p.m_gchunk;
  a.chunk_seg = base + p.m_chunk_seg;
  a.gck = base + p.m_gck;
  a.n_chunks = static_cast<int32_t>(p.total_chunks);
  a.n_seg = p.n_seg;
  a.h_qk = h_qk;
  a.h_v = h_v;
  a.scale = scale;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // Checkpoints and the chunk tables: at bf16 d = 128 from the forward scan
  // kernel (32-token chunks, all segments in one launch from the given final
  // states; prep then only clears dq, dk), else from the prep and states
  // kernels.
  const bool ck_fwd = d_k == 128 && d_v == 128 && dtype == TREE_DTYPE_BF16;
  {
    hipError_t e = tg::launch_scan_backward_prep(a, d_k, dtype, !ck_fwd, !ck_fwd, st);
    if (e == hipSuccess && ck_fwd) {
      tg::ScanArgs c{};
      c.q = q;
      c.k = k;
      c.v = v;
      c.g = g;
      c.beta = beta;
      c.init = init_states;
      c.root_idx = a.root_idx;
      c.states = const_cast<float*>(states);  // read only in this pass
      c.seg_off = a.seg_off;
      c.parent = a.parent;
      c.items = base + p.m_order;  // every segment, level by level
      c.n_items = p.n_seg;
      c.h_qk = h_qk;
      c.h_v = h_v;
      c.scale = scale;
      c.ckpt = a.hws;
      c.gck = a.gck;
      c.tws = a.tws;
      c.gchunk = a.gchunk;
      e = tg::launch_scan_d128_checkpoints(c, st);
    }
    if (e != hipSuccess) return hip_fail("tree_gdn_scan_backward: launch", e);
  }
  // Deepest level first: a parent sums its children's start-state gradients.
  for (int32_t l = p.n_levels - 1; l >= (pairwise ? -1 : 0); --l) {
    const int32_t ld = l + 1;  // the level below, whose second heads run now
    a.items = l >= 0 ? base + p.m_order + p.level_start[l] : nullptr;
    a.n_items = l >= 0 ? p.level_start[l + 1] - p.level_start[l] : 0;
    a.head_step = pairwise ? 2 : 1;
    a.head_off = 0;
    a.dq_accum = 0;
    a.items2 = nullptr;
    a.n_items2 = 0;
    if (pairwise && ld < p.n_levels) {
      a.items2 = base + p.m_order + p.level_start[ld];
      a.n_items2 = p.level_start[ld + 1] - p.level_start[ld];
      a.head_off2 = 1;
      a.dq_accum2 = 1;
    }
    const hipError_t e = tg::launch_scan_backward_level(a, d_k, dtype, st);
    if (e != hipSuccess) return hip_fail("tree_gdn_scan_backward: launch", e);
  }
  if (grouped) {
    const int group = h_v / h_qk;
    hipError_t e = tg::launch_head_group_sum(a.dq, dq, n_tokens, h_qk, group, d_k, st);
    if (e == hipSuccess) e = tg::launch_head_group_sum(a.dk, dk, n_tokens, h_qk, group, d_k, st);
    if (e != hipSuccess) return hip_fail("tree_gdn_scan_backward: launch", e);
  }
  return TREE_OK;
}

int tree_ssd_scan(const void* x, const float* dt, const float* A, const void* B, const void* C, const float* D,
                  void* y, const float* init_states, float* states, int64_t n_tokens, int32_t n_groups,
                  int32_t n_heads, int32_t d_state, int32_t head_dim, int32_t dtype, const tree_plan_t* plan,
                  const void* dplan, size_t dplan_bytes, void* ws, size_t ws_bytes, void* stream) {
  if (!plan || !x || !dt || !A || !B || !C || !y || !dplan)
    return fail(TREE_ERR_INVALID_ARG, "tree_ssd_scan: null argument");
  const tg::Plan& p = plan->p;
  if (n_tokens != p.n_tokens)
    return fail(TREE_ERR_SIZE, "tree_ssd_scan: n_tokens %lld != plan tokens %lld", static_cast<long long>(n_tokens),
                static_cast<long long>(p.n_tokens));
  if (n_groups <= 0 || n_heads <= 0 || d_state <= 0 || head_dim <= 0)
    return fail(TREE_ERR_INVALID_ARG, "tree_ssd_scan: head counts and sizes must be > 0");
  if (n_heads % n_groups != 0)
    return fail(TREE_ERR_UNSUPPORTED, "tree_ssd_scan: n_heads %d is not a multiple of n_groups %d", n_heads, n_groups);
  if (!dtype_ok(dtype)) return fail(TREE_ERR_INVALID_ARG, "tree_ssd_scan: bad dtype %d", dtype);
  if (!tg::ssd_supported(d_state, head_dim, dtype))
    return fail(TREE_ERR_UNSUPPORTED, "tree_ssd_scan: d_state=%d head_dim=%d dtype=%d not compiled in", d_state,
                head_dim, dtype);
  const size_t need = tree_scan_workspace_bytes(plan, n_heads, d_state, head_dim, states != nullptr);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(TREE_ERR_WORKSPACE, "tree_ssd_scan: workspace has %zu bytes, needs %zu", ws ? ws_bytes : 0, need);
  if (const int rc = check_dplan(plan, dplan, dplan_bytes, "tree_ssd_scan")) return rc;
  const int32_t* base = static_cast<const int32_t*>(dplan);
  tg::SsdArgs a{};
  a.x = x;
  a.dt = dt;
  a.A = A;
  a.B = B;
  a.C = C;
  a.D = D;
  a.y = y;
  a.init = init_states;
  a.states = states;
  a.slots = static_cast<float*>(ws);
  a.seg_off = base + p.m_seg_off;
  a.parent = base + p.m_parent;
  a.slot = base + p.m_slot;
  a.root_idx = base + p.m_root;
  a.n_groups = n_groups;
  a.n_heads = n_heads;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  for (int32_t l = 0; l < p.n_levels; ++l) {
    a.items = base + p.m_order + p.level_start[l];
    a.n_items = p.level_start[l + 1] - p.level_start[l];
    const hipError_t e = tg::launch_ssd_scan(a, d_state, head_dim, dtype, st);
    if (e != hipSuccess) return hip_fail("tree_ssd_scan: launch", e);
  }
  return TREE_OK;
}

const char* tree_last_error(void) { return g_err.c_str(); }

}  // extern "C"
