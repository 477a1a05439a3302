// C ABI of the MoE layer forward: host-side validation, workspace layout and
// kernel launches.  Every device buffer is the caller's; nothing here
// allocates, copies to the host or synchronises.
#include "moe.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"

using moe::WKind;

namespace {

thread_local std::string g_err;

moe_status fail(moe_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

moe_status hip_fail(hipError_t e, const char* where) {
  g_err = std::string(where) + ": " + hipGetErrorString(e);
  return MOE_ERR_HIP;
}

// benchmark timing state (moe_profile_start / moe_profile_stop)
struct Profile {
  std::mutex mu;
  std::vector<hipEvent_t> ev;   // 4 per call
  int used = 0;
  bool on = false;
} g_prof;

void profile_slot(hipEvent_t (&ev)[4]) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  for (auto& e : ev) e = nullptr;
  if (!g_prof.on || (size_t)(g_prof.used + 1) * 4 > g_prof.ev.size()) return;
  for (int i = 0; i < 4; ++i) ev[i] = g_prof.ev[g_prof.used * 4 + i];
  ++g_prof.used;
}

size_t align_up(size_t n) { return (n + 255) & ~size_t(255); }

int expert_end(const moe_params* p) { return p->expert_end == 0 ? p->n_experts : p->expert_end; }
bool full_range(const moe_params* p) { return p->expert_begin == 0 && expert_end(p) == p->n_experts; }

// Workspace carve-up (offsets in bytes, each 256-byte aligned).
struct Layout {
  size_t logits, rpart, topk_idx, topk_w, counts, offsets, sorted_token, row_of, perm, sched;
  size_t h, hscale, hs, hsscale, xq, xs, out, shared_out, total;
};

size_t act_size(const moe_params* p) { return p->act_dtype == MOE_F32 ? 4 : 2; }

constexpr int kMaxWidth = 65536;   // largest dim, inter and shared_inter

WKind wkind(const moe_params* p) {
  return p->weight_dtype == MOE_FP8_E4M3 ? WKind::FP8
         : p->weight_dtype == MOE_BF16   ? WKind::BF16
                                         : WKind::F32;
}

Layout layout(const moe_params* p, int64_t T) {
  Layout L{};
  const size_t R = (size_t)T * p->topk, E = p->n_experts, asz = act_size(p);
  const bool fp8 = p->weight_dtype == MOE_FP8_E4M3;
  const size_t hsz = fp8 ? 1 : asz;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o += align_up(bytes); return at; };
  L.logits = take((size_t)T * E * 4);
  const int splits = p->act_dtype == MOE_F32 ? 1 : moe::router_splits((int)T, (int)E, p->dim, nullptr);
  L.rpart = take(splits > 1 ? (size_t)splits * T * E * 4 : 0);   // K-split router partials
  L.topk_idx = take(R * 4);
  L.topk_w = take(R * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.sorted_token = take(R * 4);
  L.row_of = take(R * 4);
  L.perm = take(moe::permute_scratch_bytes((int)T, (int)E));
  L.sched = take((size_t)moe::kSchedInts((int)E) * 4);
  L.h = take(R * p->inter * hsz);
  L.hscale = take(fp8 ? R * (p->inter / 128) * 4 : 0);
  L.hs = take((size_t)T * p->shared_inter * hsz);
  L.hsscale = take(fp8 ? (size_t)T * (p->shared_inter / 128) * 4 : 0);
  L.xq = take(fp8 ? (size_t)T * p->dim : 0);
  L.xs = take(fp8 ? (size_t)T * (p->dim / 128) * 4 : 0);
  L.out = take(R * p->dim * asz);
  L.shared_out = take((size_t)T * p->dim * asz);
  L.total = o;
  return L;
}

moe_status validate(const moe_params* p, int64_t T) {
  if (p == nullptr) return fail(MOE_ERR_INVALID_ARG, "params is NULL");
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T < 0");
  if (T >= (int64_t)1 << 24) return fail(MOE_ERR_UNSUPPORTED, "T >= 2^24 tokens");
  const int E = p->n_experts, G = p->n_groups;
  if (E < 1) return fail(MOE_ERR_INVALID_ARG, "n_experts < 1");
  if (E > moe::kMaxExperts) return fail(MOE_ERR_UNSUPPORTED, "n_experts > 512");
  if (G < 1 || E % G != 0) return fail(MOE_ERR_INVALID_ARG, "n_experts must be a multiple of n_groups >= 1");
  if (G > moe::kMaxGroups) return fail(MOE_ERR_UNSUPPORTED, "n_groups > 64");
  if (p->topk_groups < 1 || p->topk_groups > G)
    return fail(MOE_ERR_INVALID_ARG, "topk_groups must be in [1, n_groups]");
  if (p->topk < 1 || p->topk > p->topk_groups * (E / G))
    return fail(MOE_ERR_INVALID_ARG, "topk must be in [1, topk_groups * n_experts / n_groups]");
  if (p->topk > moe::kMaxTopk) return fail(MOE_ERR_UNSUPPORTED, "topk > 32");
  if (p->score_func != MOE_SCORE_SIGMOID && p->score_func != MOE_SCORE_SOFTMAX)
    return fail(MOE_ERR_INVALID_ARG, "unknown score_func");
  if (p->accumulate != MOE_ACC_F32 && p->accumulate != MOE_ACC_LAYER)
    return fail(MOE_ERR_INVALID_ARG, "unknown accumulate mode");
  const int eend = p->expert_end == 0 ? E : p->expert_end;
  if (p->expert_begin < 0 || p->expert_begin > eend || eend > E)
    return fail(MOE_ERR_INVALID_ARG, "expert range must satisfy 0 <= expert_begin <= expert_end <= n_experts");
  if (p->dim < 1 || p->inter < 1 || p->shared_inter < 0)
    return fail(MOE_ERR_INVALID_ARG, "dim and inter must be >= 1, shared_inter >= 0");
  if (p->dim > kMaxWidth || p->inter > kMaxWidth || p->shared_inter > kMaxWidth)
    return fail(MOE_ERR_UNSUPPORTED, "dim, inter and shared_inter must be <= 65536");
  const bool f32 = p->act_dtype == MOE_F32 && p->router_dtype == MOE_F32 && p->weight_dtype == MOE_F32;
  const bool bf = p->act_dtype == MOE_BF16 && p->router_dtype == MOE_BF16 &&
                  (p->weight_dtype == MOE_BF16 || p->weight_dtype == MOE_FP8_E4M3);
  if (!f32 && !bf) return fail(MOE_ERR_UNSUPPORTED, "unsupported dtype combination");
  const int q = p->weight_dtype == MOE_FP8_E4M3 ? 128 : 64;
  if (p->dim % q || p->inter % q || p->shared_inter % q)
    return fail(MOE_ERR_UNSUPPORTED, q == 128 ? "dim, inter, shared_inter must be multiples of 128 for fp8"
                                              : "dim, inter, shared_inter must be multiples of 64");
  return MOE_OK;
}

// Every launch of the expert step must fit a dispatch's 32-bit work-item count.
moe_status check_launch_size(const moe_params* p, int64_t T, bool shared) {
  const long items = moe::ffn_max_items((int)T, p->topk, p->n_experts, p->dim, p->inter,
                                        p->shared_inter, wkind(p), shared);
  if (items > moe::kMaxLaunchItems)
    return fail(MOE_ERR_UNSUPPORTED, "T and the widths give an expert launch of more than 2^32 - 1 work-items");
  return MOE_OK;
}

moe_status check_ws(const moe_params* p, int64_t T, void* ws, size_t ws_bytes) {
  const size_t need = layout(p, T).total;
  if (ws == nullptr || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace smaller than moe_workspace_size() (" +
                                       std::to_string(need) + " bytes)");
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0)
    return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return MOE_OK;
}

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

moe_status bias_rule(const moe_params* p, const float* bias) {
  if (bias != nullptr && p->n_groups > 1 && p->n_experts / p->n_groups < 2)
    return fail(MOE_ERR_INVALID_ARG, "a bias with n_groups > 1 needs >= 2 experts per group (top-2 group score)");
  return MOE_OK;
}

moe_status do_gate(const moe_params* p, int64_t T, const void* x, const void* wr,
                   const float* bias, int32_t* idx, float* w, void* ws, hipStream_t st) {
  const Layout L = layout(p, T);
  hipError_t e = moe::launch_gate(x, wr, p->act_dtype == MOE_F32, bias, (int)T, p->dim,
                                  p->n_experts, p->n_groups, p->topk_groups, p->topk,
                                  p->score_func == MOE_SCORE_SOFTMAX, p->route_scale,
                                  at<float>(ws, L.logits), at<float>(ws, L.rpart), idx, w, st);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "gate launch");
}

moe_status do_permute(const moe_params* p, int64_t T, const int32_t* idx, int32_t* counts,
                      int32_t* offsets, int32_t* sorted_token, int32_t* row_of, void* ws,
                      hipStream_t st) {
  const Layout L = layout(p, T);
  hipError_t e = moe::launch_permute(idx, (int)T, p->topk, p->n_experts, counts, offsets,
                                     sorted_token, row_of, at<int32_t>(ws, L.perm), st);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "permute launch");
}

// The parts of an expert-step problem every call shares: shapes, weights,
// workspace buffers.  The caller sets what runs (routed / shared / combine).
moe::FfnProblem ffn_problem(const moe_params* p, int64_t T, const void* x, const moe_weights* w,
                            void* ws) {
  const Layout L = layout(p, T);
  moe::FfnProblem f{};
  f.x = x;
  f.w1 = w->w1; f.w3 = w->w3; f.w2 = w->w2;
  f.w1s = w->w1_scale; f.w3s = w->w3_scale; f.w2s = w->w2_scale;
  if (p->shared_inter > 0) {
    f.ws1 = w->ws1; f.ws3 = w->ws3; f.ws2 = w->ws2;
    f.ws1s = w->ws1_scale; f.ws3s = w->ws3_scale; f.ws2s = w->ws2_scale;
  }
  f.h = at<void>(ws, L.h);
  f.hscale = at<float>(ws, L.hscale);
  f.hs = at<void>(ws, L.hs);
  f.hsscale = at<float>(ws, L.hsscale);
  f.xq = at<uint8_t>(ws, L.xq);
  f.xs = at<float>(ws, L.xs);
  f.sched = at<int32_t>(ws, L.sched);
  f.ntok = (int)T; f.dim = p->dim; f.E = p->n_experts; f.topk = p->topk;
  f.inter = p->inter; f.inter_s = p->shared_inter;
  f.e_begin = p->expert_begin; f.e_end = expert_end(p);
  f.act_f32 = p->act_dtype == MOE_F32;
  f.wkind = wkind(p);
  f.shared_down = moe::SharedDown::None;
  return f;
}

moe_status run_ffn(moe::FfnProblem& f, hipStream_t st) {
  profile_slot(f.ev);
  hipError_t e = moe::launch_ffn(f, st);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "expert launch");
}

// The shared expert and the combine (moe_combine, and the end of moe_forward,
// where f already holds the routed work).  With a shared expert and at most
// kRegSlots experts per token the combine is fused into the shared expert's
// down projection; otherwise the shared output goes through the workspace
// and the stand-alone combine adds it.
moe_status shared_and_combine(const moe_params* p, int64_t T, moe::FfnProblem& f,
                              const moe::CombineArgs& c, void* ws, hipStream_t st) {
  const Layout L = layout(p, T);
  const bool shared = p->shared_inter > 0;
  const bool fuse = shared && moe::ffn_can_fuse_combine(p->topk);
  f.shared_up = shared;
  f.shared_down = fuse ? moe::SharedDown::Combine : shared ? moe::SharedDown::Store : moe::SharedDown::None;
  f.comb = c;
  f.shared_out = shared ? at<void>(ws, L.shared_out) : nullptr;
  moe_status s = MOE_OK;
  if (f.routed || shared) s = run_ffn(f, st);
  if (s != MOE_OK || fuse) return s;
  hipError_t e = moe::launch_combine(c, f.shared_out, (int)T, p->dim, p->act_dtype == MOE_F32, st);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "combine launch");
}

moe::CombineArgs combine_args(const moe_params* p, const void* expert_out, const int32_t* row_of,
                              const float* topk_w, void* y, const int32_t* offsets) {
  moe::CombineArgs c{};
  c.out = expert_out;
  c.row_of = row_of;
  c.w = topk_w;
  c.y = y;
  c.offsets = full_range(p) ? nullptr : offsets;
  c.e_begin = p->expert_begin;
  c.e_end = expert_end(p);
  c.topk = p->topk;
  c.layer_acc = p->accumulate == MOE_ACC_LAYER;
  return c;
}

moe_status check_weights(const moe_params* p, const moe_weights* w, bool need_router,
                         bool need_shared, bool need_routed = true) {
  if (w == nullptr) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  if (need_router && w->w_router == nullptr) return fail(MOE_ERR_INVALID_ARG, "w_router is NULL");
  const bool fp8 = p->weight_dtype == MOE_FP8_E4M3;
  if (need_routed) {
    if (!w->w1 || !w->w3 || !w->w2) return fail(MOE_ERR_INVALID_ARG, "w1/w3/w2 must be non-NULL");
    if (fp8 && (!w->w1_scale || !w->w3_scale || !w->w2_scale))
      return fail(MOE_ERR_INVALID_ARG, "fp8 weights need w1/w3/w2 scales");
  }
  if (need_shared && p->shared_inter > 0) {
    if (!w->ws1 || !w->ws3 || !w->ws2) return fail(MOE_ERR_INVALID_ARG, "shared_inter > 0 needs ws1/ws3/ws2");
    if (fp8 && (!w->ws1_scale || !w->ws3_scale || !w->ws2_scale))
      return fail(MOE_ERR_INVALID_ARG, "fp8 shared weights need scales");
  }
  return MOE_OK;
}

}  // namespace

void moe::set_last_error(const char* msg) { g_err = msg; }

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_err.c_str(); }

moe_status moe_profile_start(int32_t max_calls) {
  g_err.clear();
  if (max_calls < 1 || max_calls > 100000) return fail(MOE_ERR_INVALID_ARG, "max_calls must be in [1, 100000]");
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (g_prof.on) return fail(MOE_ERR_INVALID_ARG, "profiling already started");
  g_prof.ev.assign((size_t)max_calls * 4, nullptr);
  for (auto& e : g_prof.ev) {
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      for (auto& d : g_prof.ev) if (d) (void)hipEventDestroy(d);
      g_prof.ev.clear();
      return hip_fail(r, "hipEventCreate");
    }
  }
  g_prof.used = 0;
  g_prof.on = true;
  return MOE_OK;
}

moe_status moe_profile_stop(int32_t* calls, float* up_ms, float* down_ms) {
  g_err.clear();
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (!g_prof.on) return fail(MOE_ERR_INVALID_ARG, "profiling not started");
  float up = 0.f, dn = 0.f;
  moe_status s = MOE_OK;
  for (int c = 0; c < g_prof.used && s == MOE_OK; ++c) {
    hipEvent_t* e = &g_prof.ev[(size_t)c * 4];
    float a = 0.f, b = 0.f;
    hipError_t r = hipEventSynchronize(e[3]);
    if (r == hipSuccess) r = hipEventElapsedTime(&a, e[0], e[1]);
    if (r == hipSuccess) r = hipEventElapsedTime(&b, e[2], e[3]);
    if (r != hipSuccess) s = hip_fail(r, "profile events");
    up += a;
    dn += b;
  }
  for (auto& e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.clear();
  if (calls) *calls = g_prof.used;
  if (up_ms) *up_ms = up;
  if (down_ms) *down_ms = dn;
  g_prof.used = 0;
  g_prof.on = false;
  return s;
}

moe_status moe_workspace_size(const moe_params* p, int64_t T, size_t* bytes) {
  g_err.clear();
  moe_status s = validate(p, T);
  if (s != MOE_OK) return s;
  if (bytes == nullptr) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = layout(p, T).total;
  return MOE_OK;
}

moe_status moe_gate(const moe_params* p, int64_t T, const void* x, const void* w_router,
                    const float* bias, int32_t* topk_idx, float* topk_w, void* workspace,
                    size_t workspace_bytes, void* stream) {
  g_err.clear();
  moe_status s = validate(p, T);
  if (s != MOE_OK) return s;
  if ((s = bias_rule(p, bias)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !topk_idx || !topk_w) return fail(MOE_ERR_INVALID_ARG, "NULL pointer argument");
  if ((s = check_ws(p, T, workspace, workspace_bytes)) != MOE_OK) return s;
  return do_gate(p, T, x, w_router, bias, topk_idx, topk_w, workspace, (hipStream_t)stream);
}

moe_status moe_permute(const moe_params* p, int64_t T, const int32_t* topk_idx, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_token, int32_t* row_of, void* workspace,
                       size_t workspace_bytes, void* stream) {
  g_err.clear();
  moe_status s = validate(p, T);
  if (s != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if (!topk_idx || !counts || !offsets || !sorted_token || !row_of)
    return fail(MOE_ERR_INVALID_ARG, "NULL pointer argument");
  if ((s = check_ws(p, T, workspace, workspace_bytes)) != MOE_OK) return s;
  return do_permute(p, T, topk_idx, counts, offsets, sorted_token, row_of, workspace,
                    (hipStream_t)stream);
}

moe_status moe_expert_ffn(const moe_params* p, int64_t T, const void* x,
                          const int32_t* sorted_token, const int32_t* offsets,
                          const moe_weights* w, void* expert_out, void* workspace,
                          size_t workspace_bytes, void* stream) {
  g_err.clear();
  moe_status s = validate(p, T);
  if (s != MOE_OK) return s;
  if ((s = check_launch_size(p, T, false)) != MOE_OK) return s;
  if ((s = check_weights(p, w, false, false)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if (!x || !sorted_token || !offsets || !expert_out) return fail(MOE_ERR_INVALID_ARG, "NULL pointer argument");
  if ((s = check_ws(p, T, workspace, workspace_bytes)) != MOE_OK) return s;
  moe::FfnProblem f = ffn_problem(p, T, x, w, workspace);
  f.routed = true;
  f.sorted_token = sorted_token;
  f.offsets = offsets;
  f.out = expert_out;
  return run_ffn(f, (hipStream_t)stream);
}

moe_status moe_combine(const moe_params* p, int64_t T, const void* x, const void* expert_out,
                       const int32_t* row_of, const float* topk_w, const moe_weights* w, void* y,
                       void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  moe_status s = validate(p, T);
  if (s != MOE_OK) return s;
  if (!full_range(p)) return fail(MOE_ERR_UNSUPPORTED, "moe_combine needs the full expert range");
  const bool shared = p->shared_inter > 0;
  if (shared) {
    if ((s = check_weights(p, w, false, true, false)) != MOE_OK) return s;
    if ((s = check_launch_size(p, T, true)) != MOE_OK) return s;
  }
  if (T == 0) return MOE_OK;
  if (!expert_out || !row_of || !topk_w || !y) return fail(MOE_ERR_INVALID_ARG, "NULL pointer argument");
  if (shared && !x) return fail(MOE_ERR_INVALID_ARG, "x is NULL (needed by the shared expert)");
  if ((s = check_ws(p, T, workspace, workspace_bytes)) != MOE_OK) return s;
  const moe::CombineArgs c = combine_args(p, expert_out, row_of, topk_w, y, nullptr);
  moe::FfnProblem f = shared ? ffn_problem(p, T, x, w, workspace) : moe::FfnProblem{};
  f.routed = false;
  return shared_and_combine(p, T, f, c, workspace, (hipStream_t)stream);
}

moe_status moe_quant_fp8(const void* x, int64_t rows, int32_t cols, uint8_t* q, float* scales,
                         void* stream) {
  g_err.clear();
  if (rows < 0 || cols < 128 || cols % 128 != 0)
    return fail(MOE_ERR_INVALID_ARG, "rows >= 0 and cols a positive multiple of 128 required");
  // 16 work-items per 1x128 block; a dispatch counts at most 2^32 - 1
  if (rows > (((int64_t)1 << 28) - 16) / (cols / 128))
    return fail(MOE_ERR_UNSUPPORTED, "rows * cols / 128 must be <= 2^28 - 16");
  if (rows == 0) return MOE_OK;
  if (!x || !q || !scales) return fail(MOE_ERR_INVALID_ARG, "NULL pointer argument");
  hipError_t e = moe::launch_quant_x(static_cast<const uint16_t*>(x), (int)rows, cols, q, scales,
                                     (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "quantiser launch");
}

moe_status moe_pack_weights(const void* src, int64_t rows, int64_t row_bytes, void* dst,
                            void* stream) {
  g_err.clear();
  if (rows < 0 || rows % 16 != 0 || row_bytes <= 0 || row_bytes % 64 != 0)
    return fail(MOE_ERR_INVALID_ARG, "rows a multiple of 16 and row_bytes a positive multiple of 64 required");
  if (rows == 0) return MOE_OK;
  if (!src || !dst) return fail(MOE_ERR_INVALID_ARG, "NULL pointer argument");
  if (src == dst) return fail(MOE_ERR_INVALID_ARG, "src and dst must be distinct buffers");
  hipError_t e = moe::launch_pack_weights(static_cast<const uint8_t*>(src), rows, row_bytes,
                                          static_cast<uint8_t*>(dst), (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "pack launch");
}

moe_status moe_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  g_err.clear();
  if (!buf || !sink) return fail(MOE_ERR_INVALID_ARG, "NULL pointer argument");
  if (bytes == 0 || bytes % 16 != 0) return fail(MOE_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
  hipError_t e = moe::launch_stream_read(buf, bytes, sink, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "stream-read launch");
}

moe_status moe_forward(const moe_params* p, int64_t T, const void* x, const moe_weights* w,
                       void* y, int32_t* topk_idx, float* topk_w, int32_t* counts,
                       void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  moe_status s = validate(p, T);
  if (s != MOE_OK) return s;
  if ((s = check_weights(p, w, true, true)) != MOE_OK) return s;
  if ((s = bias_rule(p, w->bias)) != MOE_OK) return s;
  if ((s = check_launch_size(p, T, p->shared_inter > 0)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if (!x || !y) return fail(MOE_ERR_INVALID_ARG, "NULL pointer argument");
  if ((s = check_ws(p, T, workspace, workspace_bytes)) != MOE_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  const Layout L = layout(p, T);
  int32_t* idx = topk_idx ? topk_idx : at<int32_t>(workspace, L.topk_idx);
  float* wt = topk_w ? topk_w : at<float>(workspace, L.topk_w);
  int32_t* cnt = counts ? counts : at<int32_t>(workspace, L.counts);
  int32_t* off = at<int32_t>(workspace, L.offsets);
  int32_t* st_tok = at<int32_t>(workspace, L.sorted_token);
  int32_t* row_of = at<int32_t>(workspace, L.row_of);
  void* out = at<void>(workspace, L.out);
  if ((s = do_gate(p, T, x, w->w_router, w->bias, idx, wt, workspace, st)) != MOE_OK) return s;
  if ((s = do_permute(p, T, idx, cnt, off, st_tok, row_of, workspace, st)) != MOE_OK) return s;
  moe::FfnProblem f = ffn_problem(p, T, x, w, workspace);
  f.routed = true;
  f.sorted_token = st_tok;
  f.offsets = off;
  f.out = out;
  return shared_and_combine(p, T, f, combine_args(p, out, row_of, wt, y, off), workspace, st);
}

}  // extern "C"
