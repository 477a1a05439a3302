// Internal launchers of the MoE kernels (host side).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "combine.h"

namespace moe {

constexpr int kMaxExperts = 512;

// Sets the thread's moe_last_error() text (moe_api.cpp).
void set_last_error(const char* msg);
constexpr int kMaxTopk = 32;
constexpr int kMaxGroups = 64;

// gate.hip
// K splits of the bf16 router for these sizes (1 = none); rpart must then hold
// splits * ntok * E floats.
int router_splits(int ntok, int E, int dim, int* steps_per_split);
hipError_t launch_gate(const void* x, const void* wr, bool f32, const float* bias, int ntok,
                       int dim, int E, int n_groups, int topk_groups, int topk, bool softmax,
                       float route_scale, float* logits, float* rpart, int32_t* topk_idx,
                       float* topk_w, hipStream_t st);

// permute.hip
size_t permute_scratch_bytes(int ntok, int E);
hipError_t launch_permute(const int32_t* idx, int ntok, int topk, int E, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_token, int32_t* row_of,
                          int32_t* scratch, hipStream_t st);

// ffn.hip
enum class WKind { F32, BF16, FP8 };

// What the shared expert's down projection does with its output.
enum class SharedDown { None, Store, Combine };

struct FfnProblem {
  const void* x;               // [T, dim] act dtype (bf16 or f32)
  const uint8_t* xq;           // fp8 path: [T, dim] e4m3 codes of x
  const float* xs;             // fp8 path: [T, dim/128] scales
  const int32_t* sorted_token; // [T*topk]
  const int32_t* offsets;      // [E+1]
  const void *w1, *w3, *w2;    // routed weights
  const float *w1s, *w3s, *w2s;
  const void *ws1, *ws3, *ws2; // shared weights (NULL = no shared expert)
  const float *ws1s, *ws3s, *ws2s;
  void* h;                     // routed h [T*topk, inter] (bf16 / f32 / e4m3)
  float* hscale;               // fp8: routed h scales [T*topk, inter/128]
  void* hs;                    // shared h [T, inter_s]
  float* hsscale;              // fp8: shared h scales [T, inter_s/128]
  void* out;                   // routed outputs [T*topk, dim] act dtype
  void* shared_out;            // shared outputs [T, dim] act dtype (SharedDown::Store)
  int32_t* sched;              // scratch, 3 * (E + 2) ints
  int ntok, dim, E, topk, inter, inter_s;
  int e_begin, e_end;          // routed experts computed: [e_begin, e_end)
  bool act_f32;
  WKind wkind;
  bool routed;                 // compute the routed experts (offsets, sorted_token, out)
  bool shared_up;              // the shared expert's up projection (needs ws1, ws3, hs)
  SharedDown shared_down;      // its down projection: skipped, stored, or fused with the combine
  CombineArgs comb;            // SharedDown::Combine: the routed rows, weights and y
  hipEvent_t ev[4];            // optional timing: up start/end, down start/end (or null)
};

// The fused combine needs the token's slots sorted in registers.
inline bool ffn_can_fuse_combine(int topk) { return topk <= kRegSlots; }

size_t ffn_h_bytes(int ntok, int topk, int inter, int inter_s, WKind wk, bool act_f32);
hipError_t launch_ffn(const FfnProblem& p, hipStream_t st);
// A launch counts its work-items (workgroups x threads) in 32 bits.
constexpr long kMaxLaunchItems = 0xFFFFFFFFL;
// Work-items of the largest launch launch_ffn makes for these shapes (host only).
long ffn_max_items(int ntok, int topk, int E, int dim, int inter, int inter_s, WKind wk,
                   bool has_shared);
constexpr int kSchedInts(int E) { return 3 * (E + 2); }
hipError_t launch_quant_x(const uint16_t* x, int ntok, int dim, uint8_t* xq, float* xs,
                          hipStream_t st);

// pack.hip
hipError_t launch_pack_weights(const uint8_t* src, int64_t rows, int64_t row_bytes, uint8_t* dst,
                               hipStream_t st);

// calib.hip (measurement only): one streaming read of bytes (multiple of 16)
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st);

// combine.hip: the stand-alone combine, y = cast(sum_k w O + S) with the
// arithmetic of combine.h; shared_out may be NULL (no shared expert).
hipError_t launch_combine(const CombineArgs& c, const void* shared_out, int ntok, int dim,
                          bool act_f32, hipStream_t st);

}  // namespace moe
