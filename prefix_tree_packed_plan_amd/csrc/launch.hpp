// Internal kernel launchers shared by api.cpp and the .hip files.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tg {

struct ConvArgs {
  const void* x;
  const void* w;
  const void* bias;  // may be null
  void* y;
  int32_t n_tok;
  int32_t channels;
  int32_t width;  // 1..4
  int32_t dtype;  // TREE_DTYPE_*
  int32_t act;    // TREE_ACT_*
  const int32_t* seg_off;  // device, n_seg + 1
  const int32_t* hist;     // device, n_seg * (width - 1)
  int32_t n_seg;
  const void* init_ctx;    // [n_roots, width - 1, channels] or null (zeros)
  void* ctx_out;           // [n_seg, width - 1, channels] or null
  const int32_t* ctx_src;  // device, n_seg * (width - 1)
};

// Returns hipSuccess or the launch error.
hipError_t launch_conv(const ConvArgs& a, hipStream_t stream);

struct ConvBwdArgs {
  const void* x;
  const void* w;
  const void* bias;      // may be null
  const void* dy;
  const void* init_ctx;  // may be null
  void* dx;
  float* dw;             // [C, W]
  float* dbias;          // [C] or null
  float* dinit_ctx;      // [n_roots, W-1, C] or null
  float* heads;          // workspace [n_seg (W-1), C]: dz of each segment's first W-1 tokens
  float* part;           // workspace [n_part, C, W + 1]: per-block dw, dbias partials
  int32_t n_part;
  int32_t n_tok;
  int32_t channels;
  int32_t width;
  int32_t dtype;
  int32_t act;
  int32_t n_seg;
  int32_t n_roots;
  const int32_t* seg_off;
  const int32_t* hist;
  const int32_t* fut_off;  // [n_seg (W-1) + 1]
  const int32_t* fut;      // head rows m steps past a segment's end
  const int32_t* ent_off;  // [n_seg (W-1) + 1]
  const int32_t* ent;      // head rows m steps after a segment's start
  const int32_t* roots;    // [n_roots], segment order
};

hipError_t launch_conv_backward(const ConvBwdArgs& a, hipStream_t stream);

struct ScanArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  void* o;
  const float* init;  // [n_roots, h_v, d_k, d_v] initial states of the roots, or null (zeros)
  const int32_t* root_idx;  // root rank of each segment, -1 for a non-root
  float* states;  // [n_seg, h_v, d_k, d_v] or null
  float* slots;   // [n_parents, h_v, d_k, d_v] when states is null
  const int32_t* seg_off;
  const int32_t* parent;
  const int32_t* slot;
  const int32_t* items;     // segments of this launch (level mode)
  const int32_t* walk_off;  // rescan walks: walk w is walk[walk_off[w] .. walk_off[w+1]-1]
  const int32_t* walk;      // segment index (owned) or its complement (not owned)
  int32_t n_items;          // segments (level mode) or walks (rescan mode)
  int32_t h_qk;
  int32_t h_v;
  float scale;
  float* ckpt;              // checkpoint pass: the scan backward's checkpoint slots
  const int32_t* gck;       // checkpoint pass: first slot of each segment
  float* tws;               // checkpoint pass: T, KK, QK of every 16-token chunk [total_chunks, h_v, 3, 16, 16]
  const int32_t* gchunk;    // checkpoint pass: first 16-token chunk of each segment
};

// One launch over `n_items` work items x h_v value heads: segments of one
// level (paths = false) or rescan walks (paths = true).  Returns
// hipErrorInvalidValue for a head size that is not compiled in.
hipError_t launch_scan(const ScanArgs& a, int d_k, int d_v, int dtype, bool paths, hipStream_t stream);

// bf16, d_k = d_v = 128: the DMA-fed kernel (gdn_scan_d128.hip).
hipError_t launch_scan_d128(const ScanArgs& a, bool paths, hipStream_t stream);
// The same kernel as the scan backward's checkpoint pass: every segment of
// `items` from its parent's final state in `states` (read only; `init` for
// roots), writing the start state of every kBwdCkpt-th 16-token chunk (every
// 128 tokens) to ckpt at slot gck[seg] + j, as 16x16 tiles in the lanes'
// accumulator order, and every 16-token chunk's T, KK and QK to tws (the
// prep kernel's tables); no output.
hipError_t launch_scan_d128_checkpoints(const ScanArgs& a, hipStream_t stream);

// Whether (d_k, d_v, dtype) has a compiled scan kernel.
bool scan_supported(int d_k, int d_v, int dtype);

// The scan backward keeps the start state of every kBwdCkpt-th chunk of a
// segment (a checkpoint) and re-runs the chunks between two checkpoints
// forward when it reaches them.
constexpr int kBwdCkpt = 8;

// Cache-policy operand of the buffer load/store builtins on gfx950: bit 1 is
// NT (non-temporal), which L2 keeps as the first line to evict.  For data a
// work-group reads or writes exactly once.
constexpr int kCacheNT = 2;

struct ScanBwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const void* dout;
  const float* dstates;  // [n_seg, h_v, d, d] or null
  const float* init;     // [n_roots, h_v, d, d] or null (zeros)
  const float* states;   // the forward's final states [n_seg, h_v, d, d]
  float* dq;             // [N, dq_heads, d]
  float* dk;             // [N, dq_heads, d]
  float* dv;             // [N, h_v, d]
  float* dg;             // [N, h_v]
  float* dbeta;          // [N, h_v]
  float* dinit;          // [n_roots, h_v, d, d] or null
  float* hws;            // workspace: checkpoint start states, every kBwdCkpt-th chunk of a segment
                         // (segment s's j-th at slot gck[s] + j) [total_ckpts, h_v, d, d]
  float* scr;            // workspace: per level work-group, the start states of the chunks after a
                         // checkpoint, re-run from it [n_items * h_v, kBwdCkpt - 1, d, d]
  float* tws;            // workspace: chunk T, KK, QK [total_chunks, h_v, 3, 16, 16]
  float* dsseg;          // workspace: start-state gradients [n_seg, h_v, d, d]
  const int32_t* seg_off;
  const int32_t* parent;
  const int32_t* root_idx;
  const int32_t* kid_off;
  const int32_t* kid;
  const int32_t* gchunk;
  const int32_t* chunk_seg;
  const int32_t* gck;    // first checkpoint slot of each segment
  int32_t n_chunks;      // total chunks (prep launch)
  int32_t n_seg;         // segments (states launch)
  // A level launch runs two groups of work items: value heads head_off,
  // head_off + head_step, ... of the n_items segments at items (group 0),
  // then those from head_off2 of the n_items2 segments at items2 (group 1).
  // A group with dq_accum set adds its part of dq, dk instead of storing it.
  const int32_t* items;
  int32_t n_items;
  const int32_t* items2;
  int32_t n_items2;
  int32_t head_step;
  int32_t head_off, head_off2;
  int32_t dq_accum, dq_accum2;
  int32_t h_qk;
  int32_t h_v;
  int32_t dq_heads;      // h_qk (dq, dk written per q/k head) or h_v (per value head)
  float scale;
};

// Scan backward (gdn_backward.hip); d = d_k = d_v.  The prep launches compute
// every chunk's T, KK and QK (state-free) and the checkpoint start states;
// then the level launches, deepest level first.
// Prep (T, KK, QK of every chunk, when `tables`) and, with `states`, the
// checkpoint pass of the states kernel.
hipError_t launch_scan_backward_prep(const ScanBwdArgs& a, int d, int dtype, bool tables, bool states,
                                     hipStream_t stream);
hipError_t launch_scan_backward_level(const ScanBwdArgs& a, int d, int dtype, hipStream_t stream);
// dst[t, j] = sum_m src[t, j group + m] over [n_tok, h_qk * group, d] fp32.
hipError_t launch_head_group_sum(const float* src, float* dst, int64_t n_tok, int h_qk, int group, int d,
                                 hipStream_t stream);
bool scan_backward_supported(int d_k, int d_v, int dtype);

struct SsdArgs {
  const void* x;       // [N, n_heads, head_dim]
  const float* dt;     // [N, n_heads], after softplus
  const float* A;      // [n_heads], < 0
  const void* B;       // [N, n_groups, d_state]
  const void* C;       // [N, n_groups, d_state]
  const float* D;      // [n_heads] or null
  void* y;             // [N, n_heads, head_dim]
  const float* init;   // [n_roots, n_heads, d_state, head_dim] or null (zeros)
  float* states;       // [n_seg, n_heads, d_state, head_dim] or null
  float* slots;        // [n_parents, n_heads, d_state, head_dim] when states is null
  const int32_t* seg_off;
  const int32_t* parent;
  const int32_t* slot;
  const int32_t* root_idx;
  const int32_t* items;  // segments of this level
  int32_t n_items;
  int32_t n_groups;
  int32_t n_heads;
};

// Mamba2 (SSD) forward over one trie level (ssd_scan.hip).
hipError_t launch_ssd_scan(const SsdArgs& a, int d_state, int head_dim, int dtype, hipStream_t stream);
bool ssd_supported(int d_state, int head_dim, int dtype);

}  // namespace tg
