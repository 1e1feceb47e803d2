// Host-side trie plan (no HIP headers: this file and plan.cpp build and run
// without a GPU).
//
// The tree-recurrence 0.1.0 project page ("How a tree runs") makes one such
// plan on the host per forward pass and runs every kernel on it: segment
// offsets, the level schedule that lets every segment start from its
// parent's final state ("Tree Training" section 3.2, Eq. 10: parents precede
// children), and the conv history table that gives each segment the last
// W-1 inputs of its own path (section 3.2, Eq. 11).
//
// History entries: h >= 0 is a packed token row; h < 0 is position
// -1 - h of the roots' caller-given contexts (root r, context row j, oldest
// first: code -1 - (r (W-1) + j)), which read as zeros when no context is
// given.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

namespace tg {

struct Plan {
  int32_t n_seg = 0;
  int32_t width = 0;  // conv width W
  int64_t n_tokens = 0;
  int32_t n_roots = 0, n_leaves = 0, n_parents = 0, n_levels = 0;
  int64_t path_tokens = 0, max_path_tokens = 0;

  std::vector<int32_t> parents, lens, seg_off, depth, slot, hist;
  // root_idx[s]: rank of root s among the roots in segment order, -1 for a
  // non-root.  ctx_src[s][j]: source of the j-th (oldest first) of the W-1
  // path inputs ending at segment s's last token, coded like hist.
  std::vector<int32_t> root_idx, ctx_src;
  std::vector<int32_t> level_start;  // n_levels + 1
  std::vector<int32_t> order;        // segments by (level, length desc, index)

  // Rescan walks: one per leaf, longest path first (ties by leaf index).
  // Walk w is entries path_seg[path_off[w] .. path_off[w+1]-1], the segments
  // of the leaf's root path from the root down; an entry is the segment
  // index when this walk owns the segment's outputs and state (the walk of
  // the lowest-indexed leaf below it), its bitwise complement otherwise.
  // Empty (and paths_ok false) when the table would exceed kMaxPathEntries.
  static constexpr int64_t kMaxPathEntries = int64_t(1) << 26;
  bool paths_ok = false;
  int64_t path_entries = 0;  // sum over leaves of (depth + 1)
  std::vector<int32_t> path_off, path_seg;

  // Conv backward: "head" rows h = s (W-1) + j name token j < W-1 of segment
  // s.  ent[s][m] (CSR over s (W-1) + m) lists the head rows of the tokens
  // m steps after segment s's first token along any path (s's own token m
  // if it has one, else the children's, recursively); fut[s][m] those m + 1
  // steps after s's last token, i.e. the union of the children's ent[c][m].
  // roots: the roots in segment order.
  std::vector<int32_t> ent_off, ent, fut_off, fut, roots;

  // Scan backward: kid[kid_off[s] .. kid_off[s+1]-1] are segment s's
  // children in index order (the fixed order in which their start-state
  // gradients are summed into s's final-state gradient).  gchunk[s] is the
  // offset of s's first kBwdChunk-token chunk among all chunks in segment
  // order, chunk_seg[c] the segment of chunk c (total_chunks of them).
  // The backward keeps the start state of every kBwdCkpt-th chunk of a
  // segment; gck[s] is the offset of s's first such checkpoint among all of
  // them in segment order (total_ckpts of them).
  static constexpr int32_t kBwdChunk = 16;
  static constexpr int32_t kBwdCkpt = 8;
  std::vector<int32_t> kid_off, kid, gchunk, chunk_seg, gck;
  int64_t total_chunks = 0;
  int64_t total_ckpts = 0;

  // Device copy: one int32 array; element offsets of each table inside it.
  std::vector<int32_t> mirror;
  size_t m_seg_off = 0, m_parent = 0, m_slot = 0, m_hist = 0, m_order = 0, m_root = 0, m_ctx = 0;
  size_t m_path_off = 0, m_path_seg = 0;
  size_t m_ent_off = 0, m_ent = 0, m_fut_off = 0, m_fut = 0, m_roots = 0;
  size_t m_kid_off = 0, m_kid = 0, m_gchunk = 0, m_chunk_seg = 0, m_gck = 0;

  size_t device_bytes() const { return mirror.size() * sizeof(int32_t); }
};

// The fork/rescan choice (TREE_SCHED_LEVEL or TREE_SCHED_RESCAN) for a
// launch priced at `min_saved` scanned tokens (>= 0).
int32_t choose_schedule(const Plan& p, int64_t min_saved);

// Returns 0 or a negative TREE_ERR_* code; on failure *err holds a message.
int build_plan(const int32_t* parents, const int32_t* seg_lens, int32_t n_seg,
               int32_t conv_width, Plan* out, std::string* err);

}  // namespace tg
