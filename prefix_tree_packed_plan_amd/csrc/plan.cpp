// Host-side trie plan.  See plan.hpp.
#include "plan.hpp"

#include <algorithm>
#include <cstdio>

#include "../../include/tree_gdn.h"

namespace tg {

namespace {
std::string fmt(const char* f, long a, long b = 0, long c = 0) {
  char buf[256];
  std::snprintf(buf, sizeof(buf), f, a, b, c);
  return buf;
}
}  // namespace

int build_plan(const int32_t* parents, const int32_t* seg_lens, int32_t n_seg,
               int32_t conv_width, Plan* out, std::string* err) {
  if (!parents || !seg_lens || !out) {
    *err = "tree_plan: null pointer argument";
    return TREE_ERR_INVALID_ARG;
  }
  if (n_seg <= 0) {
    *err = fmt("tree_plan: n_seg must be >= 1 (got %ld)", n_seg);
    return TREE_ERR_BAD_TREE;
  }
  if (conv_width < 1 || conv_width > 8) {
    *err = fmt("tree_plan: conv_width must be in 1..8 (got %ld)", conv_width);
    return TREE_ERR_INVALID_ARG;
  }
  Plan p;
  p.n_seg = n_seg;
  p.width = conv_width;
  p.parents.assign(parents, parents + n_seg);
  p.lens.assign(seg_lens, seg_lens + n_seg);

  // Validate and take offsets: parents precede children, so one forward pass
  // over the segments gives depths and path lengths too.
  p.seg_off.assign(n_seg + 1, 0);
  p.depth.assign(n_seg, 0);
  std::vector<int64_t> path_len(n_seg, 0);
  std::vector<int32_t> n_children(n_seg, 0);
  int64_t total = 0;
  for (int32_t i = 0; i < n_seg; ++i) {
    const int32_t par = p.parents[i];
    if (par < -1 || par >= i) {
      *err = fmt("tree_plan: parents[%ld] = %ld is not in [-1, %ld)", i, par, i);
      return TREE_ERR_BAD_TREE;
    }
    if (p.lens[i] <= 0) {
      *err = fmt("tree_plan: seg_lens[%ld] = %ld must be >= 1", i, p.lens[i]);
      return TREE_ERR_BAD_TREE;
    }
    p.seg_off[i] = static_cast<int32_t>(total);
    total += p.lens[i];
    if (total >= (int64_t(1) << 31)) {
      *err = "tree_plan: total token count must be < 2^31";
      return TREE_ERR_BAD_TREE;
    }
    if (par >= 0) {
      p.depth[i] = p.depth[par] + 1;
      path_len[i] = path_len[par] + p.lens[i];
      n_children[par] += 1;
    } else {
      path_len[i] = p.lens[i];
      p.n_roots += 1;
    }
  }
  p.seg_off[n_seg] = static_cast<int32_t>(total);
  p.n_tokens = total;

  // Leaves, path statistics and state slots (one per segment with children).
  p.slot.assign(n_seg, -1);
  for (int32_t i = 0; i < n_seg; ++i) {
    if (n_children[i] == 0) {
      p.n_leaves += 1;
      p.path_tokens += path_len[i];
      p.max_path_tokens = std::max(p.max_path_tokens, path_len[i]);
    } else {
      p.slot[i] = p.n_parents++;
    }
  }

  // Levels: by depth, longest segment first inside a level (ties by index),
  // so the longest work items of a level are dispatched first.
  int32_t max_depth = 0;
  for (int32_t i = 0; i < n_seg; ++i) max_depth = std::max(max_depth, p.depth[i]);
  p.n_levels = max_depth + 1;
  p.order.resize(n_seg);
  for (int32_t i = 0; i < n_seg; ++i) p.order[i] = i;
  std::stable_sort(p.order.begin(), p.order.end(), [&](int32_t a, int32_t b) {
    if (p.depth[a] != p.depth[b]) return p.depth[a] < p.depth[b];
    return p.lens[a] > p.lens[b];
  });
  p.level_start.assign(p.n_levels + 1, 0);
  for (int32_t i = 0; i < n_seg; ++i) p.level_start[p.depth[i] + 1] += 1;
  for (int32_t l = 0; l < p.n_levels; ++l) p.level_start[l + 1] += p.level_start[l];

  // Conv history: the W-1 packed rows preceding segment i on its path are the
  // last W-1 entries of (hist[parent] ++ rows of parent); -1 pads at a root.
  const int32_t H = conv_width - 1;
  p.hist.assign(static_cast<size_t>(n_seg) * H, -1);
  std::vector<int32_t> ext;
  for (int32_t i = 0; i < n_seg && H > 0; ++i) {
    const int32_t par = p.parents[i];
    if (par < 0) continue;
    ext.assign(p.hist.begin() + static_cast<size_t>(par) * H,
               p.hist.begin() + static_cast<size_t>(par + 1) * H);
    const int32_t take = std::min(p.lens[par], H);
    for (int32_t j = p.lens[par] - take; j < p.lens[par]; ++j) ext.push_back(p.seg_off[par] + j);
    std::copy(ext.end() - H, ext.end(), p.hist.begin() + static_cast<size_t>(i) * H);
  }

  // Device mirror.
  p.m_seg_off = 0;
  p.m_parent = p.m_seg_off + n_seg + 1;
  p.m_slot = p.m_parent + n_seg;
  p.m_hist = p.m_slot + n_seg;
  p.m_order = p.m_hist + p.hist.size();
  p.mirror.resize(p.m_order + n_seg);
  std::copy(p.seg_off.begin(), p.seg_off.end(), p.mirror.begin() + p.m_seg_off);
  std::copy(p.parents.begin(), p.parents.end(), p.mirror.begin() + p.m_parent);
  std::copy(p.slot.begin(), p.slot.end(), p.mirror.begin() + p.m_slot);
  std::copy(p.hist.begin(), p.hist.end(), p.mirror.begin() + p.m_hist);
  std::copy(p.order.begin(), p.order.end(), p.mirror.begin() + p.m_order);

  *out = std::move(p);
  return TREE_OK;
}

}  // namespace tg
