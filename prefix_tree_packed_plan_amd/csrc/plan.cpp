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

int32_t choose_schedule(const Plan& p, int64_t min_saved) {
  // Forking saves the prefix tokens a rescan scans more than once and costs
  // one launch per level beyond the first.
  const int64_t saved = p.path_tokens - p.n_tokens;
  const int64_t extra = p.n_levels - 1;
  if (!p.paths_ok || extra == 0) return TREE_SCHED_LEVEL;
  const bool fork = min_saved == 0 || saved / extra >= min_saved;
  return fork ? TREE_SCHED_LEVEL : TREE_SCHED_RESCAN;
}

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
  // Conv history rows s (W-1) + j are int32 in every table and kernel.
  if (static_cast<int64_t>(n_seg) * (conv_width - 1) >= (int64_t(1) << 31)) {
    *err = fmt("tree_plan: n_seg (W-1) must be < 2^31 (got %ld segments, W = %ld)", n_seg, conv_width);
    return TREE_ERR_BAD_TREE;
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

  // Roots in segment order.
  p.root_idx.assign(n_seg, -1);
  for (int32_t i = 0, r = 0; i < n_seg; ++i)
    if (p.parents[i] < 0) p.root_idx[i] = r++;

  // Conv history: the W-1 rows preceding segment i on its path are the last
  // W-1 entries of (hist[parent] ++ rows of parent); a root's are its
  // context positions -1 - (r (W-1) + j).  ctx_src[i] is the same for the
  // W-1 rows ending at segment i's last token: the last W-1 entries of
  // (hist[i] ++ rows of i).
  const int32_t H = conv_width - 1;
  p.hist.assign(static_cast<size_t>(n_seg) * H, -1);
  p.ctx_src.assign(static_cast<size_t>(n_seg) * H, -1);
  std::vector<int32_t> ext;
  auto tail = [&](int32_t s, int32_t* dst) {  // last H of (hist[s] ++ rows of s)
    ext.assign(p.hist.begin() + static_cast<size_t>(s) * H, p.hist.begin() + static_cast<size_t>(s + 1) * H);
    const int32_t take = std::min(p.lens[s], H);
    for (int32_t j = p.lens[s] - take; j < p.lens[s]; ++j) ext.push_back(p.seg_off[s] + j);
    std::copy(ext.end() - H, ext.end(), dst);
  };
  for (int32_t i = 0; i < n_seg && H > 0; ++i) {
    const int32_t par = p.parents[i];
    int32_t* hi = p.hist.data() + static_cast<size_t>(i) * H;
    if (par < 0) {
      for (int32_t j = 0; j < H; ++j) hi[j] = -1 - (p.root_idx[i] * H + j);
    } else {
      tail(par, hi);
    }
    tail(i, p.ctx_src.data() + static_cast<size_t>(i) * H);
  }

  // Rescan walks (the fork-free alternative of the tree-recurrence 0.1.0
  // project page, "How a tree runs": every root-to-leaf path is scanned
  // whole, and each segment keeps the outputs of one path through it).
  // A segment is owned by the lowest-indexed leaf below it: walking the
  // segments backwards, a leaf owns itself and a parent takes the smallest
  // owner among its children.
  for (int32_t i = 0; i < n_seg; ++i)
    if (n_children[i] == 0) p.path_entries += p.depth[i] + 1;
  p.paths_ok = p.path_entries <= Plan::kMaxPathEntries;
  if (p.paths_ok) {
    std::vector<int32_t> owner(n_seg, n_seg), leaves;
    for (int32_t i = n_seg - 1; i >= 0; --i) {
      if (n_children[i] == 0) owner[i] = i;
      if (p.parents[i] >= 0) owner[p.parents[i]] = std::min(owner[p.parents[i]], owner[i]);
    }
    for (int32_t i = 0; i < n_seg; ++i)
      if (n_children[i] == 0) leaves.push_back(i);
    std::stable_sort(leaves.begin(), leaves.end(),
                     [&](int32_t a, int32_t b) { return path_len[a] > path_len[b]; });
    p.path_off.assign(1, 0);
    p.path_seg.reserve(static_cast<size_t>(p.path_entries));
    std::vector<int32_t> up;
    for (const int32_t leaf : leaves) {
      up.clear();
      for (int32_t s = leaf; s >= 0; s = p.parents[s]) up.push_back(s);
      for (auto it = up.rbegin(); it != up.rend(); ++it) p.path_seg.push_back(owner[*it] == leaf ? *it : ~*it);
      p.path_off.push_back(static_cast<int32_t>(p.path_seg.size()));
    }
  }

  // Conv backward head tables: ent bottom-up (children have larger indices).
  {
    std::vector<std::vector<int32_t>> kids(n_seg);
    for (int32_t i = 0; i < n_seg; ++i)
      if (p.parents[i] >= 0) kids[p.parents[i]].push_back(i);
      else p.roots.push_back(i);
    std::vector<std::vector<int32_t>> ent(static_cast<size_t>(n_seg) * std::max(H, 1));
    for (int32_t i = n_seg - 1; i >= 0 && H > 0; --i) {
      for (int32_t m = 0; m < H; ++m) {
        auto& e = ent[static_cast<size_t>(i) * H + m];
        if (m < p.lens[i]) {
          e.push_back(i * H + m);
        } else {
          for (const int32_t c : kids[i]) {
            const auto& ce = ent[static_cast<size_t>(c) * H + (m - p.lens[i])];
            e.insert(e.end(), ce.begin(), ce.end());
          }
        }
      }
    }
    // Both CSR tables are indexed with int32 offsets on the device.
    size_t n_ent = 0, n_fut = 0;
    for (int32_t i = 0; i < n_seg && H > 0; ++i)
      for (int32_t m = 0; m < H; ++m) {
        n_ent += ent[static_cast<size_t>(i) * H + m].size();
        for (const int32_t c : kids[i]) n_fut += ent[static_cast<size_t>(c) * H + m].size();
      }
    if (n_ent >= (size_t(1) << 31) || n_fut >= (size_t(1) << 31)) {
      *err = "tree_plan: conv backward head tables exceed 2^31 entries";
      return TREE_ERR_BAD_TREE;
    }
    p.ent.reserve(n_ent);
    p.fut.reserve(n_fut);
    p.ent_off.assign(1, 0);
    p.fut_off.assign(1, 0);
    for (int32_t i = 0; i < n_seg && H > 0; ++i) {
      for (int32_t m = 0; m < H; ++m) {
        const auto& e = ent[static_cast<size_t>(i) * H + m];
        p.ent.insert(p.ent.end(), e.begin(), e.end());
        p.ent_off.push_back(static_cast<int32_t>(p.ent.size()));
        for (const int32_t c : kids[i]) {
          const auto& ce = ent[static_cast<size_t>(c) * H + m];
          p.fut.insert(p.fut.end(), ce.begin(), ce.end());
        }
        p.fut_off.push_back(static_cast<int32_t>(p.fut.size()));
      }
    }
  }

  // Scan backward: children lists and chunk offsets.
  p.kid_off.assign(n_seg + 1, 0);
  for (int32_t i = 0; i < n_seg; ++i)
    if (p.parents[i] >= 0) p.kid_off[p.parents[i] + 1] += 1;
  for (int32_t i = 0; i < n_seg; ++i) p.kid_off[i + 1] += p.kid_off[i];
  p.kid.assign(p.kid_off[n_seg], 0);
  {
    std::vector<int32_t> fill(p.kid_off.begin(), p.kid_off.end() - 1);
    for (int32_t i = 0; i < n_seg; ++i)
      if (p.parents[i] >= 0) p.kid[fill[p.parents[i]]++] = i;
  }
  p.gchunk.assign(n_seg, 0);
  p.gck.assign(n_seg, 0);
  for (int32_t i = 0; i < n_seg; ++i) {
    p.gchunk[i] = static_cast<int32_t>(p.total_chunks);
    p.gck[i] = static_cast<int32_t>(p.total_ckpts);
    const int32_t nc = (p.lens[i] + Plan::kBwdChunk - 1) / Plan::kBwdChunk;
    for (int32_t j = 0; j < nc; ++j) p.chunk_seg.push_back(i);
    p.total_chunks += nc;
    p.total_ckpts += (nc + Plan::kBwdCkpt - 1) / Plan::kBwdCkpt;
  }

  // Device mirror.
  p.m_seg_off = 0;
  p.m_parent = p.m_seg_off + n_seg + 1;
  p.m_slot = p.m_parent + n_seg;
  p.m_hist = p.m_slot + n_seg;
  p.m_order = p.m_hist + p.hist.size();
  p.m_root = p.m_order + n_seg;
  p.m_ctx = p.m_root + n_seg;
  p.m_path_off = p.m_ctx + p.ctx_src.size();
  p.m_path_seg = p.m_path_off + p.path_off.size();
  p.m_ent_off = p.m_path_seg + p.path_seg.size();
  p.m_ent = p.m_ent_off + p.ent_off.size();
  p.m_fut_off = p.m_ent + p.ent.size();
  p.m_fut = p.m_fut_off + p.fut_off.size();
  p.m_roots = p.m_fut + p.fut.size();
  p.m_kid_off = p.m_roots + p.roots.size();
  p.m_kid = p.m_kid_off + p.kid_off.size();
  p.m_gchunk = p.m_kid + p.kid.size();
  p.m_chunk_seg = p.m_gchunk + p.gchunk.size();
  p.m_gck = p.m_chunk_seg + p.chunk_seg.size();
  p.mirror.resize(p.m_gck + p.gck.size());
  std::copy(p.seg_off.begin(), p.seg_off.end(), p.mirror.begin() + p.m_seg_off);
  std::copy(p.parents.begin(), p.parents.end(), p.mirror.begin() + p.m_parent);
  std::copy(p.slot.begin(), p.slot.end(), p.mirror.begin() + p.m_slot);
  std::copy(p.hist.begin(), p.hist.end(), p.mirror.begin() + p.m_hist);
  std::copy(p.order.begin(), p.order.end(), p.mirror.begin() + p.m_order);
  std::copy(p.root_idx.begin(), p.root_idx.end(), p.mirror.begin() + p.m_root);
  std::copy(p.ctx_src.begin(), p.ctx_src.end(), p.mirror.begin() + p.m_ctx);
  std::copy(p.path_off.begin(), p.path_off.end(), p.mirror.begin() + p.m_path_off);
  std::copy(p.path_seg.begin(), p.path_seg.end(), p.mirror.begin() + p.m_path_seg);
  std::copy(p.ent_off.begin(), p.ent_off.end(), p.mirror.begin() + p.m_ent_off);
  std::copy(p.ent.begin(), p.ent.end(), p.mirror.begin() + p.m_ent);
  std::copy(p.fut_off.begin(), p.fut_off.end(), p.mirror.begin() + p.m_fut_off);
  std::copy(p.fut.begin(), p.fut.end(), p.mirror.begin() + p.m_fut);
  std::copy(p.roots.begin(), p.roots.end(), p.mirror.begin() + p.m_roots);
  std::copy(p.kid_off.begin(), p.kid_off.end(), p.mirror.begin() + p.m_kid_off);
  std::copy(p.kid.begin(), p.kid.end(), p.mirror.begin() + p.m_kid);
  std::copy(p.gchunk.begin(), p.gchunk.end(), p.mirror.begin() + p.m_gchunk);
  std::copy(p.chunk_seg.begin(), p.chunk_seg.end(), p.mirror.begin() + p.m_chunk_seg);
  std::copy(p.gck.begin(), p.gck.end(), p.mirror.begin() + p.m_gck);

  *out = std::move(p);
  return TREE_OK;
}

}  // namespace tg
