// Host plan checker, built with AddressSanitizer and UBSan by
// test_plan_sanitize.py (host code only: plan.cpp and this file, no HIP).
//
// Random forests and degenerate shapes (one segment, chains of one-token
// segments, stars, forests of roots, every conv width) go through
// tg::build_plan; every table is compared with a brute-force reading of the
// trie built here by enumerating root-to-leaf token paths:
//   - hist / ctx_src: the W-1 path rows before a segment's first token and up
//     to its last, preceded by the root's context codes ("Tree Training"
//     section 3.2, Eq. 11: each token sees only the inputs of its own path);
//   - the level order: parents before children (Eq. 10), longest first;
//   - rescan walks: one per leaf, its root path, one owner per segment;
//   - conv backward heads: the segment-head tokens m steps along each path.
// Invalid tries and arguments must fail with the documented codes without
// reading past the arrays they were given.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <set>
#include <string>
#include <utility>
#include <vector>

#include "plan.hpp"
#include "tree_gdn.h"

namespace {

int g_fail = 0;

#define CHECK(cond, ...)                                         \
  do {                                                           \
    if (!(cond)) {                                               \
      std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);                         \
      std::fprintf(stderr, "\n");                                \
      if (++g_fail > 20) std::exit(1);                           \
      return;                                                    \
    }                                                            \
  } while (0)

// splitmix64: a seeded generator for the shapes.
struct Rng {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  int32_t below(int32_t n) { return static_cast<int32_t>(next() % static_cast<uint64_t>(n)); }
};

struct Trie {
  std::vector<int32_t> parents, lens;
};

// One token of a path: (segment, position in segment).
using Tok = std::pair<int32_t, int32_t>;

void check_plan(const Trie& t, int32_t W, const char* name) {
  const int32_t n = static_cast<int32_t>(t.parents.size());
  const int32_t H = W - 1;
  tg::Plan p;
  std::string err;
  const int rc = tg::build_plan(t.parents.data(), t.lens.data(), n, W, &p, &err);
  CHECK(rc == TREE_OK, "%s W=%d: build_plan failed: %s", name, W, err.c_str());

  // Children, depths, roots, leaves, offsets.
  std::vector<std::vector<int32_t>> kids(n);
  std::vector<int32_t> depth(n, 0), root_rank(n, -1), off(n + 1, 0);
  int32_t n_roots = 0;
  for (int32_t i = 0; i < n; ++i) {
    off[i + 1] = off[i] + t.lens[i];
    if (t.parents[i] >= 0) {
      kids[t.parents[i]].push_back(i);
      depth[i] = depth[t.parents[i]] + 1;
    } else {
      root_rank[i] = n_roots++;
    }
  }
  CHECK(p.n_seg == n && p.width == W && p.n_roots == n_roots, "%s: header fields", name);
  CHECK(p.n_tokens == off[n], "%s: n_tokens", name);
  for (int32_t i = 0; i <= n; ++i) CHECK(p.seg_off[i] == off[i], "%s: seg_off[%d]", name, i);
  for (int32_t i = 0; i < n; ++i) CHECK(p.root_idx[i] == root_rank[i], "%s: root_idx[%d]", name, i);

  // Paths: the segment chain from the root to each segment.
  auto chain = [&](int32_t s) {
    std::vector<int32_t> c;
    for (int32_t u = s; u >= 0; u = t.parents[u]) c.push_back(u);
    std::reverse(c.begin(), c.end());
    return c;
  };
  auto path_len = [&](int32_t s) {
    int64_t L = 0;
    for (const int32_t u : chain(s)) L += t.lens[u];
    return L;
  };

  // Stats.
  int32_t leaves = 0, slots = 0, max_depth = 0;
  int64_t ptok = 0, maxp = 0, entries = 0;
  for (int32_t i = 0; i < n; ++i) {
    max_depth = std::max(max_depth, depth[i]);
    if (kids[i].empty()) {
      ++leaves;
      ptok += path_len(i);
      maxp = std::max(maxp, path_len(i));
      entries += depth[i] + 1;
      CHECK(p.slot[i] == -1, "%s: leaf %d has a slot", name, i);
    } else {
      CHECK(p.slot[i] == slots, "%s: slot[%d] = %d, want %d", name, i, p.slot[i], slots);
      ++slots;
    }
  }
  CHECK(p.n_leaves == leaves && p.n_parents == slots && p.n_levels == max_depth + 1, "%s: counts", name);
  CHECK(p.path_tokens == ptok && p.max_path_tokens == maxp && p.path_entries == entries, "%s: path stats", name);

  // Level order: a permutation, grouped by depth, longest first, ties by index.
  CHECK(static_cast<int32_t>(p.level_start.size()) == max_depth + 2, "%s: level_start size", name);
  std::vector<int32_t> seen(n, 0);
  for (int32_t l = 0; l <= max_depth; ++l) {
    for (int32_t k = p.level_start[l]; k < p.level_start[l + 1]; ++k) {
      const int32_t s = p.order[k];
      CHECK(s >= 0 && s < n && !seen[s]++, "%s: order[%d] = %d", name, k, s);
      CHECK(depth[s] == l, "%s: segment %d at level %d, depth %d", name, s, l, depth[s]);
      if (k > p.level_start[l]) {
        const int32_t q = p.order[k - 1];
        CHECK(t.lens[q] > t.lens[s] || (t.lens[q] == t.lens[s] && q < s), "%s: level %d order", name, l);
      }
    }
  }
  CHECK(p.level_start[0] == 0 && p.level_start[max_depth + 1] == n, "%s: level_start ends", name);

  // Conv history from the token path: the root's W-1 context codes, then the
  // path's rows.
  for (int32_t s = 0; s < n; ++s) {
    const std::vector<int32_t> c = chain(s);
    std::vector<int32_t> rows;
    for (int32_t j = 0; j < H; ++j) rows.push_back(-1 - (root_rank[c[0]] * H + j));
    for (const int32_t u : c) {
      if (u == s) {
        for (int32_t j = 0; j < H; ++j)
          CHECK(p.hist[static_cast<size_t>(s) * H + j] == rows[rows.size() - H + j], "%s W=%d: hist[%d][%d] = %d, want %d",
                name, W, s, j, p.hist[static_cast<size_t>(s) * H + j], rows[rows.size() - H + j]);
      }
      for (int32_t j = 0; j < t.lens[u]; ++j) rows.push_back(off[u] + j);
    }
    for (int32_t j = 0; j < H; ++j)
      CHECK(p.ctx_src[static_cast<size_t>(s) * H + j] == rows[rows.size() - H + j], "%s W=%d: ctx_src[%d][%d]", name, W, s, j);
  }

  // Rescan walks: one per leaf, longest first (ties by leaf index), each the
  // leaf's root path; segment s owned by the walk of its lowest leaf.
  CHECK(p.paths_ok == (entries <= tg::Plan::kMaxPathEntries), "%s: paths_ok", name);
  if (p.paths_ok) {
    std::vector<int32_t> low(n, n);  // lowest-indexed leaf below (or at) s
    for (int32_t l = 0; l < n; ++l)
      if (kids[l].empty())
        for (const int32_t u : chain(l)) low[u] = std::min(low[u], l);
    CHECK(static_cast<int32_t>(p.path_off.size()) == leaves + 1 && p.path_off[0] == 0, "%s: path_off size", name);
    std::vector<int32_t> owned(n, 0), walked(n, 0);
    int64_t prev_len = -1;
    int32_t prev_leaf = -1;
    for (int32_t w = 0; w < leaves; ++w) {
      const int32_t b = p.path_off[w], e = p.path_off[w + 1];
      CHECK(e > b, "%s: empty walk %d", name, w);
      const int32_t last = p.path_seg[e - 1] >= 0 ? p.path_seg[e - 1] : ~p.path_seg[e - 1];
      CHECK(last >= 0 && last < n && kids[last].empty() && !walked[last]++, "%s: walk %d leaf", name, w);
      const std::vector<int32_t> c = chain(last);
      CHECK(static_cast<int32_t>(c.size()) == e - b, "%s: walk %d length", name, w);
      for (int32_t k = 0; k < e - b; ++k) {
        const int32_t v = p.path_seg[b + k];
        const int32_t s = v >= 0 ? v : ~v;
        CHECK(s == c[k], "%s: walk %d entry %d", name, w, k);
        CHECK((v >= 0) == (low[s] == last), "%s: walk %d owner flag of %d", name, w, s);
        if (v >= 0) owned[s] += 1;
      }
      const int64_t L = path_len(last);
      CHECK(prev_len < 0 || L < prev_len || (L == prev_len && last > prev_leaf), "%s: walk order", name);
      prev_len = L;
      prev_leaf = last;
    }
    for (int32_t s = 0; s < n; ++s) CHECK(owned[s] == 1, "%s: segment %d owned %d times", name, s, owned[s]);
  }

  // Children lists and chunk tables.
  for (int32_t s = 0; s < n; ++s) {
    const std::vector<int32_t> got(p.kid.begin() + p.kid_off[s], p.kid.begin() + p.kid_off[s + 1]);
    CHECK(got == kids[s], "%s: kid list of %d", name, s);
  }
  int64_t chunks = 0, ckpts = 0;
  for (int32_t s = 0; s < n; ++s) {
    CHECK(p.gchunk[s] == chunks, "%s: gchunk[%d]", name, s);
    CHECK(p.gck[s] == ckpts, "%s: gck[%d]", name, s);
    const int32_t nc = (t.lens[s] + tg::Plan::kBwdChunk - 1) / tg::Plan::kBwdChunk;
    for (int32_t j = 0; j < nc; ++j) CHECK(p.chunk_seg[chunks + j] == s, "%s: chunk_seg", name);
    chunks += nc;
    for (int32_t j = 0; j < nc; j += tg::Plan::kBwdCkpt) ++ckpts;  // chunks 0, 8, 16, ... of the segment
  }
  CHECK(p.total_chunks == chunks && static_cast<int64_t>(p.chunk_seg.size()) == chunks, "%s: total_chunks", name);
  CHECK(p.total_ckpts == ckpts && static_cast<int64_t>(p.gck.size()) == n, "%s: total_ckpts", name);
  std::vector<int32_t> roots;
  for (int32_t s = 0; s < n; ++s)
    if (t.parents[s] < 0) roots.push_back(s);
  CHECK(p.roots == roots, "%s: roots", name);

  // Conv backward heads.  Walk every root-to-leaf token path; the token at
  // path position q + m (q = a segment's first or one past its last token)
  // is a head row c (W-1) + j when j < W-1.
  if (H > 0) {
    std::vector<std::set<int32_t>> ent(static_cast<size_t>(n) * H), fut(static_cast<size_t>(n) * H);
    for (int32_t l = 0; l < n; ++l) {
      if (!kids[l].empty()) continue;
      std::vector<Tok> toks;
      for (const int32_t u : chain(l))
        for (int32_t j = 0; j < t.lens[u]; ++j) toks.emplace_back(u, j);
      for (size_t q = 0; q < toks.size(); ++q) {
        const int32_t s = toks[q].first, j = toks[q].second;
        for (int32_t m = 0; m < H; ++m) {
          const size_t a = j == 0 ? q + m : size_t(-1);
          const size_t f = j == t.lens[s] - 1 ? q + 1 + m : size_t(-1);
          if (a < toks.size() && toks[a].second < H)
            ent[static_cast<size_t>(s) * H + m].insert(toks[a].first * H + toks[a].second);
          if (f < toks.size() && toks[f].second < H)
            fut[static_cast<size_t>(s) * H + m].insert(toks[f].first * H + toks[f].second);
        }
      }
    }
    CHECK(static_cast<int64_t>(p.ent_off.size()) == int64_t(n) * H + 1, "%s: ent_off size", name);
    CHECK(static_cast<int64_t>(p.fut_off.size()) == int64_t(n) * H + 1, "%s: fut_off size", name);
    for (size_t r = 0; r < static_cast<size_t>(n) * H; ++r) {
      std::vector<int32_t> g(p.ent.begin() + p.ent_off[r], p.ent.begin() + p.ent_off[r + 1]);
      std::sort(g.begin(), g.end());
      CHECK(std::adjacent_find(g.begin(), g.end()) == g.end() && std::set<int32_t>(g.begin(), g.end()) == ent[r],
            "%s W=%d: ent row %zu", name, W, r);
      std::vector<int32_t> h(p.fut.begin() + p.fut_off[r], p.fut.begin() + p.fut_off[r + 1]);
      std::sort(h.begin(), h.end());
      CHECK(std::adjacent_find(h.begin(), h.end()) == h.end() && std::set<int32_t>(h.begin(), h.end()) == fut[r],
            "%s W=%d: fut row %zu", name, W, r);
    }
  }

  // The device mirror holds every table at its offset.
  auto same = [&](const std::vector<int32_t>& v, size_t at) {
    return at + v.size() <= p.mirror.size() && std::equal(v.begin(), v.end(), p.mirror.begin() + at);
  };
  CHECK(same(p.seg_off, p.m_seg_off) && same(p.parents, p.m_parent) && same(p.slot, p.m_slot) &&
            same(p.hist, p.m_hist) && same(p.order, p.m_order) && same(p.root_idx, p.m_root) &&
            same(p.ctx_src, p.m_ctx) && same(p.path_off, p.m_path_off) && same(p.path_seg, p.m_path_seg) &&
            same(p.ent_off, p.m_ent_off) && same(p.ent, p.m_ent) && same(p.fut_off, p.m_fut_off) &&
            same(p.fut, p.m_fut) && same(p.roots, p.m_roots) && same(p.kid_off, p.m_kid_off) &&
            same(p.kid, p.m_kid) && same(p.gchunk, p.m_gchunk) && same(p.chunk_seg, p.m_chunk_seg) &&
            same(p.gck, p.m_gck) && p.m_gck + p.gck.size() == p.mirror.size(),
        "%s: device mirror", name);
}

// A random forest: parent drawn from the last `reach` segments (deep when
// small, bushy when large), a root with probability 1/root_every.
Trie random_trie(Rng& g, int32_t n, int32_t max_len, int32_t reach, int32_t root_every) {
  Trie t;
  for (int32_t i = 0; i < n; ++i) {
    int32_t par = -1;
    if (i > 0 && g.below(root_every) != 0) par = i - 1 - g.below(std::min(i, reach));
    t.parents.push_back(par);
    t.lens.push_back(1 + g.below(max_len));
  }
  return t;
}

void expect_error(const int32_t* par, const int32_t* lens, int32_t n, int32_t W, int code, const char* name) {
  tg::Plan p;
  std::string err;
  const int rc = tg::build_plan(par, lens, n, W, &p, &err);
  CHECK(rc == code && !err.empty(), "%s: rc %d, want %d", name, rc, code);
}

void bad_inputs() {
  const int32_t ok_par[3] = {-1, 0, 0}, ok_len[3] = {4, 2, 3};
  expect_error(nullptr, ok_len, 3, 4, TREE_ERR_INVALID_ARG, "null parents");
  expect_error(ok_par, nullptr, 3, 4, TREE_ERR_INVALID_ARG, "null lens");
  expect_error(ok_par, ok_len, 0, 4, TREE_ERR_BAD_TREE, "no segments");
  expect_error(ok_par, ok_len, -5, 4, TREE_ERR_BAD_TREE, "negative n_seg");
  expect_error(ok_par, ok_len, 3, 0, TREE_ERR_INVALID_ARG, "width 0");
  expect_error(ok_par, ok_len, 3, 9, TREE_ERR_INVALID_ARG, "width 9");
  const int32_t self_par[3] = {-1, 1, 0}, fwd_par[3] = {-1, 2, 0}, low_par[3] = {-1, -2, 0};
  expect_error(self_par, ok_len, 3, 4, TREE_ERR_BAD_TREE, "self parent");
  expect_error(fwd_par, ok_len, 3, 4, TREE_ERR_BAD_TREE, "forward parent");
  expect_error(low_par, ok_len, 3, 4, TREE_ERR_BAD_TREE, "parent below -1");
  const int32_t zero_len[3] = {4, 0, 3}, neg_len[3] = {4, 2, -1};
  expect_error(ok_par, zero_len, 3, 4, TREE_ERR_BAD_TREE, "zero length");
  expect_error(ok_par, neg_len, 3, 4, TREE_ERR_BAD_TREE, "negative length");
  // Token count at 2^31: rejected at the segment that reaches it.
  const int32_t big_par[2] = {-1, 0}, big_len[2] = {0x40000000, 0x40000000};
  expect_error(big_par, big_len, 2, 4, TREE_ERR_BAD_TREE, "2^31 tokens");
  // n_seg (W-1) >= 2^31 is rejected before the arrays are read (they hold
  // three entries here; the sanitizer flags any read past them).
  expect_error(ok_par, ok_len, 400000000, 8, TREE_ERR_BAD_TREE, "history rows past int32");
}

}  // namespace

int main() {
  Rng g{20251202};
  int32_t cases = 0;
  // Degenerate shapes at every width.
  for (int32_t W = 1; W <= 8; ++W) {
    check_plan({{-1}, {1}}, W, "one token");
    check_plan({{-1}, {37}}, W, "one segment");
    Trie chain, star, roots, comb;
    for (int32_t i = 0; i < 12; ++i) {
      chain.parents.push_back(i - 1);
      chain.lens.push_back(1);
      star.parents.push_back(i == 0 ? -1 : 0);
      star.lens.push_back(i == 0 ? 2 : 1 + i % 3);
      roots.parents.push_back(-1);
      roots.lens.push_back(1 + i % 5);
      comb.parents.push_back(i == 0 ? -1 : (i % 2 ? i - 1 : i - 2));
      comb.lens.push_back(1 + (i * 7) % 4);
    }
    check_plan(chain, W, "chain of one-token segments");
    check_plan(star, W, "star");
    check_plan(roots, W, "forest of roots");
    check_plan(comb, W, "comb");
    cases += 6;
  }
  // Random forests.
  for (int32_t it = 0; it < 400; ++it) {
    const int32_t n = 1 + g.below(it < 300 ? 40 : 400);
    const int32_t max_len = 1 + g.below(it % 3 == 0 ? 3 : 60);
    const int32_t reach = 1 + g.below(it % 2 ? 3 : 50);
    const int32_t root_every = 2 + g.below(40);
    check_plan(random_trie(g, n, max_len, reach, root_every), 1 + g.below(8), "random");
    ++cases;
  }
  // A deep spine with many leaves: the rescan walk table exceeds its cap.
  {
    Trie t;
    const int32_t spine = 9000, fan = 7500;
    for (int32_t i = 0; i < spine; ++i) {
      t.parents.push_back(i - 1);
      t.lens.push_back(1);
    }
    for (int32_t i = 0; i < fan; ++i) {
      t.parents.push_back(spine - 1);
      t.lens.push_back(2);
    }
    tg::Plan p;
    std::string err;
    if (tg::build_plan(t.parents.data(), t.lens.data(), spine + fan, 4, &p, &err) != TREE_OK || p.paths_ok ||
        !p.path_seg.empty() || tg::choose_schedule(p, 0) != TREE_SCHED_LEVEL) {
      std::fprintf(stderr, "FAIL: capped rescan table\n");
      ++g_fail;
    }
    ++cases;
  }
  bad_inputs();
  if (g_fail) {
    std::fprintf(stderr, "%d failures\n", g_fail);
    return 1;
  }
  std::printf("plan_fuzz: %d plans checked, all tables match\n", cases);
  return 0;
}
