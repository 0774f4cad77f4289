// Host topology builder.  Sources: page "NCCL 专家课程 13：Tree、双树、层次化
// 连接与真实交叉区间", sections "Btree 的 bit 构造", "双树：偶数 mirror，奇数
// shift", "节点内先形成链" (chain order and head pattern), "节点间连接",
// "从 GRAPH 日志复原 active tree"; page "NCCL代码分析", section "Tree搜索"
// (the three intra-node tree patterns).
#include "topology.h"

#include <cstdio>
#include <cstdlib>

namespace emu {

namespace {

// Hangs node m, reached with span s, below `parent`, then its subtree: the
// lower child sits s/2 below m, the upper child t above m for the largest
// power of two t <= s/2 that still names a node; the children's spans are
// s/2 and t.
void hang(std::vector<NodeTreeEdges>& t, int n, int parent, int m, int span, int type) {
  t[m] = {parent, -1, -1, type};
  const int half = span / 2;
  if (half == 0) return;
  t[m].child0 = m - half;   // m is a multiple of span, so m - half >= 0
  hang(t, n, m, m - half, half, 0);
  int up = half;
  while (up > 0 && m + up >= n) up /= 2;
  if (up > 0) {
    t[m].child1 = m + up;
    hang(t, n, m, m + up, up, 1);
  }
}

}  // namespace

// The node-level binary tree, top down.  The bit construction of the pages
// puts node r (lowest set bit b) at height log2(b): its parent is the nearer
// node of the next height, its children sit at r -/+ b/2.  Read from the
// root down that is a nest of power-of-two halves: node 0 is the root and
// has one child, the largest power of two p below n, which spans (0, 2p);
// every node splits what it spans into a lower and an upper half and
// hangs the middle node of each.  Where the upper half runs past n its
// middle node moves down to the largest power-of-two offset that exists.
std::vector<NodeTreeEdges> node_btree(int n) {
  std::vector<NodeTreeEdges> t(n > 0 ? n : 0, NodeTreeEdges{-1, -1, -1, -1});
  if (n <= 1) return t;
  int p = 1;
  while (2 * p < n) p *= 2;
  t[0].child1 = p;
  hang(t, n, 0, p, p, 1);
  return t;
}

// The double binary tree: tree 1 is tree 0 with every node index relabelled
// (mirror x -> n-1-x for even n, shift x -> x+1 mod n for odd n), child
// slots and child types carried over unchanged.
std::array<std::vector<NodeTreeEdges>, 2> node_dtree(int n) {
  std::array<std::vector<NodeTreeEdges>, 2> t;
  t[0] = node_btree(n);
  auto relabel = [n](int x) { return x < 0 ? -1 : (n % 2 == 1 ? (x + 1) % n : n - 1 - x); };
  t[1].assign(t[0].size(), NodeTreeEdges{-1, -1, -1, -1});
  for (int x = 0; x < n; ++x) {
    const NodeTreeEdges& e = t[0][x];
    t[1][relabel(x)] = {relabel(e.parent), relabel(e.child0), relabel(e.child1), e.child_type};
  }
  return t;
}

static int log2_floor(int x) {
  int out = 0;
  while (x >= 2) { x >>= 1; ++out; }
  return out;
}

// Attach a child to the first empty slot; false if all three are taken.
static bool attach_down(RankRecord& rec, int child) {
  if (child < 0) return true;
  for (int s = 0; s < 3; ++s) {
    if (rec.down[s] == -1) { rec.down[s] = child; return true; }
  }
  return false;
}

bool check_channel(const ChannelTopology& ch) {
  const int n = (int)ch.ranks.size();
  int roots = 0, edges = 0, root = -1;
  for (int r = 0; r < n; ++r) {
    const RankRecord& rec = ch.ranks[r];
    if (rec.up == -1) { ++roots; root = r; }
    else {
      if (rec.up < 0 || rec.up >= n) return false;
      const RankRecord& p = ch.ranks[rec.up];
      if (p.down[0] != r && p.down[1] != r && p.down[2] != r) return false;
    }
    int nchild = 0;
    for (int s = 0; s < 3; ++s) {
      const int c = rec.down[s];
      if (c == -1) continue;
      if (c < 0 || c >= n || ch.ranks[c].up != r) return false;
      ++nchild;
    }
    if (nchild > (rec.up == -1 ? 2 : 3)) return false;
    edges += nchild;
  }
  if (roots != 1 || edges != n - 1) return false;
  for (int r = 0; r < n; ++r) {
    int x = r, steps = 0;
    while (ch.ranks[x].up != -1) {
      x = ch.ranks[x].up;
      if (++steps > n) return false;   // cycle
    }
    if (x != root) return false;
  }
  return true;
}

// Chain positions of the parent, child0 and child1 heads of a node.
static bool head_positions(int pattern, int pos[3]) {
  switch (pattern) {
    case EMU_PATTERN_TREE: pos[0] = 0; pos[1] = 0; pos[2] = 0; return true;
    case EMU_PATTERN_SPLIT_TREE: pos[0] = 0; pos[1] = 1; pos[2] = 1; return true;
    case EMU_PATTERN_BALANCED_TREE: pos[0] = 0; pos[1] = 1; pos[2] = 0; return true;
    default: return false;
  }
}

int build_topology(int nranks, int nnodes, int nchannels, int pattern, const int* intra, Topology* out) {
  if (nranks < 1 || nranks > kMaxRanks || nnodes < 1 || nranks % nnodes != 0 ||
      nchannels < 1 || nchannels > kMaxChannels)
    return EMU_ERR_INVALID_ARGUMENT;
  const int L = nranks / nnodes;
  int pos[3];
  if (!head_positions(pattern, pos)) return EMU_ERR_INVALID_ARGUMENT;
  if (pos[1] >= L || pos[2] >= L) return EMU_ERR_INVALID_ARGUMENT;
  if (intra) {
    // every node's part of every row is a permutation of that node's ranks
    for (int c = 0; c < nchannels; ++c)
      for (int node = 0; node < nnodes; ++node) {
        uint64_t seen = 0;
        for (int i = 0; i < L; ++i) {
          const int r = intra[(size_t)c * nranks + node * L + i];
          if (r < node * L || r >= (node + 1) * L || (seen >> (r - node * L) & 1)) return EMU_ERR_INVALID_ARGUMENT;
          seen |= (uint64_t)1 << (r - node * L);
        }
      }
  }
  Topology topo;
  topo.nranks = nranks;
  topo.nnodes = nnodes;
  topo.nchannels = nchannels;
  topo.pattern = pattern;
  topo.depth_approx = L - 1 + log2_floor(nnodes);
  const std::array<std::vector<NodeTreeEdges>, 2> node_trees = node_dtree(nnodes);
  const int first_half = (nchannels + 1) / 2;
  for (int c = 0; c < nchannels; ++c) {
    ChannelTopology ch;
    ch.tree_index = c < first_half ? 0 : 1;
    ch.order.resize(nranks);
    for (int i = 0; i < nranks; ++i) ch.order[i] = intra ? intra[(size_t)c * nranks + i] : i;
    ch.ranks.assign(nranks, RankRecord{});
    // chain inside every node, in the channel's order
    auto at = [&](int node, int i) { return ch.order[node * L + i]; };
    for (int node = 0; node < nnodes; ++node) {
      for (int i = 0; i < L; ++i) {
        const int r = at(node, i);
        ch.ranks[r].up = i > 0 ? at(node, i - 1) : -1;
        ch.ranks[r].down[0] = i < L - 1 ? at(node, i + 1) : -1;
      }
    }
    // node-level edges between heads: a node's parent head goes up to the
    // parent node's child0 or child1 head (by child type); a child head
    // takes the child node's parent head, child0 before child1.
    for (int node = 0; node < nnodes; ++node) {
      const NodeTreeEdges& e = node_trees[ch.tree_index][node];
      if (e.parent != -1) ch.ranks[at(node, pos[0])].up = at(e.parent, pos[1 + e.child_type]);
      if (e.child0 != -1 && !attach_down(ch.ranks[at(node, pos[1])], at(e.child0, pos[0]))) return EMU_ERR_INTERNAL;
      if (e.child1 != -1 && !attach_down(ch.ranks[at(node, pos[2])], at(e.child1, pos[0]))) return EMU_ERR_INTERNAL;
    }
    if (!check_channel(ch)) return EMU_ERR_INTERNAL;
    ch.depth.assign(nranks, 0);
    ch.height = 0;
    for (int r = 0; r < nranks; ++r) {
      int x = r, d = 0;
      while (ch.ranks[x].up != -1) { x = ch.ranks[x].up; ++d; }
      ch.depth[r] = d;
      if (d > ch.height) ch.height = d;
      if (d == 0) ch.root = r;
    }
    // ids of the distinct orders and record sets seen so far
    ch.ring_id = topo.nrings;
    ch.tree_id = topo.ntrees;
    for (const ChannelTopology& o : topo.channels) {
      if (o.order == ch.order) { ch.ring_id = o.ring_id; break; }
    }
    for (const ChannelTopology& o : topo.channels) {
      bool same = true;
      for (int r = 0; r < nranks && same; ++r) {
        const RankRecord &a = o.ranks[r], &b = ch.ranks[r];
        same = a.up == b.up && a.down[0] == b.down[0] && a.down[1] == b.down[1] && a.down[2] == b.down[2];
      }
      if (same) { ch.tree_id = o.tree_id; break; }
    }
    if (ch.ring_id == topo.nrings) ++topo.nrings;
    if (ch.tree_id == topo.ntrees) ++topo.ntrees;
    topo.channels.push_back(std::move(ch));
  }
  if (const char* dbg = std::getenv("EMU_DEBUG")) {
    if (dbg[0] == '1') {
      // One line per (channel, rank) in the shape of the GRAPH log line:
      // child slots -> rank -> parent.
      for (int c = 0; c < nchannels; ++c)
        for (int r = 0; r < nranks; ++r) {
          const RankRecord& rec = topo.channels[c].ranks[r];
          std::fprintf(stderr, "EMU Trees [%d] %d/%d/%d->%d->%d\n", c, rec.down[0], rec.down[1],
                       rec.down[2], r, rec.up);
        }
    }
  }
  *out = std::move(topo);
  return EMU_SUCCESS;
}

}  // namespace emu
