// Host topology builder.  Sources: page "NCCL 专家课程 13：Tree、双树、层次化
// 连接与真实交叉区间", sections "Btree 的 bit 构造", "双树：偶数 mirror，奇数
// shift", "节点内先形成链" (chain order and head pattern), "节点间连接",
// "从 GRAPH 日志复原 active tree"; page "NCCL代码分析", section "Tree搜索"
// (the three intra-node tree patterns).
#include "topology.h"

#include <cstdio>
#include <cstdlib>

namespace emu {

NodeTreeEdges node_btree(int n, int r) {
  // Lowest set bit of r among the powers of two below n; for r = 0 the scan
  // runs through and ends at the smallest power of two >= n.
  int bit = 1;
  while (bit < n && !(bit & r)) bit <<= 1;
  if (r == 0) return {-1, -1, n > 1 ? (bit >> 1) : -1, -1};
  int parent = (r ^ bit) | (bit << 1);   // clear the low bit, set the next one
  if (parent >= n) parent = r ^ bit;       // that node does not exist: only clear
  NodeTreeEdges e;
  e.parent = parent;
  e.child_type = r < parent ? 0 : 1;
  const int half = bit >> 1;
  e.child0 = half > 0 ? r - half : -1;
  e.child1 = -1;
  for (int off = half; off > 0; off >>= 1) {   // upper child: shrink until it exists
    if (r + off < n) { e.child1 = r + off; break; }
  }
  return e;
}

std::array<NodeTreeEdges, 2> node_dtree(int n, int r) {
  std::array<NodeTreeEdges, 2> t;
  t[0] = node_btree(n, r);
  NodeTreeEdges s;
  if (n % 2 == 1) {
    // odd: build at r-1 (mod n), move every id up by one
    s = node_btree(n, (r - 1 + n) % n);
    auto back = [n](int x) { return x < 0 ? -1 : (x + 1) % n; };
    s.parent = back(s.parent); s.child0 = back(s.child0); s.child1 = back(s.child1);
  } else {
    // even: build at the mirrored index n-1-r, mirror the ids back
    s = node_btree(n, n - 1 - r);
    auto back = [n](int x) { return x < 0 ? -1 : n - 1 - x; };
    s.parent = back(s.parent); s.child0 = back(s.child0); s.child1 = back(s.child1);
  }
  t[1] = s;
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
  std::vector<std::array<NodeTreeEdges, 2>> node_trees(nnodes);
  for (int m = 0; m < nnodes; ++m) node_trees[m] = node_dtree(nnodes, m);
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
      const NodeTreeEdges& e = node_trees[node][ch.tree_index];
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
