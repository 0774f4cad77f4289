// Host topology builder: node-level double binary tree, intra-node chain in
// each channel's order, head pattern, per-channel tree records.
#pragma once

#include <array>
#include <vector>

#include "common.h"

namespace emu {

struct NodeTreeEdges {
  int parent;      // -1 at the root
  int child0;      // -1 if absent
  int child1;      // -1 if absent
  int child_type;  // 0: below its parent, 1: above; -1 at the root
};

// Binary tree over node indices 0..n-1, one entry per node (page "NCCL 专家
// 课程 13", section "Btree 的 bit 构造").
std::vector<NodeTreeEdges> node_btree(int n);
// Tree 0 and tree 1 of the double binary tree, one entry per node each
// (section "双树：偶数 mirror，奇数 shift").
std::array<std::vector<NodeTreeEdges>, 2> node_dtree(int n);

struct RankRecord {
  int up = -1;
  int down[3] = {-1, -1, -1};
};

struct ChannelTopology {
  int tree_index = 0;               // which node-level tree
  std::vector<int> order;           // ring / chain order: node 0's ranks, then node 1's, ...
  std::vector<RankRecord> ranks;    // per rank
  std::vector<int> depth;           // distance from the root, per rank
  int root = 0;
  int height = 0;                   // max depth
  int ring_id = 0;                  // index of this channel's order among the distinct ones
  int tree_id = 0;                  // index of this channel's records among the distinct trees
};

struct Topology {
  int nranks = 0, nnodes = 0, nchannels = 0;
  int pattern = EMU_PATTERN_TREE;
  int depth_approx = 0;             // nranks/nnodes - 1 + floor(log2 nnodes)
  int nrings = 0;                   // distinct ring orders over the channels
  int ntrees = 0;                   // distinct tree record sets over the channels
  std::vector<ChannelTopology> channels;
};

// Builds and validates.  `intra` is NULL (identity) or nchannels rows of
// nranks ranks, each node's part a permutation of that node's ranks.
// Returns EMU_SUCCESS, EMU_ERR_INVALID_ARGUMENT or EMU_ERR_INTERNAL (record
// overflow or a failed structural check).
int build_topology(int nranks, int nnodes, int nchannels, int pattern, const int* intra, Topology* out);
inline int build_topology(int nranks, int nnodes, int nchannels, Topology* out) {
  return build_topology(nranks, nnodes, nchannels, EMU_PATTERN_TREE, nullptr, out);
}

// Structural checks: parent/child symmetry, one root, N-1 edges, no cycle,
// every rank reaches the root, at most 2 children at the root and 3 elsewhere.
bool check_channel(const ChannelTopology& ch);

}  // namespace emu
