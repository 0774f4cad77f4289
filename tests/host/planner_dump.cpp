// Test driver: dumps the host planner's output for one shape as JSON on
// stdout, for tests/test_host_planner.py to check against the oracle.
// Built with plain g++ (and sanitizers) from the host-only planner sources.
//
// usage: planner_dump nranks nnodes nchannels chunk_bytes esz count pattern intra
//   pattern  0 tree, 1 split, 2 balanced
//   intra    "-" for identity orders, else nchannels*nranks comma-separated ranks
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../double_binary_tree_amd/csrc/plan.h"
#include "../../double_binary_tree_amd/csrc/topology.h"

using namespace emu;

static void print_orders(const char* name, const FusedOrders& o, const std::vector<Tile>& tiles) {
  std::printf("\"%s\": {\"mode\": %d, \"rotate_perm\": [", name, o.mode);
  for (int j = 0; j < kMaxRanks; ++j) std::printf("%s%u", j ? "," : "", o.rotate_perm[j]);
  std::printf("], \"rows\": [");
  for (size_t i = 0; i < o.rows.size(); ++i) std::printf("%s%u", i ? "," : "", o.rows[i]);
  std::printf("], \"base\": [");
  for (size_t i = 0; i < o.base.size(); ++i) std::printf("%s%u", i ? "," : "", o.base[i]);
  std::printf("], \"tiles\": [");
  for (size_t i = 0; i < tiles.size(); ++i)
    std::printf("%s[%llu,%u,%u]", i ? "," : "", (unsigned long long)tiles[i].start, tiles[i].nelem,
                tiles[i].variant);
  std::printf("]},");
}

int main(int argc, char** argv) {
  if (argc != 9) {
    std::fprintf(stderr, "usage: %s nranks nnodes nchannels chunk_bytes esz count pattern intra\n", argv[0]);
    return 2;
  }
  const int n = std::atoi(argv[1]), m = std::atoi(argv[2]), nch = std::atoi(argv[3]);
  const uint64_t chunk_bytes = std::strtoull(argv[4], nullptr, 10);
  const int esz = std::atoi(argv[5]);
  const uint64_t count = std::strtoull(argv[6], nullptr, 10);
  const int pattern = std::atoi(argv[7]);
  std::vector<int> intra;
  if (std::strcmp(argv[8], "-") != 0) {
    for (const char* p = argv[8]; *p;) {
      char* end = nullptr;
      intra.push_back((int)std::strtol(p, &end, 10));
      p = (*end == ',') ? end + 1 : end;
    }
    if (intra.size() != (size_t)n * nch) {
      std::fprintf(stderr, "intra needs %d entries\n", n * nch);
      return 2;
    }
  }
  const uint64_t unit = 16 / esz, chunk = chunk_bytes / esz;
  Topology topo;
  if (int e = build_topology(n, m, nch, pattern, intra.empty() ? nullptr : intra.data(), &topo)) {
    std::printf("{\"error\": %d}\n", e);
    return 0;
  }
  std::printf("{\"nrings\": %d, \"ntrees\": %d, \"ring_id\": [", topo.nrings, topo.ntrees);
  for (int c = 0; c < nch; ++c) std::printf("%s%d", c ? "," : "", topo.channels[c].ring_id);
  std::printf("], \"tree_id\": [");
  for (int c = 0; c < nch; ++c) std::printf("%s%d", c ? "," : "", topo.channels[c].tree_id);
  std::printf("],");
  // fused orders and tiles, both algorithms, tile of 256 vectors
  for (int algo = 0; algo < 2; ++algo) {
    const Algo a = algo == 0 ? Algo::Ring : Algo::Tree;
    FusedOrders orders;
    if (int e = build_fused_orders(topo, a, &orders)) {
      std::printf("\"fused_%s\": {\"error\": %d},", algo == 0 ? "ring" : "tree", e);
      continue;
    }
    std::vector<Tile> tiles;
    build_fused_tiles(topo, a, orders, count, unit, chunk, 256 * unit, &tiles);
    print_orders(algo == 0 ? "fused_ring" : "fused_tree", orders, tiles);
  }
  // reduce-scatter / all-gather with a block of count rounded down to whole units
  {
    const uint64_t block = count / unit * unit;
    FusedOrders ring_orders;
    build_fused_orders(topo, Algo::Ring, &ring_orders);
    for (int coll = kReduceScatter; coll <= kAllGather; ++coll) {
      std::vector<Tile> tiles;
      build_fused_coll_tiles(topo, (Coll)coll, ring_orders, block, unit, 256 * unit, &tiles);
      print_orders(coll == kReduceScatter ? "fused_rs" : "fused_ag", ring_orders, tiles);
    }
    std::vector<RingLoopBlock> loops;
    std::vector<RingTask> tasks;
    std::vector<uint32_t> orders;
    const uint64_t slice = 64 * unit;
    build_ring_coll_tasks(topo, block, unit, chunk, slice, &loops, &tasks, &orders);
    std::printf("\"coll_block\": %llu, \"coll_blocks\": [", (unsigned long long)block);
    for (size_t i = 0; i < loops.size(); ++i)
      std::printf("%s[%llu,%u,%u]", i ? "," : "", (unsigned long long)loops[i].offset, loops[i].nelem,
                  loops[i].first_cell);
    std::printf("], \"coll_tasks\": [");
    for (size_t i = 0; i < tasks.size(); ++i)
      std::printf("%s[%u,%u,%u]", i ? "," : "", tasks[i].loop, tasks[i].slice, tasks[i].ring);
    std::printf("], \"coll_orders\": [");
    for (size_t i = 0; i < orders.size(); ++i) std::printf("%s%u", i ? "," : "", orders[i]);
    std::printf("],");
  }
  // stepwise ring loop table and tasks, slice of 64 lanes x 1 vector
  {
    std::vector<RingLoopBlock> loops;
    std::vector<RingTask> tasks;
    std::vector<uint32_t> orders;
    const uint64_t slice = 64 * unit;
    build_ring_tasks(topo, count, unit, chunk, slice, &loops, &tasks, &orders);
    std::printf("\"ring_slice\": %llu, \"ring_blocks\": [", (unsigned long long)slice);
    for (size_t i = 0; i < loops.size(); ++i)
      std::printf("%s[%llu,%u,%u]", i ? "," : "", (unsigned long long)loops[i].offset, loops[i].nelem,
                  loops[i].first_cell);
    std::printf("], \"ring_tasks\": [");
    for (size_t i = 0; i < tasks.size(); ++i)
      std::printf("%s[%u,%u,%u,%u]", i ? "," : "", tasks[i].loop, tasks[i].slice, tasks[i].ring, tasks[i].nslices);
    std::printf("], \"ring_orders\": [");
    for (size_t i = 0; i < orders.size(); ++i) std::printf("%s%u", i ? "," : "", orders[i]);
    std::printf("],");
  }
  // stepwise tree tasks
  {
    std::vector<TreeTask> tasks;
    std::vector<TreeNode> nodes;
    const uint64_t slice = 64 * unit;
    build_tree_tasks(topo, count, unit, slice, 37, &tasks, &nodes);
    std::printf("\"tree_slice\": %llu, \"tree_tasks\": [", (unsigned long long)slice);
    for (size_t i = 0; i < tasks.size(); ++i)
      std::printf("%s[%llu,%u,%u]", i ? "," : "", (unsigned long long)tasks[i].start, tasks[i].nelem,
                  tasks[i].channel);
    std::printf("], \"tree_nodes\": [");
    for (size_t i = 0; i < nodes.size(); ++i)
      std::printf("%s[%d,%d,%d,%d,%d]", i ? "," : "", nodes[i].up, nodes[i].down[0], nodes[i].down[1],
                  nodes[i].down[2], nodes[i].depth);
    std::printf("],");
  }
  // compiled tree program of every channel
  std::printf("\"programs\": [");
  for (int c = 0; c < nch; ++c) {
    uint8_t perm[kMaxRanks], instr[kMaxRanks];
    int nregs = 0;
    bool pure = false;
    const int e = compile_tree_program(topo.channels[c], perm, instr, &nregs, &pure);
    std::printf("%s{\"channel\": %d, \"error\": %d, \"nregs\": %d, \"pure\": %d, \"perm\": [", c ? "," : "", c, e,
                nregs, pure ? 1 : 0);
    for (int i = 0; i < n; ++i) std::printf("%s%u", i ? "," : "", perm[i]);
    std::printf("], \"instr\": [");
    for (int i = 0; i < n; ++i) std::printf("%s%u", i ? "," : "", instr[i]);
    std::printf("]}");
  }
  std::printf("]}\n");
  return 0;
}
