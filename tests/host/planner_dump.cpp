// Test driver: dumps the host planner's output for one shape as JSON on
// stdout, for tests/test_host_planner.py to check against the oracle.
// Built with plain g++ (and sanitizers) from the host-only planner sources.
//
// usage: planner_dump nranks nnodes nchannels chunk_bytes esz count
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../double_binary_tree_amd/csrc/plan.h"
#include "../../double_binary_tree_amd/csrc/topology.h"

using namespace emu;

int main(int argc, char** argv) {
  if (argc != 7) {
    std::fprintf(stderr, "usage: %s nranks nnodes nchannels chunk_bytes esz count\n", argv[0]);
    return 2;
  }
  const int n = std::atoi(argv[1]), m = std::atoi(argv[2]), nch = std::atoi(argv[3]);
  const uint64_t chunk_bytes = std::strtoull(argv[4], nullptr, 10);
  const int esz = std::atoi(argv[5]);
  const uint64_t count = std::strtoull(argv[6], nullptr, 10);
  const uint64_t unit = 16 / esz, chunk = chunk_bytes / esz;
  Topology topo;
  if (int e = build_topology(n, m, nch, &topo)) {
    std::printf("{\"error\": %d}\n", e);
    return 0;
  }
  std::printf("{");
  // fused tiles, both algorithms, tile of 256 vectors
  for (int algo = 0; algo < 2; ++algo) {
    std::vector<Tile> tiles;
    build_fused_tiles(topo, algo == 0 ? Algo::Ring : Algo::Tree, count, unit, chunk, 256 * unit, &tiles);
    std::printf("\"tiles_%s\": [", algo == 0 ? "ring" : "tree");
    for (size_t i = 0; i < tiles.size(); ++i)
      std::printf("%s[%llu,%u,%u]", i ? "," : "", (unsigned long long)tiles[i].start, tiles[i].nelem,
                  tiles[i].variant);
    std::printf("],");
  }
  // stepwise ring loop table and tasks, slice of 64 lanes x 1 vector
  {
    std::vector<RingLoopBlock> loops;
    std::vector<RingTask> tasks;
    const uint64_t slice = 64 * unit;
    build_ring_tasks(topo, count, unit, chunk, slice, &loops, &tasks);
    std::printf("\"ring_slice\": %llu, \"ring_blocks\": [", (unsigned long long)slice);
    for (size_t i = 0; i < loops.size(); ++i)
      std::printf("%s[%llu,%u,%u]", i ? "," : "", (unsigned long long)loops[i].offset, loops[i].nelem,
                  loops[i].first_cell);
    std::printf("], \"ring_tasks\": [");
    for (size_t i = 0; i < tasks.size(); ++i) std::printf("%s[%u,%u]", i ? "," : "", tasks[i].loop, tasks[i].slice);
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
  // fused tree programs of tree 0 and tree 1
  std::printf("\"programs\": [");
  for (int t = 0; t < 2; ++t) {
    const ChannelTopology* ch = &topo.channels[0];
    for (const auto& c : topo.channels)
      if (c.tree_index == t) { ch = &c; break; }
    uint8_t perm[kMaxRanks], instr[kMaxRanks];
    int nregs = 0;
    bool pure = false;
    const int e = compile_tree_program(*ch, perm, instr, &nregs, &pure);
    std::printf("%s{\"tree\": %d, \"error\": %d, \"nregs\": %d, \"pure\": %d, \"perm\": [", t ? "," : "", ch->tree_index,
                e, nregs, pure ? 1 : 0);
    for (int i = 0; i < n; ++i) std::printf("%s%u", i ? "," : "", perm[i]);
    std::printf("], \"instr\": [");
    for (int i = 0; i < n; ++i) std::printf("%s%u", i ? "," : "", instr[i]);
    std::printf("]}");
  }
  std::printf("]}\n");
  return 0;
}
