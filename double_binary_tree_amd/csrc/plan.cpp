// Host planner.  Sources: page "NCCL 专家课程 13：Tree、双树、层次化连接与真实
// 交叉区间", section "前置知识" (disjoint channel ranges named by grid offset,
// channel count and chunk count) and section "runTreeSplit 如何流水" (the
// chunk loop of the tree); page "all-reduce 每张卡要发多少数据? ring 和 tree 有
// 什么区别?", section "手撕代码" (the ring's n nearly equal parts, the first
// ones larger).  The exact split rule is not printed on the pages; the rule
// here cuts the message into 16-byte units and deals them out the way
// numpy's array_split deals items.
#include "plan.h"

#include <algorithm>
#include <functional>
#include <string>

namespace emu {

static uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

std::vector<Range> channel_ranges(uint64_t count, uint64_t unit, int nch) {
  const uint64_t units = ceil_div(count, unit);
  const uint64_t base = units / nch, extra = units % nch;
  std::vector<Range> out;
  uint64_t u0 = 0;
  for (int c = 0; c < nch; ++c) {
    const uint64_t nu = base + ((uint64_t)c < extra ? 1 : 0);
    const uint64_t s = std::min(u0 * unit, count), e = std::min((u0 + nu) * unit, count);
    out.push_back({s, e - s});
    u0 += nu;
  }
  return out;
}

std::vector<Range> tree_chunks(const Range& ch, uint64_t chunk_count) {
  std::vector<Range> out;
  for (uint64_t e = 0; e < ch.count; e += chunk_count)
    out.push_back({ch.offset + e, std::min(chunk_count, ch.count - e)});
  return out;
}

std::vector<std::vector<Range>> ring_loops(const Range& ch, int nranks, uint64_t chunk_count,
                                           uint64_t unit) {
  std::vector<std::vector<Range>> loops;
  const uint64_t loop_size = (uint64_t)nranks * chunk_count;
  for (uint64_t start = 0; start < ch.count; start += loop_size) {
    const uint64_t len = std::min(loop_size, ch.count - start);
    const uint64_t units = ceil_div(len, unit);
    const uint64_t base = units / nranks, extra = units % nranks;
    std::vector<Range> blocks;
    uint64_t u0 = 0;
    for (int k = 0; k < nranks; ++k) {
      const uint64_t nu = base + ((uint64_t)k < extra ? 1 : 0);
      const uint64_t s = std::min(u0 * unit, len), e = std::min((u0 + nu) * unit, len);
      blocks.push_back({ch.offset + start + s, e - s});
      u0 += nu;
    }
    loops.push_back(std::move(blocks));
  }
  return loops;
}

namespace {

// Segments (start, length, variant) in element order, adjacent segments of
// equal variant merged.
struct Segments {
  struct Seg { uint64_t start, len; uint32_t variant; };
  std::vector<Seg> segs;
  void push(uint64_t s, uint64_t n, uint32_t v) {
    if (n == 0) return;
    if (!segs.empty() && segs.back().variant == v && segs.back().start + segs.back().len == s)
      segs.back().len += n;
    else
      segs.push_back({s, n, v});
  }
  // Cut at global multiples of the tile size, so that full tiles start on a
  // tile-size (>= 4 KiB) boundary of every rank buffer and each wave's
  // accesses cover whole cache lines; only the pieces next to a segment
  // boundary are short.
  void cut(uint64_t tile_elems, std::vector<Tile>* out) const {
    out->clear();
    for (const Seg& s : segs) {
      uint64_t pos = s.start;
      const uint64_t end = s.start + s.len;
      while (pos < end) {
        const uint64_t next = std::min(end, (pos / tile_elems + 1) * tile_elems);
        out->push_back({pos, (uint32_t)(next - pos), s.variant});
        pos = next;
      }
    }
  }
};

int position_of(const ChannelTopology& ch, int rank) {
  for (size_t p = 0; p < ch.order.size(); ++p)
    if (ch.order[p] == rank) return (int)p;
  return 0;
}

}  // namespace

void build_fused_tiles(const Topology& topo, Algo algo, const FusedOrders& orders, uint64_t count,
                       uint64_t unit, uint64_t chunk_count, uint64_t tile_elems, std::vector<Tile>* out) {
  Segments sg;
  auto push = [&](uint64_t s, uint64_t n, uint32_t v) { sg.push(s, n, v); };
  const std::vector<Range> chans = channel_ranges(count, unit, topo.nchannels);
  for (int c = 0; c < topo.nchannels; ++c) {
    if (algo == Algo::Ring) {
      for (const auto& blocks : ring_loops(chans[c], topo.nranks, chunk_count, unit))
        for (int k = 0; k < topo.nranks; ++k) push(blocks[k].offset, blocks[k].count, orders.base[c] + (uint32_t)k);
    } else {
      push(chans[c].offset, chans[c].count, orders.base[c]);
    }
  }
  sg.cut(tile_elems, out);
}

void build_fused_coll_tiles(const Topology& topo, Coll coll, const FusedOrders& ring_orders, uint64_t block,
                            uint64_t unit, uint64_t tile_elems, std::vector<Tile>* out) {
  const int n = topo.nranks;
  Segments sg;
  if (coll == kAllGather) {
    for (int k = 0; k < n; ++k) sg.push((uint64_t)k * block, block, (uint32_t)k << 16);
  } else {
    const std::vector<Range> chans = channel_ranges(block, unit, topo.nchannels);
    for (int r = 0; r < n; ++r)
      for (int c = 0; c < topo.nchannels; ++c) {
        const uint32_t k = (uint32_t)((position_of(topo.channels[c], r) + 1) % n);
        sg.push((uint64_t)r * block + chans[c].offset, chans[c].count, (uint32_t)r << 16 | (ring_orders.base[c] + k));
      }
  }
  sg.cut(tile_elems, out);
}

void build_ring_coll_tasks(const Topology& topo, uint64_t block, uint64_t unit, uint64_t chunk_count,
                           uint64_t slice_elems, std::vector<RingLoopBlock>* loops, std::vector<RingTask>* tasks,
                           std::vector<uint32_t>* orders) {
  const int n = topo.nranks;
  loops->clear();
  tasks->clear();
  orders->assign((size_t)topo.nrings * kMaxRanks, 0);
  for (const ChannelTopology& c : topo.channels)
    for (int p = 0; p < n; ++p) (*orders)[(size_t)c.ring_id * kMaxRanks + p] = (uint32_t)c.order[p];
  uint32_t loop_id = 0;
  const std::vector<Range> chans = channel_ranges(block, unit, topo.nchannels);
  for (int c = 0; c < topo.nchannels; ++c) {
    const ChannelTopology& ch = topo.channels[c];
    for (const Range& piece : tree_chunks(chans[c], chunk_count)) {
      uint64_t nslices = 0;
      for (int k = 0; k < n; ++k) {
        const uint64_t d = (uint64_t)ch.order[(k + n - 1) % n];   // data block of step block k
        const uint64_t off = d * block + piece.offset;
        loops->push_back({off, (uint32_t)piece.count, (uint32_t)(off / slice_elems)});
        nslices = std::max(nslices, ceil_div(off + piece.count, slice_elems) - off / slice_elems);
      }
      for (uint64_t q = 0; q < nslices; ++q)
        tasks->push_back({loop_id, (uint32_t)q, (uint32_t)ch.ring_id, (uint32_t)nslices});
      ++loop_id;
    }
  }
}

int build_fused_orders(const Topology& topo, Algo algo, FusedOrders* out) {
  const int n = topo.nranks;
  FusedOrders o;
  o.base.assign(topo.nchannels, 0);
  for (int j = 0; j < kMaxRanks; ++j) o.rotate_perm[j] = (uint8_t)(j < n ? j : 0);
  if (algo == Algo::Ring) {
    // Ring block k of channel c folds the ranks order[k], order[k+1], ...
    if (topo.nrings == 1) {
      o.mode = kRotate;
      for (int j = 0; j < n; ++j) o.rotate_perm[j] = (uint8_t)topo.channels[0].order[j];
    } else {
      o.mode = kFold;
      o.rows.assign((size_t)topo.nrings * kRowLen, 0);
      for (const ChannelTopology& ch : topo.channels) {
        uint32_t* row = &o.rows[(size_t)ch.ring_id * kRowLen];
        for (int j = 0; j < 2 * n; ++j) row[j] = (uint32_t)ch.order[j % n];
      }
      for (int c = 0; c < topo.nchannels; ++c) o.base[c] = (uint32_t)topo.channels[c].ring_id << 8;
    }
    *out = std::move(o);
    return EMU_SUCCESS;
  }
  // Tree: one program per distinct record set.
  std::vector<uint8_t> perm((size_t)topo.ntrees * kMaxRanks), instr((size_t)topo.ntrees * kMaxRanks);
  std::vector<bool> done(topo.ntrees, false);
  bool all_pure = true;
  for (const ChannelTopology& ch : topo.channels) {
    if (done[ch.tree_id]) continue;
    done[ch.tree_id] = true;
    int nregs = 0;
    bool pure = false;
    if (int e = compile_tree_program(ch, &perm[(size_t)ch.tree_id * kMaxRanks],
                                     &instr[(size_t)ch.tree_id * kMaxRanks], &nregs, &pure))
      return e;
    all_pure = all_pure && pure;
  }
  if (topo.ntrees == 1 && all_pure) {
    o.mode = kRotate;   // one chain: a left fold over the permuted pointers, variant 0
    for (int j = 0; j < n; ++j) o.rotate_perm[j] = perm[j];
  } else {
    o.mode = all_pure ? kFold : kProgram;
    o.rows.assign((size_t)topo.ntrees * kRowLen, 0);
    for (int t = 0; t < topo.ntrees; ++t)
      for (int j = 0; j < n; ++j)
        o.rows[(size_t)t * kRowLen + j] =
            (uint32_t)perm[(size_t)t * kMaxRanks + j] | (uint32_t)instr[(size_t)t * kMaxRanks + j] << 8;
    for (int c = 0; c < topo.nchannels; ++c) o.base[c] = (uint32_t)topo.channels[c].tree_id << 8;
  }
  *out = std::move(o);
  return EMU_SUCCESS;
}

// ---------------------------------------------------------------------------
// Fused tree program.
//
// The tree fold of a rank is acc = x_r, then acc = acc op v(child) for its
// children in slot order, every op rounded (this order is the reading of the
// pages' "receive the children, reduce with the local input" step).  That
// defines an expression tree of binary ops.  Because one rounded add or max
// gives the same bits with its operands swapped, each op may evaluate either
// operand first; the program evaluates the operand that needs more
// registers first (Sethi-Ullman), so a chain needs one register and the
// hierarchical trees a handful.
namespace {

struct Expr {
  int leaf = -1;          // rank for a leaf
  int a = -1, b = -1;     // operands of an op node (indices into the pool)
  int need = 1;
};

struct Insn {
  int kind;   // 0 load, 1 fold input, 2 fold register (R[d] = R[d] op R[d+1])
  int d;
  int rank;
};

}  // namespace

int compile_tree_program(const ChannelTopology& ch, uint8_t perm[kMaxRanks],
                         uint8_t instr[kMaxRanks], int* nregs, bool* pure_fold) {
  const int n = (int)ch.ranks.size();
  std::vector<Expr> pool;
  std::function<int(int)> build = [&](int r) -> int {
    Expr leaf;
    leaf.leaf = r;
    pool.push_back(leaf);
    int acc = (int)pool.size() - 1;
    for (int s = 0; s < 3; ++s) {
      const int c = ch.ranks[r].down[s];
      if (c == -1) continue;
      const int sub = build(c);
      Expr op;
      op.a = acc;
      op.b = sub;
      const Expr& ea = pool[acc];
      const Expr& eb = pool[sub];
      if (ea.leaf >= 0 && eb.leaf >= 0) op.need = 1;
      else if (eb.leaf >= 0) op.need = ea.need;
      else if (ea.leaf >= 0) op.need = eb.need;
      else op.need = std::min(std::max(ea.need, eb.need + 1), std::max(eb.need, ea.need + 1));
      pool.push_back(op);
      acc = (int)pool.size() - 1;
    }
    return acc;
  };
  const int root_expr = build(ch.root);

  std::vector<Insn> code;
  std::function<void(int, int)> gen = [&](int e, int d) {
    const Expr& x = pool[e];
    if (x.leaf >= 0) { code.push_back({0, d, x.leaf}); return; }
    const Expr& ea = pool[x.a];
    const Expr& eb = pool[x.b];
    if (eb.leaf >= 0) { gen(x.a, d); code.push_back({1, d, eb.leaf}); return; }
    if (ea.leaf >= 0) { gen(x.b, d); code.push_back({1, d, ea.leaf}); return; }
    const int first = ea.need >= eb.need ? x.a : x.b;
    const int second = first == x.a ? x.b : x.a;
    gen(first, d);
    gen(second, d + 1);
    code.push_back({2, d, -1});
  };
  gen(root_expr, 0);

  // Pack: one record per consumed input, register folds attached to the
  // input that precedes them (they always come as a cascade d-1, d-2, ...).
  int j = -1, maxd = 0;
  int pops = 0;
  for (const Insn& in : code) {
    maxd = std::max(maxd, in.d);
    if (in.kind == 2) {
      if (j < 0) return EMU_ERR_INTERNAL;
      const int d_in = (instr[j] >> 1) & 7;
      if (in.d != d_in - 1 - pops) return EMU_ERR_INTERNAL;
      ++pops;
      if (pops > 15) return EMU_ERR_INTERNAL;
      instr[j] = (uint8_t)((instr[j] & 0x0F) | (pops << 4));
      continue;
    }
    ++j;
    if (j >= n || in.d >= kMaxRegs) return EMU_ERR_INTERNAL;
    pops = 0;
    perm[j] = (uint8_t)in.rank;
    instr[j] = (uint8_t)((in.kind == 1 ? 1 : 0) | (in.d << 1));
  }
  if (j != n - 1) return EMU_ERR_INTERNAL;
  *nregs = maxd + 1;
  if (*nregs > kMaxRegs) return EMU_ERR_INTERNAL;

  bool pure = (instr[0] == 0);
  for (int i = 1; i < n; ++i) pure = pure && instr[i] == 1;
  *pure_fold = pure;

  // Self-check: run the packed program on canonical strings where
  // op(p, q) = "(" min(p,q) "," max(p,q) ")"; it must spell the same
  // expression as the fold definition with every op's operands unordered.
  std::function<std::string(int)> canon = [&](int e) -> std::string {
    const Expr& x = pool[e];
    if (x.leaf >= 0) return std::to_string(x.leaf);
    std::string p = canon(x.a), q = canon(x.b);
    if (q < p) std::swap(p, q);
    return "(" + p + "," + q + ")";
  };
  auto opc = [](const std::string& p, const std::string& q) {
    return p < q ? "(" + p + "," + q + ")" : "(" + q + "," + p + ")";
  };
  std::vector<std::string> R(kMaxRegs);
  for (int i = 0; i < n; ++i) {
    const int d = (instr[i] >> 1) & 7;
    const std::string x = std::to_string(perm[i]);
    R[d] = (instr[i] & 1) ? opc(R[d], x) : x;
    for (int p = 1; p <= (instr[i] >> 4); ++p) R[d - p] = opc(R[d - p], R[d - p + 1]);
  }
  if (R[0] != canon(root_expr)) return EMU_ERR_INTERNAL;
  return EMU_SUCCESS;
}

void build_ring_tasks(const Topology& topo, uint64_t count, uint64_t unit, uint64_t chunk_count,
                      uint64_t slice_elems, std::vector<RingLoopBlock>* loops,
                      std::vector<RingTask>* tasks, std::vector<uint32_t>* orders) {
  loops->clear();
  tasks->clear();
  orders->assign((size_t)topo.nrings * kMaxRanks, 0);
  for (const ChannelTopology& c : topo.channels)
    for (int p = 0; p < topo.nranks; ++p) (*orders)[(size_t)c.ring_id * kMaxRanks + p] = (uint32_t)c.order[p];
  uint32_t loop_id = 0;
  const std::vector<Range> chans = channel_ranges(count, unit, topo.nchannels);
  for (int c = 0; c < topo.nchannels; ++c) {
    const Range& ch = chans[c];
    const uint32_t ring = (uint32_t)topo.channels[c].ring_id;
    for (const auto& blocks : ring_loops(ch, topo.nranks, chunk_count, unit)) {
      // slices of a block = the slice-size cells of the global grid it overlaps
      uint64_t nslices = 0;
      for (const Range& b : blocks) {
        loops->push_back({b.offset, (uint32_t)b.count, (uint32_t)(b.offset / slice_elems)});
        if (b.count)
          nslices = std::max(nslices, ceil_div(b.offset + b.count, slice_elems) - b.offset / slice_elems);
      }
      for (uint64_t q = 0; q < nslices; ++q) tasks->push_back({loop_id, (uint32_t)q, ring, (uint32_t)nslices});
      ++loop_id;
    }
  }
}

std::vector<uint32_t> ring_channel_loops(const Topology& topo, uint64_t count, uint64_t unit, uint64_t chunk_count) {
  std::vector<uint32_t> out;
  uint32_t first = 0;
  const std::vector<Range> chans = channel_ranges(count, unit, topo.nchannels);
  for (int c = 0; c < topo.nchannels; ++c) {
    const uint32_t nloops = (uint32_t)ring_loops(chans[c], topo.nranks, chunk_count, unit).size();
    out.push_back(first);
    out.push_back(first + nloops);
    first += nloops;
  }
  return out;
}

void build_tree_tasks(const Topology& topo, uint64_t count, uint64_t unit, uint64_t slice_elems,
                      uint64_t target_tasks, std::vector<TreeTask>* tasks,
                      std::vector<TreeNode>* nodes, uint64_t min_cells) {
  tasks->clear();
  const std::vector<Range> chans = channel_ranges(count, unit, topo.nchannels);
  // Adjacent channels with the same tree records are contiguous ranges of
  // the message with identical per-element orders; each such segment is one
  // stream of slices.  It is cut, at slice-cell boundaries, into pieces of
  // nearly equal size, one pipeline per workgroup, so that the pipeline's
  // fill and drain are paid once per piece rather than once per chunk
  // (chunking never changes an element's order).
  struct Seg { uint64_t start, end; int channel; };
  std::vector<Seg> segs;
  for (int c = 0; c < topo.nchannels; ++c) {
    if (chans[c].count == 0) continue;
    if (!segs.empty() && topo.channels[segs.back().channel].tree_id == topo.channels[c].tree_id &&
        segs.back().end == chans[c].offset)
      segs.back().end = chans[c].offset + chans[c].count;
    else
      segs.push_back({chans[c].offset, chans[c].offset + chans[c].count, c});
  }
  uint64_t total_cells = 0;
  for (const Seg& g : segs) total_cells += ceil_div(g.end, slice_elems) - g.start / slice_elems;
  if (target_tasks == 0) target_tasks = 1;
  // Cells per task: even split of all cells, and few enough elements that a
  // task's length fits the 32-bit field.
  uint64_t per_task = std::max<uint64_t>(std::max<uint64_t>(1, min_cells), ceil_div(total_cells, target_tasks));
  per_task = std::min<uint64_t>(per_task, ((uint64_t)1 << 31) / slice_elems);
  for (const Seg& g : segs) {
    uint64_t pos = g.start;
    while (pos < g.end) {
      const uint64_t next = std::min(g.end, (pos / slice_elems + per_task) * slice_elems);
      tasks->push_back({pos, (uint32_t)(next - pos), (uint32_t)g.channel});
      pos = next;
    }
  }
  nodes->assign((size_t)topo.nchannels * topo.nranks, TreeNode{});
  for (int c = 0; c < topo.nchannels; ++c)
    for (int r = 0; r < topo.nranks; ++r) {
      const RankRecord& rec = topo.channels[c].ranks[r];
      TreeNode& tn = (*nodes)[(size_t)c * topo.nranks + r];
      tn.up = (int8_t)rec.up;
      for (int s = 0; s < 3; ++s) tn.down[s] = (int8_t)rec.down[s];
      tn.depth = (int8_t)topo.channels[c].depth[r];
    }
}

}  // namespace emu
