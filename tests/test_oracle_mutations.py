"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in the oracle (monkeypatched for the test
only: a wrong index, a dropped or swapped term, a flipped sign, a wrong
rounding) and runs the pins that should notice it; at least one must fail.
This checks the pins, not the oracle: the unmodified oracle passes them all
in the other test files."""

import numpy as np
import pytest

import oracle.collectives as C
import oracle.costmodel as CM
import oracle.numerics as N
import oracle.partition as P
import oracle.ring as R
import oracle.topology as T
import oracle.tree as TR
import tests.test_oracle_collectives as tc
import tests.test_oracle_costmodel as tcm
import tests.test_oracle_numerics as tn
import tests.test_oracle_partition as tp
import tests.test_oracle_ring_tree as trt
import tests.test_oracle_topology as tt

_btree, _dtree, _build, _heads = T.btree, T.dtree, T.build_topology, T.head_positions
_rs, _ag = R.ring_reduce_scatter_steps, R.ring_all_gather_steps
_channels, _loops = P.channel_ranges, P.ring_loops
_f32_to_bf16, _combine = N.f32_to_bf16, N.combine
_reduce_scatter = C.reduce_scatter
_verdict, _relative, _busbw = CM.verdict, CM.relative, CM.busbw


# --- mutants ---------------------------------------------------------------

def btree_parent_only_clears(n, r):
    p, c0, c1, ct = _btree(n, r)
    if r == 0:
        return p, c0, c1, ct
    parent = r ^ (r & -r)
    return parent, c0, c1, 0 if r < parent else 1


def btree_child_type_inverted(n, r):
    p, c0, c1, ct = _btree(n, r)
    return p, c0, c1, None if ct is None else 1 - ct


def dtree_odd_mirrored(n, r):
    t0 = _btree(n, r)
    p, c0, c1, ct = _btree(n, n - 1 - r)
    back = lambda x: -1 if x == -1 else n - 1 - x    # noqa: E731
    return t0, (back(p), back(c0), back(c1), ct)


def dtree_shift_reversed(n, r):
    if n % 2 == 0:
        return _dtree(n, r)
    t0 = _btree(n, r)
    p, c0, c1, ct = _btree(n, (r + 1) % n)
    back = lambda x: -1 if x == -1 else (x - 1) % n    # noqa: E731
    return t0, (back(p), back(c0), back(c1), ct)


def chain_reversed(nranks, nnodes, nchannels, pattern="tree", intra=None):
    L = nranks // nnodes
    rows = intra if intra is not None else [list(range(nranks))] * nchannels
    rev = [[x for m in range(nnodes) for x in reversed(row[m * L:(m + 1) * L])] for row in rows]
    return _build(nranks, nnodes, nchannels, pattern, rev)


def ring_order_ignored(nranks, nnodes, nchannels, pattern="tree", intra=None):
    topo = _build(nranks, nnodes, nchannels, pattern, intra)
    for ch in topo.channels:
        ch.order = list(range(nranks))
    return topo


def balanced_heads_swapped(pattern):
    return (0, 0, 1) if pattern == "balanced" else _heads(pattern)


def rs_sends_next_block(bufs, combine, copy, trace=None, sent=None, size=None):
    n = len(bufs)
    for s in range(n - 1):
        out = [copy(bufs[r][(r - s + 1) % n]) for r in range(n)]
        for r in range(n):
            dst, b = (r + 1) % n, (r - s + 1) % n
            bufs[dst][b] = combine(bufs[dst][b], out[r])
            if sent is not None:
                sent[r] += size(out[r])
        if trace is not None:
            trace.append((("RS", s + 1), [[copy(b) for b in row] for row in bufs]))


def ag_keeps_own_copy(bufs, copy, trace=None, sent=None, size=None):
    n = len(bufs)
    for s in range(n - 1):
        if trace is not None:
            trace.append((("AG", s + 1), [[copy(b) if b is not None else None for b in row] for row in bufs]))


def tree_children_first(inputs, up, down, combine, copy, sent=None, size=None):
    n = len(inputs)
    memo = {}

    def v(r):
        if r not in memo:
            kids = [c for c in down[r] if c != -1]
            acc = None
            for c in kids:
                acc = v(c) if acc is None else combine(acc, v(c))
            memo[r] = copy(inputs[r]) if acc is None else combine(acc, inputs[r])
        return memo[r]
    root = next(r for r in range(n) if up[r] == -1)
    return [copy(v(root)) for _ in range(n)]


def channels_extra_to_last(count, unit, nchannels):
    units = P.ceil_div(count, unit)
    base, extra = divmod(units, nchannels)
    out, u0 = [], 0
    for c in range(nchannels):
        nu = base + (1 if c >= nchannels - extra else 0)
        s, e = min(u0 * unit, count), min((u0 + nu) * unit, count)
        out.append((s, e - s))
        u0 += nu
    return out


def loops_extra_to_last(grid_offset, channel_count, nranks, chunk_count, unit):
    out = []
    for blocks in _loops(grid_offset, channel_count, nranks, chunk_count, unit):
        lens = [ln for _, ln in blocks][::-1]
        pos, new = blocks[0][0], []
        for ln in lens:
            new.append((pos, ln))
            pos += ln
        out.append(new)
    return out


def bf16_truncates(x):
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    return (u >> 16).astype(np.uint16)


def i32_saturates(dtype, op, acc, x):
    if dtype == "i32" and op == "sum":
        s = np.asarray(acc).astype(np.int64) + np.asarray(x).astype(np.int64)
        return np.clip(s, -(1 << 31), (1 << 31) - 1).astype(np.int32)
    return _combine(dtype, op, acc, x)


def max_ignores_signed_zero(dtype, op, acc, x):
    if op == "max" and dtype not in ("i32", "i64"):
        a, b = N.to_f64(acc, dtype), N.to_f64(x, dtype)
        return np.where(b > a, x, acc)
    return _combine(dtype, op, acc, x)


def rs_block_off_by_one(inputs, nnodes, nchannels, chunk_bytes, dtype, op, intra=None, stats=None):
    # rank r ends with block r+1 (the ring's raw placement) instead of its own
    out = _reduce_scatter(inputs, nnodes, nchannels, chunk_bytes, dtype, op, intra, stats)
    n = len(out)
    return [out[(r + 1) % n] for r in range(n)]


def tie_threshold_ten_percent(t_ring, t_tree, tie=0.05):
    return _verdict(t_ring, t_tree, 0.10)


def relative_flipped(t_tree, t_ring):
    return _relative(t_ring, t_tree)


def busbw_without_factor(nbytes, seconds, n):
    return nbytes / seconds


# --- cases: (name, patches, pins) -------------------------------------------

def _pins(*fns):
    return fns


CASES = [
    ("btree parent only clears the low bit", [(T, "btree", btree_parent_only_clears)],
     _pins(tt.test_probe_table_roots_depths_overlap, tt.test_four_node_trees_match_drawings)),
    ("btree child type inverted", [(T, "btree", btree_child_type_inverted)],
     _pins(tt.test_head_patterns_hand_worked_3x2)),
    ("odd double tree mirrored instead of shifted", [(T, "dtree", dtree_odd_mirrored)],
     _pins(tt.test_probe_table_roots_depths_overlap)),
    ("odd shift in the wrong direction", [(T, "dtree", dtree_shift_reversed)],
     _pins(tt.test_probe_table_roots_depths_overlap, tt.test_head_patterns_hand_worked_3x2)),
    ("intra-node chain reversed", [(T, "build_topology", chain_reversed)],
     _pins(tt.test_chain_roles_and_depth, trt.test_chain_fold_order_pin)),
    ("ring walks rank ids instead of the channel order", [(T, "build_topology", ring_order_ignored)],
     _pins(trt.test_permuted_ring_fold_order_pin)),
    ("balanced pattern heads swapped", [(T, "head_positions", balanced_heads_swapped)],
     _pins(tt.test_head_patterns_hand_worked_3x2)),
    ("reduce-scatter sends the next block", [(R, "ring_reduce_scatter_steps", rs_sends_next_block)],
     _pins(trt.test_ring_four_rank_step_table, trt.test_ring_fold_order_pin)),
    ("all-gather never overwrites", [(R, "ring_all_gather_steps", ag_keeps_own_copy)],
     _pins(trt.test_ring_four_rank_step_table, trt.test_two_rank_example_ring_and_tree)),
    ("tree folds the children before the own input", [(TR, "tree_allreduce_chunk", tree_children_first)],
     _pins(lambda: trt.test_head_pattern_fold_order_pin("tree"))),
    ("channel split gives the extra units to the last channels", [(P, "channel_ranges", channels_extra_to_last)],
     _pins(tp.test_channel_example_twelve_channels, lambda: tp.test_channel_ranges_cover_disjoint_aligned(4))),
    ("ring loop split gives the extra units to the last rank-chunks", [(P, "ring_loops", loops_extra_to_last)],
     _pins(tp.test_ring_loops_unit_one_is_array_split)),
    ("bf16 rounding truncates", [(N, "f32_to_bf16", bf16_truncates)],
     _pins(tn.test_bf16_rounding_against_grid_search)),
    ("integer sums saturate", [(N, "combine", i32_saturates)],
     _pins(tn.test_integer_sums_wrap)),
    ("float max ignores the sign of zero", [(N, "combine", max_ignores_signed_zero)],
     _pins(tn.test_max_bf16_and_signed_zero)),
    ("reduce-scatter hands rank r block r+1", [(C, "reduce_scatter", rs_block_off_by_one)],
     _pins(tc.test_reduce_scatter_float_order_pin,
           lambda: tc.test_reduce_scatter_brute_force_integers(4, 2, 2, 100, 32, "sum"))),
    ("tie threshold 10%", [(CM, "verdict", tie_threshold_ten_percent)],
     _pins(tcm.test_selected_points_relative_verdict_busbw, tcm.test_crossover_table_is_a_merge_of_tie_rule_verdicts)),
    ("relative difference of ring to tree", [(CM, "relative", relative_flipped)],
     _pins(tcm.test_selected_points_relative_verdict_busbw)),
    ("busbw without the 2(n-1)/n factor", [(CM, "busbw", busbw_without_factor)],
     _pins(tcm.test_selected_points_relative_verdict_busbw)),
]


@pytest.mark.parametrize("name,patches,pins", CASES, ids=[c[0] for c in CASES])
def test_planted_mistake_fails_a_pin(monkeypatch, name, patches, pins):
    for mod, attr, fn in patches:
        monkeypatch.setattr(mod, attr, fn)
    failures = 0
    for pin in pins:
        try:
            pin()
        except (AssertionError, T.TopologyError):   # a pin, or the structural tree assertions
            failures += 1
    assert failures > 0, f"no pin noticed: {name}"
