"""Oracle: the cost model and the decision rules of algorithm selection
(test infrastructure only).

Sources (page title, then section):

* "NCCL 专家课程 13：Tree、双树、层次化连接与真实交叉区间", section "理想成本模型":
  with per-stage cost alpha and link bandwidth B, a tree of depth D costs
  about 2*D*alpha + 2*M/B (D stages up, D down, every edge carrying the whole
  range once each way) and a ring about 2(N-1)*alpha + 2(N-1)/N * M/B.
* "all-reduce 每张卡要发多少数据? ring 和 tree 有什么区别?", sections "α–β 模型"
  and "推导 / 关键公式" (time = alpha + bytes/B per message; the ring's
  2(n-1) steps of S/n each; the ring and tree rows of the comparison table).
* "NCCL 专家课程 13", section "性能结果的判定规则" (a loser within 5% of the
  winner is a practical tie, |loser/winner - 1| < 5%) and the tables under
  "真实交叉区间" and "选定性能点" (interval merging over the size ladder, the
  relative difference (Tree/Ring - 1), busbw).
* "all-reduce 每张卡要发多少数据?", section "busbw 和 algbw 是什么?" (algbw =
  S/t, busbw = algbw * 2(n-1)/n).
* "NCCL代码分析", section "通讯时如何选择Channel" (the selection takes, per
  algorithm, a latency times a count of pipelined operations plus bytes over
  a bandwidth, and picks the smallest time).

Readings (listed in the design doc): the fitted per-stage alpha and bandwidth of
each algorithm come from a least-squares straight line t = a + b*S through
measured points, a = (stages)*alpha + L with a fixed launch cost L shared
by both algorithms, and b = (bytes factor)/B; selection picks the smaller
predicted time, ring on an exact tie.

Pins (tests/test_oracle_costmodel.py): the pages' selected points (relative
difference, verdict, busbw), the crossover table (points per interval on the
size ladder, verdicts of the margins, contiguity), closed forms of the two
formulas, and exact recovery of parameters from noiseless model data.
"""

from __future__ import annotations

import numpy as np

TIE = 0.05


def ring_stages(n: int) -> int:
    return 2 * (n - 1)


def tree_stages(depth: int) -> int:
    return 2 * depth


def ring_time(n: int, nbytes: float, alpha: float, bw: float, launch: float = 0.0) -> float:
    """2(N-1)*alpha + 2(N-1)/N * M/B (+ a fixed launch cost)."""
    return launch + ring_stages(n) * alpha + 2.0 * (n - 1) / n * nbytes / bw


def tree_time(depth: int, nbytes: float, alpha: float, bw: float, launch: float = 0.0) -> float:
    """2*D*alpha + 2*M/B (+ a fixed launch cost)."""
    return launch + tree_stages(depth) * alpha + 2.0 * nbytes / bw


def relative(t_tree: float, t_ring: float) -> float:
    """Tree relative to ring: Tree/Ring - 1 (positive: tree slower)."""
    return t_tree / t_ring - 1.0


def verdict(t_ring: float, t_tree: float, tie: float = TIE) -> str:
    """"Ring", "Tree" or "Tie" by the practical-tie rule."""
    winner, loser = (t_ring, t_tree) if t_ring <= t_tree else (t_tree, t_ring)
    if loser / winner - 1.0 < tie:
        return "Tie"
    return "Ring" if t_ring < t_tree else "Tree"


def margin(t_ring: float, t_tree: float) -> float:
    """The loser's excess over the winner, |loser/winner - 1|."""
    lo, hi = min(t_ring, t_tree), max(t_ring, t_tree)
    return hi / lo - 1.0


def intervals(sizes: list[int], verdicts: list[str]) -> list[tuple[str, int, int, int]]:
    """Merge runs of equal verdicts over increasing sizes into
    (verdict, first size, last size, points)."""
    out: list[list] = []
    for s, v in zip(sizes, verdicts):
        if out and out[-1][0] == v:
            out[-1][2] = s
            out[-1][3] += 1
        else:
            out.append([v, s, s, 1])
    return [tuple(x) for x in out]


def busbw(nbytes: float, seconds: float, n: int) -> float:
    """Bus bandwidth in bytes/s: (S/t) * 2(n-1)/n."""
    return nbytes / seconds * 2.0 * (n - 1) / n


def fit_line(sizes, times) -> tuple[float, float]:
    """Least-squares t = a + b*S, weighted by 1/t (relative errors count)."""
    s = np.asarray(sizes, dtype=np.float64)
    t = np.asarray(times, dtype=np.float64)
    w = 1.0 / t
    A = np.stack([np.ones_like(s), s], axis=1) * w[:, None]
    (a, b), *_ = np.linalg.lstsq(A, t * w, rcond=None)
    return float(a), float(b)


def params_from_fit(algo: str, n: int, depth: int, a: float, b: float, launch: float) -> tuple[float, float]:
    """(alpha, bandwidth) of the pages' formula from a fitted line t = a + b*S
    and a known launch cost: a = launch + stages*alpha, b = factor / B."""
    stages = ring_stages(n) if algo == "ring" else tree_stages(depth)
    factor = 2.0 * (n - 1) / n if algo == "ring" else 2.0
    alpha = (a - launch) / stages if stages else 0.0
    return alpha, factor / b


def select(n: int, depth: int, nbytes: float, ring: tuple, tree: tuple) -> str:
    """The algorithm with the smaller predicted time; ring on an exact tie.
    ring = (alpha, bw, launch), tree likewise."""
    tr = ring_time(n, nbytes, *ring)
    tt = tree_time(depth, nbytes, *tree)
    return "tree" if tt < tr else "ring"


def crossover(n: int, depth: int, ring: tuple, tree: tuple) -> float | None:
    """The size where the two predicted times are equal (None if parallel)."""
    ar, br, lr = ring
    at, bt, lt = tree
    a_r = lr + ring_stages(n) * ar
    a_t = lt + tree_stages(depth) * at
    b_r = 2.0 * (n - 1) / n / br
    b_t = 2.0 / bt
    if b_r == b_t:
        return None
    return (a_t - a_r) / (b_r - b_t)
