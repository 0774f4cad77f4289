"""Fit the pages' alpha-beta cost model to measured message-size sweeps.

Input: the JSON lines of ``python -m double_binary_tree_amd.sweep --jsonl``,
one or more sweeps (each line names its workload, ranks N, deepest channel
tree D, channel count and per-leg times), or the same points as a
tab-separated table (``profiles/sweep_points.txt`` holds the sweeps the
library's defaults were fitted to).

Per (workload, channel count, mode, algorithm) a straight line t = a + b*S is
fitted by least squares with relative weights, and read in the pages' form
(page "NCCL 专家课程 13", section "理想成本模型"; page "all-reduce 每张卡要发多
少数据?", section "α–β 模型"): ring t = 2(N-1)*alpha + 2(N-1)/N * S/B, tree
t = 2*D*alpha + 2*S/B.  The fixed cost of a call is folded into alpha, as
in the pages' formula.  Per shape the report gives alpha and B, the model's
crossover size and, under the 5% practical-tie rule of section "性能结果的判定
规则", the measured winner intervals next to the model's choice, and the
share of sizes where the choice is the measured winner or a tie ("agree") —
for the shape's own fit and for the 8-rank fit applied to it.

    python -m double_binary_tree_amd.costfit a.jsonl [b.jsonl ...] [--out report.md] [--defaults]
    python -m double_binary_tree_amd.costfit profiles/sweep_points.txt --defaults

``--defaults`` prints the C initialiser of the library's per-rank-class
defaults: the fits of 8 ranks at 12 channels, 16 ranks at 8 and 32 ranks at
16 (each workload's own channel count).
"""

from __future__ import annotations

import argparse
import json
import sys

import numpy as np

TIE = 0.05
MODES = ("fused", "stepwise")
CLASS_POINTS = ((8, 12), (16, 8), (32, 16))   # (ranks, channels) fitted for each rank-count class


def fit_line(sizes, times):
    s = np.asarray(sizes, dtype=np.float64)
    t = np.asarray(times, dtype=np.float64)
    w = 1.0 / t
    A = np.stack([np.ones_like(s), s], axis=1) * w[:, None]
    (a, b), *_ = np.linalg.lstsq(A, t * w, rcond=None)
    return float(a), float(b)


def stages(algo: str, n: int, depth: int) -> int:
    return 2 * (n - 1) if algo == "ring" else 2 * depth


def factor(algo: str, n: int) -> float:
    return 2.0 * (n - 1) / n if algo == "ring" else 2.0


def to_params(algo: str, n: int, depth: int, a: float, b: float):
    """(alpha us per stage, bandwidth bytes/us) of the pages' formula."""
    return a / stages(algo, n, depth), factor(algo, n) / b


def predict(algo: str, n: int, depth: int, alpha: float, bw: float, nbytes: float) -> float:
    return stages(algo, n, depth) * alpha + factor(algo, n) * nbytes / bw


def verdict(t_ring: float, t_tree: float) -> str:
    lo, hi = min(t_ring, t_tree), max(t_ring, t_tree)
    if hi / lo - 1.0 < TIE:
        return "tie"
    return "ring" if t_ring < t_tree else "tree"


def human(nbytes: float) -> str:
    nbytes = int(nbytes)
    for unit, div in (("GiB", 1 << 30), ("MiB", 1 << 20), ("KiB", 1 << 10)):
        if nbytes >= div:
            return f"{nbytes // div} {unit}"
    return f"{nbytes} B"


def intervals(pairs):
    out = []
    for s, v in pairs:
        if out and out[-1][0] == v:
            out[-1][2] = s
        else:
            out.append([v, s, s])
    return out


def agreement(pts, mode, n, depth, ring, tree):
    """Share of sizes where the model picks the measured winner or a tie,
    and the model's picks."""
    chosen = []
    ok = 0
    for r in pts:
        s = r["bytes"]
        pick = "tree" if predict("tree", n, depth, *tree, s) < predict("ring", n, depth, *ring, s) else "ring"
        chosen.append((s, pick))
        m = verdict(r[f"ring_{mode}"], r[f"tree_{mode}"])
        ok += m in ("tie", pick)
    return ok / len(pts), chosen


def analyse(rows):
    res = {}
    shapes = sorted({(r["workload"], r["nranks"], r["depth"], r["nch"]) for r in rows}, key=lambda x: (x[1], x[3]))
    for wl, n, depth, nch in shapes:
        pts = sorted((r for r in rows if r["workload"] == wl and r["nch"] == nch), key=lambda r: r["bytes"])
        sizes = [r["bytes"] for r in pts]
        for mode in MODES:
            fits = {}
            for algo in ("ring", "tree"):
                times = [r[f"{algo}_{mode}"] for r in pts]
                a, b = fit_line(sizes, times)
                alpha, bw = to_params(algo, n, depth, a, b)
                pred = [a + b * s for s in sizes]
                err = float(np.median(np.abs(np.array(pred) / np.array(times) - 1)))
                fits[algo] = {"a_us": a, "b_us_per_byte": b, "alpha_us": alpha, "bw": bw, "median_rel_err": err}
            ar, br = fits["ring"]["a_us"], fits["ring"]["b_us_per_byte"]
            at, bt = fits["tree"]["a_us"], fits["tree"]["b_us_per_byte"]
            cross = (at - ar) / (br - bt) if br != bt else None
            measured = [(r["bytes"], verdict(r[f"ring_{mode}"], r[f"tree_{mode}"])) for r in pts]
            agree, chosen = agreement(pts, mode, n, depth, (fits["ring"]["alpha_us"], fits["ring"]["bw"]),
                                      (fits["tree"]["alpha_us"], fits["tree"]["bw"]))
            res[(wl, n, depth, nch, mode)] = {"fits": fits, "crossover_bytes": cross, "pts": pts,
                                              "measured": intervals(measured), "chosen": intervals(chosen),
                                              "agreement": agree}
    return res


def fit_of(res, n, nch, mode):
    for (wl, rn, depth, rc, m), r in res.items():
        if rn == n and rc == nch and m == mode:
            return r
    return None


def report(res, srcs) -> str:
    lines = ["# Cost model fitted to the message-size sweeps (one MI355X)\n\n",
             f"Command: `python -m double_binary_tree_amd.costfit {' '.join(srcs)} --out <this file>` on the "
             "points of `python -m double_binary_tree_amd.sweep --workload <w> --jsonl` (graph-replayed "
             "launches, library buffer placement). Per shape, mode and algorithm a least-squares line t = a + b·S "
             "(relative weights), read as ring t = 2(N−1)·α + 2(N−1)/N·S/B and tree t = 2·D·α + 2·S/B with the "
             "shape's N and deepest channel tree D; the fixed cost of a call is folded into α. Measured winners "
             "use the 5% practical-tie rule; \"agree\" is the share of sizes where the model's pick is the "
             "measured winner or a tie, with the shape's own fit and with the 8-rank, 12-channel fit applied "
             "to the shape (the single default the library had before it kept one per rank-count class).\n\n",
             "| workload | N | D | nch | mode | algo | α µs/stage | B GB/s | median \\|fit/measured − 1\\| | "
             "crossover | agree (own fit) | agree (8-rank fit) |\n",
             "|---|---|---|---|---|---|---|---|---|---|---|---|\n"]
    for (wl, n, depth, nch, mode), r in res.items():
        ref = fit_of(res, 8, 12, mode)
        if ref is not None:
            f8 = ref["fits"]
            agree8, _ = agreement(r["pts"], mode, n, depth, (f8["ring"]["alpha_us"], f8["ring"]["bw"]),
                                  (f8["tree"]["alpha_us"], f8["tree"]["bw"]))
            a8 = f"{100 * agree8:.0f}%"
        else:
            a8 = "–"
        cross = r["crossover_bytes"]
        cx = "none" if cross is None or cross <= 0 else human(cross)
        for algo in ("ring", "tree"):
            f = r["fits"][algo]
            lines.append(f"| {wl} | {n} | {depth} | {nch} | {mode} | {algo} | {f['alpha_us']:.3f} | "
                         f"{f['bw'] / 1e3:.1f} | {100 * f['median_rel_err']:.1f}% | {cx} | "
                         f"{100 * r['agreement']:.0f}% | {a8} |\n")
    lines.append("\n## Measured winners (5% tie rule) and the model's choice (own fit)\n\n")
    for (wl, n, depth, nch, mode), r in res.items():
        meas = "; ".join(f"{v} {human(a)}–{human(b)}" for v, a, b in r["measured"])
        cho = "; ".join(f"{v} {human(a)}–{human(b)}" for v, a, b in r["chosen"])
        lines.append(f"* {wl}, {mode}, {nch} channel(s): measured {meas}. Model picks {cho}.\n")
    lines.append("\nThe straight line cannot follow the cache regime (2·N·S below the 256 MB Infinity Cache "
                 "runs partly from cache, and the smallest sizes are launch-bound), which is why the fit error is "
                 "large at the small end; the pages offer the formula to make falsifiable predictions, not to "
                 "replace measurement.\n")
    return "".join(lines)


def defaults(res) -> str:
    out = []
    for n, nch in CLASS_POINTS:
        parts = []
        for mode in ("stepwise", "fused"):
            r = fit_of(res, n, nch, mode)
            if r is None:
                return f"missing the sweep of {n} ranks at {nch} channels"
            f = r["fits"]
            parts.append("{{%.6g, %.6g}, {%.6g, %.6g}}" % (f["ring"]["alpha_us"], f["ring"]["bw"],
                                                         f["tree"]["alpha_us"], f["tree"]["bw"]))
        out.append("    {" + ", ".join(parts) + "},   // " + f"{n} ranks, {nch} channels")
    return "\n".join(out)


def read_points(path: str):
    """Sweep points: JSON lines of the sweep, or its tab-separated table
    (header line, then one point per line; '#' lines are comments)."""
    with open(path, encoding="utf-8") as f:
        lines = [ln.rstrip("\n") for ln in f if ln.strip() and not ln.startswith("#")]
    if lines and lines[0].lstrip().startswith("{"):
        return [json.loads(ln) for ln in lines]
    head = lines[0].split("\t")
    out = []
    for ln in lines[1:]:
        row = {}
        for k, v in zip(head, ln.split("\t")):
            try:
                row[k] = int(v)
            except ValueError:
                try:
                    row[k] = float(v)
                except ValueError:
                    row[k] = v
        out.append(row)
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("jsonl", nargs="+")
    ap.add_argument("--out", default=None)
    ap.add_argument("--defaults", action="store_true")
    args = ap.parse_args()
    rows = []
    for path in args.jsonl:
        rows += read_points(path)
    res = analyse(rows)
    text = report(res, args.jsonl)
    if args.out:
        with open(args.out, "w", encoding="utf-8") as f:
            f.write(text)
    print(text)
    if args.defaults:
        print(defaults(res))
    return 0


if __name__ == "__main__":
    sys.exit(main())
