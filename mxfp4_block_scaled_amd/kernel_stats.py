"""Per-kernel statistics of a rocprofv3 run, from its SQLite output.

    python -m mxfp4_block_scaled_amd.kernel_stats <run>_results.db [--skip N] [--pmc]

Kernel trace (default): per kernel the number of dispatches, then mean / median /
min / max duration in microseconds over the dispatches left after dropping each
kernel's first N (the warm-up calls, whose clocks and caches are not yet in their
steady state), as a Markdown table. With --pmc: the counter values per dispatch
(mean over the dispatches after the first N) of a --pmc run."""

import argparse
import collections
import sqlite3
import statistics


def _rows(db, table, cols):
    cur = db.cursor()
    have = [r[1] for r in cur.execute(f"pragma table_info({table})")]
    ix = {c: have.index(c) for c in cols if c in have}
    return [tuple(r[ix[c]] for c in cols if c in ix) for r in cur.execute(f"select * from {table}")], ix


def kernel_table(path, skip):
    db = sqlite3.connect(path)
    rows, ix = _rows(db, "kernels", ["name", "kernel_name", "start", "end"])
    name_i = 0
    per = collections.defaultdict(list)
    for r in sorted(rows, key=lambda r: r[-2]):
        per[r[name_i]].append((r[-1] - r[-2]) / 1000.0)
    out = ["| kernel | dispatches (kept) | mean µs | median µs | min µs | max µs |", "|---|---|---|---|---|---|"]
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        kept = v[skip:] if len(v) > skip else v
        out.append(f"| `{k[:110]}` | {len(v)} ({len(kept)}) | {statistics.mean(kept):.2f} | "
                   f"{statistics.median(kept):.2f} | {min(kept):.2f} | {max(kept):.2f} |")
    return "\n".join(out)


def pmc_table(path, skip):
    db = sqlite3.connect(path)
    cur = db.cursor()
    cols = [r[1] for r in cur.execute("pragma table_info(counters_collection)")]
    i_name, i_ctr, i_val, i_disp = (cols.index(c) for c in ("kernel_name", "counter_name", "value", "dispatch_id"))
    per = collections.defaultdict(list)
    for r in sorted(cur.execute("select * from counters_collection").fetchall(), key=lambda r: r[i_disp]):
        per[(r[i_name], r[i_ctr])].append(r[i_val])
    out = ["| kernel | counter | dispatches (kept) | mean per dispatch |", "|---|---|---|---|"]
    for (k, c), v in sorted(per.items()):
        kept = v[skip:] if len(v) > skip else v
        out.append(f"| `{k[:110]}` | {c} | {len(v)} ({len(kept)}) | {statistics.mean(kept):.1f} |")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("db")
    ap.add_argument("--skip", type=int, default=0, help="first dispatches of each kernel to leave out")
    ap.add_argument("--pmc", action="store_true", help="counter values of a --pmc run")
    a = ap.parse_args()
    print(pmc_table(a.db, a.skip) if a.pmc else kernel_table(a.db, a.skip))


if __name__ == "__main__":
    main()
