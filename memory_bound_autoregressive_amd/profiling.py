"""Summaries of rocprofv3 CSV output for the decode-step kernels.

Every profile is taken with `--output-format csv` (for example `rocprofv3 --kernel-trace --stats
--output-format csv -d DIR -o run -- python3 bench.py ...`): the profiler's default output format
has ended a finished run with a segmentation fault in its own exit path.

  python -m memory_bound_autoregressive_amd.profiling stats    <kernel_stats.csv> <out.md> --command "..."
  python -m memory_bound_autoregressive_amd.profiling counters <counter_collection.csv> <out.md> --command "..."
  python -m memory_bound_autoregressive_amd.profiling traffic  --fetch F.csv --write W.csv \
        --cal-fetch CF.csv --cal-write CW.csv --copy-bytes B --kernel SUBSTR --out traffic.json

`traffic` turns the FETCH_SIZE / WRITE_SIZE counters (KiB per dispatch) of one kernel into HBM
bytes per launch. Each counter is scaled by the factor that makes it read right on a plain device
copy of known size (the copy reads B bytes and writes B bytes), measured in the same way on the
same machine. The result records the digest of the kernel sources it was measured on, so a
later change to the kernels invalidates it.

--context-start C records the contexts the dispatches ran at: the kernel's i-th dispatch (in
Dispatch_Id order) attended C + i + 1 positions, as in a bench.py --no-trace run where every launch
is one token. With --fit-context the per-dispatch bytes are also fitted by least squares to
a + b x context (b: KV traffic per cached token; a: the context-independent part); that needs the
dispatches to span a wide range of contexts.
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import sys


def _rows(path: str):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def stats_table(path: str, top: int = 16) -> str:
    rows = _rows(path)
    out = ["| kernel | calls | avg us | min us | max us | share of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows[:top]:
        out.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} % |")
    return "\n".join(out)


def counter_means(path: str) -> dict:
    """{kernel name: {counter: (dispatches, mean value per dispatch)}}"""
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in _rows(path):
        agg[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: (len(v), sum(v) / len(v)) for c, v in d.items()} for k, d in agg.items()}


def counters_table(path: str) -> str:
    out = ["| kernel | counter | dispatches | mean per dispatch |", "|---|---|---|---|"]
    for k, d in sorted(counter_means(path).items(), key=lambda kv: kv[0]):
        for c, (n, mean) in d.items():
            out.append(f"| `{k[:90]}` | {c} | {n} | {mean:.1f} |")
    return "\n".join(out)


def _one(path: str, kernel: str, counter: str) -> float:
    hits = [(n, m) for k, d in counter_means(path).items() if kernel in k for c, (n, m) in d.items() if c == counter]
    if not hits:
        raise SystemExit(f"no {counter} rows for a kernel matching {kernel!r} in {path}")
    tot = sum(n for n, _ in hits)
    return sum(n * m for n, m in hits) / tot


# sources of the GEMV kernels of the kernel chain, and of the single-launch step
GEMV_SOURCES = ("bw_gemv.hip", "bw_common.h", "bw_dot.h", "bw_internal.h")
STEP_SOURCES = ("bw_persist.hip", "bw_common.h", "bw_dot.h", "bw_lanes.h", "bw_mfma.h", "bw_internal.h")


def _copy(path: str, kernel: str, counter: str) -> float:
    """Mean counter value of the large dispatches of the copy kernel (other, small uses of the
    same kernel in the calibration run, such as argument uploads, are left out)."""
    vals = [float(r["Counter_Value"]) for r in _rows(path) if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not vals:
        raise SystemExit(f"no {counter} rows for {kernel!r} in {path}")
    big = [v for v in vals if v >= 0.5 * max(vals)]
    return sum(big) / len(big)


def _per_dispatch(path: str, kernel: str, counter: str) -> list[float]:
    rows = [r for r in _rows(path) if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not rows or "Dispatch_Id" not in rows[0]:
        raise SystemExit(f"no per-dispatch {counter} rows (with Dispatch_Id) for {kernel!r} in {path}")
    by_id = collections.defaultdict(float)
    for r in rows:  # one row per dispatch (a counter summed over its instances)
        by_id[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    return [by_id[k] for k in sorted(by_id)]


def _linfit(y: list[float], c0: int = 0) -> tuple[float, float, float]:
    """least squares y[i] = a + b (c0 + i + 1); returns (a, b, rms residual)"""
    n = len(y)
    xs = [c0 + i + 1.0 for i in range(n)]
    mx, my = sum(xs) / n, sum(y) / n
    sxx = sum((x - mx) ** 2 for x in xs)
    b = sum((x - mx) * (v - my) for x, v in zip(xs, y)) / sxx
    a = my - b * mx
    rms = (sum((v - a - b * x) ** 2 for x, v in zip(xs, y)) / n) ** 0.5
    return a, b, rms


def traffic(fetch: str, write: str, cal_fetch: str, cal_write: str, copy_bytes: int, kernel: str,
            copy_kernel: str = "copyBuffer", sources: tuple[str, ...] = GEMV_SOURCES,
            fit_context: bool = False, context_start: int | None = None) -> dict:
    from .build import source_digest
    kib = 1024.0
    cf = _copy(cal_fetch, copy_kernel, "FETCH_SIZE") * kib
    cw = _copy(cal_write, copy_kernel, "WRITE_SIZE") * kib
    f_scale, w_scale = copy_bytes / cf, copy_bytes / cw
    kf = _one(fetch, kernel, "FETCH_SIZE") * kib
    kw = _one(write, kernel, "WRITE_SIZE") * kib
    res = {"kernel": kernel, "fetch_kib_per_dispatch": kf / kib, "write_kib_per_dispatch": kw / kib,
           "copy_bytes": copy_bytes, "copy_fetch_kib": cf / kib, "copy_write_kib": cw / kib,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "hbm_bytes_per_launch": kf * f_scale + kw * w_scale, "kernel_sources": list(sources),
           "kernel_source_digest": source_digest(sources)}
    if context_start is not None:
        n = len(_per_dispatch(fetch, kernel, "FETCH_SIZE"))
        res["contexts"] = [context_start + 1, context_start + n]
    if fit_context:
        c0 = context_start or 0
        fv = _per_dispatch(fetch, kernel, "FETCH_SIZE")
        wv = _per_dispatch(write, kernel, "WRITE_SIZE")
        n = min(len(fv), len(wv))
        tot = [fv[i] * kib * f_scale + wv[i] * kib * w_scale for i in range(n)]
        a, b, rms = _linfit(tot, c0)
        res["fit"] = {"bytes_at_context_0": a, "bytes_per_context_token": b, "contexts": [c0 + 1, c0 + n],
                      "rms_residual_bytes": rms,
                      "model": "HBM bytes of one launch = bytes_at_context_0 + bytes_per_context_token x context"}
    return res


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("out")
    s.add_argument("--command", required=True)
    s.add_argument("--title", default="rocprofv3 kernel statistics")
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("out")
    c.add_argument("--command", required=True)
    c.add_argument("--title", default="rocprofv3 counters")
    t = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--cal-fetch", "--cal-write", "--kernel", "--out"):
        t.add_argument(a, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--sources", default="step", choices=("step", "gemv"))
    t.add_argument("--fit-context", action="store_true")
    t.add_argument("--context-start", type=int, default=None)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        text = f"# {a.title}\n\nCommand:\n\n```\n{a.command}\n```\n\n{stats_table(a.csv)}\n"
    elif a.cmd == "counters":
        text = f"# {a.title}\n\nCommand:\n\n```\n{a.command}\n```\n\n{counters_table(a.csv)}\n"
    else:
        res = traffic(a.fetch, a.write, a.cal_fetch, a.cal_write, a.copy_bytes, a.kernel,
                      sources=STEP_SOURCES if a.sources == "step" else GEMV_SOURCES, fit_context=a.fit_context,
                      context_start=a.context_start)
        with open(a.out, "w") as f:
            json.dump(res, f, indent=1)
        print(json.dumps(res))
        return 0
    with open(a.out, "w") as f:
        f.write(text)
    print(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
