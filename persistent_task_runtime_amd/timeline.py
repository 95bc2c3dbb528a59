"""Per-task timeline of a persistent run, for inspection in Perfetto or
chrome://tracing, and the waiting time at every operator boundary.

The pages list a profiling mode that shows when each task of the megakernel
ran ("Mirage Persistent Kernel: Compiling LLMs into a MegaKernel",
agentlenshq.com, "Highlights"; the German hysenlabs.com review, section "Der
dokumentierte Einstieg mit Mirage Persistent Kernel").  Here the records
come from the device trace (`mpk_read_trace`, launch option trace = 1 or 2)
or from the host simulator (`mpk_simulate`), and are laid out with one lane
per worker CU, grouped by XCD when the device reported it.

Host-side formatting only: no part of the decode runs here.
"""
from __future__ import annotations

import json
from typing import Dict, List, Optional, Sequence

import numpy as np

# s_memrealtime counts at 100 MHz on MI355X: 10 ns per tick
DEVICE_NS_PER_TICK = 10.0
_ABSENT = (0, 0xFFFFFFFFFFFFFFFF)


def op_labels(kinds: Sequence[int], names: Optional[Dict[int, str]] = None) -> List[str]:
    """One label per operator of a decoder graph (the argmax task gets the
    index len(kinds)).  Linear operators of a layer alternate as o / down."""
    from . import (MPK_OP_ATTENTION, MPK_OP_EMBED, MPK_OP_LINEAR_RESIDUAL, MPK_OP_LMHEAD_ARGMAX,
                   MPK_OP_RMSNORM_GATEUP, MPK_OP_RMSNORM_LINEAR)

    base = {MPK_OP_EMBED: "embed", MPK_OP_RMSNORM_LINEAR: "qkv", MPK_OP_ATTENTION: "attention",
            MPK_OP_RMSNORM_GATEUP: "gate_up", MPK_OP_LMHEAD_ARGMAX: "lm_head"}
    if names:
        base.update(names)
    out, lin = [], 0
    for k in kinds:
        if k in base:
            out.append(base[k])
        elif k == MPK_OP_LINEAR_RESIDUAL:  # o_proj, then down_proj, in each layer
            out.append("o_proj" if lin % 2 == 0 else "down_proj")
            lin += 1
        else:
            out.append("op%d" % k)
    return out + ["argmax"]


def _present(t) -> bool:
    return int(t) not in _ABSENT


def task_events(records: np.ndarray, tasks, labels: Sequence[str],
                ns_per_tick: float = DEVICE_NS_PER_TICK) -> List[dict]:
    """Chrome trace events for the records that ran (task >= 0).

    Each task becomes a complete event ("ph": "X") on the lane of its worker
    (tid) within its XCD (pid; 0 when the record holds no XCC id).  When the
    record holds a ready time, the part before it (waiting for inputs and
    staging them) is a nested "wait" event.  Times are microseconds from the
    earliest start in the records."""
    ran = records[records["task"] >= 0]
    if len(ran) == 0:
        return []
    t0 = int(ran["t_start"].min())
    us = ns_per_tick / 1000.0
    ev = []
    for r in ran:
        ti = tasks[int(r["task"])]
        name = labels[ti.op] if ti.op < len(labels) else "op%d" % ti.op
        pid = int(r["xcc_id"]) & 0xF if "xcc_id" in r.dtype.names else 0
        ts = (int(r["t_start"]) - t0) * us
        dur = max(0.0, (int(r["t_end"]) - int(r["t_start"])) * us)
        args = {"iteration": int(r["iteration"]), "task": int(r["task"]), "tile": int(ti.tile),
                "rows": [int(ti.row0), int(ti.row0) + int(ti.nrows)]}
        if ti.split >= 0:
            args["split"] = int(ti.split)
        if int(r["start_ticket"]) != 0xFFFFFFFF:  # taken under trace = 1 only
            args["tickets"] = [int(r["start_ticket"]), int(r["end_ticket"])]
        ev.append({"name": name, "cat": "task", "ph": "X", "pid": pid, "tid": int(ti.worker),
                   "ts": ts, "dur": dur, "args": args})
        if "t_ready" in r.dtype.names and _present(r["t_ready"]):
            ready = int(r["t_ready"])
            if int(r["t_start"]) <= ready <= int(r["t_end"]):
                ev.append({"name": "wait", "cat": "wait", "ph": "X", "pid": pid, "tid": int(ti.worker),
                           "ts": ts, "dur": (ready - int(r["t_start"])) * us,
                           "args": {"iteration": int(r["iteration"]), "op": name}})
    return ev


def chrome_trace(records: np.ndarray, tasks, labels: Sequence[str],
                 ns_per_tick: float = DEVICE_NS_PER_TICK) -> dict:
    """The whole trace-event document: task events plus lane names."""
    ev = task_events(records, tasks, labels, ns_per_tick)
    lanes = sorted({(e["pid"], e["tid"]) for e in ev})
    meta = []
    for pid in sorted({p for p, _ in lanes}):
        meta.append({"name": "process_name", "ph": "M", "pid": pid, "args": {"name": "XCD %d" % pid}})
    for pid, tid in lanes:
        meta.append({"name": "thread_name", "ph": "M", "pid": pid, "tid": tid,
                     "args": {"name": "CU worker %d" % tid}})
    return {"traceEvents": meta + ev, "displayTimeUnit": "ns"}


def write_chrome_trace(path: str, records: np.ndarray, tasks, labels: Sequence[str],
                       ns_per_tick: float = DEVICE_NS_PER_TICK) -> int:
    """Write the trace-event JSON to path; returns the number of task events."""
    doc = chrome_trace(records, tasks, labels, ns_per_tick)
    with open(path, "w") as f:
        json.dump(doc, f)
    return sum(1 for e in doc["traceEvents"] if e.get("cat") == "task")


def boundary_gaps(records: np.ndarray, tasks, num_tasks: int, chain: Sequence[int],
                  ns_per_tick: float = DEVICE_NS_PER_TICK) -> Dict[str, np.ndarray]:
    """Per (iteration, boundary) of the operator chain a -> b, in microseconds:

    - "first_start": first start of b minus the last end of a (negative when
      a CU already waits at b while a is still running);
    - "last_start":  last start of b minus the last end of a;
    - "span_b":      last end of b minus the last end of a (the boundary plus
      b's own duration: the critical path of the chain runs through these);
    - "last_ready":  last time a task of b had all its inputs, minus the last
      end of a (how long b's inputs took to arrive);
    - "work_med", "work_max": median and maximum over b's tasks of end minus
      ready (a task's own work once its inputs are there).

    Arrays have shape [iterations, len(chain) - 1]; operators whose tasks
    did not run in an iteration (e.g. attention splits beyond the context)
    count only the tasks that did."""
    recs = records.reshape(-1, num_tasks)
    by_op: Dict[int, List[int]] = {}
    for i in range(num_tasks):
        by_op.setdefault(tasks[i].op, []).append(i)
    us = ns_per_tick / 1000.0
    n_it, n_b = recs.shape[0], len(chain) - 1
    out = {k: np.full((n_it, n_b), np.nan)
           for k in ("first_start", "last_start", "span_b", "last_ready", "work_med", "work_max")}
    for s in range(n_it):
        r = recs[s]
        for k, (a, b) in enumerate(zip(chain, chain[1:])):
            ra = r[by_op[a]]
            rb = r[by_op[b]]
            ra = ra[ra["task"] >= 0]
            rb = rb[rb["task"] >= 0]
            if len(ra) == 0 or len(rb) == 0:
                continue
            end_a = int(ra["t_end"].max())
            out["first_start"][s, k] = (int(rb["t_start"].min()) - end_a) * us
            out["last_start"][s, k] = (int(rb["t_start"].max()) - end_a) * us
            out["span_b"][s, k] = (int(rb["t_end"].max()) - end_a) * us
            ready = rb[rb["t_ready"] != np.iinfo(np.uint64).max]
            if len(ready):
                out["last_ready"][s, k] = (int(ready["t_ready"].max()) - end_a) * us
                work = (ready["t_end"].astype(np.int64) - ready["t_ready"].astype(np.int64)) * us
                out["work_med"][s, k] = float(np.median(work))
                out["work_max"][s, k] = float(work.max())
    return out


def gap_histogram(values: np.ndarray, edges_us: Sequence[float] = (0, 1, 2, 4, 8, 16, 32, 64)) -> Dict[str, int]:
    """Counts of finite gap values per bin [e_i, e_{i+1}); values below the
    first edge and at or above the last one get bins of their own."""
    v = np.asarray(values, dtype=np.float64).ravel()
    v = v[np.isfinite(v)]
    e = list(edges_us)
    hist = {"<%g" % e[0]: int((v < e[0]).sum())}
    for lo, hi in zip(e, e[1:]):
        hist["[%g,%g)" % (lo, hi)] = int(((v >= lo) & (v < hi)).sum())
    hist[">=%g" % e[-1]] = int((v >= e[-1]).sum())
    return hist


def main(argv=None) -> int:
    """Trace a run on the GPU and write its timeline:

        python -m persistent_task_runtime_amd.timeline --workload qwen3_8b \\
            --warmup 38 --iters 8 --out timeline.json

    The first --warmup iterations run untraced-in-the-output (same launch
    options), then --iters traced iterations are exported; a table of the
    boundary gaps per operator (median over iterations and layers) is
    printed."""
    import argparse
    import time

    ap = argparse.ArgumentParser(description=main.__doc__.splitlines()[0])
    ap.add_argument("--workload", default="qwen3_8b", choices=("tiny", "qwen3_8b", "qwen3_8b_long"))
    ap.add_argument("--warmup", type=int, default=None, help="default: the prompt iterations (2 for long)")
    ap.add_argument("--iters", type=int, default=8)
    ap.add_argument("--out", default="timeline.json")
    ap.add_argument("--batch", type=int, default=1, choices=(1, 2, 8),
                    help="requests decoded together (qwen3_8b: each with its own seeded 39-id prompt)")
    args = ap.parse_args(argv)

    import torch

    import synth
    from . import load_library, mpk_get_graph_info, mpk_read_trace
    from . import runner

    load_library()  # before the GPU runtime initialises (see load_library)

    if args.workload == "qwen3_8b_long":
        warm = 2 if args.warmup is None else args.warmup
    else:
        warm = int(synth.workload(args.workload).prompt_len[0]) - 1 if args.warmup is None else args.warmup
    w = synth.workload(args.workload, n_iter=warm + args.iters)
    if args.batch > 1:
        w = synth.Workload(w.name + "_b%d" % args.batch, w.shape, args.batch, w.n_iter, w.tokens_width,
                           np.repeat(w.prompt_len[:1], args.batch), np.repeat(w.step0[:1], args.batch),
                           kv_prefill=w.kv_prefill, seed=w.seed, gains=w.gains)
    model = runner.DeviceModel(w.shape, weights=synth.make_model(w.shape, seed=w.seed))
    sess = runner.Session(w, model, trace=2)
    if warm:
        sess.run(warm)
    torch.cuda.synchronize()
    sess.check_status()
    t = time.time()
    sess.run(args.iters)
    torch.cuda.synchronize()
    sess.check_status()
    wall = (time.time() - t) * 1e3
    info = mpk_get_graph_info(sess.exe.graph)
    NT = info.num_tasks
    tasks = [info.tasks[i] for i in range(NT)]
    kinds = [o.kind for o in sess.exe.spec.ops]
    labels = op_labels(kinds)
    tr = mpk_read_trace(sess.exe.exe, args.iters * NT)
    n = write_chrome_trace(args.out, tr, tasks, labels)
    from . import MPK_OP_EMBED

    chain = [i for i, k in enumerate(kinds) if k != MPK_OP_EMBED] + [len(kinds)]
    gaps = boundary_gaps(tr, tasks, NT, chain)
    print("%d task events over %d iterations (%.3f ms/iteration traced) -> %s"
          % (n, args.iters, wall / args.iters, args.out))
    cols = ("first_start", "last_start", "span_b", "last_ready", "work_med", "work_max")
    print("%-10s" % "operator" + "".join("%13s" % c for c in ("first_start", "last_start", "span", "last_ready",
                                                             "work_med", "work_max")))
    per = {}
    for k, b in enumerate(chain[1:]):
        per.setdefault(labels[b], []).append(k)
    for name, ks in per.items():
        med = [float(np.nanmedian(gaps[f][:, ks])) for f in cols]
        print("%-10s" % name + "".join("%10.2f us" % v for v in med))
    print("boundary span histogram (us):", gap_histogram(gaps["span_b"]))
    sess.close()
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
