"""The timeline export (Chrome trace-event JSON, boundary gaps) on records
from the host simulator of the dependency protocol (no GPU)."""
import json
from types import SimpleNamespace

import numpy as np

import synth
import persistent_task_runtime_amd as mpk
from persistent_task_runtime_amd import timeline

from test_builder import build, info_arrays


def _simulated(n_iter=3):
    g, spec = build(synth.TINY, num_cus=32, tokens_width=16, max_seq=16)
    sim = 0
    try:
        info, tasks, _, _, _ = info_arrays(g)
        toks = np.full((1, 16), -1, np.int32)
        toks[0, :4] = [1, 2, 3, 4]
        sim = mpk.mpk_sim_create(g, np.zeros(1, np.int32), toks, np.array([4], np.int32))
        tr = mpk.mpk_simulate(sim, info.num_tasks, n_iter, 0, seed=3, jitter_us=50, timeout_ms=20000)
        # copies: the task table belongs to the graph, destroyed below
        tasks = [SimpleNamespace(**{f: getattr(t, f) for f in ("op", "tile", "worker", "row0", "nrows", "split")})
                 for t in tasks]
        return tr, tasks, info.num_tasks, [o.kind for o in spec.ops]
    finally:
        mpk.mpk_sim_destroy(sim)
        mpk.mpk_destroy_graph(g)


def test_labels_follow_the_decoder_order():
    kinds = [mpk.MPK_OP_EMBED] + [mpk.MPK_OP_RMSNORM_LINEAR, mpk.MPK_OP_ATTENTION, mpk.MPK_OP_LINEAR_RESIDUAL,
                                  mpk.MPK_OP_RMSNORM_GATEUP, mpk.MPK_OP_LINEAR_RESIDUAL] * 2 + \
        [mpk.MPK_OP_LMHEAD_ARGMAX]
    lab = timeline.op_labels(kinds)
    assert lab == ["embed"] + ["qkv", "attention", "o_proj", "gate_up", "down_proj"] * 2 + ["lm_head", "argmax"]


def test_every_task_is_one_event_on_its_workers_lane(tmp_path):
    tr, tasks, NT, kinds = _simulated()
    labels = timeline.op_labels(kinds)
    path = str(tmp_path / "t.json")
    n = timeline.write_chrome_trace(path, tr, tasks, labels, ns_per_tick=1.0)  # simulator times are ns
    doc = json.load(open(path))
    ev = [e for e in doc["traceEvents"] if e.get("cat") == "task"]
    assert n == len(ev) == int((tr["task"] >= 0).sum()) == 3 * NT
    seen = set()
    for e in ev:
        t = tasks[e["args"]["task"]]
        assert e["tid"] == t.worker and e["name"] == labels[t.op] and e["dur"] >= 0
        seen.add((e["args"]["iteration"], e["args"]["task"]))
    assert len(seen) == len(ev)
    # a worker runs its queue in order: its events never overlap
    lanes = {}
    for e in ev:
        lanes.setdefault((e["pid"], e["tid"]), []).append((e["ts"], e["ts"] + e["dur"]))
    for spans in lanes.values():
        spans.sort()
        for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
            assert a1 <= b0 + 1e-6
    names = {(m["pid"], m["tid"]) for m in doc["traceEvents"] if m.get("name") == "thread_name"}
    assert names == set(lanes)


def test_boundary_gaps_and_histogram():
    tr, tasks, NT, kinds = _simulated()
    chain = [i for i, k in enumerate(kinds) if k != mpk.MPK_OP_EMBED] + [len(kinds)]
    g = timeline.boundary_gaps(tr, tasks, NT, chain, ns_per_tick=1.0)
    assert g["span_b"].shape == (3, len(chain) - 1)
    assert np.isfinite(g["span_b"]).all()
    assert (g["last_start"] >= g["first_start"]).all()
    assert (g["span_b"] >= g["last_start"]).all()
    h = timeline.gap_histogram(g["span_b"])
    assert sum(h.values()) == g["span_b"].size


def test_histogram_bins():
    h = timeline.gap_histogram(np.array([-1.0, 0.0, 0.5, 3.0, 100.0, np.nan]), edges_us=(0, 1, 4))
    assert h == {"<0": 1, "[0,1)": 2, "[1,4)": 1, ">=4": 1}
