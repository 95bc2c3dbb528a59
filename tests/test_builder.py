"""Host-side tests of the C ABI: exported symbols, argument validation, the
task-graph builder's tiling, events and queues, and the dependency protocol
run on host threads (no GPU: the builder never touches device memory, so the
"device" pointers here are placeholders)."""
import json
import os
import re

import numpy as np
import pytest

import synth
import persistent_task_runtime_amd as mpk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return mpk.load_library()


def test_library_exports_every_declared_symbol(lib):
    hdr = open(os.path.join(ROOT, "include", "mpk.h")).read()
    declared = set(re.findall(r"^\s*(?:int|void|const char\s*\*)\s*(mpk_[a-z_]+)\s*\(", hdr, re.M))
    assert declared == set(mpk.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


class FakePtrs(dict):
    """Distinct 256-byte-aligned placeholder addresses per name."""

    def __missing__(self, key):
        v = 0x7F0000000000 + (len(self) + 1) * 0x1000000
        self[key] = v
        return v


def build(shape, B=1, tokens_width=64, max_seq=64, num_cus=256, layers=None, logits_iters=0,
          with_embedding=True, with_lm_head=True, launch=None, rows_per_request=1):
    ptrs = FakePtrs()
    spec, meta = mpk.qwen3_graph(shape, B, ptrs, tokens_width, max_seq, layers=layers,
                                 logits_iters=logits_iters, with_embedding=with_embedding,
                                 with_lm_head=with_lm_head, x_in_ptr=ptrs["x_in"],
                                 rows_per_request=rows_per_request)
    g = mpk.mpk_build_graph(mpk.model_cfg(shape, B, max_seq), launch or mpk.launch_cfg(num_cus),
                            spec.c_tensors(), spec.ops, meta)
    return g, spec


def info_arrays(g):
    info = mpk.mpk_get_graph_info(g)
    tasks = [info.tasks[i] for i in range(info.num_tasks)]
    ev_cnt = [info.event_count[i] for i in range(info.num_events)]
    ev_op = [info.event_op[i] for i in range(info.num_events)]
    qlen = [info.queue_len[w] for w in range(info.num_queues)]
    queues = [[info.queues[w * info.max_queue + k] for k in range(qlen[w])] for w in range(info.num_queues)]
    return info, tasks, ev_cnt, ev_op, queues


def test_full_model_tiles_fill_every_cu():
    g, spec = build(synth.QWEN3_8B, tokens_width=551, max_seq=551)
    try:
        info, tasks, ev_cnt, ev_op, queues = info_arrays(g)
        per_op = {}
        for t in tasks:
            per_op.setdefault(t.op, []).append(t)
        kinds = [o.kind for o in spec.ops]
        argmax_op = len(spec.ops)
        assert info.num_ops == len(spec.ops) + 1 and info.sink_op == argmax_op
        # every GEMV-type operator has exactly one tile per CU, except the
        # o projection (the consumer of attention): its tiles take the 256 - 72
        # workers without an attention task (72 = 8 kv heads x 9 splits), which
        # prefetch ahead while the attention runs
        for i, k in enumerate(kinds):
            if k == mpk.MPK_OP_EMBED:
                assert i not in per_op
                continue
            if k == mpk.MPK_OP_ATTENTION:
                assert sorted(t.worker for t in per_op[i]) == list(range(72))
                continue
            after_attn = i > 0 and kinds[i - 1] == mpk.MPK_OP_ATTENTION
            want = list(range(72, 256)) if after_attn else list(range(256))
            assert sorted(t.worker for t in per_op[i]) == want, (i, k)
        # row split of the named shapes (P1 "The API": blocks a multiple of the workers)
        rows = {mpk.MPK_OP_RMSNORM_LINEAR: 24, mpk.MPK_OP_RMSNORM_GATEUP: 96}
        for i, k in enumerate(kinds):
            if k in rows:
                assert {t.nrows for t in per_op[i]} == {rows[k]}
            if k == mpk.MPK_OP_LINEAR_RESIDUAL:
                after_attn = kinds[i - 1] == mpk.MPK_OP_ATTENTION
                assert {t.nrows for t in per_op[i]} == ({22, 23} if after_attn else {16})
                assert sum(t.nrows for t in per_op[i]) == 4096
            if k == mpk.MPK_OP_LMHEAD_ARGMAX:
                assert {t.nrows for t in per_op[i]} == {593, 594}
                assert sum(t.nrows for t in per_op[i]) == 151936
        # attention: 8 kv heads x ceil(551 / 64) = 9 splits at batch 1
        attn = per_op[2]
        assert sorted((t.nrows, t.split) for t in attn) == [(j, c) for j in range(8) for c in range(9)]
        # one argmax task, on worker 0, last in its queue
        assert len(per_op[argmax_op]) == 1 and per_op[argmax_op][0].worker == 0
        assert tasks[queues[0][-1]].op == argmax_op
        # operator order on every queue: per layer an attention task or an o
        # tile (never both), and qkv, gate/up, down; the LM head on each
        for w, q in enumerate(queues):
            ops = [tasks[t].op for t in q]
            assert ops == sorted(ops)
            n_attn = sum(kinds[o] == mpk.MPK_OP_ATTENTION for o in ops if o < argmax_op)
            n_o = sum(o > 0 and kinds[o - 1] == mpk.MPK_OP_ATTENTION for o in ops if o < argmax_op)
            assert (n_attn, n_o) == ((36, 0) if w < 72 else (0, 36)), w
            assert sum(kinds[o] != mpk.MPK_OP_ATTENTION for o in ops if o < argmax_op) == 36 * 3 + n_o + 1
        # events: one flag per tile (GEMV, LM head), per (request, kv head) merge, 1 for argmax
        for e, (c, op) in enumerate(zip(ev_cnt, ev_op)):
            after_attn = op > 0 and op < argmax_op and kinds[op - 1] == mpk.MPK_OP_ATTENTION
            want = 1 if op == argmax_op else {mpk.MPK_OP_ATTENTION: 8}.get(kinds[op], 184 if after_attn else 256)
            assert c == want
    finally:
        mpk.mpk_destroy_graph(g)


def test_dependencies_follow_the_decoder_chain():
    g, spec = build(synth.TINY)
    try:
        info, tasks, ev_cnt, ev_op, queues = info_arrays(g)
        kinds = [o.kind for o in spec.ops]
        deps = {}
        for t in tasks:
            d = tuple(sorted((ev_op[t.dep_event[k]], t.dep_prev[k]) for k in range(3) if t.dep_event[k] >= 0))
            deps.setdefault(t.op, set()).add(d)
        assert all(len(v) == 1 for v in deps.values())
        deps = {k: next(iter(v)) for k, v in deps.items()}
        sink = info.sink_op
        assert sink == len(kinds)  # the argmax task after the LM head
        # op 0 is the (task-less) embedding; layer 0 QKV waits for the previous iteration's argmax
        assert deps[1] == ((sink, 1),)
        for i in range(2, len(kinds) + 1):
            assert deps[i] == ((i - 1, 0),), (i, deps[i])
    finally:
        mpk.mpk_destroy_graph(g)


def test_split_rule_checked_for_cus():
    # P1 "How MPK Works": workers + (local + remote schedulers) / 4 = #SMs; the
    # pages' example GPU has 108 SMs (P4 "工作机制").
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_numbers.json")))
    n = gold["a100_sm_count"]["value"]
    ok = mpk.launch_cfg(n, sched_mode=mpk.MPK_SCHED_DEDICATED, num_workers=n - 8, num_schedulers=32)
    g, _ = build(synth.TINY, launch=ok, num_cus=n)
    mpk.mpk_destroy_graph(g)
    for nw, ns in ((n - 8, 30), (n - 7, 32), (n, 4)):
        bad = mpk.launch_cfg(n, sched_mode=mpk.MPK_SCHED_DEDICATED, num_workers=nw, num_schedulers=ns)
        with pytest.raises(mpk.MPKError) as e:
            build(synth.TINY, launch=bad, num_cus=n)
        assert e.value.code == mpk.MPK_ERR_SPLIT
    # co-resident mode: one scheduler wavefront per worker CU
    with pytest.raises(mpk.MPKError) as e:
        build(synth.TINY, launch=mpk.launch_cfg(256, num_workers=200))
    assert e.value.code == mpk.MPK_ERR_SPLIT


def test_shape_and_graph_errors_are_reported():
    shape = synth.TINY
    ptrs = FakePtrs()
    spec, meta = mpk.qwen3_graph(shape, 1, ptrs, 64, 64)
    mcfg, lcfg = mpk.model_cfg(shape, 1, 64), mpk.launch_cfg(256)
    # wrong dtype
    t = spec.c_tensors()
    t[spec.index["l0.wq"]].dtype = mpk.MPK_F32
    with pytest.raises(mpk.MPKError) as e:
        mpk.mpk_build_graph(mcfg, lcfg, t, spec.ops, meta)
    assert e.value.code == mpk.MPK_ERR_DTYPE
    # wrong shape
    t = spec.c_tensors()
    t[spec.index["l1.wo"]].dims[1] = 255
    with pytest.raises(mpk.MPKError) as e:
        mpk.mpk_build_graph(mcfg, lcfg, t, spec.ops, meta)
    assert e.value.code == mpk.MPK_ERR_SHAPE
    # misaligned attached pointer
    t = spec.c_tensors()
    t[spec.index["l0.wk"]].dev_ptr = ptrs["l0.wk"] + 2
    with pytest.raises(mpk.MPKError) as e:
        mpk.mpk_build_graph(mcfg, lcfg, t, spec.ops, meta)
    assert e.value.code == mpk.MPK_ERR_ALIGN
    # operator reading an activation before its producer
    ops = list(spec.ops)
    ops[1], ops[2] = ops[2], ops[1]
    with pytest.raises(mpk.MPKError) as e:
        mpk.mpk_build_graph(mcfg, lcfg, spec.c_tensors(), ops, meta)
    assert e.value.code == mpk.MPK_ERR_GRAPH
    # LM head not last
    ops = list(spec.ops)
    ops.append(ops[1])
    with pytest.raises(mpk.MPKError) as e:
        mpk.mpk_build_graph(mcfg, lcfg, spec.c_tensors(), ops, meta)
    assert e.value.code in (mpk.MPK_ERR_GRAPH,)
    # a head size the attention kernel is not built for
    m96 = mpk.model_cfg(shape, 1, 64)
    m96.head_dim = 96
    with pytest.raises(mpk.MPKError) as e:
        mpk.mpk_build_graph(m96, lcfg, spec.c_tensors(), spec.ops, meta)
    assert e.value.code == mpk.MPK_ERR_SHAPE and "head_dim" in mpk.mpk_last_error()
    # too many tiles for the rows
    ops = list(spec.ops)
    ops[1].num_tiles = 256
    with pytest.raises(mpk.MPKError) as e:
        mpk.mpk_build_graph(mcfg, lcfg, spec.c_tensors(), ops, meta)
    assert e.value.code == mpk.MPK_ERR_SHAPE
    assert "tiles" in mpk.mpk_last_error()


def test_null_arguments_are_rejected(lib):
    import ctypes

    assert lib.mpk_run_steps(None, 1, None) == mpk.MPK_ERR_INVALID_ARG
    assert lib.mpk_get_status(None, None, None, None) == mpk.MPK_ERR_INVALID_ARG
    out = ctypes.c_void_p()
    assert lib.mpk_compile(None, 0, ctypes.byref(out)) == mpk.MPK_ERR_INVALID_ARG
    assert lib.mpk_build_graph(None, None, None, 0, None, 0, None, ctypes.byref(out)) == mpk.MPK_ERR_INVALID_ARG
    assert "NULL" in mpk.mpk_last_error()
    lib.mpk_destroy_exec(None)
    lib.mpk_destroy_graph(None)


def test_stream_read_arguments_are_checked_before_any_launch(lib):
    """The read-ceiling probe refuses bad arguments on the host (these calls
    never reach the device: the addresses are never dereferenced)."""
    fake, sink = 1 << 20, 1 << 21
    unit = 128 * 1024
    assert lib.mpk_stream_read(None, unit, 256, sink, None) == mpk.MPK_ERR_INVALID_ARG
    assert lib.mpk_stream_read(fake, unit, 256, None, None) == mpk.MPK_ERR_INVALID_ARG
    assert lib.mpk_stream_read(fake, unit, 0, sink, None) == mpk.MPK_ERR_INVALID_ARG
    assert lib.mpk_stream_read(fake, 0, 256, sink, None) == mpk.MPK_ERR_SHAPE
    assert lib.mpk_stream_read(fake, unit + 16, 256, sink, None) == mpk.MPK_ERR_SHAPE
    assert "131072" in mpk.mpk_last_error()
    assert lib.mpk_stream_read(fake + 8, unit, 256, sink, None) == mpk.MPK_ERR_ALIGN


def test_single_layer_graph_without_embedding_or_lm_head():
    sh = synth.ModelShape(1, 4096, 32, 8, 128, 12288, 151936)
    g, spec = build(sh, tokens_width=514, max_seq=513, with_embedding=False, with_lm_head=False)
    try:
        info, tasks, ev_cnt, ev_op, queues = info_arrays(g)
        assert info.sink_op == len(spec.ops) - 1
        first = [t for t in tasks if t.op == 0]
        # no producer: waits for the previous iteration's last operator
        assert {(ev_op[t.dep_event[0]], t.dep_prev[0]) for t in first} == {(info.sink_op, 1)}
    finally:
        mpk.mpk_destroy_graph(g)


def test_more_attention_groups_than_workers_is_a_shape_error():
    # B x n_kv attention groups need one worker each at least (an owner split
    # must never queue behind another group's split)
    sh = synth.ModelShape(1, 1024, 16, 16, 64, 256, 256)
    with pytest.raises(mpk.MPKError) as e:
        build(sh, num_cus=8)
    assert e.value.code == mpk.MPK_ERR_SHAPE and "attention" in mpk.mpk_last_error()
    g, _ = build(sh, num_cus=16)
    mpk.mpk_destroy_graph(g)


def test_host_run_check_follows_the_start_of_run_rule():
    """mpk_check_run: positions inside tokens and the KV cache; every id the
    run reads from tokens (the one at step, then the prompt ids it feeds
    forward) inside the vocabulary; generated slots past the prompt are not
    read."""
    V = synth.TINY.vocab
    g, spec = build(synth.TINY, B=2, tokens_width=64, max_seq=60)
    try:
        toks = np.full((2, 64), -1, np.int32)
        toks[0, :10] = 5
        toks[1, :4] = 7
        plen = np.array([10, 4], np.int32)
        step = np.zeros(2, np.int32)
        mpk.mpk_check_run(g, step, toks, plen, 30)
        bad = toks.copy()
        bad[0, 9] = V
        with pytest.raises(mpk.MPKError) as e:
            mpk.mpk_check_run(g, step, bad, plen, 30)
        assert e.value.code == mpk.MPK_ERR_SHAPE and "request 0" in str(e.value) and "position 9" in str(e.value)
        mpk.mpk_check_run(g, step, bad, plen, 9)  # position 9 is not read by 9 iterations from 0
        bad = toks.copy()
        bad[1, 2] = -3
        with pytest.raises(mpk.MPKError) as e:
            mpk.mpk_check_run(g, step, bad, plen, 3)
        assert "request 1" in str(e.value)
        # a generating request reads only the id at its position
        s2 = np.array([10, 4], np.int32)
        t2 = toks.copy()
        t2[0, 10] = 1
        t2[1, 4] = 2
        mpk.mpk_check_run(g, s2, t2, plen, 20)
        t2[1, 4] = V + 1
        with pytest.raises(mpk.MPKError):
            mpk.mpk_check_run(g, s2, t2, plen, 20)
        # positions: tokens width 64, KV capacity 60
        with pytest.raises(mpk.MPKError, match="leaves"):
            mpk.mpk_check_run(g, np.array([0, 4], np.int32), toks, plen, 61)
        with pytest.raises(mpk.MPKError, match="leaves"):
            mpk.mpk_check_run(g, np.array([-1, 4], np.int32), toks, plen, 1)
    finally:
        mpk.mpk_destroy_graph(g)


def test_rows_per_request_graph_and_run_rule():
    """Batched prompt ingestion (rows_per_request R): B rows are R positions
    of B / R requests - meta tensors and K/V caches per request, activations
    and attention tasks per row - and a run must end inside the prompt:
    step + R n <= prompt_len - 1, every consumed id in the vocabulary."""
    V = synth.TINY.vocab
    g, spec = build(synth.TINY, B=2, tokens_width=64, max_seq=60, rows_per_request=2)
    try:
        assert spec.tensors[spec.index["tokens"]].dims == (1, 64)
        assert spec.tensors[spec.index["l0.kcache"]].dims[0] == 1
        info, tasks, _, _, _ = info_arrays(g)
        att = [t for t in tasks if t.split >= 0]
        assert {t.row0 for t in att} == {0, 1}  # one attention group per row
        toks = np.full((1, 64), -1, np.int32)
        toks[0, :39] = 3
        plen = np.array([39], np.int32)
        mpk.mpk_check_run(g, np.array([0], np.int32), toks, plen, 19)  # positions 0..37
        with pytest.raises(mpk.MPKError, match="past the prompt"):
            mpk.mpk_check_run(g, np.array([0], np.int32), toks, plen, 20)
        with pytest.raises(mpk.MPKError, match="past the prompt"):
            mpk.mpk_check_run(g, np.array([1], np.int32), toks, plen, 19)
        bad = toks.copy()
        bad[0, 37] = V
        with pytest.raises(mpk.MPKError, match="position 37"):
            mpk.mpk_check_run(g, np.array([0], np.int32), bad, plen, 19)
    finally:
        mpk.mpk_destroy_graph(g)
    # rows must be 1, 2 or 8 and divisible into requests
    with pytest.raises(mpk.MPKError) as e:
        build(synth.TINY, B=4, rows_per_request=4)
    assert e.value.code == mpk.MPK_ERR_SHAPE


def test_batch8_tiles_and_refusals():
    """Batch 8 (the MFMA linear tasks): the same row tiles as batch 1 for QKV
    (24 rows = two 16-row blocks), o (16), gate/up (48 pairs) and the LM head
    (593/594); down split in K three ways,
    attention 8 requests x 8 kv heads x 4 splits = 256 tasks; input widths
    must be multiples of 4096 (the 256-wide tiny decoder is refused), and
    batch sizes other than 1, 2 and 8 are refused."""
    g, spec = build(synth.QWEN3_8B, B=8, tokens_width=4096, max_seq=800)
    try:
        info, tasks, _, _, _ = info_arrays(g)
        kinds = [o.kind for o in spec.ops]
        rows = {}
        for t in tasks:
            if t.op < len(kinds):
                rows.setdefault(kinds[t.op], set()).add(t.nrows)
        assert rows[mpk.MPK_OP_RMSNORM_LINEAR] == {24}
        assert rows[mpk.MPK_OP_RMSNORM_GATEUP] == {96}
        assert rows[mpk.MPK_OP_LMHEAD_ARGMAX] == {593, 594}
        attn = [t for t in tasks if t.op == 2]
        assert len(attn) == 256 and {t.row0 for t in attn} == set(range(8))
        assert {t.split for t in attn} == {0, 1, 2, 3}
        # o: 256 tiles of 16 rows; down (K = 12288) splits K in three: 85
        # row groups of 48-49 rows x splits 0, 1, 2 (one 4096-column pass each)
        o_ops = {i for i, k in enumerate(kinds) if k == mpk.MPK_OP_LINEAR_RESIDUAL and kinds[i - 1] == mpk.MPK_OP_ATTENTION}
        down_ops = {i for i, k in enumerate(kinds) if k == mpk.MPK_OP_LINEAR_RESIDUAL} - o_ops
        assert {t.nrows for t in tasks if t.op in o_ops} == {16}
        assert {t.split for t in tasks if t.op in o_ops} == {-1}
        for op in down_ops:
            dt = [t for t in tasks if t.op == op]
            assert len(dt) == 255 and {t.nrows for t in dt} == {48, 49}
            groups = {}
            for t in dt:
                groups.setdefault((t.row0, t.nrows), []).append(t.split)
            assert len(groups) == 85 and all(sorted(v) == [0, 1, 2] for v in groups.values())
            assert sum(n for _, n in groups) == 4096 and len({t.worker for t in dt}) == 255
    finally:
        mpk.mpk_destroy_graph(g)
    g, _ = build(synth.workload("narrow8").shape, B=8, tokens_width=26, max_seq=26)
    mpk.mpk_destroy_graph(g)
    with pytest.raises(mpk.MPKError) as e:
        build(synth.TINY, B=8)
    assert e.value.code == mpk.MPK_ERR_SHAPE and "4096" in str(e.value)
    with pytest.raises(mpk.MPKError) as e:
        build(synth.TINY, B=3)
    assert e.value.code == mpk.MPK_ERR_SHAPE
