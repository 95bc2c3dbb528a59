"""The host model of the device protocol (mpk_simulate): stamped words, the
per-launch stamp base, owner-split gathers and K/V rows stored before the
word that orders their readers, run on host threads over the builder's own
operator and task tables (no GPU).

Positions 58..69 of a tiny decoder with 32 CUs: the attention context grows
from one split of 64 positions to two at position 64, so the split that
owns the position (and gathers the other's partial) changes mid-run."""
import numpy as np
import pytest

import synth
import persistent_task_runtime_amd as mpk

from test_builder import build, info_arrays

NONE = 0xFFFFFFFF
WIDTH = MAX_SEQ = 200
P0 = 58


def _graph():
    g, spec = build(synth.TINY, num_cus=32, tokens_width=WIDTH, max_seq=MAX_SEQ)
    return g, spec


def _meta():
    toks = np.full((1, WIDTH), -1, np.int32)
    toks[0, :P0 + 1] = synth.uniform_ids(0, "sim.prompt", P0 + 1, synth.TINY.vocab)
    return np.array([P0], np.int32), toks, np.array([20], np.int32)


@pytest.fixture
def sim():
    g, spec = _graph()
    step, toks, plen = _meta()
    s = mpk.mpk_sim_create(g, step, toks, plen, kv_filled=P0)
    yield g, spec, s
    mpk.mpk_sim_destroy(s)
    mpk.mpk_destroy_graph(g)


def _run(g, s, n, base, **kw):
    info = mpk.mpk_get_graph_info(g)
    return mpk.mpk_simulate(s, info.num_tasks, n, base, **kw).reshape(n, info.num_tasks)


def test_every_data_edge_is_ordered_under_jitter(sim):
    g, spec, s = sim
    n = 12
    tr = _run(g, s, n, 1000, seed=7, jitter_us=300, timeout_ms=20000)
    info, tasks, _, _, _ = info_arrays(g)
    NT = info.num_tasks
    assert (tr["task"] == np.arange(NT)[None, :]).all(), "every task exactly once per iteration"
    kinds = [o.kind for o in spec.ops]
    by_op = {}
    for i, t in enumerate(tasks):
        by_op.setdefault(t.op, []).append(i)
    sh = synth.TINY
    d, G = sh.head_dim, sh.n_q // sh.n_kv

    def group_rows(j):
        rows = set(range(j * G * d, (j + 1) * G * d))
        rows |= set(range(sh.n_q * d + j * d, sh.n_q * d + (j + 1) * d))
        rows |= set(range((sh.n_q + sh.n_kv) * d + j * d, (sh.n_q + sh.n_kv) * d + (j + 1) * d))
        return rows

    # edges from the decoder's operator order (not from the builder's tables):
    # embed -> [qkv -> attention -> o -> gate/up -> down] x L -> LM head -> argmax -> next iteration
    chain = [i for i, k in enumerate(kinds) if k != mpk.MPK_OP_EMBED] + [len(kinds)]
    two_splits = 0
    for it in range(n):
        st = tr[it]["start_ticket"]
        for a, b in zip(chain, chain[1:]):
            pa = [t for t in by_op[a] if st[t] != NONE]
            pb = [t for t in by_op[b] if st[t] != NONE]
            assert pa and pb
            if b < len(kinds) and kinds[b] == mpk.MPK_OP_ATTENTION:
                two_splits += len(pb) == 2 * sh.n_kv
                for t in pb:
                    rows = group_rows(tasks[t].nrows)
                    prod = [q for q in pa if rows & set(range(tasks[q].row0, tasks[q].row0 + tasks[q].nrows))]
                    assert prod and max(st[q] for q in prod) < st[t]
            else:
                assert max(st[t] for t in pa) < min(st[t] for t in pb), (it, a, b)
        if it:
            prev = tr[it - 1]["start_ticket"][by_op[chain[-1]]].max()
            assert prev < tr[it]["start_ticket"][by_op[chain[0]]].min()
    # the splits cover positions 0 .. p - 1: 58..64 take one split, 65..69 two
    # (the owner gathers the other)
    assert two_splits == 5 * 2  # 5 iterations x 2 layers
    step, toks = mpk.mpk_sim_read_meta(s, 1, WIDTH)
    assert step[0] == P0 + n
    assert ((toks[0, P0 + 1:P0 + n + 1] >= 0) & (toks[0, P0 + 1:P0 + n + 1] < synth.TINY.vocab)).all()
    assert (toks[0, P0 + n + 1:] == -1).all()


def test_buffers_reused_across_launches_never_pass_a_stale_word(sim):
    g, spec, s = sim
    # consecutive launches, stamp base advanced by each launch's iterations (as
    # the library does): every word a task accepts is this iteration's
    _run(g, s, 5, 100, seed=1, jitter_us=100, timeout_ms=20000)
    _run(g, s, 4, 105, seed=2, jitter_us=100, timeout_ms=20000)
    # a base that repeats the last launch's stamps: the words that launch left
    # behind carry the stamp the next launch waits for, and are caught
    with pytest.raises(mpk.MPKError) as e:
        _run(g, s, 3, 108, seed=3, jitter_us=0, timeout_ms=20000)
    assert e.value.code == mpk.MPK_ERR_GRAPH and "not this iteration" in str(e.value)


def test_kv_row_stored_after_the_publish_is_caught(sim):
    g, spec, s = sim
    with pytest.raises(mpk.MPKError) as e:
        _run(g, s, 4, 10, fault=mpk.MPK_SIM_FAULT_KV_AFTER_PUBLISH, timeout_ms=20000)
    assert e.value.code == mpk.MPK_ERR_GRAPH and "K/V row" in str(e.value)


def test_a_skipped_wait_is_caught(sim):
    g, spec, s = sim
    with pytest.raises(mpk.MPKError) as e:
        _run(g, s, 3, 10, fault=mpk.MPK_SIM_FAULT_SKIP_WAIT, timeout_ms=20000)
    assert e.value.code == mpk.MPK_ERR_GRAPH


def test_a_word_never_published_times_out_and_the_next_launch_recovers(sim):
    g, spec, s = sim
    with pytest.raises(mpk.MPKError) as e:
        _run(g, s, 3, 10, fault=mpk.MPK_SIM_FAULT_DROP_PUBLISH, timeout_ms=300)
    assert e.value.code == mpk.MPK_ERR_DEVICE_TIMEOUT
    # relaunch from the state the stopped run left (a fresh stamp base)
    step, _ = mpk.mpk_sim_read_meta(s, 1, WIDTH)
    _run(g, s, 3, 20, seed=4, jitter_us=50, timeout_ms=20000)
    step2, _ = mpk.mpk_sim_read_meta(s, 1, WIDTH)
    assert step2[0] == step[0] + 3


def test_start_of_run_rule_applies(sim):
    g, spec, s = sim
    with pytest.raises(mpk.MPKError) as e:
        _run(g, s, WIDTH, 10)
    assert e.value.code == mpk.MPK_ERR_SHAPE


def test_batch8_split_k_graph_runs_under_jitter():
    """Batch 8 with the down projection split in K (FFN 12288: three
    4096-column splits per row group, the last one merging the others'
    partial sums): one decoder layer on 256 CUs, 8 requests at their own
    positions, three iterations under random per-task jitter.  Every task
    runs once per iteration (the merging splits wait for the partials, none
    takes a stale word), and step and tokens advance."""
    sh = synth.ModelShape(1, 4096, 32, 8, 128, 12288, 4096)
    B, width = 8, 40
    g, spec = build(sh, B=B, num_cus=256, tokens_width=width, max_seq=width)
    try:
        info, tasks, _, _, _ = info_arrays(g)
        kinds = [o.kind for o in spec.ops]
        down = [i for i, k in enumerate(kinds) if k == mpk.MPK_OP_LINEAR_RESIDUAL][-1]
        assert {t.split for t in tasks if t.op == down} == {0, 1, 2}
        step = np.arange(10, 10 + B, dtype=np.int32)
        toks = np.full((B, width), -1, np.int32)
        for r in range(B):
            toks[r, :step[r] + 1] = synth.uniform_ids(0, "sim8.%d" % r, int(step[r]) + 1, sh.vocab)
        plen = step + 1
        s = mpk.mpk_sim_create(g, step, toks, plen, kv_filled=int(step.max()))
        try:
            n = 3
            tr = mpk.mpk_simulate(s, info.num_tasks, n, 500, seed=3, jitter_us=100,
                                  timeout_ms=60000).reshape(n, info.num_tasks)
            assert (tr["task"] == np.arange(info.num_tasks)[None, :]).all()
            st, tk = mpk.mpk_sim_read_meta(s, B, width)
            assert np.array_equal(st, step + n)
            for r in range(B):
                gen = tk[r, int(step[r]) + 1:int(step[r]) + n + 1]
                assert ((gen >= 0) & (gen < sh.vocab)).all()
        finally:
            mpk.mpk_sim_destroy(s)
    finally:
        mpk.mpk_destroy_graph(g)


def test_batch2_hidden640_graph_runs_under_jitter():
    """The decoder of the hidden-640 GPU parity case at batch 2 (10 q / 5 kv
    heads, FFN 1920, 2 layers, 256 CUs): both requests from position 0 (prompts
    of 12 and 9 ids), 24 iterations under random per-task jitter, then a second
    launch on the same buffers with the stamp base advanced.  Every task runs
    once per iteration with no stale word accepted, and step and the tokens
    past each prompt advance."""
    sh = synth.ModelShape(layers=2, hidden=640, n_q=10, n_kv=5, head_dim=64, ffn=1920, vocab=1024)
    B, width = 2, 40
    g, spec = build(sh, B=B, num_cus=256, tokens_width=width, max_seq=width)
    try:
        info = mpk.mpk_get_graph_info(g)
        plen = np.array([12, 9], np.int32)
        step = np.zeros(B, np.int32)
        toks = np.full((B, width), -1, np.int32)
        for r in range(B):
            toks[r, :plen[r]] = synth.uniform_ids(0, "sim640.%d" % r, int(plen[r]), sh.vocab)
        s = mpk.mpk_sim_create(g, step, toks, plen, kv_filled=0)
        try:
            base = 3000
            for n, seed in ((24, 11), (8, 12)):
                tr = mpk.mpk_simulate(s, info.num_tasks, n, base, seed=seed, jitter_us=60,
                                      timeout_ms=60000).reshape(n, info.num_tasks)
                assert (tr["task"] == np.arange(info.num_tasks)[None, :]).all()
                base += n
            st, tk = mpk.mpk_sim_read_meta(s, B, width)
            assert np.array_equal(st, step + 32)
            for r in range(B):
                assert np.array_equal(tk[r, :plen[r]], toks[r, :plen[r]]), "prompt slots unchanged"
                gen = tk[r, int(plen[r]):33]
                assert ((gen >= 0) & (gen < sh.vocab)).all()
                assert (tk[r, 33:] == -1).all()
        finally:
            mpk.mpk_sim_destroy(s)
    finally:
        mpk.mpk_destroy_graph(g)


def test_full_qwen3_8b_graph_runs_under_jitter():
    """The benchmark's own graph at full size (36 layers, 151936-id LM head,
    batch 1, 256 CUs: 37121 tasks per iteration) across the end of a
    39-token prompt: position 37 consumes a prompt id, 38 the last one and
    writes the first generated id, 39 the next; then one more launch (position
    40) with the stamp base advanced.  Every task runs once per iteration and no stale word is
    accepted."""
    sh = synth.QWEN3_8B
    width, P = 64, 39
    g, spec = build(sh, B=1, num_cus=256, tokens_width=width, max_seq=width)
    try:
        info = mpk.mpk_get_graph_info(g)
        toks = np.full((1, width), -1, np.int32)
        toks[0, :P] = synth.uniform_ids(0, "simfull", P, sh.vocab)
        s = mpk.mpk_sim_create(g, np.array([P - 2], np.int32), toks, np.array([P], np.int32), kv_filled=P - 2)
        try:
            base = 7000
            for n, seed in ((3, 5), (1, 6)):
                tr = mpk.mpk_simulate(s, info.num_tasks, n, base, seed=seed, jitter_us=20,
                                      timeout_ms=120000).reshape(n, info.num_tasks)
                assert (tr["task"] == np.arange(info.num_tasks)[None, :]).all()
                base += n
            st, tk = mpk.mpk_sim_read_meta(s, 1, width)
            assert st[0] == P + 2
            assert np.array_equal(tk[0, :P], toks[0, :P])
            assert ((tk[0, P:P + 3] >= 0) & (tk[0, P:P + 3] < sh.vocab)).all()
            assert (tk[0, P + 3:] == -1).all()
        finally:
            mpk.mpk_sim_destroy(s)
    finally:
        mpk.mpk_destroy_graph(g)


def test_long_context_graph_runs_under_jitter():
    """The long-context benchmark's graph (full model, K/V filled to 32768
    positions, 256 CUs): every layer's attention runs 32 splits per kv head,
    the owner split gathering the other 31 partials.  Three iterations from
    position 32768 under jitter: every attention split runs in every
    iteration, no stale word is accepted, step and tokens advance."""
    sh = synth.QWEN3_8B
    width, P0 = 32800, 32768
    g, spec = build(sh, B=1, num_cus=256, tokens_width=width, max_seq=width)
    try:
        info, tasks, _, _, _ = info_arrays(g)
        kinds = [o.kind for o in spec.ops]
        att = [i for i, t in enumerate(tasks) if t.op < len(kinds) and kinds[t.op] == mpk.MPK_OP_ATTENTION]
        assert len(att) == sh.layers * sh.n_kv * 32
        toks = np.full((1, width), -1, np.int32)
        toks[0, :P0 + 1] = synth.uniform_ids(0, "simlong", P0 + 1, sh.vocab)
        s = mpk.mpk_sim_create(g, np.array([P0], np.int32), toks, np.array([20], np.int32), kv_filled=P0)
        try:
            n = 3
            tr = mpk.mpk_simulate(s, info.num_tasks, n, 9000, seed=8, jitter_us=20,
                                  timeout_ms=120000).reshape(n, info.num_tasks)
            assert (tr["task"] == np.arange(info.num_tasks)[None, :]).all()
            assert (tr["start_ticket"][:, att] != NONE).all()
            st, tk = mpk.mpk_sim_read_meta(s, 1, width)
            assert st[0] == P0 + n
            assert np.array_equal(tk[0, :P0 + 1], toks[0, :P0 + 1])
            assert ((tk[0, P0 + 1:P0 + n + 1] >= 0) & (tk[0, P0 + 1:P0 + n + 1] < sh.vocab)).all()
            assert (tk[0, P0 + n + 1:] == -1).all()
        finally:
            mpk.mpk_sim_destroy(s)
    finally:
        mpk.mpk_destroy_graph(g)


def test_batch8_full_graph_runs_under_jitter():
    """The batch-8 benchmark's graph at full size (36 layers, down projection
    split in K, 256 CUs: 46301 tasks per iteration), eight requests each at
    the last position of its own prompt (lengths 16 to 512): two iterations
    under jitter write every request's first two generated ids; no stale word
    is accepted."""
    sh = synth.QWEN3_8B
    B, width = 8, 600
    g, spec = build(sh, B=B, num_cus=256, tokens_width=width, max_seq=width)
    try:
        info = mpk.mpk_get_graph_info(g)
        plen = np.array([16, 512, 100, 37, 250, 64, 65, 400], np.int32)
        step = plen - 1
        toks = np.full((B, width), -1, np.int32)
        for r in range(B):
            toks[r, :plen[r]] = synth.uniform_ids(0, "simb8.%d" % r, int(plen[r]), sh.vocab)
        s = mpk.mpk_sim_create(g, step, toks, plen, kv_filled=int(step.max()))
        try:
            n = 2
            tr = mpk.mpk_simulate(s, info.num_tasks, n, 12000, seed=9, jitter_us=20,
                                  timeout_ms=120000).reshape(n, info.num_tasks)
            assert (tr["task"] == np.arange(info.num_tasks)[None, :]).all()
            st, tk = mpk.mpk_sim_read_meta(s, B, width)
            assert np.array_equal(st, step + n)
            for r in range(B):
                p = int(plen[r])
                assert np.array_equal(tk[r, :p], toks[r, :p])
                assert ((tk[r, p:p + n] >= 0) & (tk[r, p:p + n] < sh.vocab)).all()
                assert (tk[r, p + n:] == -1).all()
        finally:
            mpk.mpk_sim_destroy(s)
    finally:
        mpk.mpk_destroy_graph(g)
