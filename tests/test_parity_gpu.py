"""GPU parity: the persistent kernel against the CPU oracle on the same seeded
inputs, through the C ABI.

Bar (the parity contract of the decode path): per-step logits within max-abs
5e-2 of the oracle; greedy token ids equal wherever the oracle's top-2 margin
exceeds 0.1; step advanced exactly; task-dependency order exact.  The oracle
runs teacher-forced on the GPU's own token sequence (oracle/parity.py), so
every iteration of every request is compared; each test asserts how many
iterations it compared and a floor on the margin-checked ones, and logs both.
"""
import time

import numpy as np
import pytest

import oracle
import synth
from oracle import parity
import persistent_task_runtime_amd as mpk
from persistent_task_runtime_amd import timeline

pytestmark = pytest.mark.gpu

LOGIT_TOL = parity.LOGIT_TOL


@pytest.fixture(scope="module")
def torch_dev(rocm_device):
    import torch

    return torch


def log(msg):
    print(msg, flush=True)


def check_against_oracle(w, n_iter, weights, res, min_checked=0, min_written=0, chunk=0, kv=None):
    """Teacher-forced oracle on the GPU's tokens; the full protocol; floors on
    the compared and margin-checked counts."""
    om = oracle.Model(w.shape, weights)
    K = V = None
    if kv is not None:
        K, V = kv
    elif w.kv_prefill:
        K, V = synth.make_kv_prefill(w.shape, w.batch, w.max_seq, w.kv_prefill, seed=w.seed)
    t0 = time.time()
    ol, oam, omg = parity.teacher_forced(om, w.shape, res["tokens"], w.step0, n_iter, w.max_seq, K, V,
                                         chunk=chunk, progress=log)
    rep = parity.compare(synth.make_tokens(w), w.prompt_len, w.step0, n_iter, res["logits"], res["tokens"],
                         res["step"], ol, oam, omg)
    log("%s: %s (oracle %.1f s)" % (w.name, rep, time.time() - t0))
    assert rep.compared == w.batch * n_iter
    assert rep.checked >= min_checked, "only %d margin-checked decisions" % rep.checked
    assert rep.checked_written >= min_written, "only %d margin-checked written tokens" % rep.checked_written
    return rep


def run_tiny(torch, gains="ones", n_iter=None, per_op=False, trace=False, seed=0):
    from persistent_task_runtime_amd import runner

    w = synth.workload("tiny", seed=seed, gains=gains)
    n_iter = n_iter or w.n_iter
    weights = synth.make_model(w.shape, seed=w.seed, gains=w.gains)
    model = runner.DeviceModel(w.shape, weights=weights)
    res = runner.run_workload(w, n_iter, want_logits=True, per_op=per_op, trace=trace, model=model)
    return w, weights, res


@pytest.mark.parametrize("gains", ["ones", "random"])
def test_tiny_greedy_matches_oracle(torch_dev, gains):
    """The tiny decoder over its whole workload: 38 prompt iterations and 32
    generated tokens, every iteration compared."""
    log("tiny greedy, gains=%s" % gains)
    w, weights, res = run_tiny(torch_dev, gains)
    # (the oracle's own greedy run margin-checks 51-52 of 70 decisions, 32 on written ids)
    check_against_oracle(w, w.n_iter, weights, res, min_checked=35, min_written=20)
    res["session"].close()


def test_megakernel_equals_per_op_bitwise(torch_dev):
    log("megakernel vs per-op")
    n = 20
    _, _, a = run_tiny(torch_dev, n_iter=n)
    _, _, b = run_tiny(torch_dev, n_iter=n, per_op=True)
    assert np.array_equal(a["tokens"], b["tokens"])
    assert np.array_equal(a["logits"].view(np.uint32), b["logits"].view(np.uint32))
    a["session"].close(), b["session"].close()


def test_real_width_megakernel_equals_per_op_and_oracle(torch_dev):
    """Real-width operators (a Qwen3-8B layer and a 16384-id head, every
    streaming operator on the fast whole-group path): several persistent runs
    and the one-launch-per-operator path give bit-identical activations,
    logits and tokens, and the logits match the oracle.  Each row is computed
    by one wavefront with fixed arithmetic, whichever wavefront takes it, so
    any difference is a race (such a race showed as one wrong row in a few
    runs out of 24)."""
    from persistent_task_runtime_amd import runner

    log("real-width: wide1")
    w = synth.workload("wide1", gains="random")
    weights = synth.make_model(w.shape, seed=w.seed, gains=w.gains)
    model = runner.DeviceModel(w.shape, weights=weights)
    ref = runner.run_workload(w, w.n_iter, want_logits=True, model=model, per_op=True)
    for rep in range(6):
        got = runner.run_workload(w, w.n_iter, want_logits=True, model=model)
        assert np.array_equal(got["tokens"], ref["tokens"]), rep
        bad = np.nonzero(got["logits"].view(np.uint32) != ref["logits"].view(np.uint32))
        assert len(bad[0]) == 0, "run %d: %d logits differ, first (iter, req, id) %s" % (
            rep, len(bad[0]), list(zip(*bad))[:4])
        got["session"].close()
    check_against_oracle(w, w.n_iter, weights, ref, min_checked=4, min_written=3)
    ref["session"].close()


def test_run_to_run_deterministic_and_resumable(torch_dev):
    import torch
    from persistent_task_runtime_amd import runner

    log("resume a + b == a + b")
    w = synth.workload("tiny")
    weights = synth.make_model(w.shape, seed=w.seed)
    model = runner.DeviceModel(w.shape, weights=weights)
    s1 = runner.Session(w, model, logits_iters=30)
    s1.run(30)
    torch.cuda.synchronize()
    s1.check_status()
    l_all = s1.logits.cpu().numpy().copy()
    toks_all = s1.tokens.cpu().numpy()
    kc_all = s1.kc[0].cpu().numpy()
    s2 = runner.Session(w, model, logits_iters=30)
    s2.run(12)
    torch.cuda.synchronize()
    l_a = s2.logits.cpu().numpy()[:12].copy()
    s2.run(18)
    torch.cuda.synchronize()
    s2.check_status()
    l_b = s2.logits.cpu().numpy()[:18]
    assert np.array_equal(np.concatenate([l_a, l_b]).view(np.uint32), l_all.view(np.uint32))
    assert np.array_equal(s2.tokens.cpu().numpy(), toks_all)
    assert np.array_equal(s2.kc[0].cpu().numpy(), kc_all)
    assert int(s2.step.cpu()[0]) == 30
    s1.close(), s2.close()


@pytest.mark.parametrize("static", [False, True])
def test_packed_words_cleared_before_their_stamps_repeat(torch_dev, static):
    """The packed hand-over words (one 32-bit word per element: value and an
    8-bit stamp, st mod 255 + 1) left by a run could look current to a later
    run whose first stamp is 255 after theirs.  Exec A runs 6 iterations,
    exec C exactly 254, so A's next first stamp has the same 8-bit stamp as
    every packed word A left; A must clear them first (and in the static
    array, where C's words overlay A's, because C used it last): its 6 + 24
    iterations equal bitwise one run of 30 of a fresh exec."""
    import torch
    from persistent_task_runtime_amd import runner

    w = synth.workload("tiny")
    weights = synth.make_model(w.shape, seed=w.seed)
    model = runner.DeviceModel(w.shape, weights=weights)
    ref = runner.Session(w, model, logits_iters=30)
    ref.run(30, static=static)
    torch.cuda.synchronize()
    ref.check_status()
    l_ref = ref.logits.cpu().numpy().copy()
    toks_ref = ref.tokens.cpu().numpy()
    ref.close()
    wc = synth.Workload("tiny_c", w.shape, 1, n_iter=254, tokens_width=300, prompt_len=w.prompt_len.copy(),
                        step0=np.zeros(1, np.int32))
    c = runner.Session(wc, model)
    a = runner.Session(w, model, logits_iters=30)
    a.run(6, static=static)
    torch.cuda.synchronize()
    l_a = a.logits.cpu().numpy()[:6].copy()
    c.run(254, static=static)
    torch.cuda.synchronize()
    c.check_status()
    a.run(24, static=static)
    torch.cuda.synchronize()
    a.check_status()
    l_b = a.logits.cpu().numpy()[:24]
    assert np.array_equal(np.concatenate([l_a, l_b]).view(np.uint32), l_ref.view(np.uint32))
    assert np.array_equal(a.tokens.cpu().numpy(), toks_ref)
    a.close(), c.close()


def test_trace_orders_every_dependency(torch_dev):
    log("trace order")
    n = 6
    w, weights, res = run_tiny(torch_dev, n_iter=n, trace=True)
    sess = res["session"]
    info = mpk.mpk_get_graph_info(sess.exe.graph)
    NT = info.num_tasks
    tr = mpk.mpk_read_trace(sess.exe.exe, n * NT).reshape(n, NT)
    assert (tr["task"] == np.arange(NT)[None, :]).all(), "each task exactly once per iteration"
    tasks = [info.tasks[i] for i in range(NT)]
    kinds = [o.kind for o in sess.exe.spec.ops]
    by_op = {}
    for i, t in enumerate(tasks):
        by_op.setdefault(t.op, []).append(i)
    # A task's start ticket is taken once every word it reads is present and
    # before it stores any output, so for every data dependency the
    # producer's ticket is below the consumer's.  Decoder edges: [QKV ->
    # attention -> o_proj -> gate/up -> down] x L -> LM head -> argmax ->
    # next iteration's first QKV (its embedding read waits for the token).
    NONE = 0xFFFFFFFF
    chain = [i for i, k in enumerate(kinds) if k != mpk.MPK_OP_EMBED] + [len(kinds)]  # + argmax task
    sh = w.shape
    d, G = sh.head_dim, sh.n_q // sh.n_kv

    def group_rows(j):
        """virtual QKV rows an attention task of kv head j reads"""
        rows = set(range(j * G * d, (j + 1) * G * d))
        rows |= set(range(sh.n_q * d + j * d, sh.n_q * d + (j + 1) * d))
        rows |= set(range((sh.n_q + sh.n_kv) * d + j * d, (sh.n_q + sh.n_kv) * d + (j + 1) * d))
        return rows

    for s in range(n):
        st = tr[s]["start_ticket"]
        for a, b in zip(chain, chain[1:]):
            pa = [t for t in by_op[a] if st[t] != NONE]
            pb = [t for t in by_op[b] if st[t] != NONE]
            assert pa and pb
            if a < len(kinds) and kinds[a] == mpk.MPK_OP_RMSNORM_LINEAR and \
                    b < len(kinds) and kinds[b] == mpk.MPK_OP_ATTENTION:
                for t in pb:
                    rows = group_rows(tasks[t].nrows)
                    prod = [q for q in pa if rows & set(range(tasks[q].row0, tasks[q].row0 + tasks[q].nrows))]
                    assert prod and max(st[q] for q in prod) < st[t]
            else:
                assert max(st[t] for t in pa) < min(st[t] for t in pb), (s, a, b)
        if s:
            prev = tr[s - 1]["start_ticket"][by_op[chain[-1]]].max()
            assert prev < tr[s]["start_ticket"][by_op[chain[0]]].min()
    # one workgroup per CU: scheduler wavefronts report distinct (XCC, SE, SH, CU)
    ids = set()
    for t in range(NT):
        hw, xcc = int(tr[0]["hw_id"][t]), int(tr[0]["xcc_id"][t])
        ids.add((tasks[t].worker, xcc & 0xF, (hw >> 8) & 0xFF))  # XCC, (SE, SH, CU)
    per_worker = {}
    for wk, *cu in ids:
        per_worker.setdefault(wk, set()).add(tuple(cu))
    assert all(len(v) == 1 for v in per_worker.values())
    cus = [next(iter(v)) for v in per_worker.values()]
    assert len(set(cus)) == len(cus), "two workers shared a CU"
    # the timeline export of the same records: one event per task on its
    # worker's lane, lanes never overlapping, every boundary measured
    doc = timeline.chrome_trace(tr.reshape(-1), tasks, timeline.op_labels(kinds))
    ev = [e for e in doc["traceEvents"] if e.get("cat") == "task"]
    assert len(ev) == n * NT
    lanes = {}
    for e in ev:
        assert e["tid"] == tasks[e["args"]["task"]].worker
        lanes.setdefault((e["pid"], e["tid"]), []).append((e["ts"], e["ts"] + e["dur"]))
    for spans in lanes.values():
        spans.sort()
        assert all(a1 <= b0 + 1e-3 for (_, a1), (b0, _) in zip(spans, spans[1:]))
    gaps = timeline.boundary_gaps(tr.reshape(-1), tasks, NT, chain)
    assert np.isfinite(gaps["span_b"]).all() and (gaps["span_b"] > 0).all()
    sess.close()


def test_batch_rows_match_single_requests(torch_dev):
    import torch
    from persistent_task_runtime_amd import runner

    log("batch 2 vs batch 1")
    base = synth.workload("tiny")
    n = 16
    P = np.array([7, 12], np.int32)
    w2 = synth.Workload("b2", base.shape, 2, n, 40, P, np.zeros(2, np.int32))
    weights = synth.make_model(base.shape, seed=0)
    model = runner.DeviceModel(base.shape, weights=weights)
    r2 = runner.run_workload(w2, n, want_logits=True, model=model)
    toks2 = synth.make_tokens(w2)
    for r in range(2):
        w1 = synth.Workload("b1", base.shape, 1, n, 40, P[r:r + 1], np.zeros(1, np.int32))
        s1 = runner.Session(w1, model, logits_iters=n)
        s1.tokens.copy_(torch.from_numpy(toks2[r:r + 1]).to(s1.tokens.device))
        s1.run(n)
        torch.cuda.synchronize()
        s1.check_status()
        assert np.array_equal(s1.tokens.cpu().numpy()[0], r2["tokens"][r])
        np.testing.assert_allclose(s1.logits.cpu().numpy()[:, 0], r2["logits"][:, r], rtol=0, atol=1e-5)
        s1.close()
    check_against_oracle(w2, n, weights, r2, min_checked=17, min_written=10)
    r2["session"].close()


def test_batch2_real_width_matches_single_requests_and_oracle(torch_dev):
    """Batch 2 at the real widths (a Qwen3-8B layer, 16384-id head): each row
    of the batch equals the request run alone (same tokens, logits within
    1e-5), and both match the oracle."""
    import torch
    from persistent_task_runtime_amd import runner

    log("batch 2 vs batch 1, wide1")
    base = synth.workload("wide1", gains="random")
    n = 9
    P = np.array([4, 6], np.int32)
    w2 = synth.Workload("wide1_b2", base.shape, 2, n, 12, P, np.zeros(2, np.int32), gains="random")
    weights = synth.make_model(base.shape, seed=0, gains="random")
    model = runner.DeviceModel(base.shape, weights=weights)
    r2 = runner.run_workload(w2, n, want_logits=True, model=model)
    toks2 = synth.make_tokens(w2)
    for r in range(2):
        w1 = synth.Workload("wide1_b1", base.shape, 1, n, 12, P[r:r + 1], np.zeros(1, np.int32), gains="random")
        s1 = runner.Session(w1, model, logits_iters=n)
        s1.tokens.copy_(torch.from_numpy(toks2[r:r + 1]).to(s1.tokens.device))
        s1.run(n)
        torch.cuda.synchronize()
        s1.check_status()
        assert np.array_equal(s1.tokens.cpu().numpy()[0], r2["tokens"][r])
        np.testing.assert_allclose(s1.logits.cpu().numpy()[:, 0], r2["logits"][:, r], rtol=0, atol=1e-5)
        s1.close()
    check_against_oracle(w2, n, weights, r2, min_checked=9, min_written=5)
    r2["session"].close()


def test_start_of_run_check_rejects_bad_ids_and_positions(torch_dev):
    """mpk_run_steps checks the meta tensors on the device before the run: a
    prompt id outside the vocabulary at a position the run would feed forward,
    or a position that leaves the tokens tensor, stops the run before any
    iteration (MPK_ERR_SHAPE, iteration -1, the request as task) and leaves
    tokens, step and the K/V cache unchanged.  The host rule (mpk_check_run)
    agrees."""
    import torch
    from persistent_task_runtime_amd import runner

    log("start-of-run check")
    w = synth.workload("tiny")
    model = runner.DeviceModel(w.shape, weights=synth.make_model(w.shape, seed=0))
    s = runner.Session(w, model)
    toks = s.tokens.cpu().numpy().copy()
    bad = toks.copy()
    bad[0, 20] = w.shape.vocab  # a prompt id the 25-iteration run would feed forward at position 20
    s.tokens.copy_(torch.from_numpy(bad).to(s.tokens.device))
    with pytest.raises(mpk.MPKError) as e:
        mpk.mpk_check_run(s.exe.graph, np.zeros(1, np.int32), bad, w.prompt_len, 25)
    assert e.value.code == mpk.MPK_ERR_SHAPE and "position 20" in str(e.value)
    kc0 = s.kc[0].cpu().numpy().copy()
    s.run(25)
    torch.cuda.synchronize()
    assert s.exe.status() == (mpk.MPK_ERR_SHAPE, -1, 0)
    assert int(s.step.cpu()[0]) == 0
    assert np.array_equal(s.tokens.cpu().numpy(), bad)
    assert np.array_equal(s.kc[0].cpu().numpy(), kc0)
    # a run that stops before position 20 reads no id there: accepted
    mpk.mpk_check_run(s.exe.graph, np.zeros(1, np.int32), bad, w.prompt_len, 20)
    s.run(20)
    torch.cuda.synchronize()
    s.check_status()
    assert int(s.step.cpu()[0]) == 20
    # the position would leave the tokens tensor
    s.tokens.copy_(torch.from_numpy(toks).to(s.tokens.device))
    s.step.fill_(w.tokens_width - 3)
    s.run(3)
    torch.cuda.synchronize()
    assert s.exe.status()[0] == mpk.MPK_ERR_SHAPE
    assert int(s.step.cpu()[0]) == w.tokens_width - 3
    s.close()


def test_dedicated_scheduler_mode_matches_coresident(torch_dev):
    """The pages' worker / scheduler split (workers + schedulers / 4 = CUs):
    tiles on the worker CUs only, the argmax task on the first scheduler CU.
    Same tokens and logits (within 1e-5) as the co-resident mode, and the
    oracle's."""
    import torch
    from persistent_task_runtime_amd import runner

    log("dedicated scheduler mode")
    w = synth.workload("tiny")
    weights = synth.make_model(w.shape, seed=0)
    model = runner.DeviceModel(w.shape, weights=weights)
    n = w.n_iter
    ref = runner.run_workload(w, n, want_logits=True, model=model)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    launch = mpk.launch_cfg(cus, sched_mode=mpk.MPK_SCHED_DEDICATED, num_workers=cus - 8, num_schedulers=32)
    got = runner.run_workload(w, n, want_logits=True, model=model, launch=launch)
    info = mpk.mpk_get_graph_info(got["session"].exe.graph)
    assert (info.num_workers, info.num_queues) == (cus - 8, cus)
    assert np.array_equal(got["tokens"], ref["tokens"])
    np.testing.assert_allclose(got["logits"], ref["logits"], rtol=0, atol=1e-5)
    check_against_oracle(w, n, weights, got, min_checked=35, min_written=20)
    ref["session"].close(), got["session"].close()


def test_watchdog_and_abort_end_the_run(torch_dev):
    import torch
    from persistent_task_runtime_amd import runner

    log("watchdog / abort")
    w = synth.workload("tiny")
    model = runner.DeviceModel(w.shape, weights=synth.make_model(w.shape, seed=0))
    # a 1 ns spin limit: the first wait that is not already satisfied expires
    s = runner.Session(w, model, spin_timeout_ns=1)
    s.run(5)
    torch.cuda.synchronize()
    code, it, task = s.exe.status()
    assert code == mpk.MPK_ERR_DEVICE_TIMEOUT and it >= 0 and task >= 0
    s.close()
    # a stop request raised before the run ends it at the first wait
    s = runner.Session(w, model)
    mpk.mpk_set_abort(s.exe.exe, 1)
    s.run(5)
    torch.cuda.synchronize()
    code, it, task = s.exe.status()
    assert code == mpk.MPK_ERR_ABORTED
    mpk.mpk_set_abort(s.exe.exe, 0)
    s.run(3)
    torch.cuda.synchronize()
    s.check_status()
    s.close()


@pytest.mark.parametrize("ctx", [0, 1, 15, 16, 63, 64, 65, 512, 1000, 10300, 32768])
def test_one_layer_matches_oracle(torch_dev, ctx):
    """One Qwen3-8B-shaped layer, KV cache pre-filled N(0,1) to ctx positions,
    input h ~ N(0,1), one decode step at position ctx.  The attention splits
    fold the ctx cached positions in steps of 16 (position ctx itself is the
    owner's own partial), cut into splits of at least 64 positions: 0 (an
    empty cache: only the new position), 1, 15 and 16 (one step, ragged or
    whole), 63 / 64 / 65 (the last step ragged, whole, a single position;
    65 also takes a second split, merged by the owner), 512, 1000 (several
    splits, ragged), 10300 (32 splits of 321-322 positions, the two-step ring
    wrapping), 32768 (32 splits of 1024)."""
    import torch
    from persistent_task_runtime_amd import runner

    log("one 8B layer, context %d" % ctx)
    w = synth.workload("one_layer", tokens_width=ctx + 2, prompt_len=np.array([ctx + 1], np.int32),
                       step0=np.array([ctx], np.int32), kv_prefill=ctx)
    sh = w.shape
    weights = synth.make_model(sh, seed=w.seed, with_embedding=False)
    x = synth.normal_f32(w.seed, "one_layer.h", (1, sh.hidden), 1.0)
    K, V = synth.make_kv_prefill(sh, 1, w.max_seq, w.kv_prefill, seed=w.seed)
    model = runner.DeviceModel(sh, weights=weights)
    x_dev = torch.from_numpy(x).to("cuda:0")
    sess = runner.Session(w, model, kv=(K, V), x_in=x_dev)
    sess.run(1)
    torch.cuda.synchronize()
    sess.check_status()
    h_gpu = sess.x_out.cpu().numpy()[0].astype(np.float64)
    k_gpu = sess.kc[0].cpu().numpy().view(np.uint16)[0]
    v_gpu = sess.vc[0].cpu().numpy().view(np.uint16)[0]
    om = oracle.Model(sh, weights)
    st = oracle.State(sh, np.zeros((1, ctx + 2), np.int32), w.step0, w.prompt_len, w.max_seq, K, V)
    h_or = oracle.layer(om, 0, st, 0, ctx, x[0])
    err = float(np.max(np.abs(h_gpu - h_or)))
    log("h max-abs err %.3g (|h| max %.3g)" % (err, np.max(np.abs(h_or))))
    assert err <= LOGIT_TOL
    # the new K/V row: equal, or one bf16 step apart where the fp32 values straddle a rounding boundary
    for nm, got, want in (("K", k_gpu, st.kcache[0, 0]), ("V", v_gpu, st.vcache[0, 0])):
        a = synth.bf16_bits_to_f32(got[:, ctx]).astype(np.float64)
        b = synth.bf16_bits_to_f32(want[:, ctx]).astype(np.float64)
        bad = np.abs(a - b) > 2.0 ** -7 * np.maximum(np.abs(b), 1e-30)
        where = [(j, int(i), a[j, i], b[j, i]) for j, i in zip(*np.nonzero(bad))][:8]
        assert not bad.any(), "%s row %d: %d elements off, first (head, dim, gpu, oracle): %s" % (
            nm, ctx, int(bad.sum()), where)
        assert np.array_equal(got[:, :ctx], want[:, :ctx]), "pre-filled positions untouched"
    sess.close()


@pytest.fixture(scope="module")
def full_weights():
    """The full model's seeded weights (15.1 GB of bf16), shared by the two
    full-size tests."""
    t0 = time.time()
    wts = synth.make_model(synth.QWEN3_8B, seed=0)
    log("full model weights generated in %.1f s" % (time.time() - t0))
    return wts


@pytest.mark.timeout(900)
def test_full_model_prompt_and_generated_tokens(torch_dev, full_weights):
    """Full Qwen3-8B-shaped model (36 layers, tied 151936-row LM head) on the
    benchmark's workload start: the 39-token seeded prompt (38 ingesting
    iterations) and 8 generated tokens, one persistent launch, every
    iteration compared against the teacher-forced oracle."""
    from persistent_task_runtime_amd import runner

    sh = synth.QWEN3_8B
    P, gen = 39, 8
    n = (P - 1) + gen
    w = synth.Workload("qwen3_8b_prompt39", sh, 1, n, P + gen + 4, np.array([P], np.int32), np.zeros(1, np.int32))
    weights = full_weights
    log("full model: uploading")
    model = runner.DeviceModel(sh, weights=weights)
    res = runner.run_workload(w, n, want_logits=True, model=model)
    res["session"].close()
    del model
    log("gpu done; oracle")
    check_against_oracle(w, n, weights, res, min_checked=20, min_written=3, chunk=8)


@pytest.mark.timeout(900)
def test_benchmark_launch_plan_end_of_generation(torch_dev, full_weights):
    """The benchmark's own plan at full size: the 39-token prompt through the
    one-launch-per-operator path, then the 512 generated tokens as eight
    persistent launches of 64 iterations.  Sampled outputs the oracle
    computes one by one: the last six iterations (positions 544-549, the
    end of the eighth launch) against the oracle teacher-forced on the GPU's
    tokens, with the GPU's own K/V rows of positions 0-543 as its cache;
    step, the prompt slots and the slots past the last one written are
    checked whole, and every generated id is a vocabulary id."""
    import torch
    from persistent_task_runtime_amd import runner

    sh = synth.QWEN3_8B
    P, K, L, n_chk = 39, 512, 64, 6
    n_prompt = P - 1
    total = n_prompt + K
    width = total + 2
    w = synth.Workload("qwen3_8b", sh, 1, n_iter=total, tokens_width=width, prompt_len=np.array([P], np.int32),
                       step0=np.zeros(1, np.int32))
    log("benchmark plan: uploading")
    model = runner.DeviceModel(sh, weights=full_weights)
    sess = runner.Session(w, model, max_seq=width, logits_iters=L)
    sess.run(n_prompt, per_op=True)
    torch.cuda.synchronize()
    sess.check_status()
    for i in range(K // L):
        log("benchmark plan: launch %d of %d iterations" % (i, L))
        sess.run(L)
    torch.cuda.synchronize()
    sess.check_status()
    tokens = sess.tokens.cpu().numpy()
    step = sess.step.cpu().numpy()
    logits = sess.logits.cpu().numpy()  # the last launch's iterations: positions total - L .. total - 1
    p0 = total - n_chk
    kv = []
    for cache in (sess.kc, sess.vc):
        a = np.stack([cache[l].cpu().numpy().view(np.uint16) for l in model.layer_ids])[:, :, :, :total]
        a[:, :, :, p0:] = 0  # the oracle writes its own rows from p0 on
        kv.append(np.ascontiguousarray(a))
    sess.close()
    del model
    assert int(step[0]) == total
    gen = tokens[0, P:total + 1]
    assert ((gen >= 0) & (gen < sh.vocab)).all()
    w_end = synth.Workload("qwen3_8b_end", sh, 1, n_iter=n_chk, tokens_width=width,
                           prompt_len=np.array([P], np.int32), step0=np.array([p0], np.int32))
    res = {"tokens": tokens, "step": step, "logits": logits[L - n_chk:]}
    log("gpu done; oracle at positions %d-%d" % (p0, total - 1))
    check_against_oracle(w_end, n_chk, full_weights, res, min_checked=1, min_written=1, kv=tuple(kv))


@pytest.mark.timeout(900)
def test_long_context_benchmark_plan_end(torch_dev, full_weights):
    """The long-context benchmark's own plan at full size: K/V pre-filled
    N(0,1) to 32768 positions, 2 warm-up iterations, then two persistent
    launches of 63 (positions 32770-32895).  Sampled outputs the oracle
    computes one by one: the last six iterations (positions 32890-32895)
    against the oracle teacher-forced on the GPU's tokens, with the GPU's own
    K/V rows (the prefill and the rows the run wrote) as its cache; at least
    one of them with a token decision (top-2 margin above 0.1)."""
    import torch
    from persistent_task_runtime_amd import runner

    w = synth.workload("qwen3_8b_long")
    sh = w.shape
    L, n_chk = 63, 6
    total = int(w.step0[0]) + 2 + 2 * L
    log("long-context benchmark plan: uploading (K/V prefill per layer)")
    model = runner.DeviceModel(sh, weights=full_weights)
    sess = runner.Session(w, model, logits_iters=L)
    sess.run(2)
    for i in range(2):
        log("long-context benchmark plan: launch %d of %d iterations" % (i, L))
        sess.run(L)
    torch.cuda.synchronize()
    sess.check_status()
    tokens = sess.tokens.cpu().numpy()
    step = sess.step.cpu().numpy()
    logits = sess.logits.cpu().numpy()  # the last launch's iterations
    p0 = total - n_chk
    kv = []
    for cache in (sess.kc, sess.vc):
        a = np.stack([cache[l].cpu().numpy().view(np.uint16) for l in model.layer_ids])
        a[:, :, :, p0:] = 0  # the oracle writes its own rows from p0 on
        kv.append(np.ascontiguousarray(a))
    S = sess.max_seq
    sess.close()
    del model
    assert int(step[0]) == total
    gen = tokens[0, int(w.step0[0]) + 1:total + 1]
    assert ((gen >= 0) & (gen < sh.vocab)).all()
    log("gpu done; oracle at positions %d-%d" % (p0, total - 1))
    om = oracle.Model(sh, full_weights)
    t0 = time.time()
    p0a = np.array([p0], np.int32)
    ol, oam, omg = parity.teacher_forced(om, sh, tokens, p0a, n_chk, S, kv[0], kv[1], chunk=1, progress=log)
    del kv
    rep = parity.compare(synth.make_tokens(w), w.prompt_len, p0a, n_chk, logits[L - n_chk:], tokens, step,
                         ol, oam, omg)
    log("qwen3_8b_long end: %s (oracle %.1f s)" % (rep, time.time() - t0))
    assert rep.compared == n_chk and rep.checked >= 1, str(rep)


@pytest.mark.timeout(900)
def test_long_context_sampled_steps(torch_dev, full_weights):
    """The long-context configuration: the full model with each layer's K/V
    cache pre-filled N(0,1) to 32768 positions, decoding at positions
    32768 .. 32771 (the attention splits then hold ~1024 positions each).
    Four iterations against the oracle: the first consumes the seeded token
    at position 32768, the others the generated ones."""
    from persistent_task_runtime_amd import runner

    n = 4
    w = synth.workload("qwen3_8b_long", n_iter=n)
    assert w.seed == 0
    weights = full_weights
    log("long context: uploading (K/V prefill per layer)")
    model = runner.DeviceModel(w.shape, weights=weights)
    res = runner.run_workload(w, n, want_logits=True, model=model)
    res["session"].close()
    del model
    log("gpu done; oracle")
    check_against_oracle(w, n, weights, res, min_checked=1, min_written=1, chunk=1)
