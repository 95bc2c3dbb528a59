"""Batched prompt ingestion on the GPU (mpk_meta rows_per_request R > 1):
every iteration takes R consecutive prompt positions of the request as R
rows (each row's attention covers the cache before the chunk plus the
chunk's rows up to its own, from their q/k/v words), then the remaining
prompt positions and the generated tokens go one per iteration through the
ordinary decode run.

Parity: the logits of every position - the chunk rows and the decode
iterations - against the oracle decoding the same tokens one position at a
time, teacher-forced on the GPU's sequence, with the full protocol of
oracle/parity.py (logits within 5e-2, greedy ids where the oracle's margin
exceeds 0.1, step exact, prompt slots unchanged).  R = 2 runs on the batch-2
vector kernels (tiny model), R = 8 on the batch-8 MFMA kernels (hidden
4096)."""
import time

import numpy as np
import pytest

import oracle
import synth
from oracle import parity
import persistent_task_runtime_amd as mpk

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


def prefill_then_decode(w, model, rows, n_gen):
    """Chunks of `rows` positions while they fit before the prompt's last
    position, then one position per iteration to the end of n_gen generated
    tokens.  Returns the GPU state and the logits of every consumed position
    in order ([positions, 1, V])."""
    import torch
    from persistent_task_runtime_amd import runner

    P = int(w.prompt_len[0])
    sess = runner.Session(w, model, logits_iters=P - 1 + n_gen)
    pc = runner.PromptChunks(sess, 0, rows, logits_iters=max(1, (P - 1) // rows))
    nch = pc.chunks_left()
    assert nch == (P - 1) // rows
    t0 = time.time()
    pc.run(nch)
    torch.cuda.synchronize()
    pc.check_status()
    sess.check_status()
    assert int(sess.step[0].item()) == nch * rows
    rest = (P - 1 - nch * rows) + n_gen
    sess.run(rest)
    torch.cuda.synchronize()
    sess.check_status()
    log("%s: %d chunks of %d positions, then %d iterations (%.2f s)" % (w.name, nch, rows, rest, time.time() - t0))
    chunk_logits = pc.logits.cpu().numpy()[:nch].reshape(nch * rows, 1, -1)
    logits = np.concatenate([chunk_logits, sess.logits.cpu().numpy()[:rest]])
    out = {"tokens": sess.tokens.cpu().numpy(), "step": sess.step.cpu().numpy(), "logits": logits,
           "n": nch * rows + rest, "chunks": nch}
    pc.close()
    sess.close()
    return out


def check(w, weights, res, min_checked, min_written, chunk=0):
    om = oracle.Model(w.shape, weights)
    n = res["n"]
    t0 = time.time()
    ol, oam, omg = parity.teacher_forced(om, w.shape, res["tokens"], w.step0, n, w.max_seq, chunk=chunk,
                                         progress=log)
    rep = parity.compare(synth.make_tokens(w), w.prompt_len, w.step0, n, res["logits"], res["tokens"],
                         res["step"], ol, oam, omg)
    log("%s: %s (oracle %.1f s)" % (w.name, rep, time.time() - t0))
    assert rep.compared == n
    assert rep.checked >= min_checked and rep.checked_written >= min_written, str(rep)
    return rep


# Two-row chunks of the tiny decoder are off the GPU for now: a build of the
# attention task with the merging split fixed at the group's last task (since
# taken out) stopped this case with a dependency-wait timeout and then a GPU
# memory fault, and the cause was not found.  The batch-2 kernels are again
# byte-identical to the build these tests passed on, but the case stays off
# the GPU until a cause is shown.
SKIP_R2 = pytest.mark.skip(reason="two-row chunked ingestion faulted the GPU with a since-removed attention "
                                  "change; off the GPU until the cause is shown")


@SKIP_R2
def test_tiny_prompt_in_chunks_of_two(rocm_device):
    from persistent_task_runtime_amd import runner

    w0 = synth.workload("tiny")
    P, gen = int(w0.prompt_len[0]), 24
    w = synth.Workload("tiny_chunks2", w0.shape, 1, P - 1 + gen, P + gen + 4, w0.prompt_len.copy(),
                       np.zeros(1, np.int32))
    weights = synth.make_model(w.shape, seed=w.seed, gains=w.gains)
    model = runner.DeviceModel(w.shape, weights=weights)
    res = prefill_then_decode(w, model, 2, gen)
    assert res["chunks"] == (P - 1) // 2
    check(w, weights, res, min_checked=40, min_written=15)


def test_prompt_in_chunks_of_eight_at_hidden_4096(rocm_device):
    """Two layers at the widths the batch-8 MFMA tasks take: 27-id prompt
    (3 chunks of 8 positions, 2 more prompt iterations), 6 generated."""
    from persistent_task_runtime_amd import runner

    sh = synth.ModelShape(2, 4096, 32, 8, 128, 4096, 4096)
    P, gen = 27, 6
    w = synth.Workload("narrow_chunks8", sh, 1, P - 1 + gen, P + gen + 4, np.array([P], np.int32),
                       np.zeros(1, np.int32), gains="random")
    weights = synth.make_model(sh, seed=w.seed, gains=w.gains)
    model = runner.DeviceModel(sh, weights=weights)
    res = prefill_then_decode(w, model, 8, gen)
    assert res["chunks"] == 3
    check(w, weights, res, min_checked=18, min_written=4)


@SKIP_R2
def test_chunks_past_the_prompt_are_refused(rocm_device):
    """A run whose chunks would reach the prompt's last position stops at its
    start with MPK_ERR_SHAPE (device check), leaving step unchanged."""
    import torch
    from persistent_task_runtime_amd import runner

    w = synth.workload("tiny")
    P = int(w.prompt_len[0])
    model = runner.DeviceModel(w.shape, weights=synth.make_model(w.shape, seed=w.seed))
    sess = runner.Session(w, model)
    pc = runner.PromptChunks(sess, 0, 2)
    pc.run((P - 1) // 2 + 1)
    torch.cuda.synchronize()
    code, it, task = pc.exe.status()
    assert code == mpk.MPK_ERR_SHAPE and it == -1 and task == 0
    assert int(sess.step[0].item()) == 0
    pc.run((P - 1) // 2)
    torch.cuda.synchronize()
    assert pc.exe.status()[0] == 0
    assert int(sess.step[0].item()) == P - 1 - (P - 1) % 2
    pc.close()
    sess.close()


@pytest.fixture(scope="module")
def full_weights_pf():
    t0 = time.time()
    wts = synth.make_model(synth.QWEN3_8B, seed=0)
    log("full model weights generated in %.1f s" % (time.time() - t0))
    return wts


@pytest.mark.timeout(900)
def test_full_model_prompt_in_chunks_of_eight(rocm_device, full_weights_pf):
    """The benchmark's 39-id prompt on the full model: 4 chunks of 8
    positions, 6 prompt iterations, 4 generated tokens, every position
    against the oracle."""
    from persistent_task_runtime_amd import runner

    sh = synth.QWEN3_8B
    P, gen = 39, 4
    w = synth.Workload("qwen3_8b_chunks8", sh, 1, P - 1 + gen, P + gen + 4, np.array([P], np.int32),
                       np.zeros(1, np.int32))
    model = runner.DeviceModel(sh, weights=full_weights_pf)
    res = prefill_then_decode(w, model, 8, gen)
    del model
    assert res["chunks"] == 4
    check(w, full_weights_pf, res, min_checked=15, min_written=1, chunk=8)
