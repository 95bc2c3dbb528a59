"""The teacher-forced comparison (oracle/parity.py) on the CPU: the oracle
fed its own greedy sequence reproduces its own logits bitwise, and each kind
of mistake the protocol is there to catch (a wrong written token at a
high-margin step, a logit off by more than the tolerance, a wrong step, a
touched prompt slot, a write past the run) fails it."""
import numpy as np
import pytest

import oracle
import synth
from oracle import parity


@pytest.fixture(scope="module")
def tiny_run():
    w = synth.workload("tiny")
    n = 50
    weights = synth.make_model(w.shape, seed=0)
    om = oracle.Model(w.shape, weights)
    st = oracle.State(w.shape, synth.make_tokens(w), w.step0, w.prompt_len, w.max_seq)
    lg, am, mg = oracle.decode(om, st, n)
    return w, n, om, st, lg, am, mg


def test_teacher_forced_on_own_greedy_is_bitwise_identical(tiny_run):
    w, n, om, st, lg, am, mg = tiny_run
    tl, tam, tmg = parity.teacher_forced(om, w.shape, st.tokens, w.step0, n, w.max_seq)
    assert np.array_equal(tl, lg) and np.array_equal(tam, am) and np.array_equal(tmg, mg)
    # in chunks, with progress lines
    seen = []
    cl, _, _ = parity.teacher_forced(om, w.shape, st.tokens, w.step0, n, w.max_seq, chunk=16,
                                     progress=seen.append)
    assert np.array_equal(cl, lg) and len(seen) == 4


def test_compare_accepts_the_oracle_and_counts(tiny_run):
    w, n, om, st, lg, am, mg = tiny_run
    rep = parity.compare(synth.make_tokens(w), w.prompt_len, w.step0, n, lg.astype(np.float32), st.tokens,
                         st.step, lg, am, mg)
    assert rep.compared == n
    assert rep.checked == int((mg[:, 0] > parity.MARGIN).sum())
    gen = np.arange(n) + 1 >= int(w.prompt_len[0])
    assert rep.checked_written == int(((mg[:, 0] > parity.MARGIN) & gen).sum())
    assert rep.worst < 1e-6


def test_compare_catches_planted_mistakes(tiny_run):
    w, n, om, st, lg, am, mg = tiny_run
    p0 = synth.make_tokens(w)
    g_l = lg.astype(np.float32)

    def run(l=g_l, t=st.tokens, s=st.step):
        return parity.compare(p0, w.prompt_len, w.step0, n, l, t, s, lg, am, mg)

    # a written token that disagrees at a step whose oracle margin exceeds 0.1
    gen_steps = [s for s in range(n) if s + 1 >= int(w.prompt_len[0]) and mg[s, 0] > parity.MARGIN]
    t = st.tokens.copy()
    s = gen_steps[0]
    t[0, s + 1] = (t[0, s + 1] + 1) % w.shape.vocab
    with pytest.raises(AssertionError, match="token"):
        run(t=t)
    # a logit off by more than the tolerance
    l = g_l.copy()
    l[3, 0, 17] += 0.06
    with pytest.raises(AssertionError, match="logits"):
        run(l=l)
    # step not advanced by exactly n
    with pytest.raises(AssertionError, match="step"):
        run(s=st.step + 1)
    # a prompt slot changed
    t = st.tokens.copy()
    t[0, 5] = (t[0, 5] + 1) % w.shape.vocab
    with pytest.raises(AssertionError):
        run(t=t)
    # a slot written past the run
    t = st.tokens.copy()
    t[0, n + 1] = 3
    with pytest.raises(AssertionError, match="past"):
        run(t=t)
