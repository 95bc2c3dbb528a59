"""Pins for the CPU oracle: closed forms, invariants, brute force.

Each test ties one oracle function to something other than itself, chosen so
that a plausible mistake (a dropped term, a wrong sign or index, a transposed
operand, eps in the wrong place, the wrong RoPE pairing or GQA grouping, gate
and up swapped) fails at least one of them.
"""
import math
import os
import subprocess
import sys

import numpy as np
import pytest
from scipy.special import expit
from scipy.special import softmax as sp_softmax

import oracle
import synth

RNG = np.random.default_rng(1234)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Exact bf16 bit patterns for values already representable in bf16."""
    f = np.asarray(x, dtype=np.float32)
    b = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(synth.bf16_bits_to_f32(b), f), "value not exactly representable in bf16"
    return b


def rand_bf16(shape, std=1.0):
    """Random values that are exactly bf16 (truncate float32 to its top 16 bits)."""
    f = (RNG.standard_normal(shape) * std).astype(np.float32)
    b = (f.view(np.uint32) >> 16).astype(np.uint16)
    return b, synth.bf16_bits_to_f32(b).astype(np.float64)


# ---- bf16 -------------------------------------------------------------------

def test_bf16_widening_known_patterns():
    assert oracle.bf16_to_f64(0x3F80) == 1.0
    assert oracle.bf16_to_f64(0xC040) == -3.0
    assert oracle.bf16_to_f64(0x3F81) == 1.0 + 2.0 ** -7
    assert oracle.bf16_to_f64(0x0001) == 2.0 ** -133
    assert oracle.bf16_to_f64(0x7F80) == math.inf


def test_bf16_rounding_is_nearest_even():
    assert oracle.f32_to_bf16(1.0 + 2.0 ** -8) == 0x3F80           # tie -> even (down)
    assert oracle.f32_to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82       # tie -> even (up)
    assert oracle.f32_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -20) == 0x3F81
    assert oracle.f32_to_bf16(-(1.0 + 2.0 ** -8 + 2.0 ** -20)) == 0xBF81
    assert oracle.f32_to_bf16(3.0) == 0x4040


# ---- RMSNorm ----------------------------------------------------------------

@pytest.mark.parametrize("c,eps", [(1e-3, 1e-6), (2.5, 1e-6), (-0.7, 0.5)])
def test_rmsnorm_constant_vector_closed_form(c, eps):
    n = 64
    gain_vals = np.array([1.0, -2.0, 0.5, 3.0] * 16, np.float32)
    y = oracle.rmsnorm(np.full(n, c), bf16_bits(gain_vals), eps)
    expect = gain_vals.astype(np.float64) * c / math.sqrt(c * c + eps)
    np.testing.assert_allclose(y, expect, rtol=1e-14, atol=0)


def test_rmsnorm_unit_rms_and_scale_invariance():
    x = RNG.standard_normal(4096)
    ones = np.full(4096, synth.BF16_ONE, np.uint16)
    y = oracle.rmsnorm(x, ones, 0.0)
    assert abs(math.sqrt(np.mean(y * y)) - 1.0) < 1e-13
    y2 = oracle.rmsnorm(37.5 * x, ones, 0.0)
    np.testing.assert_allclose(y, y2, rtol=1e-13, atol=1e-15)
    g_bits, g = rand_bf16(4096)
    yg = oracle.rmsnorm(x, g_bits, 0.0)
    np.testing.assert_allclose(yg, g * y, rtol=1e-14, atol=1e-300)


# ---- linear -----------------------------------------------------------------

def test_linear_hand_example():
    W = bf16_bits(np.array([[1, 2, 3], [4, 5, 6]], np.float32))
    y = oracle.linear(W, [1.0, 2.0, 3.0])
    assert y.tolist() == [14.0, 32.0]


def test_linear_one_hot_rows_copy_exactly():
    cols = 257
    perm = RNG.permutation(cols)[:31]
    W = np.zeros((31, cols), np.float32)
    W[np.arange(31), perm] = 1.0
    x = RNG.standard_normal(cols)
    y = oracle.linear(bf16_bits(W), x)
    assert np.array_equal(y, x[perm])


def test_linear_matches_library_matmul():
    Wb, Wf = rand_bf16((300, 1000), std=0.02)
    x = RNG.standard_normal(1000)
    y = oracle.linear(Wb, x)
    ref = Wf @ x
    bound = 1000 * 2.0 ** -52 * (np.abs(Wf) @ np.abs(x))
    assert np.all(np.abs(y - ref) <= bound + 1e-300)


# ---- RoPE -------------------------------------------------------------------

def test_rope_position_zero_is_identity():
    x = RNG.standard_normal(128)
    assert np.array_equal(oracle.rope(x, 0, 1e6), x)


def test_rope_half_split_pairs_keep_their_norm():
    d = 128
    x = RNG.standard_normal(d)
    y = oracle.rope(x, 517, 1e6)
    h = d // 2
    np.testing.assert_allclose(x[:h] ** 2 + x[h:] ** 2, y[:h] ** 2 + y[h:] ** 2, rtol=1e-13)
    np.testing.assert_allclose(np.linalg.norm(x), np.linalg.norm(y), rtol=1e-14)


def test_rope_pair_zero_turns_by_position_radians():
    d, p = 64, 3
    e0 = np.zeros(d)
    e0[0] = 1.0
    y = oracle.rope(e0, p, 1e6)
    assert abs(y[0] - math.cos(3.0)) < 1e-15 and abs(y[d // 2] - math.sin(3.0)) < 1e-15
    others = np.delete(y, [0, d // 2])
    assert np.all(others == 0.0)


def test_rope_hand_evaluated_frequency():
    # d = 4, theta = 100: pair 1 turns by p * 100^(-2/4) = p / 10 radians.
    x = np.array([0.0, 1.0, 0.0, 0.0])
    y = oracle.rope(x, 5, 100.0)
    np.testing.assert_allclose(y, [0.0, math.cos(0.5), 0.0, math.sin(0.5)], atol=1e-15)


def test_rope_composes_and_is_relative():
    d = 128
    q, k = RNG.standard_normal(d), RNG.standard_normal(d)
    a, b = 301, 45
    np.testing.assert_allclose(oracle.rope(oracle.rope(q, a, 1e6), b, 1e6),
                               oracle.rope(q, a + b, 1e6), rtol=1e-9, atol=1e-11)
    lhs = oracle.rope(q, a, 1e6) @ oracle.rope(k, b, 1e6)
    rhs = oracle.rope(q, a - b, 1e6) @ k
    assert abs(lhs - rhs) < 1e-10


# ---- softmax / attention -------------------------------------------------------

def test_softmax_closed_form_and_invariants():
    np.testing.assert_allclose(oracle.softmax([0.0, math.log(3.0)]), [0.25, 0.75], rtol=1e-15)
    s = RNG.standard_normal(333) * 5
    w = oracle.softmax(s)
    assert abs(w.sum() - 1.0) < 1e-14
    np.testing.assert_allclose(oracle.softmax(s + 123.0), w, rtol=1e-12)


def test_attention_single_position_returns_v():
    d = 128
    Kb, _ = rand_bf16((1, d))
    Vb, Vf = rand_bf16((1, d))
    out = oracle.attention_head(RNG.standard_normal(d), Kb, Vb)
    assert np.array_equal(out, Vf[0])


def test_attention_identical_keys_give_mean_of_v():
    d, n = 64, 9
    Kb, _ = rand_bf16((1, d))
    Kb = np.repeat(Kb, n, axis=0)
    Vb, Vf = rand_bf16((n, d))
    out = oracle.attention_head(RNG.standard_normal(d), Kb, Vb)
    np.testing.assert_allclose(out, Vf.mean(axis=0), rtol=1e-13, atol=1e-15)


def test_attention_scale_is_inverse_sqrt_d():
    # Scores differ by sqrt(d) * ln 3 / sqrt(d) = ln 3  ->  weights 1/4, 3/4.
    d = 64
    K = np.zeros((2, d), np.float32)
    K[1, 0] = 1.0
    q = np.zeros(d)
    q[0] = math.sqrt(d) * math.log(3.0)
    Vb, Vf = rand_bf16((2, d))
    out = oracle.attention_head(q, bf16_bits(K), Vb)
    np.testing.assert_allclose(out, 0.25 * Vf[0] + 0.75 * Vf[1], rtol=1e-13, atol=1e-15)


def test_attention_matches_brute_force_library_route():
    for (d, n) in [(64, 1), (64, 7), (128, 40)]:
        Kb, Kf = rand_bf16((n, d))
        Vb, Vf = rand_bf16((n, d))
        q = RNG.standard_normal(d)
        ref = sp_softmax(Kf @ q / math.sqrt(d)) @ Vf
        np.testing.assert_allclose(oracle.attention_head(q, Kb, Vb), ref, rtol=1e-11, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    n_q, n_kv, d, n = 8, 2, 64, 13
    Kb, _ = rand_bf16((n_kv, n, d))
    Vb, _ = rand_bf16((n_kv, n, d))
    q = RNG.standard_normal((n_q, d))
    gqa = oracle.gqa_attention(q, Kb, Vb)
    g = n_q // n_kv
    mha = oracle.gqa_attention(q, np.repeat(Kb, g, axis=0), np.repeat(Vb, g, axis=0))
    assert np.array_equal(gqa, mha)


def test_gqa_grouping_is_contiguous():
    # V of kv head j is the constant j; one position -> head h returns h // group.
    n_q, n_kv, d = 8, 4, 64
    V = np.zeros((n_kv, 1, d), np.float32)
    for j in range(n_kv):
        V[j] = j
    Kb, _ = rand_bf16((n_kv, 1, d))
    out = oracle.gqa_attention(RNG.standard_normal((n_q, d)), Kb, bf16_bits(V))
    assert [out[h, 0] for h in range(n_q)] == [h // 2 for h in range(n_q)]


def test_gqa_attends_only_first_n_positions():
    n_kv, d, stride = 2, 64, 10
    Kb, _ = rand_bf16((n_kv, stride, d))
    Vb, _ = rand_bf16((n_kv, stride, d))
    q = RNG.standard_normal((4, d))
    a = oracle.gqa_attention(q, Kb, Vb, n=6)
    Kb2, Vb2 = Kb.copy(), Vb.copy()
    Kb2[:, 6:] = 0x4000
    Vb2[:, 6:] = 0x4000
    assert np.array_equal(a, oracle.gqa_attention(q, Kb2, Vb2, n=6))


# ---- SiLU / argmax ----------------------------------------------------------

def test_silu_identities():
    assert oracle.silu(0.0) == 0.0
    for x in RNG.standard_normal(50) * 4:
        assert abs((oracle.silu(x) - oracle.silu(-x)) - x) < 1e-14
        assert abs(oracle.silu(x) - x * expit(x)) < 1e-14


def test_argmax_ties_take_lowest_index_and_margin():
    v = np.array([1.0, 5.0, 2.0, 5.0, 4.5])
    i, m = oracle.argmax(v)
    assert i == 1 and m == 0.0
    i, m = oracle.argmax(np.array([0.0, -1.0, 3.0, 2.75]))
    assert i == 2 and m == 0.25
    x = RNG.standard_normal(10000)
    assert oracle.argmax(x)[0] == int(np.argmax(x))


# ---- whole-decoder special cases ---------------------------------------------

def _tiny_state(shape, prompt, width, B=1, n_layers=None):
    toks = np.full((B, width), -1, np.int32)
    toks[:, :len(prompt)] = prompt
    return oracle.State(shape, toks, np.zeros(B, np.int32), np.full(B, len(prompt), np.int32),
                        max_seq=width, n_layers=n_layers)


def test_decoder_without_mixing_is_a_closed_form_bigram():
    # Wo = Wd = 0: attention and FFN add nothing, the residual stays E[t] and
    # logits = E . RMSNorm(E[t]; final_norm).  Pins embedding, final norm,
    # LM head, argmax, and the step / tokens rules.
    shape = synth.TINY
    w = synth.make_model(shape, seed=3, gains="random", zero=("wo", "wd"))
    model = oracle.Model(shape, w)
    prompt = synth.uniform_ids(3, "p", 5, shape.vocab)
    st = _tiny_state(shape, prompt, 12)
    logits, am, mg = oracle.decode(model, st, 9)
    Ef = synth.bf16_bits_to_f32(w["E"]).astype(np.float64)
    gf = synth.bf16_bits_to_f32(w["final_norm"]).astype(np.float64)
    toks = st.tokens[0]
    assert np.array_equal(toks[:5], prompt)
    assert st.step[0] == 9
    assert np.all(toks[10:] == -1)
    for s in range(9):
        e = Ef[toks[s]]
        z = gf * e / math.sqrt(np.mean(e * e) + shape.rms_eps)
        ref = Ef @ z
        np.testing.assert_allclose(logits[s, 0], ref, rtol=1e-10, atol=1e-12)
        assert am[s, 0] == int(np.argmax(ref))
        if s + 1 >= 5:
            assert toks[s + 1] == am[s, 0]


def test_ffn_closed_form_one_layer():
    # One layer with Wo = 0: h_out = e + Wd (silu(Wg b) * (Wu b)), b = RMSNorm(e).
    shape = synth.ModelShape(1, 256, 4, 2, 64, 768, 1024)
    w = synth.make_model(shape, seed=5, gains="random", zero=("wo",))
    model = oracle.Model(shape, w)
    st = _tiny_state(shape, [7], 4)
    e = synth.bf16_bits_to_f32(w["E"][7]).astype(np.float64)
    h = oracle.layer(model, 0, st, 0, 0, e)
    f = lambda k: synth.bf16_bits_to_f32(w["l0." + k]).astype(np.float64)
    b = f("ffn_norm") * e / math.sqrt(np.mean(e * e) + shape.rms_eps)
    g, u = f("wg") @ b, f("wu") @ b
    ref = e + f("wd") @ (g * expit(g) * u)
    np.testing.assert_allclose(h, ref, rtol=1e-10, atol=1e-13)


def test_attention_block_closed_form_with_zero_queries():
    # Wq = Wk = 0 -> q = k = 0 after QK-norm -> uniform attention weights:
    # o_h = mean over positions of V[kv head of h]; Wd = 0 removes the FFN, so
    # h_out = h + Wo o.  The current position's V is bf16(float32(Wv a)).
    shape = synth.ModelShape(1, 256, 4, 2, 64, 768, 1024)
    w = synth.make_model(shape, seed=6, gains="random", zero=("wq", "wk", "wd"))
    model = oracle.Model(shape, w)
    pos = 5
    K, V = synth.make_kv_prefill(shape, 1, 8, pos, seed=6)
    toks = np.zeros((1, 8), np.int32)
    st = oracle.State(shape, toks, np.zeros(1, np.int32), np.ones(1, np.int32), 8, K, V)
    h0 = RNG.standard_normal(256)
    h = oracle.layer(model, 0, st, 0, pos, h0)
    f = lambda k: synth.bf16_bits_to_f32(w["l0." + k]).astype(np.float64)
    a = f("attn_norm") * h0 / math.sqrt(np.mean(h0 * h0) + shape.rms_eps)
    v_cur = (f("wv") @ a).astype(np.float32)
    v_cur = synth.bf16_bits_to_f32(np.array([oracle.f32_to_bf16(x) for x in v_cur], np.uint16))
    Vall = synth.bf16_bits_to_f32(st.vcache[0, 0]).astype(np.float64)   # [n_kv, 8, d]
    assert np.array_equal(Vall[:, pos].reshape(-1), v_cur.astype(np.float64))
    o = np.concatenate([Vall[hh // 2, :pos + 1].mean(axis=0) for hh in range(4)])
    np.testing.assert_allclose(h, h0 + f("wo") @ o, rtol=1e-10, atol=1e-12)
    # k = 0 exactly after QK-norm and RoPE -> cached keys are +-0
    assert np.all((st.kcache[0, 0, :, pos] & 0x7FFF) == 0)


def test_prompt_positions_are_never_overwritten():
    shape = synth.TINY
    w = synth.make_model(shape, seed=2)
    model = oracle.Model(shape, w)
    prompt = synth.uniform_ids(2, "p", 10, shape.vocab)
    st = _tiny_state(shape, prompt, 10)
    _, am, _ = oracle.decode(model, st, 9, want_logits=False)
    assert np.array_equal(st.tokens[0], prompt) and st.step[0] == 9


def test_decode_rejects_positions_outside_the_tensors():
    shape = synth.TINY
    model = oracle.Model(shape, synth.make_model(shape, seed=2))
    st = _tiny_state(shape, [1, 2], 4)
    with pytest.raises(ValueError):
        oracle.decode(model, st, 4, want_logits=False)


def test_batch_rows_are_independent():
    shape = synth.TINY
    w = synth.make_model(shape, seed=4)
    model = oracle.Model(shape, w)
    pa = synth.uniform_ids(4, "a", 6, shape.vocab)
    pb = synth.uniform_ids(4, "b", 6, shape.vocab)
    toks = np.full((2, 14), -1, np.int32)
    toks[0, :6], toks[1, :6] = pa, pb
    st2 = oracle.State(shape, toks, np.zeros(2, np.int32), np.full(2, 6, np.int32), 14)
    l2, _, _ = oracle.decode(model, st2, 12)
    for r, p in enumerate([pa, pb]):
        st1 = _tiny_state(shape, p, 14)
        l1, _, _ = oracle.decode(model, st1, 12)
        assert np.array_equal(l1[:, 0], l2[:, r])
        assert np.array_equal(st1.tokens[0], st2.tokens[r])


def test_kv_cache_resume_is_bitwise():
    # decode(a) then decode(b) == decode(a + b): all state lives in tokens,
    # step and the cache.
    shape = synth.TINY
    model = oracle.Model(shape, synth.make_model(shape, seed=8))
    prompt = synth.uniform_ids(8, "p", 4, shape.vocab)
    s1 = _tiny_state(shape, prompt, 16)
    la, _, _ = oracle.decode(model, s1, 6)
    lb, _, _ = oracle.decode(model, s1, 7)
    s2 = _tiny_state(shape, prompt, 16)
    lab, _, _ = oracle.decode(model, s2, 13)
    assert np.array_equal(np.concatenate([la, lb]), lab)
    assert np.array_equal(s1.tokens, s2.tokens) and np.array_equal(s1.kcache, s2.kcache)


def test_thread_count_does_not_change_bits():
    code = ("import numpy as np, synth, oracle\n"
            "sh = synth.TINY\n"
            "m = oracle.Model(sh, synth.make_model(sh, seed=9))\n"
            "t = np.full((1, 12), -1, np.int32); t[0, :3] = [5, 6, 7]\n"
            "st = oracle.State(sh, t, np.zeros(1, np.int32), np.full(1, 3, np.int32), 12)\n"
            "l, a, g = oracle.decode(m, st, 10)\n"
            "import sys; sys.stdout.buffer.write(l.tobytes())\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    outs = []
    for nt in ("1", "5"):
        env = dict(os.environ, OMP_NUM_THREADS=nt, PYTHONPATH=root)
        outs.append(subprocess.run([sys.executable, "-c", code], env=env, check=True,
                                   capture_output=True).stdout)
    assert outs[0] == outs[1] and len(outs[0]) == 10 * 1024 * 8


def test_layer_wiring_from_pinned_components():
    # The layer is the composition of the pinned parts in the order
    # RMSNorm -> QKV -> per-head QK-norm -> RoPE (q and k) -> bf16 cache ->
    # GQA attention -> Wo + residual -> RMSNorm -> SwiGLU -> Wd + residual.
    shape = synth.ModelShape(1, 256, 4, 2, 64, 768, 1024)
    w = synth.make_model(shape, seed=11, gains="random")
    model = oracle.Model(shape, w)
    pos, S = 6, 8
    K, V = synth.make_kv_prefill(shape, 1, S, pos, seed=11)
    st = oracle.State(shape, np.zeros((1, S), np.int32), np.zeros(1, np.int32),
                      np.ones(1, np.int32), S, K, V)
    h0 = RNG.standard_normal(256)
    h = oracle.layer(model, 0, st, 0, pos, h0)
    f = lambda k: synth.bf16_bits_to_f32(w["l0." + k]).astype(np.float64)
    g = lambda k: w["l0." + k]
    eps, th, d = shape.rms_eps, shape.rope_theta, 64
    a = oracle.rmsnorm(h0, g("attn_norm"), eps)
    q = (f("wq") @ a).reshape(4, d)
    k = (f("wk") @ a).reshape(2, d)
    v = (f("wv") @ a).reshape(2, d)
    q = np.stack([oracle.rope(oracle.rmsnorm(x, g("q_norm"), eps), pos, th) for x in q])
    k = np.stack([oracle.rope(oracle.rmsnorm(x, g("k_norm"), eps), pos, th) for x in k])
    to_bf16 = np.vectorize(lambda x: oracle.f32_to_bf16(float(np.float32(x))), otypes=[np.uint16])
    assert np.array_equal(st.kcache[0, 0, :, pos], to_bf16(k))
    assert np.array_equal(st.vcache[0, 0, :, pos], to_bf16(v))
    Kc, Vc = K[0, 0].copy(), V[0, 0].copy()
    Kc[:, pos], Vc[:, pos] = to_bf16(k), to_bf16(v)
    o = oracle.gqa_attention(q, Kc, Vc, n=pos + 1).reshape(-1)
    h1 = h0 + f("wo") @ o
    b = oracle.rmsnorm(h1, g("ffn_norm"), eps)
    gg, uu = f("wg") @ b, f("wu") @ b
    ref = h1 + f("wd") @ (gg * expit(gg) * uu)
    np.testing.assert_allclose(h, ref, rtol=1e-10, atol=1e-12)


# ---- symmetries of the composed decoder --------------------------------------
# Relabelling that the definition says cannot matter: FFN units, kv heads with
# their query groups, query heads within a group, hidden dimensions.  The
# whole multi-layer decoder must give the same logits (fp64; only the order of
# a few sums changes).  A wrong GQA grouping, a transposed projection, a gain
# applied to the wrong axis or gate/up paired with the wrong down column breaks
# one of them.

def _scaled(bits, k):
    """bf16 bits times 2**k, exactly (only the exponent moves)."""
    f = synth.bf16_bits_to_f32(bits).astype(np.float32) * np.float32(2.0 ** k)
    out = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(synth.bf16_bits_to_f32(out), f)
    return out


def _mixing_model(shape, seed):
    # sharper attention and a stronger FFN than N(0, 0.02) gives, so that the
    # permutations act on a decoder far from linear
    w = synth.make_model(shape, seed=seed, gains="random")
    for l in range(shape.layers):
        for key_, k in (("wq", 3), ("wk", 3), ("wg", 2), ("wu", 2), ("wo", 1), ("wd", 1)):
            n = "l%d.%s" % (l, key_)
            w[n] = _scaled(w[n], k)
    return w


def _prompt_logits(shape, w, seed, n=10):
    prompt = synth.uniform_ids(seed, "sym", n, shape.vocab)
    st = _tiny_state(shape, prompt, n + 2)
    logits, _, _ = oracle.decode(oracle.Model(shape, w), st, n - 1)
    return logits[:, 0]


def _heads(a, d, order):
    """Row blocks of d rows, taken in `order`."""
    return np.ascontiguousarray(np.concatenate([a[h * d:(h + 1) * d] for h in order], axis=0))


SYM_SHAPES = [synth.ModelShape(2, 256, 4, 2, 64, 768, 1024), synth.ModelShape(2, 192, 6, 2, 64, 320, 512)]


@pytest.mark.parametrize("shape", SYM_SHAPES, ids=["tiny", "q_rows_ne_hidden"])
def test_decoder_invariant_under_ffn_unit_permutation(shape):
    w = _mixing_model(shape, 21)
    ref = _prompt_logits(shape, w, 21)
    p = np.random.default_rng(5).permutation(shape.ffn)
    v = dict(w)
    for l in range(shape.layers):
        v["l%d.wg" % l] = np.ascontiguousarray(w["l%d.wg" % l][p])
        v["l%d.wu" % l] = np.ascontiguousarray(w["l%d.wu" % l][p])
        v["l%d.wd" % l] = np.ascontiguousarray(w["l%d.wd" % l][:, p])
    np.testing.assert_allclose(_prompt_logits(shape, v, 21), ref, rtol=0, atol=1e-9 * np.abs(ref).max())
    # the same permutation on the gate rows alone is not a symmetry
    u = dict(w)
    u["l0.wg"] = np.ascontiguousarray(w["l0.wg"][p])
    assert np.abs(_prompt_logits(shape, u, 21) - ref).max() > 1e-4 * np.abs(ref).max()


@pytest.mark.parametrize("shape", SYM_SHAPES, ids=["tiny", "q_rows_ne_hidden"])
def test_decoder_invariant_under_head_relabelling(shape):
    # kv head j' of the new model is old kv head sig[j'], with its query group;
    # inside every group the query heads are taken in the order tau
    d, G = shape.head_dim, shape.n_q // shape.n_kv
    w = _mixing_model(shape, 22)
    ref = _prompt_logits(shape, w, 22)
    rng = np.random.default_rng(6)
    sig = rng.permutation(shape.n_kv)
    while shape.n_kv > 1 and (sig == np.arange(shape.n_kv)).all():
        sig = rng.permutation(shape.n_kv)
    tau = rng.permutation(G)
    qorder = [int(sig[j]) * G + int(tau[i]) for j in range(shape.n_kv) for i in range(G)]
    v = dict(w)
    for l in range(shape.layers):
        v["l%d.wq" % l] = _heads(w["l%d.wq" % l], d, qorder)
        v["l%d.wk" % l] = _heads(w["l%d.wk" % l], d, sig)
        v["l%d.wv" % l] = _heads(w["l%d.wv" % l], d, sig)
        v["l%d.wo" % l] = np.ascontiguousarray(_heads(w["l%d.wo" % l].T, d, qorder).T)
    np.testing.assert_allclose(_prompt_logits(shape, v, 22), ref, rtol=0, atol=1e-9 * np.abs(ref).max())
    # moving the query heads without their kv heads changes the result
    u = dict(w)
    for l in range(shape.layers):
        u["l%d.wq" % l] = v["l%d.wq" % l]
        u["l%d.wo" % l] = v["l%d.wo" % l]
    assert np.abs(_prompt_logits(shape, u, 22) - ref).max() > 1e-4 * np.abs(ref).max()


@pytest.mark.parametrize("shape", SYM_SHAPES, ids=["tiny", "q_rows_ne_hidden"])
def test_decoder_invariant_under_hidden_permutation(shape):
    # the residual stream's coordinates relabelled everywhere they appear:
    # embedding columns, every RMSNorm gain over the hidden axis, the input
    # columns of q/k/v/gate/up and the output rows of o/down
    w = _mixing_model(shape, 23)
    ref = _prompt_logits(shape, w, 23)
    r = np.random.default_rng(7).permutation(shape.hidden)
    v = dict(w)
    v["E"] = np.ascontiguousarray(w["E"][:, r])
    v["final_norm"] = np.ascontiguousarray(w["final_norm"][r])
    for l in range(shape.layers):
        for key_ in ("attn_norm", "ffn_norm"):
            v["l%d.%s" % (l, key_)] = np.ascontiguousarray(w["l%d.%s" % (l, key_)][r])
        for key_ in ("wq", "wk", "wv", "wg", "wu"):
            v["l%d.%s" % (l, key_)] = np.ascontiguousarray(w["l%d.%s" % (l, key_)][:, r])
        for key_ in ("wo", "wd"):
            v["l%d.%s" % (l, key_)] = np.ascontiguousarray(w["l%d.%s" % (l, key_)][r])
    np.testing.assert_allclose(_prompt_logits(shape, v, 23), ref, rtol=0, atol=1e-9 * np.abs(ref).max())
    # the permutation left out of one gain vector is not a symmetry
    u = dict(v)
    u["l1.ffn_norm"] = w["l1.ffn_norm"]
    assert np.abs(_prompt_logits(shape, u, 23) - ref).max() > 1e-4 * np.abs(ref).max()
