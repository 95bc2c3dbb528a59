"""CPU ORACLE (test infrastructure only): ctypes binding of ``oracle.c``.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` import this package.  The GPU path never does.

Every function here forwards to the fp64 C oracle; no arithmetic of the
decoder happens in Python.  See ``oracle.c`` for the definition each function
follows and the passage of the pages it cites.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

c_i32, c_i64, c_f64, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (plain C, OpenMP over output rows only)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
                               "-shared", "-fPIC", os.path.join(_HERE, "oracle.c"), "-o", tmp,
                               "-lm"])
        os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        L = ctypes.CDLL(_SO)
        L.orc_bf16_to_f64.restype = c_f64
        L.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        L.orc_rmsnorm.restype = None
        L.orc_rmsnorm.argtypes = [c_i32, c_vp, c_vp, c_f64, c_vp]
        L.orc_linear.restype = None
        L.orc_linear.argtypes = [c_i32, c_i32, c_vp, c_vp, c_vp]
        L.orc_rope.restype = None
        L.orc_rope.argtypes = [c_i32, c_f64, c_i64, c_vp]
        L.orc_softmax.restype = None
        L.orc_softmax.argtypes = [c_i32, c_vp, c_vp]
        L.orc_attention_head.restype = None
        L.orc_attention_head.argtypes = [c_i32, c_i32, c_vp, c_vp, c_vp, c_vp]
        L.orc_gqa_attention.restype = None
        L.orc_gqa_attention.argtypes = [c_i32, c_i32, c_i32, c_i32, c_i64, c_vp, c_vp, c_vp, c_vp]
        L.orc_silu.restype = c_f64
        L.orc_silu.argtypes = [c_f64]
        L.orc_argmax.restype = c_i32
        L.orc_argmax.argtypes = [c_i32, c_vp, c_vp]
        L.orc_layer.restype = None
        L.orc_layer.argtypes = [c_vp, c_i32, c_vp, c_i32, c_i32, c_vp]
        L.orc_lm_head.restype = None
        L.orc_lm_head.argtypes = [c_vp, c_vp, c_vp]
        L.orc_decode.restype = c_i32
        L.orc_decode.argtypes = [c_vp, c_vp, c_i32, c_vp, c_vp, c_vp]
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags.c_contiguous
    return a.ctypes.data


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


# ---- components ---------------------------------------------------------------

def bf16_to_f64(bits: int) -> float:
    return lib().orc_bf16_to_f64(bits)


def f32_to_bf16(x: float) -> int:
    return lib().orc_f32_to_bf16(x)


def rmsnorm(x, gain_bits: np.ndarray, eps: float) -> np.ndarray:
    x = _f64(x)
    g = np.ascontiguousarray(gain_bits, dtype=np.uint16)
    y = np.empty_like(x)
    lib().orc_rmsnorm(x.size, _p(x), _p(g), eps, _p(y))
    return y


def linear(W_bits: np.ndarray, x) -> np.ndarray:
    W = np.ascontiguousarray(W_bits, dtype=np.uint16)
    x = _f64(x)
    rows, cols = W.shape
    assert x.size == cols
    y = np.empty(rows, dtype=np.float64)
    lib().orc_linear(rows, cols, _p(W), _p(x), _p(y))
    return y


def rope(x, pos: int, theta: float) -> np.ndarray:
    y = _f64(x).copy()
    lib().orc_rope(y.size, theta, pos, _p(y))
    return y


def softmax(s) -> np.ndarray:
    s = _f64(s)
    w = np.empty_like(s)
    lib().orc_softmax(s.size, _p(s), _p(w))
    return w


def attention_head(q, K_bits: np.ndarray, V_bits: np.ndarray) -> np.ndarray:
    q = _f64(q)
    K = np.ascontiguousarray(K_bits, dtype=np.uint16)
    V = np.ascontiguousarray(V_bits, dtype=np.uint16)
    n, d = K.shape
    out = np.empty(d, dtype=np.float64)
    lib().orc_attention_head(d, n, _p(q), _p(K), _p(V), _p(out))
    return out


def gqa_attention(q, K_bits: np.ndarray, V_bits: np.ndarray, n: Optional[int] = None) -> np.ndarray:
    """q [n_q, d]; K, V [n_kv, stride, d] bf16 bits; attends positions [0, n)."""
    q = _f64(q)
    K = np.ascontiguousarray(K_bits, dtype=np.uint16)
    V = np.ascontiguousarray(V_bits, dtype=np.uint16)
    n_q, d = q.shape
    n_kv, stride, _ = K.shape
    n = stride if n is None else n
    out = np.empty((n_q, d), dtype=np.float64)
    lib().orc_gqa_attention(n_q, n_kv, d, n, stride, _p(q), _p(K), _p(V), _p(out))
    return out


def silu(g: float) -> float:
    return lib().orc_silu(g)


def argmax(v):
    v = _f64(v)
    m = ctypes.c_double()
    i = lib().orc_argmax(v.size, _p(v), ctypes.byref(m))
    return i, m.value


# ---- model / state ------------------------------------------------------------

class _Model(ctypes.Structure):
    _fields_ = [("layers", c_i32), ("hidden", c_i32), ("n_q", c_i32), ("n_kv", c_i32),
                ("head_dim", c_i32), ("ffn", c_i32), ("vocab", c_i32),
                ("rms_eps", c_f64), ("rope_theta", c_f64),
                ("E", c_vp), ("final_norm", c_vp)] + [
        (n, ctypes.POINTER(c_vp)) for n in ("attn_norm", "wq", "wk", "wv", "q_norm", "k_norm",
                                             "wo", "ffn_norm", "wg", "wu", "wd")]


class _State(ctypes.Structure):
    _fields_ = [("batch", c_i32), ("tokens_width", c_i32), ("max_seq", c_i32),
                ("tokens", c_vp), ("step", c_vp), ("prompt_len", c_vp),
                ("kcache", c_vp), ("vcache", c_vp)]


_PER_LAYER = ("attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "ffn_norm", "wg", "wu", "wd")


class Model:
    """Holds references to the weight arrays (bf16 bits) and the C struct."""

    def __init__(self, shape, weights: Dict[str, np.ndarray], layers=None):
        self.shape = shape
        self.w = weights
        self.layer_ids = list(range(shape.layers)) if layers is None else list(layers)
        L = len(self.layer_ids)
        self._keep = []
        s = _Model()
        s.layers, s.hidden, s.n_q, s.n_kv = L, shape.hidden, shape.n_q, shape.n_kv
        s.head_dim, s.ffn, s.vocab = shape.head_dim, shape.ffn, shape.vocab
        s.rms_eps, s.rope_theta = shape.rms_eps, shape.rope_theta
        if "E" in weights:
            s.E = _p(weights["E"])
            s.final_norm = _p(weights["final_norm"])
        for name in _PER_LAYER:
            arr = (c_vp * L)(*[_p(weights["l%d.%s" % (l, name)]) for l in self.layer_ids])
            self._keep.append(arr)
            setattr(s, name, ctypes.cast(arr, ctypes.POINTER(c_vp)))
        self.s = s


class State:
    """tokens / step / prompt_len and a bf16 KV cache [L][B][n_kv][max_seq][d]."""

    def __init__(self, shape, tokens: np.ndarray, step: np.ndarray, prompt_len: np.ndarray,
                 max_seq: int, kcache: Optional[np.ndarray] = None,
                 vcache: Optional[np.ndarray] = None, n_layers: Optional[int] = None):
        L = shape.layers if n_layers is None else n_layers
        self.tokens = np.ascontiguousarray(tokens, dtype=np.int32).copy()
        self.step = np.ascontiguousarray(step, dtype=np.int32).copy()
        self.prompt_len = np.ascontiguousarray(prompt_len, dtype=np.int32).copy()
        B = self.tokens.shape[0]
        kv_shape = (L, B, shape.n_kv, max_seq, shape.head_dim)
        self.kcache = np.zeros(kv_shape, np.uint16) if kcache is None else np.ascontiguousarray(kcache).copy()
        self.vcache = np.zeros(kv_shape, np.uint16) if vcache is None else np.ascontiguousarray(vcache).copy()
        assert self.kcache.shape == kv_shape and self.vcache.shape == kv_shape
        s = _State()
        s.batch, s.tokens_width, s.max_seq = B, self.tokens.shape[1], max_seq
        s.tokens, s.step, s.prompt_len = _p(self.tokens), _p(self.step), _p(self.prompt_len)
        s.kcache, s.vcache = _p(self.kcache), _p(self.vcache)
        self.s = s


def layer(model: Model, l_index: int, state: State, r: int, pos: int, h) -> np.ndarray:
    """One decoder layer (index into the model's layer list); returns the new h."""
    h = _f64(h).copy()
    lib().orc_layer(ctypes.byref(model.s), l_index, ctypes.byref(state.s), r, pos, _p(h))
    return h


def lm_head(model: Model, h) -> np.ndarray:
    h = _f64(h)
    out = np.empty(model.shape.vocab, np.float64)
    lib().orc_lm_head(ctypes.byref(model.s), _p(h), _p(out))
    return out


def decode(model: Model, state: State, n_iter: int, want_logits: bool = True):
    """Greedy decode; returns (logits [n_iter,B,V] or None, argmax [n_iter,B], margin)."""
    B, V = state.tokens.shape[0], model.shape.vocab
    logits = np.empty((n_iter, B, V), np.float64) if want_logits else None
    am = np.empty((n_iter, B), np.int32)
    mg = np.empty((n_iter, B), np.float64)
    rc = lib().orc_decode(ctypes.byref(model.s), ctypes.byref(state.s), n_iter,
                          _p(logits) if want_logits else None, _p(am), _p(mg))
    if rc != 0:
        raise ValueError("oracle decode: position outside tokens / KV cache")
    return logits, am, mg
