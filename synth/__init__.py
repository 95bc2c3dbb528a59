"""Seeded synthetic workloads: shapes and random inputs, nothing else.

Both the GPU path and the CPU oracle take their inputs from here.  The module
generates random numbers and names the workload shapes; it computes no step of
the decoder.  Values come from ``synth.c`` (counter-based, so any slice of any
tensor can be regenerated on its own with identical bits).

Workloads (the shapes follow the Qwen3-8B demo model that the pages name; the
pages give no weights, so weights are seeded random, see ``make_model``):

* ``tiny``        2 layers, hidden 256, 4 q / 2 kv heads of 64, FFN 768,
                  vocab 1024; 39 random prompt ids, 32 greedy tokens.
* ``one_layer``   one Qwen3-8B-shaped layer, KV cache pre-filled to 512
                  positions with N(0,1) bf16, fp32 input h ~ N(0,1), one step.
* ``wide1``       one Qwen3-8B-shaped layer with a 16384-id tied embedding /
                  LM head; 4 random prompt ids, 5 greedy tokens.
* ``narrow8``     2 layers at the widths the batch-8 linear tasks take (hidden
                  4096, 32 q / 8 kv heads of 128, FFN 4096) with a 4096-id
                  vocabulary; batch 8, prompt lengths uniform in [3, 10],
                  greedy to 14 iterations.
* ``qwen3_8b``    36 layers + tied 151936-row embedding / LM head, batch 1,
                  39 random prompt ids, 512 greedy tokens.
* ``qwen3_8b_b8`` same model at batch 8, prompt lengths uniform in [16, 512],
                  tokens [8, 4096], 256 greedy tokens per request.
* ``qwen3_8b_long`` same model, batch 1, KV cache pre-filled to 32768
                  positions with N(0,1) bf16, 128 greedy tokens.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile synth.c into libsynth.so with gcc (OpenMP)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC",
                               os.path.join(_HERE, "synth.c"), "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        lib = ctypes.CDLL(_SO)
        u64, i64 = ctypes.c_uint64, ctypes.c_int64
        lib.synth_key.restype = u64
        lib.synth_key.argtypes = [u64, ctypes.c_char_p]
        for fn in (lib.synth_normal_bf16, lib.synth_normal_f32):
            fn.restype = None
            fn.argtypes = [u64, u64, u64, ctypes.c_double, ctypes.c_double, ctypes.c_void_p]
        lib.synth_uniform_ids.restype = None
        lib.synth_uniform_ids.argtypes = [u64, u64, u64, ctypes.c_uint32, ctypes.c_void_p]
        lib.synth_uniform_int.restype = None
        lib.synth_uniform_int.argtypes = [u64, u64, u64, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_void_p]
        _lib = lib
    return _lib


def key(seed: int, name: str) -> int:
    return _load().synth_key(seed, name.encode())


def normal_bf16(seed: int, name: str, shape, std: float, mean: float = 0.0,
                out: Optional[np.ndarray] = None) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(mean, std) samples, round-to-nearest-even."""
    n = int(np.prod(shape))
    if out is None:
        out = np.empty(shape, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.size == n and out.flags.c_contiguous
    _load().synth_normal_bf16(key(seed, name), 0, n, mean, std, out.ctypes.data)
    return out


def normal_bf16_into(seed: int, name: str, ptr: int, n: int, std: float, mean: float = 0.0,
                     start: int = 0) -> None:
    """Write elements [start, start+n) of the stream into host memory at ``ptr``."""
    _load().synth_normal_bf16(key(seed, name), start, n, mean, std, ptr)


def normal_f32(seed: int, name: str, shape, std: float, mean: float = 0.0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(shape, dtype=np.float32)
    _load().synth_normal_f32(key(seed, name), 0, n, mean, std, out.ctypes.data)
    return out


def uniform_ids(seed: int, name: str, n: int, vocab: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load().synth_uniform_ids(key(seed, name), 0, n, vocab, out.ctypes.data)
    return out


def uniform_int(seed: int, name: str, n: int, lo: int, hi: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load().synth_uniform_int(key(seed, name), 0, n, lo, hi, out.ctypes.data)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (a bit shift, no rounding)."""
    return (b.astype(np.uint32) << 16).view(np.float32)


BF16_ONE = 0x3F80


@dataclass(frozen=True)
class ModelShape:
    layers: int
    hidden: int
    n_q: int
    n_kv: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float = 1e-6
    rope_theta: float = 1e6

    @property
    def q_rows(self) -> int:
        return self.n_q * self.head_dim

    @property
    def kv_rows(self) -> int:
        return self.n_kv * self.head_dim

    def layer_weight_bytes(self) -> int:
        H, d = self.hidden, self.head_dim
        mats = (self.q_rows + 2 * self.kv_rows) * H + H * self.q_rows + 3 * self.ffn * H
        vecs = 2 * H + 2 * d
        return 2 * (mats + vecs)

    def streamed_weight_bytes(self) -> int:
        """bf16 bytes read once per decode iteration: all layers, final norm and
        the tied LM head (the input embedding is a one-row gather)."""
        return self.layers * self.layer_weight_bytes() + 2 * self.hidden + 2 * self.vocab * self.hidden


TINY = ModelShape(layers=2, hidden=256, n_q=4, n_kv=2, head_dim=64, ffn=768, vocab=1024)
QWEN3_8B = ModelShape(layers=36, hidden=4096, n_q=32, n_kv=8, head_dim=128, ffn=12288,
                      vocab=151936)


@dataclass
class Workload:
    name: str
    shape: ModelShape
    batch: int
    n_iter: int                 # decode iterations (prompt ingestion included)
    tokens_width: int           # tokens[batch, tokens_width]
    prompt_len: np.ndarray      # [batch] int32
    step0: np.ndarray           # [batch] int32, position consumed by the first iteration
    kv_prefill: int = 0         # positions [0, kv_prefill) of the KV cache pre-filled N(0,1)
    seed: int = 0
    gains: str = "ones"
    notes: str = ""
    extra: Dict = field(default_factory=dict)

    @property
    def max_seq(self) -> int:
        """KV capacity needed: every position consumed plus one."""
        return int((self.step0 + self.n_iter).max())


def weight_std(shape: ModelShape) -> float:
    return 0.02


def make_tokens(w: Workload) -> np.ndarray:
    """tokens[B, width] int32: prompt ids (uniform in [0, vocab)), the rest -1."""
    toks = np.full((w.batch, w.tokens_width), -1, dtype=np.int32)
    for r in range(w.batch):
        P = int(w.prompt_len[r])
        toks[r, :P] = uniform_ids(w.seed, "prompt.%d" % r, P, w.shape.vocab)
    if w.kv_prefill:
        # A pre-filled cache stands for positions whose ids are never consumed;
        # the id at the first consumed position is a seeded uniform id.
        for r in range(w.batch):
            p0 = int(w.step0[r])
            toks[r, p0] = uniform_ids(w.seed, "start.%d" % r, 1, w.shape.vocab)[0]
    return toks


def workload(name: str, seed: int = 0, gains: str = "ones", **over) -> Workload:
    if name == "tiny":
        P = 39
        w = Workload("tiny", TINY, 1, n_iter=(P - 1) + 32, tokens_width=P + 32,
                     prompt_len=np.array([P], np.int32), step0=np.zeros(1, np.int32),
                     seed=seed, gains=gains)
    elif name == "one_layer":
        sh = ModelShape(1, 4096, 32, 8, 128, 12288, 151936)
        w = Workload("one_layer", sh, 1, n_iter=1, tokens_width=514,
                     prompt_len=np.array([513], np.int32), step0=np.array([512], np.int32),
                     kv_prefill=512, seed=seed, gains=gains)
    elif name == "wide1":
        # Qwen3-8B layer and head widths, one layer, a 16384-id vocabulary: every
        # streaming operator of the full model's kinds at its real width
        P = 4
        sh = ModelShape(1, 4096, 32, 8, 128, 12288, 16384)
        w = Workload("wide1", sh, 1, n_iter=(P - 1) + 5, tokens_width=P + 5,
                     prompt_len=np.array([P], np.int32), step0=np.zeros(1, np.int32),
                     seed=seed, gains=gains)
    elif name == "narrow8":
        B = 8
        sh = ModelShape(2, 4096, 32, 8, 128, 4096, 4096)
        P = uniform_int(seed, "narrow8.prompt_len", B, 3, 10)
        w = Workload("narrow8", sh, B, n_iter=14, tokens_width=26, prompt_len=P,
                     step0=np.zeros(B, np.int32), seed=seed, gains=gains)
    elif name == "qwen3_8b":
        P = 39
        w = Workload("qwen3_8b", QWEN3_8B, 1, n_iter=(P - 1) + 512, tokens_width=P + 512,
                     prompt_len=np.array([P], np.int32), step0=np.zeros(1, np.int32),
                     seed=seed, gains=gains)
    elif name == "qwen3_8b_b8":
        B = 8
        P = uniform_int(seed, "prompt_len", B, 16, 512)
        w = Workload("qwen3_8b_b8", QWEN3_8B, B, n_iter=256, tokens_width=4096,
                     prompt_len=P, step0=(P - 1).astype(np.int32), seed=seed, gains=gains,
                     notes="prompts ingested before the timed lockstep iterations")
    elif name == "qwen3_8b_long":
        ctx = 32768
        w = Workload("qwen3_8b_long", QWEN3_8B, 1, n_iter=128, tokens_width=ctx + 129,
                     prompt_len=np.array([ctx + 1], np.int32), step0=np.array([ctx], np.int32),
                     kv_prefill=ctx, seed=seed, gains=gains)
    else:
        raise KeyError(name)
    for k, v in over.items():
        setattr(w, k, v)
    return w


def layer_names(l: int):
    return {
        "attn_norm": "l%d.attn_norm" % l, "wq": "l%d.wq" % l, "wk": "l%d.wk" % l,
        "wv": "l%d.wv" % l, "q_norm": "l%d.q_norm" % l, "k_norm": "l%d.k_norm" % l,
        "wo": "l%d.wo" % l, "ffn_norm": "l%d.ffn_norm" % l, "wg": "l%d.wg" % l,
        "wu": "l%d.wu" % l, "wd": "l%d.wd" % l,
    }


def _gain(seed, name, n, gains):
    if gains == "ones":
        return np.full(n, BF16_ONE, dtype=np.uint16)
    if gains == "random":
        return normal_bf16(seed, name, (n,), std=0.1, mean=1.0)
    raise ValueError(gains)


def make_model(shape: ModelShape, seed: int = 0, gains: str = "ones",
               zero: tuple = (), layers=None, with_embedding: bool = True) -> Dict[str, np.ndarray]:
    """All weights as bf16 bit arrays (uint16), row-major [out, in].

    Matrices are N(0, 0.02); RMSNorm gains are 1 (``gains='ones'``) or N(1, 0.1)
    (``gains='random'``).  Names listed in ``zero`` (e.g. ``'wo'``) are all-zero
    matrices in every layer, for closed-form special cases.
    """
    H, d, F = shape.hidden, shape.head_dim, shape.ffn
    std = weight_std(shape)
    m: Dict[str, np.ndarray] = {}
    if with_embedding:
        m["E"] = normal_bf16(seed, "E", (shape.vocab, H), std)
        m["final_norm"] = _gain(seed, "final_norm", H, gains)
    dims = {"wq": (shape.q_rows, H), "wk": (shape.kv_rows, H), "wv": (shape.kv_rows, H),
            "wo": (H, shape.q_rows), "wg": (F, H), "wu": (F, H), "wd": (H, F)}
    for l in (range(shape.layers) if layers is None else layers):
        n = layer_names(l)
        m[n["attn_norm"]] = _gain(seed, n["attn_norm"], H, gains)
        m[n["ffn_norm"]] = _gain(seed, n["ffn_norm"], H, gains)
        m[n["q_norm"]] = _gain(seed, n["q_norm"], d, gains)
        m[n["k_norm"]] = _gain(seed, n["k_norm"], d, gains)
        for key_, dim in dims.items():
            if key_ in zero:
                m[n[key_]] = np.zeros(dim, dtype=np.uint16)
            else:
                m[n[key_]] = normal_bf16(seed, n[key_], dim, std)
    return m


def make_kv_prefill(shape: ModelShape, batch: int, max_seq: int, n_fill: int, seed: int = 0,
                    layers=None):
    """K and V caches, bf16 bits [L][B][n_kv][max_seq][d]; positions < n_fill are
    N(0,1), the rest zero."""
    L = shape.layers if layers is None else len(layers)
    K = np.zeros((L, batch, shape.n_kv, max_seq, shape.head_dim), dtype=np.uint16)
    V = np.zeros_like(K)
    if n_fill:
        for li, l in enumerate(range(shape.layers) if layers is None else layers):
            for r in range(batch):
                for j in range(shape.n_kv):
                    K[li, r, j, :n_fill] = normal_bf16(seed, "kcache.%d.%d.%d" % (l, r, j),
                                                       (n_fill, shape.head_dim), 1.0)
                    V[li, r, j, :n_fill] = normal_bf16(seed, "vcache.%d.%d.%d" % (l, r, j),
                                                       (n_fill, shape.head_dim), 1.0)
    return K, V
