"""Python binding of the MI355X persistent decode megakernel (libmpk.so).

Argument marshalling only: the functions below have the names of the C ABI in
``include/mpk.h`` and forward to it through ctypes.  ``qwen3_graph`` lays out
the tensor table and operator list of a Qwen3-style decoder (the demo model
the pages name) from device pointers; every step of the decode runs in the
library's kernels.

Sources: the pages on Mirage Persistent Kernel ("MPK") describe the Python
surface this mirrors: a PersistentKernel configured with worker and
scheduler counts, step and tokens meta tensors, attached or library-allocated
tensors, fused operators such as rmsnorm_linear_layer, then compile() and a
call to run (page "Mirage Persistent Kernel: Fusing Multi-GPU LLM Inference
into One Kernel Launch", sections "How MPK Works", "Getting Started" and
"The API").
"""
from __future__ import annotations

import atexit
import ctypes
import os
import sys
import weakref
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmpk.so")

# ---- status codes and enums (mpk.h) -------------------------------------------
MPK_OK = 0
MPK_ERR_INVALID_ARG = -1
MPK_ERR_SHAPE = -2
MPK_ERR_DTYPE = -3
MPK_ERR_ALIGN = -4
MPK_ERR_SPLIT = -5
MPK_ERR_NOT_CORESIDENT = -6
MPK_ERR_HIP = -7
MPK_ERR_DEVICE_TIMEOUT = -8
MPK_ERR_ABORTED = -9
MPK_ERR_STATE = -10
MPK_ERR_GRAPH = -11

MPK_BF16, MPK_F32, MPK_I32 = 1, 2, 3
MPK_SCHED_CORESIDENT, MPK_SCHED_DEDICATED = 0, 1
MPK_OP_EMBED = 1
MPK_OP_RMSNORM_LINEAR = 2
MPK_OP_ATTENTION = 3
MPK_OP_LINEAR_RESIDUAL = 4
MPK_OP_RMSNORM_GATEUP = 5
MPK_OP_LMHEAD_ARGMAX = 6

c_i32, c_i64, c_u32, c_u64, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p


class mpk_model_cfg(ctypes.Structure):
    _fields_ = [("num_layers", c_i32), ("hidden", c_i32), ("n_q_heads", c_i32),
                ("n_kv_heads", c_i32), ("head_dim", c_i32), ("ffn", c_i32), ("vocab", c_i32),
                ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("max_batch", c_i32), ("max_seq", c_i32)]


class mpk_launch_cfg(ctypes.Structure):
    _fields_ = [("num_cus", c_i32), ("num_workers", c_i32), ("num_schedulers", c_i32),
                ("sched_mode", c_i32), ("trace", c_i32), ("reserved", c_i32),
                ("spin_timeout_ns", c_u64)]


class mpk_tensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("dtype", c_i32), ("ndim", c_i32),
                ("dims", c_i64 * 4), ("dev_ptr", c_vp)]


class mpk_op(ctypes.Structure):
    _fields_ = [("kind", c_i32), ("layer", c_i32), ("in_", c_i32 * 5), ("out", c_i32 * 1),
                ("num_tiles", c_i32)]


class mpk_meta(ctypes.Structure):
    _fields_ = [("tokens", c_i32), ("step", c_i32), ("prompt_len", c_i32), ("num_requests", c_i32),
                ("rows_per_request", c_i32)]


class mpk_trace_record(ctypes.Structure):
    _fields_ = [("task", c_i32), ("iteration", c_i32), ("start_ticket", c_u32),
                ("end_ticket", c_u32), ("t_start", c_u64), ("t_end", c_u64),
                ("hw_id", c_u32), ("xcc_id", c_u32), ("t_ready", c_u64)]


class mpk_task_info(ctypes.Structure):
    _fields_ = [("op", c_i32), ("tile", c_i32), ("worker", c_i32), ("row0", c_i32),
                ("nrows", c_i32), ("split", c_i32), ("dep_event", c_i32 * 3),
                ("dep_count", c_i32 * 3), ("dep_prev", c_i32 * 3), ("out_event", c_i32)]


class mpk_graph_info(ctypes.Structure):
    _fields_ = [("num_tasks", c_i32), ("num_events", c_i32), ("num_workers", c_i32),
                ("max_queue", c_i32), ("num_ops", c_i32), ("sink_op", c_i32), ("num_queues", c_i32),
                ("tasks", ctypes.POINTER(mpk_task_info)), ("event_count", ctypes.POINTER(c_i32)),
                ("event_op", ctypes.POINTER(c_i32)), ("queue_len", ctypes.POINTER(c_i32)),
                ("queues", ctypes.POINTER(c_i32))]


MPK_SIM_NO_FAULT, MPK_SIM_FAULT_KV_AFTER_PUBLISH, MPK_SIM_FAULT_SKIP_WAIT, MPK_SIM_FAULT_DROP_PUBLISH = 0, 1, 2, 3


class mpk_sim_cfg(ctypes.Structure):
    _fields_ = [("num_iterations", c_i32), ("iter_base", c_u32), ("seed", c_u32), ("jitter_us", c_i32),
                ("timeout_ms", c_i32), ("fault", c_i32)]


TRACE_DTYPE_FIELDS = [("task", "<i4"), ("iteration", "<i4"), ("start_ticket", "<u4"),
                      ("end_ticket", "<u4"), ("t_start", "<u8"), ("t_end", "<u8"),
                      ("hw_id", "<u4"), ("xcc_id", "<u4"), ("t_ready", "<u8")]


class MPKError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("mpk error %d: %s" % (code, msg))
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libmpk.so (built by ``persistent_task_runtime_amd.build``).  There is
    no fallback: without the library nothing runs."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        from . import build as _build
        _build.build(force=False)
    # Load order: torch ships its own HIP runtime, and a process holds one
    # runtime per soname (the first loaded) to which every HIP library binds.
    # torch, which provides the device memory and streams, is imported first,
    # so the library always runs on torch's runtime.  (Importing torch does
    # not initialise the GPU.)
    try:
        import torch  # noqa: F401
    except ImportError:  # then the system HIP runtime
        pass
    L = ctypes.CDLL(path)
    P = ctypes.POINTER
    sig = {
        "mpk_build_graph": (c_i32, [P(mpk_model_cfg), P(mpk_launch_cfg), P(mpk_tensor), c_i32,
                                    P(mpk_op), c_i32, P(mpk_meta), P(c_vp)]),
        "mpk_compile": (c_i32, [c_vp, c_i32, P(c_vp)]),
        "mpk_run_steps": (c_i32, [c_vp, c_i32, c_vp]),
        "mpk_run_steps_static": (c_i32, [c_vp, c_i32, c_vp]),
        "mpk_run_steps_per_op": (c_i32, [c_vp, c_i32, c_vp]),
        "mpk_get_status": (c_i32, [c_vp, P(c_i32), P(c_i32), P(c_i32)]),
        "mpk_set_abort": (c_i32, [c_vp, c_i32]),
        "mpk_read_trace": (c_i32, [c_vp, c_vp, ctypes.c_size_t, P(ctypes.c_size_t)]),
        "mpk_get_graph_info": (c_i32, [c_vp, P(mpk_graph_info)]),
        "mpk_sim_create": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_i32, P(c_vp)]),
        "mpk_simulate": (c_i32, [c_vp, P(mpk_sim_cfg), c_vp]),
        "mpk_sim_read_meta": (c_i32, [c_vp, c_vp, c_vp]),
        "mpk_sim_destroy": (None, [c_vp]),
        "mpk_check_run": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_i32]),
        "mpk_get_tensor_ptr": (c_i32, [c_vp, c_i32, P(c_vp)]),
        "mpk_destroy_exec": (None, [c_vp]),
        "mpk_destroy_graph": (None, [c_vp]),
        "mpk_stream_read": (c_i32, [c_vp, ctypes.c_uint64, c_i32, c_vp, c_vp]),
        "mpk_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


EXPORTED = ["mpk_build_graph", "mpk_compile", "mpk_run_steps", "mpk_run_steps_static", "mpk_run_steps_per_op",
            "mpk_get_status", "mpk_set_abort", "mpk_read_trace", "mpk_get_graph_info",
            "mpk_sim_create", "mpk_simulate", "mpk_sim_read_meta", "mpk_sim_destroy",
            "mpk_check_run", "mpk_get_tensor_ptr", "mpk_destroy_exec", "mpk_destroy_graph",
            "mpk_stream_read", "mpk_last_error"]


def mpk_last_error() -> str:
    return load_library().mpk_last_error().decode(errors="replace")


def _check(rc: int):
    if rc != MPK_OK:
        raise MPKError(rc, mpk_last_error())


# ---- thin wrappers with the C names ------------------------------------------------

def mpk_build_graph(model: mpk_model_cfg, launch: mpk_launch_cfg, tensors: Sequence[mpk_tensor],
                    ops: Sequence[mpk_op], meta: mpk_meta) -> int:
    T = (mpk_tensor * len(tensors))(*tensors)
    O = (mpk_op * len(ops))(*ops)
    out = c_vp()
    _check(load_library().mpk_build_graph(ctypes.byref(model), ctypes.byref(launch), T, len(tensors),
                                          O, len(ops), ctypes.byref(meta), ctypes.byref(out)))
    return out.value


def mpk_compile(graph: int, device: int = 0) -> int:
    out = c_vp()
    _check(load_library().mpk_compile(graph, device, ctypes.byref(out)))
    return out.value


def mpk_run_steps(exe: int, num_iterations: int, stream: int = 0) -> None:
    _check(load_library().mpk_run_steps(exe, num_iterations, stream))


def mpk_run_steps_static(exe: int, num_iterations: int, stream: int = 0) -> None:
    _check(load_library().mpk_run_steps_static(exe, num_iterations, stream))


def mpk_run_steps_per_op(exe: int, num_iterations: int, stream: int = 0) -> None:
    _check(load_library().mpk_run_steps_per_op(exe, num_iterations, stream))


def mpk_get_status(exe: int) -> Tuple[int, int, int]:
    c, i, t = c_i32(), c_i32(), c_i32()
    _check(load_library().mpk_get_status(exe, ctypes.byref(c), ctypes.byref(i), ctypes.byref(t)))
    return c.value, i.value, t.value


def mpk_set_abort(exe: int, flag: int) -> None:
    _check(load_library().mpk_set_abort(exe, flag))


def mpk_read_trace(exe: int, n_records: int):
    import numpy as np
    buf = np.empty(n_records, dtype=np.dtype(TRACE_DTYPE_FIELDS))
    written = ctypes.c_size_t()
    _check(load_library().mpk_read_trace(exe, buf.ctypes.data, buf.nbytes, ctypes.byref(written)))
    return buf[: written.value // buf.dtype.itemsize]


def mpk_get_graph_info(graph: int) -> mpk_graph_info:
    info = mpk_graph_info()
    _check(load_library().mpk_get_graph_info(graph, ctypes.byref(info)))
    return info


def mpk_sim_create(graph: int, step, tokens, prompt_len, kv_filled: int = 0) -> int:
    import numpy as np
    a = [np.ascontiguousarray(v, dtype=np.int32) for v in (step, tokens, prompt_len)]
    out = c_vp()
    _check(load_library().mpk_sim_create(graph, a[0].ctypes.data, a[1].ctypes.data, a[2].ctypes.data,
                                         kv_filled, ctypes.byref(out)))
    return out.value


def mpk_simulate(sim: int, num_tasks: int, num_iterations: int, iter_base: int, seed: int = 0,
                 jitter_us: int = 0, timeout_ms: int = 5000, fault: int = MPK_SIM_NO_FAULT):
    """One simulated launch; returns the trace records [num_iterations * num_tasks]."""
    import numpy as np
    cfg = mpk_sim_cfg(num_iterations, iter_base, seed, jitter_us, timeout_ms, fault)
    buf = np.empty(num_iterations * num_tasks, dtype=np.dtype(TRACE_DTYPE_FIELDS))
    _check(load_library().mpk_simulate(sim, ctypes.byref(cfg), buf.ctypes.data))
    return buf


def mpk_sim_read_meta(sim: int, batch: int, width: int):
    import numpy as np
    step = np.empty(batch, np.int32)
    toks = np.empty((batch, width), np.int32)
    _check(load_library().mpk_sim_read_meta(sim, step.ctypes.data, toks.ctypes.data))
    return step, toks


def mpk_sim_destroy(sim: int) -> None:
    if sim:
        load_library().mpk_sim_destroy(sim)


def mpk_check_run(graph: int, step, tokens, prompt_len, num_iterations: int) -> None:
    import numpy as np
    a = [np.ascontiguousarray(v, dtype=np.int32) for v in (step, tokens, prompt_len)]
    _check(load_library().mpk_check_run(graph, a[0].ctypes.data, a[1].ctypes.data, a[2].ctypes.data,
                                        num_iterations))


def mpk_get_tensor_ptr(exe: int, tensor_id: int) -> int:
    p = c_vp()
    _check(load_library().mpk_get_tensor_ptr(exe, tensor_id, ctypes.byref(p)))
    return p.value or 0


def mpk_stream_read(src_ptr: int, nbytes: int, workgroups: int, sink_ptr: int, stream: int) -> None:
    _check(load_library().mpk_stream_read(src_ptr, nbytes, workgroups, sink_ptr, stream))


def mpk_destroy_exec(exe: int) -> None:
    if exe:
        load_library().mpk_destroy_exec(exe)


def mpk_destroy_graph(graph: int) -> None:
    if graph:
        load_library().mpk_destroy_graph(graph)


# ---- graph layout for a Qwen3-style decoder (marshalling only) ---------------------

@dataclass
class TensorRef:
    """A tensor-table entry: dtype, dims and a device address (0 = library-owned)."""
    name: str
    dtype: int
    dims: Tuple[int, ...]
    ptr: int = 0


class GraphSpec:
    """Tensor table + operator list under construction."""

    def __init__(self):
        self.tensors: List[TensorRef] = []
        self.index: Dict[str, int] = {}
        self.ops: List[mpk_op] = []

    def tensor(self, name: str, dtype: int, dims, ptr: int = 0) -> int:
        if name in self.index:
            raise ValueError("duplicate tensor " + name)
        self.index[name] = len(self.tensors)
        self.tensors.append(TensorRef(name, dtype, tuple(int(d) for d in dims), int(ptr)))
        return self.index[name]

    def op(self, kind: int, layer: int, ins: Sequence[int], out: int, num_tiles: int = 0):
        o = mpk_op()
        o.kind, o.layer, o.num_tiles = kind, layer, num_tiles
        ins = list(ins) + [-1] * (5 - len(ins))
        for i, v in enumerate(ins):
            o.in_[i] = v
        o.out[0] = out
        self.ops.append(o)

    def c_tensors(self) -> List[mpk_tensor]:
        out = []
        self._names = []
        for t in self.tensors:
            ct = mpk_tensor()
            nm = t.name.encode()
            self._names.append(nm)
            ct.name = nm
            ct.dtype, ct.ndim = t.dtype, len(t.dims)
            for i in range(4):
                ct.dims[i] = t.dims[i] if i < len(t.dims) else 1
            ct.dev_ptr = t.ptr or None
            out.append(ct)
        return out


def model_cfg(shape, max_batch: int, max_seq: int) -> mpk_model_cfg:
    m = mpk_model_cfg()
    m.num_layers, m.hidden, m.n_q_heads, m.n_kv_heads = shape.layers, shape.hidden, shape.n_q, shape.n_kv
    m.head_dim, m.ffn, m.vocab = shape.head_dim, shape.ffn, shape.vocab
    m.rms_eps, m.rope_theta = shape.rms_eps, shape.rope_theta
    m.max_batch, m.max_seq = max_batch, max_seq
    return m


def launch_cfg(num_cus: int, trace: bool = False, spin_timeout_ns: int = 0,
               sched_mode: int = MPK_SCHED_CORESIDENT, num_workers: int = 0,
               num_schedulers: int = 0) -> mpk_launch_cfg:
    l = mpk_launch_cfg()
    l.num_cus, l.num_workers, l.num_schedulers = num_cus, num_workers, num_schedulers
    l.sched_mode, l.trace, l.spin_timeout_ns = sched_mode, int(trace), spin_timeout_ns
    return l


_LAYER_KEYS = ("attn_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "ffn_norm", "wg", "wu", "wd")


def qwen3_graph(shape, batch: int, ptrs: Dict[str, int], tokens_width: int, max_seq: int,
                layers: Optional[Sequence[int]] = None, with_embedding: bool = True,
                with_lm_head: bool = True, logits_iters: int = 0, x_in_ptr: int = 0,
                x_out_ptr: int = 0, rows_per_request: int = 1) -> Tuple[GraphSpec, mpk_meta]:
    """Tensor table and operator list of a Qwen3-style decoder, in layer order.

    ``batch`` is the rows B of an iteration: B / rows_per_request requests,
    each taking rows_per_request consecutive positions per iteration (> 1:
    batched prompt ingestion, see mpk_meta).  ``ptrs`` maps weight names
    (``E``, ``final_norm``, ``l{i}.wq`` ...), the KV caches (``l{i}.kcache`` /
    ``l{i}.vcache``, each [requests, n_kv, max_seq, d] bf16), ``tokens``,
    ``step``, ``prompt_len`` (per request) and optionally ``logits`` to
    device addresses.  Without the embedding the first layer reads the f32
    tensor at ``x_in_ptr`` ([B, hidden]); without the LM head the last layer
    writes ``x_out_ptr`` when given.  Activations between operators are
    library-owned."""
    g = GraphSpec()
    H, d, F = shape.hidden, shape.head_dim, shape.ffn
    B = batch
    if rows_per_request < 1 or B % rows_per_request:
        raise ValueError("rows_per_request must divide the rows per iteration")
    NR = B // rows_per_request
    layer_ids = list(range(shape.layers)) if layers is None else list(layers)
    tok = g.tensor("tokens", MPK_I32, (NR, tokens_width), ptrs["tokens"])
    stp = g.tensor("step", MPK_I32, (NR,), ptrs["step"])
    pl = g.tensor("prompt_len", MPK_I32, (NR,), ptrs["prompt_len"])
    meta = mpk_meta()
    meta.tokens, meta.step, meta.prompt_len, meta.num_requests = tok, stp, pl, NR
    meta.rows_per_request = rows_per_request
    if with_embedding:
        E = g.tensor("E", MPK_BF16, (shape.vocab, H), ptrs["E"])
        x = g.tensor("x0", MPK_F32, (B, H))
        g.op(MPK_OP_EMBED, -1, [E], x)
    else:
        x = g.tensor("x_in", MPK_F32, (B, H), x_in_ptr)
    qkv_w = (shape.n_q + 2 * shape.n_kv) * d
    for li, l in enumerate(layer_ids):
        w = {k: g.tensor("l%d.%s" % (l, k), MPK_BF16, dims, ptrs["l%d.%s" % (l, k)])
             for k, dims in (("attn_norm", (H,)), ("wq", (shape.q_rows, H)), ("wk", (shape.kv_rows, H)),
                             ("wv", (shape.kv_rows, H)), ("q_norm", (d,)), ("k_norm", (d,)),
                             ("wo", (H, shape.q_rows)), ("ffn_norm", (H,)), ("wg", (F, H)),
                             ("wu", (F, H)), ("wd", (H, F)))}
        kc = g.tensor("l%d.kcache" % l, MPK_BF16, (NR, shape.n_kv, max_seq, d), ptrs["l%d.kcache" % l])
        vc = g.tensor("l%d.vcache" % l, MPK_BF16, (NR, shape.n_kv, max_seq, d), ptrs["l%d.vcache" % l])
        qkv = g.tensor("l%d.qkv" % l, MPK_F32, (B, qkv_w))
        o = g.tensor("l%d.o" % l, MPK_F32, (B, shape.q_rows))
        h1 = g.tensor("l%d.h_attn" % l, MPK_F32, (B, H))
        m = g.tensor("l%d.m" % l, MPK_F32, (B, F))
        last = li == len(layer_ids) - 1
        h2 = g.tensor("l%d.h_out" % l, MPK_F32, (B, H),
                      x_out_ptr if (last and not with_lm_head) else 0)
        g.op(MPK_OP_RMSNORM_LINEAR, l, [x, w["attn_norm"], w["wq"], w["wk"], w["wv"]], qkv)
        g.op(MPK_OP_ATTENTION, l, [qkv, w["q_norm"], w["k_norm"], kc, vc], o)
        g.op(MPK_OP_LINEAR_RESIDUAL, l, [o, w["wo"], x], h1)
        g.op(MPK_OP_RMSNORM_GATEUP, l, [h1, w["ffn_norm"], w["wg"], w["wu"]], m)
        g.op(MPK_OP_LINEAR_RESIDUAL, l, [m, w["wd"], h1], h2)
        x = h2
    if with_lm_head:
        fn = g.tensor("final_norm", MPK_BF16, (H,), ptrs["final_norm"])
        E_id = g.index["E"] if "E" in g.index else g.tensor("E", MPK_BF16, (shape.vocab, H), ptrs["E"])
        lg = -1
        if logits_iters:
            lg = g.tensor("logits", MPK_F32, (logits_iters, B, shape.vocab), ptrs["logits"])
        g.op(MPK_OP_LMHEAD_ARGMAX, -1, [x, fn, E_id], lg)
    return g, meta


# Executables still open when the interpreter exits are closed by an atexit
# hook, which runs while the HIP runtime (and any profiler attached to it) is
# still intact; a finaliser running later, during interpreter teardown, makes
# no HIP call.
_live = weakref.WeakSet()


@atexit.register
def _close_live_executables():
    for e in list(_live):
        e.close()


class Executable:
    """Owns a built graph and its compiled executable."""

    def __init__(self, spec: GraphSpec, meta: mpk_meta, model: mpk_model_cfg,
                 launch: mpk_launch_cfg, device: int = 0):
        self.spec = spec
        self.exe = 0
        self.graph = mpk_build_graph(model, launch, spec.c_tensors(), spec.ops, meta)
        try:
            self.exe = mpk_compile(self.graph, device)
        except Exception:
            mpk_destroy_graph(self.graph)
            self.graph = 0
            raise
        _live.add(self)

    def tensor_ptr(self, name: str) -> int:
        return mpk_get_tensor_ptr(self.exe, self.spec.index[name])

    def run(self, n_iter: int, stream: int = 0):
        mpk_run_steps(self.exe, n_iter, stream)

    def run_per_op(self, n_iter: int, stream: int = 0):
        mpk_run_steps_per_op(self.exe, n_iter, stream)

    def status(self):
        return mpk_get_status(self.exe)

    def close(self):
        mpk_destroy_exec(getattr(self, "exe", 0))
        mpk_destroy_graph(getattr(self, "graph", 0))
        self.exe = self.graph = 0
        _live.discard(self)

    def __del__(self, _finalizing=sys.is_finalizing):
        # (bound at definition: module globals may already be cleared when
        # an executable is collected during interpreter shutdown)
        if _finalizing():
            return
        try:
            self.close()
        except Exception:
            pass
