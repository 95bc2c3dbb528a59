"""Device-side setup for a synthetic workload: weights, KV caches and meta
tensors in HBM, a compiled graph, and runs of the persistent kernel.

Marshalling only (torch allocates device memory and copies inputs in); the
decode itself runs in libmpk.so.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

import synth
import persistent_task_runtime_amd as mpk


def _dev():
    import torch

    if not torch.cuda.is_available():
        raise RuntimeError("persistent_task_runtime_amd needs a ROCm GPU (none visible)")
    return torch.device("cuda:0")


def upload_bf16(arr: np.ndarray):
    import torch

    assert arr.dtype == np.uint16
    return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(_dev())


class DeviceModel:
    """Weights of a Qwen3-style decoder in HBM (bf16 stored as int16 tensors).

    Weights come either from a dict of bf16 bit arrays (``weights``) or are
    generated tensor by tensor from the seeded generator and uploaded, so the
    full-size model never needs a complete host copy."""

    def __init__(self, shape, seed: int = 0, gains: str = "ones",
                 weights: Optional[Dict[str, np.ndarray]] = None, layers=None,
                 with_embedding: bool = True):
        import torch

        self.shape = shape
        self.t: Dict[str, "torch.Tensor"] = {}
        self.layer_ids = list(range(shape.layers)) if layers is None else list(layers)
        if weights is not None:
            for k, v in weights.items():
                self.t[k] = upload_bf16(v)
            return
        if with_embedding:
            for k, v in synth.make_model(shape, seed, gains, layers=[], with_embedding=True).items():
                self.t[k] = upload_bf16(v)
        for l in self.layer_ids:
            for k, v in synth.make_model(shape, seed, gains, layers=[l], with_embedding=False).items():
                self.t[k] = upload_bf16(v)
            torch.cuda.synchronize()

    def ptrs(self) -> Dict[str, int]:
        return {k: v.data_ptr() for k, v in self.t.items()}

    def bytes(self) -> int:
        return sum(v.numel() * v.element_size() for v in self.t.values())


class Session:
    """KV caches, meta tensors and a compiled executable for one workload."""

    def __init__(self, w: "synth.Workload", model: DeviceModel, logits_iters: int = 0,
                 trace: bool = False, max_seq: Optional[int] = None, kv=None,
                 spin_timeout_ns: int = 0, x_in=None, launch=None):
        import torch

        dev = _dev()
        self.w = w
        sh = w.shape
        self.max_seq = max_seq or w.max_seq
        B = w.batch
        self.tokens = torch.from_numpy(synth.make_tokens(w)).to(dev)
        self.step = torch.from_numpy(w.step0.astype(np.int32)).to(dev)
        self.prompt_len = torch.from_numpy(w.prompt_len.astype(np.int32)).to(dev)
        self.kc, self.vc = {}, {}
        for li, l in enumerate(model.layer_ids):
            if kv is not None:
                K, V = kv
                self.kc[l] = upload_bf16(K[li])
                self.vc[l] = upload_bf16(V[li])
            elif w.kv_prefill:
                K, V = synth.make_kv_prefill(sh, B, self.max_seq, w.kv_prefill, seed=w.seed, layers=[l])
                self.kc[l] = upload_bf16(K[0])
                self.vc[l] = upload_bf16(V[0])
            else:
                self.kc[l] = torch.zeros((B, sh.n_kv, self.max_seq, sh.head_dim), dtype=torch.int16, device=dev)
                self.vc[l] = torch.zeros_like(self.kc[l])
        ptrs = model.ptrs()
        for l in model.layer_ids:
            ptrs["l%d.kcache" % l] = self.kc[l].data_ptr()
            ptrs["l%d.vcache" % l] = self.vc[l].data_ptr()
        ptrs.update(tokens=self.tokens.data_ptr(), step=self.step.data_ptr(),
                    prompt_len=self.prompt_len.data_ptr())
        self.logits = None
        with_lm = "E" in model.t
        if logits_iters and with_lm:
            self.logits = torch.zeros((logits_iters, B, sh.vocab), dtype=torch.float32, device=dev)
            ptrs["logits"] = self.logits.data_ptr()
        self.x_in = x_in
        self.x_out = None
        if not with_lm:
            self.x_out = torch.zeros((B, sh.hidden), dtype=torch.float32, device=dev)
        spec, meta = mpk.qwen3_graph(sh, B, ptrs, self.tokens.shape[1], self.max_seq,
                                     layers=model.layer_ids, with_embedding=with_lm,
                                     with_lm_head=with_lm, logits_iters=logits_iters if with_lm else 0,
                                     x_in_ptr=x_in.data_ptr() if x_in is not None else 0,
                                     x_out_ptr=self.x_out.data_ptr() if self.x_out is not None else 0)
        num_cus = torch.cuda.get_device_properties(dev).multi_processor_count
        mcfg = mpk.model_cfg(sh, B, self.max_seq)
        lcfg = launch if launch is not None else mpk.launch_cfg(num_cus, trace=trace,
                                                                  spin_timeout_ns=spin_timeout_ns)
        self.model = model
        self.exe = mpk.Executable(spec, meta, mcfg, lcfg)

    def run(self, n_iter: int, per_op: bool = False, stream=None, static: bool = False):
        import torch

        s = torch.cuda.current_stream() if stream is None else stream
        if per_op:
            self.exe.run_per_op(n_iter, s.cuda_stream)
        elif static:
            mpk.mpk_run_steps_static(self.exe.exe, n_iter, s.cuda_stream)
        else:
            self.exe.run(n_iter, s.cuda_stream)

    def replace_request(self, r: int, prompt) -> None:
        """Slot r takes a new request between runs (the request that held it
        leaves): its tokens row becomes the new prompt (-1 past it), its step
        0 and its prompt length len(prompt).  The other slots go on where
        they were.  The slot's K/V cache is not cleared: the new request
        reads a position only after it has written it.  Ordered with the runs
        on the current stream."""
        import torch

        prompt = np.asarray(prompt, dtype=np.int32)
        W = self.tokens.shape[1]
        if not 1 <= prompt.size < W:
            raise ValueError("prompt of %d ids does not fit a tokens row of %d" % (prompt.size, W))
        row = np.full(W, -1, np.int32)
        row[:prompt.size] = prompt
        dev = self.tokens.device
        self.tokens[r].copy_(torch.from_numpy(row).to(dev))
        self.step[r:r + 1].fill_(0)
        self.prompt_len[r:r + 1].fill_(int(prompt.size))

    def check_status(self):
        code, it, task = self.exe.status()
        if code != 0:
            raise mpk.MPKError(code, "device status at iteration %d task %d" % (it, task))

    def close(self):
        self.exe.close()


class RequestView:
    """Request r of a batched Session as a batch-1 executable over views of
    the session's own tensors (its tokens row, step and prompt_len entries,
    and its slice of every layer's K/V cache, contiguous in the
    [B, n_kv, S, d] layout): runs of it advance that request in place, e.g.
    to ingest its prompt before batched decoding."""

    def __init__(self, sess: "Session", r: int):
        import torch

        sh, m = sess.w.shape, sess.model
        ptrs = m.ptrs()
        for l in m.layer_ids:
            ptrs["l%d.kcache" % l] = sess.kc[l][r].data_ptr()
            ptrs["l%d.vcache" % l] = sess.vc[l][r].data_ptr()
        ptrs.update(tokens=sess.tokens[r].data_ptr(), step=sess.step[r:r + 1].data_ptr(),
                    prompt_len=sess.prompt_len[r:r + 1].data_ptr())
        spec, meta = mpk.qwen3_graph(sh, 1, ptrs, sess.tokens.shape[1], sess.max_seq, layers=m.layer_ids)
        num_cus = torch.cuda.get_device_properties(_dev()).multi_processor_count
        self.exe = mpk.Executable(spec, meta, mpk.model_cfg(sh, 1, sess.max_seq), mpk.launch_cfg(num_cus))

    def run(self, n_iter: int, stream=None):
        import torch

        s = torch.cuda.current_stream() if stream is None else stream
        self.exe.run(n_iter, s.cuda_stream)

    def close(self):
        self.exe.close()


class PromptChunks:
    """Batched prompt ingestion for request r of a Session: every iteration
    takes `rows` consecutive prompt positions of the request as `rows` rows
    (mpk_meta rows_per_request), over views of the session's own tensors
    (its tokens row, step and prompt_len entries, its K/V caches), so a run
    advances the request in place by `rows` positions per iteration.  With
    logits_iters > 0 the logits of every row are kept ([iteration, row, V]:
    row i of iteration s is position step + rows s + i)."""

    def __init__(self, sess: "Session", r: int, rows: int = 8, logits_iters: int = 0):
        import torch

        sh, m = sess.w.shape, sess.model
        self.sess, self.r, self.rows = sess, r, rows
        ptrs = m.ptrs()
        for l in m.layer_ids:
            ptrs["l%d.kcache" % l] = sess.kc[l][r].data_ptr()
            ptrs["l%d.vcache" % l] = sess.vc[l][r].data_ptr()
        ptrs.update(tokens=sess.tokens[r].data_ptr(), step=sess.step[r:r + 1].data_ptr(),
                    prompt_len=sess.prompt_len[r:r + 1].data_ptr())
        self.logits = None
        if logits_iters:
            self.logits = torch.zeros((logits_iters, rows, sh.vocab), dtype=torch.float32, device=_dev())
            ptrs["logits"] = self.logits.data_ptr()
        spec, meta = mpk.qwen3_graph(sh, rows, ptrs, sess.tokens.shape[1], sess.max_seq, layers=m.layer_ids,
                                     logits_iters=logits_iters, rows_per_request=rows)
        num_cus = torch.cuda.get_device_properties(_dev()).multi_processor_count
        self.exe = mpk.Executable(spec, meta, mpk.model_cfg(sh, rows, sess.max_seq), mpk.launch_cfg(num_cus))

    def chunks_left(self) -> int:
        """Whole chunks that fit before the prompt's last position (batched
        ingestion generates no token: the last prompt position is decoded)."""
        step = int(self.sess.step[self.r].item())
        plen = int(self.sess.prompt_len[self.r].item())
        return max(0, (plen - 1 - step) // self.rows)

    def run(self, n_iter: int, stream=None):
        import torch

        s = torch.cuda.current_stream() if stream is None else stream
        self.exe.run(n_iter, s.cuda_stream)

    def check_status(self):
        """Raises MPKError if the last chunk run stopped on the device (after
        the stream has been synchronised)."""
        code, it, task = self.exe.status()
        if code != 0:
            raise mpk.MPKError(code, "chunk run: device status at iteration %d task %d" % (it, task))

    def close(self):
        self.exe.close()


def run_workload(w: "synth.Workload", n_iter: int, want_logits: bool = False, per_op: bool = False,
                 trace: bool = False, model: Optional[DeviceModel] = None, launch=None) -> dict:
    import torch

    model = model or DeviceModel(w.shape, w.seed, w.gains)
    sess = Session(w, model, logits_iters=n_iter if want_logits else 0, trace=trace, launch=launch)
    sess.run(n_iter, per_op=per_op)
    torch.cuda.synchronize()
    sess.check_status()
    out = {"tokens": sess.tokens.cpu().numpy(), "step": sess.step.cpu().numpy()}
    if want_logits:
        lg = sess.logits.cpu().numpy()
        out["logits"] = lg
        out["argmax"] = lg.argmax(axis=-1).astype(np.int32)
    out["session"] = sess
    return out
