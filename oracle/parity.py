"""CPU ORACLE (test infrastructure only): teacher-forced comparison of a GPU
decode against the oracle.

Only ``tests/`` and ``__graft_entry__.smoke()`` use this module.

Protocol (the readings of the parity contract for the decode path):

* The oracle runs teacher-forced on the GPU's own token sequence: the GPU's
  final ``tokens`` row is handed to the oracle as a prompt that covers every
  position the run consumed, so at every iteration the oracle computes the
  logits of the same context the GPU saw, and one low-margin divergence
  cannot cascade into later iterations.
* At every iteration and request: logits max-abs error <= 5e-2; the token the
  GPU chose (the id it wrote into ``tokens`` once the prompt is consumed,
  the argmax of its logits while it is still ingesting the prompt) equals
  the oracle's argmax wherever the oracle's top-2 margin exceeds 0.1.
* After the run: ``step`` advanced by exactly the iteration count, the
  prompt's slots unchanged, the slots past the last written one untouched.

The decode iterations (P1 "How MPK Works": the runtime advances ``step``
after each decoding iteration and ``tokens[num_requests, seq_length]`` holds
prompt and generated ids) are the oracle's ``decode``.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Optional

import numpy as np

from . import Model, State, decode

LOGIT_TOL = 5e-2
MARGIN = 0.1


@dataclass
class ParityReport:
    compared: int        # (iteration, request) pairs whose logits were compared
    checked: int         # of those, margin-checked token decisions
    checked_written: int  # margin-checked decisions on ids the GPU wrote into tokens
    worst: float         # max-abs logit error over everything compared

    def __str__(self):
        return ("compared %d iterations, %d margin-checked (%d on written tokens), worst logit err %.3g"
                % (self.compared, self.checked, self.checked_written, self.worst))


def teacher_forced(model: Model, shape, gpu_tokens: np.ndarray, step0: np.ndarray, n_iter: int,
                   max_seq: int, kcache=None, vcache=None, chunk: int = 0,
                   progress: Optional[Callable[[str], None]] = None):
    """Oracle logits, argmax and top-2 margin [n_iter, B(, V)] on the GPU's token
    sequence: every consumed position holds the GPU's id, and every position
    is treated as prompt so the oracle writes no id of its own.  ``chunk``
    > 0 decodes in chunks of that many iterations (progress lines between)."""
    toks = np.ascontiguousarray(gpu_tokens, dtype=np.int32).copy()
    B = toks.shape[0]
    plen = np.full(B, toks.shape[1], np.int32)  # everything is prompt: never overwritten
    st = State(shape, toks, step0, plen, max_seq, kcache, vcache)
    if chunk <= 0:
        return decode(model, st, n_iter)
    parts = []
    done = 0
    while done < n_iter:
        n = min(chunk, n_iter - done)
        parts.append(decode(model, st, n))
        done += n
        if progress:
            progress("oracle: %d / %d iterations" % (done, n_iter))
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(3))


def compare(prompt_tokens: np.ndarray, prompt_len: np.ndarray, step0: np.ndarray, n_iter: int,
            g_logits: np.ndarray, g_tokens: np.ndarray, g_step: np.ndarray,
            o_logits: np.ndarray, o_am: np.ndarray, o_mg: np.ndarray,
            tol: float = LOGIT_TOL, margin: float = MARGIN) -> ParityReport:
    """Checks the protocol above; raises AssertionError naming the first
    failing (request, iteration).  prompt_tokens is the tokens tensor the run
    started from ([B, width], prompt ids and -1 elsewhere)."""
    B = g_tokens.shape[0]
    compared = checked = written = 0
    worst = 0.0
    for r in range(B):
        P = int(prompt_len[r])
        for s in range(n_iter):
            p = int(step0[r]) + s
            err = float(np.max(np.abs(g_logits[s, r].astype(np.float64) - o_logits[s, r])))
            worst = max(worst, err)
            assert err <= tol, "request %d iteration %d (position %d): logits max-abs error %g" % (r, s, p, err)
            compared += 1
            generating = p + 1 >= P
            g_tok = int(g_tokens[r, p + 1]) if generating else int(np.argmax(g_logits[s, r]))
            if o_mg[s, r] > margin:
                checked += 1
                written += int(generating)
                assert g_tok == int(o_am[s, r]), (
                    "request %d iteration %d (position %d): token %d vs oracle %d (oracle margin %g)"
                    % (r, s, p, g_tok, o_am[s, r], o_mg[s, r]))
        assert int(g_step[r]) == int(step0[r]) + n_iter, "request %d: step %d, expected %d" % (
            r, int(g_step[r]), int(step0[r]) + n_iter)
        assert np.array_equal(g_tokens[r, :P], prompt_tokens[r, :P]), "request %d: prompt slots changed" % r
        last = int(step0[r]) + n_iter  # the last slot an iteration may write
        assert np.array_equal(g_tokens[r, last + 1:], prompt_tokens[r, last + 1:]), (
            "request %d: slots past position %d were written" % (r, last))
    return ParityReport(compared, checked, written, worst)
