"""GPU parity at widths without packed words (hidden 640, FFN 1920), batch 1
and 2, against the CPU oracle through the C ABI; the bar and the oracle
protocol are those of test_parity_gpu.py, whose helpers this file uses.

Collected after the other parity files on purpose: in one of five full runs
of the GPU suite the batch-2 case had logits 0.089 off the oracle at one
(iteration, request), cause not found.  Run late, a recurrence is reported
without hiding, under ``pytest -x``, every test collected after it.
"""
import numpy as np
import pytest

import synth
from test_parity_gpu import check_against_oracle, torch_dev  # noqa: F401 (fixture)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("batch", [1, 2])
def test_widths_without_packed_words_match_oracle(torch_dev, batch):
    """Widths that are not multiples of 256 (hidden 640, FFN 1920, 10 q / 5 kv
    heads): no operator input gets packed words, so every linear task gathers
    the 64-bit stamped words (global->LDS DMA where they fit, the register
    path otherwise).  Prompt plus generated tokens against the oracle, at
    batch 1 and 2."""
    from persistent_task_runtime_amd import runner

    sh = synth.ModelShape(layers=2, hidden=640, n_q=10, n_kv=5, head_dim=64, ffn=1920, vocab=1024)
    P = np.array([12, 9][:batch], np.int32)
    n = 24
    w = synth.Workload("w640_b%d" % batch, sh, batch, n, n + 4, P, np.zeros(batch, np.int32), gains="random")
    weights = synth.make_model(sh, seed=w.seed, gains=w.gains)
    model = runner.DeviceModel(sh, weights=weights)
    res = runner.run_workload(w, n, want_logits=True, model=model)
    check_against_oracle(w, n, weights, res, min_checked=8 * batch, min_written=4 * batch)
    res["session"].close()
