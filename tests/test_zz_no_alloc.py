"""mpk_run_steps_static: the allocation-free run (its scratch in the
library's static device array, shared by every call on the GPU) gives the
same tokens, step, logits and K/V caches, bit for bit, as mpk_run_steps on
the same graph and inputs; twice in a row, the second call on a smaller
graph (over what the first left in the array).  Oversized and traced graphs
are refused before anything is launched."""
import numpy as np
import pytest

import synth
import persistent_task_runtime_amd as mpk

pytestmark = pytest.mark.gpu


def _run_pair(model, w, n):
    import torch
    from persistent_task_runtime_amd import runner

    out = []
    for static in (False, True):
        s = runner.Session(w, model, logits_iters=n)
        s.run(n, static=static)
        torch.cuda.synchronize()
        s.check_status()
        out.append({"tokens": s.tokens.cpu().numpy(), "step": s.step.cpu().numpy(),
                    "logits": s.logits.cpu().numpy(),
                    "kv": [np.concatenate([s.kc[l].cpu().numpy().ravel(), s.vc[l].cpu().numpy().ravel()])
                           for l in model.layer_ids]})
        s.close()
    a, b = out
    assert np.array_equal(a["tokens"], b["tokens"]) and np.array_equal(a["step"], b["step"])
    assert np.array_equal(a["logits"].view(np.uint32), b["logits"].view(np.uint32))
    for x, y in zip(a["kv"], b["kv"]):
        assert np.array_equal(x, y)
    assert int(b["step"][0]) == int(w.step0[0]) + n
    return b


def test_static_run_equals_run_steps_twice_second_smaller(rocm_device):
    from persistent_task_runtime_amd import runner

    w = synth.workload("tiny")
    print("allocation-free run: tiny, 2 layers, 48 iterations", flush=True)
    m2 = runner.DeviceModel(w.shape, weights=synth.make_model(w.shape, seed=0))
    _run_pair(m2, w, 48)
    print("allocation-free run: tiny, 1 layer, 20 iterations", flush=True)
    m1 = runner.DeviceModel(w.shape, weights=synth.make_model(w.shape, seed=1, layers=[0]), layers=[0])
    _run_pair(m1, w, 20)


def test_static_run_refuses_oversized_and_traced_graphs(rocm_device):
    import torch
    from persistent_task_runtime_amd import runner

    from test_builder import FakePtrs

    # an 80-layer 8B-wide graph at 4096 positions: its run scratch (stamped
    # words and split partials of every layer) is beyond 64 MiB.  Attached
    # pointers are placeholders: nothing is launched.
    sh = synth.ModelShape(80, 4096, 32, 8, 128, 12288, 151936)
    spec, meta = mpk.qwen3_graph(sh, 1, FakePtrs(), 4100, 4096)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    exe = mpk.Executable(spec, meta, mpk.model_cfg(sh, 1, 4096), mpk.launch_cfg(cus))
    with pytest.raises(mpk.MPKError) as e:
        mpk.mpk_run_steps_static(exe.exe, 1, 0)
    assert e.value.code == mpk.MPK_ERR_SHAPE and "static array" in str(e.value)
    exe.close()
    # a traced graph would need its trace buffer allocated
    w = synth.workload("tiny")
    model = runner.DeviceModel(w.shape, weights=synth.make_model(w.shape, seed=0))
    s = runner.Session(w, model, trace=True)
    with pytest.raises(mpk.MPKError) as e:
        s.run(4, static=True)
    assert e.value.code == mpk.MPK_ERR_INVALID_ARG
    s.close()
