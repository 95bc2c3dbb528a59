"""bench.py's launch planning under a short command line
(``bench.py --gpus 1 --steps 20 --warmup 5``): any --steps is accepted, the
timed region is the configured 512-token generation split into persistent
launches (the last one takes the remainder), and the prompt is ingested
before it whatever --warmup says."""
import pytest

import bench


def test_plan_covers_every_iteration_with_a_remainder_launch():
    assert bench.plan_launches(512, 64) == [64] * 8
    assert bench.plan_launches(20, 64) == [20]
    assert bench.plan_launches(130, 64) == [64, 64, 2]
    for n in (1, 7, 63, 64, 65, 511, 512, 1000):
        for L in (1, 5, 64, 100):
            p = bench.plan_launches(n, L)
            assert sum(p) == n and all(0 < x <= L for x in p) and all(x == L for x in p[:-1])
    with pytest.raises(ValueError):
        bench.plan_launches(0, 64)


def test_short_command_times_the_configured_generation():
    # --steps 20 still times all 512 generated tokens
    assert bench.timed_tokens(20) == 512
    assert bench.timed_tokens(512) == 512
    assert bench.timed_tokens(600) == 600
    assert bench.plan_launches(bench.timed_tokens(20), 64) == [64] * 8


def test_short_argv_parses_and_plans():
    a = bench.parse_args(["--gpus", "1", "--steps", "20", "--warmup", "5"])
    assert (a.gpus, a.steps, a.warmup, a.workload) == (1, 20, 5, "qwen3_8b")
    K = bench.timed_tokens(a.steps)
    launches = bench.plan_launches(K, a.launch_iters)
    assert sum(launches) == 512 and launches == [64] * 8
    # the committed traffic figure applies to 64-iteration launches
    assert launches[0] == bench.TRAFFIC["iters_per_launch"]


def test_every_configuration_has_a_workload():
    """The five configurations: tiny decoder, one layer, the full model at
    batch 1 (default), batch 8 and long context."""
    for wl in ("tiny", "one_layer", "qwen3_8b", "b8", "long"):
        assert bench.parse_args(["--workload", wl]).workload == wl


def test_one_layer_bytes_per_step():
    import synth

    sh = synth.ModelShape(1, 4096, 32, 8, 128, 12288, 151936)
    # 385.9 MB of weights; K/V: 8 kv heads x 128 dims x bf16 x (K, V) per position
    assert sh.layer_weight_bytes() == 2 * (4096 * 6144 + 4096 * 4096 + 3 * 12288 * 4096) + 2 * (2 * 4096 + 2 * 128)
    assert bench.layer_bytes(sh, 512) - sh.layer_weight_bytes() == 513 * 8 * 128 * 4
