"""Benchmark: greedy decode of the Qwen3-8B-shaped model at batch 1 on one
MI355X through the persistent kernel.

Workload: 36 layers (hidden 4096, 32 q / 8 kv heads of 128, FFN 12288) and a
tied 151936-row embedding / LM head, seeded N(0, 0.02) bf16 weights, a
39-token seeded prompt and greedy decoding (the pages' Figure 1 workload:
39-token prompt, 512 generated tokens).  A step is one decode iteration:
every layer, the LM head, the argmax and the step/tokens advance for the one
request.  The warm-up steps ingest the prompt (untimed); the timed steps are
the generating ones (defaults: 38 warm-up, 512 timed, in launches of 64
iterations).

Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ms/token decode latency at batch 1 (Qwen3-8B shape) + % of HBM roofline"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, GB/s
# HBM bytes per 64-iteration launch of the persistent kernel from rocprofv3
# FETCH_SIZE + WRITE_SIZE, each scaled by a plain 1 GiB copy's readings
# (profiles/mpk_persistent_qwen3_8b_b1_hbm_counters.md).  Reported only while
# the code the counters were taken on is unchanged: the digest covers the
# device code, its tables and the graph builder, comments and layout
# stripped.
TRAFFIC = {"gb_per_launch": 977.3, "iters_per_launch": 64, "code_digest": "657feaa963ac04b5"}
CODE_FILES = ("runtime.hip", "mpk_internal.h", "builder.cpp")


def code_digest() -> str:
    """sha256 (16 hex digits) of the C/HIP sources in CODE_FILES with
    comments removed and whitespace collapsed (string literals are kept
    as they are; none of these files has a comment marker inside one)."""
    import hashlib
    import re

    h = hashlib.sha256()
    for name in CODE_FILES:
        src = open(os.path.join(ROOT, "persistent_task_runtime_amd", "csrc", name)).read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(name.encode() + b"\0" + " ".join(src.split()).encode() + b"\0")
    return h.hexdigest()[:16]


def measured_traffic(iters_per_launch: int):
    try:
        dig = code_digest()
    except OSError:
        return None
    if dig != TRAFFIC["code_digest"] or iters_per_launch != TRAFFIC["iters_per_launch"]:
        return None
    return TRAFFIC["gb_per_launch"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kv_bytes_per_position(sh) -> int:
    """bf16 K and V of one position over all layers."""
    return sh.layers * sh.n_kv * sh.head_dim * 2 * 2


def iteration_bytes(sh, p: int) -> int:
    """Algorithmic HBM bytes of one decode iteration at position p (batch 1):
    every weight byte once (the embedding is a one-row gather, the tied LM head
    is streamed whole), the K/V rows of positions < p read, the K/V row of p
    written, the embedding row read."""
    return sh.streamed_weight_bytes() + kv_bytes_per_position(sh) * (p + 1) + 2 * sh.hidden


def copy_calibration(n_bytes: int = 1 << 30) -> None:
    """A plain device copy of n_bytes (torch's copy kernel): run under
    rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE it gives the counters' bytes for a
    known amount of traffic, the factor that scales the megakernel's counters."""
    import torch

    src = torch.empty(n_bytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("copied %d bytes 3 times" % n_bytes)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512, help="timed decode iterations")
    ap.add_argument("--warmup", type=int, default=38,
                    help="untimed iterations before the timed ones (the prompt)")
    ap.add_argument("--launch-iters", type=int, default=64,
                    help="iterations per persistent launch in the timed region")
    ap.add_argument("--per-op-steps", type=int, default=64)
    ap.add_argument("--cpu-iters", type=int, default=6)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-op", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration for profiles)")
    ap.add_argument("--workload", choices=("qwen3_8b", "long"), default="qwen3_8b",
                    help="long: the same model with each layer's K/V cache pre-filled N(0,1) to "
                         "32768 positions, 128 decode iterations from there (attention-heavy)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import persistent_task_runtime_amd as mpk
    from persistent_task_runtime_amd import runner

    assert torch.cuda.is_available(), "no GPU visible"
    if args.workload == "long":
        return bench_long(args)
    sh = synth.QWEN3_8B
    P = 39
    K, W, L = args.steps, args.warmup, args.launch_iters
    if K % L:
        sys.exit("--steps must be a multiple of --launch-iters")
    total = W + K
    width = max(P + 512 + 1, total + 2)
    w = synth.Workload("qwen3_8b", sh, 1, n_iter=total, tokens_width=width,
                       prompt_len=np.array([P], np.int32), step0=np.zeros(1, np.int32))
    t0 = time.time()
    weights = synth.make_model(sh, seed=0)
    log("weights generated in %.1f s" % (time.time() - t0))
    model = runner.DeviceModel(sh, weights=weights)
    torch.cuda.synchronize()
    log("uploaded %.2f GB in %.1f s" % (model.bytes() / 1e9, time.time() - t0))
    if args.copy_calibration:
        copy_calibration()

    stream = torch.cuda.current_stream()
    sess = runner.Session(w, model, max_seq=width)
    if W:
        # the prompt goes through the one-launch-per-operator path: the same
        # task bodies, bitwise the same state, and no persistent launch of
        # another length in the profile of the timed one
        sess.run(W, per_op=True)
        torch.cuda.synchronize()
        sess.check_status()
    n_launch = K // L
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_launch)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        sess.run(L)
        b.record(stream)
    torch.cuda.synchronize()
    sess.check_status()
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    ms = ev[0][0].elapsed_time(ev[-1][1])
    ms_tok = ms / K
    step_now = int(sess.step.cpu()[0])
    assert step_now == total, (step_now, total)
    toks = sess.tokens.cpu().numpy()[0]
    assert (toks[: total + 1] >= 0).all()
    alg_bytes = sum(iteration_bytes(sh, W + i) for i in range(K))
    # roofline of the dominant kernel: algorithmic bytes per launch / mean launch duration
    launch_avg = sum(launch_ms) / n_launch
    achieved = (alg_bytes / n_launch) / (launch_avg / 1e3) / 1e9
    bound_ms = alg_bytes / K / (HBM_PEAK_GBS * 1e9) * 1e3
    log("persistent: %.4f ms/token over %d launches of %d iterations (mean launch %.3f ms), "
        "%.1f GB/s algorithmic (%.1f%% of %.0f GB/s)"
        % (ms_tok, n_launch, L, launch_avg, achieved, 100 * achieved / HBM_PEAK_GBS, HBM_PEAK_GBS))
    sess.close()

    per_op = None
    if not args.no_per_op:
        Kp = min(args.per_op_steps, K)
        s2 = runner.Session(w, model, max_seq=width)
        s2.run(W, per_op=True)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        s2.run(Kp, per_op=True)
        e1.record(stream)
        torch.cuda.synchronize()
        s2.check_status()
        per_op = e0.elapsed_time(e1) / Kp
        log("one launch per operator: %.4f ms/token over %d steps" % (per_op, Kp))
        s2.close()

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        n_cpu = args.cpu_iters
        om = oracle.Model(sh, weights)
        st = oracle.State(sh, synth.make_tokens(w), w.step0, w.prompt_len, n_cpu + 1)
        t1 = time.time()
        oracle.decode(om, st, n_cpu, want_logits=False)
        dt = time.time() - t1
        cores = int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))
        cpu = {"value": dt / n_cpu * 1e3, "unit": "ms/token", "cores": cores, "kind": "oracle",
               "sample": "%d greedy decode iterations (positions 0-%d) of the same model and prompt, "
                         "fp64 C oracle, OpenMP over output rows" % (n_cpu, n_cpu - 1)}
        log("cpu oracle: %.1f ms/token on %d threads" % (cpu["value"], cores))

    out = {
        "metric": METRIC,
        "value": round(ms_tok, 5),
        "unit": "ms/token",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_tok, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "qwen3_8b_batch1_prompt39_greedy", "layers": sh.layers,
                   "hidden": sh.hidden, "q_heads": sh.n_q, "kv_heads": sh.n_kv, "head_dim": sh.head_dim,
                   "ffn": sh.ffn, "vocab": sh.vocab, "tied_lm_head": True, "batch": 1,
                   "prompt_tokens": P, "generated_tokens": K, "iterations_per_launch": L,
                   "weights": "bf16 N(0,0.02) seeded", "kv_cache": "bf16"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(L)},
        "kernel": "mpk_persistent<1>",
        "traffic_unit": "GB per launch",
        "launch_ms": round(launch_avg, 4),
        "bound_ms_per_token": round(bound_ms, 5),
        "frac_of_bound": round(bound_ms / ms_tok, 4),
        "per_op_ms_per_token": round(per_op, 5) if per_op else None,
        "speedup_vs_per_op": round(per_op / ms_tok, 3) if per_op else None,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_long(args):
    """The long-context configuration: 128 iterations from position 32768
    over a K/V cache pre-filled N(0,1) (no prompt, no per-operator leg)."""
    import numpy as np
    import torch

    import synth
    from persistent_task_runtime_amd import runner

    sh = synth.QWEN3_8B
    K = 128
    L = (K - 2) // 2  # two timed launches after two warm-up iterations
    w = synth.workload("qwen3_8b_long", n_iter=K)
    p0 = int(w.step0[0])
    t0 = time.time()
    weights = synth.make_model(sh, seed=w.seed)
    model = runner.DeviceModel(sh, weights=weights)
    sess = runner.Session(w, model)  # generates and uploads the K/V prefill
    torch.cuda.synchronize()
    log("weights and K/V prefill ready in %.1f s" % (time.time() - t0))
    stream = torch.cuda.current_stream()
    sess.run(2)  # warm-up: the first two iterations (not timed)
    torch.cuda.synchronize()
    sess.check_status()
    n_launch = (K - 2) // L
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_launch)]
    for a, b in ev:
        a.record(stream)
        sess.run(L)
        b.record(stream)
    torch.cuda.synchronize()
    sess.check_status()
    n_timed = n_launch * L
    ms = ev[0][0].elapsed_time(ev[-1][1])
    ms_tok = ms / n_timed
    launch_avg = sum(a.elapsed_time(b) for a, b in ev) / n_launch
    alg_bytes = sum(iteration_bytes(sh, p0 + 2 + i) for i in range(n_timed))
    achieved = (alg_bytes / n_launch) / (launch_avg / 1e3) / 1e9
    bound_ms = alg_bytes / n_timed / (HBM_PEAK_GBS * 1e9) * 1e3
    log("long context: %.4f ms/token over %d launches of %d iterations from position %d, "
        "%.1f GB/s algorithmic (%.1f%% of %.0f GB/s)"
        % (ms_tok, n_launch, L, p0 + 2, achieved, 100 * achieved / HBM_PEAK_GBS, HBM_PEAK_GBS))
    sess.close()
    out = {
        "metric": METRIC, "value": round(ms_tok, 5), "unit": "ms/token", "n_gpus": 1, "steps": n_timed,
        "warmup": 2, "ms_per_step": round(ms_tok, 5), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "qwen3_8b_batch1_kv32768_greedy", "layers": sh.layers, "hidden": sh.hidden,
                   "q_heads": sh.n_q, "kv_heads": sh.n_kv, "head_dim": sh.head_dim, "ffn": sh.ffn,
                   "vocab": sh.vocab, "tied_lm_head": True, "batch": 1, "kv_prefill": p0,
                   "iterations_per_launch": L, "weights": "bf16 N(0,0.02) seeded",
                   "kv_cache": "bf16, N(0,1) pre-filled"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
        "kernel": "mpk_persistent<1>", "launch_ms": round(launch_avg, 4),
        "bound_ms_per_token": round(bound_ms, 5), "frac_of_bound": round(bound_ms / ms_tok, 4),
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
