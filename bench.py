"""Benchmark: greedy decode of the Qwen3-8B-shaped model at batch 1 on one
MI355X through the persistent kernel.

Workload: 36 layers (hidden 4096, 32 q / 8 kv heads of 128, FFN 12288) and a
tied 151936-row embedding / LM head, seeded N(0, 0.02) bf16 weights, a
39-token seeded prompt and greedy decoding (the pages' Figure 1 workload:
39-token prompt, 512 generated tokens).  A step is one decode iteration:
every layer, the LM head, the argmax and the step/tokens advance for the one
request.

Order of a run: --warmup persistent iterations on the same executable
(untimed; step, tokens and the prompt are then restored), the 38 prompt
iterations through the one-launch-per-operator path (untimed, whatever
--warmup says: the prompt is input, not the measured work), then the timed
generating iterations as persistent launches of --launch-iters iterations
(the last launch takes the remainder).  The timed region covers the whole
configured generation: max(--steps, 512) tokens, so a short --steps
(say 20) still measures the 512-token workload; "steps" in the output is the
number of iterations actually timed.

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
# HBM bytes per 64-iteration launch of the persistent kernel (mean over the
# eight launches of the benchmark, as roofline.achieved) from rocprofv3
# FETCH_SIZE + WRITE_SIZE, each scaled by a plain 1 GiB copy's readings
# (profiles/mpk_persistent_qwen3_8b_b1_hbm_counters.md).  Reported only while
# the code the counters were taken on is unchanged: the digest covers the
# device code, its tables and the graph builder, comments and layout
# stripped.
TRAFFIC = {"gb_per_launch": 977.93, "iters_per_launch": 64, "code_digest": "f9aeeb7ca1c414d2"}
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


GENERATED_TOKENS = 512  # the configured workload: 512 greedy tokens after a 39-token prompt
PROMPT_TOKENS = 39


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def log_native_maps():
    """Address ranges of the repository's native libraries and the HIP / HSA
    runtimes in this process (stderr), to attribute any frame of a crash
    report printed after the program's last line."""
    spans = {}
    try:
        for line in open("/proc/self/maps"):
            f = line.split()
            if len(f) < 6:
                continue
            path = f[5]
            if path.startswith(ROOT) or any(k in path for k in ("libamdhip64", "libhsa-runtime64", "libgomp")):
                lo, hi = (int(x, 16) for x in f[0].split("-"))
                a, b = spans.get(path, (lo, hi))
                spans[path] = (min(a, lo), max(b, hi))
    except OSError:
        return
    for path, (lo, hi) in sorted(spans.items(), key=lambda kv: kv[1]):
        log("native map %#x-%#x %s" % (lo, hi, path))


def plan_launches(n_iter: int, per_launch: int):
    """Lengths of the persistent launches that cover n_iter iterations: as many
    launches of per_launch as fit, then one with the remainder."""
    if n_iter <= 0 or per_launch <= 0:
        raise ValueError("iterations and iterations per launch must be positive")
    full, rest = divmod(n_iter, per_launch)
    return [per_launch] * full + ([rest] if rest else [])


def timed_tokens(steps: int) -> int:
    """Generated tokens in the timed region: the whole configured generation,
    or more when --steps asks for more."""
    return max(steps, GENERATED_TOKENS)


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


def stream_ceiling(n_bytes: int = 4 << 30, workgroups=(256, 512, 768, 1024, 2048), reps: int = 5):
    """Measured HBM read ceiling: mpk_stream_read (16-byte nontemporal loads,
    the weight streams' load form) over a buffer much larger than the
    256 MB last-level cache, timed with HIP events on the stream it runs
    on; the best launch shape's median rate in GB/s."""
    import torch

    import persistent_task_runtime_amd as mpk

    buf = torch.zeros(n_bytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    best = None
    for wg in workgroups:
        rates = []
        for i in range(reps + 2):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            mpk.mpk_stream_read(buf.data_ptr(), n_bytes, wg, sink.data_ptr(), stream.cuda_stream)
            b.record(stream)
            b.synchronize()
            if i >= 2:
                rates.append(n_bytes / (a.elapsed_time(b) / 1e3) / 1e9)
        med = sorted(rates)[len(rates) // 2]
        log("stream read: %d workgroups, %.1f GB/s (median of %d)" % (wg, med, reps))
        if best is None or med > best[0]:
            best = (med, wg)
    del buf, sink
    torch.cuda.synchronize()
    return {"gbs": round(best[0], 1), "workgroups": best[1], "bytes": n_bytes,
            "probe": "mpk_stream_read: one read of a 4 GiB buffer, 16-byte nontemporal loads"}


def with_ceiling(roofline: dict, ceiling) -> dict:
    """The roofline object plus the measured read ceiling and the achieved
    rate's fraction of it."""
    if ceiling:
        roofline["ceiling_gbs"] = ceiling["gbs"]
        roofline["frac_of_ceiling"] = round(roofline["achieved"] / ceiling["gbs"], 4)
        roofline["ceiling_probe"] = ceiling["probe"]
    return roofline


def parse_args(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=GENERATED_TOKENS,
                    help="timed generated tokens (at least the configured 512 are timed)")
    ap.add_argument("--warmup", type=int, default=5,
                    help="untimed persistent iterations before the prompt is ingested")
    ap.add_argument("--launch-iters", type=int, default=64,
                    help="iterations per persistent launch in the timed region (last launch: remainder)")
    ap.add_argument("--per-op-steps", type=int, default=64)
    ap.add_argument("--cpu-iters", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-op", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the HBM read-ceiling probe")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prompt-ingestion comparison (one position per iteration vs chunks of 8)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration for profiles)")
    ap.add_argument("--workload", choices=("qwen3_8b", "long", "b8", "tiny", "one_layer"), default="qwen3_8b",
                    help="long: the same model with each layer's K/V cache pre-filled N(0,1) to "
                         "32768 positions, 128 decode iterations from there (attention-heavy); "
                         "b8: batch 8, prompt lengths uniform in [16, 512] ingested per request, "
                         "then 256 lockstep greedy iterations (MFMA linear tasks)")
    return ap.parse_args(argv)


def bench_prefill(sess, n_prompt, restart, stream, rows=8):
    """Prompt ingestion (positions 0 .. P-2, untimed in the decode figure):
    one position per persistent iteration, against chunks of `rows`
    positions per iteration (rows_per_request: the batch-8 kernels) followed
    by the remaining positions one at a time.  Each is warmed up once, then
    timed with HIP events around its launches."""
    import torch
    from persistent_task_runtime_amd import runner

    pc = runner.PromptChunks(sess, 0, rows)
    restart()
    nch = pc.chunks_left()
    rest = n_prompt - rows * nch

    def one_by_one():
        sess.run(n_prompt)

    def chunked():
        pc.run(nch)
        if rest:
            sess.run(rest)

    out = {}
    for name, fn in (("one_per_iteration", one_by_one), ("chunked", chunked)):
        restart()
        fn()
        torch.cuda.synchronize()
        restart()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        sess.check_status()
        code = pc.exe.status()[0]
        assert code == 0, "prompt chunks: device status %d" % code
        assert int(sess.step.cpu()[0]) == n_prompt
        out[name] = a.elapsed_time(b)
    pc.close()
    res = {"positions": n_prompt, "rows_per_iteration": rows, "chunk_iterations": nch,
           "decode_iterations": rest, "ms_chunked": round(out["chunked"], 3),
           "ms_one_per_iteration": round(out["one_per_iteration"], 3),
           "speedup": round(out["one_per_iteration"] / out["chunked"], 3)}
    log("prompt ingestion (%d positions): %.3f ms one per iteration, %.3f ms in %d chunks of %d + %d "
        "iterations (%.2fx)" % (n_prompt, out["one_per_iteration"], out["chunked"], nch, rows, rest,
                                res["speedup"]))
    return res


def main():
    args = parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import persistent_task_runtime_amd as mpk
    from persistent_task_runtime_amd import runner

    # The native libraries are opened before the GPU runtime initialises, so
    # they map above the address range it reserves, like every other HIP
    # library of the process; their exit-time destructors (a HIP library's
    # unregisters its device code) then run in the usual order.
    mpk.load_library()
    synth._load()
    assert torch.cuda.is_available(), "no GPU visible"
    if args.workload == "long":
        return bench_long(args)
    if args.workload == "tiny":
        return bench_tiny(args)
    if args.workload == "one_layer":
        return bench_one_layer(args)
    if args.workload == "b8":
        return bench_b8(args)
    sh = synth.QWEN3_8B
    P = PROMPT_TOKENS
    K, W = timed_tokens(args.steps), args.warmup
    launches = plan_launches(K, args.launch_iters)
    # iterations at positions 0 .. P-2 consume prompt ids and write nothing;
    # the iteration at P-1 consumes the last prompt id and yields the first
    # generated token, so the timed iterations are positions P-1 .. P-2+K
    n_prompt = P - 1
    total = n_prompt + K
    width = max(total + 2, W + 2)
    if K != args.steps:
        log("timing the configured %d generated tokens (--steps %d asks for fewer)" % (K, args.steps))
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
    toks0 = sess.tokens.clone()

    def restart():
        """step, tokens back to the prompt (the K/V rows are rewritten as the
        positions are consumed again)"""
        sess.step.zero_()
        sess.tokens.copy_(toks0)

    def ingest_prompt():
        # the prompt goes through the one-launch-per-operator path: the same
        # task bodies, bitwise the same state, and no persistent launch of
        # another length in the profile of the timed ones
        sess.run(n_prompt, per_op=True)
        torch.cuda.synchronize()
        sess.check_status()

    if W:
        sess.run(W)
        torch.cuda.synchronize()
        sess.check_status()
        restart()
        log("warm-up: %d persistent iterations" % W)
    ingest_prompt()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in launches]
    torch.cuda.synchronize()
    for (a, b), L in zip(ev, launches):
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
    assert (toks[: total + 1] >= 0).all() and (toks[: total + 1] < sh.vocab).all()
    # roofline of the dominant kernel: algorithmic bytes per launch / mean
    # launch duration (HIP events on the launch stream)
    pos = n_prompt
    launch_bytes = []
    for L in launches:
        launch_bytes.append(sum(iteration_bytes(sh, pos + i) for i in range(L)))
        pos += L
    alg_bytes = sum(launch_bytes)
    achieved = sum(b / (t / 1e3) for b, t in zip(launch_bytes, launch_ms)) / len(launches) / 1e9
    launch_avg = sum(launch_ms) / len(launches)
    bound_ms = alg_bytes / K / (HBM_PEAK_GBS * 1e9) * 1e3
    log("persistent: %.4f ms/token over %d launches %s (mean launch %.3f ms), "
        "%.1f GB/s algorithmic (%.1f%% of %.0f GB/s)"
        % (ms_tok, len(launches), launches, launch_avg, achieved, 100 * achieved / HBM_PEAK_GBS, HBM_PEAK_GBS))

    per_op = None
    if not args.no_per_op:
        Kp = min(args.per_op_steps, K)
        restart()
        ingest_prompt()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        sess.run(Kp, per_op=True)
        e1.record(stream)
        torch.cuda.synchronize()
        sess.check_status()
        per_op = e0.elapsed_time(e1) / Kp
        log("one launch per operator: %.4f ms/token over %d steps" % (per_op, Kp))
    prefill = None
    if not args.no_prefill:
        prefill = bench_prefill(sess, n_prompt, restart, stream)
    sess.close()
    del sess, model
    torch.cuda.synchronize()
    ceiling = None if args.no_ceiling else stream_ceiling()

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
                   "prompt_tokens": P, "generated_tokens": K, "iterations_per_launch": launches[0],
                   "launches": len(launches),
                   "weights": "bf16 N(0,0.02) seeded", "kv_cache": "bf16"},
        "roofline": with_ceiling({"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                                  "traffic": measured_traffic(launches[0]) if len(set(launches)) == 1 else None},
                                 ceiling),
        "kernel": "mpk_persistent<1>",
        "traffic_unit": "GB per launch",
        "launch_ms": round(launch_avg, 4),
        "bound_ms_per_token": round(bound_ms, 5),
        "frac_of_bound": round(bound_ms / ms_tok, 4),
        "per_op_ms_per_token": round(per_op, 5) if per_op else None,
        "speedup_vs_per_op": round(per_op / ms_tok, 3) if per_op else None,
        "prompt_ingestion": prefill,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    log_native_maps()


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
    del sess
    torch.cuda.synchronize()
    ceiling = None if args.no_ceiling else stream_ceiling()
    out = {
        "metric": METRIC, "value": round(ms_tok, 5), "unit": "ms/token", "n_gpus": 1, "steps": n_timed,
        "warmup": 2, "ms_per_step": round(ms_tok, 5), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "qwen3_8b_batch1_kv32768_greedy", "layers": sh.layers, "hidden": sh.hidden,
                   "q_heads": sh.n_q, "kv_heads": sh.n_kv, "head_dim": sh.head_dim, "ffn": sh.ffn,
                   "vocab": sh.vocab, "tied_lm_head": True, "batch": 1, "kv_prefill": p0,
                   "iterations_per_launch": L, "weights": "bf16 N(0,0.02) seeded",
                   "kv_cache": "bf16, N(0,1) pre-filled"},
        "roofline": with_ceiling({"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
                                 ceiling),
        "kernel": "mpk_persistent<1>", "launch_ms": round(launch_avg, 4),
        "bound_ms_per_token": round(bound_ms, 5), "frac_of_bound": round(bound_ms / ms_tok, 4),
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def bench_b8(args):
    """Batch 8: 8 requests with seeded prompt lengths uniform in [16, 512]
    (tokens [8, 4096]); each prompt is ingested at batch 1 into the batch-8
    session's own tensors (untimed), then the 8 requests decode in lockstep,
    each at its own position, 256 greedy iterations timed in launches of
    --launch-iters.  A step is one batch-8 iteration (a token for each of the
    8 requests)."""
    import numpy as np
    import torch

    import synth
    from persistent_task_runtime_amd import runner

    sh = synth.QWEN3_8B
    K = 256
    w = synth.workload("qwen3_8b_b8")
    P = w.prompt_len.astype(np.int64)
    launches = plan_launches(K, args.launch_iters)
    t0 = time.time()
    weights = synth.make_model(sh, seed=w.seed)
    model = runner.DeviceModel(sh, weights=weights)
    sess = runner.Session(w, model)
    torch.cuda.synchronize()
    log("weights and batch-8 session ready in %.1f s" % (time.time() - t0))
    # prompts: request r alone (batch 1) over positions 0 .. P_r - 2, in the
    # batch-8 tensors; then step[r] = P_r - 1 (the first batched iteration
    # consumes the last prompt id)
    t1 = time.time()
    sess.step.zero_()
    for r in range(w.batch):
        view = runner.RequestView(sess, r)
        view.run(int(P[r]) - 1)
        torch.cuda.synchronize()
        code, it, task = view.exe.status()
        assert code == 0, (r, code, it, task)
        view.close()
    step0 = sess.step.cpu().numpy()
    assert np.array_equal(step0, P - 1), (step0, P - 1)
    toks0 = sess.tokens.clone()
    log("prompts (%d ids) ingested at batch 1 in %.1f s" % (int(P.sum()), time.time() - t1))
    stream = torch.cuda.current_stream()
    if args.warmup:
        sess.run(args.warmup)
        torch.cuda.synchronize()
        sess.check_status()
        sess.step.copy_(torch.from_numpy(step0.astype(np.int32)).to(sess.step.device))
        sess.tokens.copy_(toks0)
        log("warm-up: %d batch-8 iterations" % args.warmup)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in launches]
    torch.cuda.synchronize()
    for (a, b), L in zip(ev, launches):
        a.record(stream)
        sess.run(L)
        b.record(stream)
    torch.cuda.synchronize()
    sess.check_status()
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    ms = ev[0][0].elapsed_time(ev[-1][1])
    ms_it = ms / K
    assert np.array_equal(sess.step.cpu().numpy(), step0 + K)
    toks = sess.tokens.cpu().numpy()
    for r in range(w.batch):
        gen = toks[r, int(P[r]):int(P[r]) + K]
        assert ((gen >= 0) & (gen < sh.vocab)).all()
    kvp = kv_bytes_per_position(sh)

    def it_bytes(s):
        return sh.streamed_weight_bytes() + sum(kvp * (int(step0[r]) + s + 1) + 2 * sh.hidden for r in range(8))

    pos = 0
    launch_bytes = []
    for L in launches:
        launch_bytes.append(sum(it_bytes(pos + i) for i in range(L)))
        pos += L
    alg = sum(launch_bytes)
    achieved = sum(b / (t / 1e3) for b, t in zip(launch_bytes, launch_ms)) / len(launches) / 1e9
    bound_ms = alg / K / (HBM_PEAK_GBS * 1e9) * 1e3
    tok_s = 8 * K / (ms / 1e3)
    log("batch 8: %.4f ms/iteration (%.1f tokens/s) over launches %s, %.1f GB/s algorithmic (%.1f%% of %.0f "
        "GB/s), bound %.4f ms/iteration" % (ms_it, tok_s, launches, achieved, 100 * achieved / HBM_PEAK_GBS,
                                            HBM_PEAK_GBS, bound_ms))
    sess.close()
    del sess, model
    torch.cuda.synchronize()
    ceiling = None if args.no_ceiling else stream_ceiling()
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        n_cpu = 2
        om = oracle.Model(sh, weights)
        wc = synth.Workload("b8_cpu", sh, 8, n_cpu, n_cpu + 2, np.full(8, n_cpu + 1, np.int32),
                            np.zeros(8, np.int32))
        st = oracle.State(sh, synth.make_tokens(wc), wc.step0, wc.prompt_len, n_cpu + 1)
        t2 = time.time()
        oracle.decode(om, st, n_cpu, want_logits=False)
        dt = time.time() - t2
        cores = int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))
        cpu = {"value": dt / n_cpu * 1e3, "unit": "ms/iteration", "cores": cores, "kind": "oracle",
               "sample": "%d batch-8 iterations (8 requests each, positions 0-%d) of the same model, fp64 C "
                         "oracle, OpenMP over output rows" % (n_cpu, n_cpu - 1)}
        log("cpu oracle: %.1f ms per batch-8 iteration on %d threads" % (cpu["value"], cores))
    out = {
        "metric": "ms/iteration decode latency at batch 8 (Qwen3-8B shape) + % of HBM roofline",
        "value": round(ms_it, 5), "unit": "ms/iteration", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_it, 5), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 MFMA (hi/lo inputs), f32 accumulate", "data": "synthetic",
        "config": {"workload": "qwen3_8b_batch8_prompts16to512_greedy", "layers": sh.layers, "hidden": sh.hidden,
                   "q_heads": sh.n_q, "kv_heads": sh.n_kv, "head_dim": sh.head_dim, "ffn": sh.ffn,
                   "vocab": sh.vocab, "tied_lm_head": True, "batch": 8,
                   "prompt_lengths": [int(x) for x in P], "generated_tokens_per_request": K,
                   "iterations_per_launch": launches[0], "weights": "bf16 N(0,0.02) seeded", "kv_cache": "bf16"},
        "tokens_per_s": round(tok_s, 1),
        "roofline": with_ceiling({"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
                                 ceiling),
        "kernel": "mpk_persistent<8>", "launch_ms": round(sum(launch_ms) / len(launches), 4),
        "bound_ms_per_iteration": round(bound_ms, 5), "frac_of_bound": round(bound_ms / ms_it, 4),
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)



def timed_runs(sess, n_iter: int, reps: int, restart, per_op: bool = False):
    """reps launches of n_iter iterations, each after restart() (stream-ordered
    copies, outside the events); durations in ms from HIP events on the launch
    stream."""
    import torch

    stream = torch.cuda.current_stream()
    out = []
    for _ in range(reps):
        restart()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        sess.run(n_iter, per_op=per_op)
        b.record(stream)
        b.synchronize()
        sess.check_status()
        out.append(a.elapsed_time(b))
    return out


def bench_tiny(args):
    """The tiny decoder (2 layers, hidden 256, 4 q / 2 kv heads of 64, FFN
    768, vocab 1024; 39-id prompt and 32 greedy tokens): its whole workload,
    70 decode iterations, as one persistent launch, repeated.  Its 3.7 MB of
    weights stay in the last-level cache, so this measures the runtime's
    latency per operator phase (12 phases per iteration: 2 layers x 5, the LM
    head and the argmax), not bandwidth."""
    import numpy as np

    import synth
    from persistent_task_runtime_amd import runner

    w = synth.workload("tiny")
    sh, n = w.shape, w.n_iter
    weights = synth.make_model(sh, seed=w.seed, gains=w.gains)
    model = runner.DeviceModel(sh, weights=weights)
    sess = runner.Session(w, model)
    toks0 = sess.tokens.clone()

    def restart():
        sess.step.zero_()
        sess.tokens.copy_(toks0)

    timed_runs(sess, n, 1, restart)  # warm-up
    reps = 9
    ms = sorted(timed_runs(sess, n, reps, restart))
    ms_it = ms[reps // 2] / n
    per_op = sorted(timed_runs(sess, n, 3, restart, per_op=True))[1] / n
    phases = sh.layers * 5 + 2
    alg = sum(iteration_bytes(sh, p) for p in range(n)) / n
    achieved = alg / (ms_it / 1e3) / 1e9
    log("tiny: %.4f ms/iteration (median of %d launches of %d), %.2f us per phase; one launch per operator "
        "%.4f ms/iteration" % (ms_it, reps, n, ms_it * 1e3 / phases, per_op))
    sess.close()
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        om = oracle.Model(sh, weights)
        st = oracle.State(sh, synth.make_tokens(w), w.step0, w.prompt_len, w.max_seq)
        t1 = time.time()
        oracle.decode(om, st, n, want_logits=False)
        dt = time.time() - t1
        cores = int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))
        cpu = {"value": dt / n * 1e3, "unit": "ms/iteration", "cores": cores, "kind": "oracle",
               "sample": "the whole 70-iteration workload, fp64 C oracle, OpenMP over output rows"}
    out = {
        "metric": "ms/iteration decode latency (tiny 2-layer decoder) + us per operator phase",
        "value": round(ms_it, 5), "unit": "ms/iteration", "n_gpus": 1, "steps": n * reps, "warmup": n,
        "ms_per_step": round(ms_it, 5), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "tiny_2layer_prompt39_greedy32", "layers": sh.layers, "hidden": sh.hidden,
                   "q_heads": sh.n_q, "kv_heads": sh.n_kv, "head_dim": sh.head_dim, "ffn": sh.ffn,
                   "vocab": sh.vocab, "tied_lm_head": True, "batch": 1, "iterations_per_launch": n,
                   "weights": "bf16 N(0,0.02) seeded", "kv_cache": "bf16"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 5), "traffic": None},
        "note": "latency-bound: the weights stay in the last-level cache; us_per_phase is the figure of merit",
        "phases_per_iteration": phases, "us_per_phase": round(ms_it * 1e3 / phases, 3),
        "per_op_ms_per_iteration": round(per_op, 5), "speedup_vs_per_op": round(per_op / ms_it, 3),
        "kernel": "mpk_persistent<1>", "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def layer_bytes(sh, p: int) -> int:
    """Algorithmic HBM bytes of one decoder layer's decode step at position p
    (batch 1): the layer's weights once, K/V rows 0 .. p - 1 read and row p
    written."""
    return sh.layer_weight_bytes() + sh.n_kv * sh.head_dim * 2 * 2 * (p + 1)


def bench_one_layer(args):
    """One Qwen3-8B-shaped decoder layer (hidden 4096, 32 q / 8 kv heads of
    128, FFN 12288, bf16 weights), K/V pre-filled N(0,1) to 512 positions,
    input h ~ N(0,1): the layer's decode step at positions 512 .. 575 as 64
    iterations of one persistent launch (each iteration attends to the
    positions before it and writes its own K/V row; the 385.9 MB of weights
    exceed the 256 MB last-level cache and are streamed with nontemporal
    loads, so every iteration reads them from HBM)."""
    import numpy as np
    import torch

    import synth
    from persistent_task_runtime_amd import runner

    sh = synth.ModelShape(1, 4096, 32, 8, 128, 12288, 151936)
    n, p0 = 64, 512
    w = synth.Workload("one_layer_bench", sh, 1, n, p0 + n + 2, np.array([p0 + 1], np.int32),
                       np.array([p0], np.int32), kv_prefill=p0)
    weights = synth.make_model(sh, seed=0, with_embedding=False)
    x = torch.from_numpy(synth.normal_f32(0, "one_layer_bench.h", (1, sh.hidden), 1.0)).to("cuda:0")
    K, V = synth.make_kv_prefill(sh, 1, w.max_seq, p0, seed=0)
    model = runner.DeviceModel(sh, weights=weights)
    sess = runner.Session(w, model, kv=(K, V), x_in=x)

    def restart():  # no argmax in the graph: step stays at 512, every launch covers 512 .. 575
        pass

    timed_runs(sess, n, 1, restart)  # warm-up
    reps = 5
    ms = sorted(timed_runs(sess, n, reps, restart))
    ms_med = ms[reps // 2]
    us_it = ms_med * 1e3 / n
    per_op = sorted(timed_runs(sess, n, 3, restart, per_op=True))[1] * 1e3 / n
    alg = sum(layer_bytes(sh, p0 + i) for i in range(n))
    achieved = alg / (ms_med / 1e3) / 1e9
    bound_us = alg / n / (HBM_PEAK_GBS * 1e9) * 1e6
    log("one layer: %.2f us/iteration (median of %d launches of %d), %.1f GB/s algorithmic (%.1f%% of %.0f "
        "GB/s), bound %.2f us; one launch per operator %.2f us" % (us_it, reps, n, achieved,
                                                               100 * achieved / HBM_PEAK_GBS, HBM_PEAK_GBS,
                                                               bound_us, per_op))
    sess.close()
    del sess, model
    torch.cuda.synchronize()
    ceiling = None if args.no_ceiling else stream_ceiling()
    out = {
        "metric": "us per decode step of one Qwen3-8B-shaped layer + % of HBM roofline",
        "value": round(us_it, 3), "unit": "us/iteration", "n_gpus": 1, "steps": n * reps, "warmup": n,
        "ms_per_step": round(us_it / 1e3, 6), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "qwen3_8b_one_layer_kv512", "hidden": sh.hidden, "q_heads": sh.n_q,
                   "kv_heads": sh.n_kv, "head_dim": sh.head_dim, "ffn": sh.ffn, "batch": 1,
                   "positions": [p0, p0 + n - 1], "iterations_per_launch": n,
                   "weights": "bf16 N(0,0.02) seeded", "kv_cache": "bf16, N(0,1) pre-filled to 512",
                   "input": "h ~ N(0,1)"},
        "roofline": with_ceiling({"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
                                 ceiling),
        "kernel": "mpk_persistent<1>", "bound_us_per_iteration": round(bound_us, 3),
        "frac_of_bound": round(bound_us / us_it, 4), "per_op_us_per_iteration": round(per_op, 3),
        "speedup_vs_per_op": round(per_op / us_it, 3), "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
