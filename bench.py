"""Decode-step benchmark: 32 stacked Ling-shaped MoE layers + the FP8 LM head, batch 1.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers 32] [--no-breakdown] [--no-cpu]

A step is one decode pass through the whole hot path: for each of the 32
layers the RMS norm of the residual stream, the router GEMV with top-8 of 512,
the MXFP4 routed (8) + shared SwiGLU experts and the bf16 residual add, then
the FP8 head (157,184 x 2,560) with the fused greedy argmax.  Inputs (51.5 GB
of MXFP4 experts, the quantized head and 2,000 seeded tokens) are resident in
HBM before timing; the timed steps are one captured HIP graph with one node
per step, each reading its own resident token and writing its own argmax
slot, so every timed step is read back and checked against an eager call
afterwards.

Prints one JSON line (rank 0) with the µs per step, the achieved HBM rate of
the step's algorithmic bytes, the roofline object of the dominant kernel (the
single-launch decode step), the standalone FP8 head kernel's rate, the 4-token
verify pass through all layers and the head, a per-component breakdown (one
MoE layer over 100 seeded cold inputs at 1 and 4 tokens, the FP8 and BF16
heads, the sampling epilogue at the GSM8K settings, the load-time quantizer,
the W4A8 layer at 1 and 4 tokens, the grouped layer at 16 tokens in bf16 and
W4A8), a pure-read bandwidth probe, and the CPU oracle on three of the timed
steps (every layer checked against the device, teacher-forced) with its time
per step at one BLAS thread and at all cores, plus its time per unit of the
smaller workloads.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--head-reps", type=int, default=200)
    ap.add_argument("--kernel-reps", type=int, default=200)
    ap.add_argument("--breakdown-reps", type=int, default=100,
                    help="samples per breakdown row (at most the workload's seeded inputs); small values serve "
                         "hardware-counter runs")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB device-to-device 3 times (a plain copy "
                         "kernel of known size, used to scale hardware byte counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    from weight_streaming_expert_amd import configs, inputs, ops

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = configs.DECODE_STEP
    m = wl.moe
    L = args.layers
    H, I, E, k, V = m.H, m.I, m.E, m.k, configs.LM_HEAD.V

    # ------------------------------------------------------------------ resident inputs
    t0 = time.time()
    shapes = dict(w13c=(L, E, 2 * I, H // 2), w13s=(L, E, 2 * I, H // 32), w2c=(L, E, H, I // 2), w2s=(L, E, H, I // 32))
    dw = {key: torch.empty(s, dtype=torch.uint8, device=dev) for key, s in shapes.items()}
    router = torch.empty((L, E, H), dtype=torch.bfloat16, device=dev)
    sh = [torch.empty((L,) + s[2:], dtype=torch.uint8, device=dev) for s in
          (shapes["w13c"], shapes["w13s"], shapes["w2c"], shapes["w2s"])]
    # one pinned host staging buffer per tensor, refilled for every layer (first-touch of
    # fresh host memory costs more than generating the bytes)
    stage_t = {key: torch.empty(s[1:], dtype=torch.uint8, pin_memory=True) for key, s in shapes.items()}
    stage = {key: t.numpy() for key, t in stage_t.items()}
    for l in range(L):
        lw = inputs.layer_weights(wl, l, out=stage)
        for key in shapes:
            dw[key][l].copy_(stage_t[key])
        router[l].copy_(torch.from_numpy(lw["router"].view(np.int16)).view(torch.bfloat16))
        for i in range(4):
            sh[i][l].copy_(torch.from_numpy(lw["shared"][i]))
        if l % 4 == 3:
            log(f"generated {l + 1}/{L} layers ({time.time() - t0:.0f} s)")
    del stage, stage_t
    stack = ops.MoeStackTensors(router, dw["w13c"], dw["w13s"], dw["w2c"], dw["w2s"], shared=tuple(sh), k=k)
    resident = sum(t.numel() * t.element_size() for t in list(dw.values()) + sh + [router])
    head_w_host = inputs.head_weights(configs.LM_HEAD)
    head_w = torch.from_numpy(head_w_host.view(np.int16)).view(torch.bfloat16).to(dev)
    torch.cuda.synchronize()
    # load-time quantization (timed once, cold)
    qs, qe = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    qs.record()
    head = ops.Fp8LmHead.quantize(head_w)
    qe.record()
    torch.cuda.synchronize()
    quant_us = qs.elapsed_time(qe) * 1e3
    n_tok = wl.steps
    tokens = torch.from_numpy(np.concatenate([inputs.activations(wl, s) for s in range(n_tok)]).view(np.int16)) \
        .view(torch.bfloat16).to(dev).reshape(n_tok, 1, H)
    log(f"resident: {resident / 1e9:.2f} GB MoE + {head.q.numel() / 1e9:.3f} GB head; setup {time.time() - t0:.0f} s")

    # ------------------------------------------------------------------ decode step graphs
    # One graph node per step: step s reads its own resident token and writes
    # its own argmax slot (the residual stream and logits buffers are shared),
    # so every timed step's result can be read back and checked afterwards.
    W, K = args.warmup, args.steps
    h_out = torch.empty((1, H), dtype=torch.bfloat16, device=dev)
    logits = torch.empty((1, V), dtype=torch.float32, device=dev)
    am_hist = torch.full((W + K,), -2, dtype=torch.int32, device=dev)
    ws = ops.workspace(ops.decode_step_workspace_bytes(1, H, I, E, k, V), dev)

    def step(s, slot, argmax_buf=am_hist):
        ops.moe_decode_step(tokens[s % n_tok], stack, head, ws=ws,
                            out=dict(h=h_out, logits=logits, argmax=argmax_buf[slot:slot + 1]))

    step(0, 0)                                                   # eager once (also warms the code objects)
    torch.cuda.synchronize()

    def capture(first, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s in range(first, first + n):
                step(s, s)
        return g

    gw = capture(0, W) if W > 0 else None
    gt = capture(W, K)
    torch.cuda.synchronize()
    if gw is not None:
        gw.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    gt.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / K
    step_bytes = L * configs.moe_layer_bytes(m, k) + configs.head_bytes(V, H, 1, True)
    us_step = ms_step * 1e3
    gbps = step_bytes / (us_step * 1e-6) / 1e9
    log(f"decode step: {us_step:.1f} us, {gbps:.0f} GB/s ({100 * gbps / PEAK_GBPS:.1f}% of 8 TB/s)")
    # the timed steps: every argmax read back, each checked against an eager
    # call on the same token (a failed wait would show as -1)
    h_last, logits_last = h_out.clone(), logits.clone()
    timed_am = am_hist[W:].cpu().numpy()
    am_eager = torch.full((K,), -2, dtype=torch.int32, device=dev)
    for j in range(K):
        step(W + j, j, am_eager)
    torch.cuda.synchronize()
    eager_am = am_eager.cpu().numpy()
    timed_valid = bool(np.all(timed_am >= 0) and np.array_equal(timed_am, eager_am))
    log(f"timed steps valid: {timed_valid} ({int(np.sum(timed_am < 0))} failed, "
        f"{int(np.sum(timed_am != eager_am))} differ from eager)")

    # ------------------------------------------------------------------ dominant kernel: the one-launch step
    # Ten back-to-back steps per graph: the average launch duration of the
    # step kernel itself, measured with events on the launch stream.
    am_k = torch.full((10,), -2, dtype=torch.int32, device=dev)
    gk = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gk):
        for j in range(10):
            step(W + j, j, am_k)
    gk.replay()
    torch.cuda.synchronize()
    reps = max(1, args.kernel_reps // 10)
    e0.record()
    for _ in range(reps):
        gk.replay()
    e1.record()
    torch.cuda.synchronize()
    k_us = e0.elapsed_time(e1) * 1e3 / (10 * reps)
    k_gbps = step_bytes / (k_us * 1e-6) / 1e9
    probe = read_probe(torch, ops, dev)
    roofline = {"kernel": "decode_step_kernel (one launch: 32 MoE layers + FP8 head with argmax)", "bound": "hbm",
                "achieved": round(k_gbps, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                "frac": round(k_gbps / PEAK_GBPS, 4), "traffic": step_traffic_bytes(),
                "bytes_per_launch": step_bytes, "us_per_launch": round(k_us, 2),
                "frac_of_read_probe": round(k_gbps / probe["GBps"], 4)}
    log(f"step kernel: {k_us:.1f} us per launch, {k_gbps:.0f} GB/s; read probe {probe['GBps']:.0f} GB/s")

    # ------------------------------------------------------------------ the verify pass through the whole stack
    # Four resident tokens per step through all layers and the head (the
    # multi-token-prediction verify shape), ten steps per graph; the last
    # step's outputs are checked bit for bit against an eager call.
    n4 = max(1, n_tok // 4)
    tok4 = tokens.reshape(n_tok, H)[torch.arange(4 * n4, device=dev) % n_tok].reshape(n4, 4, H)
    ws4 = ops.workspace(ops.decode_step_workspace_bytes(4, H, I, E, k, V), dev)
    out4 = dict(h=torch.empty((4, H), dtype=torch.bfloat16, device=dev),
                logits=torch.empty((4, V), dtype=torch.float32, device=dev),
                argmax=torch.empty((4,), dtype=torch.int32, device=dev))
    ops.moe_decode_step(tok4[0], stack, head, ws=ws4, out=out4)
    torch.cuda.synchronize()
    g4 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g4):
        for j in range(10):
            ops.moe_decode_step(tok4[j % n4], stack, head, ws=ws4, out=out4)
    g4.replay()
    torch.cuda.synchronize()
    v_reps = 5
    e0.record()
    for _ in range(v_reps):
        g4.replay()
    e1.record()
    torch.cuda.synchronize()
    v_us = e0.elapsed_time(e1) * 1e3 / (10 * v_reps)
    g_h, g_am = out4["h"].clone(), out4["argmax"].clone()
    ops.moe_decode_step(tok4[9 % n4], stack, head, ws=ws4, out=out4)
    torch.cuda.synchronize()
    v_ok = bool(torch.equal(g_h, out4["h"]) and torch.equal(g_am, out4["argmax"]))
    # algorithmic bytes of each of the ten steps: every layer's distinct
    # routed experts (from a traced eager call) + shared expert + router, and
    # the head
    v_bytes = []
    for j in range(10):
        ids = ops.moe_decode_step(tok4[j % n4], stack, head, ws=ws4, trace=True)["ids_trace"].cpu().numpy()
        v_bytes.append(sum(configs.moe_layer_bytes(m, len(np.unique(ids[l]))) for l in range(L))
                       + configs.head_bytes(V, H, 4, True))
    v_gbps = float(np.mean(v_bytes)) / (v_us * 1e-6) / 1e9
    verify_step = {"tokens_per_step": 4, "us_per_step": round(v_us, 2), "over_one_token_step": round(v_us / k_us, 3),
                   "bytes_per_step": int(np.mean(v_bytes)), "achieved_GBps": round(v_gbps, 1),
                   "frac_of_peak": round(v_gbps / PEAK_GBPS, 4), "graph_equals_eager": v_ok,
                   "note": "4 seeded resident tokens per step through all layers (per-phase launches) and the FP8 "
                           "head with argmax; ten steps per graph, warm replays"}
    log(f"verify step (4 tokens): {v_us:.1f} us ({v_us / k_us:.2f}x the one-token step), {v_gbps:.0f} GB/s, "
        f"graph == eager: {v_ok}")
    del ws4

    # ------------------------------------------------------------------ the FP8 LM head kernel on its own
    u = torch.from_numpy(inputs.activations(wl, 0).view(np.int16)).view(torch.bfloat16).to(dev)
    hws = ops.workspace(ops.lm_head_workspace_bytes(1, V, H), dev)
    hlog = torch.empty((1, V), dtype=torch.float32, device=dev)
    ham = torch.empty((1,), dtype=torch.int32, device=dev)

    def head_call():
        ops._lib.call("lm_head_gemv_fp8_argmax", ops._p(head.q), ops._p(head.s), V, H, ops._p(u), 1,
                      ops._p(hlog), ops._p(ham), ops._p(hws), hws.numel(), ops._stream(dev))

    gh = torch.cuda.CUDAGraph()
    head_call()
    torch.cuda.synchronize()
    with torch.cuda.graph(gh):
        for _ in range(10):
            head_call()
    gh.replay()
    torch.cuda.synchronize()
    reps = max(1, args.head_reps // 10)
    e0.record()
    for _ in range(reps):
        gh.replay()
    e1.record()
    torch.cuda.synchronize()
    head_us = e0.elapsed_time(e1) * 1e3 / (10 * reps)
    head_bytes = configs.head_bytes(V, H, 1, True)
    head_gbps = head_bytes / (head_us * 1e-6) / 1e9
    head_kernel = {"kernel": "lm_head_wide_kernel<fp8> (FP8 LM-head GEMV + argmax, 1 token, standalone)", "bound": "hbm",
                   "achieved": round(head_gbps, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                   "frac": round(head_gbps / PEAK_GBPS, 4), "bytes_per_launch": head_bytes,
                   "us_per_launch": round(head_us, 2), "frac_of_read_probe": round(head_gbps / probe["GBps"], 4)}
    log(f"fp8 head: {head_us:.1f} us, {head_gbps:.0f} GB/s")

    result = {
        "metric": "µs per decode step & achieved HBM GB/s (% of peak), MoE layer + FP8 LM head",
        "value": round(us_step, 2), "unit": "µs", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_step, 5), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4/fp8 weights, bf16 activations, f32 accumulate", "data": "synthetic (seeded), resident in HBM",
        "config": {"workload": wl.name, "layers": L, "hidden": H, "experts": E, "top_k": k, "expert_intermediate": I,
                   "vocab": V, "tokens_per_step": 1, "seeded_tokens": n_tok, "resident_bytes": resident + head.q.numel(),
                   "step_bytes": step_bytes},
        "achieved_GBps": round(gbps, 1), "frac_of_peak": round(gbps / PEAK_GBPS, 4),
        "timed_steps_valid": timed_valid,
        "timed_steps_checked": {"steps": K, "argmax_negative": int(np.sum(timed_am < 0)),
                                "differ_from_eager": int(np.sum(timed_am != eager_am))},
        "roofline": roofline,
        "head_kernel": head_kernel,
        "verify_step": verify_step,
        "read_probe": probe,
    }

    if not args.no_breakdown:
        result["breakdown"] = breakdown(torch, ops, configs, inputs, dev, stack, head, head_w, wl, quant_us, probe,
                                        reps=args.breakdown_reps)
    if not args.no_cpu:
        # the timed steps whose every layer is checked against the oracle: the
        # first, middle and last of the timed range (the last one's residual
        # stream and logits are the timed graph's own final outputs)
        picks = [W, W + K // 2, W + K - 1] if K >= 3 else [W + j for j in range(K)]
        graph_out = dict(step=W + K - 1, h=h_last, logits=logits_last)
        cpu, par = step_oracle(torch, ops, configs, inputs, stack, head, wl, tokens, n_tok, picks, timed_am, W,
                               graph_out, step_bytes)
        cpu["per_unit"] = oracle_per_unit(torch, ops, configs, inputs, dev, stack, head)
        result["cpu_baseline"] = cpu
        result["parity_32_layers"] = par
    print(json.dumps(result), flush=True)
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: 3 x {args.calib_copy_mib} MiB device-to-device")


def read_probe(torch, ops, dev, gib=1, reps=10):
    """The library's plain streaming-read kernel over a 1 GiB buffer: the rate a
    pure read reaches on this GPU (median of `reps` launches)."""
    n = gib << 30
    buf = torch.ones(n // 8, dtype=torch.int64, device=dev)
    out = torch.zeros(1, dtype=torch.int32, device=dev)

    def call():
        ops._lib.call("wsx_read_probe", ops._p(buf), n, ops._p(out), ops._stream(dev))

    call()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        # five back-to-back launches per sample, so the host's launch latency
        # is not counted as GPU time
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(5):
            call()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3 / 5)
    us = float(np.median(ts))
    del buf
    return {"kernel": "read_probe_kernel (16-byte nontemporal loads, 8 in flight per thread, 2048 workgroups)", "bytes": n,
            "median_us": round(us, 2), "GBps": round(n / (us * 1e-6) / 1e9, 1),
            "frac_of_peak": round(n / (us * 1e-6) / 1e9 / PEAK_GBPS, 4)}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_step_kernel_hbm_counters.md")
STEP_SOURCES = ("weight_streaming_expert_amd/csrc/decode_step_kernel.h", "weight_streaming_expert_amd/csrc/decode_step.hip",
                "weight_streaming_expert_amd/csrc/wsx_device.h")


def step_source_digest():
    """sha256 over the step kernel's sources, to tell whether recorded counters still apply."""
    import hashlib
    h = hashlib.sha256()
    for f in STEP_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def step_traffic_bytes():
    """HBM bytes per launch of the step kernel, from the recorded FETCH_SIZE and
    WRITE_SIZE counter runs (scaled by a plain copy of known size); None when no
    record exists or the kernel's sources changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and line.startswith("- `"):
            key, val = line[3:].split("`", 1)
            rec[key] = val.split(":", 1)[1].strip().strip("`")
    if rec.get("sources_sha256") != step_source_digest():
        return None
    try:
        return int(rec["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _timed_graph(torch, fn, flush=None, reps=100, before=None, after=None):
    """µs of a captured graph replayed `reps` times, each after an optional
    per-sample input update `before(i)` and cache flush (outside the timed
    interval); `after(i)` runs once the sample has completed.  Returns the
    per-sample times."""
    g = torch.cuda.CUDAGraph()
    if before is not None:
        before(0)
    fn()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    ts = []
    for i in range(reps):
        if before is not None:
            before(i)
        if flush is not None:
            flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
        if after is not None:
            after(i)
    return np.array(ts)


def _stats(ts, bytes_per_sample=None, probe=None):
    d = dict(samples=int(len(ts)), median_us=round(float(np.median(ts)), 2),
             p10_us=round(float(np.percentile(ts, 10)), 2), p90_us=round(float(np.percentile(ts, 90)), 2))
    if bytes_per_sample is not None:
        b = np.broadcast_to(np.asarray(bytes_per_sample, dtype=np.float64), ts.shape)
        rate = b / (ts * 1e-6) / 1e9
        d.update(bytes=int(np.median(b)), GBps=round(float(np.median(rate)), 1),
                 frac_of_peak=round(float(np.median(rate)) / PEAK_GBPS, 4))
        if probe is not None:
            d["frac_of_read_probe"] = round(float(np.median(rate)) / probe["GBps"], 4)
    return d


def breakdown(torch, ops, configs, inputs, dev, stack, head, head_w, wl, quant_us, probe, reps=100):
    m = wl.moe
    H, I, E, k, V = m.H, m.I, m.E, m.k, head.V
    flush_buf = torch.ones(1 << 27, dtype=torch.int64, device=dev)   # 1 GiB

    def flush():
        # a read-only sweep: it evicts the caches without leaving dirty lines
        # whose write-back would land inside the next timed kernel
        flush_buf.sum()

    def bf16_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    out = {}
    # what the timing itself costs: the same sweep, events and graph replay
    # around one small launch of the library (the read probe over 64 KiB), so
    # the rows below can also be read net of it (net_median_us)
    pbuf = torch.ones(1 << 13, dtype=torch.int64, device=dev)
    pout = torch.zeros(1, dtype=torch.int32, device=dev)
    ts = _timed_graph(torch, lambda: ops._lib.call("wsx_read_probe", ops._p(pbuf), pbuf.numel() * 8, ops._p(pout),
                                                   ops._stream(dev)), flush, reps=reps)
    out["harness_overhead"] = _stats(ts)
    out["harness_overhead"]["note"] = ("event pair and graph replay after the 1 GiB sweep around one 64 KiB read-probe "
                                       "launch; included in every row's median_us")
    # one MoE layer of the resident stack (layer 0), timed per seeded input
    # with a cold cache: 100 one-token inputs (the single-layer workload) and
    # 100 four-token verify passes
    layer = dict(router=stack.w_router[0], w13c=stack.w13_codes[0], w13s=stack.w13_scales[0],
                 w2c=stack.w2_codes[0], w2s=stack.w2_scales[0], shared=tuple(t[0] for t in stack.shared))
    rows = ((configs.MOE_LAYER, "moe_layer_t1", ops.moe_expert_gemv_mxfp4),
            (configs.VERIFY, "moe_layer_verify_t4", ops.moe_expert_gemv_mxfp4),
            (configs.MOE_LAYER, "moe_layer_w4a8_t1", ops.moe_expert_gemv_w4a8),
            (configs.VERIFY, "moe_layer_w4a8_verify_t4", ops.moe_expert_gemv_w4a8),
            (configs.GROUPED16, "moe_layer_grouped_t16", ops.moe_expert_gemv_mxfp4),
            (configs.GROUPED16, "moe_layer_w4a8_grouped_t16", ops.moe_expert_gemv_w4a8))
    for wlx, name, experts in rows:
        T = wlx.T
        xs = [bf16_dev(inputs.activations(wlx, s)) for s in range(min(wlx.steps, reps))]
        x = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        res = torch.empty_like(x)
        ws = ops.workspace(ops.moe_workspace_bytes(T, H, I, E, k), dev)
        held = {}
        n_active = []

        def layer_call():
            rr = ops.moe_route_topk(x, layer["router"], k, ws=ws)
            experts(x, layer["w13c"], layer["w13s"], layer["w2c"], layer["w2s"], rr["expert_list"], rr["slot_w"], k,
                    shared=layer["shared"], residual=res, ws=ws)
            held["el"] = rr["expert_list"]

        def before(i):
            x.copy_(xs[i])
            res.copy_(xs[i])

        ts = _timed_graph(torch, layer_call, flush, reps=len(xs), before=before,
                          after=lambda i: n_active.append(int(held["el"][0])))
        na = np.array(n_active)
        t = _stats(ts, [configs.moe_layer_bytes(m, int(n)) for n in na], probe)
        t.update(distinct_experts=dict(min=int(na.min()), median=float(np.median(na)), max=int(na.max())),
                 inputs=f"{len(xs)} seeded inputs of {wlx.name}, each after a 1 GiB read-only sweep")
        out[name] = t
    # the FP8 head on 100 seeded cold tokens, and on 4 rows (the verify pass)
    xh = [bf16_dev(inputs.activations(configs.LM_HEAD, s)) for s in range(configs.LM_HEAD.steps)]
    for T in (1, 4):
        x = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        hws = ops.workspace(ops.lm_head_workspace_bytes(T, V, H), dev)
        rows = lambda i, T=T: torch.cat([xh[(i * T + j) % len(xh)] for j in range(T)])
        ts = _timed_graph(torch, lambda: head.gemv_argmax(x, ws=hws), flush, reps=reps,
                          before=lambda i, x=x, rows=rows: x.copy_(rows(i)))
        out[f"lm_head_fp8_t{T}"] = _stats(ts, configs.head_bytes(V, H, T, True), probe)
    x = bf16_dev(inputs.normal_bf16((wl.seed, 8), (4, H), 1.0))
    # the sampling epilogue at the GSM8K settings (temperature 0.6, top-k 29,
    # top-p 0.95): the sampler alone on resident logits, and head + sampler
    for T in (1, 4):
        xt = x[:T].contiguous()
        u = torch.from_numpy(inputs.uniform_f32((wl.seed, 9, T), (T,))).to(dev)
        logits_t, _ = head.gemv_argmax(xt)
        sws = ops.workspace(ops._lib.load().wsx_sample_workspace_bytes(T, V, 29), dev)
        ts = _timed_graph(torch, lambda: ops.lm_sample_topk_topp(logits_t, 0.6, 29, 0.95, u, ws=sws), flush, reps=reps)
        t = _stats(ts)
        t.update(bytes=T * V * 4)
        out[f"sample_topk_topp_t{T}"] = t
        fws = ops.workspace(ops._lib.load().wsx_lm_head_sample_workspace_bytes(T, V, H, 29), dev)
        ts = _timed_graph(torch, lambda: ops.lm_head_gemv_fp8_sample(head.q, head.s, xt, 0.6, 29, 0.95, u, ws=fws),
                          flush, reps=reps)
        out[f"lm_head_fp8_sample_t{T}"] = _stats(ts, configs.head_bytes(V, H, T, True), probe)
    hws = ops.workspace(ops.lm_head_workspace_bytes(1, V, H), dev)
    x1 = torch.empty((1, H), dtype=torch.bfloat16, device=dev)
    ts = _timed_graph(torch, lambda: ops.lm_head_gemv_bf16_argmax(head_w, x1, ws=hws), flush, reps=reps,
                      before=lambda i: x1.copy_(xh[i % len(xh)]))
    out["lm_head_bf16_t1"] = _stats(ts, configs.head_bytes(V, H, 1, False), probe)
    out["bf16_over_fp8_time"] = round(out["lm_head_bf16_t1"]["median_us"] / out["lm_head_fp8_t1"]["median_us"], 3)
    # load-time quantizer kernel alone (outputs preallocated, cold cache), plus
    # the first call's time including the 403 MB output allocation
    qq, qsc = torch.empty_like(head.q), torch.empty_like(head.s)
    ts = _timed_graph(torch, lambda: ops._lib.call("lm_head_quantize_fp8", ops._p(head_w), V, H, ops._p(qq),
                                                   ops._p(qsc), ops._stream(dev)), flush, reps=min(20, reps))
    assert torch.equal(qq, head.q) and torch.equal(qsc, head.s)
    t = _stats(ts, V * H * 2 + V * H + V * 4, probe)
    t.update(first_call_incl_alloc_us=round(quant_us, 1))
    out["quantize_fp8"] = t
    base = out["harness_overhead"]["median_us"]
    for name, d in out.items():
        if name != "harness_overhead" and isinstance(d, dict) and "median_us" in d:
            d["net_median_us"] = round(d["median_us"] - base, 2)
            if "bytes" in d and d["net_median_us"] > 0:
                d["net_frac_of_peak"] = round(d["bytes"] / (d["net_median_us"] * 1e-6) / 1e9 / PEAK_GBPS, 4)
    out["verify_over_decode_layer"] = round(out["moe_layer_verify_t4"]["median_us"] / out["moe_layer_t1"]["median_us"], 3)
    out["w4a8_over_bf16_layer_t1"] = round(out["moe_layer_w4a8_t1"]["median_us"] / out["moe_layer_t1"]["median_us"], 3)
    del flush_buf
    return out


def _thread_ctx(n):
    import contextlib
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:                                            # pragma: no cover
        return contextlib.nullcontext()
    return threadpool_limits(limits=n)


def step_oracle(torch, ops, configs, inputs, stack, head, wl, tokens, n_tok, picks, timed_am, W, graph_out,
                step_bytes):
    """The CPU oracle on three of the timed steps, every layer teacher-forced.

    Each picked step is rerun eagerly with traces (h_l, u_l, routing of every
    layer); its argmax must equal what the timed graph wrote for that step, and
    for the last timed step the residual stream and logits must equal the
    timed graph's own final outputs bit for bit.  Then, for every one of the
    32 layers, the oracle recomputes the norm, the router logits and top-k,
    the experts for the device's routing and the residual add, and the head
    on the last normalized stream; each stage is checked against the device.
    The first pick is timed with one BLAS thread, the others with all cores;
    expert regeneration is not timed."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import parity as P
    from oracle import compare as C
    from oracle import head as OH
    from oracle import moe as OM
    m = wl.moe
    L, k, I = stack.L, m.k, m.I
    ncores = len(os.sched_getaffinity(0))
    traces = []
    for s in picks:
        o = ops.moe_decode_step(tokens[s % n_tok], stack, head, trace=True)
        torch.cuda.synchronize()
        assert int(o["argmax"][0]) == int(timed_am[s - W]), "traced step differs from the timed graph's argmax"
        if s == graph_out["step"]:
            assert torch.equal(o["h"], graph_out["h"]) and torch.equal(o["logits"], graph_out["logits"]), \
                "traced step differs from the timed graph's outputs"
        traces.append(dict(h=P.bits(o["h_trace"]), u=P.bits(o["u_trace"]), ids=P.np_(o["ids_trace"]),
                           w=P.np_(o["w_trace"]), logits=P.np_(o["logits"]), argmax=P.np_(o["argmax"])))
    threads = [1] + [ncores] * (len(picks) - 1)
    t_layers = [0.0] * len(picks)
    t_head = [0.0] * len(picks)
    worst = dict(y_rel=0.0, logit_rel=0.0)
    near_ties = 0
    for l in range(L):
        wr = P.router_values(inputs.router_weights(wl, l))
        shared = inputs.expert_weights(wl, l, inputs.SHARED)
        need = sorted(set(int(e) for tr in traces for e in tr["ids"][l].reshape(-1)))
        experts = {e: inputs.expert_weights(wl, l, e) for e in need}
        get = experts.__getitem__
        for j, tr in enumerate(traces):
            ht, ut, ids, wts = tr["h"], tr["u"], tr["ids"][l], tr["w"][l]
            with _thread_ctx(threads[j]):
                t0 = time.perf_counter()
                u_ref = OM.rmsnorm_bf16(ht[l])
                ref_logits = OM.router_logits(ut[l], wr)
                OM.route(ref_logits, k)
                y_ref = P.moe_y_ref(ut[l], ids, wts, get, shared, I)
                OM.residual_bf16(ht[l], y_ref)
                t_layers[j] += time.perf_counter() - t0
            del u_ref
            P.check_norm(ht[l], ut[l])
            near_ties += P.check_routing(ut[l], wr, k, ids, wts)
            P.check_h_next(ht[l], y_ref, ht[l + 1])
    qh, sh = P.np_(head.q), P.np_(head.s)
    for j, tr in enumerate(traces):
        with _thread_ctx(threads[j]):
            t0 = time.perf_counter()
            ref = OH.head_logits(qh, sh, tr["u"][L])
            OH.greedy_argmax(ref)
            t_head[j] = time.perf_counter() - t0
        P.check_norm(tr["h"][L], tr["u"][L])
        ok, r = C.fp_close(tr["logits"], ref)
        assert ok, f"head logits off by {r:.3e} x RMS"
        worst["logit_rel"] = max(worst["logit_rel"], r)
        ok, ties = C.check_argmax(tr["argmax"], ref)
        assert ok, "argmax mismatch"
        near_ties += ties
    per_step = [tl + th for tl, th in zip(t_layers, t_head)]
    cpu = {"value": round(per_step[0] * 1e6, 0), "unit": "µs per decode step", "cores": 1, "kind": "oracle",
           "sample": f"{len(picks)} timed steps, all {L} layers + the FP8 head each, fp64 numpy; the first with "
                     f"1 BLAS thread, the others with {ncores}; expert regeneration not timed",
           "all_cores": {"value": round(float(np.mean(per_step[1:])) * 1e6, 0) if len(per_step) > 1 else None,
                         "cores": ncores},
           "layer_s_1_thread": round(t_layers[0] / L, 3), "head_s_1_thread": round(t_head[0], 3),
           "cpu": _cpu_name(), "host_cores_visible": ncores}
    par = {"steps_checked": [int(s) for s in picks], "layers_per_step": L, "result": "ok",
           "near_tie_tokens": int(near_ties), "head_logits_worst_rel": round(worst["logit_rel"], 6),
           "graph_outputs_equal_traced": True}
    return cpu, par


def oracle_per_unit(torch, ops, configs, inputs, dev, stack, head):
    """Oracle seconds per unit of each workload, with 1 BLAS thread and with all
    cores: the tiny decode (MoE layer + 4096-row head) per token, one Ling
    MoE layer per token, the FP8 head per token, one 4-token verify layer."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import parity as P
    from oracle import head as OH
    from oracle import moe as OM
    ncores = len(os.sched_getaffinity(0))
    res = {}

    def timed(fn, n):
        out = {}
        for th in (1, ncores):
            with _thread_ctx(th):
                t0 = time.perf_counter()
                for i in range(n):
                    fn(i)
                out[f"s_per_unit_{th}_threads"] = round((time.perf_counter() - t0) / n, 4)
        out["units_timed"] = n
        return out

    tw = configs.TINY
    tl = inputs.layer_weights(tw, 0)
    tq, ts_ = OH.quantize_fp8(inputs.head_weights(tw, K=tw.moe.H))
    get_t = lambda e: (tl["w13c"][e], tl["w13s"][e], tl["w2c"][e], tl["w2s"][e])

    def tiny(i):
        x = inputs.activations(tw, i)
        r = OM.moe_layer(x, P.router_values(tl["router"]), tw.moe.k, get_t, tl["shared"], x, tw.moe.I)
        OH.greedy_argmax(OH.head_logits(tq, ts_, r["h"]))

    res["tiny_decode"] = timed(tiny, tw.steps)
    lw = configs.MOE_LAYER
    wr = P.router_values(inputs.router_weights(configs.DECODE_STEP, 0))
    sh = inputs.expert_weights(configs.DECODE_STEP, 0, inputs.SHARED)
    cache = {}

    def get_l(e):
        if e not in cache:
            cache[e] = inputs.expert_weights(configs.DECODE_STEP, 0, e)
        return cache[e]

    def layer_t(wlx):
        def run(i):
            x = inputs.activations(wlx, i)
            OM.moe_layer(x, wr, lw.moe.k, get_l, sh, x, lw.moe.I)
        return run

    for i in range(3):                                     # regenerate the experts outside the timing
        x = inputs.activations(lw, i)
        for e in OM.route(OM.router_logits(x, wr), lw.moe.k)[0].reshape(-1):
            get_l(int(e))
    res["moe_layer_t1"] = timed(layer_t(lw), 3)
    vx = inputs.activations(configs.VERIFY, 0)
    for e in OM.route(OM.router_logits(vx, wr), lw.moe.k)[0].reshape(-1):
        get_l(int(e))
    res["moe_layer_verify_t4"] = timed(layer_t(configs.VERIFY), 1)
    qh, shs = P.np_(head.q), P.np_(head.s)
    res["lm_head_fp8_t1"] = timed(lambda i: OH.greedy_argmax(OH.head_logits(qh, shs, inputs.activations(configs.LM_HEAD, i))), 2)
    return res


def _cpu_name():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
