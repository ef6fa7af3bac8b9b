"""Decode-step benchmark: 32 stacked Ling-shaped MoE layers + the FP8 LM head, batch 1.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers 32] [--no-breakdown] [--no-cpu]

A step is one decode pass through the whole hot path: for each of the 32
layers the RMS norm of the residual stream, the router GEMV with top-8 of 512,
the MXFP4 routed (8) + shared SwiGLU experts and the bf16 residual add, then
the FP8 head (157,184 x 2,560) with the fused greedy argmax.  Inputs (51.5 GB
of MXFP4 experts, the quantized head and 2,000 seeded tokens) are resident in
HBM before timing; each step is one replay of a captured HIP graph on one
stream, preceded by a 5 KB device copy of that step's token.

Prints one JSON line (rank 0) with the µs per step, the achieved HBM rate of
the step's algorithmic bytes, the roofline object of the dominant kernel (the
single-launch decode step), the standalone FP8 head kernel's rate, a
per-component breakdown (one MoE layer with a cold cache, the FP8 and BF16
heads, the 4-token verify pass, the sampling epilogue at the GSM8K settings,
the load-time quantizer) and the CPU-oracle
baseline timed on a bounded sample of the same workload.
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
    host_layer0 = None
    for l in range(L):
        lw = inputs.layer_weights(wl, l, out=stage)
        for key in shapes:
            dw[key][l].copy_(stage_t[key])
        router[l].copy_(torch.from_numpy(lw["router"].view(np.int16)).view(torch.bfloat16))
        for i in range(4):
            sh[i][l].copy_(torch.from_numpy(lw["shared"][i]))
        if l == 0:
            host_layer0 = {key: v.copy() if isinstance(v, np.ndarray) else v for key, v in lw.items()}
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

    # ------------------------------------------------------------------ decode step graph
    h_in = torch.empty((1, H), dtype=torch.bfloat16, device=dev)
    out = dict(h=torch.empty((1, H), dtype=torch.bfloat16, device=dev),
               logits=torch.empty((1, V), dtype=torch.float32, device=dev),
               argmax=torch.empty((1,), dtype=torch.int32, device=dev))
    ws = ops.workspace(ops.decode_step_workspace_bytes(1, H, I, E, k, V), dev)
    h_in.copy_(tokens[0])
    ops.moe_decode_step(h_in, stack, head, ws=ws, out=out)        # eager once (also warms the code objects)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.moe_decode_step(h_in, stack, head, ws=ws, out=out)
    torch.cuda.synchronize()

    def run_steps(n, start):
        for s in range(n):
            h_in.copy_(tokens[(start + s) % n_tok])
            g.replay()

    run_steps(args.warmup, 0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run_steps(args.steps, args.warmup)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    step_bytes = L * configs.moe_layer_bytes(m, k) + configs.head_bytes(V, H, 1, True)
    us_step = ms_step * 1e3
    gbps = step_bytes / (us_step * 1e-6) / 1e9
    log(f"decode step: {us_step:.1f} us, {gbps:.0f} GB/s ({100 * gbps / PEAK_GBPS:.1f}% of 8 TB/s)")

    # ------------------------------------------------------------------ dominant kernel: the one-launch step
    # Ten back-to-back steps per graph, no token copies between them: the
    # average launch duration of the step kernel itself.
    gk = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gk):
        for _ in range(10):
            ops.moe_decode_step(h_in, stack, head, ws=ws, out=out)
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
    roofline = {"kernel": "decode_step_kernel (one launch: 32 MoE layers + FP8 head with argmax)", "bound": "hbm",
                "achieved": round(k_gbps, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                "frac": round(k_gbps / PEAK_GBPS, 4), "traffic": step_traffic_bytes(),
                "bytes_per_launch": step_bytes, "us_per_launch": round(k_us, 2)}
    log(f"step kernel: {k_us:.1f} us per launch, {k_gbps:.0f} GB/s")

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
                   "us_per_launch": round(head_us, 2)}
    log(f"fp8 head: {head_us:.1f} us, {head_gbps:.0f} GB/s")

    result = {
        "metric": "µs per decode step & achieved HBM GB/s (% of peak), MoE layer + FP8 LM head",
        "value": round(us_step, 2), "unit": "µs", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4/fp8 weights, bf16 activations, f32 accumulate", "data": "synthetic (seeded), resident in HBM",
        "config": {"workload": wl.name, "layers": L, "hidden": H, "experts": E, "top_k": k, "expert_intermediate": I,
                   "vocab": V, "tokens_per_step": 1, "seeded_tokens": n_tok, "resident_bytes": resident + head.q.numel(),
                   "step_bytes": step_bytes},
        "achieved_GBps": round(gbps, 1), "frac_of_peak": round(gbps / PEAK_GBPS, 4),
        "roofline": roofline,
        "head_kernel": head_kernel,
    }

    if not args.no_breakdown:
        result["breakdown"] = breakdown(torch, ops, configs, inputs, dev, stack, head, head_w, host_layer0, wl,
                                        quant_us)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(torch, ops, configs, inputs, dev, stack, head, host_layer0, wl, step_bytes)
    print(json.dumps(result), flush=True)
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: 3 x {args.calib_copy_mib} MiB device-to-device")


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_step_kernel_hbm_counters.md")
STEP_SOURCES = ("weight_streaming_expert_amd/csrc/decode_step.hip", "weight_streaming_expert_amd/csrc/wsx_device.h")


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


def _timed_graph(torch, fn, flush=None, reps=100):
    """Median µs of a captured graph replayed `reps` times, each after an
    optional cache flush (outside the timed interval)."""
    g = torch.cuda.CUDAGraph()
    fn()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    ts = []
    for _ in range(reps):
        if flush is not None:
            flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    ts = np.array(ts)
    return dict(median_us=round(float(np.median(ts)), 2), p10_us=round(float(np.percentile(ts, 10)), 2),
                p90_us=round(float(np.percentile(ts, 90)), 2))


def breakdown(torch, ops, configs, inputs, dev, stack, head, head_w, lw0, wl, quant_us):
    m = wl.moe
    H, I, E, k, V = m.H, m.I, m.E, m.k, head.V
    flush_buf = torch.ones(1 << 27, dtype=torch.int64, device=dev)   # 1 GiB

    def flush():
        # a read-only sweep: it evicts the caches without leaving dirty lines
        # whose write-back would land inside the next timed kernel
        flush_buf.sum()

    out = {}
    layer = dict(router=stack.w_router[0], w13c=stack.w13_codes[0], w13s=stack.w13_scales[0],
                 w2c=stack.w2_codes[0], w2s=stack.w2_scales[0], shared=tuple(t[0] for t in stack.shared))
    for T, name in ((1, "moe_layer_t1"), (4, "moe_layer_verify_t4")):
        x = torch.from_numpy(inputs.normal_bf16((wl.seed, 7, T), (T, H), 1.0).view(np.int16)).view(torch.bfloat16).to(dev)
        res = x.clone()
        ws = ops.workspace(ops.moe_workspace_bytes(T, H, I, E, k), dev)
        r = ops.moe_route_topk(x, layer["router"], k, ws=ws)
        torch.cuda.synchronize()
        n_active = int(r["expert_list"][0])

        def layer_call():
            rr = ops.moe_route_topk(x, layer["router"], k, ws=ws)
            ops.moe_expert_gemv_mxfp4(x, layer["w13c"], layer["w13s"], layer["w2c"], layer["w2s"], rr["expert_list"],
                                      rr["slot_w"], k, shared=layer["shared"], residual=res, ws=ws)

        t = _timed_graph(torch, layer_call, flush)
        b = configs.moe_layer_bytes(m, n_active)
        t.update(bytes=b, active_experts=n_active, GBps=round(b / (t["median_us"] * 1e-6) / 1e9, 1))
        out[name] = t
    x = torch.from_numpy(inputs.normal_bf16((wl.seed, 8), (4, H), 1.0).view(np.int16)).view(torch.bfloat16).to(dev)
    for T in (1, 4):
        xt = x[:T].contiguous()
        hws = ops.workspace(ops.lm_head_workspace_bytes(T, V, H), dev)
        t = _timed_graph(torch, lambda: head.gemv_argmax(xt, ws=hws), flush)
        b = configs.head_bytes(V, H, T, True)
        t.update(bytes=b, GBps=round(b / (t["median_us"] * 1e-6) / 1e9, 1))
        out[f"lm_head_fp8_t{T}"] = t
    # the sampling epilogue at the GSM8K settings (temperature 0.6, top-k 29,
    # top-p 0.95): the sampler alone on resident logits, and head + sampler
    for T in (1, 4):
        xt = x[:T].contiguous()
        u = torch.from_numpy(inputs.uniform_f32((wl.seed, 9, T), (T,))).to(dev)
        logits_t, _ = head.gemv_argmax(xt)
        sws = ops.workspace(ops._lib.load().wsx_sample_workspace_bytes(T, V, 29), dev)
        t = _timed_graph(torch, lambda: ops.lm_sample_topk_topp(logits_t, 0.6, 29, 0.95, u, ws=sws), flush)
        t.update(bytes=T * V * 4)
        out[f"sample_topk_topp_t{T}"] = t
        fws = ops.workspace(ops._lib.load().wsx_lm_head_sample_workspace_bytes(T, V, H, 29), dev)
        t = _timed_graph(torch, lambda: ops.lm_head_gemv_fp8_sample(head.q, head.s, xt, 0.6, 29, 0.95, u, ws=fws),
                         flush)
        b = configs.head_bytes(V, H, T, True)
        t.update(bytes=b, GBps=round(b / (t["median_us"] * 1e-6) / 1e9, 1))
        out[f"lm_head_fp8_sample_t{T}"] = t
    hws = ops.workspace(ops.lm_head_workspace_bytes(1, V, H), dev)
    x1 = x[:1].contiguous()
    t = _timed_graph(torch, lambda: ops.lm_head_gemv_bf16_argmax(head_w, x1, ws=hws), flush)
    b = configs.head_bytes(V, H, 1, False)
    t.update(bytes=b, GBps=round(b / (t["median_us"] * 1e-6) / 1e9, 1))
    out["lm_head_bf16_t1"] = t
    out["bf16_over_fp8_time"] = round(t["median_us"] / out["lm_head_fp8_t1"]["median_us"], 3)
    # load-time quantizer kernel alone (outputs preallocated, cold cache), plus
    # the first call's time including the 403 MB output allocation
    qq, qsc = torch.empty_like(head.q), torch.empty_like(head.s)
    t = _timed_graph(torch, lambda: ops._lib.call("lm_head_quantize_fp8", ops._p(head_w), V, H, ops._p(qq),
                                                  ops._p(qsc), ops._stream(dev)), flush, reps=20)
    assert torch.equal(qq, head.q) and torch.equal(qsc, head.s)
    qb = V * H * 2 + V * H + V * 4
    t.update(bytes=qb, GBps=round(qb / (t["median_us"] * 1e-6) / 1e9, 1), first_call_incl_alloc_us=round(quant_us, 1))
    out["quantize_fp8"] = t
    out["verify_over_decode_layer"] = round(out["moe_layer_verify_t4"]["median_us"] / out["moe_layer_t1"]["median_us"], 3)
    del flush_buf
    return out


def cpu_baseline(torch, ops, configs, inputs, dev, stack, head, lw0, wl, step_bytes):
    """The CPU oracle (fp64 numpy, one BLAS thread) on a bounded sample of the
    decode step: one token through the first 2 layers (teacher-forced on the
    GPU's own residual stream) and the full head; the per-step figure scales the
    layer time to all layers.  The same sample is checked against the GPU."""
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:                                            # pragma: no cover
        threadpool_limits = None
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import parity as P
    from oracle import head as OH
    m = wl.moe
    L_s = 2
    h0 = inputs.activations(wl, 0)
    out = ops.moe_decode_step(P.to_dev_bf16(h0), stack, head, trace=True)
    torch.cuda.synchronize()
    ht, ut = P.bits(out["h_trace"]), P.bits(out["u_trace"])
    ids, wts = P.np_(out["ids_trace"]), P.np_(out["w_trace"])
    qh, sh = P.np_(head.q), P.np_(head.s)
    lws = [lw0] + [inputs.layer_weights(wl, l) for l in range(1, L_s)]
    import contextlib
    ctx = threadpool_limits(limits=1) if threadpool_limits else contextlib.nullcontext()
    t_layers = 0.0
    with ctx:
        for l in range(L_s):
            lw = lws[l]
            get = lambda e, lw=lw: (lw["w13c"][e], lw["w13s"][e], lw["w2c"][e], lw["w2s"][e])
            t0 = time.perf_counter()
            from oracle import moe as OM
            u = OM.rmsnorm_bf16(ht[l])
            logits = OM.router_logits(u, P.router_values(lw["router"]))
            rid, rw = OM.route(logits, m.k)
            y = P.moe_y_ref(u, rid, rw, get, lw["shared"], m.I)
            OM.residual_bf16(ht[l], y)
            t_layers += time.perf_counter() - t0
            # parity of the sampled layer (teacher-forced on the GPU's stream)
            P.check_norm(ht[l], ut[l])
            P.check_routing(ut[l], P.router_values(lw["router"]), m.k, ids[l], wts[l])
            P.check_h_next(ht[l], P.moe_y_ref(ut[l], ids[l], wts[l], get, lw["shared"], m.I), ht[l + 1])
        t0 = time.perf_counter()
        ref = OH.head_logits(qh, sh, ut[-1])
        OH.greedy_argmax(ref)
        t_head = time.perf_counter() - t0
        P.check_head(qh, sh, ut[-1], P.np_(out["logits"]), P.np_(out["argmax"]))
        parity = "ok"
    L = stack.L
    per_step_s = t_layers / L_s * L + t_head
    return {"value": round(per_step_s * 1e6, 0), "unit": "µs per decode step", "cores": 1, "kind": "oracle",
            "sample": f"1 token: {L_s} of {L} MoE layers (scaled x{L / L_s:g}) + the full FP8 head, fp64 numpy, "
                      f"1 BLAS thread; measured {t_layers:.2f} s layers + {t_head:.2f} s head",
            "parity_on_sample": parity,
            "cpu": _cpu_name(), "host_cores_visible": len(os.sched_getaffinity(0))}


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
