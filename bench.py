"""Benchmark of the MoE-layer decode hot path on one MI355X.

Default workload: the 80B-A3B-shaped decode chain -- hidden 2048, 512 experts,
top-10, expert and shared intermediate 512, int4 group-64 weights, bf16
activations, 1 token through 48 distinct chained layers (pre-RMSNorm, MoE
layer, residual add).  A step is one token through all 48 layers.  The input
rotates over 8 seeded vectors so the routed experts change between steps and
the 43.5 GB slab cannot be served from the 256 MB Infinity Cache.  Each
rotation is one captured hipGraph of the whole chain.

Prints ONE JSON line (see the keys below).  ``value`` is the chain throughput
in tokens/s; the HBM figures use the algorithmic bytes of the step: router
weights, the routed experts' blobs actually selected, the shared blob and its
gate vector, and the activations in and out of each layer.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense bf16 / fp16 matrix-core peak of MI355X
N_ROTATE = 8


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default="decode_80b",
                   help="decode_80b (default), decode_35b, batched_80b, batched_80b_int8, "
                        "prefill_35b, tiny; the token mixers: gdn_80b, gdn_batched, att_80b, "
                        "att_batched; pool_80b: decode through an expert slot pool over pinned "
                        "host memory")
    p.add_argument("--layers", type=int, default=0, help="override the number of layers")
    p.add_argument("--cpu-layers", type=int, default=-1,
                   help="layers of the oracle's timed sample (default: the whole chain for "
                        "batch-1 decode, 1 layer otherwise; 0: skip the CPU baseline)")
    p.add_argument("--no-roofline", action="store_true", help="skip the per-launch event pass")
    p.add_argument("--dense-q4", action="store_true",
                   help="router rows and shared gate in 4 bits (MOE_FLAG_DENSE_Q4)")
    p.add_argument("--pool-frac", type=float, default=0.25,
                   help="pool_80b: slots as a fraction of the experts of the pack")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="also run one device-to-device copy of this many MiB (a reference "
                        "kernel of known traffic for hardware byte counters)")
    return p.parse_args()


def algorithmic_bytes(cfg, wl, unique_per_layer):
    """Bytes the method must move once per step (no re-reads, no scratch)."""
    T, E, H = cfg.n_tokens, cfg.n_experts, cfg.hidden
    act = 4 if cfg.act == "f32" else 2
    blob = int(wl.layout.blob_bytes)
    sblob = int(wl.slayout.blob_bytes)
    per_layer = []
    for U in unique_per_layer:
        if wl.dense_q4:
            # router rows and shared gate: 4-bit codes + (scale, bias) words
            R = E + 1
            b = R * H // 2 + R * (H // 64) * 4
        else:
            b = E * H * 4 + H * 4            # router weights and shared gate vector (fp32)
        b += E * 4 if cfg.zipf_s else 0      # router bias
        b += U * blob                        # routed experts, each read once
        b += sblob                           # shared expert blob
        b += 2 * T * H * act                 # x_hat in, out out
        per_layer.append(b)
    return per_layer


def algorithmic_flops(cfg):
    """Flops of one layer (a multiply-add counts 2): per token the router's E
    rows and the shared-gate row, gate, up and down of the k routed experts,
    and of the shared expert."""
    T, E, H, k, I, Is = (cfg.n_tokens, cfg.n_experts, cfg.hidden, cfg.top_k, cfg.inter,
                         cfg.shared_inter)
    per_token = 2 * ((E + (1 if Is else 0)) * H + k * 3 * H * I + 3 * H * Is)
    return T * per_token


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the MoE layer is measured on one MI355X's share of the work)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import int4_group_quantized_moe_amd as moe
    import synth
    import workload
    from synth import configs
    from synth import mixers as sm

    if args.config in sm.GDN_CONFIGS or args.config in sm.ATT_CONFIGS:
        return mixer_bench(args)
    if args.config == "pool_80b":
        return pool_bench(args)
    cfg = configs.CONFIGS[args.config]
    if args.layers:
        cfg = cfg.with_(layers=args.layers)
    torch.cuda.set_device(0)
    moe.lib()
    t0 = time.time()
    print(f"# building {cfg.name}: {cfg.layers} layers, T={cfg.n_tokens}", file=sys.stderr,
          flush=True)
    wl = workload.Workload(cfg, dense_q4=args.dense_q4)
    print(f"# built in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    d = wl.desc
    L, T = cfg.layers, cfg.n_tokens
    xs = [workload.act_tensor(cfg, synth.activations(cfg, variant=r)) for r in range(N_ROTATE)]
    x = torch.empty_like(xs[0])
    x_hat = torch.empty_like(x)
    out = torch.empty_like(x)
    ws = wl.workspace()
    stream = torch.cuda.Stream()

    def load_input(r):
        x.copy_(xs[r])

    def forward():
        moe.moe_chain_forward(d, L, x, wl.router_all, wl.router_bias, wl.slab, wl.slot_tables,
                              wl.shared, wl.shared_stride, x_hat, out, ws)

    def chain(r):
        load_input(r)
        forward()

    # eager run: routing statistics (unique experts per layer) per rotation
    pi, pw, pg = moe.moe_workspace_routing(d, ws)
    idx_off = pi - ws.data_ptr()
    uniq = np.zeros((N_ROTATE, L))
    for r in range(N_ROTATE):
        x.copy_(xs[r])
        for layer in range(L):
            moe.moe_rmsnorm(d, x, out if layer else None, x_hat)
            rw, rb, st, sh = wl.layer_args(layer)
            moe.moe_layer_forward(d, x_hat, rw, rb, wl.slab, st, sh, out, ws)
            idx = ws[idx_off: idx_off + 4 * T * cfg.top_k].view(torch.int32)
            uniq[r, layer] = torch.unique(idx).numel()
    torch.cuda.synchronize()
    bytes_per_rot = [sum(algorithmic_bytes(cfg, wl, uniq[r])) for r in range(N_ROTATE)]

    # one captured graph per input rotation; eager launches if the chain's
    # launch cannot be captured
    graphs = []
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for r in range(N_ROTATE):
            chain(r)                     # warm the capture stream
        torch.cuda.synchronize()
        try:
            for r in range(N_ROTATE):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    chain(r)
                graphs.append(g)
        except Exception as e:          # noqa: BLE001
            print(f"# graph capture unavailable ({type(e).__name__}); timing eager launches",
                  file=sys.stderr, flush=True)
            graphs = []
    torch.cuda.synchronize()
    mode = "hipgraph" if graphs else "eager"

    def step(s):
        if graphs:
            graphs[s % N_ROTATE].replay()
        else:
            chain(s % N_ROTATE)

    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # warmup + timed region
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for s in range(args.steps):
        step(s)
    ev1.record()
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / args.steps
    step_bytes = sum(bytes_per_rot[s % N_ROTATE] for s in range(args.steps)) / args.steps
    tokens_per_s = T / (ms_per_step / 1e3)
    gbps = step_bytes / (ms_per_step / 1e3) / 1e9
    step_flops = algorithmic_flops(cfg) * L
    tflops = step_flops / (ms_per_step / 1e3) / 1e12

    # correctness guards of the timed state: finite residual stream, and no
    # bounded wait of the persistent chain expired in any timed call
    assert torch.isfinite(x.float()).all(), "non-finite output"
    check_chain_status(moe, d, ws, "timed region")

    roofline = None
    if not args.no_roofline:
        roofline = chain_roofline(cfg, load_input, forward, bytes_per_rot, step_flops,
                                  dense_q4=args.dense_q4)
        check_chain_status(moe, d, ws, "roofline pass")

    # release the captured graphs (they hold the persistent chain launch)
    # and drain the device while the runtime is whole, not at interpreter exit
    for g in graphs:
        g.reset()
    graphs.clear()
    torch.cuda.synchronize()

    cpu = None
    n_cpu = args.cpu_layers if args.cpu_layers >= 0 else (L if T == 1 else 1)
    if n_cpu > 0:
        cpu = cpu_baseline(cfg, min(n_cpu, L), dense_q4=args.dense_q4)

    line = {
        "metric": "MoE-layer decode tokens/s and achieved HBM GB/s (% of peak), 1 GPU",
        "value": round(tokens_per_s, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"int{cfg.bits} weights x {cfg.act} activations, fp32 accumulate",
        "data": "synthetic",
        "config": {
            "workload": describe(cfg, args.dense_q4),
            "tokens_per_step": T,
            "layers": L,
            "input_rotations": N_ROTATE,
            "launch": mode,
            "unique_experts_per_layer_mean": round(float(uniq.mean()), 2),
        },
        "hbm_gbps": round(gbps, 1),
        "hbm_frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": int(step_bytes),
        "mfma_tflops": round(tflops, 2),
        "mfma_frac_of_peak": round(tflops / MFMA_PEAK_TFLOPS, 4),
        "algorithmic_flops_per_step": int(step_flops),
        "us_per_layer": round(ms_per_step * 1e3 / L, 3),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    line["config"]["bits"] = cfg.bits
    print(json.dumps(line), flush=True)


def check_chain_status(moe, d, ws, what):
    """Fail the run if the persistent chain's status word reports an expired
    wait between workgroups (that call's results would be invalid)."""
    import torch
    off = moe.moe_chain_status(d, ws) - ws.data_ptr()
    torch.cuda.synchronize()
    st = int(ws[off:off + 4].view(torch.int32).item())
    if st != 0:
        raise SystemExit(f"chain status word {st:#x} after the {what}: a bounded wait expired")


def describe(cfg, dense_q4=False):
    return (f"{cfg.name}: hidden {cfg.hidden}, {cfg.n_experts} experts top-{cfg.top_k}, "
            f"inter {cfg.inter}, shared {cfg.shared_inter} (sigmoid gate), int{cfg.bits} "
            f"group {cfg.group}, {cfg.act} activations, {cfg.n_tokens} token(s), "
            f"{cfg.layers} chained layer(s)"
            + (", router and shared gate int4 group 64" if dense_q4 else ""))


def chain_kernel_name(cfg, dense_q4=False):
    """The instantiation of the persistent chain kernel that runs this
    configuration (as the library dispatches it; the last argument selects
    the 4-bit dense router rows)."""
    shared = "true" if cfg.shared_inter else "false"
    epl = 4 if cfg.n_experts <= 256 else 8
    spec = (cfg.n_experts, cfg.top_k) in ((256, 8), (512, 10)) and cfg.shared_inter
    ec, kc = (cfg.n_experts, cfg.top_k) if spec else (0, 0)
    dq = "true" if dense_q4 else "false"
    return (f"chain_kernel<4, 8, {shared}, {cfg.inter}, {cfg.shared_inter or 512}, {epl}, {ec}, "
            f"{kc}, {dq}>")


def chain_roofline(cfg, load_input, forward, bytes_per_rot, flops, reps=64, dense_q4=False):
    """Average duration of one moe_chain_forward launch (for batch-1 bf16
    int4 decode this is the single persistent kernel that streams every
    layer's weights), timed with HIP events on the launch stream around the
    library call only (the input copy before it is outside the interval).
    The stream is first held by a device-side sleep so that all launches are
    queued before the first one runs and the intervals contain no host gaps."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    torch.cuda.synchronize()
    torch.cuda._sleep(50_000_000)
    for i in range(reps):
        load_input(i % N_ROTATE)
        evs[i][0].record()
        forward()
        evs[i][1].record()
    torch.cuda.synchronize()
    durs = [a.elapsed_time(b) * 1e-3 for a, b in evs]
    avg_s = sum(durs) / len(durs)
    srt = sorted(durs)
    pct = {q: srt[min(len(srt) - 1, int(q / 100 * len(srt)))] * 1e6 for q in (10, 50, 90)}
    avg_b = sum(bytes_per_rot[i % N_ROTATE] for i in range(reps)) / reps
    achieved = avg_b / avg_s / 1e9
    persistent = cfg.n_tokens == 1 and cfg.act == "bf16" and cfg.bits == 4
    # (the counter summaries in profiles/ are of the fp32-router kernel)
    traffic = measured_traffic(cfg) if persistent and not dense_q4 else None
    if flops / avg_b > MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9):
        # above the ridge point (a prefill chunk): the matrix cores bound it
        tf = flops / avg_s / 1e12
        return {"bound": "mfma",
                "kernel": "moe_chain_forward: all kernels of one chain step (bf16 MFMA grouped "
                          "GEMMs, fp32 accumulate)",
                "achieved": round(tf, 2), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tf / MFMA_PEAK_TFLOPS, 4), "traffic": None,
                "avg_launch_us": round(avg_s * 1e6, 3),
                "launch_us_p10_p50_p90": [round(pct[10], 3), round(pct[50], 3),
                                          round(pct[90], 3)],
                "flops_per_launch": int(flops), "bytes_per_launch": int(avg_b),
                "launches": reps}
    return {"bound": "hbm",
            "kernel": (f"{chain_kernel_name(cfg, dense_q4)}: the persistent decode-chain kernel, "
                       f"one launch per {cfg.layers}-layer step" if persistent else
                       "moe_chain_forward: all kernels of one chain step"),
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
            "avg_launch_us": round(avg_s * 1e6, 3),
            "launch_us_p10_p50_p90": [round(pct[10], 3), round(pct[50], 3), round(pct[90], 3)],
            "bytes_per_launch": int(avg_b),
            "launches": reps}


def measured_traffic(cfg):
    """HBM bytes per launch of the decode-chain kernel from the hardware-counter
    summary in profiles/ (FETCH_SIZE + WRITE_SIZE, calibrated on a copy of
    known size), or None when there is none for this workload or the kernel's
    sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"chain_kernel_{cfg.name}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path, encoding="utf-8"):
        if " = " in line:
            key, val = line.strip().split(" = ", 1)
            fields[key] = val
    h = hashlib.sha256()
    for f in ("chain.hip", "decode_common.h"):
        with open(os.path.join(ROOT, "int4_group_quantized_moe_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if fields.get("kernel_source_sha256") != h.hexdigest():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(cfg, n_layers, dense_q4=False):
    """The C++ fp64 oracle, as it is, on a bounded sample: the first n_layers
    layers of the same chain for the bench's first input (the inputs of the
    selected experts are generated by an untimed first pass), on every host
    thread OpenMP is given, then on one thread for the first layer; tokens/s
    scaled to the full chain."""
    import numpy as np

    import oracle
    import synth
    from oracle import cpp
    O = cpp.default()
    inputs = [oracle.LayerInputs(cfg, l, dense_q4=dense_q4) for l in range(n_layers)]
    x0 = synth.activations(cfg)

    def run(layers):
        x = x0.astype(np.float64)
        for l in range(layers):
            xh = O.chain_prologue(x, cfg.rms_eps, cfg.act)
            r = oracle.oracle_layer(inputs[l], xh)
            x = O.chain_epilogue(x, r["out"], cfg.act)
        return x

    run(n_layers)                         # draws and caches the routed experts' inputs
    threads = O.num_threads()
    reps = 0
    t0 = time.perf_counter()
    while True:                           # repeat the sample for about 10 s of CPU work
        run(n_layers)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or reps >= 64:
            break
    per_layer = dt / (reps * n_layers)
    tokens_per_s = cfg.n_tokens / (per_layer * cfg.layers)
    per_layer_1t = None
    if per_layer * threads < 30.0:        # keep the one-thread figure within the sample budget
        try:
            O.set_num_threads(1)
            t0 = time.perf_counter()
            run(1)
            per_layer_1t = time.perf_counter() - t0
        finally:
            O.set_num_threads(threads)
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo", encoding="utf-8"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(tokens_per_s, 6), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{cfg.n_tokens} token(s) through layers 0..{n_layers - 1} of {cfg.layers}, "
                      f"{reps} time(s) (C++ fp64 oracle, OpenMP, {threads} threads; {dt:.2f}s); "
                      f"scaled to the {cfg.layers}-layer chain",
            "seconds_per_layer": round(per_layer, 5),
            "seconds_per_layer_1_thread": round(per_layer_1t, 5) if per_layer_1t else None,
            "speedup_vs_1_thread": round(per_layer_1t / per_layer, 2) if per_layer_1t else None,
            "cpu_model": model, "nproc": os.cpu_count()}


def pool_bench(args):
    """Batch-1 decode through an expert slot pool (include/moe_pool.h): the
    80B-A3B shape, the whole 48-layer pack in pinned host memory, and a slab
    of pool_frac x (48 x 512) slots in HBM.  Per layer: RMSNorm and the
    router on the GPU, the routing read back, moe_pool_require (copies of the
    missed blobs over the host link), the experts on the pool's slab.  A step
    is one token through all layers; warm-up tokens fill the pool first.
    Each (token, layer) reads its own independent N(0, 1) input row rather
    than the previous layer's residual: with random weights the residual
    stream of every token converges to one direction after a few layers (the
    group biases give each expert an input-independent output), so deep
    layers would route every token alike and the hit rate would measure that
    artefact.  Expert popularity is set by an additive Zipf(s) router bias: s = 0 is
    uniform routing, s = 1.1 concentrates each layer on a few experts; the
    headline is s = 0.5.  Reported: tokens/s, the hit rate (the pages quote
    43-70%) and a sweep over skews and pool sizes."""
    import numpy as np
    import torch

    import int4_group_quantized_moe_amd as moe
    import synth
    import workload
    from synth import configs
    torch.cuda.set_device(0)
    moe.lib()
    cfg = configs.BATCHED_80B.with_(name="pool_80b", n_tokens=1)
    if args.layers:
        cfg = cfg.with_(layers=args.layers)
    L, E, k, H = cfg.layers, cfg.n_experts, cfg.top_k, cfg.hidden
    t0 = time.time()
    wl = workload.Workload(cfg)
    d = wl.desc
    stride = wl.stride
    pack = torch.empty(L * E * stride, dtype=torch.uint8, pin_memory=True)
    pack.copy_(wl.slab)
    torch.cuda.synchronize()
    del wl.slab                      # the pack lives on the host only
    torch.cuda.empty_cache()
    print(f"# pack of {pack.numel() / 1e9:.1f} GB in pinned host memory ({time.time() - t0:.1f}s)",
          file=sys.stderr, flush=True)
    ws = wl.workspace()
    idx = torch.empty(1, k, dtype=torch.int32, device="cuda")
    wt = torch.empty(1, k, dtype=torch.float32, device="cuda")
    gam = torch.empty(1, dtype=torch.float32, device="cuda")
    n_rows = 4096            # distinct (token, layer) inputs before a repeat
    xs = workload.act_tensor(cfg, synth.activations(cfg, variant=1, n_tokens=n_rows))
    xh, out = torch.empty_like(xs[:1]), torch.empty_like(xs[:1])
    wsg = [wl.shared[l][wl.slayout.shared_gate_offset:
                        wl.slayout.shared_gate_offset + 4 * H].view(torch.float32)
           for l in range(L)]

    def set_skew(zs):
        for l in range(L):
            b = synth.router_bias(cfg.with_(zipf_s=zs), l) if zs else np.zeros(E, np.float32)
            wl.router_bias[l].copy_(torch.from_numpy(b))

    def run(frac, steps, warm):
        n_slots = max(k, int(frac * L * E))
        pslab = torch.empty(n_slots * stride, dtype=torch.uint8, device="cuda")
        tables = torch.zeros(L, E, dtype=torch.int32, device="cuda")
        pool = moe.MoePool(d, L, n_slots, pack, stride, pslab, tables)

        def token(s):
            for l in range(L):
                r = (s * L + l) % n_rows
                rw, rb, _, sh = wl.layer_args(l)
                moe.moe_residual_rmsnorm(d, xs[r:r + 1], None, xh)
                moe.moe_router_topk(d, xh, rw, rb, wsg[l], idx, wt, gam, ws)
                need = sorted(set(idx.cpu().numpy().ravel().tolist()))   # synchronises
                pool.require(l, need)
                moe.moe_experts_forward(d, xh, idx, wt, gam, pslab, tables[l], sh, out, ws)

        for s in range(warm):
            token(s)
        torch.cuda.synchronize()
        st0 = pool.stats()
        t1 = time.perf_counter()
        for s in range(warm, warm + steps):
            token(s)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t1
        st1 = pool.stats()
        look = st1["lookups"] - st0["lookups"]
        hits = st1["hits"] - st0["hits"]
        res = {"pool_frac": frac, "slots": n_slots, "tokens_per_s": round(steps / dt, 2),
               "hit_rate": round(hits / max(look, 1), 4),
               "misses_per_layer": round((look - hits) / (steps * L), 2),
               "mib_copied_per_token": round((st1["bytes_copied"] - st0["bytes_copied"])
                                             / steps / 2 ** 20, 1)}
        assert torch.isfinite(out.float()).all()
        del pool, pslab, tables
        torch.cuda.empty_cache()
        return res, dt / steps

    sweep = []
    main_res = s_per_tok = None
    for zs in (0.5, 0.0, 1.1):
        set_skew(zs)
        for frac in (0.25, 0.1, 0.5):
            headline = zs == 0.5 and frac == args.pool_frac
            r, spt = run(frac, args.steps if headline else max(8, args.steps // 2), args.warmup)
            r["zipf_s"] = zs
            sweep.append(r)
            print(f"# zipf {zs} pool {frac}: {r}", file=sys.stderr, flush=True)
            if headline:
                main_res, s_per_tok = r, spt
    if main_res is None:
        main_res, s_per_tok = sweep[0], 1.0 / sweep[0]["tokens_per_s"]
    line = {
        "metric": "MoE decode through an expert slot pool: tokens/s and hit rate, 1 GPU",
        "value": main_res["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(s_per_tok * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int4 weights x bf16 activations, fp32 accumulate", "data": "synthetic",
        "config": {"workload": (f"pool_80b: hidden {H}, {E} experts top-{k} with a Zipf(0.5) "
                                f"router bias, {L} layers, 1 token, an independent input per layer; the pack "
                                f"({pack.numel() / 1e9:.1f} GB) in pinned host memory, "
                                f"{main_res['slots']} HBM slots"),
                   "pool_frac": main_res["pool_frac"], "zipf_s": 0.5},
        "hit_rate": main_res["hit_rate"], "pages_hit_rate_range": [0.43, 0.70],
        "misses_per_layer": main_res["misses_per_layer"],
        "mib_copied_per_token": main_res["mib_copied_per_token"],
        "sweep": sweep, "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def mixer_bench(args):
    """One decode step of a token mixer (Gated DeltaNet or gated GQA
    attention) per step, inputs rotating over 8 steps' worth; HBM-bound, so
    reported as algorithmic bytes per step over the step time against 8 TB/s."""
    import numpy as np
    import torch

    import int4_group_quantized_moe_amd as moe
    from oracle import mixer_oracle as mx
    from synth import device as sd
    from synth import mixers as sm
    torch.cuda.set_device(0)
    moe.lib()
    stream = torch.cuda.current_stream().cuda_stream

    def bf16(x):
        return torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda().to(torch.bfloat16)

    def uniform(spec):
        seed, t, layer, n, lo, hi = spec
        buf = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        sd.fill_uniform_bf16(seed, t, layer, 0xFFFFFE, n, lo, hi, buf, stream)
        return buf

    if args.config in sm.GDN_CONFIGS:
        cfg = sm.GDN_CONFIGS[args.config]
        B, Hk, Hv, dk, dv = cfg.n_seqs, cfg.n_k_heads, cfg.n_v_heads, cfg.d_k, cfg.d_v
        d = moe.make_gdn_desc(B, Hk, Hv, dk, dv)
        state = uniform(sm.gdn_state_spec(cfg)).float().view(B, Hv, dv, dk)
        ins = [sm.gdn_inputs(cfg, r) for r in range(N_ROTATE)]
        dev = [(bf16(i["q"]), bf16(i["k"]), bf16(i["v"]), torch.from_numpy(i["g"]).cuda(),
                torch.from_numpy(i["beta"]).cuda()) for i in ins]
        out = torch.empty(B, Hv, dv, dtype=torch.bfloat16, device="cuda")

        def step(s):
            q, k, v, g, b = dev[s % N_ROTATE]
            moe.moe_gdn_decode(d, q, k, v, g, b, state, out)

        step_bytes = B * Hv * dv * dk * 8 + B * (2 * Hk * dk * 2 + 2 * Hv * dv * 2 + Hv * 8)
        kernel = f"gdn_decode_kernel<{dk}>"
        workload = (f"{cfg.name}: Gated DeltaNet decode step, {B} sequence(s), {Hk} q/k heads, "
                    f"{Hv} v heads, d_k {dk}, d_v {dv}, fp32 state")

        def cpu_sample():
            i0 = ins[0]
            S = sm.gdn_state(cfg, seqs=[0]).astype(np.float64)
            t0 = time.perf_counter()
            reps = 0
            while True:
                mx.gdn_step(S, i0["q"][:1], i0["k"][:1], i0["v"][:1], i0["g"][:1], i0["beta"][:1])
                reps += 1
                if time.perf_counter() - t0 > 5.0:
                    break
            dt = (time.perf_counter() - t0) / reps
            return 1.0 / dt, f"one sequence's step (all {Hv} heads), numpy float64, {reps} reps"
    else:
        cfg = sm.ATT_CONFIGS[args.config]
        B, Hq, Hkv, D, N = cfg.n_seqs, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.max_len
        d = moe.make_attn_desc(B, Hq, Hkv, D, N)
        K = uniform(sm.attn_cache_spec(cfg, "k"))
        V = uniform(sm.attn_cache_spec(cfg, "v"))
        lengths = sm.attn_lengths(cfg)
        lens = torch.from_numpy(lengths).cuda()
        qs = [sm.attn_query(cfg, r) for r in range(N_ROTATE)]
        dev = [(bf16(x["q"]), bf16(x["gate"])) for x in qs]
        out = torch.empty(B, Hq, D, dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(max(moe.moe_attn_workspace_bytes(d), 256), dtype=torch.uint8,
                         device="cuda")

        def step(s):
            q, g = dev[s % N_ROTATE]
            moe.moe_attn_decode(d, q, g, K, V, lens, out, ws)

        step_bytes = int(lengths.astype(np.int64).sum()) * Hkv * D * 2 * 2 + B * Hq * D * 2 * 3
        kernel = f"attn_chunk_kernel<{D}, {8 if Hq // Hkv <= 8 else 16}> + attn_merge_kernel<{D}>"
        workload = (f"{cfg.name}: gated GQA attention decode, {B} sequence(s), {Hq} q heads, "
                    f"{Hkv} kv heads, head dim {D}, cache lengths "
                    f"{'ragged up to' if cfg.ragged else ''} {N} (bf16 cache)")

        def cpu_sample():
            b = int(np.argmax(lengths))
            n = int(lengths[b])
            kv = [(sm.attn_cache(cfg, "k", b, c, n), sm.attn_cache(cfg, "v", b, c, n))
                  for c in range(Hkv)]
            t0 = time.perf_counter()
            reps = 0
            while True:
                mx.attn_decode(qs[0]["q"][b:b + 1], qs[0]["gate"][b:b + 1],
                               lambda i, c, nn: kv[c], [n], Hkv)
                reps += 1
                if time.perf_counter() - t0 > 5.0:
                    break
            dt = (time.perf_counter() - t0) / reps
            return 1.0 / dt, f"sequence {b} ({n} positions, all heads), numpy float64, {reps} reps"

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda._sleep(20_000_000)             # queue every launch before the first runs
    for s in range(args.steps):
        evs[s][0].record()
        step(s)
        evs[s][1].record()
    torch.cuda.synchronize()
    durs = sorted(a.elapsed_time(b) for a, b in evs)
    ms = sum(durs) / len(durs)
    gbps = step_bytes / (ms / 1e3) / 1e9
    cpu = None
    if args.cpu_layers != 0:
        import os as _os
        rate, sample = cpu_sample()
        cpu = {"value": round(rate, 3), "unit": "sequence-steps/s", "cores": 1, "kind": "oracle",
               "sample": sample, "nproc": _os.cpu_count()}
    line = {
        "metric": "token-mixer decode step: sequences/s and achieved HBM GB/s (% of peak), 1 GPU",
        "value": round(cfg.n_seqs / (ms / 1e3), 3),
        "unit": "sequence-steps/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 activations and cache, fp32 state and arithmetic",
        "data": "synthetic",
        "config": {"workload": workload},
        "hbm_gbps": round(gbps, 1),
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": None, "avg_launch_us": round(ms * 1e3, 3),
                     "launch_us_p10_p50_p90": [round(durs[int(q / 100 * (len(durs) - 1))] * 1e3, 3)
                                               for q in (10, 50, 90)],
                     "bytes_per_launch": int(step_bytes)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
