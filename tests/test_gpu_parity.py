"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Every case prints its name before touching the GPU.  Inputs are seeded
synthetic workloads (synth); the oracle reads the generator's logical arrays
on the host, never the packed slab.
"""
import gc

import numpy as np
import pytest

import oracle
import synth
from synth import configs
from tests.parity import check_out, check_routing, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int4_group_quantized_moe_amd as moe
    from synth import device as sd
    moe.lib()          # must load: there is no fallback path
    sd.lib()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _moe():
    import int4_group_quantized_moe_amd as moe
    return moe


def _wl():
    import workload
    return workload


def _free():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def chain_status(d, ws) -> int:
    """The persistent chain's status word in ws (bit 0: a bounded wait
    between workgroups expired).  Synchronises."""
    moe = _moe()
    off = moe.moe_chain_status(d, ws) - ws.data_ptr()
    torch.cuda.synchronize()
    return int(ws[off:off + 4].view(torch.int32).item())


def chain(d, L, x, w_args, x_hat, out, ws):
    """moe_chain_forward, then a check that no bounded wait expired."""
    moe = _moe()
    moe.moe_chain_forward(d, L, x, *w_args, x_hat, out, ws)
    assert chain_status(d, ws) == 0, "chain status word set: a bounded wait expired"


# ---------------------------------------------------------------------------
# generator and packer


@pytest.mark.parametrize("cfgname,expert", [("tiny", 3), ("decode_80b", 77), ("batched_80b_int8", 5),
                                            ("decode_35b", synth.SHARED_EXPERT)])
def test_device_fill_matches_host_generator(cfgname, expert):
    from synth import device as sd
    cfg = configs.CONFIGS[cfgname]
    say(f"[fill] {cfgname} expert {expert}")
    H, G = cfg.hidden, cfg.group
    I = cfg.shared_inter if expert == synth.SHARED_EXPERT else cfg.inter
    qg = torch.empty(1, I, H, dtype=torch.uint8, device="cuda")
    qu, qd = torch.empty_like(qg), torch.empty(1, H, I, dtype=torch.uint8, device="cuda")
    sbg = torch.empty(1, 2, I, H // G, dtype=torch.int16, device="cuda")
    sbu, sbd = torch.empty_like(sbg), torch.empty(1, 2, H, I // G, dtype=torch.int16, device="cuda")
    sd.fill_experts(cfg, 2, expert, 1, I, qg, qu, qd, sbg, sbu, sbd,
                    torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = synth.expert_arrays(cfg, 2, expert)
    assert np.array_equal(qg[0].cpu().numpy(), ref["qg"])
    assert np.array_equal(qu[0].cpu().numpy(), ref["qu"])
    assert np.array_equal(qd[0].cpu().numpy(), ref["qd"])
    for t, (s, b) in ((sbg, ("sg", "bg")), (sbu, ("su", "bu")), (sbd, ("sd", "bd"))):
        got = t[0].cpu().numpy().view(np.uint16)
        assert np.array_equal(got[0], ref[s]) and np.array_equal(got[1], ref[b])


@pytest.mark.parametrize("cfgname", ["tiny", "decode_80b", "batched_80b_int8"])
def test_device_packer_matches_host_packer(cfgname):
    moe, wl = _moe(), _wl()
    cfg = configs.CONFIGS[cfgname]
    say(f"[pack] {cfgname}")
    d = wl.desc_for(cfg)
    w = wl.Workload(cfg, n_layers=1, batch=8)
    L = w.layout
    for e in (0, cfg.n_experts - 1):
        a = synth.expert_arrays(cfg, 0, e)
        host = np.zeros(L.blob_bytes, np.uint8)
        moe.moe_pack_expert(d, cfg.inter, a["qg"], a["qu"], a["qd"],
                            np.stack([a["sg"], a["bg"]]), np.stack([a["su"], a["bu"]]),
                            np.stack([a["sd"], a["bd"]]), None, host)
        slot = int(w.slot_tables_np[0, e])
        dev = w.slab[slot * w.stride: slot * w.stride + L.blob_bytes].cpu().numpy()
        assert np.array_equal(dev, host), e
    a = synth.expert_arrays(cfg, 0, synth.SHARED_EXPERT)
    host = np.zeros(w.slayout.shared_bytes, np.uint8)
    moe.moe_pack_expert(d, cfg.shared_inter, a["qg"], a["qu"], a["qd"],
                        np.stack([a["sg"], a["bg"]]), np.stack([a["su"], a["bu"]]),
                        np.stack([a["sd"], a["bd"]]), synth.shared_gate_weight(cfg, 0), host)
    assert np.array_equal(w.shared[0].cpu().numpy(), host)
    del w
    _free()


# ---------------------------------------------------------------------------
# router


@pytest.mark.parametrize("cfgname", ["tiny", "decode_35b", "decode_80b", "batched_80b",
                                     "prefill_35b"])
def test_router_topk_parity(cfgname):
    moe, wl = _moe(), _wl()
    cfg = configs.CONFIGS[cfgname]
    say(f"[router] {cfgname} T={cfg.n_tokens}")
    d = wl.desc_for(cfg)
    T, E, k, H = cfg.n_tokens, cfg.n_experts, cfg.top_k, cfg.hidden
    x_np = synth.activations(cfg)
    if cfg.act == "bf16":   # router input of a chained layer: a normalised, stored x_hat
        x_np = oracle.chain_prologue(x_np, cfg.rms_eps, "bf16").astype(np.float32)
    x = wl.act_tensor(cfg, x_np)
    Wr = synth.router_weight(cfg, 0)
    rb = synth.router_bias(cfg, 0)
    wsg = synth.shared_gate_weight(cfg, 0)
    Wr_d = torch.from_numpy(Wr).cuda()
    rb_d = torch.from_numpy(rb).cuda() if rb is not None else None
    wsg_d = torch.from_numpy(wsg).cuda()
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    gam = torch.empty(T, dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.moe_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    moe.moe_router_topk(d, x, Wr_d, rb_d, wsg_d, idx, w, gam, ws)
    torch.cuda.synchronize()
    l, ridx, rw, gap = oracle.route(x_np.astype(np.float64), Wr, rb, k)
    ref = {"logits": l, "idx": ridx, "w": rw, "gap": gap}
    _, _, n_ties = check_routing(idx.cpu().numpy(), w.cpu().numpy(), ref, k, gam.cpu().numpy(),
                                 oracle.shared_gate(x_np.astype(np.float64), wsg))
    say(f"  tokens with gap < 1e-5: {n_ties}")


# ---------------------------------------------------------------------------
# whole layer


def run_layer(w, cfg, x, i=0, desc=None):
    moe = _moe()
    d = desc or w.desc
    out = torch.empty_like(x)
    ws = w.workspace(d)
    rw, rb, st, sh = w.layer_args(i)
    moe.moe_layer_forward(d, x, rw, rb, w.slab, st, sh, out, ws)
    pi, pw, pg = moe.moe_workspace_routing(d, ws)
    T, k = d.n_tokens, d.top_k
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    wt = torch.empty(T, k, dtype=torch.float32, device="cuda")
    g = torch.empty(T, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    # copy the routing out of the workspace (device addresses inside ws)
    base = ws.data_ptr()
    idx.copy_(ws[pi - base: pi - base + 4 * T * k].view(torch.int32).view(T, k))
    wt.copy_(ws[pw - base: pw - base + 4 * T * k].view(torch.float32).view(T, k))
    g.copy_(ws[pg - base: pg - base + 4 * T].view(torch.float32))
    torch.cuda.synchronize()
    return out, idx, wt, g


def check_layer(cfg, layer, x_hat_np, out, idx, wt, g, what):
    inp = oracle.LayerInputs(cfg, layer)
    ref = oracle.oracle_layer(inp, x_hat_np.astype(np.float64))
    use_idx, use_w, n_ties = check_routing(idx.cpu().numpy(), wt.cpu().numpy(), ref, cfg.top_k,
                                           g.cpu().numpy(), ref["gamma"])
    if n_ties:
        ref = oracle.oracle_layer(inp, x_hat_np.astype(np.float64), routing=(use_idx, use_w))
    return check_out(out.float().cpu().numpy(), ref["out"], cfg.act, what)


def test_tiny_layer_parity():
    moe, wl = _moe(), _wl()
    cfg = configs.TINY
    say("[layer] tiny fp32 T=4")
    w = wl.Workload(cfg, n_layers=1)
    x_np = synth.activations(cfg)
    x = wl.act_tensor(cfg, x_np)
    out, idx, wt, g = run_layer(w, cfg, x)
    check_layer(cfg, 0, x_np, out, idx, wt, g, "tiny")
    # router + experts called separately give the same bits
    d = w.desc
    ws = w.workspace()
    rw, rb, st, sh = w.layer_args(0)
    idx2 = torch.empty_like(idx)
    w2 = torch.empty_like(wt)
    g2 = torch.empty_like(g)
    wsg = sh[w.slayout.shared_gate_offset: w.slayout.shared_gate_offset + 4 * cfg.hidden].view(torch.float32)
    moe.moe_router_topk(d, x, rw, rb, wsg, idx2, w2, g2, ws)
    out2 = torch.empty_like(out)
    moe.moe_experts_forward(d, x, idx2, w2, g2, w.slab, st, sh, out2, ws)
    torch.cuda.synchronize()
    assert torch.equal(idx2, idx) and torch.equal(w2, wt) and torch.equal(g2, g)
    assert torch.equal(out2, out)
    del w
    _free()


@pytest.mark.parametrize("cfgname,check_layers", [("decode_35b", (0, 1, 19, 39)),
                                                  ("decode_80b", (0, 1, 30, 47))])
def test_decode_chain_parity(cfgname, check_layers):
    """Batch-1 decode through every layer of the chain, teacher-forced: the
    chain entry point is called one layer at a time (the kernels the benchmark
    runs), and layer l of the oracle takes the GPU's own x_l / x_hat_l."""
    moe, wl = _moe(), _wl()
    cfg = configs.CONFIGS[cfgname]
    say(f"[chain] {cfgname}: building {cfg.layers} layers")
    w = wl.Workload(cfg)
    d = w.desc
    T, k = 1, cfg.top_k
    x0_np = synth.activations(cfg)
    x = wl.act_tensor(cfg, x0_np)
    xh = torch.empty_like(x)
    out = torch.empty_like(x)
    ws = w.workspace()
    pi, pw, pg = moe.moe_workspace_routing(d, ws)
    base = ws.data_ptr()
    for i in range(cfg.layers):
        checking = i in check_layers
        x_before = x.clone() if checking else None
        rw, rb, st, sh = w.layer_args(i)
        moe.moe_chain_forward(d, 1, x, rw, rb, w.slab, st, sh, w.shared_stride, xh, out, ws)
        if not checking:
            continue
        say(f"  layer {i}")
        assert chain_status(d, ws) == 0
        xb = wl.to_f64(x_before)
        xh_ref = oracle.chain_prologue(xb, cfg.rms_eps, cfg.act)
        assert np.all(np.abs(wl.to_f64(xh) - xh_ref) <= np.abs(xh_ref) * 2.0 ** -7), "rmsnorm"
        idx = ws[pi - base: pi - base + 4 * T * k].view(torch.int32).view(T, k)
        wt = ws[pw - base: pw - base + 4 * T * k].view(torch.float32).view(T, k)
        g = ws[pg - base: pg - base + 4 * T].view(torch.float32)
        check_layer(cfg, i, wl.to_f64(xh), out, idx, wt, g, f"{cfgname} layer {i}")
        x_ref = oracle.chain_epilogue(xb, wl.to_f64(out), cfg.act)
        assert np.array_equal(wl.to_f64(x), x_ref), "residual"
    torch.cuda.synchronize()
    # the whole chain in one call runs the same kernels: bit-equal residual
    say("  chain entry point, all layers")
    assert chain_status(d, ws) == 0
    xc = wl.act_tensor(cfg, x0_np)
    chain(d, cfg.layers, xc, (w.router_w, w.router_bias, w.slab, w.slot_tables, w.shared,
                              w.shared_stride), torch.empty_like(xc), torch.empty_like(xc), ws)
    assert torch.equal(xc, x)
    assert torch.isfinite(xc.float()).all()
    # and a single layer through moe_layer_forward equals the oracle as well
    rw, rb, st, sh = w.layer_args(0)
    xh0 = wl.act_tensor(cfg, oracle.chain_prologue(x0_np, cfg.rms_eps, cfg.act).astype(np.float32))
    o, idx, wt, g = run_layer(w, cfg, xh0, 0)
    check_layer(cfg, 0, wl.to_f64(xh0), o, idx, wt, g, f"{cfgname} layer_forward")
    del w
    _free()


def test_decode_massive_ties():
    """All-zero router: every logit ties, so top-k must take experts 0..k-1
    with weights 1/k (more ties than the fast candidate path holds)."""
    moe, wl = _moe(), _wl()
    cfg = configs.DECODE_35B
    say("[ties] zero router, E=256")
    w = wl.Workload(cfg, n_layers=1)
    w.router_w.zero_()
    x = wl.act_tensor(cfg, oracle.chain_prologue(synth.activations(cfg), 1e-6, "bf16").astype(np.float32))
    out, idx, wt, g = run_layer(w, cfg, x)
    assert idx[0].tolist() == list(range(cfg.top_k))
    assert torch.allclose(wt[0], torch.full_like(wt[0], 1.0 / cfg.top_k), rtol=1e-6)
    inp = oracle.LayerInputs(cfg, 0, overrides={"router_w": np.zeros((cfg.n_experts, cfg.hidden), np.float32)})
    ref = oracle.oracle_layer(inp, wl.to_f64(x))
    check_out(out.float().cpu().numpy(), ref["out"], cfg.act, "ties")
    del w
    _free()


@pytest.mark.parametrize("top_k", [4, 6])
def test_chain_other_top_k(top_k):
    """The persistent chain for a top-k it has no specialised kernel for (the
    kernel built with k and E read at run time), one layer against the
    oracle, and two chained layers equal to two single-layer calls."""
    moe, wl = _moe(), _wl()
    cfg = configs.DECODE_35B.with_(name=f"decode_35b_top{top_k}", top_k=top_k, layers=2)
    say(f"[chain] E=256 top-{top_k}")
    w = wl.Workload(cfg)
    d = w.desc
    x0_np = synth.activations(cfg)
    x = wl.act_tensor(cfg, x0_np)
    xh = torch.empty_like(x)
    out = torch.empty_like(x)
    ws = w.workspace()
    pi, pw, pg = moe.moe_workspace_routing(d, ws)
    base = ws.data_ptr()
    for i in range(cfg.layers):
        x_before = x.clone()
        rw, rb, st, sh = w.layer_args(i)
        chain(d, 1, x, (rw, rb, w.slab, st, sh, w.shared_stride), xh, out, ws)
        idx = ws[pi - base: pi - base + 4 * top_k].view(torch.int32).view(1, top_k)
        wt = ws[pw - base: pw - base + 4 * top_k].view(torch.float32).view(1, top_k)
        g = ws[pg - base: pg - base + 4].view(torch.float32)
        check_layer(cfg, i, wl.to_f64(xh), out, idx, wt, g, f"top-{top_k} layer {i}")
        assert np.array_equal(wl.to_f64(x), oracle.chain_epilogue(wl.to_f64(x_before), wl.to_f64(out), cfg.act))
    xc = wl.act_tensor(cfg, x0_np)
    chain(d, cfg.layers, xc, (w.router_w, w.router_bias, w.slab, w.slot_tables, w.shared,
                              w.shared_stride), torch.empty_like(xc), torch.empty_like(xc), ws)
    assert torch.equal(xc, x)
    del w
    _free()


@pytest.mark.parametrize("cfgname", ["decode_35b", "decode_80b"])
def test_chain_boundary_ties(cfgname):
    """The persistent chain when a few more than k experts tie for the top
    logit (fewer than 64 candidates, so the ranked-candidate path, not the
    argmax fallback): the set is the k lowest indices of the tied experts
    and every weight is 1/k."""
    moe, wl = _moe(), _wl()
    cfg = configs.CONFIGS[cfgname]
    E, H, k = cfg.n_experts, cfg.hidden, cfg.top_k
    say(f"[chain boundary ties] {cfgname}")
    w = wl.Workload(cfg, n_layers=1)
    rng = np.random.default_rng(11)
    tied = np.sort(rng.choice(E, size=k + 4, replace=False))
    x0_np = synth.activations(cfg)
    # a row along x_hat: its logit (about 0.05 H) is far above every other
    rw_np = w.router_w.view(E, H).cpu().numpy().copy()
    rw_np[tied] = (0.05 * oracle.chain_prologue(x0_np, cfg.rms_eps, cfg.act)).astype(np.float32)[0]
    w.router_w.view(E, H).copy_(torch.from_numpy(rw_np))
    d = w.desc
    x = wl.act_tensor(cfg, x0_np)
    xh = torch.empty_like(x)
    out = torch.empty_like(x)
    ws = w.workspace()
    pi, pw, pg = moe.moe_workspace_routing(d, ws)
    base = ws.data_ptr()
    rw, rb, st, sh = w.layer_args(0)
    chain(d, 1, x, (rw, rb, w.slab, st, sh, w.shared_stride), xh, out, ws)
    idx = ws[pi - base: pi - base + 4 * k].view(torch.int32)
    wt = ws[pw - base: pw - base + 4 * k].view(torch.float32)
    assert idx.tolist() == tied[:k].tolist()
    assert torch.allclose(wt, torch.full_like(wt, 1.0 / k), rtol=1e-6)
    inp = oracle.LayerInputs(cfg, 0, overrides={"router_w": rw_np})
    ref = oracle.oracle_layer(inp, wl.to_f64(xh))
    assert ref["idx"][0].tolist() == tied[:k].tolist()
    check_out(out.float().cpu().numpy(), ref["out"], cfg.act, "chain boundary ties")
    del w
    _free()


@pytest.mark.parametrize("cfgname", ["decode_35b", "decode_80b"])
def test_chain_massive_ties(cfgname):
    """The persistent chain on an all-zero router: every logit ties, so the
    expert set is 0..k-1 (k rounds of wave argmax, not the candidate path),
    reported in index order with weights 1/k."""
    moe, wl = _moe(), _wl()
    cfg = configs.CONFIGS[cfgname]
    say(f"[chain ties] zero router, {cfgname}")
    w = wl.Workload(cfg, n_layers=1)
    w.router_w.zero_()
    d = w.desc
    k = cfg.top_k
    x0_np = synth.activations(cfg)
    x = wl.act_tensor(cfg, x0_np)
    xh = torch.empty_like(x)
    out = torch.empty_like(x)
    ws = w.workspace()
    pi, pw, pg = moe.moe_workspace_routing(d, ws)
    base = ws.data_ptr()
    rw, rb, st, sh = w.layer_args(0)
    chain(d, 1, x, (rw, rb, w.slab, st, sh, w.shared_stride), xh, out, ws)
    idx = ws[pi - base: pi - base + 4 * k].view(torch.int32)
    wt = ws[pw - base: pw - base + 4 * k].view(torch.float32)
    assert idx.tolist() == list(range(k))
    assert torch.allclose(wt, torch.full_like(wt, 1.0 / k), rtol=1e-6)
    inp = oracle.LayerInputs(cfg, 0, overrides={"router_w": np.zeros((cfg.n_experts, cfg.hidden), np.float32)})
    ref = oracle.oracle_layer(inp, wl.to_f64(xh))
    check_out(out.float().cpu().numpy(), ref["out"], cfg.act, "chain ties")
    del w
    _free()


@pytest.mark.parametrize("cfgname", ["batched_80b", "batched_80b_int8"])
def test_batched_parity(cfgname):
    """64 tokens with a Zipf router bias: token->expert bucketing path."""
    moe, wl = _moe(), _wl()
    cfg = configs.CONFIGS[cfgname]
    say(f"[batched] {cfgname}")
    w = wl.Workload(cfg, n_layers=2)
    d = w.desc
    x = wl.act_tensor(cfg, synth.activations(cfg))
    xh = torch.empty_like(x)
    out = None
    for i in range(2):
        moe.moe_rmsnorm(d, x, out, xh)
        o, idx, wt, g = run_layer(w, cfg, xh, i)
        uniq = len(np.unique(idx.cpu().numpy()))
        say(f"  layer {i}: {uniq} unique experts")
        check_layer(cfg, i, wl.to_f64(xh), o, idx, wt, g, f"{cfgname} layer {i}")
        # token independence: a row of the batch equals the token alone
        d1 = wl.desc_for(cfg, n_tokens=1)
        for t in (0, 17, 63):
            o1, idx1, _, _ = run_layer(w, cfg, xh[t:t + 1].contiguous(), i, desc=d1)
            assert sorted(idx1[0].tolist()) == sorted(idx[t].tolist())
            a, b = o1[0].double(), o[t].double()
            rms = float(torch.sqrt(torch.mean(b * b)))
            assert float((a - b).abs().max()) <= 2e-2 * rms, t
        out = o
    del w
    _free()


@pytest.mark.parametrize("cfgname", ["batched_80b", "batched_80b_int8", "tiny_t40"])
def test_batched_chain_fused_epilogue(cfgname):
    """The chain entry point at 64 tokens fuses the residual add and the next
    layer's RMSNorm into the combine.  One layer must equal RMSNorm + layer
    forward + residual bit for bit; over two layers the fused x_hat must be
    the RMSNorm of x_1 (to one bf16 rounding: the sum of squares is taken in
    another order), and layer 1's output and residual bit-equal to the layer
    forward run on that x_hat.  Layer 1 is then checked against the oracle,
    teacher-forced on the fused x_hat."""
    moe, wl = _moe(), _wl()
    # tiny_t40: the tiny fp32 layer at 40 tokens (bucketed GEMV path, fp32 epilogue)
    cfg = (configs.TINY.with_(n_tokens=40, layers=2) if cfgname == "tiny_t40"
           else configs.CONFIGS[cfgname])
    say(f"[batched chain] {cfgname}")
    w = wl.Workload(cfg, n_layers=2)
    d = w.desc
    ws = w.workspace()
    x0 = wl.act_tensor(cfg, synth.activations(cfg))

    def run_chain(L):
        xc, xh, out = x0.clone(), torch.empty_like(x0), torch.empty_like(x0)
        chain(d, L, xc, (w.router_w, w.router_bias, w.slab, w.slot_tables, w.shared,
                         w.shared_stride), xh, out, ws)
        return xc, xh, out

    # one layer: RMSNorm, layer, residual through the separate entry points
    x1, _, out1 = run_chain(1)
    xb, xhb = x0.clone(), torch.empty_like(x0)
    moe.moe_residual_rmsnorm(d, xb, None, xhb)
    ob, _, _, _ = run_layer(w, cfg, xhb, 0)
    moe.moe_residual_rmsnorm(d, xb, ob, torch.empty_like(x0))
    torch.cuda.synchronize()
    assert torch.equal(out1, ob), "layer 0 output"
    assert torch.equal(x1, xb), "layer 0 residual"

    # two layers: x_hat after the call is layer 1's input, from the fused norm
    x2, xh1, out2 = run_chain(2)
    xr, xh_ref = x1.clone(), torch.empty_like(x0)
    moe.moe_rmsnorm(d, xr, None, xh_ref)
    torch.cuda.synchronize()
    a, b = wl.to_f64(xh1), wl.to_f64(xh_ref)
    assert np.all(np.abs(a - b) <= np.abs(b) * 2.0 ** -7), "fused rmsnorm"
    o1, idx, wt, g = run_layer(w, cfg, xh1, 1)
    xe = x1.clone()
    moe.moe_rmsnorm(d, xe, o1, torch.empty_like(x0))
    torch.cuda.synchronize()
    assert torch.equal(out2, o1), "layer 1 output"
    assert torch.equal(x2, xe), "layer 1 residual"
    check_layer(cfg, 1, wl.to_f64(xh1), o1, idx, wt, g, f"{cfgname} chain layer 1")
    del w
    _free()


def test_prefill_parity():
    """4096-token chunk, one layer through moe_layer_forward (the call the
    benchmark times): the routing of every token and every output row against
    the oracle (each expert dequantised once and applied to its bucket)."""
    moe, wl = _moe(), _wl()
    cfg = configs.PREFILL_35B
    say("[prefill] 4096 tokens, every row")
    w = wl.Workload(cfg, n_layers=1)
    x_np = oracle.chain_prologue(synth.activations(cfg), cfg.rms_eps, "bf16").astype(np.float32)
    x = wl.act_tensor(cfg, x_np)
    out, idx, wt, g = run_layer(w, cfg, x)
    counts = np.bincount(idx.cpu().numpy().ravel(), minlength=cfg.n_experts)
    say(f"  tokens per expert: mean {counts.mean():.1f} min {counts.min()} max {counts.max()}; "
        f"{int(np.sum(counts % 128 <= 64))} experts end in a tile of at most 64 rows")
    check_layer(cfg, 0, x_np, out, idx, wt, g, "prefill all 4096 tokens")
    del w
    _free()


def test_slot_permutation_invariance():
    """Experts moved to other slots (and the slot table with them) give the
    same bits: the analogue of cache-vs-disk identity."""
    moe, wl = _moe(), _wl()
    cfg = configs.DECODE_35B
    say("[slots] permutation invariance")
    outs = []
    for perm in (None, 99):
        w = wl.Workload(cfg, n_layers=1, permute_seed=perm)
        x = wl.act_tensor(cfg, synth.activations(cfg, n_tokens=16))
        r = []
        for T in (1, 16):
            d = wl.desc_for(cfg, n_tokens=T)
            r.append(run_layer(w, cfg, x[:T].contiguous(), 0, desc=d)[0].clone())
        outs.append(r)
        del w
        _free()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_determinism():
    moe, wl = _moe(), _wl()
    cfg = configs.DECODE_35B
    say("[determinism]")
    w = wl.Workload(cfg, n_layers=1)
    x = wl.act_tensor(cfg, synth.activations(cfg, n_tokens=32))
    for T in (1, 32):
        d = wl.desc_for(cfg, n_tokens=T)
        a = run_layer(w, cfg, x[:T].contiguous(), 0, desc=d)[0].clone()
        b = run_layer(w, cfg, x[:T].contiguous(), 0, desc=d)[0].clone()
        assert torch.equal(a, b)
    del w
    _free()


@pytest.mark.parametrize("T,k", [(1, 1), (4, 16), (8, 2), (9, 2), (63, 3), (64, 2), (65, 4),
                                 (100, 2)])
def test_edge_cases_tiny(T, k):
    """Ragged token counts around the small-batch/bucketed boundary and the
    64-token bucketing blocks, k = 1 and k = E."""
    wl = _wl()
    cfg = configs.TINY.with_(n_tokens=T, top_k=k)
    say(f"[edge] T={T} k={k}")
    w = wl.Workload(cfg, n_layers=1)
    x_np = synth.activations(cfg)
    x = wl.act_tensor(cfg, x_np)
    out, idx, wt, g = run_layer(w, cfg, x)
    check_layer(cfg, 0, x_np, out, idx, wt, g, f"T={T} k={k}")
    if k == cfg.n_experts:
        assert np.array_equal(np.sort(idx.cpu().numpy(), 1), np.tile(np.arange(k), (T, 1)))
    del w
    _free()


def test_zero_tokens_no_op():
    moe, wl = _moe(), _wl()
    cfg = configs.TINY
    say("[edge] T=0")
    w = wl.Workload(cfg, n_layers=1)
    d0 = wl.desc_for(cfg, n_tokens=0)
    out = torch.full((1, cfg.hidden), 7.0, device="cuda")
    rw, rb, st, sh = w.layer_args(0)
    moe.moe_layer_forward(d0, out, rw, rb, w.slab, st, sh, out, w.workspace())
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    del w
    _free()


def test_rmsnorm_parity():
    moe, wl = _moe(), _wl()
    say("[rmsnorm]")
    cfg = configs.DECODE_35B.with_(n_tokens=5)
    d = wl.desc_for(cfg)
    rng = np.random.default_rng(3)
    x_np = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(rng.standard_normal((5, 2048)) * 30))
    o_np = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(rng.standard_normal((5, 2048)) * 200))
    x = wl.act_tensor(cfg, x_np)
    o = wl.act_tensor(cfg, o_np)
    xh = torch.empty_like(x)
    moe.moe_rmsnorm(d, x, o, xh)
    torch.cuda.synchronize()
    x_ref = oracle.chain_epilogue(x_np, o_np, "bf16")
    assert np.array_equal(wl.to_f64(x), x_ref)
    xh_ref = oracle.chain_prologue(x_ref, cfg.rms_eps, "bf16")
    assert np.all(np.abs(wl.to_f64(xh) - xh_ref) <= np.abs(xh_ref) * 2.0 ** -7)


@pytest.mark.parametrize("T,k,bits", [(256, 2, 4), (300, 4, 4), (300, 3, 8), (1000, 16, 4)])
def test_grouped_mfma_path_tiny(T, k, bits):
    """bf16 batches of >= 256 tokens run the grouped MFMA GEMMs: ragged expert
    buckets (partial 128-row tiles), int4 and int8, k up to E."""
    wl = _wl()
    cfg = configs.TINY.with_(n_tokens=T, top_k=k, bits=bits, act="bf16")
    say(f"[mfma] tiny bf16 T={T} k={k} int{bits}")
    w = wl.Workload(cfg, n_layers=1)
    x_np = synth.activations(cfg)
    x = wl.act_tensor(cfg, x_np)
    out, idx, wt, g = run_layer(w, cfg, x)
    check_layer(cfg, 0, x_np, out, idx, wt, g, f"mfma T={T} k={k} int{bits}")
    del w
    _free()


def test_grouped_mfma_dynamic_range():
    """Tokens whose activation rows differ by 2^5 either way share the grouped
    GEMMs' 128-row tiles, so h (fp16 after one power-of-two scale per tile and
    128-column block) spans about 2^20 within a tile, and the partial rows
    (fp16 with a scale per 32-row x 64-column block) as much; each scale's
    rows are checked against the oracle on their own size.  (The tile's h scale
    keeps 11 significant bits for values within 2^-29 of the tile's largest:
    rows of one tile more than about 2^14 apart in input scale lose
    precision.)  The oracle takes the routing the GPU chose: at scaled logits
    the lower softmax weights are tiny and carry the logits' fp32 rounding,
    which the routing tests check at ordinary scale."""
    wl = _wl()
    cfg = configs.TINY.with_(n_tokens=300, top_k=3, bits=4, act="bf16")
    say("[mfma] tiny bf16 T=300 rows scaled by 2^-5, 1, 2^5")
    w = wl.Workload(cfg, n_layers=1)
    group = np.arange(cfg.n_tokens) % 3
    x_np = synth.activations(cfg).astype(np.float64) * (2.0 ** (5 * (group - 1)))[:, None]
    x = wl.act_tensor(cfg, x_np.astype(np.float32))
    out, idx, wt, g = run_layer(w, cfg, x)
    inp = oracle.LayerInputs(cfg, 0)
    ref = oracle.oracle_layer(inp, x_np, routing=(idx.cpu().numpy(),
                                                  wt.cpu().numpy().astype(np.float64)))
    got = out.float().cpu().numpy()
    for s in range(3):
        rows = group == s
        check_out(got[rows], ref["out"][rows], cfg.act, f"rows scaled by 2^{5 * (s - 1)}")
    del w
    _free()


@pytest.mark.parametrize("cfgname,T", [("batched_80b", 320), ("batched_80b_int8", 300)])
def test_grouped_mfma_path_80b(cfgname, T):
    """80B-shaped layer with a Zipf-skewed router (one bucket holds most tokens)
    through the grouped MFMA GEMMs; every output row against the oracle."""
    wl = _wl()
    cfg = configs.CONFIGS[cfgname].with_(n_tokens=T)
    say(f"[mfma] {cfgname} T={T}")
    w = wl.Workload(cfg, n_layers=1)
    x_np = oracle.chain_prologue(synth.activations(cfg), cfg.rms_eps, "bf16").astype(np.float32)
    x = wl.act_tensor(cfg, x_np)
    out, idx, wt, g = run_layer(w, cfg, x)
    counts = np.bincount(idx.cpu().numpy().ravel(), minlength=cfg.n_experts)
    say(f"  largest bucket {counts.max()} tokens, {np.count_nonzero(counts)} experts used")
    check_layer(cfg, 0, x_np, out, idx, wt, g, f"{cfgname} T={T} every row")
    # moe_layer_forward takes the activations' group sums from the router GEMM;
    # router + experts called separately compute them in their own kernel: the
    # same bits either way
    moe = _moe()
    d = w.desc
    ws = w.workspace()
    rw, rb, st, sh = w.layer_args(0)
    idx2, w2, g2 = torch.empty_like(idx), torch.empty_like(wt), torch.empty_like(g)
    wsg = sh[w.slayout.shared_gate_offset: w.slayout.shared_gate_offset + 4 * cfg.hidden].view(torch.float32)
    moe.moe_router_topk(d, x, rw, rb, wsg, idx2, w2, g2, ws)
    out2 = torch.empty_like(out)
    moe.moe_experts_forward(d, x, idx2, w2, g2, w.slab, st, sh, out2, ws)
    torch.cuda.synchronize()
    assert torch.equal(idx2, idx) and torch.equal(w2, wt) and torch.equal(g2, g)
    assert torch.equal(out2, out)
    del w
    _free()


@pytest.mark.parametrize("T,k", [(15, 2), (16, 2), (17, 3), (40, 16), (127, 4), (128, 2),
                                 (129, 5)])
def test_bf16_batch_thresholds(T, k):
    """bf16 batches around the MFMA router threshold (16 tokens; K split over
    logit planes below 1024 tokens) and the grouped-GEMM tile edges (128-row
    tiles; tiles of at most 64 rows split K between the wave rows).  Every
    bucket of at least 1 token runs on the grouped MFMA GEMMs."""
    wl = _wl()
    cfg = configs.TINY.with_(n_tokens=T, top_k=k, act="bf16")
    say(f"[thresholds] tiny bf16 T={T} k={k}")
    w = wl.Workload(cfg, n_layers=1)
    x_np = synth.activations(cfg)
    x = wl.act_tensor(cfg, x_np)
    out, idx, wt, g = run_layer(w, cfg, x)
    counts = np.bincount(idx.cpu().numpy().ravel(), minlength=cfg.n_experts)
    say(f"  bucket sizes {sorted(counts.tolist())}")
    check_layer(cfg, 0, x_np, out, idx, wt, g, f"thresholds T={T} k={k}")
    # same layer again: bitwise identical
    out2 = run_layer(w, cfg, x)[0]
    assert torch.equal(out, out2)
    del w
    _free()


@pytest.mark.parametrize("cfgname", ["batched_80b", "batched_80b_int8"])
def test_batched_deep_layers(cfgname):
    """The 64-token Zipf-routed chain through all 48 layers, one layer per
    chain call, teacher-forced at layers 0, 1, 24 and 47: the deep layers'
    routing concentrates on few experts, so their buckets are the largest."""
    moe, wl = _moe(), _wl()
    cfg = configs.CONFIGS[cfgname]
    say(f"[batched deep] {cfgname}: building {cfg.layers} layers")
    w = wl.Workload(cfg)
    d = w.desc
    ws = w.workspace()
    x = wl.act_tensor(cfg, synth.activations(cfg))
    xh, out = torch.empty_like(x), torch.empty_like(x)
    pi, pw, pg = moe.moe_workspace_routing(d, ws)
    base = ws.data_ptr()
    T, k = cfg.n_tokens, cfg.top_k
    for i in range(cfg.layers):
        x_before = x.clone() if i in (0, 1, 24, 47) else None
        rw, rb, st, sh = w.layer_args(i)
        chain(d, 1, x, (rw, rb, w.slab, st, sh, w.shared_stride), xh, out, ws)
        if x_before is None:
            continue
        torch.cuda.synchronize()
        idx = ws[pi - base: pi - base + 4 * T * k].view(torch.int32).view(T, k)
        wt = ws[pw - base: pw - base + 4 * T * k].view(torch.float32).view(T, k)
        g = ws[pg - base: pg - base + 4 * T].view(torch.float32)
        counts = np.bincount(idx.cpu().numpy().ravel(), minlength=cfg.n_experts)
        say(f"  layer {i}: {np.count_nonzero(counts)} unique experts, largest bucket "
            f"{counts.max()} tokens")
        xb = wl.to_f64(x_before)
        xh_ref = oracle.chain_prologue(xb, cfg.rms_eps, cfg.act)
        assert np.all(np.abs(wl.to_f64(xh) - xh_ref) <= np.abs(xh_ref) * 2.0 ** -7), "rmsnorm"
        check_layer(cfg, i, wl.to_f64(xh), out, idx, wt, g, f"{cfgname} layer {i}")
        assert np.array_equal(wl.to_f64(x), oracle.chain_epilogue(xb, wl.to_f64(out), cfg.act))
    del w
    _free()


@pytest.mark.parametrize("cfgname,T", [("decode_35b", 2), ("decode_35b", 5), ("decode_80b", 8),
                                       ("batched_80b_int8", 5), ("batched_80b", 3)])
def test_small_bf16_batches(cfgname, T):
    """bf16 batches of 2 to 8 tokens: the per-pair GEMV path (no bucketing),
    against the oracle, and each row equal to its token alone."""
    wl = _wl()
    cfg = configs.CONFIGS[cfgname].with_(n_tokens=T)
    say(f"[small batch] {cfgname} T={T} int{cfg.bits}")
    w = wl.Workload(cfg, n_layers=1)
    x_np = oracle.chain_prologue(synth.activations(cfg), cfg.rms_eps, "bf16").astype(np.float32)
    x = wl.act_tensor(cfg, x_np)
    out, idx, wt, g = run_layer(w, cfg, x)
    check_layer(cfg, 0, x_np, out, idx, wt, g, f"{cfgname} T={T}")
    d1 = wl.desc_for(cfg, n_tokens=1)
    for t in (0, T - 1):
        o1, idx1, _, _ = run_layer(w, cfg, x[t:t + 1].contiguous(), 0, desc=d1)
        assert sorted(idx1[0].tolist()) == sorted(idx[t].tolist())
    del w
    _free()


def test_int8_batch1_decode():
    """int8 codes at batch 1 (the three-kernel decode path with 8-bit codes)
    through moe_layer_forward and a two-layer chain, against the oracle."""
    moe, wl = _moe(), _wl()
    cfg = configs.BATCHED_80B_INT8.with_(n_tokens=1, layers=2)
    say("[int8 T=1] 80B shape, int8")
    w = wl.Workload(cfg)
    d = w.desc
    x0_np = synth.activations(cfg)
    xh0 = oracle.chain_prologue(x0_np, cfg.rms_eps, "bf16").astype(np.float32)
    out, idx, wt, g = run_layer(w, cfg, wl.act_tensor(cfg, xh0))
    check_layer(cfg, 0, xh0, out, idx, wt, g, "int8 T=1 layer_forward")
    ws = w.workspace()
    pi, pw, pg = moe.moe_workspace_routing(d, ws)
    base = ws.data_ptr()
    x = wl.act_tensor(cfg, x0_np)
    xh, o = torch.empty_like(x), torch.empty_like(x)
    for i in range(cfg.layers):
        xb = wl.to_f64(x)
        rw, rb, st, sh = w.layer_args(i)
        chain(d, 1, x, (rw, rb, w.slab, st, sh, w.shared_stride), xh, o, ws)
        torch.cuda.synchronize()
        k = cfg.top_k
        idx = ws[pi - base: pi - base + 4 * k].view(torch.int32).view(1, k)
        wt = ws[pw - base: pw - base + 4 * k].view(torch.float32).view(1, k)
        g = ws[pg - base: pg - base + 4].view(torch.float32)
        check_layer(cfg, i, wl.to_f64(xh), o, idx, wt, g, f"int8 T=1 chain layer {i}")
        assert np.array_equal(wl.to_f64(x), oracle.chain_epilogue(xb, wl.to_f64(o), cfg.act))
    del w
    _free()


@pytest.mark.parametrize("T,bits", [(20, 4), (70, 8), (9, 4)])
def test_bf16_bucketed_gemv_hidden_384(T, bits):
    """bf16 batches of more than 8 tokens whose hidden size (384) the grouped
    MFMA GEMMs do not take: every bucket on the bucketed GEMV kernels."""
    wl = _wl()
    cfg = configs.TINY.with_(n_tokens=T, hidden=384, act="bf16", bits=bits, top_k=3)
    say(f"[gemv H=384] bf16 T={T} int{bits}")
    w = wl.Workload(cfg, n_layers=1)
    x_np = synth.activations(cfg)
    x = wl.act_tensor(cfg, x_np)
    out, idx, wt, g = run_layer(w, cfg, x)
    check_layer(cfg, 0, x_np, out, idx, wt, g, f"H=384 T={T} int{bits}")
    del w
    _free()


@pytest.mark.parametrize("cfgname,T,hidden", [("batched_80b", 9, 2048), ("batched_80b", 33, 2048),
                                              ("batched_80b_int8", 47, 2048),
                                              ("decode_35b", 40, 2048),
                                              ("batched_80b", 24, 1024),
                                              ("batched_80b_int8", 64, 1024)])
def test_one_block_grouped_gemms(cfgname, T, hidden):
    """Batches of 9..64 bf16 tokens (one token block) run the grouped GEMMs
    whose workgroups request their whole weight tile up front: ragged buckets
    of 1..64 rows (one or two 32-row MFMA blocks), the shared expert's T rows,
    hidden 2048 and 1024 (8 or 4 quantisation groups per wave), int4 and
    int8; every output row and the routing against the oracle, and a second
    call bit-equal to the first."""
    wl = _wl()
    cfg = configs.CONFIGS[cfgname].with_(n_tokens=T, hidden=hidden)
    say(f"[one block] {cfgname} T={T} H={hidden}")
    w = wl.Workload(cfg, n_layers=1)
    x_np = oracle.chain_prologue(synth.activations(cfg), cfg.rms_eps, "bf16").astype(np.float32)
    x = wl.act_tensor(cfg, x_np)
    out, idx, wt, g = run_layer(w, cfg, x)
    counts = np.bincount(idx.cpu().numpy().ravel(), minlength=cfg.n_experts)
    say(f"  {np.count_nonzero(counts)} experts, largest bucket {counts.max()}")
    check_layer(cfg, 0, x_np, out, idx, wt, g, f"{cfgname} T={T} H={hidden}")
    out2 = run_layer(w, cfg, x)[0]
    assert torch.equal(out, out2)
    del w
    _free()
