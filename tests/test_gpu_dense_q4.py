"""The 4-bit dense path (MOE_FLAG_DENSE_Q4: router rows and shared gate as
int4 group-64 codes with bf16 scale and bias) against the fp64 oracle,
through the C ABI.

The oracle routes with the values the codes encode (its own dequantisation,
w = s q + b per group); the GPU reads the packed dense blob.  Covered: the
router entry point (GEMV router, MFMA router at 4096 tokens), whole layers on
every dispatch path (batch-1 decode kernels, one token block, grouped GEMMs,
fp32 tokens) and chains of layers.
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
    moe.lib()
    sd.lib()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _free():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _routing_from_ws(moe, d, ws):
    pi, pw, pg = moe.moe_workspace_routing(d, ws)
    T, k = d.n_tokens, d.top_k
    base = ws.data_ptr()
    torch.cuda.synchronize()
    idx = ws[pi - base: pi - base + 4 * T * k].view(torch.int32).view(T, k).clone()
    wt = ws[pw - base: pw - base + 4 * T * k].view(torch.float32).view(T, k).clone()
    g = ws[pg - base: pg - base + 4 * T].view(torch.float32).clone()
    return idx, wt, g


def _check(cfg, layer, x_np, out, idx, wt, g, what):
    inp = oracle.LayerInputs(cfg, layer, dense_q4=True)
    ref = oracle.oracle_layer(inp, np.asarray(x_np, np.float64))
    use_idx, use_w, n_ties = check_routing(idx.cpu().numpy(), wt.cpu().numpy(), ref, cfg.top_k,
                                           g.cpu().numpy(), ref["gamma"])
    if n_ties:
        ref = oracle.oracle_layer(inp, np.asarray(x_np, np.float64), routing=(use_idx, use_w))
    return check_out(out.float().cpu().numpy(), ref["out"], cfg.act, what)


def _input(cfg, T):
    import workload as wl
    x_np = synth.activations(cfg, n_tokens=T)
    if cfg.act == "bf16":
        x_np = oracle.chain_prologue(x_np, cfg.rms_eps, "bf16").astype(np.float32)
    return x_np, wl.act_tensor(cfg, x_np)


@pytest.mark.parametrize("cfgname,T", [("tiny", 4), ("decode_35b", 1), ("batched_80b", 64),
                                       ("prefill_35b", 4096)])
def test_dense_router_topk(cfgname, T):
    """moe_router_topk on the dense blob: the rows dequantised once per call
    for the GEMV router (small T) or the MFMA router (4096 tokens)."""
    import int4_group_quantized_moe_amd as moe
    import workload as wl
    cfg = configs.CONFIGS[cfgname].with_(n_tokens=T)
    say(f"[dense router] {cfgname} T={T}")
    w = wl.Workload(cfg, n_layers=1, dense_q4=True)
    d = wl.desc_for(cfg, n_tokens=T, dense_q4=True)
    x_np, x = _input(cfg, T)
    rw, rb, _, _ = w.layer_args(0)
    idx = torch.empty(T, cfg.top_k, dtype=torch.int32, device="cuda")
    wt = torch.empty(T, cfg.top_k, dtype=torch.float32, device="cuda")
    g = torch.empty(T, dtype=torch.float32, device="cuda")
    moe.moe_router_topk(d, x, rw, rb, None, idx, wt, g, w.workspace(d))
    torch.cuda.synchronize()
    inp = oracle.LayerInputs(cfg, 0, dense_q4=True)
    xs = np.asarray(x_np, np.float64)
    l, ridx, rwt, gap = oracle.route(xs, inp.router_w, inp.router_bias, cfg.top_k)
    ref = {"logits": l, "idx": ridx, "w": rwt, "gap": gap}
    _, _, n_ties = check_routing(idx.cpu().numpy(), wt.cpu().numpy(), ref, cfg.top_k,
                                 g.cpu().numpy(), oracle.shared_gate(xs, inp.w_sg))
    say(f"  tokens with gap < 1e-5: {n_ties}")
    # a gate vector passed beside the dense blob is an argument error
    with pytest.raises(moe.MoeError):
        moe.moe_router_topk(d, x, rw, rb, w.shared[0], idx, wt, g, w.workspace(d))
    del w
    _free()


@pytest.mark.parametrize("cfgname,T", [("tiny", 4), ("decode_35b", 1), ("decode_80b", 1),
                                       ("batched_80b", 64), ("batched_80b", 300),
                                       ("batched_80b_int8", 40), ("decode_35b", 5)])
def test_dense_layer(cfgname, T):
    """moe_layer_forward with the dense blob as its router argument: the
    batch-1 decode kernels read the 4-bit rows directly, the other paths
    through the per-call fp32 copy."""
    import int4_group_quantized_moe_amd as moe
    import workload as wl
    cfg = configs.CONFIGS[cfgname].with_(n_tokens=T)
    say(f"[dense layer] {cfgname} T={T}")
    w = wl.Workload(cfg, n_layers=1, dense_q4=True)
    d = wl.desc_for(cfg, n_tokens=T, dense_q4=True)
    x_np, x = _input(cfg, T)
    rw, rb, st, sh = w.layer_args(0)
    out = torch.empty_like(x)
    ws = w.workspace(d)
    moe.moe_layer_forward(d, x, rw, rb, w.slab, st, sh, out, ws)
    idx, wt, g = _routing_from_ws(moe, d, ws)
    _check(cfg, 0, x_np, out, idx, wt, g, f"dense {cfgname} T={T}")
    # the shared blob's fp32 gate vector is not read: zeroing it changes nothing
    sh2 = sh.clone()
    off = int(w.slayout.shared_gate_offset)
    sh2[off:off + 4 * cfg.hidden].zero_()
    out2 = torch.empty_like(x)
    moe.moe_layer_forward(d, x, rw, rb, w.slab, st, sh2, out2, w.workspace(d))
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    del w
    _free()


@pytest.mark.parametrize("cfgname,T,L", [("decode_80b", 1, 3), ("batched_80b", 64, 2)])
def test_dense_chain(cfgname, T, L):
    """moe_chain_forward over dense blobs laid out `bytes` apart: each layer
    against the oracle (one-layer calls), and the whole chain in one call
    bit-equal to them."""
    import int4_group_quantized_moe_amd as moe
    import workload as wl
    cfg = configs.CONFIGS[cfgname].with_(n_tokens=T, layers=L)
    say(f"[dense chain] {cfgname} T={T} L={L}")
    w = wl.Workload(cfg, n_layers=L, dense_q4=True)
    d = wl.desc_for(cfg, n_tokens=T, dense_q4=True)
    x0_np = synth.activations(cfg, n_tokens=T)
    x = wl.act_tensor(cfg, x0_np)
    xh, out = torch.empty_like(x), torch.empty_like(x)
    ws = w.workspace(d)
    for i in range(L):
        xb = wl.to_f64(x)
        rw, rb, st, sh = w.layer_args(i)
        moe.moe_chain_forward(d, 1, x, rw, rb, w.slab, st, sh, w.shared_stride, xh, out, ws)
        idx, wt, g = _routing_from_ws(moe, d, ws)
        xh_ref = oracle.chain_prologue(xb, cfg.rms_eps, cfg.act)
        assert np.all(np.abs(wl.to_f64(xh) - xh_ref) <= np.abs(xh_ref) * 2.0 ** -7), "rmsnorm"
        _check(cfg, i, wl.to_f64(xh), out, idx, wt, g, f"dense chain {cfgname} layer {i}")
        assert np.array_equal(wl.to_f64(x), oracle.chain_epilogue(xb, wl.to_f64(out), cfg.act))
    xc = wl.act_tensor(cfg, x0_np)
    moe.moe_chain_forward(d, L, xc, w.router_all, w.router_bias, w.slab, w.slot_tables, w.shared,
                          w.shared_stride, torch.empty_like(xc), torch.empty_like(xc),
                          w.workspace(d))
    torch.cuda.synchronize()
    assert torch.equal(xc, x)
    del w
    _free()
