"""GPU test of the expert slot pool (include/moe_pool.h): decode through a
pool much smaller than the expert pack, with the pack in pinned host memory.

Per layer the router runs on the GPU, the routed experts are made resident
by moe_pool_require (host-to-device copies of the missed blobs, slot-table
updates on the same stream), and moe_experts_forward runs on the pool's slab.
Every output must be bit-equal to the same call on the fully resident slab
(the same kernels read the same blob bytes from other slots), and each
loaded slot must hold exactly the packed blob."""
import gc

import numpy as np
import pytest

import synth
from synth import configs
from tests.parity import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int4_group_quantized_moe_amd as moe
    moe.lib()
    yield
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfgname,T,n_slots,tokens", [("decode_35b", 1, 24, 4),
                                                     ("batched_80b", 64, 120, 2)])
def test_pool_streaming_decode(cfgname, T, n_slots, tokens):
    import int4_group_quantized_moe_amd as moe
    import workload as wl
    from oracle.pool_oracle import SlotPool
    cfg = configs.CONFIGS[cfgname].with_(layers=3, n_tokens=T)
    say(f"[pool] {cfgname} T={T}: {cfg.layers} layers x {cfg.n_experts} experts, {n_slots} slots")
    w = wl.Workload(cfg)
    d = w.desc
    L, E, k, H = cfg.layers, cfg.n_experts, cfg.top_k, cfg.hidden
    stride = w.stride
    pack = torch.empty(L * E * stride, dtype=torch.uint8, pin_memory=True)
    pack.copy_(w.slab)
    torch.cuda.synchronize()
    pslab = torch.empty(n_slots * stride, dtype=torch.uint8, device="cuda")
    tables = torch.zeros(L, E, dtype=torch.int32, device="cuda")
    pool = moe.MoePool(d, L, n_slots, pack, stride, pslab, tables)
    ref = SlotPool(n_slots)
    ws = w.workspace()
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    wt = torch.empty(T, k, dtype=torch.float32, device="cuda")
    gam = torch.empty(T, dtype=torch.float32, device="cuda")
    for tok in range(tokens):
        x = wl.act_tensor(cfg, synth.activations(cfg, variant=tok))
        xh = torch.empty_like(x)
        o_pool, o_ref = torch.empty_like(x), torch.empty_like(x)
        for layer in range(L):
            moe.moe_residual_rmsnorm(d, x, o_ref if layer else None, xh)
            rw, rb, st, sh = w.layer_args(layer)
            wsg = sh[w.slayout.shared_gate_offset: w.slayout.shared_gate_offset + 4 * H].view(
                torch.float32)
            moe.moe_router_topk(d, xh, rw, rb, wsg, idx, wt, gam, ws)
            torch.cuda.synchronize()
            need = sorted(set(idx.cpu().numpy().ravel().tolist()))
            missed = pool.require(layer, need)
            loads = ref.require(layer, need)
            assert missed == len(loads)
            moe.moe_experts_forward(d, xh, idx, wt, gam, pslab, tables[layer], sh, o_pool, ws)
            moe.moe_experts_forward(d, xh, idx, wt, gam, w.slab, st, sh, o_ref, ws)
            torch.cuda.synchronize()
            assert torch.equal(o_pool, o_ref), (tok, layer)
            for e, s in loads[:3]:
                assert pool.slot(layer, e) == s
                blob = pslab[s * stride: s * stride + w.layout.blob_bytes]
                src = w.slab[int(w.slot_tables_np[layer, e]) * stride:][:w.layout.blob_bytes]
                assert torch.equal(blob, src), (layer, e)
    st = pool.stats()
    say(f"  {st['lookups']} lookups, hit rate {st['hits'] / st['lookups']:.3f}, "
        f"{st['evictions']} evictions, {st['bytes_copied'] / 2 ** 20:.1f} MiB copied")
    assert (st["hits"], st["misses"], st["evictions"]) == (ref.hits, ref.misses, ref.evictions)
    assert st["bytes_copied"] == st["misses"] * w.layout.blob_bytes
    del pool, w
    gc.collect()
    torch.cuda.empty_cache()
