"""The no-allocation entry point (moe_layer_forward_noalloc) against
moe_layer_forward, through the C ABI.

Collected last (this file's name sorts after every other test file).  Each
case makes two calls in a row on the library's scratch, the second with
fewer tokens, so that the second starts from the first's leftover contents;
each output must equal moe_layer_forward's on a fresh zero-filled workspace
bit for bit (the same kernels run).
"""
import gc

import numpy as np
import pytest

import oracle
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
    moe.lib()          # must load: there is no fallback path
    yield
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfgname,T1,T2", [("batched_80b", 128, 20), ("batched_80b_int8", 64, 9),
                                           ("tiny", 40, 9), ("decode_35b", 5, 1),
                                           ("decode_80b", 16, 1)])
def test_noalloc_matches_layer_forward(cfgname, T1, T2):
    import int4_group_quantized_moe_amd as moe
    import workload as wl
    base = configs.CONFIGS[cfgname]
    cfg = base.with_(n_tokens=T1)
    say(f"[noalloc] {cfgname} T={T1} then T={T2}")
    w = wl.Workload(cfg, n_layers=1)
    x_np = synth.activations(cfg)
    if cfg.act == "bf16":
        x_np = oracle.chain_prologue(x_np, cfg.rms_eps, "bf16").astype(np.float32)
    x = wl.act_tensor(cfg, x_np)
    rw, rb, st, sh = w.layer_args(0)
    for T in (T1, T2):
        d = wl.desc_for(cfg, n_tokens=T)
        assert moe.moe_workspace_bytes(d) <= moe.MOE_NOALLOC_SCRATCH_BYTES
        xt = x[:T].contiguous()
        ref = torch.empty_like(xt)
        moe.moe_layer_forward(d, xt, rw, rb, w.slab, st, sh, ref, w.workspace(d))
        got = torch.full_like(xt, float("nan"))
        moe.moe_layer_forward_noalloc(d, xt, rw, rb, w.slab, st, sh, got)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"T={T}"
        say(f"  T={T}: equal to moe_layer_forward")
    del w
    gc.collect()
    torch.cuda.empty_cache()


def test_noalloc_rejects_calls_beyond_the_scratch():
    """A call whose workspace exceeds the scratch returns MOE_ERR_TOO_LARGE
    before anything is enqueued (no pointer is read)."""
    import int4_group_quantized_moe_amd as moe
    import workload as wl
    cfg = configs.PREFILL_35B
    d = wl.desc_for(cfg, n_tokens=4096)
    assert moe.moe_workspace_bytes(d) > moe.MOE_NOALLOC_SCRATCH_BYTES
    dummy = torch.zeros(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer_forward_noalloc(d, dummy, dummy, None, dummy, dummy, dummy, dummy)
    assert e.value.status == moe.MOE_ERR_TOO_LARGE
