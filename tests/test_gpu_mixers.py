"""GPU parity of the token mixers (include/moe_mixers.h) against the fp64
oracle (oracle/mixer_oracle.py), through the C ABI.

Tolerances (derived from fp32 arithmetic on values of order 1):
* Gated DeltaNet state: every element within 1e-4 absolute of the oracle
  (each element is alpha S + c k_j with c from a 128-term fp32 dot product:
  worst-case accumulation error 128 x 2^-24 x sum |S k| ~ 1e-4, typical 1e-6;
  a wrong term moves elements by 0.1 or more);
* outputs stored in bf16: max |err| beyond the storage rounding (2^-8 |ref|)
  <= 2e-3 x rms(out) (the benchmark spec's fp32 bar, since every step computes in fp32).
"""
import gc

import numpy as np
import pytest

from oracle import mixer_oracle as mx
from synth import mixers as sm
from tests.parity import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

STATE_ATOL = 1e-4
OUT_TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int4_group_quantized_moe_amd as moe
    moe.lib()          # must load: there is no fallback path
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _moe():
    import int4_group_quantized_moe_amd as moe
    return moe


def bf16_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda().to(torch.bfloat16)


def check_bf16_out(got, ref, what):
    got = got.float().cpu().numpy().astype(np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), what
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.maximum(np.abs(got - ref) - 2.0 ** -8 * np.abs(ref), 0.0)
    say(f"  {what}: max err beyond bf16 storage {err.max() / rms:.3g} rms (tol {OUT_TOL})")
    assert err.max() <= OUT_TOL * rms, what


def fill_uniform(spec, dtype_out=torch.float32):
    from synth import device as sd
    seed, t, layer, n, lo, hi = spec
    buf = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    sd.fill_uniform_bf16(seed, t, layer, 0xFFFFFE, n, lo, hi, buf,
                         torch.cuda.current_stream().cuda_stream)
    return buf if dtype_out == torch.bfloat16 else buf.to(dtype_out)


# ---------------------------------------------------------------------------
# Gated DeltaNet


def _gdn_run(cfg, seqs_checked, steps):
    moe = _moe()
    d = moe.make_gdn_desc(cfg.n_seqs, cfg.n_k_heads, cfg.n_v_heads, cfg.d_k, cfg.d_v)
    B, Hv, dv, dk = cfg.n_seqs, cfg.n_v_heads, cfg.d_v, cfg.d_k
    state = fill_uniform(sm.gdn_state_spec(cfg)).view(B, Hv, dv, dk)
    # the device fill and the host generator agree bit for bit
    host0 = sm.gdn_state(cfg, seqs=seqs_checked)
    assert np.array_equal(state[list(seqs_checked)].cpu().numpy(), host0.astype(np.float32))
    out = torch.empty(B, Hv, dv, dtype=torch.bfloat16, device="cuda")
    S_ref = host0.astype(np.float64)
    for step in range(steps):
        inp = sm.gdn_inputs(cfg, step)
        S_before = state[list(seqs_checked)].double().cpu().numpy()
        moe.moe_gdn_decode(d, bf16_dev(inp["q"]), bf16_dev(inp["k"]), bf16_dev(inp["v"]),
                           torch.from_numpy(inp["g"]).cuda(), torch.from_numpy(inp["beta"]).cuda(),
                           state, out)
        torch.cuda.synchronize()
        sel = list(seqs_checked)
        # teacher-forced: the oracle steps from the GPU's own state
        S2, o = mx.gdn_step(S_before, inp["q"][sel], inp["k"][sel], inp["v"][sel], inp["g"][sel],
                            inp["beta"][sel])
        got = state[sel].double().cpu().numpy()
        dS = np.abs(got - S2).max()
        say(f"  step {step}: max |state err| {dS:.3g}")
        assert dS <= STATE_ATOL
        check_bf16_out(out[sel], o, f"{cfg.name} step {step} output")
        # and the free-running oracle chain from the initial state
        S_ref, _ = mx.gdn_step(S_ref, inp["q"][sel], inp["k"][sel], inp["v"][sel], inp["g"][sel],
                               inp["beta"][sel])
    drift = np.abs(state[list(seqs_checked)].double().cpu().numpy() - S_ref).max()
    say(f"  after {steps} steps: max |state - free-running oracle| {drift:.3g}")
    assert drift <= steps * STATE_ATOL


@pytest.mark.parametrize("cfgname,seqs,steps", [("gdn_tiny", (0, 1, 2), 4),
                                                ("gdn_80b", (0,), 3),
                                                ("gdn_batched", (0, 17, 63), 2)])
def test_gdn_decode_parity(cfgname, seqs, steps):
    cfg = sm.GDN_CONFIGS[cfgname]
    say(f"[gdn] {cfgname} B={cfg.n_seqs} Hk={cfg.n_k_heads} Hv={cfg.n_v_heads} "
        f"dk={cfg.d_k} dv={cfg.d_v}")
    _gdn_run(cfg, seqs, steps)


@pytest.mark.parametrize("dk,dv,hk,hv", [(256, 32, 1, 3), (128, 48, 4, 4)])
def test_gdn_other_shapes(dk, dv, hk, hv):
    cfg = sm.GDN_TINY.with_(name=f"gdn_{dk}_{dv}", d_k=dk, d_v=dv, n_k_heads=hk, n_v_heads=hv,
                            n_seqs=2)
    say(f"[gdn] dk={dk} dv={dv} Hk={hk} Hv={hv}")
    _gdn_run(cfg, (0, 1), 2)


def test_gdn_delta_identity_on_device():
    """alpha = beta = 1 (g = 0) and a key along e_j: column j of the new
    state equals v (to the fp32 rounding of S + (v - S)); every other column
    keeps its bits."""
    moe = _moe()
    cfg = sm.GDN_TINY.with_(n_seqs=1)
    d = moe.make_gdn_desc(1, cfg.n_k_heads, cfg.n_v_heads, cfg.d_k, cfg.d_v, eps=0.0)
    rng = np.random.default_rng(5)
    S0 = rng.uniform(-0.5, 0.5, (1, cfg.n_v_heads, cfg.d_v, cfg.d_k)).astype(np.float32)
    state = torch.from_numpy(S0).cuda()
    q = bf16_dev(rng.standard_normal((1, cfg.n_k_heads, cfg.d_k)))
    kk = np.zeros((1, cfg.n_k_heads, cfg.d_k), np.float32)
    kk[0, :, 7] = 2.0
    v = rng.standard_normal((1, cfg.n_v_heads, cfg.d_v)).astype(np.float32)
    vb = bf16_dev(v)
    out = torch.empty(1, cfg.n_v_heads, cfg.d_v, dtype=torch.bfloat16, device="cuda")
    moe.moe_gdn_decode(d, q, bf16_dev(kk), vb, torch.zeros(1, cfg.n_v_heads).cuda(),
                       torch.ones(1, cfg.n_v_heads).cuda(), state, out)
    torch.cuda.synchronize()
    S1 = state.cpu().numpy()
    vv = vb.float().cpu().numpy()
    assert np.allclose(S1[0, :, :, 7], vv[0], rtol=0, atol=2e-7)
    others = [c for c in range(cfg.d_k) if c != 7]
    assert np.array_equal(S1[0][:, :, others], S0[0][:, :, others])


# ---------------------------------------------------------------------------
# gated GQA attention


def _attn_run(cfg, lengths, seqs_checked):
    moe = _moe()
    d = moe.make_attn_desc(cfg.n_seqs, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.max_len)
    B, Hq, Hkv, D, N = cfg.n_seqs, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.max_len
    qg = sm.attn_query(cfg)
    K = fill_uniform(sm.attn_cache_spec(cfg, "k"), torch.bfloat16).view(B, Hkv, N, D)
    V = fill_uniform(sm.attn_cache_spec(cfg, "v"), torch.bfloat16).view(B, Hkv, N, D)
    lens = torch.from_numpy(np.asarray(lengths, np.int32)).cuda()
    out = torch.empty(B, Hq, D, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(moe.moe_attn_workspace_bytes(d), 256), dtype=torch.uint8, device="cuda")
    moe.moe_attn_decode(d, bf16_dev(qg["q"]), bf16_dev(qg["gate"]), K, V, lens, out, ws)
    torch.cuda.synchronize()
    sel = list(seqs_checked)
    b0 = sel[0]
    # the device cache equals the host generator's rows
    assert np.array_equal(K[b0, 0, :5].float().cpu().numpy(), sm.attn_cache(cfg, "k", b0, 0, 5))
    lens_sel = [int(lengths[b]) for b in sel]

    def get_kv(i, c, n):
        b = sel[i]
        return sm.attn_cache(cfg, "k", b, c, n), sm.attn_cache(cfg, "v", b, c, n)

    ref = mx.attn_decode(qg["q"][sel], qg["gate"][sel], get_kv, lens_sel, Hkv)
    check_bf16_out(out[sel], ref, f"{cfg.name} lengths {lens_sel}")


@pytest.mark.parametrize("cfgname", ["att_tiny", "att_80b"])
def test_attn_decode_parity(cfgname):
    cfg = sm.ATT_CONFIGS[cfgname]
    lengths = sm.attn_lengths(cfg)
    say(f"[attn] {cfgname} B={cfg.n_seqs} Hq={cfg.n_q_heads} Hkv={cfg.n_kv_heads} "
        f"D={cfg.head_dim} lengths {lengths.tolist()[:8]}")
    _attn_run(cfg, lengths, range(cfg.n_seqs))


def test_attn_decode_batched_sampled():
    cfg = sm.ATT_BATCHED
    lengths = sm.attn_lengths(cfg)
    seqs = sorted({int(np.argmin(lengths)), int(np.argmax(lengths)), 0, 31, 63})
    say(f"[attn] att_batched B=64, checked sequences {seqs} lengths {lengths[seqs].tolist()}")
    _attn_run(cfg, lengths, seqs)


@pytest.mark.parametrize("lengths,hq,hkv,D", [((1, 256, 257), 4, 2, 64), ((512, 255, 1), 2, 2, 128),
                                             ((300, 7, 513), 16, 1, 256),
                                             ((256,), 16, 16, 64)])
def test_attn_edges(lengths, hq, hkv, D):
    """Chunk boundaries (255, 256, 257, 512, 513 positions), a single
    position, one query head per kv head and 16 per kv head."""
    cfg = sm.ATT_TINY.with_(name="att_edge", n_seqs=len(lengths), n_q_heads=hq, n_kv_heads=hkv,
                            head_dim=D, max_len=max(lengths) + 3)
    say(f"[attn edge] lengths {lengths} Hq={hq} Hkv={hkv} D={D}")
    _attn_run(cfg, np.array(lengths, np.int32), range(len(lengths)))
