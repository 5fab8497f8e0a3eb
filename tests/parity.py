"""Comparison rules between the HIP path and the fp64 oracle.

* top-k index sets must match exactly unless the oracle's gap between the
  k-th and (k+1)-th logits is below 1e-5; then the GPU's set must still be a
  valid top-k within that gap, and the output is re-checked against the
  oracle run with the GPU's routing;
* routing weights: relative tolerance 1e-5 (per expert);
* layer output: max |err| <= 2e-3 * rms(out) for fp32 activations and
  <= 2e-2 * rms(out) for bf16, rms over the layer's [T x H] output, with
  the error counted beyond the unit roundoff of storing the output in the
  activation dtype (an output element of 20 rms stored in bf16 alone carries
  up to 20 * 2^-8 = 0.08 rms of rounding error).
"""
from __future__ import annotations

import numpy as np

import oracle

GAP_EPS = 1e-5
W_RTOL = 1e-5
OUT_TOL = {"f32": 2e-3, "bf16": 2e-2}


def say(*a):
    print(*a, flush=True)


def check_routing(idx_gpu, w_gpu, ref, k, gamma_gpu=None, gamma_ref=None):
    """Returns the per-token list of the routing to recheck the output with
    (the oracle's, or the GPU's set where the oracle's gap is < 1e-5)."""
    idx_gpu = np.asarray(idx_gpu)
    w_gpu = np.asarray(w_gpu, np.float64)
    T = idx_gpu.shape[0]
    p = oracle.softmax(ref["logits"])
    use_idx = np.array(ref["idx"])
    use_w = np.array(ref["w"], np.float64)
    n_ties = 0
    for t in range(T):
        g = set(idx_gpu[t].tolist())
        o = set(ref["idx"][t].tolist())
        assert len(g) == k, (t, idx_gpu[t])
        if ref["gap"][t] >= GAP_EPS:
            assert g == o, f"token {t}: gpu {sorted(g)} oracle {sorted(o)} gap {ref['gap'][t]}"
        else:
            n_ties += 1
            l = ref["logits"][t]
            kth = np.sort(l)[::-1][k - 1]
            assert all(l[e] >= kth - GAP_EPS for e in g), (t, sorted(g))
            use_idx[t] = idx_gpu[t]
            use_w[t] = oracle.renormalize(p[t], idx_gpu[t])
        # weights by expert
        ref_w = {int(e): use_w[t][j] for j, e in enumerate(use_idx[t])}
        for j, e in enumerate(idx_gpu[t]):
            r = ref_w[int(e)]
            assert abs(w_gpu[t, j] - r) <= W_RTOL * abs(r), (t, int(e), w_gpu[t, j], r)
        assert abs(w_gpu[t].sum() - 1.0) < 1e-5
        # GPU order: logit descending
        l = ref["logits"][t]
        for j in range(k - 1):
            assert l[idx_gpu[t, j]] >= l[idx_gpu[t, j + 1]] - GAP_EPS
    if gamma_gpu is not None:
        gg = np.asarray(gamma_gpu, np.float64)
        assert np.allclose(gg, gamma_ref, rtol=1e-5, atol=1e-6), (gg, gamma_ref)
    return use_idx, use_w, n_ties


def check_out(got, ref, act, what=""):
    """max|got - ref| <= tol * rms(ref), where the error is measured beyond the
    rounding that storing the output in the activation dtype must add:
    |got - ref| - u * |ref|  with u = 2^-8 (bf16, 8 significant bits) or 2^-24 (fp32), the unit
    roundoff of round-to-nearest storage."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what
    rms = float(np.sqrt(np.mean(ref * ref)))
    u = 2.0 ** -8 if act == "bf16" else 2.0 ** -24
    raw = np.abs(got - ref)
    err = np.maximum(raw - u * np.abs(ref), 0.0)
    tol = OUT_TOL[act] * rms
    worst = np.unravel_index(np.argmax(err), err.shape)
    say(f"  {what}: max|err| beyond storage rounding {err.max():.4g} = {err.max() / rms:.3g} rms "
        f"(tol {OUT_TOL[act]}); raw max|err| {raw.max() / rms:.3g} rms; "
        f"max|out| {np.abs(ref).max() / rms:.3g} rms; worst token {worst[0]}")
    assert err.max() <= tol, f"{what}: max err {err.max()} > {tol} (rms {rms}) at {worst}"
    return err.max() / rms
