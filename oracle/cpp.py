"""The C++ fp64 oracle (``moe_oracle.cpp``) behind the numpy oracle's API.

TEST INFRASTRUCTURE ONLY (see the package docstring).  ``CppOracle`` loads
one build of ``liboracle.so`` and offers the same functions, with the same
arguments and results, as ``oracle.moe_oracle``; the module-level functions
are those of the default build.  This file only converts arrays and calls
the library: every step of the layer is computed in C++.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import build as _build

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_D = ctypes.c_double


class _Expert(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("qg", "qu", "qd", "sg", "bg", "su", "bu", "sd", "bd")] + \
               [("inter", _I64)]


def _arr(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a):
    return a.ctypes.data_as(_P) if a is not None else None


_SIGS = {
    "orc_num_threads": ([], ctypes.c_int),
    "orc_set_num_threads": ([ctypes.c_int], None),
    "orc_bf16_to_f64": ([_P, _I64, _P], None),
    "orc_round_bf16": ([_D], _D),
    "orc_round_act": ([_P, _I64, ctypes.c_int, _P], None),
    "orc_dequantize": ([_P, _P, _P, _I64, _I64, _I64, _P], None),
    "orc_router_logits": ([_P, _P, _P, _I64, _I64, _I64, _P], None),
    "orc_softmax": ([_P, _I64, _I64, _P], None),
    "orc_topk": ([_P, _I64, _I64, _P, _P], None),
    "orc_renormalize": ([_P, _P, _I64, _P], None),
    "orc_silu_array": ([_P, _I64, _P], None),
    "orc_sigmoid_array": ([_P, _I64, _P], None),
    "orc_expert_ffn": ([_P, _I64, _I64, ctypes.POINTER(_Expert), _I64, _P], None),
    "orc_shared_gate": ([_P, _P, _I64, _I64, _P], None),
    "orc_route": ([_P, _P, _P, _I64, _I64, _I64, _I64, _P, _P, _P, _P], None),
    "orc_combine": ([_P, _I64, _I64, _P, _P, _I64, ctypes.POINTER(_Expert), _I64, _I64, _P,
                     ctypes.POINTER(_Expert), _P], None),
    "orc_rmsnorm": ([_P, _I64, _I64, _D, _P], None),
    "orc_chain_prologue": ([_P, _I64, _I64, _D, ctypes.c_int, _P], None),
    "orc_chain_epilogue": ([_P, _P, _I64, ctypes.c_int, _P], None),
    "orc_bucket": ([_P, _I64, _I64, _I64, _P, _P, _P], None),
}

_ACT = {"f32": 0, "bf16": 1}


class CppOracle:
    """One build of the C++ oracle, with the numpy oracle's function API."""

    def __init__(self, path: str | None = None):
        self.path = path or _build.ensure_built()
        h = ctypes.CDLL(self.path)
        for name, (argtypes, restype) in _SIGS.items():
            fn = getattr(h, name)
            fn.argtypes = argtypes
            fn.restype = restype
        self._h = h

    # threads ---------------------------------------------------------------
    def num_threads(self) -> int:
        return int(self._h.orc_num_threads())

    def set_num_threads(self, n: int) -> None:
        self._h.orc_set_num_threads(int(n))

    # number formats ----------------------------------------------------------
    def bf16_to_f64(self, bits) -> np.ndarray:
        b = _arr(bits, np.uint16)
        out = np.empty(b.shape, np.float64)
        self._h.orc_bf16_to_f64(_p(b), b.size, _p(out))
        return out

    def round_to_bf16(self, v) -> np.ndarray:
        return self.round_act(v, "bf16")

    def round_act(self, v, act: str) -> np.ndarray:
        if act not in _ACT:
            raise ValueError(act)
        a = _arr(v, np.float64)
        out = np.empty(a.shape, np.float64)
        self._h.orc_round_act(_p(a), a.size, _ACT[act], _p(out))
        return out

    # the layer, step by step -------------------------------------------------
    def dequantize(self, q, scale_bits, bias_bits, group: int) -> np.ndarray:
        q = _arr(q, np.uint8)
        rows, cols = q.shape
        s, b = _arr(scale_bits, np.uint16), _arr(bias_bits, np.uint16)
        assert s.shape == (rows, cols // group) and b.shape == s.shape
        W = np.empty((rows, cols), np.float64)
        self._h.orc_dequantize(_p(q), _p(s), _p(b), rows, cols, group, _p(W))
        return W

    def router_logits(self, x_hat, router_w, router_bias=None) -> np.ndarray:
        x = _arr(x_hat, np.float64)
        Wr = _arr(router_w, np.float64)
        rb = _arr(router_bias, np.float64) if router_bias is not None else None
        T, H = x.shape
        E = Wr.shape[0]
        l = np.empty((T, E), np.float64)
        self._h.orc_router_logits(_p(x), _p(Wr), _p(rb), T, E, H, _p(l))
        return l

    def softmax(self, l) -> np.ndarray:
        a = _arr(l, np.float64)
        E = a.shape[-1]
        out = np.empty(a.shape, np.float64)
        self._h.orc_softmax(_p(a), a.size // E, E, _p(out))
        return out

    def topk(self, l_row, k: int):
        l = _arr(l_row, np.float64)
        sel = np.empty(k, np.int64)
        gap = _D()
        self._h.orc_topk(_p(l), l.shape[0], k, _p(sel), ctypes.byref(gap))
        return sel, float(gap.value)

    def renormalize(self, p_row, sel) -> np.ndarray:
        p = _arr(p_row, np.float64)
        s = _arr(sel, np.int64)
        w = np.empty(s.shape[0], np.float64)
        self._h.orc_renormalize(_p(p), _p(s), s.shape[0], _p(w))
        return w

    def silu(self, g) -> np.ndarray:
        a = _arr(g, np.float64)
        out = np.empty(a.shape, np.float64)
        self._h.orc_silu_array(_p(a), a.size, _p(out))
        return out

    def sigmoid(self, v) -> np.ndarray:
        a = _arr(v, np.float64)
        out = np.empty(a.shape, np.float64)
        self._h.orc_sigmoid_array(_p(a), a.size, _p(out))
        return out

    @staticmethod
    def _expert(arrays: dict, keep: list) -> _Expert:
        ex = _Expert()
        for key in ("qg", "qu", "qd"):
            a = _arr(arrays[key], np.uint8)
            keep.append(a)
            setattr(ex, key, a.ctypes.data)
        for key in ("sg", "bg", "su", "bu", "sd", "bd"):
            a = _arr(arrays[key], np.uint16)
            keep.append(a)
            setattr(ex, key, a.ctypes.data)
        ex.inter = np.asarray(arrays["qg"]).shape[0]
        return ex

    def expert_ffn(self, x_hat, arrays: dict, group: int) -> np.ndarray:
        x = _arr(x_hat, np.float64)
        n, H = x.shape
        keep: list = []
        ex = self._expert(arrays, keep)
        y = np.empty((n, H), np.float64)
        self._h.orc_expert_ffn(_p(x), n, H, ctypes.byref(ex), group, _p(y))
        return y

    def shared_gate(self, x_hat, w_sg) -> np.ndarray:
        x = _arr(x_hat, np.float64)
        T, H = x.shape
        w = _arr(w_sg, np.float64)
        g = np.empty(T, np.float64)
        self._h.orc_shared_gate(_p(x), _p(w), T, H, _p(g))
        return g

    def route(self, x_hat, router_w, router_bias, k: int):
        x = _arr(x_hat, np.float64)
        Wr = _arr(router_w, np.float64)
        rb = _arr(router_bias, np.float64) if router_bias is not None else None
        T, H = x.shape
        E = Wr.shape[0]
        l = np.empty((T, E), np.float64)
        idx = np.empty((T, k), np.int64)
        w = np.empty((T, k), np.float64)
        gap = np.empty(T, np.float64)
        self._h.orc_route(_p(x), _p(Wr), _p(rb), T, E, H, k, _p(l), _p(idx), _p(w), _p(gap))
        return l, idx, w, gap

    def combine(self, x_hat, idx, w, get_expert, group: int, gamma=None,
                shared=None) -> np.ndarray:
        x = _arr(x_hat, np.float64)
        T, H = x.shape
        idx = _arr(idx, np.int64)
        k = idx.shape[1]
        wt = _arr(w, np.float64)
        E = int(idx.max()) + 1 if idx.size else 1
        keep: list = []
        table = (_Expert * E)()
        for e in np.unique(idx):
            table[int(e)] = self._expert(get_expert(int(e)), keep)
        sh = None
        g = None
        if shared is not None:
            sh = ctypes.byref(self._expert(shared, keep))
            g = _arr(gamma, np.float64)
        out = np.empty((T, H), np.float64)
        self._h.orc_combine(_p(x), T, H, _p(idx), _p(wt), k, table, E, group, _p(g), sh, _p(out))
        return out

    def moe_layer(self, x_hat, router_w, router_bias, w_sg, get_expert, shared, k: int,
                  group: int, routing=None) -> dict:
        logits, idx, w, gap = self.route(x_hat, router_w, router_bias, k)
        if routing is not None:
            idx, w = np.asarray(routing[0]), np.asarray(routing[1], np.float64)
        gamma = self.shared_gate(x_hat, w_sg) if shared is not None else None
        out = self.combine(x_hat, idx, w, get_expert, group, gamma, shared)
        return {"logits": logits, "idx": idx, "w": w, "gap": gap, "gamma": gamma, "out": out}

    # the chain around the layer ------------------------------------------------
    def rmsnorm(self, x, eps: float) -> np.ndarray:
        a = _arr(x, np.float64)
        H = a.shape[-1]
        out = np.empty(a.shape, np.float64)
        self._h.orc_rmsnorm(_p(a), a.size // H, H, float(eps), _p(out))
        return out

    def chain_prologue(self, x, eps: float, act: str) -> np.ndarray:
        a = _arr(x, np.float64)
        H = a.shape[-1]
        out = np.empty(a.shape, np.float64)
        self._h.orc_chain_prologue(_p(a), a.size // H, H, float(eps), _ACT[act], _p(out))
        return out

    def chain_epilogue(self, x, out, act: str) -> np.ndarray:
        a = _arr(x, np.float64)
        o = _arr(out, np.float64)
        r = np.empty(a.shape, np.float64)
        self._h.orc_chain_epilogue(_p(a), _p(o), a.size, _ACT[act], _p(r))
        return r

    # bucketing -------------------------------------------------------------
    def bucket(self, idx, n_experts: int):
        a = _arr(idx, np.int64)
        T, k = a.shape
        counts = np.empty(n_experts, np.int64)
        offsets = np.empty(n_experts + 1, np.int64)
        pairs = np.empty((T * k, 2), np.int64)
        self._h.orc_bucket(_p(a), T, k, n_experts, _p(counts), _p(offsets), _p(pairs))
        return counts, offsets, pairs


_default: CppOracle | None = None


def default() -> CppOracle:
    """The oracle of the normal build (compiled on first use if missing)."""
    global _default
    if _default is None:
        _default = CppOracle()
    return _default


def __getattr__(name):
    # module-level access to the default build's functions: oracle.cpp.route(...)
    if name.startswith("_"):
        raise AttributeError(name)
    return getattr(default(), name)
