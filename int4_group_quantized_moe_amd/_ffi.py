"""ctypes binding of ``libmoe.so`` (the C ABI declared in include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
the library.  Tensor arguments may be torch tensors (their ``data_ptr()`` is
passed), plain integers (raw device addresses) or None (NULL).  The stream
defaults to torch's current HIP stream.  A non-zero status raises MoeError.
If the library is not built, loading raises an error: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_MISALIGNED = -3
MOE_ERR_NO_DEVICE = -4
MOE_ERR_LAUNCH = -5
MOE_ERR_TOO_LARGE = -6
MOE_NOALLOC_SCRATCH_BYTES = 32 << 20

MOE_ACT_F32 = 0
MOE_ACT_BF16 = 1

MOE_FLAG_ROUTER_BIAS = 1
MOE_FLAG_SHARED = 2
MOE_FLAG_DENSE_Q4 = 4

MOE_MAX_TOP_K = 16
MOE_MAX_EXPERTS = 1024


class MoeError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn}: {moe_status_string(status)} ({status})")


class moe_layer_desc(ctypes.Structure):
    _fields_ = [
        ("n_tokens", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("n_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("inter", ctypes.c_int32),
        ("shared_inter", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("bits", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32),
        ("reserved0", ctypes.c_int32),
        ("expert_stride", ctypes.c_int64),
        ("flags", ctypes.c_uint32),
        ("rms_eps", ctypes.c_float),
    ]


class moe_blob_layout_t(ctypes.Structure):
    _fields_ = [
        ("gu_offset", ctypes.c_int64),
        ("gu_unit_bytes", ctypes.c_int64),
        ("gu_tile_bytes", ctypes.c_int64),
        ("down_offset", ctypes.c_int64),
        ("down_unit_bytes", ctypes.c_int64),
        ("down_tile_bytes", ctypes.c_int64),
        ("blob_bytes", ctypes.c_int64),
        ("shared_gate_offset", ctypes.c_int64),
        ("shared_bytes", ctypes.c_int64),
        ("row_tile", ctypes.c_int32),
        ("kblock_cols", ctypes.c_int32),
        ("groups_per_kblock", ctypes.c_int32),
        ("reserved0", ctypes.c_int32),
    ]


class moe_dense_layout_t(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int64),
        ("words_offset", ctypes.c_int64),
        ("bytes", ctypes.c_int64),
    ]


class moe_gdn_desc(ctypes.Structure):
    _fields_ = [
        ("n_seqs", ctypes.c_int32),
        ("n_k_heads", ctypes.c_int32),
        ("n_v_heads", ctypes.c_int32),
        ("d_k", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("reserved0", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("scale", ctypes.c_float),
    ]


class moe_attn_desc(ctypes.Structure):
    _fields_ = [
        ("n_seqs", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("max_len", ctypes.c_int32),
        ("reserved0", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("reserved1", ctypes.c_float),
    ]


class moe_pool_stats_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("requests", "lookups", "hits", "misses",
                                              "evictions", "bytes_copied")]


MOE_POOL_HOST_ONLY = 1

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_DESC = ctypes.POINTER(moe_layer_desc)
_GDESC = ctypes.POINTER(moe_gdn_desc)
_ADESC = ctypes.POINTER(moe_attn_desc)

_SIGS = {
    "moe_version": ([], ctypes.c_char_p),
    "moe_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "moe_blob_layout": ([_DESC, _I32, ctypes.POINTER(moe_blob_layout_t)], ctypes.c_int),
    "moe_pack_expert": ([_DESC, _I32, _P, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "moe_dense_layout": ([_DESC, ctypes.POINTER(moe_dense_layout_t)], ctypes.c_int),
    "moe_pack_dense": ([_DESC, _P, _P, _P], ctypes.c_int),
    "moe_pack_experts_device": ([_DESC, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P],
                                ctypes.c_int),
    "moe_workspace_bytes": ([_DESC], ctypes.c_size_t),
    "moe_router_topk": ([_DESC, _P, _P, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "moe_experts_forward": ([_DESC, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "moe_layer_forward": ([_DESC, _P, _P, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "moe_layer_forward_noalloc": ([_DESC, _P, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "moe_workspace_routing": ([_DESC, _P, ctypes.POINTER(_P), ctypes.POINTER(_P),
                               ctypes.POINTER(_P)], ctypes.c_int),
    "moe_residual_rmsnorm": ([_DESC, _P, _P, _P, _P], ctypes.c_int),
    "moe_rmsnorm": ([_DESC, _P, _P, _P, _P], ctypes.c_int),
    "moe_chain_status": ([_DESC, _P, ctypes.POINTER(_P)], ctypes.c_int),
    "moe_gdn_decode": ([_GDESC, _P, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "moe_attn_workspace_bytes": ([_ADESC], ctypes.c_size_t),
    "moe_attn_decode": ([_ADESC, _P, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "moe_pool_create": ([_DESC, _I32, _I32, _P, _I64, _P, _P, ctypes.c_uint32,
                         ctypes.POINTER(_P)], ctypes.c_int),
    "moe_pool_require": ([_P, _I32, _P, _I32, _P, _P], ctypes.c_int),
    "moe_pool_stats": ([_P, ctypes.POINTER(moe_pool_stats_t)], ctypes.c_int),
    "moe_pool_slot": ([_P, _I32, _I32], ctypes.c_int32),
    "moe_pool_destroy": ([_P], None),
    "moe_chain_forward": ([_DESC, _I32, _P, _P, _P, _P, _P, _P, _I64, _P, _P, _P, _P],
                          ctypes.c_int),
}

_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
        h = ctypes.CDLL(LIB_PATH)
        for name, (argtypes, restype) in _SIGS.items():
            fn = getattr(h, name)
            fn.argtypes = argtypes
            fn.restype = restype
        _lib = h
    return _lib


def exported_symbols():
    return list(_SIGS)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    if isinstance(t, ctypes.Array) or isinstance(t, ctypes._Pointer):
        return ctypes.cast(t, ctypes.c_void_p).value
    if hasattr(t, "ctypes"):            # numpy array (host)
        return t.ctypes.data
    raise TypeError(f"cannot pass {type(t)} as a pointer")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(st: int, fn: str):
    if st != MOE_OK:
        raise MoeError(st, fn)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)


def moe_version() -> str:
    return lib().moe_version().decode()


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def moe_blob_layout(desc: moe_layer_desc, inter: int) -> moe_blob_layout_t:
    out = moe_blob_layout_t()
    _check(lib().moe_blob_layout(ctypes.byref(desc), inter, ctypes.byref(out)), "moe_blob_layout")
    return out


def moe_pack_expert(desc, inter, q_gate, q_up, q_down, sb_gate, sb_up, sb_down, shared_gate_w,
                    blob_out):
    """Host packer: numpy arrays (host memory) in, host buffer out."""
    _check(lib().moe_pack_expert(ctypes.byref(desc), inter, _ptr(q_gate), _ptr(q_up),
                                 _ptr(q_down), _ptr(sb_gate), _ptr(sb_up), _ptr(sb_down),
                                 _ptr(shared_gate_w), _ptr(blob_out)), "moe_pack_expert")


def moe_dense_layout(desc: moe_layer_desc) -> moe_dense_layout_t:
    out = moe_dense_layout_t()
    _check(lib().moe_dense_layout(ctypes.byref(desc), ctypes.byref(out)), "moe_dense_layout")
    return out


def moe_pack_dense(desc, q, sb, blob_out):
    _check(lib().moe_pack_dense(ctypes.byref(desc), _ptr(q), _ptr(sb), _ptr(blob_out)),
           "moe_pack_dense")


def moe_pack_experts_device(desc, inter, n, q_gate, q_up, q_down, sb_gate, sb_up, sb_down, slab,
                            dst_slots, stream=None):
    slots = (ctypes.c_int64 * n)(*[int(s) for s in dst_slots])
    _check(lib().moe_pack_experts_device(ctypes.byref(desc), inter, n, _ptr(q_gate), _ptr(q_up),
                                         _ptr(q_down), _ptr(sb_gate), _ptr(sb_up), _ptr(sb_down),
                                         _ptr(slab), ctypes.cast(slots, _P), _stream(stream)),
           "moe_pack_experts_device")


def moe_workspace_bytes(desc) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(desc)))


def moe_router_topk(desc, x, router_w, router_bias, shared_gate_w, topk_idx, topk_w, shared_gate,
                    ws, stream=None):
    _check(lib().moe_router_topk(ctypes.byref(desc), _ptr(x), _ptr(router_w), _ptr(router_bias),
                                 _ptr(shared_gate_w), _ptr(topk_idx), _ptr(topk_w),
                                 _ptr(shared_gate), _ptr(ws), _stream(stream)), "moe_router_topk")


def moe_experts_forward(desc, x, topk_idx, topk_w, shared_gate, expert_slab, slot_table,
                        shared_blob, out, ws, stream=None):
    _check(lib().moe_experts_forward(ctypes.byref(desc), _ptr(x), _ptr(topk_idx), _ptr(topk_w),
                                     _ptr(shared_gate), _ptr(expert_slab), _ptr(slot_table),
                                     _ptr(shared_blob), _ptr(out), _ptr(ws), _stream(stream)),
           "moe_experts_forward")


def moe_layer_forward(desc, x, router_w, router_bias, expert_slab, slot_table, shared_blob, out, ws,
                      stream=None):
    _check(lib().moe_layer_forward(ctypes.byref(desc), _ptr(x), _ptr(router_w), _ptr(router_bias),
                                   _ptr(expert_slab), _ptr(slot_table), _ptr(shared_blob),
                                   _ptr(out), _ptr(ws), _stream(stream)), "moe_layer_forward")


def moe_layer_forward_noalloc(desc, x, router_w, router_bias, expert_slab, slot_table,
                              shared_blob, out, stream=None):
    _check(lib().moe_layer_forward_noalloc(ctypes.byref(desc), _ptr(x), _ptr(router_w),
                                           _ptr(router_bias), _ptr(expert_slab), _ptr(slot_table),
                                           _ptr(shared_blob), _ptr(out), _stream(stream)),
           "moe_layer_forward_noalloc")


def moe_workspace_routing(desc, ws):
    """Device addresses (ints) of (topk_idx, topk_w, shared_gate) inside ws."""
    a, b, c = _P(), _P(), _P()
    _check(lib().moe_workspace_routing(ctypes.byref(desc), _ptr(ws), ctypes.byref(a),
                                       ctypes.byref(b), ctypes.byref(c)), "moe_workspace_routing")
    return a.value, b.value, c.value


def moe_residual_rmsnorm(desc, x_res, out, x_next, stream=None):
    _check(lib().moe_residual_rmsnorm(ctypes.byref(desc), _ptr(x_res), _ptr(out), _ptr(x_next),
                                      _stream(stream)), "moe_residual_rmsnorm")


def moe_rmsnorm(desc, x, out, x_hat, stream=None):
    _check(lib().moe_rmsnorm(ctypes.byref(desc), _ptr(x), _ptr(out), _ptr(x_hat), _stream(stream)),
           "moe_rmsnorm")


def moe_chain_status(desc, ws) -> int:
    """Device address (int) of the persistent chain's status word inside ws."""
    a = _P()
    _check(lib().moe_chain_status(ctypes.byref(desc), _ptr(ws), ctypes.byref(a)),
           "moe_chain_status")
    return a.value


def moe_chain_forward(desc, n_layers, x, router_w, router_bias, expert_slab, slot_tables,
                      shared_blobs, shared_stride, x_hat, out, ws, stream=None):
    _check(lib().moe_chain_forward(ctypes.byref(desc), n_layers, _ptr(x), _ptr(router_w),
                                   _ptr(router_bias), _ptr(expert_slab), _ptr(slot_tables),
                                   _ptr(shared_blobs), int(shared_stride), _ptr(x_hat), _ptr(out),
                                   _ptr(ws), _stream(stream)), "moe_chain_forward")


# ---------------------------------------------------------------------------
# token mixers (include/moe_mixers.h)


def make_gdn_desc(n_seqs, n_k_heads, n_v_heads, d_k, d_v, eps=1e-6, scale=0.0):
    d = moe_gdn_desc()
    d.n_seqs, d.n_k_heads, d.n_v_heads, d.d_k, d.d_v = n_seqs, n_k_heads, n_v_heads, d_k, d_v
    d.eps, d.scale = eps, scale
    return d


def make_attn_desc(n_seqs, n_q_heads, n_kv_heads, head_dim, max_len, scale=0.0):
    d = moe_attn_desc()
    d.n_seqs, d.n_q_heads, d.n_kv_heads, d.head_dim, d.max_len = (n_seqs, n_q_heads, n_kv_heads,
                                                                  head_dim, max_len)
    d.scale = scale
    return d


def moe_gdn_decode(desc, q, k, v, g, beta, state, out, stream=None):
    _check(lib().moe_gdn_decode(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                _ptr(beta), _ptr(state), _ptr(out), _stream(stream)),
           "moe_gdn_decode")


def moe_attn_workspace_bytes(desc) -> int:
    return int(lib().moe_attn_workspace_bytes(ctypes.byref(desc)))


def moe_attn_decode(desc, q, gate, k_cache, v_cache, lengths, out, ws, stream=None):
    _check(lib().moe_attn_decode(ctypes.byref(desc), _ptr(q), _ptr(gate), _ptr(k_cache),
                                 _ptr(v_cache), _ptr(lengths), _ptr(out), _ptr(ws),
                                 _stream(stream)), "moe_attn_decode")


# ---------------------------------------------------------------------------
# expert slot pool (include/moe_pool.h)


class MoePool:
    """A moe_pool handle (host object); destroyed with the Python object."""

    def __init__(self, desc, n_layers, n_slots, host_pack=None, host_stride=0, device_slab=None,
                 slot_tables=None, host_only=False):
        self._h = _P()
        _check(lib().moe_pool_create(ctypes.byref(desc), n_layers, n_slots, _ptr(host_pack),
                                     int(host_stride), _ptr(device_slab), _ptr(slot_tables),
                                     MOE_POOL_HOST_ONLY if host_only else 0,
                                     ctypes.byref(self._h)), "moe_pool_create")

    def require(self, layer, experts, stream=None) -> int:
        """Makes the experts (a sequence of ints) of `layer` resident; returns the misses."""
        arr = (ctypes.c_int32 * max(len(experts), 1))(*[int(e) for e in experts])
        missed = ctypes.c_int32(0)
        st = lib().moe_pool_require(self._h, layer, ctypes.cast(arr, _P), len(experts),
                                    ctypes.cast(ctypes.byref(missed), _P),
                                    _stream(stream) if self._needs_stream(stream) else None)
        _check(st, "moe_pool_require")
        return int(missed.value)

    @staticmethod
    def _needs_stream(stream):
        if stream is not None:
            return True
        try:
            import torch
            return torch.cuda.is_available()
        except ImportError:
            return False

    def stats(self) -> dict:
        out = moe_pool_stats_t()
        _check(lib().moe_pool_stats(self._h, ctypes.byref(out)), "moe_pool_stats")
        return {n: int(getattr(out, n)) for n, _ in moe_pool_stats_t._fields_}

    def slot(self, layer, expert) -> int:
        return int(lib().moe_pool_slot(self._h, layer, expert))

    def __del__(self):
        try:
            if self._h:
                lib().moe_pool_destroy(self._h)
                self._h = _P()
        except Exception:  # noqa: BLE001  (interpreter shutdown)
            pass
