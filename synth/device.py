"""ctypes binding of the generator's device fill (``libsynth.so``)."""
from __future__ import annotations

import ctypes
import os

from . import BIAS_HI, BIAS_LO, SCALE_HI, SCALE_LO

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsynth.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise ImportError(f"{LIB} is not built (run __graft_entry__.build())")
        h = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        h.synth_fill_experts.argtypes = [ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                         ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                         P, P, P, P, P, P, P]
        h.synth_fill_experts.restype = ctypes.c_int
        h.synth_fill_uniform_bf16.argtypes = [ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                                              ctypes.c_float, P, P]
        h.synth_fill_uniform_bf16.restype = ctypes.c_int
        _lib = h
    return _lib


def fill_experts(cfg, layer: int, expert0: int, n: int, inter: int, qg, qu, qd, sbg, sbu, sbd,
                 stream: int):
    """Logical arrays of experts expert0..expert0+n-1 of one layer into device
    tensors (see synth_fill.hip for the shapes)."""
    st = lib().synth_fill_experts(cfg.seed, cfg.bits, cfg.hidden, inter, layer, expert0, n,
                                  SCALE_LO, SCALE_HI, BIAS_LO, BIAS_HI, qg.data_ptr(),
                                  qu.data_ptr(), qd.data_ptr(), sbg.data_ptr(), sbu.data_ptr(),
                                  sbd.data_ptr(), stream)
    if st != 0:
        raise RuntimeError(f"synth_fill_experts failed: hip error {st}")


def fill_uniform_bf16(seed: int, tensor: int, layer: int, expert: int, n: int, lo: float,
                      hi: float, out, stream: int):
    """Elements [0, n) of one bf16-uniform stream into a device tensor (bf16
    or int16 storage of n elements)."""
    st = lib().synth_fill_uniform_bf16(seed, tensor, layer, expert, n, lo, hi, out.data_ptr(),
                                       stream)
    if st != 0:
        raise RuntimeError(f"synth_fill_uniform_bf16 failed: hip error {st}")
