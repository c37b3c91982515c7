"""CPU oracle for the KDA decode / verify step -- test infrastructure only.

Only the tests, the smoke check and the bench's CPU-baseline leg use this
package.  It wraps `kda_oracle.c` (plain single-threaded C, built with gcc)
through ctypes and shares nothing with the GPU library: no code, header,
table or helper.  What the C file computes, and which reading of the KDA page
(vllm ... cutedsl.kda.wide, class KdaWide) each step follows, is stated there.

Parity pinned: every stage is pinned by `tests/test_oracle_pins.py` against
invariants, closed forms, special cases and an independent float64 matrix
formulation; see the header of that file for which pin covers which step.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.environ.get("KDA_ORACLE_LIB") or os.path.join(_HERE, "libkda_oracle.so")
_lib = None

HEAD_DIM = 128


def build(force: bool = True, src: str = _SRC, lib: str = None) -> str:
    """Compiles the oracle with gcc (no fused operations, no fast-math).
    `src`/`lib` let a test build a deliberately altered copy elsewhere."""
    lib = lib or _LIB
    if force or not os.path.exists(lib):
        tmp = lib + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-o", tmp, src, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    return lib


class _Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in
                ("B", "H", "N", "W", "T", "slot_stride", "record", "has_bias", "conv_f32")] + \
               [(n, ctypes.c_float) for n in ("lower_bound", "scale", "eps")] + \
               [(n, ctypes.c_void_p) for n in
                ("x", "conv_w", "conv_b", "conv_state", "f_a", "beta", "a_log", "dt_bias",
                 "slots", "accepted", "state", "out", "gate", "norm_w", "f_b", "rec_u",
                 "rec_kg")]


_TAP_FLOAT = ("q", "k", "v", "raw_g", "decay", "beta", "q_hat", "k_hat", "u")
_TAP_DOUBLE = ("o_exact", "o_abs")


class _Taps(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _TAP_FLOAT + _TAP_DOUBLE + ("o_bf",)]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.kda_oracle_run.restype = ctypes.c_int
        lib.kda_oracle_run.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(_Taps)]
        lib.kda_oracle_replay.restype = ctypes.c_int
        lib.kda_oracle_replay.argtypes = [ctypes.c_void_p]
        lib.kda_oracle_silu_bf16.restype = ctypes.c_float
        lib.kda_oracle_silu_bf16.argtypes = [ctypes.c_float]
        lib.kda_oracle_decay.restype = ctypes.c_float
        lib.kda_oracle_decay.argtypes = [ctypes.c_float] * 4
        lib.kda_oracle_gated_rmsnorm.restype = None
        lib.kda_oracle_gated_rmsnorm.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_float,
                                                 ctypes.c_void_p]
        _lib = lib
    return _lib


_LAYOUT = {  # key -> dtype the C side reads
    "x": np.uint16, "conv_w": np.uint16, "conv_b": np.uint16, "conv_state": np.uint16,
    "f_a": np.uint16, "beta": np.uint16, "a_log": np.float32, "dt_bias": np.float32,
    "slots": np.int32, "accepted": np.int32, "state": np.float32, "out": np.uint16,
    "gate": np.uint16, "norm_w": np.uint16, "f_b": np.uint16, "rec_u": np.float32,
    "rec_kg": np.uint16,
}


def _ptr(p, key):
    a = p.get(key)
    if a is None:
        return None
    want = np.float32 if key == "conv_state" and p.get("conv_f32") else _LAYOUT[key]
    if a.dtype != want or not a.flags["C_CONTIGUOUS"]:
        raise TypeError(f"oracle operand {key}: need contiguous {want.__name__}")
    return a.ctypes.data


def run(p: dict, items=None, taps: bool = False):
    """Runs the step on the host arrays of problem `p` (see
    linear_attention_decode_03_amd.inputs for the layouts), updating `state`,
    `conv_state`, `out` and the record buffers in place.  `items` restricts
    the run to those item ids (b * H + h).  Returns the taps dict when
    `taps` is true, else None."""
    lib = _load()
    prob = _Problem(**{n: int(p[n]) for n in
                       ("B", "H", "N", "W", "T", "slot_stride", "record", "has_bias")},
                    conv_f32=int(p.get("conv_f32", 0)),
                    lower_bound=float(p["lower_bound"]), scale=float(p["scale"]),
                    eps=float(p["eps"]),
                    **{k: _ptr(p, k) for k in _LAYOUT})
    shape = (p["B"], p["H"], p["T"], HEAD_DIM)
    tap_arrays = None
    taps_struct = None
    if taps:
        tap_arrays = {n: np.full(shape, np.nan, dtype=np.float32) for n in _TAP_FLOAT}
        tap_arrays["beta"] = np.full(shape[:3], np.nan, dtype=np.float32)
        for n in _TAP_DOUBLE:
            tap_arrays[n] = np.full(shape, np.nan, dtype=np.float64)
        tap_arrays["o_bf"] = np.full(shape, np.nan, dtype=np.float32)
        taps_struct = _Taps(**{n: a.ctypes.data for n, a in tap_arrays.items()})
    if items is None:
        ip, n_items = None, 0
    else:
        items = np.ascontiguousarray(np.asarray(items, dtype=np.int32))
        ip, n_items = items.ctypes.data, int(items.size)
    status = lib.kda_oracle_run(ctypes.byref(prob), int(p.get("gate_mode", 0)), ip, n_items,
                                ctypes.byref(taps_struct) if taps_struct is not None else None)
    if status:
        raise ValueError(f"oracle rejected the problem (status {status})")
    return tap_arrays


class _ReplayProblem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("B", "H", "N", "T")] + \
               [("lower_bound", ctypes.c_float)] + \
               [(n, ctypes.c_void_p) for n in
                ("rec_u", "rec_kg", "a_log", "dt_bias", "src", "dst", "n", "state")]


_REPLAY_LAYOUT = {"rec_u": np.float32, "rec_kg": np.uint16, "a_log": np.float32,
                  "dt_bias": np.float32, "src": np.int32, "dst": np.int32, "n": np.int32,
                  "state": np.float32}


def replay(r: dict):
    """RecoverSSM replay on host arrays (see kda_oracle_replay in the C file):
    r holds B, H, N, T, lower_bound and the arrays of _REPLAY_LAYOUT; `state`
    is updated in place."""
    lib = _load()
    ptrs = {}
    for k, dt in _REPLAY_LAYOUT.items():
        a = r[k]
        if a.dtype != dt or not a.flags["C_CONTIGUOUS"]:
            raise TypeError(f"replay operand {k}: need contiguous {dt.__name__}")
        ptrs[k] = a.ctypes.data
    prob = _ReplayProblem(B=int(r["B"]), H=int(r["H"]), N=int(r["N"]), T=int(r["T"]),
                          lower_bound=float(r["lower_bound"]), **ptrs)
    status = lib.kda_oracle_replay(ctypes.byref(prob))
    if status:
        raise ValueError(f"oracle rejected the replay (status {status})")


def silu_bf16(x: float) -> float:
    """The convolution's SiLU stage, x / (1 + exp(-x)) stored BF16."""
    return float(_load().kda_oracle_silu_bf16(float(x)))


def decay(a_log: float, raw_g: float, dt: float, lower_bound: float) -> float:
    """exp(lower_bound * sigmoid(exp(A_log) * (raw_g + dt_bias))) as an FP32 value."""
    return float(_load().kda_oracle_decay(float(a_log), float(raw_g), float(dt),
                                          float(lower_bound)))


def gated_rmsnorm(o_bf, gate, norm_w, eps: float) -> np.ndarray:
    """The output stage for one token of one head: o_bf float32 [128] (BF16
    values), gate and norm_w BF16 bits [128]; returns BF16 bits [128]."""
    o = np.ascontiguousarray(o_bf, dtype=np.float32)
    g = np.ascontiguousarray(gate, dtype=np.uint16)
    w = np.ascontiguousarray(norm_w, dtype=np.uint16)
    out = np.zeros(HEAD_DIM, dtype=np.uint16)
    _load().kda_oracle_gated_rmsnorm(o.ctypes.data, g.ctypes.data, w.ctypes.data,
                                     float(eps), out.ctypes.data)
    return out
