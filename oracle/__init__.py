"""CPU oracle of the sharded AdamW step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never loads it and
shares no code with it.  This module is argument marshalling (ctypes + numpy)
around ``zs_oracle.c``, a plain single-threaded C implementation written from
the pages (see ``zs_oracle.h`` for the per-function citations):

* "Data parallelism, ZeRO and FSDP" (ML Systems lesson 8): the elementwise
  AdamW of its section 5 simulator, the averaging of rank gradients (section 2
  and the Proposition "DDP is exact"), the Theorem's memory/communication
  table, and the global-norm item of its section 7.
* "Distributed Training Basics -- DDP and FSDP": ``state_bytes`` and the
  clip at the update boundary of its DDP reference program.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.environ.get("ZS_ORACLE_LIB") or os.path.join(_HERE, "libzs_oracle.so")
_SRC = os.path.join(_HERE, "zs_oracle.c")

# -ffp-contract=off: one rounding per written operation (no FMA contraction).
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-std=c11", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc into ``oracle/libzs_oracle.so``."""
    cmd = ["gcc", *CFLAGS, "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


class _Hparams(C.Structure):
    _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double),
                ("eps", C.c_double), ("weight_decay", C.c_double),
                ("step", C.c_int64), ("max_grad_norm", C.c_double)]


class _Consts(C.Structure):
    _fields_ = [(n, C.c_float) for n in ("b1", "b2", "c1", "c2", "bc1", "bc2",
                                         "lr", "wd", "eps")]


@dataclass
class Hparams:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    step: int = 1
    max_grad_norm: float = 0.0

    def _c(self) -> _Hparams:
        return _Hparams(self.lr, self.beta1, self.beta2, self.eps,
                        self.weight_decay, int(self.step), self.max_grad_norm)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = C.CDLL(_LIB_PATH)
        i64, i32, f64, f32 = C.c_int64, C.c_int32, C.c_double, C.c_float
        P = C.POINTER
        L.or_layout.argtypes = [i64, i32, i32, i64, i32, P(i64), P(i64), P(i64)]
        L.or_layout.restype = C.c_int
        L.or_state_bytes.argtypes = [f64, i32, i32, f64]
        L.or_state_bytes.restype = f64
        L.or_comm_elems.argtypes = [f64, i32]
        L.or_comm_elems.restype = f64
        L.or_comm_bytes.argtypes = [f64, i32, i32, f64]
        L.or_comm_bytes.restype = f64
        L.or_comm_elems_accum.argtypes = [f64, i32, i32]
        L.or_comm_elems_accum.restype = f64
        L.or_hsdp_state_bytes.argtypes = [f64, i32, f64]
        L.or_hsdp_state_bytes.restype = f64
        L.or_hsdp_intra_bytes.argtypes = [f64, i32, f64]
        L.or_hsdp_intra_bytes.restype = f64
        L.or_hsdp_inter_bytes.argtypes = [f64, i32, i32, f64]
        L.or_hsdp_inter_bytes.restype = f64
        L.or_bf16_rne.argtypes = [f32]
        L.or_bf16_rne.restype = C.c_uint16
        L.or_bf16_to_f32.argtypes = [C.c_uint16]
        L.or_bf16_to_f32.restype = f32
        L.or_bf16_rne_array.argtypes = [C.c_void_p, i64, C.c_void_p]
        L.or_bf16_rne_array.restype = None
        L.or_reduce_mean.argtypes = [i32, C.c_void_p, i64, C.c_void_p]
        L.or_reduce_mean.restype = None
        L.or_reduce_mean_f32in.argtypes = [i32, C.c_void_p, i64, C.c_void_p]
        L.or_reduce_mean_f32in.restype = None
        L.or_token_weights.argtypes = [i32, C.c_void_p, C.c_void_p]
        L.or_token_weights.restype = C.c_int
        L.or_reduce_weighted.argtypes = [i32, i32, C.c_void_p, C.c_void_p, i64, C.c_void_p]
        L.or_reduce_weighted.restype = None
        L.or_accumulate.argtypes = [i64, C.c_void_p, i32, i32, C.c_void_p]
        L.or_accumulate.restype = None
        L.or_sqacc_size.argtypes = []
        L.or_sqacc_size.restype = i64
        L.or_sqacc_init.argtypes = [C.c_void_p]
        L.or_sqacc_init.restype = None
        L.or_sqacc_add.argtypes = [C.c_void_p, C.c_void_p, i64]
        L.or_sqacc_add.restype = None
        L.or_sqacc_value.argtypes = [C.c_void_p]
        L.or_sqacc_value.restype = f64
        L.or_sqnorm.argtypes = [C.c_void_p, i64]
        L.or_sqnorm.restype = f64
        L.or_clip_coef.argtypes = [f64, f64]
        L.or_clip_coef.restype = f32
        L.or_make_consts.argtypes = [P(_Hparams), P(_Consts)]
        L.or_make_consts.restype = None
        L.or_adamw_f32.argtypes = [P(_Consts), i64, C.c_void_p, C.c_int, f32,
                                   C.c_void_p, C.c_void_p, C.c_void_p]
        L.or_adamw_f32.restype = None
        L.or_pack.argtypes = [i64, i64, C.c_void_p, C.c_void_p]
        L.or_pack.restype = None
        L.or_shard_step.argtypes = [i32, i64, i64, P(_Hparams), C.c_void_p, f64,
                                    C.c_void_p, C.c_void_p, C.c_void_p,
                                    C.c_void_p, P(f64), P(f32)]
        L.or_shard_step.restype = C.c_int
        L.or_reduce_mean_f64.argtypes = [i32, C.c_void_p, i64, C.c_void_p]
        L.or_reduce_mean_f64.restype = None
        L.or_adamw_f64.argtypes = [P(_Hparams), i64, C.c_void_p, C.c_void_p,
                                   C.c_void_p, C.c_void_p]
        L.or_adamw_f64.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray, dtype) -> int:
    if a.dtype != dtype or not a.flags.c_contiguous:
        raise TypeError(f"expected contiguous {np.dtype(dtype)} array, got "
                        f"{a.dtype} contiguous={a.flags.c_contiguous}")
    return a.ctypes.data


def _ptr_array(arrs, dtype):
    ptrs = (C.c_void_p * len(arrs))(*[_ptr(a, dtype) for a in arrs])
    return ptrs


# ---- layout and accounting -------------------------------------------------

def layout(psi: int, n_d: int, rank: int, align: int, stage: int = 2):
    """Return (shard_len, shard_offset, valid_len); raise ValueError(code)."""
    S, off, V = C.c_int64(), C.c_int64(), C.c_int64()
    rc = lib().or_layout(psi, n_d, rank, align, stage, C.byref(S), C.byref(off),
                         C.byref(V))
    if rc != 0:
        raise ValueError(rc)
    return S.value, off.value, V.value


def state_bytes(psi, n_d, stage, K=12.0):
    return lib().or_state_bytes(float(psi), n_d, stage, float(K))


def comm_elems(psi, stage):
    return lib().or_comm_elems(float(psi), stage)


def comm_bytes(psi, n_d, stage, bytes_per_elem=2.0):
    return lib().or_comm_bytes(float(psi), n_d, stage, float(bytes_per_elem))


def comm_elems_accum(psi, stage, m):
    return lib().or_comm_elems_accum(float(psi), stage, m)


def hsdp_state_bytes(psi, g, K=12.0):
    return lib().or_hsdp_state_bytes(float(psi), g, float(K))


def hsdp_intra_bytes(psi, g, bytes_per_elem=2.0):
    return lib().or_hsdp_intra_bytes(float(psi), g, float(bytes_per_elem))


def hsdp_inter_bytes(psi, n_d, g, bytes_per_elem=2.0):
    return lib().or_hsdp_inter_bytes(float(psi), n_d, g, float(bytes_per_elem))


# ---- elementwise pieces -----------------------------------------------------

def bf16_rne(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().or_bf16_rne_array(_ptr(x, np.float32), x.size, _ptr(out, np.uint16))
    return out


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening (bit shift); plain numpy, no arithmetic involved."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def reduce_mean(slices) -> np.ndarray:
    n = slices[0].size
    for s in slices:
        if s.size != n:
            raise ValueError("slices must have equal length")
    out = np.empty(n, dtype=np.float32)
    lib().or_reduce_mean(len(slices), _ptr_array(slices, np.uint16), n,
                         _ptr(out, np.float32))
    return out


def reduce_mean_f32(slices) -> np.ndarray:
    """Rank-order mean of fp32 slices (the fp32 reduce_dtype reading)."""
    n = slices[0].size
    for sl in slices:
        if sl.size != n:
            raise ValueError("slices must have equal length")
    out = np.empty(n, dtype=np.float32)
    lib().or_reduce_mean_f32in(len(slices), _ptr_array(slices, np.float32), n,
                               _ptr(out, np.float32))
    return out


class ZeroTokens(ValueError):
    """The global valid-token count is zero: every rank rejects the update."""


def token_weights(tokens) -> np.ndarray:
    t = np.ascontiguousarray(tokens, dtype=np.int64)
    w = np.empty(t.size, dtype=np.float32)
    rc = lib().or_token_weights(t.size, _ptr(t, np.int64), _ptr(w, np.float32))
    if rc == -2:
        raise ZeroTokens("global token count is zero")
    if rc != 0:
        raise ValueError(f"invalid token counts ({rc})")
    return w


def reduce_weighted(slices, w) -> np.ndarray:
    """Token-weighted rank-order sum of bf16 (uint16) or fp32 slices."""
    n = slices[0].size
    f32in = slices[0].dtype == np.float32
    dt = np.float32 if f32in else np.uint16
    for sl in slices:
        if sl.size != n:
            raise ValueError("slices must have equal length")
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.size != len(slices):
        raise ValueError("one weight per slice")
    out = np.empty(n, dtype=np.float32)
    lib().or_reduce_weighted(len(slices), 1 if f32in else 0, _ptr_array(slices, dt),
                             _ptr(w, np.float32), n, _ptr(out, np.float32))
    return out


def accumulate(r_j: np.ndarray, j: int, m: int, acc: np.ndarray) -> None:
    """Micro-batch j of m into the fp32 accumulator (in place); after the
    last one acc holds the step's gradient, the mean over micro-batches."""
    if r_j.size != acc.size or not (0 <= j < m):
        raise ValueError("bad accumulate call")
    lib().or_accumulate(acc.size, _ptr(r_j, np.float32), j, m, _ptr(acc, np.float32))


def sqnorm(g: np.ndarray) -> float:
    """Exactly rounded sum of g_i^2 (fp32 g)."""
    return lib().or_sqnorm(_ptr(g, np.float32) if g.size else None, g.size)


class SqAcc:
    """Exact squared-norm accumulator: add chunks in any order, read the
    exactly rounded total (the sum is exact until value())."""

    def __init__(self):
        self._buf = C.create_string_buffer(lib().or_sqacc_size())
        lib().or_sqacc_init(self._buf)

    def add(self, g: np.ndarray) -> "SqAcc":
        if g.size:
            lib().or_sqacc_add(self._buf, _ptr(g, np.float32), g.size)
        return self

    def value(self) -> float:
        return lib().or_sqacc_value(self._buf)


def clip_coef(Q: float, max_norm: float) -> np.float32:
    return np.float32(lib().or_clip_coef(float(Q), float(max_norm)))


def make_consts(h: Hparams) -> dict:
    c = _Consts()
    hc = h._c()
    lib().or_make_consts(C.byref(hc), C.byref(c))
    return {n: np.float32(getattr(c, n)) for n, _ in _Consts._fields_}


def adamw_f32(h: Hparams, g, w, m, v, coef=None) -> None:
    """In-place O4 on w, m, v (float32 arrays) with gradient g."""
    c = _Consts()
    hc = h._c()
    lib().or_make_consts(C.byref(hc), C.byref(c))
    n = g.size
    for a in (w, m, v):
        if a.size != n:
            raise ValueError("size mismatch")
    lib().or_adamw_f32(C.byref(c), n, _ptr(g, np.float32),
                       0 if coef is None else 1,
                       0.0 if coef is None else float(coef),
                       _ptr(w, np.float32), _ptr(m, np.float32),
                       _ptr(v, np.float32))


def pack(shard_len: int, w: np.ndarray) -> np.ndarray:
    out = np.empty(shard_len, dtype=np.uint16)
    if w.size > shard_len:
        raise ValueError("valid_len > shard_len")
    lib().or_pack(shard_len, w.size, _ptr(w, np.float32) if w.size else None,
                  _ptr(out, np.uint16))
    return out


def shard_step(n_d, shard_len, valid_len, h: Hparams, slices, w, m, v,
               other_sqnorm=0.0):
    """O1..O5 on one shard, in place on w, m, v.  Returns (out, q, coef)."""
    if len(slices) != n_d:
        raise ValueError("need n_d slices")
    for s in slices:
        if s.size < valid_len:
            raise ValueError("slice shorter than valid_len")
    out = np.empty(shard_len, dtype=np.uint16)
    q, coef = C.c_double(), C.c_float()
    hc = h._c()
    rc = lib().or_shard_step(n_d, shard_len, valid_len, C.byref(hc),
                             _ptr_array(slices, np.uint16), float(other_sqnorm),
                             _ptr(w, np.float32), _ptr(m, np.float32),
                             _ptr(v, np.float32), _ptr(out, np.uint16),
                             C.byref(q), C.byref(coef))
    if rc != 0:
        raise MemoryError(rc)
    return out, q.value, np.float32(coef.value)


def reduce_mean_f64(slices) -> np.ndarray:
    n = slices[0].size
    out = np.empty(n, dtype=np.float64)
    lib().or_reduce_mean_f64(len(slices), _ptr_array(slices, np.float64), n,
                             _ptr(out, np.float64))
    return out


def adamw_f64(h: Hparams, g, w, m, v) -> None:
    hc = h._c()
    lib().or_adamw_f64(C.byref(hc), g.size, _ptr(g, np.float64),
                       _ptr(w, np.float64), _ptr(m, np.float64),
                       _ptr(v, np.float64))
