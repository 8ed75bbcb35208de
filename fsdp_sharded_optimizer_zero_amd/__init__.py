"""MI355X sharded optimizer step (ZeRO-1/2/3, FSDP) -- Python binding.

Argument marshalling only: every function forwards to the C ABI of
``libzero_shard.so`` (declared in ``include/zero_shard.h``) with the same
name.  PyTorch tensors serve as device memory and streams; all arithmetic
runs in the library's HIP kernels.  There is no fallback: if the library is
missing, importing the entry points raises.
"""
from __future__ import annotations

import contextlib
import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzero_shard.so")
# test build: at most 65,536 threads per launch (every entry point splits early)
# and the step's streaming loads at every size
SMALLGRID_LIB_PATH = os.path.join(_HERE, "libzero_shard_smallgrid.so")

ZS_OK = 0
ZS_EINVAL_PSI = -1
ZS_EINVAL_ND = -2
ZS_EINVAL_RANK = -3
ZS_EINVAL_LAYOUT = -4
ZS_EALIGN = -5
ZS_EINVAL_HPARAM = -6
ZS_EINVAL_STAGE = -7
ZS_ENULL = -8
ZS_EUNSUPPORTED = -9
ZS_EWORKSPACE = -10
ZS_ELAUNCH = -11
ZS_EINVAL_REDUCE = -12
ZS_EZERO_TOKENS = -13
ZS_EINVAL_UNITS = -14
ZS_ESCRATCH = -15
ZS_SCRATCH_BYTES = 16 << 20
ZS_GRAD_BF16 = 0
ZS_GRAD_F32 = 1
ZS_MAX_RANKS = 64
ZS_OUT_GATHER = 0
ZS_OUT_SHARD = 1


class ZSError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {zs_strerror(code)} (code {code})")
        self.code = code


class zs_shard(C.Structure):
    _fields_ = [("psi", C.c_int64), ("n_d", C.c_int32), ("rank", C.c_int32),
                ("align", C.c_int64), ("shard_len", C.c_int64), ("shard_offset", C.c_int64),
                ("valid_len", C.c_int64), ("stage", C.c_int32), ("out_mode", C.c_int32)]

    def __repr__(self):
        return ("zs_shard(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_)
                + ")")


class zs_adamw(C.Structure):
    _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double),
                ("eps", C.c_double), ("weight_decay", C.c_double), ("step", C.c_int64),
                ("max_grad_norm", C.c_double)]


class zs_reduce(C.Structure):
    _fields_ = [("grad_dtype", C.c_int32), ("micro", C.c_int32), ("micro_count", C.c_int32),
                ("reserved", C.c_int32), ("rank_tokens", C.POINTER(C.c_int64))]


_lib = None


def _open(path: str):
    """Load one build of the library and declare its entry points."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with __graft_entry__.build(); "
                          "there is no CPU fallback")
    L = C.CDLL(path)
    P, vp, i32, i64, f64 = C.POINTER, C.c_void_p, C.c_int32, C.c_int64, C.c_double
    L.zs_layout.argtypes = [i64, i32, i32, i64, i32, i32, P(zs_shard)]
    L.zs_layout.restype = C.c_int
    L.zs_workspace_bytes.argtypes = [P(zs_shard)]
    L.zs_workspace_bytes.restype = C.c_size_t
    L.zs_state_bytes.argtypes = [f64, i32, i32, f64]
    L.zs_state_bytes.restype = f64
    L.zs_comm_bytes.argtypes = [f64, i32, i32, f64]
    L.zs_comm_bytes.restype = f64
    L.shard_grad_sqnorm.argtypes = [P(zs_shard), vp, vp, vp, C.c_size_t, vp, i32, vp]
    L.shard_grad_sqnorm.restype = C.c_int
    L.zs_workspace_bytes_units.argtypes = [P(zs_shard), i32]
    L.zs_workspace_bytes_units.restype = C.c_size_t
    L.shard_grad_sqnorm_units.argtypes = [P(zs_shard), i32, vp, vp, vp, C.c_size_t, vp,
                                          i32, vp]
    L.shard_grad_sqnorm_units.restype = C.c_int
    L.shard_grad_reduce.argtypes = [P(zs_shard), P(zs_reduce), vp, vp, vp, C.c_size_t,
                                    vp, i32, vp]
    L.shard_grad_reduce.restype = C.c_int
    L.zero_shard_step.argtypes = [P(zs_shard), P(zs_adamw), vp, vp, vp, f64, vp, vp, vp,
                                  vp, vp]
    L.zero_shard_step.restype = C.c_int
    L.shard_pack_gather.argtypes = [P(zs_shard), vp, vp, vp]
    L.shard_pack_gather.restype = C.c_int
    L.zs_strerror.argtypes = [C.c_int]
    L.zs_strerror.restype = C.c_char_p
    L.shard_grad_sqnorm_noalloc.argtypes = [P(zs_shard), vp, vp, vp, i32, vp]
    L.shard_grad_sqnorm_noalloc.restype = C.c_int
    L.zs_init.argtypes = []
    L.zs_init.restype = C.c_int
    return L


def lib():
    """Load libzero_shard.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _open(LIB_PATH)
    return _lib


@contextlib.contextmanager
def library(path: str):
    """Route every call of this module through another build of the same
    ABI (the small-grid test build) while the context is open."""
    global _lib
    saved = lib()
    _lib = _open(path)
    try:
        yield _lib
    finally:
        _lib = saved


def zs_strerror(code: int) -> str:
    return lib().zs_strerror(code).decode()


def _check(rc: int, what: str) -> None:
    if rc != ZS_OK:
        raise ZSError(rc, what)


_F32 = ("float32",)
_F64 = ("float64",)
_B16 = ("int16", "bfloat16", "uint16")      # bf16 bit patterns
_ANY = None


def _ptr(t, what: str = "buffer", dtypes=_ANY, min_numel: int = 0):
    """Device address of a tensor, an int address, or None.

    A torch tensor must have one of `dtypes` (torch dtype names; None: any),
    be contiguous, hold at least `min_numel` elements (what the call reads or
    writes through it) and live on the GPU; otherwise ValueError, before the
    C ABI is called.  An int is passed through unchecked."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not hasattr(t, "data_ptr"):
        raise TypeError(f"{what}: a torch tensor, an int device address or None is required")
    name = str(t.dtype).replace("torch.", "")
    if dtypes is not None and name not in dtypes:
        raise ValueError(f"{what}: dtype {name}, expected {' or '.join(dtypes)}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: the tensor must be contiguous")
    if t.numel() < min_numel:
        raise ValueError(f"{what}: {t.numel()} elements, the call needs {min_numel}")
    if not t.is_cuda:
        raise ValueError(f"{what}: a GPU tensor is required (got {t.device})")
    return t.data_ptr()


def _bytes_ptr(t, what: str, nbytes: int):
    """As _ptr for a buffer of any dtype that must hold `nbytes` bytes."""
    if t is not None and not isinstance(t, int) and hasattr(t, "numel"):
        if t.numel() * t.element_size() < nbytes:
            raise ValueError(f"{what}: {t.numel() * t.element_size()} bytes, the call needs "
                             f"{nbytes}")
    return _ptr(t, what)


def _out_len(s: "zs_shard") -> int:
    """Elements of param_out the step or the pack writes up to: the slot
    [shard_offset, shard_offset + shard_len) of the gather buffer, or the
    rank's own shard."""
    return s.shard_len + (s.shard_offset if s.out_mode == ZS_OUT_GATHER else 0)


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _slices(grad_slices, count: int, valid_len: int = 0, dtypes=_B16):
    """The host array of device pointers the C ABI reads `count` entries of
    (each slice tensor must hold valid_len elements of `dtypes`)."""
    if grad_slices is None:
        return None
    if len(grad_slices) != count:
        raise ValueError(f"{len(grad_slices)} gradient slice pointers given, {count} needed")
    arr = (C.c_void_p * count)(*[_ptr(g, f"grad_slices[{i}]", dtypes, valid_len)
                                 for i, g in enumerate(grad_slices)])
    return arr


# ---- host calls ------------------------------------------------------------------

def zs_init() -> None:
    """Per-device set-up of the current device (before capturing library
    calls into a HIP graph)."""
    _check(lib().zs_init(), "zs_init")


def zs_layout(psi: int, n_d: int, rank: int, align: int, stage: int = 2,
              out_mode: int = ZS_OUT_GATHER) -> zs_shard:
    s = zs_shard()
    _check(lib().zs_layout(psi, n_d, rank, align, stage, out_mode, C.byref(s)), "zs_layout")
    return s


def zs_workspace_bytes(s: zs_shard) -> int:
    return lib().zs_workspace_bytes(C.byref(s))


def zs_state_bytes(psi, n_d, stage, K=12.0) -> float:
    return lib().zs_state_bytes(float(psi), n_d, stage, float(K))


def zs_comm_bytes(psi, n_d, stage, bytes_per_elem=2.0) -> float:
    return lib().zs_comm_bytes(float(psi), n_d, stage, float(bytes_per_elem))


def adamw(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=1,
          max_grad_norm=0.0) -> zs_adamw:
    return zs_adamw(lr, beta1, beta2, eps, weight_decay, int(step), max_grad_norm)


# ---- device calls (enqueue on `stream`; torch tensors or raw addresses) ------------

def shard_grad_sqnorm(s: zs_shard, grad_slices, mean_out, workspace, sqnorm_out,
                      accumulate: bool = False, stream=None, workspace_bytes=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = (workspace.numel() * workspace.element_size()
                           if hasattr(workspace, "numel") else zs_workspace_bytes(s))
    V = s.valid_len
    _check(lib().shard_grad_sqnorm(C.byref(s), _slices(grad_slices, s.n_d, V),
                                   _ptr(mean_out, "mean_out", _F32, V),
                                   _bytes_ptr(workspace, "workspace", workspace_bytes),
                                   workspace_bytes, _ptr(sqnorm_out, "sqnorm_out", _F64, 1),
                                   1 if accumulate else 0, _stream(stream)),
           "shard_grad_sqnorm")


def shard_grad_sqnorm_noalloc(s: zs_shard, grad_slices, mean_out, sqnorm_out,
                              accumulate: bool = False, stream=None) -> None:
    """shard_grad_sqnorm without a workspace argument: the library's static
    per-device scratch array holds the block partials (no allocation)."""
    V = s.valid_len
    _check(lib().shard_grad_sqnorm_noalloc(C.byref(s), _slices(grad_slices, s.n_d, V),
                                           _ptr(mean_out, "mean_out", _F32, V),
                                           _ptr(sqnorm_out, "sqnorm_out", _F64, 1),
                                           1 if accumulate else 0, _stream(stream)),
           "shard_grad_sqnorm_noalloc")


def zs_workspace_bytes_units(s: zs_shard, units: int) -> int:
    return lib().zs_workspace_bytes_units(C.byref(s), units)


def shard_grad_sqnorm_units(s: zs_shard, grad_slices, mean_out, workspace, sqnorm_out,
                            accumulate: bool = False, stream=None, workspace_bytes=None) -> None:
    """grad_slices: flat list of units * n_d device pointers (unit-major);
    mean_out: None or a list of `units` fp32 buffers (entries may be None)."""
    units = len(grad_slices) // s.n_d
    if units * s.n_d != len(grad_slices):
        raise ValueError("grad_slices must hold units * n_d pointers")
    means = None
    if mean_out is not None:
        if len(mean_out) != units:
            raise ValueError("one mean buffer per unit")
        means = (C.c_void_p * units)(*[_ptr(m, f"mean_out[{u}]", _F32, s.valid_len)
                                       for u, m in enumerate(mean_out)])
    if workspace_bytes is None:
        workspace_bytes = (workspace.numel() * workspace.element_size()
                           if hasattr(workspace, "numel") else zs_workspace_bytes_units(s, units))
    _check(lib().shard_grad_sqnorm_units(C.byref(s), units,
                                         _slices(grad_slices, units * s.n_d, s.valid_len),
                                         means, _bytes_ptr(workspace, "workspace",
                                                           workspace_bytes),
                                         workspace_bytes, _ptr(sqnorm_out, "sqnorm_out", _F64, 1),
                                         1 if accumulate else 0, _stream(stream)),
           "shard_grad_sqnorm_units")


def make_reduce(grad_dtype: int = ZS_GRAD_BF16, micro: int = 0, micro_count: int = 1,
                rank_tokens=None):
    """A zs_reduce; the token array it points to is kept alive on it."""
    r = zs_reduce(grad_dtype, micro, micro_count, 0, None)
    if rank_tokens is not None:
        arr = (C.c_int64 * len(rank_tokens))(*[int(t) for t in rank_tokens])
        r.rank_tokens = C.cast(arr, C.POINTER(C.c_int64))
        r._tokens = arr
    return r


def shard_grad_reduce(s: zs_shard, r: zs_reduce, grad_slices, grad_out, workspace=None,
                      sqnorm_out=None, accumulate: bool = False, stream=None,
                      workspace_bytes=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = (workspace.numel() * workspace.element_size()
                           if hasattr(workspace, "numel") else
                           (zs_workspace_bytes(s) if workspace is not None else 0))
    tokens = getattr(r, "_tokens", None)
    if r.rank_tokens and (tokens is None or len(tokens) != s.n_d):
        raise ValueError(f"rank_tokens must hold n_d = {s.n_d} counts")
    V = s.valid_len
    gtypes = _F32 if r.grad_dtype == ZS_GRAD_F32 else _B16
    _check(lib().shard_grad_reduce(C.byref(s), C.byref(r), _slices(grad_slices, s.n_d, V, gtypes),
                                   _ptr(grad_out, "grad_out", _F32, V),
                                   _bytes_ptr(workspace, "workspace", workspace_bytes),
                                   workspace_bytes, _ptr(sqnorm_out, "sqnorm_out", _F64, 1),
                                   1 if accumulate else 0, _stream(stream)),
           "shard_grad_reduce")


def zero_shard_step(s: zs_shard, h: zs_adamw, grad_slices=None, mean_in=None, sqnorm=None,
                    other_sqnorm: float = 0.0, master=None, exp_avg=None, exp_avg_sq=None,
                    param_out=None, stream=None) -> None:
    V = s.valid_len
    _check(lib().zero_shard_step(C.byref(s), C.byref(h), _slices(grad_slices, s.n_d, V),
                                 _ptr(mean_in, "mean_in", _F32, V),
                                 _ptr(sqnorm, "sqnorm", _F64, 1), float(other_sqnorm),
                                 _ptr(master, "master", _F32, V),
                                 _ptr(exp_avg, "exp_avg", _F32, V),
                                 _ptr(exp_avg_sq, "exp_avg_sq", _F32, V),
                                 _ptr(param_out, "param_out", _B16, _out_len(s)),
                                 _stream(stream)), "zero_shard_step")


def shard_pack_gather(s: zs_shard, master, param_out, stream=None) -> None:
    _check(lib().shard_pack_gather(C.byref(s), _ptr(master, "master", _F32, s.valid_len),
                                   _ptr(param_out, "param_out", _B16, _out_len(s)),
                                   _stream(stream)), "shard_pack_gather")


def build(verbose: bool = False) -> str:
    from . import _build
    return _build.build(verbose)
