"""Seeded synthetic inputs for the sharded optimizer step.

The one module that serves both the CPU oracle's side and the GPU side.  It
holds none of the optimizer step's arithmetic: it only draws the inputs
(fp32 master weights and moments, per-rank bf16 gradients) from the counter
based generator defined in ``zsg_def.h``.  The host library fills numpy
arrays (threaded); the device library fills GPU buffers in place.  Both give
the same bits for the same (seed, stream, rank, step, index).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

from .workloads import WORKLOADS, Workload, grad_stream, state_stream  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libzsg_host.so")
DEV_LIB = os.path.join(_HERE, "libzsg_device.so")

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-ffp-contract=off", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-std=c++17"]


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def build(verbose: bool = False) -> None:
    """Build the host (gcc) and device (hipcc, gfx950) generator libraries."""
    cmds = [
        ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11",
         "-pthread", "-Wall", "-o", HOST_LIB + ".tmp", os.path.join(_HERE, "zsg_host.c"), "-lm"],
        ["hipcc", *HIP_FLAGS, "-o", DEV_LIB + ".tmp", os.path.join(_HERE, "zsg_device.hip")],
    ]
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd))
        subprocess.run(cmd, check=True)
    os.replace(HOST_LIB + ".tmp", HOST_LIB)
    os.replace(DEV_LIB + ".tmp", DEV_LIB)


_host = None
_dev = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"{HOST_LIB} missing: run __graft_entry__.build()")
        L = C.CDLL(HOST_LIB)
        u64, u32, i64, f64, vp, ci = C.c_uint64, C.c_uint32, C.c_int64, C.c_double, C.c_void_p, C.c_int
        L.zsg_fill_f32.argtypes = [u64, u32, u32, u32, f64, ci, i64, i64, vp, ci]
        L.zsg_fill_bf16.argtypes = [u64, u32, u32, u32, f64, f64, f64, i64, i64, vp, ci]
        L.zsg_gather_f32.argtypes = [u64, u32, u32, u32, f64, ci, vp, i64, vp, ci]
        L.zsg_gather_bf16.argtypes = [u64, u32, u32, u32, f64, f64, f64, vp, i64, vp, ci]
        for f in (L.zsg_fill_f32, L.zsg_fill_bf16, L.zsg_gather_f32, L.zsg_gather_bf16):
            f.restype = ci
        _host = L
    return _host


def _dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"{DEV_LIB} missing: run __graft_entry__.build()")
        L = C.CDLL(DEV_LIB)
        u64, u32, i64, f64, vp, ci = C.c_uint64, C.c_uint32, C.c_int64, C.c_double, C.c_void_p, C.c_int
        L.zsg_dev_fill_f32.argtypes = [u64, u32, u32, u32, f64, ci, i64, i64, vp, vp]
        L.zsg_dev_fill_bf16.argtypes = [u64, u32, u32, u32, f64, f64, f64, i64, i64, vp, vp]
        L.zsg_dev_fill_f32.restype = ci
        L.zsg_dev_fill_bf16.restype = ci
        _dev = L
    return _dev


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


# ---- host ---------------------------------------------------------------------

def host_f32(seed, stream, rank, step, sigma, start, n, absval=False, out=None,
             threads=None) -> np.ndarray:
    """fp32 sigma*N(0,1) (|.| if absval) for elements start .. start+n-1."""
    if out is None:
        out = np.empty(n, np.float32)
    assert out.dtype == np.float32 and out.size == n and out.flags.c_contiguous
    _check(_host_lib().zsg_fill_f32(seed, stream, rank, step, float(sigma), int(absval),
                                    start, n, out.ctypes.data, threads or default_threads()),
           "zsg_fill_f32")
    return out


def host_bf16(seed, stream, rank, step, sigma, start, n, p_out=0.0, sigma_out=0.0,
              out=None, threads=None) -> np.ndarray:
    """bf16 bit patterns (uint16) of sigma*N(0,1), outliers with prob p_out."""
    if out is None:
        out = np.empty(n, np.uint16)
    assert out.dtype == np.uint16 and out.size == n and out.flags.c_contiguous
    _check(_host_lib().zsg_fill_bf16(seed, stream, rank, step, float(sigma), float(p_out),
                                     float(sigma_out), start, n, out.ctypes.data,
                                     threads or default_threads()), "zsg_fill_bf16")
    return out


def host_f32_at(seed, stream, rank, step, sigma, idx, absval=False, threads=None):
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, np.float32)
    _check(_host_lib().zsg_gather_f32(seed, stream, rank, step, float(sigma), int(absval),
                                      idx.ctypes.data, idx.size, out.ctypes.data,
                                      threads or default_threads()), "zsg_gather_f32")
    return out


def host_bf16_at(seed, stream, rank, step, sigma, idx, p_out=0.0, sigma_out=0.0,
                 threads=None):
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, np.uint16)
    _check(_host_lib().zsg_gather_bf16(seed, stream, rank, step, float(sigma), float(p_out),
                                       float(sigma_out), idx.ctypes.data, idx.size,
                                       out.ctypes.data, threads or default_threads()),
           "zsg_gather_bf16")
    return out


# ---- device (torch tensors as plain device memory) ------------------------------

def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return int(stream)


def dev_f32(t, seed, stream, rank, step, sigma, start, absval=False, hip_stream=None):
    """Fill the float32 device tensor t (contiguous) with elements start..start+numel-1."""
    import torch
    assert t.is_cuda and t.dtype == torch.float32 and t.is_contiguous()
    _check(_dev_lib().zsg_dev_fill_f32(seed, stream, rank, step, float(sigma), int(absval),
                                       start, t.numel(), t.data_ptr(),
                                       _stream_handle(hip_stream)), "zsg_dev_fill_f32")
    return t


def dev_bf16(t, seed, stream, rank, step, sigma, start, p_out=0.0, sigma_out=0.0,
             hip_stream=None):
    """Fill the 2-byte device tensor t (bfloat16/int16/uint16) in place."""
    assert t.is_cuda and t.element_size() == 2 and t.is_contiguous()
    _check(_dev_lib().zsg_dev_fill_bf16(seed, stream, rank, step, float(sigma), float(p_out),
                                        float(sigma_out), start, t.numel(), t.data_ptr(),
                                        _stream_handle(hip_stream)), "zsg_dev_fill_bf16")
    return t
