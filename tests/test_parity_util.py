"""The element-by-element comparison behind the full-size parity tests, as
host logic (no GPU): on the oracle's own step of a small shard it counts
nothing; a one-ulp change in w, m, v or the bf16 output is counted and stays
within the bars; an error past the fp32 or bf16 bar, or any change in the
stored gradient, fails.  CPU tensors stand in for the device arrays."""
import dataclasses
import types

import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_zero_amd as Z
import oracle as O
from zsgen.workloads import WORKLOADS
from parity_util import (compare_unit_full, compare_unit_streamed, hparams, host_state,
                         oracle_sqnorm_chunked)

CHUNK = 100_000     # several chunks and a ragged last one over the 262,144-parameter shard


def _oracle_run(clip: bool):
    """A stand-in `run` whose unit holds the oracle's result of one step of
    the tiny workload (optionally with a clip), plus that workload, its
    gradient, squared norm and clip coefficient."""
    wl = WORKLOADS["tiny"]
    if clip:
        wl = dataclasses.replace(wl, max_grad_norm=0.1)   # the norm is ~0.26
    s = Z.zs_layout(wl.psi, wl.n_d, wl.rank, wl.align, wl.stage)
    V, off = s.valid_len, s.shard_offset
    q, g = oracle_sqnorm_chunked(wl, 0, wl.t0, off, V, keep_all=True)
    coef = O.clip_coef(q, wl.max_grad_norm) if clip else None
    w, m, v = host_state(wl, 0, off, V)
    O.adamw_f32(hparams(wl, wl.t0), g, w, m, v, coef=coef)
    out = np.full(wl.n_d * s.shard_len, 0x7FC1, np.uint16)
    out[off:off + V] = O.bf16_rne(w)
    unit = types.SimpleNamespace(w=torch.from_numpy(w), m=torch.from_numpy(m),
                                 v=torch.from_numpy(v),
                                 out=torch.from_numpy(out.view(np.int16)),
                                 mean=torch.from_numpy(g.copy()))
    return types.SimpleNamespace(shard=s, units_data=[unit]), wl, g, q, coef


def _bump(t: torch.Tensor, i: int, ulps: int):
    """Move element i of an fp32 or bf16-bits tensor by `ulps` bit steps."""
    if t.dtype == torch.float32:
        t.view(torch.int32)[i] += ulps
    else:
        t[i] += ulps


@pytest.mark.parametrize("clip", [False, True])
def test_full_compare_counts_nothing_on_the_oracle_result(clip):
    run, wl, g, q, coef = _oracle_run(clip)
    if clip:
        assert coef < 1, "the clip binds"
    assert compare_unit_full("oracle", wl, run, 0, wl.t0, g, coef, chunk=CHUNK) == 0
    q2, nb = compare_unit_streamed("oracle", wl, run, 0, wl.t0, coef, chunk=CHUNK)
    assert nb == 0 and q2 == q


def test_full_compare_counts_one_ulp_changes():
    run, wl, g, _, coef = _oracle_run(True)
    d, off = run.units_data[0], run.shard.shard_offset
    V = run.shard.valid_len
    # one element in the first chunk, one at a chunk boundary, one in the ragged tail
    _bump(d.w, 7, 1)
    _bump(d.m, CHUNK, -1)
    _bump(d.v, V - 1, 1)
    _bump(d.out, off + 2 * CHUNK + 5, 1)
    assert compare_unit_full("planted", wl, run, 0, wl.t0, g, coef, chunk=CHUNK) == 4
    assert compare_unit_streamed("planted", wl, run, 0, wl.t0, coef, chunk=CHUNK)[1] == 4


@pytest.mark.parametrize("array,i,ulps", [("w", 3, 1 << 10), ("m", 150_000, -(1 << 12)),
                                          ("v", 262_143, 1 << 9), ("out", 11, 2),
                                          ("mean", 100_001, 1)])
def test_full_compare_fails_past_the_bars(array, i, ulps):
    run, wl, g, _, coef = _oracle_run(True)
    d = run.units_data[0]
    j = i + run.shard.shard_offset if array == "out" else i
    _bump(getattr(d, array), j, ulps)
    with pytest.raises(AssertionError):
        compare_unit_full("planted", wl, run, 0, wl.t0, g, coef, chunk=CHUNK)
