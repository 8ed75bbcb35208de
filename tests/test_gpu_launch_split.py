"""The multi-launch path of every entry point, on the small-grid test build.

A dispatch counts its work-items in 32 bits, so the library splits a shard
whose grid would be longer into several launches (from 8.6e9 parameters on:
shards that fit the 288 GB of one MI355X once the state is small, e.g. the
norm of a large N_d = 1 shard).  The test build libzero_shard_smallgrid.so is
the same source with at most 65,536 threads per launch: 524,288 parameters
per launch of the clip pass and of a step with 8 parameters per lane, 262,144
of the streaming step from a stored gradient (4 per lane).  Shards of 1-2 million
parameters with a ragged tail then cross several launch boundaries (the last
launch of the 64-slice clip pass has 13 blocks, so the XCD-contiguous block
mapping meets a grid that is not a multiple of 8).  The test build also takes
the step's streaming cache policy (non-temporal loads, sc1 and nt stores) at
every size, which the normal build uses only for steps that move 512 MiB or
more: the comparison with the normal build covers both policies.

Each output must equal the oracle's bit for bit (the squared norm within the
oracle's bar, Q_REL_BAR), equal the normal build's bit for bit, and leave
every byte outside its range untouched.  Run on an MI355X:  pytest -m gpu -s
"""
import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_zero_amd as Z
import oracle as O
from fsdp_sharded_optimizer_zero_amd._build import SMALLGRID_THREADS
from parity_util import Q_REL_BAR, coef_is_robust, log
from reduce_util import run_reduce_case

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC1                     # bf16 NaN pattern nothing in the step writes
F32_GUARD = np.uint32(0x7FC00ABC)     # fp32 NaN pattern nothing writes
GUARD = 64
PARAMS_PER_LAUNCH = SMALLGRID_THREADS * 8


@pytest.fixture(autouse=True)
def _free_gpu_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _bf16_slices(rng, n_d, V):
    return [O.bf16_rne(rng.normal(0, 1e-3, V).astype(np.float32)) for _ in range(n_d)]


def _rows(slices, S, V):
    """Device [n_d, S] bf16 rows; beyond V they hold +Inf the kernels must not read."""
    rows = torch.full((len(slices), S), 0x7F80, dtype=torch.int16)
    for r, sl in enumerate(slices):
        rows[r, :V] = torch.from_numpy(sl[:V].view(np.int16))
    return rows.cuda()


def _guarded(x):
    """fp32 array on the device with GUARD NaN-pattern words after it."""
    buf = np.full(x.size + GUARD, F32_GUARD, np.uint32)
    buf[:x.size] = x.view(np.uint32)
    return torch.from_numpy(buf.view(np.float32)).cuda()


def _f32(t, n):
    return t.cpu().numpy()[:n].copy()


def _guard_intact(t, n):
    return bool(np.all(t.cpu().numpy().view(np.uint32)[n:] == F32_GUARD))


def _clip_then_step(path, s, slices, w0, m0, v0, h, reread=False):
    """shard_grad_sqnorm (mean stored) then zero_shard_step(mean_in) with the
    build at `path`, or with `reread` the norm alone then the step from the
    slices; returns the host copies of every output."""
    S, V, n_d = s.shard_len, s.valid_len, s.n_d
    rows = _rows(slices, S, V)
    ptrs = [rows.data_ptr() + 2 * S * r for r in range(n_d)]
    mean = _guarded(np.zeros(V, np.float32))
    w, m, v = _guarded(w0), _guarded(m0), _guarded(v0)
    out = torch.full((n_d * S,), SENTINEL, dtype=torch.int16, device="cuda")
    ws = torch.empty(Z.zs_workspace_bytes(s) // 8, dtype=torch.float64, device="cuda")
    sq = torch.zeros(1, dtype=torch.float64, device="cuda")
    with Z.library(path):
        if reread:
            Z.shard_grad_sqnorm(s, ptrs, None, ws, sq)
            Z.zero_shard_step(s, h, grad_slices=ptrs, sqnorm=sq, master=w, exp_avg=m,
                              exp_avg_sq=v, param_out=out)
        else:
            Z.shard_grad_sqnorm(s, ptrs, mean, ws, sq)
            Z.zero_shard_step(s, h, mean_in=mean, sqnorm=sq, master=w, exp_avg=m,
                              exp_avg_sq=v, param_out=out)
    torch.cuda.synchronize()
    assert all(_guard_intact(t, V) for t in (mean, w, m, v)), "wrote past valid_len"
    return dict(mean=_f32(mean, V), w=_f32(w, V), m=_f32(m, V), v=_f32(v, V),
                out=out.cpu().numpy().view(np.uint16).copy(), q=float(sq.item()))


@pytest.mark.parametrize("n_d,per_rank,tail,max_norm,reread", [(8, 1_600_000, 5, 1.0, False),
                                                               (64, 1_100_000, 13, 1.0, False),
                                                               (8, 1_600_000, 5, 0.0, False),
                                                               (8, 1_600_000, 5, 1.0, True)])
def test_split_clip_pass_and_step(n_d, per_rank, tail, max_norm, reread):
    """The clip pass with the mean stored, then the step from the stored mean
    (with the global clip, or without one: max_norm 0); or the norm alone,
    then the clipped step from the slices (re-read schedule).  Against the
    normal build and the oracle."""
    psi = n_d * per_rank - tail
    rank = n_d - 1                                  # the ragged last rank
    s = Z.zs_layout(psi, n_d, rank, 8, 2)
    S, V, base = s.shard_len, s.valid_len, s.shard_offset
    assert V < S and S > 2 * PARAMS_PER_LAUNCH
    rng = np.random.default_rng(1000 + n_d)
    slices = _bf16_slices(rng, n_d, V)
    w0 = rng.normal(0, 0.02, V).astype(np.float32)
    m0 = rng.normal(0, 1e-4, V).astype(np.float32)
    v0 = np.abs(rng.normal(0, 1e-6, V)).astype(np.float32)
    zh = Z.adamw(lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1, step=1000,
                 max_grad_norm=max_norm)
    oh = O.Hparams(lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1, step=1000,
                   max_grad_norm=max_norm)
    log(f"split clip+step n_d={n_d} V={V} S={S} max_norm={max_norm} reread={reread}: "
        f"{-(-S // PARAMS_PER_LAUNCH)} step launches")
    small = _clip_then_step(Z.SMALLGRID_LIB_PATH, s, slices, w0, m0, v0, zh, reread)
    normal = _clip_then_step(Z.LIB_PATH, s, slices, w0, m0, v0, zh, reread)
    for k in (("w", "m", "v") if reread else ("mean", "w", "m", "v")):
        assert np.array_equal(small[k].view(np.uint32), normal[k].view(np.uint32)), k
    assert np.array_equal(small["out"], normal["out"])
    assert small["q"] == normal["q"], "same partials in the same order"

    w, m, v = w0.copy(), m0.copy(), v0.copy()
    out, q, coef = O.shard_step(n_d, S, V, oh, slices, w, m, v)
    if not reread:
        assert np.array_equal(small["mean"].view(np.uint32),
                              O.reduce_mean(slices).view(np.uint32))
    assert abs(small["q"] - q) <= Q_REL_BAR * q
    if max_norm > 0:
        assert coef_is_robust(q, oh.max_grad_norm), "draw another seed"
    for k, ref in (("w", w), ("m", m), ("v", v)):
        assert np.array_equal(small[k].view(np.uint32), ref.view(np.uint32)), k
    assert np.array_equal(small["out"][base:base + S], out)
    assert np.all(np.delete(small["out"], np.arange(base, base + S)) == SENTINEL)


def test_split_fused_step_and_pack():
    """zero_shard_step from the slices (no clip) and shard_pack_gather."""
    n_d, psi = 4, 4 * 1_300_000 - 3
    s = Z.zs_layout(psi, n_d, 3, 8, 2)
    S, V, base = s.shard_len, s.valid_len, s.shard_offset
    rng = np.random.default_rng(77)
    slices = _bf16_slices(rng, n_d, V)
    w0 = rng.normal(0, 0.02, V).astype(np.float32)
    zh = Z.adamw(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=3)
    oh = O.Hparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=3)
    rows = _rows(slices, S, V)
    ptrs = [rows.data_ptr() + 2 * S * r for r in range(n_d)]
    zeros = np.zeros(V, np.float32)
    w, m, v = _guarded(w0), _guarded(zeros), _guarded(zeros)
    out = torch.full((n_d * S,), SENTINEL, dtype=torch.int16, device="cuda")
    packed = torch.full((S,), SENTINEL, dtype=torch.int16, device="cuda")
    so = Z.zs_layout(psi, n_d, 3, 8, 3, Z.ZS_OUT_SHARD)
    with Z.library(Z.SMALLGRID_LIB_PATH):
        Z.zero_shard_step(s, zh, grad_slices=ptrs, master=w, exp_avg=m, exp_avg_sq=v,
                          param_out=out)
        Z.shard_pack_gather(so, w, packed)
    torch.cuda.synchronize()
    ow, om, ov = w0.copy(), zeros.copy(), zeros.copy()
    oout, _, _ = O.shard_step(n_d, S, V, oh, slices, ow, om, ov)
    for name, got, ref in (("w", w, ow), ("m", m, om), ("v", v, ov)):
        assert _guard_intact(got, V), name
        assert np.array_equal(_f32(got, V).view(np.uint32), ref.view(np.uint32)), name
    gout = out.cpu().numpy().view(np.uint16)
    assert np.array_equal(gout[base:base + S], oout)
    assert np.all(np.delete(gout, np.arange(base, base + S)) == SENTINEL)
    assert np.array_equal(packed.cpu().numpy().view(np.uint16), O.pack(S, ow))


def test_split_units():
    """shard_grad_sqnorm_units over 3 units: the block partials of unit u sit
    at u * blocks, each unit split over several launches."""
    n_d, units, psi = 4, 3, 4 * 1_200_000 - 7
    s = Z.zs_layout(psi, n_d, 3, 8, 2)
    S, V = s.shard_len, s.valid_len
    rng = np.random.default_rng(5)
    all_slices = [_bf16_slices(rng, n_d, V) for _ in range(units)]
    rows = [_rows(sl, S, V) for sl in all_slices]
    ptrs = [r.data_ptr() + 2 * S * k for r in rows for k in range(n_d)]
    results = {}
    for path in (Z.SMALLGRID_LIB_PATH, Z.LIB_PATH):
        means = [_guarded(np.zeros(V, np.float32)) for _ in range(units)]
        ws = torch.empty(Z.zs_workspace_bytes_units(s, units) // 8, dtype=torch.float64,
                         device="cuda")
        sq = torch.zeros(1, dtype=torch.float64, device="cuda")
        with Z.library(path):
            Z.shard_grad_sqnorm_units(s, ptrs, means, ws, sq)
        torch.cuda.synchronize()
        assert all(_guard_intact(t, V) for t in means)
        results[path] = ([_f32(t, V) for t in means], float(sq.item()))
    (small_means, small_q), (normal_means, normal_q) = results.values()
    assert small_q == normal_q
    acc = O.SqAcc()
    for u in range(units):
        ref = O.reduce_mean(all_slices[u])
        assert np.array_equal(small_means[u].view(np.uint32), ref.view(np.uint32)), u
        assert np.array_equal(normal_means[u].view(np.uint32), ref.view(np.uint32)), u
        acc.add(ref)
    assert abs(small_q - acc.value()) <= Q_REL_BAR * acc.value()


@pytest.mark.parametrize("f32,tokens,m", [(True, None, 1), (False, [3, 0, 5, 9], 1),
                                          (False, None, 3), (True, [1, 2, 3, 4], 2)])
def test_split_reduce_modes(f32, tokens, m):
    """shard_grad_reduce: fp32 slices, token weights, micro-batch accumulation."""
    with Z.library(Z.SMALLGRID_LIB_PATH):
        run_reduce_case(4 * 1_100_000 - 9, 4, 3, f32, tokens, m, seed=31 + m)
