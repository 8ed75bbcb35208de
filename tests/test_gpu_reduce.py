"""GPU parity of shard_grad_reduce: fp32 gradient slices, token-weighted
ranks and ZeRO-2 gradient accumulation, through the C ABI, against the CPU
oracle (or_reduce_mean_f32in, or_reduce_weighted, or_accumulate).

Every expected value comes from the oracle on inputs drawn by the host side of
the seeded generator or by numpy on the host.  The reductions and the
accumulator are bit-exact by construction (the same fp32 operations in the
same order), and that is what is asserted; the squared norm is within 1e-12
of the oracle's exactly rounded sum.  Run on an MI355X:  pytest -m gpu -s
"""
import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_zero_amd as Z
import oracle as O
from fsdp_sharded_optimizer_zero_amd.runner import ShardRun
from zsgen.workloads import NEXT, WORKLOADS
from parity_util import Q_REL_BAR, coef_is_robust, compare_unit_full, log, oracle_sqnorm_chunked
from reduce_util import (F32_SENTINEL, GUARD, draw_slices, oracle_reduce, rows_on_device,
                         run_reduce_case)

pytestmark = pytest.mark.gpu

@pytest.fixture(autouse=True)
def _free_gpu_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_reduce_ragged_every_mode():
    n = 0
    for psi in (1, 9, 1000, 4099, 100_003):
        for n_d in (1, 3, 8, 64):
            if n_d == 64 and psi > 4099:
                continue
            for rank in sorted({0, n_d - 1}):
                for f32 in (False, True):
                    for weighted in (False, True):
                        tokens = None
                        if weighted:
                            tokens = [(7 * r + 3) % 11 for r in range(n_d)]
                            if sum(tokens) == 0:
                                tokens[0] = 1
                        for m in (1, 3):
                            run_reduce_case(psi, n_d, rank, f32, tokens, m, seed=n)
                            n += 1
    log(f"shard_grad_reduce: {n} ragged cases bit-exact")


def test_reduce_bf16_mean_is_the_sqnorm_path():
    """m = 1, bf16, no weights: the same bits as shard_grad_sqnorm."""
    rng = np.random.default_rng(31)
    s = Z.zs_layout(1_000_003, 8, 5, 8, 2)
    S, V = s.shard_len, s.valid_len
    sl = draw_slices(rng, 8, V, False)
    rows = rows_on_device(sl, 8, S, V, False)
    ptrs = [rows.data_ptr() + 2 * S * r for r in range(8)]
    a = torch.empty(V, dtype=torch.float32, device="cuda")
    b = torch.empty(V, dtype=torch.float32, device="cuda")
    ws = torch.empty(Z.zs_workspace_bytes(s) // 8, dtype=torch.float64, device="cuda")
    qa = torch.zeros(1, dtype=torch.float64, device="cuda")
    qb = torch.zeros(1, dtype=torch.float64, device="cuda")
    Z.shard_grad_sqnorm(s, ptrs, a, ws, qa)
    Z.shard_grad_reduce(s, Z.make_reduce(), ptrs, b, ws, qb)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert float(qa.item()) == float(qb.item())


def test_reduce_token_worked_example_on_gpu():
    """Ranks with 2 and 6 valid tokens, local mean gradients 3 and 1: 1.5."""
    s = Z.zs_layout(16, 2, 0, 8, 2)
    V = s.valid_len
    for f32 in (False, True):
        sl = ([np.full(V, 3.0, np.float32), np.full(V, 1.0, np.float32)] if f32 else
              [O.bf16_rne(np.full(V, 3.0, np.float32)), O.bf16_rne(np.full(V, 1.0, np.float32))])
        rows = rows_on_device(sl, 2, s.shard_len, V, f32)
        es = 4 if f32 else 2
        ptrs = [rows.data_ptr(), rows.data_ptr() + es * s.shard_len]
        out = torch.zeros(V, dtype=torch.float32, device="cuda")
        Z.shard_grad_reduce(s, Z.make_reduce(Z.ZS_GRAD_F32 if f32 else Z.ZS_GRAD_BF16,
                                             rank_tokens=[2, 6]), ptrs, out)
        torch.cuda.synchronize()
        assert bool((out == 1.5).all())


def test_reduce_zero_tokens_rejects_and_writes_nothing():
    rng = np.random.default_rng(32)
    s = Z.zs_layout(5000, 4, 2, 8, 2)
    S, V = s.shard_len, s.valid_len
    rows = rows_on_device(draw_slices(rng, 4, V, False), 4, S, V, False)
    ptrs = [rows.data_ptr() + 2 * S * r for r in range(4)]
    out = torch.full((V,), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(Z.ZSError) as e:
        Z.shard_grad_reduce(s, Z.make_reduce(rank_tokens=[0, 0, 0, 0]), ptrs, out)
    assert e.value.code == Z.ZS_EZERO_TOKENS
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


@pytest.mark.parametrize("name", NEXT)
def test_next_workloads_full_size(name):
    """One optimizer step of the 7B ZeRO-2 shard with fp32 slices, token
    weights, or 4 accumulated micro-batches: the oracle's squared norm over
    the whole shard, then every element of w, m, v, the bf16 slot and the
    stored gradient against the oracle's step from its own gradient."""
    wl = WORKLOADS[name]
    log(f"{name}: allocating and filling on the device")
    run = ShardRun(wl)
    run.fill_state(out_fill=0x7FC1)
    run.fill_grads(wl.t0)
    run.step(wl.t0)
    torch.cuda.synchronize()
    gq = float(run.sqnorm.item())
    V, s = run.V, run.shard
    log(f"{name}: GPU Q={gq:.6g}; oracle squared norm over {V:,} params")
    oq, og = oracle_sqnorm_chunked(wl, 0, wl.t0, s.shard_offset, V, keep_all=True)
    log(f"{name}: oracle Q={oq:.17g} GPU Q={gq:.17g}")
    assert abs(gq - oq) <= Q_REL_BAR * oq
    coef = O.clip_coef(oq, wl.max_grad_norm)
    nb = compare_unit_full(name, wl, run, 0, wl.t0, og, coef)
    del og
    d = run.units_data[0]
    assert bool((d.out[:s.shard_offset] == 0x7FC1).all())
    assert bool((d.out[s.shard_offset + s.shard_len:] == 0x7FC1).all())
    if coef_is_robust(oq, wl.max_grad_norm):
        assert nb == 0


@pytest.mark.parametrize("n_d,units", [(3, 1), (8, 3), (8, 5), (64, 2)])
def test_sqnorm_units_equals_per_unit_calls(n_d, units):
    """shard_grad_sqnorm_units over several FSDP units gives the bits of one
    shard_grad_sqnorm per unit (accumulate from the second on): the same
    means and the same squared norm, with and without a prior value."""
    rng = np.random.default_rng(40 + units)
    psi = 300_007 if n_d < 64 else 40_009
    s = Z.zs_layout(psi, n_d, n_d - 1, 8, 3)
    S, V = s.shard_len, s.valid_len
    rows = [rows_on_device(draw_slices(rng, n_d, V, False), n_d, S, V, False)
            for _ in range(units)]
    ptrs = [r.data_ptr() + 2 * S * k for r in rows for k in range(n_d)]
    means_a = [torch.empty(max(V, 8), dtype=torch.float32, device="cuda") for _ in range(units)]
    means_b = [torch.empty(max(V, 8), dtype=torch.float32, device="cuda") for _ in range(units)]
    ws1 = torch.empty(Z.zs_workspace_bytes(s) // 8, dtype=torch.float64, device="cuda")
    wsu = torch.empty(Z.zs_workspace_bytes_units(s, units) // 8, dtype=torch.float64,
                      device="cuda")
    for prior in (None, 3.25):
        qa = torch.full((1,), 0.0 if prior is None else prior, dtype=torch.float64, device="cuda")
        qb = qa.clone()
        for u in range(units):
            Z.shard_grad_sqnorm(s, ptrs[u * n_d:(u + 1) * n_d], means_a[u], ws1, qa,
                                accumulate=(u > 0 or prior is not None))
        Z.shard_grad_sqnorm_units(s, ptrs, means_b, wsu, qb, accumulate=prior is not None)
        torch.cuda.synchronize()
        assert float(qa.item()) == float(qb.item()), (prior, qa.item(), qb.item())
        for a, b in zip(means_a, means_b):
            assert torch.equal(a[:V].view(torch.int32), b[:V].view(torch.int32))
    # and against the oracle's exact norm over all units
    acc = O.SqAcc()
    for r in rows:
        sl = [r[k, :V].cpu().numpy().view(np.uint16).copy() for k in range(n_d)]
        acc.add(O.reduce_mean(sl))
    oq = acc.value() + 3.25
    assert abs(float(qb.item()) - oq) <= Q_REL_BAR * oq


def _same_values(got, ref):
    """Bit for bit on finite and infinite values; NaN matched as a class (a NaN
    that an operation creates has a processor-dependent sign)."""
    gn, rn = np.isnan(got), np.isnan(ref)
    return (np.array_equal(gn, rn) and
            np.array_equal(got[~gn].view(np.uint32), ref[~rn].view(np.uint32)))


@pytest.mark.parametrize("f32,tokens,m", [(True, None, 1), (False, [3, 1, 0, 5], 1),
                                          (False, None, 3), (True, [2, 2, 0, 1], 3)])
def test_reduce_non_finite(f32, tokens, m):
    """NaN and ±Inf in single ranks' slices through shard_grad_reduce (fp32
    slices, token weights, accumulation): IEEE propagation as the oracle does
    it, in full blocks and in the tail, including Inf + (-Inf) and a
    zero-token rank holding an Inf (0 * Inf)."""
    rng = np.random.default_rng(90 + m)
    psi, n_d, rank = 4 * 3000 + 5, 4, 3
    s = Z.zs_layout(psi, n_d, rank, 8, 2)
    S, V = s.shard_len, s.valid_len
    esize = 4 if f32 else 2
    nan, inf = np.float32("nan"), np.float32("inf")
    # (rank, index, value): idx 2 gets -Inf + Inf; idx 4 puts an Inf in rank 2
    # (a zero-token rank where weighted); V - 1 sits in the tail
    poison = [(0, 0, nan), (1, 5, inf), (2, 1000, -inf), (3, 1000, inf), (3, 2047, inf),
              (1, 2047, inf), (2, 2048, inf), (0, V - 1, -inf)]
    out = torch.from_numpy(np.full(V + GUARD, F32_SENTINEL, np.uint32).view(np.float32)).cuda()
    ws = torch.empty(Z.zs_workspace_bytes(s) // 8, dtype=torch.float64, device="cuda")
    sq = torch.zeros(1, dtype=torch.float64, device="cuda")
    acc = np.empty(V, np.float32)
    for j in range(m):
        sl = draw_slices(rng, n_d, V, f32)
        if j == m - 1:
            for r, i, x in poison:
                if f32:
                    sl[r][i] = x
                else:
                    sl[r][i] = O.bf16_rne(np.array([x], np.float32))[0]
        rows = rows_on_device(sl, n_d, S, V, f32)
        ptrs = [rows.data_ptr() + esize * S * r for r in range(n_d)]
        last = j == m - 1
        r = Z.make_reduce(Z.ZS_GRAD_F32 if f32 else Z.ZS_GRAD_BF16, j, m, tokens)
        Z.shard_grad_reduce(s, r, ptrs, out, ws if last else None, sq if last else None)
        torch.cuda.synchronize()
        O.accumulate(oracle_reduce(sl, tokens, f32), j, m, acc)
        got = out.cpu().numpy()[:V]
        case = f"f32={f32} tokens={tokens} j={j}/{m}"
        assert _same_values(got, acc), case
        assert np.all(out.cpu().numpy().view(np.uint32)[V:] == F32_SENTINEL), case
        del rows
    assert np.isnan(acc).sum() >= 2 and np.isinf(acc).any()
    q = O.sqnorm(acc)
    gq = float(sq.item())
    assert np.isnan(q) and np.isnan(gq), (q, gq)
