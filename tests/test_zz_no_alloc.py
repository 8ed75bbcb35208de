"""The allocation-free clip pass, shard_grad_sqnorm_noalloc, through the C ABI:
its output must equal that of shard_grad_sqnorm (the same kernels with a
caller workspace) bit for bit -- the stored mean and the fp64 squared norm --
and match the oracle (mean bit for bit, squared norm within 1e-12 of the
exactly rounded sum), on calls in a row of decreasing size, so that what an
earlier call left in the shared static array cannot leak into a later one.
"""
import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_zero_amd as Z
import oracle as O
import zsgen
from parity_util import Q_REL_BAR, log
from reduce_util import F32_SENTINEL, GUARD, rows_on_device

pytestmark = pytest.mark.gpu


def _mean_buf(V):
    return torch.from_numpy(np.full(V + GUARD, F32_SENTINEL, np.uint32).view(np.float32)).cuda()


def _bits64(t):
    return int(t.view(torch.int64).item())


def _case(psi, n_d, rank, seed, store=True, prior=None):
    """One shard through both entry points; returns the squared norm."""
    rng = np.random.default_rng(seed)
    s = Z.zs_layout(psi, n_d, rank, 8, 2)
    S, V = s.shard_len, s.valid_len
    sl = [O.bf16_rne(rng.normal(0, 1e-3, V).astype(np.float32)) for _ in range(n_d)]
    rows = rows_on_device(sl, n_d, S, V, False)
    ptrs = [rows.data_ptr() + 2 * S * r for r in range(n_d)]
    acc = prior is not None
    init = 0.0 if prior is None else prior
    mean_a, mean_b = (_mean_buf(V), _mean_buf(V)) if store else (None, None)
    sq_a = torch.full((1,), init, dtype=torch.float64, device="cuda")
    sq_b = torch.full((1,), init, dtype=torch.float64, device="cuda")
    ws = torch.empty(Z.zs_workspace_bytes(s) // 8, dtype=torch.float64, device="cuda")
    Z.shard_grad_sqnorm(s, ptrs, mean_a, ws, sq_a, accumulate=acc)
    Z.shard_grad_sqnorm_noalloc(s, ptrs, mean_b, sq_b, accumulate=acc)
    torch.cuda.synchronize()
    case = f"psi={psi} n_d={n_d} k={rank} V={V} store={store} prior={prior}"
    assert _bits64(sq_a) == _bits64(sq_b), f"{case}: squared norm bits differ"
    og = O.reduce_mean(sl)
    oq = init + O.sqnorm(og)
    gq = float(sq_b.item())
    assert abs(gq - oq) <= Q_REL_BAR * max(oq, 1e-300), f"{case}: {gq} vs oracle {oq}"
    if store:
        a = mean_a.cpu().numpy().view(np.uint32)
        b = mean_b.cpu().numpy().view(np.uint32)
        assert np.array_equal(a, b), f"{case}: means differ"
        assert np.array_equal(b[:V], og.view(np.uint32)), f"{case}: mean vs oracle"
        assert np.all(b[V:] == F32_SENTINEL), f"{case}: wrote past valid_len"
    log(f"noalloc == workspace call, {case}: Q={gq:.6g}")
    return gq


def test_noalloc_equals_workspace_call_in_decreasing_sizes():
    # 3M parameters over 8 slices (733 blocks), then 64 slices of 200K, 3
    # slices of 100K accumulated onto a prior value, a norm-only call, one
    # partial vector, and an empty shard
    _case(8 * 3_000_011, 8, 5, seed=1)
    _case(64 * 200_003, 64, 63, seed=2)
    _case(3 * 100_003, 3, 2, seed=3, prior=0.25)
    _case(4 * 50_001, 4, 1, seed=4, store=False)
    _case(4 * 5, 4, 2, seed=5)
    assert _case(9, 4, 3, seed=6) == 0.0


def test_noalloc_at_its_largest_shard():
    """The largest shard the static array serves (2,146,959,360 parameters:
    room for the partials of 128-thread blocks, the smallest the clip pass
    runs, and their group sums; this bf16 call runs 256-thread blocks) gives the workspace call's
    squared norm bit for bit; one vector more is rejected before anything is
    enqueued."""
    vmax = 2_146_959_360
    s = Z.zs_layout(vmax, 1, 0, 8, 0)
    assert Z.zs_workspace_bytes(s) == Z.ZS_SCRATCH_BYTES
    g = torch.empty(vmax, dtype=torch.int16, device="cuda")
    zsgen.dev_bf16(g, 9, 4, 0, 1, 1e-3, 0)
    ws = torch.empty(Z.zs_workspace_bytes(s) // 8, dtype=torch.float64, device="cuda")
    sq_a = torch.zeros(1, dtype=torch.float64, device="cuda")
    sq_b = torch.zeros(1, dtype=torch.float64, device="cuda")
    Z.shard_grad_sqnorm(s, [g], None, ws, sq_a)
    Z.shard_grad_sqnorm_noalloc(s, [g], None, sq_b)
    torch.cuda.synchronize()
    assert _bits64(sq_a) == _bits64(sq_b)
    big = Z.zs_layout(vmax + 8, 1, 0, 8, 0)
    with pytest.raises(Z.ZSError) as e:
        # the raw address, so that the library's own size check answers (the
        # binding would refuse the tensor as too short for this shard first)
        Z.shard_grad_sqnorm_noalloc(big, [g.data_ptr()], None, sq_b)
    assert e.value.code == Z.ZS_ESCRATCH
    assert _bits64(sq_a) == _bits64(sq_b)
    # a smaller call right after, against the oracle
    _case(8 * 1_000_003, 8, 0, seed=7)
    log(f"noalloc at {vmax:,} parameters: Q={float(sq_b.item()):.6g}, equal bits")
