"""Helpers of the GPU parity tests of shard_grad_reduce (test code).

Every expected value comes from the CPU oracle on inputs drawn by numpy on the
host; the device rows hold +Inf beyond valid_len, which the kernels must not
read, and the output buffer a guard of NaN-pattern words after valid_len,
which they must not write.
"""
import numpy as np
import torch

import fsdp_sharded_optimizer_zero_amd as Z
import oracle as O
from parity_util import Q_REL_BAR

GUARD = 64
F32_SENTINEL = np.uint32(0x7FC00ABC)     # a NaN pattern the kernels never write


def rows_on_device(slices, n_d, S, V, f32):
    """Device [n_d, S] rows; beyond V they hold +Inf the kernels must not read."""
    if f32:
        rows = torch.full((n_d, S), float("inf"), dtype=torch.float32)
        for r in range(n_d):
            rows[r, :V] = torch.from_numpy(slices[r][:V])
    else:
        rows = torch.full((n_d, S), 0x7F80, dtype=torch.int16)
        for r in range(n_d):
            rows[r, :V] = torch.from_numpy(slices[r][:V].view(np.int16))
    return rows.cuda()


def oracle_reduce(slices, tokens, f32):
    if tokens is not None:
        return O.reduce_weighted(slices, O.token_weights(tokens))
    return O.reduce_mean_f32(slices) if f32 else O.reduce_mean(slices)


def draw_slices(rng, n_d, V, f32):
    if f32:
        return [rng.normal(0, 1e-3, V).astype(np.float32) for _ in range(n_d)]
    return [O.bf16_rne(rng.normal(0, 1e-3, V).astype(np.float32)) for _ in range(n_d)]


def run_reduce_case(psi, n_d, rank, f32, tokens, m, seed):
    rng = np.random.default_rng(seed)
    s = Z.zs_layout(psi, n_d, rank, 8, 2)
    S, V = s.shard_len, s.valid_len
    esize = 4 if f32 else 2
    out = torch.from_numpy(np.full(V + GUARD, F32_SENTINEL, np.uint32).view(np.float32)).cuda()
    ws = torch.empty(Z.zs_workspace_bytes(s) // 8, dtype=torch.float64, device="cuda")
    sq = torch.zeros(1, dtype=torch.float64, device="cuda")
    acc = np.empty(V, np.float32)
    for j in range(m):
        sl = draw_slices(rng, n_d, V, f32)
        rows = rows_on_device(sl, n_d, S, V, f32)
        ptrs = [rows.data_ptr() + esize * S * r for r in range(n_d)]
        last = j == m - 1
        r = Z.make_reduce(Z.ZS_GRAD_F32 if f32 else Z.ZS_GRAD_BF16, j, m, tokens)
        Z.shard_grad_reduce(s, r, ptrs, out, ws if last else None, sq if last else None)
        torch.cuda.synchronize()
        O.accumulate(oracle_reduce(sl, tokens, f32), j, m, acc)
        got = out.cpu().numpy().view(np.uint32)
        case = f"psi={psi} n_d={n_d} k={rank} f32={f32} tokens={tokens} j={j}/{m}"
        assert np.array_equal(got[:V], acc.view(np.uint32)), case
        assert np.all(got[V:] == F32_SENTINEL), f"{case}: wrote past valid_len"
        del rows
    q = O.sqnorm(acc)
    assert abs(float(sq.item()) - q) <= Q_REL_BAR * max(q, 1e-300), (psi, n_d, rank)
