"""The library from several host threads at once, each on its own stream.

The entry points keep no per-call state (the per-device LDS size and kernel
attribute are set once, thread-safely), so concurrent calls on separate
buffers and streams must give each thread exactly the bits a serial run gives.
ctypes releases the GIL during the calls, so the host code of the library runs
concurrently.  Run on an MI355X:  pytest -m gpu -s
"""
import threading

import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_zero_amd as Z
import oracle as O

pytestmark = pytest.mark.gpu

THREADS = 4
STEPS = 5


def _case(k):
    """Thread k's shard: distinct N_d (8 or 64) and rank, so both the
    two-blocks-per-CU and the one-block-per-CU clip passes run."""
    n_d = 64 if k % 2 else 8
    s = Z.zs_layout(n_d * 300_000 - 11 * k - 1, n_d, n_d - 1 - k, 8, 2)
    rng = np.random.default_rng(500 + k)
    S, V = s.shard_len, s.valid_len
    rows = np.full((n_d, S), 0x7F80, np.uint16)
    for r in range(n_d):
        rows[r, :V] = O.bf16_rne(rng.normal(0, 1e-3, V).astype(np.float32))
    w = rng.normal(0, 0.02, V).astype(np.float32)
    return s, rows, w


def _run(s, rows, w0, stream):
    n_d, S, V = s.n_d, s.shard_len, s.valid_len
    with torch.cuda.stream(stream):
        dev_rows = torch.from_numpy(rows.view(np.int16)).to("cuda", non_blocking=False)
        ptrs = [dev_rows.data_ptr() + 2 * S * r for r in range(n_d)]
        w = torch.from_numpy(w0).cuda()
        m = torch.zeros(V, device="cuda")
        v = torch.zeros(V, device="cuda")
        mean = torch.empty(V, device="cuda")
        out = torch.zeros(n_d * S, dtype=torch.int16, device="cuda")
        ws = torch.empty(Z.zs_workspace_bytes(s) // 8, dtype=torch.float64, device="cuda")
        sq = torch.zeros(1, dtype=torch.float64, device="cuda")
    for t in range(1, STEPS + 1):
        h = Z.adamw(lr=1e-3, weight_decay=0.01, step=t, max_grad_norm=0.05)
        Z.shard_grad_sqnorm(s, ptrs, mean, ws, sq, stream=stream)
        Z.zero_shard_step(s, h, mean_in=mean, sqnorm=sq, master=w, exp_avg=m, exp_avg_sq=v,
                          param_out=out, stream=stream)
    stream.synchronize()
    return [x.cpu().numpy().copy() for x in (w, m, v, out)] + [float(sq.item())]


def test_concurrent_threads_match_serial():
    cases = [_case(k) for k in range(THREADS)]
    serial = [_run(*c, torch.cuda.Stream()) for c in cases]
    results = [None] * THREADS
    errors = []
    barrier = threading.Barrier(THREADS)

    def worker(k):
        try:
            stream = torch.cuda.Stream()
            barrier.wait()
            results[k] = _run(*cases[k], stream)
        except Exception as e:       # reported below, in the main thread
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not errors, errors
    for k in range(THREADS):
        for name, a, b in zip(("w", "m", "v", "out"), results[k][:4], serial[k][:4]):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (k, name)
        assert results[k][4] == serial[k][4], k
