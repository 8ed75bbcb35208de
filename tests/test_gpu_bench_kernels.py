"""The benchmark-only kernels (libzs_benchcopy.so: not part of the ABI, but
bench.py runs them next to the step).  The copy returns its source exactly
and writes nothing past its end, on ragged lengths, launched one-shot and
with fewer blocks than spans (each block then copies several); the step
pattern adds the gradient to w, m and v, stores the high half of the new w,
and writes nothing outside its parameters.  Run on an MI355X:
pytest -m gpu -s"""
import numpy as np
import pytest
import torch

import bench

pytestmark = pytest.mark.gpu
GUARD = 64


@pytest.mark.parametrize("n16,blocks", [(1000, 4), (1000, 2), (7 * 256 + 3, 1), (5, 1),
                                        (256, 1)])
def test_copy_is_exact_and_in_bounds(n16, blocks):
    lib = bench.bench_lib()
    g = torch.Generator().manual_seed(n16 + blocks)
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (4 * n16,), dtype=torch.int32, generator=g)
    src = src.cuda()
    dst = torch.full((4 * n16 + GUARD,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    assert lib.zs_bench_copy(src.data_ptr(), dst.data_ptr(), n16, blocks, st.cuda_stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst[:4 * n16], src)
    assert bool((dst[4 * n16:] == 0x5A5A5A5A).all())


@pytest.mark.parametrize("per_cu", [6, 0])
def test_step_pattern_adds_and_stays_in_bounds(per_cu):
    lib = bench.bench_lib()
    n = 3 * 512
    rng = np.random.default_rng(per_cu)
    host = {k: rng.normal(0, 1, n + GUARD).astype(np.float32) for k in ("g", "w", "m", "v")}
    dev = {k: torch.from_numpy(a.copy()).cuda() for k, a in host.items()}
    out = torch.full((n + GUARD,), 0x1234, dtype=torch.int16, device="cuda")
    st = torch.cuda.current_stream()
    assert lib.zs_bench_step_pattern(dev["g"].data_ptr(), dev["w"].data_ptr(),
                                     dev["m"].data_ptr(), dev["v"].data_ptr(), out.data_ptr(),
                                     n, per_cu, st.cuda_stream) == 0
    torch.cuda.synchronize()
    for k in ("w", "m", "v"):
        got = dev[k].cpu().numpy()
        want = host[k][:n] + host["g"][:n]
        assert np.array_equal(got[:n].view(np.uint32), want.view(np.uint32)), k
        assert np.array_equal(got[n:].view(np.uint32), host[k][n:].view(np.uint32)), k
    hi = ((host["w"][:n] + host["g"][:n]).view(np.uint32) >> 16).astype(np.uint16)
    got_out = out.cpu().numpy().view(np.uint16)
    assert np.array_equal(got_out[:n], hi)
    assert bool((got_out[n:] == 0x1234).all())
