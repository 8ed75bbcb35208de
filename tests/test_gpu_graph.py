"""One optimizer step captured into a HIP graph (torch.cuda.CUDAGraph over
the library's calls) and replayed: every replay must equal the eager step bit
for bit.  The step enqueues only kernels (no memset, no allocation, no host
synchronisation), so it can be captured; the AdamW constants of step t are
kernel arguments and are frozen at capture, so the eager reference repeats
the same t.  Eager work and synchronisations run between the replays.  Both
builds are captured: the normal one (one launch per pass, plain step loads at
this size) and the small-grid test build (several launches per pass and the
step's streaming loads)."""
import os
import subprocess
import sys

import pytest
import torch

import fsdp_sharded_optimizer_zero_amd as Z
from fsdp_sharded_optimizer_zero_amd.runner import ShardRun
from zsgen.workloads import Workload

pytestmark = pytest.mark.gpu


def _snapshot(run):
    d = run.units_data[0]
    return [x.clone() for x in (d.w, d.m, d.v, d.out, run.sqnorm)]


def _same(a, b):
    return all(torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else
                           x.view(torch.int64) if x.dtype == torch.float64 else x,
                           y.view(torch.int32) if y.dtype == torch.float32 else
                           y.view(torch.int64) if y.dtype == torch.float64 else y)
               for x, y in zip(a, b))


@pytest.mark.parametrize("build", ["normal", "smallgrid"])
@pytest.mark.parametrize("micro", [1, 3])
def test_captured_step_replays_equal_eager(micro, build):
    path = Z.LIB_PATH if build == "normal" else Z.SMALLGRID_LIB_PATH
    with Z.library(path):
        _captured_step_replays_equal_eager(micro)


def _captured_step_replays_equal_eager(micro):
    # 1.3M parameters: 3 launches per pass in the small-grid build
    wl = Workload(name="graph", psi=5_200_003, n_d=4, rank=3, align=8, stage=2,
                  out_mode="gather", m_sigma=1e-4, v_sigma=1e-6, lr=3e-4, weight_decay=0.1,
                  max_grad_norm=0.05, t0=7, steps=1, seed=12, micro_batches=micro)
    t = wl.t0
    eager = ShardRun(wl)
    eager.fill_state(out_fill=0x7FC1)
    eager.fill_grads(t)
    graphed = ShardRun(wl)
    graphed.fill_state(out_fill=0x7FC1)
    graphed.fill_grads(t)
    torch.cuda.synchronize()
    assert _same(_snapshot(eager), _snapshot(graphed))

    # warm up on a side stream (first launches set the kernels' LDS limits),
    # then restore the state so both runs start equal
    start = _snapshot(graphed)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graphed.step(t)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    d = graphed.units_data[0]
    for dst, src in zip((d.w, d.m, d.v, d.out, graphed.sqnorm), start):
        dst.copy_(src)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.step(t)
    torch.cuda.synchronize()
    # capture executed nothing: the state is still the initial one
    assert _same(_snapshot(graphed), start)

    for k in range(4):
        eager.step(t)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum()     # unrelated eager work
        torch.cuda.synchronize()
        assert bool(torch.isfinite(junk))
        assert _same(_snapshot(eager), _snapshot(graphed)), f"replay {k} differs from eager"


def test_capture_first_after_zs_init():
    """A fresh process whose first library calls are captured, after zs_init
    (which makes the per-device set-up calls that must stay out of a
    capture): every replay equals the eager step."""
    child = os.path.join(os.path.dirname(os.path.abspath(__file__)), "capture_first_child.py")
    r = subprocess.run([sys.executable, "-u", child], capture_output=True, text=True,
                       timeout=300)
    print(r.stdout[-2000:], r.stderr[-2000:])
    assert r.returncode == 0, r.stderr[-2000:]
    assert "capture-first ok" in r.stdout
