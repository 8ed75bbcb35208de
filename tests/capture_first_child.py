"""Child process of tests/test_gpu_graph.py::test_capture_first_after_zs_init
(not a test module).

A fresh process whose first calls into the library, after zs_init, are made
under HIP-graph capture: one clipped optimizer step (clip pass + step) is
captured and replayed three times, each replay checked bit for bit against an
eager step of a second copy of the same shard, run after it.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import fsdp_sharded_optimizer_zero_amd as Z  # noqa: E402
from fsdp_sharded_optimizer_zero_amd.runner import ShardRun  # noqa: E402
from zsgen.workloads import Workload  # noqa: E402


def snapshot(run):
    d = run.units_data[0]
    return [x.clone() for x in (d.w, d.m, d.v, d.out, run.sqnorm)]


def same(a, b):
    def bits(x):
        return x.view(torch.int32) if x.dtype == torch.float32 else \
            x.view(torch.int64) if x.dtype == torch.float64 else x
    return all(torch.equal(bits(x), bits(y)) for x, y in zip(a, b))


def main():
    torch.cuda.set_device(0)
    wl = Workload(name="capture_first", psi=5_200_003, n_d=8, rank=7, align=8, stage=2,
                  out_mode="gather", m_sigma=1e-4, v_sigma=1e-6, lr=3e-4, weight_decay=0.1,
                  max_grad_norm=0.05, t0=7, steps=1, seed=13)
    t = wl.t0
    runs = [ShardRun(wl) for _ in range(2)]
    for r in runs:
        r.fill_state(out_fill=0x7FC1)
        r.fill_grads(t)
    torch.cuda.synchronize()
    eager, graphed = runs
    Z.zs_init()
    print("zs_init done; capturing the first library calls", flush=True)
    start = snapshot(graphed)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.step(t)
    torch.cuda.synchronize()
    assert same(snapshot(graphed), start), "capture executed work"
    for k in range(3):
        eager.step(t)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert same(snapshot(eager), snapshot(graphed)), f"replay {k} differs from eager"
        print(f"replay {k} equals the eager step", flush=True)
    print("capture-first ok", flush=True)


if __name__ == "__main__":
    main()
