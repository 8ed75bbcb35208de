"""Oracle-side helpers for the GPU parity tests.

Every expected value here is computed by the CPU oracle (``oracle``) from
inputs drawn by the HOST side of the seeded generator (``zsgen.host_*``);
no value produced on the GPU enters an expected value (compare_unit_full
reads the device's results only to compare them).  The GPU side fills its
own buffers with the device side of the same generator.
"""
from __future__ import annotations

import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle as O
import zsgen
from zsgen.workloads import (STREAM_EXP_AVG, STREAM_EXP_AVG_SQ, STREAM_MASTER, Workload,
                             grad_key, grad_stream)

FLT_MIN = np.float32(1.1754944e-38)
REL_BAR = 2e-6          # fp32 state: max relative error against the oracle
BF16_ULP_BAR = 1        # bf16 params: max distance in units in the last place


def log(msg):
    print(f"[parity {time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def hparams(wl: Workload, t: int) -> O.Hparams:
    return O.Hparams(lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2, eps=wl.eps,
                     weight_decay=wl.weight_decay, step=t, max_grad_norm=wl.max_grad_norm)


# ---- host inputs ----------------------------------------------------------------------

def host_state(wl: Workload, unit: int, start: int, n: int):
    w = zsgen.host_f32(wl.seed, STREAM_MASTER, unit, 0, wl.master_sigma, start, n)
    m = (np.zeros(n, np.float32) if wl.m_sigma is None else
         zsgen.host_f32(wl.seed, STREAM_EXP_AVG, unit, 0, wl.m_sigma, start, n))
    v = (np.zeros(n, np.float32) if wl.v_sigma is None else
         zsgen.host_f32(wl.seed, STREAM_EXP_AVG_SQ, unit, 0, wl.v_sigma, start, n,
                        absval=True))
    return w, m, v


def host_state_at(wl: Workload, unit: int, idx):
    w = zsgen.host_f32_at(wl.seed, STREAM_MASTER, unit, 0, wl.master_sigma, idx)
    m = (np.zeros(len(idx), np.float32) if wl.m_sigma is None else
         zsgen.host_f32_at(wl.seed, STREAM_EXP_AVG, unit, 0, wl.m_sigma, idx))
    v = (np.zeros(len(idx), np.float32) if wl.v_sigma is None else
         zsgen.host_f32_at(wl.seed, STREAM_EXP_AVG_SQ, unit, 0, wl.v_sigma, idx, absval=True))
    return w, m, v


def host_slices(wl: Workload, unit: int, t: int, start: int, n: int, j: int = 0):
    """Every rank's slice of micro-batch j of step t: bf16 bit patterns or fp32."""
    key = grad_key(t, j, wl.micro_batches)
    if wl.grad_dtype == "f32":
        return [zsgen.host_f32(wl.seed, grad_stream(unit), r, key, wl.grad_sigma, start, n)
                for r in range(wl.n_d)]
    return [zsgen.host_bf16(wl.seed, grad_stream(unit), r, key, wl.grad_sigma, start, n,
                            p_out=wl.outlier_p, sigma_out=wl.outlier_sigma)
            for r in range(wl.n_d)]


def host_slices_at(wl: Workload, unit: int, t: int, idx, j: int = 0):
    key = grad_key(t, j, wl.micro_batches)
    if wl.grad_dtype == "f32":
        return [zsgen.host_f32_at(wl.seed, grad_stream(unit), r, key, wl.grad_sigma, idx)
                for r in range(wl.n_d)]
    return [zsgen.host_bf16_at(wl.seed, grad_stream(unit), r, key, wl.grad_sigma, idx,
                               p_out=wl.outlier_p, sigma_out=wl.outlier_sigma)
            for r in range(wl.n_d)]


def oracle_reduce(wl: Workload, sl):
    """The oracle's reduction of one micro-batch's slices for this workload."""
    if wl.rank_tokens:
        return O.reduce_weighted(sl, O.token_weights(wl.rank_tokens))
    return O.reduce_mean_f32(sl) if wl.grad_dtype == "f32" else O.reduce_mean(sl)


def oracle_gradient(wl: Workload, slices_of_micro):
    """The step's gradient: the reduction of every micro-batch, accumulated."""
    m = wl.micro_batches
    if m == 1:
        return oracle_reduce(wl, slices_of_micro(0))
    acc = None
    for j in range(m):
        r = oracle_reduce(wl, slices_of_micro(j))
        if acc is None:
            acc = np.empty_like(r)
        O.accumulate(r, j, m, acc)
    return acc


# ---- oracle runs ----------------------------------------------------------------------

def oracle_full_run(wl: Workload, rank: int, steps: int, t0: int, shard, other_sqnorm=0.0):
    """Whole-shard oracle over `steps` steps of a bf16-mean workload.
    Returns (w, m, v, slot_out, qs, coefs)."""
    S, off, V = shard.shard_len, shard.shard_offset, shard.valid_len
    w, m, v = host_state(wl, 0, off, V)
    qs, coefs = [], []
    out = None
    for i in range(steps):
        t = t0 + i
        sl = host_slices(wl, 0, t, off, V)
        out, q, coef = O.shard_step(wl.n_d, S, V, hparams(wl, t), sl, w, m, v,
                                    other_sqnorm=other_sqnorm)
        qs.append(q)
        coefs.append(coef)
    return w, m, v, out, qs, coefs


def oracle_sqnorm_chunked(wl: Workload, unit: int, t: int, start: int, n: int,
                          chunk: int = 1 << 24, keep_idx=None, acc=None, keep_all=False):
    """Oracle squared norm of the mean over [start, start+n): the exact sum,
    accumulated chunk by chunk and rounded once.  The host generator fills
    chunk k+1 while the oracle reduces chunk k.  If keep_idx (sorted, relative
    to start) is given, also returns the oracle's mean at those positions;
    with keep_all, the oracle's whole gradient (fp32[n]) instead.
    Pass `acc` to keep accumulating into an existing exact accumulator (the
    global norm over several FSDP units)."""
    own = acc is None
    acc = O.SqAcc() if own else acc
    if keep_all:
        keep_idx = None
        whole = np.empty(n, np.float32)
    kept = np.empty(0 if keep_idx is None else len(keep_idx), np.float32)
    starts = list(range(0, n, chunk))

    def gen(a):
        return [host_slices(wl, unit, t, start + a, min(chunk, n - a), j)
                for j in range(wl.micro_batches)]

    with ThreadPoolExecutor(max_workers=1) as ex:
        fut = ex.submit(gen, starts[0]) if starts else None
        for ci, a in enumerate(starts):
            sls = fut.result()
            if ci + 1 < len(starts):
                fut = ex.submit(gen, starts[ci + 1])
            g = oracle_gradient(wl, lambda j: sls[j])
            acc.add(g)
            if keep_all:
                whole[a:a + len(g)] = g
            if keep_idx is not None:
                lo, hi = np.searchsorted(keep_idx, [a, a + len(g)])
                kept[lo:hi] = g[keep_idx[lo:hi] - a]
            if ci % 8 == 7:
                log(f"  oracle sqnorm {wl.name} unit {unit}: {a + len(g):,}/{n:,}")
    q = acc.value()
    if keep_all:
        return q, whole
    if keep_idx is not None:
        return q, kept
    return q


class _FullCompare:
    """Element-by-element comparison of one unit's step with the oracle,
    chunk by chunk: the oracle's AdamW (O4, with the oracle's clip
    coefficient, None for no clip) and bf16 pack (O5) from the oracle's
    gradient of the chunk and the host generator's initial state, against the
    device's w, m, v, output slot and stored gradient.  Asserts the fp32 and
    bf16 bars on every element and counts the elements that are not
    bit-identical."""

    def __init__(self, name, wl: Workload, run, unit: int, t: int, coef):
        self.name, self.wl, self.unit, self.coef = name, wl, unit, coef
        s = run.shard
        self.d = run.units_data[unit]
        self.V, self.off = s.valid_len, s.shard_offset
        self.base = self.off if wl.out_mode == "gather" else 0
        self.h = hparams(wl, t)
        self.nbit = {"w": 0, "m": 0, "v": 0, "out": 0, "gradient": 0}
        self.worst = {"w": 0.0, "m": 0.0, "v": 0.0}
        self.max_ulp = 0

    def chunk(self, a: int, gc: np.ndarray):
        name, d, n = self.name, self.d, len(gc)
        w, m, v = host_state(self.wl, self.unit, self.off + a, n)
        O.adamw_f32(self.h, gc, w, m, v, coef=self.coef)
        ob = O.bf16_rne(w)
        dev = {"w": d.w[a:a + n].cpu().numpy(), "m": d.m[a:a + n].cpu().numpy(),
               "v": d.v[a:a + n].cpu().numpy()}
        # bit-identical elements have no error: the bars are checked on the rest
        for k, ref in (("w", w), ("m", m), ("v", v)):
            diff = dev[k].view(np.uint32) != ref.view(np.uint32)
            nd = int(np.count_nonzero(diff))
            self.nbit[k] += nd
            if nd:
                e = float(rel_err(dev[k][diff], ref[diff]).max())
                self.worst[k] = max(self.worst[k], e)
                assert e <= REL_BAR, f"{name} {k}[{a}:{a + n}]: max rel err {e}"
        gout = d.out[self.base + a:self.base + a + n].cpu().numpy().view(np.uint16)
        diff = gout != ob
        nd = int(np.count_nonzero(diff))
        self.nbit["out"] += nd
        if nd:
            dist = int(bf16_ulp_dist(gout[diff], ob[diff]).max())
            self.max_ulp = max(self.max_ulp, dist)
            assert dist <= BF16_ULP_BAR, f"{name} out[{a}:{a + n}]: {dist} ulp"
        if d.mean is not None:
            gm = d.mean[a:a + n].cpu().numpy()
            self.nbit["gradient"] += int(np.count_nonzero(gm.view(np.uint32) !=
                                                          gc.view(np.uint32)))

    def finish(self) -> int:
        name, V = self.name, self.V
        for k in ("w", "m", "v"):
            log(f"  {name} {k}: max rel err {self.worst[k]:.3g}, "
                f"non-bitwise {self.nbit[k]:,}/{V:,}")
        log(f"  {name} out: max bf16 ulp {self.max_ulp}, non-bitwise {self.nbit['out']:,}/{V:,}")
        if self.d.mean is not None:
            log(f"  {name} stored gradient: non-bitwise {self.nbit['gradient']:,}/{V:,}")
            assert self.nbit["gradient"] == 0, f"{name}: stored gradient bits differ"
        return sum(self.nbit.values())


def compare_unit_full(name, wl: Workload, run, unit: int, t: int, g, coef,
                      chunk: int = 1 << 24):
    """Every element of one unit's step against the oracle (_FullCompare),
    from the oracle's whole gradient `g` (fp32[V], from
    oracle_sqnorm_chunked(keep_all=True)).  Returns the number of elements
    that are not bit-identical (all arrays)."""
    fc = _FullCompare(name, wl, run, unit, t, coef)
    for a in range(0, fc.V, chunk):
        fc.chunk(a, g[a:a + min(chunk, fc.V - a)])
    return fc.finish()


def compare_unit_streamed(name, wl: Workload, run, unit: int, t: int, coef,
                          chunk: int = 1 << 24):
    """compare_unit_full without the whole gradient in host memory: the
    oracle's gradient is drawn by the host generator and reduced chunk by
    chunk (the next chunk drawn while this one is reduced and compared), its
    exact squared norm accumulated, and each chunk's step compared at once.
    `coef` must come from the whole unit's squared norm known beforehand.
    Returns (the oracle's exactly rounded squared norm over the unit, the
    number of elements that are not bit-identical)."""
    fc = _FullCompare(name, wl, run, unit, t, coef)
    acc = O.SqAcc()
    start, n = fc.off, fc.V
    starts = list(range(0, n, chunk))

    def gen(a):
        return [host_slices(wl, unit, t, start + a, min(chunk, n - a), j)
                for j in range(wl.micro_batches)]

    with ThreadPoolExecutor(max_workers=1) as ex:
        fut = ex.submit(gen, starts[0]) if starts else None
        for ci, a in enumerate(starts):
            sls = fut.result()
            if ci + 1 < len(starts):
                fut = ex.submit(gen, starts[ci + 1])
            g = oracle_gradient(wl, lambda j: sls[j])
            del sls
            acc.add(g)
            fc.chunk(a, g)
            if ci % 8 == 7:
                log(f"  {name}: oracle step compared over {a + len(g):,}/{n:,}")
    return acc.value(), fc.finish()


def oracle_sampled_step(wl: Workload, unit: int, t: int, shard, idx, coef):
    """Oracle O1, O4, O5 at shard positions idx (relative to the shard), given
    the oracle's clip coefficient (None: no clip).  Returns (w, m, v, bf16)."""
    gidx = shard.shard_offset + np.asarray(idx, np.int64)
    g = oracle_gradient(wl, lambda j: host_slices_at(wl, unit, t, gidx, j))
    w, m, v = host_state_at(wl, unit, gidx)
    O.adamw_f32(hparams(wl, t), g, w, m, v, coef=coef)
    return w, m, v, O.bf16_rne(w), g


def sample_indices(V: int, n_random: int, seed: int, edge: int = 4096):
    """Both ends of the shard plus uniform random positions, sorted, unique."""
    if V == 0:
        return np.zeros(0, np.int64)
    rng = np.random.default_rng(seed)
    parts = [np.arange(min(edge, V)), np.arange(max(0, V - edge), V),
             rng.integers(0, V, size=n_random)]
    return np.unique(np.concatenate(parts).astype(np.int64))


# ---- comparisons ----------------------------------------------------------------------

def rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    both_nan = np.isnan(got) & np.isnan(ref)
    err = np.abs(got - ref) / np.maximum(np.abs(ref), float(FLT_MIN))
    err[both_nan] = 0.0
    err[np.isnan(err)] = np.inf
    same_inf = np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref))
    err[same_inf] = 0.0
    return err


def bf16_ulp_dist(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 steps between two bf16 bit-pattern arrays (sign-magnitude
    mapped to a monotone integer line)."""
    def line(x):
        x = x.astype(np.int64) & 0xFFFF
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(line(a) - line(b))


def assert_state_close(name, got, ref):
    e = rel_err(got, ref)
    nbit = int(np.count_nonzero(got.view(np.uint32) != ref.view(np.uint32)))
    log(f"  {name}: max rel err {e.max() if e.size else 0:.3g}, non-bitwise {nbit}/{got.size}")
    assert e.size == 0 or e.max() <= REL_BAR, f"{name}: max rel err {e.max()} > {REL_BAR}"
    return nbit


def assert_bf16_close(name, got, ref):
    got = got.astype(np.uint16)
    ref = ref.astype(np.uint16)
    d = bf16_ulp_dist(got, ref)
    nbit = int(np.count_nonzero(got != ref))
    log(f"  {name}: max bf16 ulp {d.max() if d.size else 0}, non-bitwise {nbit}/{got.size}")
    assert d.size == 0 or d.max() <= BF16_ULP_BAR
    return nbit


Q_REL_BAR = 1e-12       # GPU fp64 tree sum vs the oracle's exactly rounded sum


def coef_is_robust(Q: float, max_norm: float) -> bool:
    """True if every Q' within Q_REL_BAR of Q gives the same fp32 clip
    coefficient (so the GPU's differently rounded fp64 sum cannot change it)."""
    c = O.clip_coef(Q, max_norm)
    return (O.clip_coef(Q * (1 - Q_REL_BAR), max_norm) == c and
            O.clip_coef(Q * (1 + Q_REL_BAR), max_norm) == c)


def gpu_threads_note():
    return os.environ.get("OMP_NUM_THREADS", "")
