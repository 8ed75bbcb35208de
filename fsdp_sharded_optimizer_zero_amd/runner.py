"""One GPU's share of a sharded optimizer step, driven through the C ABI.

``ShardRun`` holds, in HBM, everything one rank needs for a step of its shard
(per FSDP unit when there are several): the N_d ranks' gradient slices of
every micro-batch (the other ranks are simulated as extra buffers on this
GPU), the fp32 master/m/v shard, the fp32 reduced gradient (clip path, or
the micro-batch accumulator), the bf16 all-gather buffer (or the rank's own
bf16 shard) and the fp64 squared norm.  Inputs come from the seeded
generator, written directly into device memory.  ``step()`` issues exactly
the library calls of one optimizer step on one stream:

* no clip:   zero_shard_step(grad_slices=...)                 per unit
* clip:      shard_grad_sqnorm(...)                 (one unit), or
             shard_grad_sqnorm_units(...)           (all FSDP units at once)
             (squared norms summed in unit order: the global norm of the
             FSDP model; the other ranks' shards enter as other_sqnorm),
             then zero_shard_step(mean_in=..., sqnorm=...)    per unit
* fp32 slices, token weights or several micro-batches:
             shard_grad_reduce(micro=j, ...) for j = 0..m-1   per unit
             (the norm on the last micro-batch only), then
             zero_shard_step(mean_in=..., sqnorm=...)         per unit
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

import zsgen
from zsgen.workloads import (STREAM_EXP_AVG, STREAM_EXP_AVG_SQ, STREAM_MASTER, Workload,
                             grad_key, grad_stream)

from . import (ZS_GRAD_BF16, ZS_GRAD_F32, ZS_OUT_GATHER, ZS_OUT_SHARD, adamw, make_reduce,
               shard_grad_reduce, shard_grad_sqnorm, shard_grad_sqnorm_units, zero_shard_step,
               zs_layout, zs_workspace_bytes, zs_workspace_bytes_units)


def _empty(n, dtype, device):
    # never a zero-size allocation: keeps every pointer non-NULL and aligned
    return torch.empty(max(int(n), 8), dtype=dtype, device=device)


@dataclass
class Unit:
    slices: torch.Tensor       # [m, n_d, pitch] int16 (bf16) or float32: micro-batch
                               # j, row r = rank r's slice, V elements used
    w: torch.Tensor
    m: torch.Tensor
    v: torch.Tensor
    mean: torch.Tensor | None
    out: torch.Tensor          # int16 [n_d*S] (gather) or [S] (shard)


class ShardRun:
    def __init__(self, wl: Workload, rank: int | None = None, device: str = "cuda",
                 units: int | None = None, store_mean: bool | None = None):
        self.wl = wl
        self.rank = wl.rank if rank is None else rank
        self.units = wl.units if units is None else units
        self.device = device
        out_mode = ZS_OUT_GATHER if wl.out_mode == "gather" else ZS_OUT_SHARD
        self.shard = zs_layout(wl.psi, wl.n_d, self.rank, wl.align, wl.stage, out_mode)
        self.clip = wl.max_grad_norm > 0
        self.micro = wl.micro_batches
        # fp32 slices, token weights and micro-batches go through the general
        # reduction, which always stores the reduced (accumulated) gradient
        self.general = wl.grad_dtype != "bf16" or bool(wl.rank_tokens) or self.micro > 1
        # the clip needs the norm before any update: store the mean, read it back
        self.store_mean = (self.clip or self.general) if store_mean is None else store_mean
        if self.general and not self.store_mean:
            raise ValueError("the general reduction needs the stored-gradient schedule")
        self.f32_grads = wl.grad_dtype == "f32"
        self.gsize = 4 if self.f32_grads else 2
        S, V, nd = self.shard.shard_len, self.shard.valid_len, wl.n_d
        out_len = nd * S if out_mode == ZS_OUT_GATHER else S
        if wl.stage == 0 and out_mode == ZS_OUT_GATHER:
            out_len = S
        self.out_len = out_len
        # Rows of the simulated ranks' slices start on a 128-byte boundary
        # (256 for fp32), as separately allocated per-rank buffers would; the
        # shard length itself need not be a multiple of 64 (the 70B shard's
        # 1,093,750,000 is not), and rows S elements apart would then start
        # off a cache-line boundary.
        self.slice_pitch = -(-S // 64) * 64
        self.units_data = []
        for _ in range(self.units):
            self.units_data.append(Unit(
                slices=torch.empty((self.micro, nd, self.slice_pitch),
                                   dtype=torch.float32 if self.f32_grads else torch.int16,
                                   device=device),
                w=_empty(V, torch.float32, device), m=_empty(V, torch.float32, device),
                v=_empty(V, torch.float32, device),
                mean=_empty(V, torch.float32, device) if self.store_mean else None,
                out=torch.empty(out_len, dtype=torch.int16, device=device)))
        # FSDP units of one layout: one clip-pass call for all of them
        self.grouped_units = self.units > 1 and not self.general
        wsb = (zs_workspace_bytes_units(self.shard, self.units) if self.grouped_units
               else zs_workspace_bytes(self.shard))
        self.workspace = torch.empty(wsb // 8, dtype=torch.float64, device=device)
        self.sqnorm = torch.zeros(1, dtype=torch.float64, device=device)
        self.t = wl.t0
        self.reduce_specs = [make_reduce(ZS_GRAD_F32 if self.f32_grads else ZS_GRAD_BF16, j,
                                         self.micro, wl.rank_tokens or None)
                             for j in range(self.micro)]

    # ---- inputs ------------------------------------------------------------------

    @property
    def V(self):
        return self.shard.valid_len

    @property
    def has_reduce_pass(self):
        """A separate reduction pass runs before the update: for the clip (the
        norm must be known first) and whenever the reduced gradient is stored."""
        return self.clip or self.store_mean

    def fill_state(self, out_fill: int | None = None):
        wl, V, off = self.wl, self.V, self.shard.shard_offset
        for u, d in enumerate(self.units_data):
            if V > 0:
                zsgen.dev_f32(d.w[:V], wl.seed, STREAM_MASTER, u, 0, wl.master_sigma, off)
                if wl.m_sigma is None:
                    d.m.zero_()
                else:
                    zsgen.dev_f32(d.m[:V], wl.seed, STREAM_EXP_AVG, u, 0, wl.m_sigma, off)
                if wl.v_sigma is None:
                    d.v.zero_()
                else:
                    zsgen.dev_f32(d.v[:V], wl.seed, STREAM_EXP_AVG_SQ, u, 0, wl.v_sigma, off,
                                  absval=True)
            if out_fill is not None:
                d.out.fill_(out_fill)

    def fill_grads(self, t: int):
        """Draw every micro-batch's slices of optimizer step t."""
        wl, V, off = self.wl, self.V, self.shard.shard_offset
        if V == 0:
            return
        for u, d in enumerate(self.units_data):
            for j in range(self.micro):
                key = grad_key(t, j, self.micro)
                for r in range(wl.n_d):
                    if self.f32_grads:
                        zsgen.dev_f32(d.slices[j, r, :V], wl.seed, grad_stream(u), r, key,
                                      wl.grad_sigma, off)
                    else:
                        zsgen.dev_bf16(d.slices[j, r, :V], wl.seed, grad_stream(u), r, key,
                                       wl.grad_sigma, off, p_out=wl.outlier_p,
                                       sigma_out=wl.outlier_sigma)

    # ---- the step -------------------------------------------------------------------

    def hparams(self, t: int):
        wl = self.wl
        return adamw(lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2, eps=wl.eps,
                     weight_decay=wl.weight_decay, step=t, max_grad_norm=wl.max_grad_norm)

    def slice_ptrs(self, d: Unit, j: int = 0):
        base = d.slices[j].data_ptr()
        return [base + self.gsize * self.slice_pitch * r for r in range(self.wl.n_d)]

    def reduce_pass(self, stream=None):
        if self.grouped_units:
            ptrs = [p for d in self.units_data for p in self.slice_ptrs(d)]
            means = [d.mean for d in self.units_data] if self.store_mean else None
            shard_grad_sqnorm_units(self.shard, ptrs, means, self.workspace, self.sqnorm,
                                    stream=stream)
            return
        for u, d in enumerate(self.units_data):
            if not self.general:
                shard_grad_sqnorm(self.shard, self.slice_ptrs(d), d.mean, self.workspace,
                                  self.sqnorm, accumulate=u > 0, stream=stream)
                continue
            for j in range(self.micro):
                norm = self.clip and j == self.micro - 1
                shard_grad_reduce(self.shard, self.reduce_specs[j], self.slice_ptrs(d, j),
                                  d.mean, self.workspace if norm else None,
                                  self.sqnorm if norm else None, accumulate=u > 0,
                                  stream=stream)

    def update_pass(self, t: int, other_sqnorm: float = 0.0, stream=None):
        h = self.hparams(t)
        for d in self.units_data:
            if self.store_mean:
                zero_shard_step(self.shard, h, mean_in=d.mean,
                                sqnorm=self.sqnorm if self.clip else None,
                                other_sqnorm=other_sqnorm, master=d.w, exp_avg=d.m,
                                exp_avg_sq=d.v, param_out=d.out, stream=stream)
            else:
                zero_shard_step(self.shard, h, grad_slices=self.slice_ptrs(d),
                                sqnorm=self.sqnorm if self.clip else None,
                                other_sqnorm=other_sqnorm, master=d.w, exp_avg=d.m,
                                exp_avg_sq=d.v, param_out=d.out, stream=stream)

    def step(self, t: int | None = None, other_sqnorm: float = 0.0, stream=None):
        """Enqueue one optimizer step of every unit at bias-correction step t."""
        t = self.t if t is None else t
        if self.has_reduce_pass:
            self.reduce_pass(stream)
        self.update_pass(t, other_sqnorm, stream)
        self.t = t + 1

    # ---- bytes the step must move (algorithmic, per step) -------------------------------

    def algorithmic_bytes(self):
        """(reduce-pass bytes, update-pass bytes) over all units.

        reduce pass: N_d bf16 reads + fp32 mean write = 2 N_d + 4 B/param
        (fp32 slices: 4 N_d; micro-batch j > 0 also reads the accumulator)
        update pass: mean read (or N_d bf16 reads) + 12 B state read + 12 B
        state write + 2 B bf16 write; pads are written too (2 B each)."""
        nd, V, S = self.wl.n_d, self.V, self.shard.shard_len
        pads = S - V
        if self.general:
            # micro-batch j reads its slices, reads the accumulator (j > 0)
            # and writes it
            red = sum((self.gsize * nd + (4 if j > 0 else 0) + 4) * V for j in range(self.micro))
            upd = (4 + 12 + 12 + 2) * V + 2 * pads
        elif self.clip and self.store_mean:
            red = (2 * nd + 4) * V
            upd = (4 + 12 + 12 + 2) * V + 2 * pads
        elif self.clip:
            red = 2 * nd * V
            upd = (2 * nd + 26) * V + 2 * pads
        else:
            red = 0
            upd = (2 * nd + 26) * V + 2 * pads
        return red * self.units, upd * self.units
