"""The synthetic workloads of the sharded optimizer step.

Each workload is one GPU's share of a data-parallel sharded AdamW step, at the
shape the pages discuss (a ZeRO-1/2 shard of a flat parameter vector, FSDP
units of a Llama-style block, a ZeRO-3 shard of a 70B model).  This file only
states sizes, hyperparameters and input distributions; it computes nothing.

Input recipe (all seeded, all synthetic): a workload's seed is its index;
master weights, moments and every rank's gradients are drawn from separate
streams of the counter-based generator at the element's index in the flat
parameter vector (so shards of one model are consistent with each other);
gradients are redrawn for every step t from (rank, t); state is drawn once.
``sigma`` is a standard deviation.  An outlier replaces the base draw of one
(rank, element) with probability ``outlier_p`` by a draw of N(0, outlier_sigma).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

# Stream ids (must match zsg_def.h).
STREAM_MASTER = 1
STREAM_EXP_AVG = 2
STREAM_EXP_AVG_SQ = 3
STREAM_GRAD = 4


def grad_stream(unit: int = 0) -> int:
    """Gradient stream of FSDP unit `unit` (rank and step go in the key)."""
    assert 0 <= unit < 1024
    return STREAM_GRAD + 16 * unit


def state_stream(which: int) -> int:
    return which


@dataclass(frozen=True)
class Workload:
    name: str
    psi: int                 # parameters of the model (or of one FSDP unit)
    n_d: int                 # data-parallel ranks
    rank: int                # the rank whose shard this GPU holds
    align: int               # shard length is a multiple of this
    stage: int               # 0 DDP, 1, 2, 3 (ZeRO stage)
    out_mode: str            # "gather": bf16[n_d*S] at k*S; "shard": bf16[S]
    units: int = 1           # FSDP units updated back to back
    master_sigma: float = 0.02
    m_sigma: Optional[float] = None      # None: zeros
    v_sigma: Optional[float] = None      # None: zeros; else |N(0, v_sigma)|
    grad_sigma: float = 1e-3
    outlier_p: float = 0.0
    outlier_sigma: float = 0.0
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    max_grad_norm: float = 0.0           # <= 0: no clip
    t0: int = 1                          # bias-correction step of the first step
    steps: int = 1
    seed: int = 0
    extra_ranks: tuple = field(default_factory=tuple)   # other ranks also tested
    grad_dtype: str = "bf16"             # "bf16" or "f32" gradient slices
    rank_tokens: tuple = ()              # () : plain mean; else valid tokens per rank
    micro_batches: int = 1               # m: micro-batches per optimizer step


def grad_key(t: int, j: int, m: int) -> int:
    """Generator step key of micro-batch j of optimizer step t (t for m = 1)."""
    return t * m + j


def _splitmix64(x: int) -> int:
    """SplitMix64 output function (Steele, Lea and Flood 2014)."""
    x = (x + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
    z = x
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
    return z ^ (z >> 31)


def token_counts(seed: int, n_d: int, seqs: int = 4, max_len: int = 4096,
                 empty_rank: int = -1) -> tuple:
    """Valid tokens per rank for a token-weighted workload: each rank holds
    `seqs` sequences whose valid lengths are uniform in [0, max_len] (the
    rest is padding); `empty_rank` holds only padding (zero tokens)."""
    out = []
    for r in range(n_d):
        n = 0
        for q in range(seqs):
            n += _splitmix64((seed << 32) ^ (r << 16) ^ q) % (max_len + 1)
        out.append(0 if r == empty_rank else n)
    return tuple(out)


WORKLOADS = {
    # Tiny flat vector, 4 ranks, no clip, 10 steps from zero moments.
    "tiny": Workload(name="tiny", psi=1_048_576, n_d=4, rank=1, align=128, stage=2,
                     out_mode="gather", lr=1e-3, weight_decay=0.01, max_grad_norm=0.0,
                     t0=1, steps=10, seed=0),
    # GPT-2-small-sized flat vector, rank 3 (and the last rank, which has a
    # padded tail), 1% gradient outliers, global clip 1.0, 5 steps.
    "gpt2_small": Workload(name="gpt2_small", psi=124_439_808, n_d=8, rank=3, align=1024,
                           stage=2, out_mode="gather", outlier_p=0.01, outlier_sigma=0.1,
                           lr=1e-3, weight_decay=0.01, max_grad_norm=1.0, t0=1, steps=5,
                           seed=1, extra_ranks=(7,)),
    # One GPU's ZeRO-2 shard of a 7B model over 8 ranks.
    "zero2_7b": Workload(name="zero2_7b", psi=7_000_000_000, n_d=8, rank=3, align=1,
                         stage=2, out_mode="gather", m_sigma=1e-4, v_sigma=1e-6,
                         lr=3e-4, weight_decay=0.1, max_grad_norm=1.0, t0=1000, steps=1,
                         seed=2),
    # FSDP / ZeRO-3, 32 Llama-style blocks (hidden 4096, FFN 14336, 32 heads,
    # 8 KV heads: 218,112,000 parameters each), rank 7 of 8 with tail padding,
    # each new bf16 shard packed into its unit's full gather buffer.
    "fsdp_llama_units": Workload(name="fsdp_llama_units", psi=218_112_000, n_d=8, rank=7,
                                 align=2048, stage=3, out_mode="gather", units=32,
                                 m_sigma=1e-4, v_sigma=1e-6, lr=3e-4, weight_decay=0.1,
                                 max_grad_norm=1.0, t0=1000, steps=1, seed=3),
    # One GPU's ZeRO-3 shard of a 70B model over 64 ranks (64 gradient slices).
    "zero3_70b": Workload(name="zero3_70b", psi=70_000_000_000, n_d=64, rank=0, align=1,
                          stage=3, out_mode="shard", m_sigma=1e-4, v_sigma=1e-6,
                          grad_sigma=5e-4, lr=1.5e-4, beta1=0.9, beta2=0.95,
                          weight_decay=0.1, max_grad_norm=1.0, t0=10, steps=1, seed=4),
    # The 7B ZeRO-2 shard with the three reductions beyond the bf16 mean:
    # fp32 gradient slices (reduce_dtype=float32); token-weighted ranks, one
    # of which holds only padding; ZeRO-2 gradient accumulation over 4
    # micro-batches (each micro-batch's slices reduced, then accumulated).
    "zero2_7b_f32grad": Workload(name="zero2_7b_f32grad", psi=7_000_000_000, n_d=8, rank=3,
                                 align=1, stage=2, out_mode="gather", m_sigma=1e-4,
                                 v_sigma=1e-6, lr=3e-4, weight_decay=0.1, max_grad_norm=1.0,
                                 t0=1000, steps=1, seed=5, grad_dtype="f32"),
    "zero2_7b_tokens": Workload(name="zero2_7b_tokens", psi=7_000_000_000, n_d=8, rank=3,
                                align=1, stage=2, out_mode="gather", m_sigma=1e-4,
                                v_sigma=1e-6, lr=3e-4, weight_decay=0.1, max_grad_norm=1.0,
                                t0=1000, steps=1, seed=6,
                                rank_tokens=token_counts(6, 8, empty_rank=5)),
    "zero2_7b_accum4": Workload(name="zero2_7b_accum4", psi=7_000_000_000, n_d=8, rank=3,
                                align=1, stage=2, out_mode="gather", m_sigma=1e-4,
                                v_sigma=1e-6, lr=3e-4, weight_decay=0.1, max_grad_norm=1.0,
                                t0=1000, steps=1, seed=7, micro_batches=4),
}

ORDER = ["tiny", "gpt2_small", "zero2_7b", "fsdp_llama_units", "zero3_70b"]
NEXT = ["zero2_7b_f32grad", "zero2_7b_tokens", "zero2_7b_accum4"]


def llama_block_params(hidden=4096, ffn=14336, heads=32, kv_heads=8) -> int:
    """Parameters of one Llama-style block: q, o (h x h), k, v (h x h*kv/heads),
    gate/up/down (3 x h x ffn), two RMSNorm weight vectors."""
    head_dim = hidden // heads
    kv = kv_heads * head_dim
    return 2 * hidden * hidden + 2 * hidden * kv + 3 * hidden * ffn + 2 * hidden
