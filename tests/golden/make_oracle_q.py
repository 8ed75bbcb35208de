#!/usr/bin/env python3
"""Write the oracle's squared gradient norm of a whole shard to
``tests/golden/oracle_q_<workload>.json``.

Only for shards too large for the oracle to finish inside a test: the 70B
ZeRO-3 shard over 64 ranks (1,093,750,000 parameters, 7e10 bf16 gradient
values) takes about half an hour on 8 host cores.  The value is the global
clip's Q of that shard ("Data parallelism, ZeRO and FSDP", section 7 "Common
mistakes": the norm of sharded gradients is taken over the squared shard
norms; the other shards enter the step as other_sqnorm, 0 here).

Calls only the CPU oracle (``oracle``) on inputs drawn by the host side of the
seeded generator (``zsgen``); nothing here touches a GPU or the HIP library.
The file records the workload's fields and the SHA-256 of the oracle and
generator sources, so that the test that reads it can tell a stale value.

    python3 tests/golden/make_oracle_q.py zero3_70b
"""
from __future__ import annotations

import dataclasses
import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(HERE))

# Sources whose arithmetic fixes the value: the oracle and the generator.
SOURCES = ["oracle/zs_oracle.c", "zsgen/zsg_def.h", "zsgen/zsg_host.c"]


def source_shas() -> dict:
    out = {}
    for rel in SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            out[rel] = hashlib.sha256(f.read()).hexdigest()
    return out


def golden_path(name: str) -> str:
    return os.path.join(HERE, f"oracle_q_{name}.json")


def workload_fields(wl) -> dict:
    return {k: (list(v) if isinstance(v, tuple) else v)
            for k, v in dataclasses.asdict(wl).items()}


def make(name: str) -> dict:
    import oracle as O
    from parity_util import log, oracle_sqnorm_chunked
    from zsgen.workloads import WORKLOADS, grad_key

    wl = WORKLOADS[name]
    if wl.units != 1:
        raise SystemExit(f"{name}: one unit only")
    S, off, V = O.layout(wl.psi, wl.n_d, wl.rank, wl.align, wl.stage)
    t0 = time.time()
    log(f"{name}: oracle squared norm over {V:,} parameters x {wl.n_d} ranks")
    q = oracle_sqnorm_chunked(wl, 0, wl.t0, off, V)
    secs = time.time() - t0
    rec = {
        "what": ("exactly rounded sum over the shard of g_i^2, g the oracle's rank-order "
                 "fp32 mean of the ranks' gradient slices (bias-correction step t0's draw)"),
        "source": ("\"Data parallelism, ZeRO and FSDP\", section 7 \"Common mistakes\" "
                   "(global norm from the squared shard norms)"),
        "script": "tests/golden/make_oracle_q.py",
        "workload": name,
        "workload_fields": workload_fields(wl),
        "layout": {"shard_len": S, "shard_offset": off, "valid_len": V},
        "grad_key": grad_key(wl.t0, 0, wl.micro_batches),
        "q": q,
        "q_hex": float.hex(q),
        "clip_coef": float(O.clip_coef(q, wl.max_grad_norm)) if wl.max_grad_norm > 0 else None,
        "sources_sha256": source_shas(),
        "oracle_seconds": round(secs, 1),
    }
    with open(golden_path(name) + ".tmp", "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    os.replace(golden_path(name) + ".tmp", golden_path(name))
    log(f"{name}: Q = {q!r} ({float.hex(q)}) in {secs:.0f} s -> {golden_path(name)}")
    return rec


if __name__ == "__main__":
    for n in sys.argv[1:] or ["zero3_70b"]:
        make(n)
