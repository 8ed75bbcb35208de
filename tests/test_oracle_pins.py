"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each test checks an oracle function against what the pages print (fixtures in
tests/golden/, each with its citation), a closed form, a special case that
reduces to a library routine (torch.optim.AdamW, clip_grad_norm_, torch's
float->bfloat16 cast, math.fsum), or brute force on tiny inputs.  The cases
are chosen so that a dropped term, a wrong sign or index, or a swapped
operand in any oracle function fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def bf16_of_exact(vals):
    """bf16 bit patterns of values that bf16 represents exactly (checked)."""
    f = np.asarray(vals, dtype=np.float32)
    h = (f.view(np.uint32) >> 16).astype(np.uint16)
    back = (h.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(back, f), "value not exact in bf16"
    return h


# ---------------------------------------------------------------- worked example

def test_worked_example_two_gpus():
    """Two GPUs, one batch: per-GPU means -1.5 and -13 average to -7.25, the
    full-batch gradient; the same with four ranks of one sample each."""
    g = golden("worked_example_two_gpus.json")
    x, y, w = (np.array(g[k], dtype=np.float64) for k in ("x", "y", "w"))
    resid = w * x - y
    grads = resid * x
    assert resid.tolist() == g["residual_per_sample"]
    assert grads.tolist() == g["grad_per_sample"]
    means = [grads[idx].mean() for idx in g["gpu_halves"]]
    assert means == g["gpu_means"]
    assert grads.mean() == g["one_gpu_full_batch_mean"]

    two = O.reduce_mean([bf16_of_exact([m]) for m in g["gpu_means"]])
    four = O.reduce_mean([bf16_of_exact([v]) for v in g["grad_per_sample"]])
    assert two[0] == np.float32(g["allreduce_mean"])
    assert four[0] == np.float32(g["allreduce_mean"])

    # The whole shard step of N_d = 2 and 4 ranks equals a one-rank step fed
    # the full-batch mean, bit for bit (Proposition "DDP is exact").
    h = O.Hparams(lr=1e-2, weight_decay=0.1, step=3, max_grad_norm=0.0)
    outs = []
    for slices in ([bf16_of_exact([m]) for m in g["gpu_means"]],
                   [bf16_of_exact([v]) for v in g["grad_per_sample"]],
                   [bf16_of_exact([g["allreduce_mean"]])]):
        w_ = np.array([1.0], np.float32)
        m_ = np.array([0.25], np.float32)
        v_ = np.array([3.0], np.float32)
        out, _, _ = O.shard_step(len(slices), 8, 1, h, slices, w_, m_, v_)
        outs.append((w_.view(np.uint32)[0], m_.view(np.uint32)[0],
                     v_.view(np.uint32)[0], out.tobytes()))
    assert outs[0] == outs[2] and outs[1] == outs[2]


# --------------------------------------------------------------------- reduction

def test_reduce_single_rank_is_identity():
    rng = np.random.default_rng(1)
    h = rng.integers(0, 1 << 16, size=4096, dtype=np.uint16)
    h = h[((h & 0x7F80) != 0x7F80)]          # drop NaN/Inf patterns
    out = O.reduce_mean([h])
    assert np.array_equal(out.view(np.uint32), O.bf16_to_f32(h).view(np.uint32))


def test_reduce_is_the_mean_not_the_sum_with_error_bound():
    rng = np.random.default_rng(2)
    for n_d in (2, 3, 5, 8, 64):
        sl = [O.bf16_rne(rng.normal(0, 1e-3, 1000).astype(np.float32))
              for _ in range(n_d)]
        got = O.reduce_mean(sl).astype(np.float64)
        vals = np.stack([O.bf16_to_f32(s).astype(np.float64) for s in sl])
        exact = vals.sum(0) / n_d       # exact: bf16 values, few binades
        bound = (n_d * np.abs(vals).sum(0) / n_d + np.abs(exact)) * 2.0 ** -23
        assert np.all(np.abs(got - exact) <= bound)


def test_reduce_power_of_two_ranks_exact_on_dyadics():
    rng = np.random.default_rng(3)
    for n_d in (1, 2, 4, 8, 16, 32, 64):
        ints = rng.integers(-200, 200, size=(n_d, 257))
        sl = [bf16_of_exact(r * 2.0 ** -10) for r in ints]
        got = O.reduce_mean(sl)
        for i in range(257):
            exact = Fraction(int(ints[:, i].sum()), 1024 * n_d)
            assert Fraction(float(got[i])) == exact


def test_reduce_rank_order():
    """Rank-order summation from rank 0: (2^24 + 1) + 1 rounds to 2^24 twice,
    whereas the reverse order would give 2^24 + 2 exactly."""
    sl = [bf16_of_exact([2.0 ** 24]), bf16_of_exact([1.0]), bf16_of_exact([1.0])]
    got = O.reduce_mean(sl)[0]
    assert got == np.float32(2.0 ** 24) / np.float32(3.0)
    assert got != np.float32(2.0 ** 24 + 2) / np.float32(3.0)


# ---------------------------------------------------------------- norm and clip

def _exact_sq_sum(vals):
    """Exact rational sum of squares of float32 values."""
    return sum((Fraction(float(x)) ** 2 for x in vals), Fraction(0))


def test_sqnorm_constant_closed_form():
    # c near 2: its squared significand is near 2^48, so more than 2^16 equal
    # terms carry out of the low 64 bits of the accumulator
    for c in (np.float32(3 * 2.0 ** -10), np.float32(1.9999999), np.float32(-1.5e-20)):
        for n in (0, 1, 7, 100_003):
            g = np.full(n, c, np.float32)
            assert O.sqnorm(g) == float(n * Fraction(float(c)) ** 2)


def test_sqnorm_is_the_exactly_rounded_sum():
    rng = np.random.default_rng(4)
    g = rng.normal(0, 1e-3, 200_001).astype(np.float32)
    g[::997] *= 1e3                         # outliers, as in the gradient workloads
    q = O.sqnorm(g)
    assert q == math.fsum(float(x) * float(x) for x in g)   # fsum: correctly rounded
    # chunks added in any order give the same exactly rounded total
    acc = O.SqAcc()
    for a in range(0, g.size, 65_536)[::-1]:
        acc.add(g[a:a + 65_536])
    assert acc.value() == q
    assert O.sqnorm(g[:0]) == 0.0


def test_sqnorm_wide_range_and_subnormals():
    vals = np.array([3.0e38, 1e-30, -2.0 ** -149, 2.0 ** -126, 1.0, -7.25, 2.0 ** -140,
                     1e19, 5e-45], np.float32)
    assert O.sqnorm(vals) == float(_exact_sq_sum(vals))
    sub = np.array([2.0 ** -149] * 3, np.float32)      # squares far below fp32 range
    assert O.sqnorm(sub) == 3 * 2.0 ** -298
    rng = np.random.default_rng(44)
    bits = rng.integers(0, 0x7F800000, size=2000, dtype=np.int64).astype(np.uint32)
    x = bits.view(np.float32)
    assert O.sqnorm(x) == float(_exact_sq_sum(x))


def test_sqnorm_ties_round_to_even():
    # 2^53 + 1 (in units of 2^-298... here units of 1): exactly between two doubles
    one = np.float32(1.0)
    big = np.full(1, np.float32(2.0 ** 26), np.float32)  # square 2^52
    g = np.concatenate([big, big, np.array([one], np.float32)])   # 2^53 + 1
    assert O.sqnorm(g) == 2.0 ** 53                                # tie -> even
    g3 = np.concatenate([g, np.array([one, one], np.float32)])     # 2^53 + 3
    assert O.sqnorm(g3) == 2.0 ** 53 + 4                           # tie -> even


def test_sqnorm_non_finite():
    assert np.isnan(O.sqnorm(np.array([1.0, np.nan, np.inf], np.float32)))
    assert O.sqnorm(np.array([1.0, -np.inf], np.float32)) == np.inf


@pytest.mark.parametrize("scale,max_norm", [(1e-3, 1.0), (1.0, 1.0), (3.0, 0.5),
                                            (1e-2, 100.0), (10.0, 2.0)])
def test_clip_against_clip_grad_norm(scale, max_norm):
    rng = np.random.default_rng(5)
    parts = [rng.normal(0, scale, n).astype(np.float32) for n in (1000, 37, 5000)]
    tens = [torch.nn.Parameter(torch.zeros(p.size, dtype=torch.float64))
            for p in parts]
    for t, p in zip(tens, parts):
        t.grad = torch.from_numpy(p.astype(np.float64))
    torch.nn.utils.clip_grad_norm_(tens, max_norm)
    torch_coef = tens[0].grad[0].item() / float(parts[0][0])
    Q = O.SqAcc()
    for p in parts:
        Q.add(p)
    coef = O.clip_coef(Q.value(), max_norm)
    if torch_coef >= 1.0 - 1e-15:
        assert coef == np.float32(1.0)
    else:
        assert abs(float(coef) - torch_coef) <= 2 * abs(torch_coef) * 2.0 ** -24


def test_clip_special_values():
    assert O.clip_coef(0.0, 1.0) == np.float32(1.0)
    assert O.clip_coef(float("inf"), 1.0) == np.float32(0.0)
    assert np.isnan(O.clip_coef(float("nan"), 1.0))
    # norm exactly at max_norm stays below 1 only through the 1e-6 guard
    assert O.clip_coef(4.0, 2.0) == np.float32(2.0 / (2.0 + 1e-6))
    # torch agrees that a NaN norm poisons every gradient
    p = torch.nn.Parameter(torch.zeros(2, dtype=torch.float64))
    p.grad = torch.tensor([float("nan"), 1.0], dtype=torch.float64)
    torch.nn.utils.clip_grad_norm_([p], 1.0)
    assert torch.isnan(p.grad).all()


# ------------------------------------------------------------------------ AdamW

HPARAM_SETS = [
    dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01),
    dict(lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1),
    dict(lr=1.5e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1),
    dict(lr=1e-2, beta1=0.5, beta2=0.9, eps=1e-2, weight_decay=0.5),
    dict(lr=0.1, beta1=0.0, beta2=0.0, eps=1e-3, weight_decay=0.0),
]


def _torch_adamw_steps(hp, w0, m0, v0, grads, t0):
    """Run torch.optim.AdamW in float64 from state (w0, m0, v0) at step t0-1."""
    p = torch.nn.Parameter(torch.from_numpy(w0.astype(np.float64)))
    opt = torch.optim.AdamW([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]),
                            eps=hp["eps"], weight_decay=hp["weight_decay"],
                            foreach=False)
    p.grad = torch.zeros_like(p)
    opt.step()                                   # creates the state
    st = opt.state[p]
    with torch.no_grad():
        p.copy_(torch.from_numpy(w0.astype(np.float64)))
    st["exp_avg"].copy_(torch.from_numpy(m0.astype(np.float64)))
    st["exp_avg_sq"].copy_(torch.from_numpy(v0.astype(np.float64)))
    st["step"].fill_(t0 - 1)
    for g in grads:
        p.grad = torch.from_numpy(g.astype(np.float64))
        opt.step()
    return (p.detach().numpy().copy(), st["exp_avg"].numpy().copy(),
            st["exp_avg_sq"].numpy().copy())


def _state(rng, n):
    w = rng.normal(0, 0.02, n)
    m = rng.normal(0, 1e-4, n)
    v = np.abs(rng.normal(0, 1e-6, n))
    return w, m, v


@pytest.mark.parametrize("hp", HPARAM_SETS)
@pytest.mark.parametrize("t0", [1, 7, 1000])
def test_adamw_f64_against_torch(hp, t0):
    rng = np.random.default_rng(6)
    n = 513
    w, m, v = _state(rng, n)
    grads = [rng.normal(0, 1e-3, n) for _ in range(4)]
    tw, tm, tv = _torch_adamw_steps(hp, w, m, v, grads, t0)
    for i, g in enumerate(grads):
        O.adamw_f64(O.Hparams(step=t0 + i, **hp), g, w, m, v)
    np.testing.assert_allclose(m, tm, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(v, tv, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(w, tw, rtol=1e-13, atol=0)


@pytest.mark.parametrize("hp", HPARAM_SETS)
@pytest.mark.parametrize("t0", [1, 10, 1000])
def test_adamw_f32_against_torch(hp, t0):
    """fp32 mode agrees with the float64 library step to fp32 rounding.  The
    update w' - w is compared on its own so that a wrong eps placement or a
    wrong decay term is not hidden by w's magnitude."""
    rng = np.random.default_rng(7)
    n = 2049
    w, m, v = (a.astype(np.float32) for a in _state(rng, n))
    g = rng.normal(0, 1e-3, n).astype(np.float32)
    tw, tm, tv = _torch_adamw_steps(hp, w, m, v, [g], t0)
    w1, m1, v1 = w.copy(), m.copy(), v.copy()
    O.adamw_f32(O.Hparams(step=t0, **hp), g, w1, m1, v1)
    u = 2.0 ** -24
    # each moment: two products and a sum in fp32, plus fp32 constants
    assert np.all(np.abs(m1 - tm) <= 6 * u * (np.abs(hp["beta1"] * m) +
                                              np.abs((1 - hp["beta1"]) * g)) + 1e-45)
    assert np.all(np.abs(v1 - tv) <= 8 * u * (np.abs(hp["beta2"] * v) +
                                              np.abs((1 - hp["beta2"]) * g * g)) + 1e-45)
    d_ref = tw - w.astype(np.float64)
    d_got = w1.astype(np.float64) - w.astype(np.float64)
    ulp_w = np.spacing(np.abs(w)).astype(np.float64)
    assert np.all(np.abs(d_got - d_ref) <= 16 * u * np.abs(d_ref) + ulp_w)


def test_adamw_f32_closed_forms():
    rng = np.random.default_rng(8)
    n = 4099
    g = rng.normal(0, 1e-3, n).astype(np.float32)
    w0, m0, v0 = (a.astype(np.float32) for a in _state(rng, n))

    # lr = 0: the weights do not move
    w, m, v = w0.copy(), m0.copy(), v0.copy()
    O.adamw_f32(O.Hparams(lr=0.0, step=5), g, w, m, v)
    assert np.array_equal(w.view(np.uint32), w0.view(np.uint32))

    # beta1 = beta2 = 0: m' = g and v' = g*g exactly, no bias correction
    w, m, v = w0.copy(), m0.copy(), v0.copy()
    O.adamw_f32(O.Hparams(lr=1e-3, beta1=0.0, beta2=0.0, eps=1e-8,
                          weight_decay=0.1, step=9), g, w, m, v)
    assert np.array_equal(m, g)
    assert np.array_equal(v, g * g)
    assert np.array_equal(np.sqrt(v), np.abs(g))

    # zero gradient from zero moments: only the decay acts, m' = v' = 0
    w = w0.copy()
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    O.adamw_f32(O.Hparams(lr=1e-3, weight_decay=0.1, step=1), np.zeros(n, np.float32),
                w, m, v)
    lr, wd = np.float32(1e-3), np.float32(0.1)
    assert np.array_equal(w, w0 - lr * (wd * w0))
    assert not m.any() and not v.any()

    # t = 1 from zero moments: the step is close to lr*(sign(g) + wd*w)
    w = w0.copy()
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    O.adamw_f32(O.Hparams(lr=1e-3, eps=1e-8, weight_decay=0.01, step=1), g, w, m, v)
    g64, w64 = g.astype(np.float64), w0.astype(np.float64)
    u = g64 / (np.abs(g64) + 1e-8) + 0.01 * w64
    ref = w64 - 1e-3 * u
    # a few fp32 roundings of the unit-size step, plus w's own rounding; a
    # wrong sign (2e-3) or a dropped decay term (~2e-7) is far outside
    tol = 8 * 2.0 ** -24 * 1e-3 * np.abs(u) + 2 * np.spacing(
        np.maximum(np.abs(w0), np.abs(w))).astype(np.float64)
    assert np.all(np.abs(w - ref) <= tol)


def test_constants_rounded_once_from_double():
    c = O.make_consts(O.Hparams(lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8,
                                weight_decay=0.1, step=1000))
    assert c["c1"] == np.float32(1.0 - 0.9)
    assert c["c1"] != np.float32(1.0) - np.float32(0.9)
    assert c["bc1"] == np.float32(1.0 - 0.9 ** 1000) == np.float32(1.0)
    assert c["bc2"] == np.float32(1.0 - 0.999 ** 1000)
    assert abs(float(c["bc2"]) - 0.6323045752290363) < 1e-7


# ---------------------------------------------------------------------- bf16

def test_bf16_rne_against_torch_structured_exhaustive():
    """Every bf16 high half, with low halves at and around the rounding
    boundary and a few random ones, against torch's float32->bfloat16."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x3FFF, 0x7FFF, 0x8000, 0x8001, 0xBFFF, 0xFFFF,
                     0x1234, 0x9ABC], dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).ravel()
    x = bits.view(np.float32)
    got = O.bf16_rne(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan_in = np.isnan(x)
    assert nan_in.sum() > 1000
    # Finite values and infinities bit for bit.  torch's CPU cast is not
    # consistent about NaN payloads (its vector path keeps high payload bits),
    # so NaN is compared as a class; the reading fixes the canonical 0x7FC0.
    assert np.array_equal(got[~nan_in], ref[~nan_in])
    assert np.all((ref[nan_in] & 0x7F80) == 0x7F80) and np.all((ref[nan_in] & 0x7F) != 0)
    assert np.all(got[nan_in] == 0x7FC0)


def test_bf16_rne_random_against_torch():
    rng = np.random.default_rng(9)
    bits = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    got = O.bf16_rne(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan_in = np.isnan(x)
    assert np.array_equal(got[~nan_in], ref[~nan_in])
    assert np.all(got[nan_in] == 0x7FC0)


# -------------------------------------------------------------------- layout

@pytest.mark.parametrize("align", [1, 2, 8, 128])
def test_layout_brute_force(align):
    for psi in list(range(1, 70)) + [127, 128, 129, 1000, 1023, 1024, 1025]:
        for n_d in range(1, 10):
            covered = np.zeros(psi, np.int32)
            S0 = None
            for k in range(n_d):
                S, off, V = O.layout(psi, n_d, k, align, stage=2)
                S0 = S if S0 is None else S0
                assert S == S0 and S % align == 0
                assert off == k * S
                assert 0 <= V <= S
                # S is the smallest multiple of align holding ceil(psi/n_d)
                need = -(-psi // n_d)
                assert S >= need and S - align < need
                covered[off:off + V] += 1
                if V < S:                       # padding only at the tail
                    assert off + V == psi or V == 0
            assert np.all(covered == 1)
            assert n_d * S0 >= psi


def test_layout_stage0_and_errors():
    assert O.layout(1000, 4, 3, 8, stage=0) == (1000, 0, 1000)
    assert O.layout(1001, 4, 0, 8, stage=0) == (1008, 0, 1001)
    for args, code in [((0, 4, 0, 8), -1), ((10, 0, 0, 8), -2), ((10, 4, 4, 8), -3),
                       ((10, 4, -1, 8), -3), ((10, 4, 0, 0), -4)]:
        with pytest.raises(ValueError) as e:
            O.layout(*args)
        assert e.value.args[0] == code
    with pytest.raises(ValueError):
        O.layout(10, 4, 0, 8, stage=4)


def test_layout_workload_shapes():
    """Shard shapes of the five workloads (derived from their stated sizes)."""
    assert O.layout(1_048_576, 4, 1, 128) == (262_144, 262_144, 262_144)
    assert O.layout(124_439_808, 8, 3, 1024) == (15_555_584, 46_666_752, 15_555_584)
    assert O.layout(124_439_808, 8, 7, 1024) == (15_555_584, 108_889_088, 15_550_720)
    assert O.layout(7_000_000_000, 8, 3, 1) == (875_000_000, 2_625_000_000, 875_000_000)
    assert O.layout(218_112_000, 8, 7, 2048) == (27_265_024, 190_855_168, 27_256_832)
    assert O.layout(70_000_000_000, 64, 0, 1, stage=3) == (1_093_750_000, 0, 1_093_750_000)


# ----------------------------------------------------------------- accounting

def test_memory_tables():
    g = golden("memory_tables.json")
    for r in g["rows"]:
        got = O.state_bytes(r["psi"], r["n_d"], r["stage"]) / 1e9
        assert abs(got - r["gb"]) <= r["tol"] + 1e-9, r
    p = g["per_param_at_4_ranks"]
    assert O.state_bytes(1, 4, 1) == p["stage1"]
    assert O.state_bytes(1, 4, 2) == p["stage2"]
    b = g["fsdp_budget_70b_64"]
    assert abs(2 * 70e9 / 64 / 1e9 - b["weights_gb"]) <= b["tol"]
    assert abs(O.state_bytes(70e9, 64, 3, K=0) / 2 / 1e9 - b["grads_gb"]) <= b["tol"]
    assert abs(12 * 70e9 / 64 / 1e9 - b["optimizer_gb"]) <= b["tol"]
    a = g["state_bytes_asserts"]
    assert O.state_bytes(7e9, 8, 3) == a["fsdp_7e9_8_equals"]
    assert O.state_bytes(50e9, 8, 3) > a["fsdp_50e9_8_exceeds"]
    bd = g["bounds_40gb_8"]
    for stage, billions in bd["params_b"].items():
        per_param = O.state_bytes(1.0, bd["n_d"], int(stage))
        assert abs(bd["gb"] / per_param - billions) <= bd["tol_b"]
    hs = g["hsdp_13b_32_g8_gb"]
    assert abs(O.hsdp_state_bytes(hs["psi"], hs["g"]) / 1e9 - hs["gb"]) < 1e-9
    # large-N_d limits of the Theorem's remark: 4 psi, 2 psi, 0
    assert abs(O.state_bytes(1.0, 10 ** 9, 1) - 4.0) < 1e-6
    assert abs(O.state_bytes(1.0, 10 ** 9, 2) - 2.0) < 1e-6
    assert O.state_bytes(1.0, 10 ** 9, 3) < 1e-6
    assert O.state_bytes(1.0, 4, 9) < 0


def test_comm_volumes():
    g = golden("comm_volumes.json")
    for r in g["ring_rows"]:
        got = O.comm_bytes(r["psi"], r["n_d"], r["stage"]) / 1e9
        assert abs(got - r["gb"]) <= r["tol"] + 1e-9, r
    z2 = g["zero2_reduce_scatter_13b_32_gb"]
    assert abs(O.comm_bytes(13e9, 32, 2) / 2 / 1e9 - z2["value"]) <= z2["tol"] + 1e-9
    for r in g["hsdp_rows"]:
        if "intra_gb" in r:
            assert abs(O.hsdp_intra_bytes(r["psi"], r["g"]) / 1e9 - r["intra_gb"]) <= r["tol"] + 1e-9
        assert abs(O.hsdp_inter_bytes(r["psi"], r["n_d"], r["g"]) / 1e9
                   - r["inter_gb"]) <= r["tol"] + 1e-9
    for r in g["times"]:
        assert abs(r["gb"] / r["gb_per_s"] - r["seconds"]) <= r.get("tol", 1e-12)
    assert O.comm_elems(1.0, 3) / O.comm_elems(1.0, 0) == g["ratio_zero3_over_ddp"]["value"]
    for m in (1, 2, 8):
        assert O.comm_elems_accum(1.0, 0, m) == 2
        assert O.comm_elems_accum(1.0, 1, m) == 2
        assert O.comm_elems_accum(1.0, 2, m) == m + 1
        assert O.comm_elems_accum(1.0, 3, m) == 3 * m


# --------------------------------------------------- the page's ZeRO-1 simulator

def _ring_sends(n_ranks, chunk_sizes):
    """Elements each rank sends in a ring reduce-scatter followed by a ring
    all-gather of chunks of the given sizes, counted transfer by transfer.
    Reduce-scatter: in round s rank k passes its running sum of chunk
    (k - s - 1) mod N to rank k + 1, so after N - 1 rounds rank k holds the
    whole sum of chunk k.  All-gather: in round s rank k passes chunk
    (k - s) mod N, starting with its own."""
    sent = [0] * n_ranks
    for s in range(n_ranks - 1):
        for k in range(n_ranks):
            sent[k] += chunk_sizes[(k - s - 1) % n_ranks]
    for s in range(n_ranks - 1):
        for k in range(n_ranks):
            sent[k] += chunk_sizes[(k - s) % n_ranks]
    return sent


def test_zero1_simulator_reproduction():
    """The ZeRO-1 experiment of "Data parallelism, ZeRO and FSDP", section 5,
    rebuilt from its statement: 4 simulated GPUs, 10 parameters, a global
    batch of 32 least-squares samples split into 4 equal micro-batches, 5
    AdamW steps.  Every rank holds all weights but the moments of its own
    slice only; each step it averages its slice of the ranks' gradients,
    updates that slice, and then every rank receives every updated slice.
    The page prints that this equals one GPU training on the whole batch
    (True, within 1e-12) and that each GPU sends 15.0 elements per step."""
    cfg = golden("comm_volumes.json")["simulator_zero1"]
    n_ranks, n_params, batch = cfg["n_gpus"], cfg["params"], cfg["batch"]
    hp = dict(lr=cfg["lr"], beta1=cfg["beta1"], beta2=cfg["beta2"], eps=cfg["eps"],
              weight_decay=cfg["wd"])
    rng = np.random.default_rng(20240805)
    feats = rng.normal(size=(batch, n_params))
    targets = rng.normal(size=batch)
    start = rng.normal(size=n_params)

    def mean_grad(w, idx):
        # the gradient of a mean loss is the mean of the per-sample gradients
        # of (x.w - y)^2 / 2, each (x.w - y) x
        per_sample = [(feats[i] @ w - targets[i]) * feats[i] for i in idx]
        return np.mean(per_sample, axis=0)

    # one GPU, the whole batch
    w1, m1, v1 = start.copy(), np.zeros(n_params), np.zeros(n_params)
    for t in range(1, cfg["steps"] + 1):
        O.adamw_f64(O.Hparams(step=t, **hp), mean_grad(w1, range(batch)), w1, m1, v1)

    # N ranks; slot k of the oracle's layout (tail padding: 3 + 3 + 3 + 1)
    slots = []
    for k in range(n_ranks):
        _, off, V = O.layout(n_params, n_ranks, k, 1, stage=1)
        slots.append(slice(off, off + V))
    per_rank = batch // n_ranks
    ranks = [{"w": start.copy(), "samples": range(k * per_rank, (k + 1) * per_rank),
              "m": np.zeros(slots[k].stop - slots[k].start),
              "v": np.zeros(slots[k].stop - slots[k].start)} for k in range(n_ranks)]
    sent_per_step = []
    for t in range(1, cfg["steps"] + 1):
        local = [mean_grad(r["w"], r["samples"]) for r in ranks]
        for k, r in enumerate(ranks):          # reduce-scatter, then the slice's update
            gk = O.reduce_mean_f64([np.ascontiguousarray(g[slots[k]]) for g in local])
            wk = np.ascontiguousarray(r["w"][slots[k]])
            O.adamw_f64(O.Hparams(step=t, **hp), gk, wk, r["m"], r["v"])
            r["w"][slots[k]] = wk
        for j, owner in enumerate(ranks):      # all-gather of the new slices
            for r in ranks:
                r["w"][slots[j]] = owner["w"][slots[j]]
        sends = _ring_sends(n_ranks, [sl.stop - sl.start for sl in slots])
        sent_per_step.append(sum(sends) / n_ranks)
    printed_true, printed_sent = cfg["prints"]
    deviation = max(np.abs(r["w"] - w1).max() for r in ranks)
    assert (deviation < cfg["max_diff_bound"]) == printed_true
    assert all(x == printed_sent for x in sent_per_step)
    # the oracle's communication formula gives the same count
    assert O.comm_bytes(n_params, n_ranks, 1, bytes_per_elem=1.0) == printed_sent


# ------------------------------------------- invariant: sharded == unsharded

def _ddp_vs_sharded(psi, n_d, align, h, grads_bf16, w0, m0, v0):
    """One unsharded step (stage 0 view) and the N_d sharded steps."""
    S0, _, V0 = O.layout(psi, n_d, 0, align, stage=0)
    w, m, v = w0.copy(), m0.copy(), v0.copy()
    q_parts = []
    Sk, _, _ = O.layout(psi, n_d, 0, align, stage=2)
    for k in range(n_d):
        _, off, V = O.layout(psi, n_d, k, align, stage=2)
        g = O.reduce_mean([np.ascontiguousarray(gr[off:off + V]) for gr in grads_bf16])
        q_parts.append(O.sqnorm(g))
    Qtot = 0.0
    for q in q_parts:
        Qtot += q
    gather = np.full(n_d * Sk, 0xFFFF, np.uint16)
    for k in range(n_d):
        _, off, V = O.layout(psi, n_d, k, align, stage=2)
        sl = [np.ascontiguousarray(gr[off:off + V]) for gr in grads_bf16]
        ws, ms, vs = (np.ascontiguousarray(a[off:off + V]) for a in (w, m, v))
        out, q, _ = O.shard_step(n_d, Sk, V, h, sl, ws, ms, vs,
                                 other_sqnorm=Qtot - q_parts[k])
        w[off:off + V], m[off:off + V], v[off:off + V] = ws, ms, vs
        gather[k * Sk:(k + 1) * Sk] = out
    wd, md, vd = w0.copy(), m0.copy(), v0.copy()
    outd, _, _ = O.shard_step(n_d, S0, V0, h, [np.ascontiguousarray(gr) for gr in grads_bf16],
                              wd, md, vd)
    return (w, m, v, gather[:psi]), (wd, md, vd, outd[:psi])


@pytest.mark.parametrize("psi", [1, 7, 1000, 4099])
@pytest.mark.parametrize("n_d", [1, 2, 3, 4, 8])
def test_sharded_equals_unsharded_no_clip(psi, n_d):
    rng = np.random.default_rng(psi * 31 + n_d)
    grads = [O.bf16_rne(rng.normal(0, 1e-3, psi).astype(np.float32)) for _ in range(n_d)]
    w0, m0, v0 = (a.astype(np.float32) for a in _state(rng, psi))
    h = O.Hparams(lr=1e-3, weight_decay=0.01, step=4)
    a, b = _ddp_vs_sharded(psi, n_d, 8, h, grads, w0, m0, v0)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


@pytest.mark.parametrize("n_d", [1, 2, 3, 8])
def test_sharded_equals_unsharded_clip_dyadic(n_d):
    """With the clip, sums are exact on small dyadic gradients, so the global
    norm from per-shard squared norms equals the one over the whole vector."""
    psi = 1001
    rng = np.random.default_rng(77 + n_d)
    grads = [bf16_of_exact(rng.integers(-64, 64, psi) * 2.0 ** -8) for _ in range(n_d)]
    w0, m0, v0 = (a.astype(np.float32) for a in _state(rng, psi))
    h = O.Hparams(lr=1e-3, weight_decay=0.01, step=2, max_grad_norm=0.5)
    a, b = _ddp_vs_sharded(psi, n_d, 8, h, grads, w0, m0, v0)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_clip_inactive_is_bitwise_no_clip():
    rng = np.random.default_rng(10)
    n_d, V = 4, 3000
    sl = [O.bf16_rne(rng.normal(0, 1e-3, V).astype(np.float32)) for _ in range(n_d)]
    w0, m0, v0 = (a.astype(np.float32) for a in _state(rng, V))
    res = []
    for mg in (0.0, 1e6):
        w, m, v = w0.copy(), m0.copy(), v0.copy()
        out, q, coef = O.shard_step(n_d, V + 8, V, O.Hparams(step=3, max_grad_norm=mg),
                                    sl, w, m, v)
        res.append((w.tobytes(), m.tobytes(), v.tobytes(), out.tobytes()))
    assert res[0] == res[1]


def test_empty_shard_writes_only_pads():
    h = O.Hparams(step=1, max_grad_norm=1.0)
    empty = np.zeros(0, np.uint16)
    w = np.zeros(0, np.float32)
    out, q, coef = O.shard_step(2, 16, 0, h, [empty, empty], w, w.copy(), w.copy())
    assert q == 0.0 and coef == np.float32(1.0)
    assert not out.any()


def test_pack_rounds_and_pads():
    w = np.array([1.0, 1.00390625, 1.01171875, -3.0e38, 1e-45], np.float32)
    out = O.pack(8, w)
    ref = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out[:5], ref)
    assert not out[5:].any()


@pytest.mark.parametrize("n_d,max_norm", [(1, 0.0), (4, 0.0), (8, 1e-3), (3, 0.01),
                                          (64, 1e-4)])
def test_shard_step_against_torch_clip_and_adamw(n_d, max_norm):
    """The whole O1..O5 composition against the library: mean of the ranks'
    bf16 gradients, clip_grad_norm_ over the shard plus the other shards'
    squared norm, torch.optim.AdamW, all in float64; the fp32 oracle must
    agree to fp32 rounding, and its bf16 output must be within one bf16 step
    of torch's rounding of the float64 weights."""
    rng = np.random.default_rng(11 + n_d)
    V, S = 3001, 3008
    sl = [O.bf16_rne(rng.normal(0, 1e-3, V).astype(np.float32)) for _ in range(n_d)]
    w0, m0, v0 = (a.astype(np.float32) for a in _state(rng, V))
    other = 2.5e-5
    hp = dict(lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
    t = 17

    g64 = np.stack([O.bf16_to_f32(s).astype(np.float64) for s in sl]).sum(0) / n_d
    if max_norm > 0:
        p = torch.nn.Parameter(torch.zeros(V, dtype=torch.float64))
        p.grad = torch.from_numpy(g64.copy())
        other_p = torch.nn.Parameter(torch.zeros(1, dtype=torch.float64))
        other_p.grad = torch.tensor([math.sqrt(other)], dtype=torch.float64)
        torch.nn.utils.clip_grad_norm_([p, other_p], max_norm)
        g64 = p.grad.numpy().copy()
    tw, tm, tv = _torch_adamw_steps(hp, w0, m0, v0, [g64], t)

    w, m, v = w0.copy(), m0.copy(), v0.copy()
    out, q, coef = O.shard_step(n_d, S, V, O.Hparams(step=t, max_grad_norm=max_norm, **hp),
                                sl, w, m, v, other_sqnorm=other)
    if max_norm > 0:
        assert coef < 1.0
    u = 2.0 ** -24
    gsc = np.abs(g64)
    assert np.all(np.abs(m - tm) <= 12 * u * (np.abs(0.9 * m0) + 0.1 * gsc) + 1e-45)
    assert np.all(np.abs(v - tv) <= 16 * u * (np.abs(0.999 * v0) + 1e-3 * gsc * gsc) + 1e-45)
    d_ref = tw - w0.astype(np.float64)
    d_got = w.astype(np.float64) - w0.astype(np.float64)
    assert np.all(np.abs(d_got - d_ref) <= 32 * u * np.abs(d_ref)
                  + np.spacing(np.abs(w0)).astype(np.float64))
    ref16 = (torch.from_numpy(tw).to(torch.bfloat16).view(torch.int16).numpy()
             .view(np.uint16).astype(np.int32))
    assert np.all(np.abs(out[:V].astype(np.int32) - ref16) <= 1)
    assert not out[V:].any()


# ------------------------------------------------- fp32 gradient slices (reduce_dtype)

def test_reduce_f32_worked_example():
    """The worked example with fp32 slices: -1.5 and -13 (two ranks), and the
    four per-sample gradients (four ranks), average to -7.25."""
    g = golden("worked_example_two_gpus.json")
    two = O.reduce_mean_f32([np.array([m], np.float32) for m in g["gpu_means"]])
    four = O.reduce_mean_f32([np.array([v], np.float32) for v in g["grad_per_sample"]])
    assert two[0] == np.float32(g["allreduce_mean"])
    assert four[0] == np.float32(g["allreduce_mean"])


def test_reduce_f32_equals_bf16_path_on_bf16_values():
    """fp32 slices holding bf16 values (the FSDP2 bf16-param / fp32-reduce
    policy widens bf16 gradients) give the bf16 reduction's bits."""
    rng = np.random.default_rng(21)
    for n_d in (1, 2, 3, 5, 8, 64):
        sl = [O.bf16_rne(rng.normal(0, 1e-3, 777).astype(np.float32)) for _ in range(n_d)]
        a = O.reduce_mean(sl)
        b = O.reduce_mean_f32([O.bf16_to_f32(x).copy() for x in sl])
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_reduce_f32_exact_and_correctly_rounded():
    """Sums of these dyadic values are exact in fp32, so the result is the
    exact mean rounded once (any N_d, power of two or not)."""
    rng = np.random.default_rng(22)
    for n_d in (1, 2, 3, 4, 7, 8, 64):
        ints = rng.integers(-(1 << 16), 1 << 16, size=(n_d, 129))
        sl = [np.ascontiguousarray((r * 2.0 ** -30).astype(np.float32)) for r in ints]
        got = O.reduce_mean_f32(sl)
        for i in range(129):
            exact = Fraction(int(ints[:, i].sum()), 1 << 30) / n_d
            assert got[i] == np.float32(float(exact))


def test_reduce_f32_rank_order():
    """1 + 2^-24 is a tie that rounds to 1, twice; the reverse order would
    give 1 + 2^-23 exactly."""
    sl = [np.array([1.0], np.float32), np.array([2.0 ** -24], np.float32),
          np.array([2.0 ** -24], np.float32)]
    got = O.reduce_mean_f32(sl)[0]
    assert got == np.float32(1.0) / np.float32(3.0)
    assert got != np.float32(1.0 + 2.0 ** -23) / np.float32(3.0)


# ------------------------------------------------------- token-weighted reduction

def test_token_weights_worked_example():
    """Two ranks with 2 and 6 valid tokens and local mean losses 3 and 1: the
    global mean is (2*3 + 6*1)/8 = 1.5, not the plain average 2."""
    w = O.token_weights([2, 6])
    assert w.tolist() == [0.25, 0.75]
    for sl in ([np.array([3.0], np.float32), np.array([1.0], np.float32)],
               [bf16_of_exact([3.0]), bf16_of_exact([1.0])]):
        assert O.reduce_weighted(sl, w)[0] == np.float32(1.5)
    assert O.reduce_mean([bf16_of_exact([3.0]), bf16_of_exact([1.0])])[0] == np.float32(2.0)


def test_token_weights_zero_token_rank_and_zero_total():
    """A zero-token rank contributes zero: the result is the other ranks'
    weighted sum exactly; a zero global count rejects the update."""
    rng = np.random.default_rng(23)
    g1 = rng.normal(0, 1e-3, 1000).astype(np.float32)
    g0 = rng.normal(0, 1e-3, 1000).astype(np.float32)
    got = O.reduce_weighted([g0, g1], O.token_weights([0, 17]))
    assert np.array_equal(got.view(np.uint32), g1.view(np.uint32))
    with pytest.raises(O.ZeroTokens):
        O.token_weights([0, 0, 0])
    with pytest.raises(ValueError):
        O.token_weights([3, -1])


def test_token_weights_rounded_once_from_double():
    """w_r = f32(n_r / T) computed in double: 16777217 is not an fp32 value,
    so dividing the fp32-rounded counts would give another weight."""
    w = O.token_weights([16777217, 1])
    T = 16777218
    assert w[0] == np.float32(16777217 / T) and w[1] == np.float32(1 / T)
    assert w[0] != np.float32(16777217) / np.float32(T)


def test_token_weights_equal_counts_is_the_mean():
    """Equal counts over a power-of-two number of ranks: w_r = 2^-k exactly,
    and scaling by 2^-k commutes with rounding, so the weighted sum is the
    plain mean bit for bit (normal values)."""
    rng = np.random.default_rng(24)
    for n_d in (1, 2, 4, 8, 64):
        sl = [O.bf16_rne(rng.normal(0, 1e-3, 513).astype(np.float32)) for _ in range(n_d)]
        got = O.reduce_weighted(sl, O.token_weights([4096] * n_d))
        assert np.array_equal(got.view(np.uint32), O.reduce_mean(sl).view(np.uint32))


def test_token_weighted_exact_on_dyadics():
    rng = np.random.default_rng(25)
    tokens = [1, 3, 0, 4]            # T = 8: weights 1/8, 3/8, 0, 4/8 exact
    w = O.token_weights(tokens)
    ints = rng.integers(-255, 256, size=(4, 200))
    sl = [bf16_of_exact(r * 2.0 ** -12) for r in ints]
    got = O.reduce_weighted(sl, w)
    for i in range(200):
        exact = sum(Fraction(tokens[r], 8) * Fraction(int(ints[r, i]), 1 << 12) for r in range(4))
        assert Fraction(float(got[i])) == exact


# ------------------------------------------------- ZeRO-2 gradient accumulation

def test_accumulate_worked_example():
    """Gradient accumulation on one rank: micro-batches [x1, x2] and [x3, x4]
    have mean gradients -1.5 and -13; accumulating both and taking the mean
    over micro-batches gives -7.25, the full-batch gradient."""
    g = golden("worked_example_two_gpus.json")
    acc = np.full(1, np.nan, np.float32)      # never read on the first micro-batch
    for j, mj in enumerate(g["gpu_means"]):
        O.accumulate(np.array([mj], np.float32), j, 2, acc)
    assert acc[0] == np.float32(g["one_gpu_full_batch_mean"])


def test_accumulate_single_micro_batch_is_identity():
    rng = np.random.default_rng(26)
    r = rng.normal(0, 1.0, 300).astype(np.float32)
    acc = np.full(300, np.nan, np.float32)
    O.accumulate(r, 0, 1, acc)
    assert np.array_equal(acc.view(np.uint32), r.view(np.uint32))


def test_accumulate_zero2_equals_ddp_accumulation_on_dyadics():
    """ZeRO-2 reduces every micro-batch and adds the reduced slices; DDP
    (no_sync) adds full local gradients and reduces once.  On values whose
    sums are exact both equal the mean over all m * N_d contributions."""
    rng = np.random.default_rng(27)
    for n_d, m in ((1, 4), (2, 2), (4, 3), (8, 4)):
        ints = rng.integers(-255, 256, size=(m, n_d, 65))
        acc = np.empty(65, np.float32)
        for j in range(m):
            r_j = O.reduce_mean([bf16_of_exact(ints[j, r] * 2.0 ** -8) for r in range(n_d)])
            O.accumulate(r_j, j, m, acc)
        for i in range(65):
            exact = Fraction(int(ints[:, :, i].sum()), 256 * n_d * m)
            if m & (m - 1) == 0:
                assert Fraction(float(acc[i])) == exact
            else:                                   # one rounding, by 1/m
                assert acc[i] == np.float32(float(exact))


def test_accumulate_micro_batch_order():
    """((2^24 + 1) + 1) / 3 in micro-batch order rounds to 2^24 / 3."""
    acc = np.empty(1, np.float32)
    for j, v in enumerate((2.0 ** 24, 1.0, 1.0)):
        O.accumulate(np.array([v], np.float32), j, 3, acc)
    assert acc[0] == np.float32(2.0 ** 24) / np.float32(3.0)
