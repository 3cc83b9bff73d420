"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names the fact it checks: a worked value the pages print, a closed
form, an identity of the mathematics, a library routine a special case reduces
to, exact rational arithmetic on tiny inputs, or finite differences.  The
``test_teeth_*`` tests plant a mistake in the oracle (on the CPU) and check
that a pin catches it.
"""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import adaln, fpmath, modulation, proj_out, residual, token_tree
from oracle.fpmath import bf16_ulp_diff, bits_to_f32, f32_to_bf16_bits, nsum
from synthetic_inputs import cancellation_tokens, make_inputs, make_mod6_inputs, make_residual_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
D = 3072


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def frac_to_f32(fr: Fraction) -> np.float32:
    """Correctly rounded float32 of an exact rational (ties to even)."""
    f = np.float32(float(fr))
    best = f
    for cand in (np.nextafter(f, np.float32(-np.inf)), np.nextafter(f, np.float32(np.inf))):
        dc = abs(Fraction(float(cand)) - fr)
        db = abs(Fraction(float(best)) - fr)
        if dc < db or (dc == db and (int(cand.view(np.uint32)) & 1) == 0):
            best = cand
    return np.float32(best)


def f32_ulps(a, b):
    """Distance in float32 ulps (monotone integer mapping)."""
    def key(v):
        u = np.asarray(v, np.float32).view(np.int32).astype(np.int64)
        return np.where(u < 0, -(u & 0x7FFFFFFF), u)
    return np.abs(key(a) - key(b))


# ------------------------------------------------------------ bf16 rounding --
def test_bf16_round_matches_torch_conversion():
    """fp32 -> bf16 is the library conversion torch.Tensor.to(bfloat16) performs."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * np.float32(7.0),
        (rng.integers(0, 2**32, 100000, dtype=np.uint64).astype(np.uint32)).view(np.float32),
        # exact ties: low 16 bits 0x8000, both parities of the kept bit
        (np.arange(0x3F800000, 0x3F800000 + (4 << 16), 1 << 15, dtype=np.uint32) | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1e-40, -1e-40, 3.4e38, -3.4e38, np.inf, -np.inf], np.float32),
    ])
    v = v[np.isfinite(v) | np.isinf(v)]
    ours = f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f64_to_bf16_single_rounding():
    """float64 -> bf16 rounds once: checked against exact rational rounding."""
    rng = np.random.default_rng(2)
    vals = list(rng.standard_normal(3000) * 3.0)
    # values a hair above / below a bf16 tie that float32 rounding would land on the tie
    for base in (1.0, 1.5, -2.25, 3.0e-3):
        b16 = float(fpmath.bits_to_f32(fpmath.f32_to_bf16_bits(np.array([base], np.float32)))[0])
        ulp = 2.0 ** (math.frexp(abs(b16))[1] - 8)
        tie = b16 + ulp / 2
        vals += [tie + ulp * 2.0 ** -30, tie - ulp * 2.0 ** -30, tie]
    vals = np.array(vals, np.float64)
    got = fpmath.f64_to_bf16_bits(vals)
    for v, g in zip(vals, got):
        fr = Fraction(float(v))
        # candidates: the two bf16 values around v
        lo = int(fpmath.f32_to_bf16_bits(np.array([v], np.float32))[0])
        cands = {(lo + d) & 0xFFFF for d in (-1, 0, 1)}
        best, bestd = None, None
        for c in sorted(cands):
            cv = float(bits_to_f32(np.array([c], np.uint16))[0])
            dist = abs(Fraction(cv) - fr)
            if bestd is None or dist < bestd or (dist == bestd and (c & 1) == 0):
                best, bestd = c, dist
        assert int(g) == best, (v, hex(int(g)), hex(best))


# ---------------------------------------------------------------- NSum (P-1) --
@pytest.mark.parametrize("kind", ["normal", "wide", "cancel", "ones_big"])
def test_nsum_within_one_ulp_of_exact(kind):
    """Sequential Neumaier sum vs math.fsum / exact rationals (correctly rounded)."""
    rng = np.random.default_rng(3)
    for trial in range(20):
        n = int(rng.integers(1, 3000))
        if kind == "normal":
            x = rng.standard_normal(n).astype(np.float32)
        elif kind == "wide":
            x = (rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n))).astype(np.float32)
        elif kind == "cancel":
            h = rng.standard_normal(n).astype(np.float32) * np.float32(1e4)
            x = np.concatenate([h, -h[::-1], rng.standard_normal(5).astype(np.float32)])
            rng.shuffle(x)
        else:
            x = np.ones(n + 2, np.float32)
            x[int(rng.integers(0, n + 2))] = np.float32(2 ** 26)
            x[int(rng.integers(0, n + 2))] -= np.float32(2 ** 26)
        exact = sum(Fraction(float(v)) for v in x)
        want = frac_to_f32(exact)
        got = nsum(x)
        assert f32_ulps(got, want) <= 1, (kind, n, got, want)
        # and it is far better than plain float32 accumulation in the cancel case
        assert abs(float(math.fsum(map(float, x))) - float(got)) <= abs(float(want)) * 2 ** -23 + 1e-30


def test_nsum_tiny_bruteforce_exact():
    """P-14: exact rational sums of a few hundred elements; NSum equals the
    correctly rounded value (it can miss by 1 ulp only in contrived cases)."""
    rng = np.random.default_rng(4)
    eq = 0
    for trial in range(200):
        n = int(rng.integers(1, 300))
        x = (rng.standard_normal(n) * np.exp2(rng.integers(-8, 8, n))).astype(np.float32)
        want = frac_to_f32(sum(Fraction(float(v)) for v in x))
        got = nsum(x)
        assert f32_ulps(got, want) <= 1
        eq += int(got == want)
    assert eq >= 198


# ------------------------------------------------------------ token tree (P-2) --
POSITIONS = [(0, 32), (0, 1), (5, 6000), (6031, 0), (31, 32), (6016, 6031), (100, 4000),
             (1, 2), (6030, 6031), (3000, 3001), (64, 96), (6015, 6016), (0, 6031), (17, 4113)]


def test_cancellation_probe_golden():
    """The pages' worked example: compensated tree 6030 for every placement,
    the sequential Neumaier reference 6030, the plain 32-way tree 6020."""
    gd = _golden("cancellation_probe.json")
    S, big = gd["S"], gd["big"]
    plain_vals = {}
    for p, q in POSITIONS:
        v = cancellation_tokens(S, p, q, big)
        assert token_tree.tree_sum(v[None, :, None])[0, 0] == np.float32(gd["compensated_tree"])
        assert nsum(v) == np.float32(gd["exact_sum"])
        plain_vals[(p, q)] = float(token_tree.plain_tree_sum(v[None, :, None])[0, 0])
    # the large tokens at leaf position 0 of different tiles: the pages' 6020
    assert plain_vals[(0, 32)] == gd["plain_tree"]
    assert plain_vals[(5, 6000)] == gd["plain_tree"] or plain_vals[(64, 96)] == gd["plain_tree"]


def test_cancellation_probe_in_three_columns_and_batch():
    """Same probe in a [B, S, 3] layout: every column, every sample gives 6030."""
    S = 6032
    cols = [cancellation_tokens(S, 0, 32), cancellation_tokens(S, 31, 6031), cancellation_tokens(S, 6016, 1)]
    x = np.stack(cols, axis=1)[None].repeat(3, axis=0)
    r = token_tree.tree_sum(x)
    assert np.all(r == np.float32(6030.0))


@pytest.mark.parametrize("S", [1, 2, 31, 32, 33, 64, 1023, 1024, 1025, 6032, 6889])
def test_tree_error_bound_random(S):
    """Tree result within the compensated-sum error bound of the exact sum."""
    rng = np.random.default_rng(5 + S)
    H = 16
    x = (rng.standard_normal((2, S, H)) * np.exp2(rng.integers(-10, 10, (2, S, H)))).astype(np.float32)
    r = token_tree.tree_sum(x)
    for b in range(2):
        for h in range(H):
            col = x[b, :, h].astype(np.float64)
            ex = math.fsum(col)
            A = float(np.abs(col).sum())
            assert abs(float(r[b, h]) - ex) <= 2 * 2 ** -24 * abs(ex) + 64 * 2 ** -48 * A + 1e-45


@pytest.mark.parametrize("S,pad", [(1, 1), (5, 27), (31, 1), (32, 1), (33, 31), (1000, 24),
                                   (1024, 1), (1025, 1023), (6032, 5000)])
def test_tree_zero_padding_neutral(S, pad):
    """P-3: appending zero tokens never changes a byte of the tree sum."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((2, S, 8)).astype(np.float32)
    xp = np.concatenate([x, np.zeros((2, pad, 8), np.float32)], axis=1)
    assert token_tree.tree_sum(x).tobytes() == token_tree.tree_sum(xp).tobytes()
    assert nsum(x, axis=1).tobytes() == nsum(xp, axis=1).tobytes()


def test_tree_levels_shape_depends_only_on_S():
    assert token_tree.tree_levels(1) == [1]
    assert token_tree.tree_levels(32) == [1]
    assert token_tree.tree_levels(33) == [2, 1]
    assert token_tree.tree_levels(4096) == [128, 4, 1]
    assert token_tree.tree_levels(6889) == [216, 7, 1]
    assert token_tree.tree_levels(40000) == [1250, 40, 2, 1]


# ----------------------------------------------------- forward / backward pins --
def _small_inputs(B, S, seed=0, **kw):
    return make_inputs(B, S, seed=seed, **kw)


def _textbook_ln(xv, eps=1e-6):
    x = xv.astype(np.float64)
    mu = x.mean(-1, keepdims=True)
    var = ((x - mu) ** 2).mean(-1, keepdims=True)
    return (x - mu) / np.sqrt(var + np.float64(np.float32(eps)))


def test_s1_token_sums_closed_form():
    """P-4: with one token, d_shift is g and d_scale is g*n, bit for bit."""
    inp = _small_inputs(2, 1, seed=7)
    f = adaln.forward(inp)
    b = adaln.backward(inp, f)
    g = bits_to_f32(inp["g"])
    assert b["d_shift"].tobytes() == g[:, 0, :].tobytes()
    assert b["d_scale"].tobytes() == (g[:, 0, :] * f["n"][:, 0, :]).astype(np.float32).tobytes()


def test_layernorm_closed_forms():
    """P-5: mean(n) = 0 and mean(n^2) = v/(v+eps); LN(20 x) = LN(x) up to eps."""
    inp = _small_inputs(1, 48, seed=8, outlier_frac=0.1)
    f = adaln.forward(inp, "fp64")
    n = f["n"][0]
    v = f["var"][0]
    assert np.all(np.abs(n.mean(-1)) < 1e-7)
    ratio = (n ** 2).mean(-1) / (v / (v + np.float32(1e-6)))
    assert np.all(np.abs(ratio - 1) < 1e-6)
    ex = dict(inp)
    xv = bits_to_f32(inp["x"]).astype(np.float64)
    ex = {k: v2 for k, v2 in inp.items()}
    ex["x_val"] = xv
    e1 = adaln.forward(ex, "exact")
    ex["x_val"] = 20.0 * xv
    e2 = adaln.forward(ex, "exact")
    assert np.max(np.abs(e1["n"] - e2["n"])) < 1e-5


def test_constant_rows_closed_form():
    """P-5b: a row of one repeated value v has mean v, variance 0, rstd =
    fp32(1 / sqrt(fp32(1e-6))) and n = 0, so out is the shift bit for bit; and
    its dx is rstd * (g m - mean(g m)) (beta drops out with n = 0), rounded
    once."""
    inp = _small_inputs(1, 5, seed=12)
    vals = np.array([0.0, 0.75, -3.0, 1.0e4, 2.0 ** -20], np.float32)
    inp["x"] = f32_to_bf16_bits(np.repeat(vals, D).reshape(1, 5, D))
    f = adaln.forward(inp)
    b = adaln.backward(inp, f)
    v = bits_to_f32(inp["x"])[0, :, 0]
    assert np.array_equal(f["mean"][0], v)
    rs = np.float32(1.0) / np.sqrt(np.float32(1e-6), dtype=np.float32)
    assert np.all(f["rstd"][0] == rs)
    assert np.array_equal(f["out_bits"], np.broadcast_to(f["emb_bits"][:, D:][:, None, :], f["out_bits"].shape))
    gm = bits_to_f32(inp["g"])[0].astype(np.float64) * f["m"][0].astype(np.float64)
    want = rs.astype(np.float64) * (gm - gm.mean(-1, keepdims=True))
    d = bf16_ulp_diff(b["dx_bits"][0], fpmath.f64_to_bf16_bits(want))
    assert d.max() <= 1


def test_identity_modulation_is_textbook_layernorm():
    """P-6: W = 0, b = 0 gives out = bf16(LayerNorm(x)); checked against a
    float64 two-pass LayerNorm; and scale = -1 gives out = shift exactly."""
    inp = _small_inputs(2, 40, seed=9, outlier_frac=0.05)
    inp["W"] = np.zeros_like(inp["W"])
    inp["bias"] = np.zeros_like(inp["bias"])
    f = adaln.forward(inp)
    want = fpmath.f64_to_bf16_bits(_textbook_ln(bits_to_f32(inp["x"])))
    d = bf16_ulp_diff(f["out_bits"], want)
    assert d.max() <= 1 and (d == 0).mean() > 0.999
    # scale = -1  ->  m = bf16(1 + -1) = 0  ->  out = bf16(0 * n + shift) = shift
    rng = np.random.default_rng(10)
    sh = f32_to_bf16_bits(rng.standard_normal(D).astype(np.float32))
    inp["bias"] = np.concatenate([f32_to_bf16_bits(np.full(D, -1.0, np.float32)), sh])
    f2 = adaln.forward(inp)
    assert np.all(f2["m"] == 0)
    assert np.array_equal(f2["out_bits"], np.broadcast_to(sh, f2["out_bits"].shape))


def _order_check(f, inp, c1, c2):
    n_tb = _textbook_ln(bits_to_f32(inp["x"]))
    right = fpmath.f64_to_bf16_bits(n_tb * (1.0 + c1) + c2)
    wrong = fpmath.f64_to_bf16_bits(n_tb * (1.0 + c2) + c1)
    dr = bf16_ulp_diff(f["out_bits"], right)
    dw = bf16_ulp_diff(f["out_bits"], wrong)
    return dr.max() <= 1 and (dw > 1).mean() > 0.5


def test_scale_shift_order():
    """P-7: emb.chunk(2) gives (scale, shift) in that order."""
    inp = _small_inputs(1, 16, seed=11)
    c1, c2 = 0.5, 0.25
    inp["W"] = np.zeros_like(inp["W"])
    inp["bias"] = np.concatenate([f32_to_bf16_bits(np.full(D, c1, np.float32)),
                                  f32_to_bf16_bits(np.full(D, c2, np.float32))])
    assert _order_check(adaln.forward(inp), inp, c1, c2)


def test_projection_matches_float64_dot():
    """P-8: emb = bf16(a W^T + b) against numpy's float64 matmul; W = [I; 0]
    and b = 0 give emb = (a | 0) exactly."""
    inp = _small_inputs(2, 1, seed=12)
    f = adaln.forward(inp)
    a = f["a"].astype(np.float64)
    W = bits_to_f32(inp["W"]).astype(np.float64)
    bias = bits_to_f32(inp["bias"]).astype(np.float64)
    want = fpmath.f64_to_bf16_bits(a @ W.T + bias)
    d = bf16_ulp_diff(f["emb_bits"], want)
    assert d.max() <= 1 and (d == 0).mean() > 0.999
    eye = np.concatenate([np.eye(D, dtype=np.float32), np.zeros((D, D), np.float32)])
    inp["W"] = f32_to_bf16_bits(eye)
    inp["bias"] = np.zeros_like(inp["bias"])
    f2 = adaln.forward(inp)
    assert np.array_equal(f2["emb_bits"][:, :D], f2["a_bits"])
    assert np.all(bits_to_f32(f2["emb_bits"][:, D:]) == 0)


def test_projection_tiny_exact_rationals():
    """P-14: tiny projection against exact rational dot products."""
    rng = np.random.default_rng(13)
    K, N, B = 24, 10, 3
    a = bits_to_f32(f32_to_bf16_bits(rng.standard_normal((B, K)).astype(np.float32)))
    W = bits_to_f32(f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.3).astype(np.float32)))
    bias = bits_to_f32(f32_to_bf16_bits((rng.standard_normal(N) * 0.1).astype(np.float32)))
    got = adaln.projection(a, W, bias, adaln.Arith("fp32"))
    for b in range(B):
        for j in range(N):
            ex = sum(Fraction(float(a[b, k])) * Fraction(float(W[j, k])) for k in range(K))
            acc = frac_to_f32(ex)
            want = f32_to_bf16_bits(np.float32(acc + bias[j]))
            assert bf16_ulp_diff(f32_to_bf16_bits(got[b, j]), want) == 0


def _proj_bwd_cancelling_case(seed=21, B=3, N=12, K=10):
    """Tiny projection-backward operands whose sums nearly cancel: sample 1
    repeats sample 0 with a negated a and a d_emb a few fp32 ulps away, row 1
    of W negates row 0 and d_emb column 1 sits a few ulps from column 0.  The
    d_emb values carry full 24-bit significands, so a product rounded to fp32
    on its own loses bits that the cancelling sum exposes."""
    rng = np.random.default_rng(seed)
    bf = lambda v: bits_to_f32(f32_to_bf16_bits(np.asarray(v, np.float32)))   # noqa: E731
    a = bf(rng.standard_normal((B, K)))
    a[1] = -a[0]
    W = bf(rng.standard_normal((N, K)) * 0.3)
    W[1] = -W[0]
    d = (rng.standard_normal((B, N)) * (1 + rng.random((B, N)))).astype(np.float32)
    steps = rng.integers(1, 9, (N,)).astype(np.int64)
    d[1] = (d[0].view(np.int32) + steps.astype(np.int32)).view(np.float32)
    d[:, 1] = (d[:, 0].view(np.int32) + np.int32(3)).view(np.float32)
    temb = bf(rng.standard_normal((B, K)))
    return d, a, W, temb


def _exact_proj_bwd(d, a, W):
    B, N = d.shape
    K = a.shape[1]
    F = lambda v: Fraction(float(v))   # noqa: E731
    dW = np.empty((N, K), np.float32)
    for j in range(N):
        for k in range(K):
            dW[j, k] = frac_to_f32(sum(F(d[b, j]) * F(a[b, k]) for b in range(B)))
    da = np.empty((B, K), np.float32)
    for b in range(B):
        for k in range(K):
            da[b, k] = frac_to_f32(sum(F(d[b, j]) * F(W[j, k]) for j in range(N)))
    return dW, da


def test_projection_backward_tiny_exact_rationals():
    """P-15: da and dW against exact rational sums of exact products, rounded
    once to fp32 (dW then to bf16), on operands that cancel."""
    d, a, W, temb = _proj_bwd_cancelling_case()
    r = adaln.proj_backward(d, a, W, temb, adaln.Arith("fp32"))
    dW_ex, da_ex = _exact_proj_bwd(d, a, W)
    assert np.array_equal(f32_to_bf16_bits(r["dW"]), f32_to_bf16_bits(dW_ex))
    assert np.array_equal(r["dW_acc"].view(np.uint32), dW_ex.view(np.uint32))
    assert np.array_equal(r["da"].view(np.uint32), da_ex.view(np.uint32))
    # dtemb before its bf16 rounding: the exact-rational da times silu'(z)
    # (sigma(z) (1 + z (1 - sigma(z))) in float64, rounded to fp32), one fp32 product
    z = temb.astype(np.float64)
    sg = 1.0 / (1.0 + np.exp(-z))
    ds = (sg * (1.0 + z * (1.0 - sg))).astype(np.float32)
    assert np.array_equal(r["dtemb_acc"].view(np.uint32), (da_ex * ds).view(np.uint32))
    assert np.array_equal(f32_to_bf16_bits(r["dtemb_acc"]), f32_to_bf16_bits(r["dtemb"]))


def test_teeth_rounded_products_caught(monkeypatch):
    """Rounding each backward product to fp32 on its own fails P-15."""
    monkeypatch.setattr(adaln.Arith, "prod",
                        lambda self, x, y: ((np.asarray(x, self.dt) * np.asarray(y, self.dt)),))
    d, a, W, temb = _proj_bwd_cancelling_case()
    r = adaln.proj_backward(d, a, W, temb, adaln.Arith("fp32"))
    dW_ex, da_ex = _exact_proj_bwd(d, a, W)
    assert not (np.array_equal(r["dW_acc"].view(np.uint32), dW_ex.view(np.uint32))
                and np.array_equal(r["da"].view(np.uint32), da_ex.view(np.uint32)))


def test_silu_worked_value_and_special_cases():
    """P-9: the review thread's worked value silu'(1) = 0.9277; silu(0) = 0,
    silu'(0) = 1/2; silu(z) -> z for large z and -> 0 for very negative z."""
    gd = _golden("silu_derivative.json")
    ar = adaln.Arith("fp32")
    z = np.array([gd["z"]], np.float32)
    v = float(adaln.dsilu(z, ar)[0])
    assert abs(v - gd["dsilu"]) < 0.5 * 10 ** -gd["digits"] + 1e-6
    assert float(adaln.dsilu(np.array([0.0], np.float32), ar)[0]) == 0.5
    assert float(adaln._silu64(np.float64(0.0))) == 0.0
    assert adaln._silu64(np.float64(60.0)) == 60.0
    assert abs(adaln._silu64(np.float64(-60.0))) < 1e-24


def test_layernorm_backward_identities():
    """P-10: sum_d dx = 0 and sum_d dx n = rstd eps/(v+eps) sum_d gy n, in exact arithmetic."""
    rng = np.random.default_rng(14)
    B, S, Dd = 2, 5, 64
    inp = {"x_val": rng.standard_normal((B, S, Dd)) * 0.01, "temb_val": rng.standard_normal((B, Dd)),
           "W_val": rng.standard_normal((2 * Dd, Dd)) * 0.02, "bias_val": rng.standard_normal(2 * Dd) * 0.01,
           "g_val": rng.standard_normal((B, S, Dd))}
    f = adaln.forward(inp, "exact")
    b = adaln.backward(inp, f, "exact")
    dx, n = b["dx"], f["n"]
    assert np.all(np.abs(dx.sum(-1)) <= 1e-12 * np.abs(dx).sum(-1))
    gy = inp["g_val"] * f["m"][:, None, :]
    lhs = (dx * n).sum(-1)
    v, eps = f["var"], np.float64(np.float32(1e-6))
    rhs = f["rstd"] * eps / (v + eps) * (gy * n).sum(-1)
    assert np.all(np.abs(lhs - rhs) <= 1e-9 * np.abs(rhs) + 1e-15)


def test_batch_sums_closed_form_at_b1():
    """P-11: with one sample, dW = bf16(d_emb (x) a) (one fp32 product each)
    and db = bf16(d_emb)."""
    inp = _small_inputs(1, 33, seed=15)
    f = adaln.forward(inp)
    b = adaln.backward(inp, f)
    de = b["d_emb"][0]
    a = f["a"][0]
    assert np.array_equal(b["dW_bits"], f32_to_bf16_bits(de[:, None] * a[None, :]))
    assert np.array_equal(b["db_bits"], f32_to_bf16_bits(de))


def _fd_inputs(seed=16, B=2, S=3, Dd=8):
    rng = np.random.default_rng(seed)
    return {"x_val": rng.standard_normal((B, S, Dd)), "temb_val": rng.standard_normal((B, Dd)),
            "W_val": rng.standard_normal((2 * Dd, Dd)) * 0.3, "bias_val": rng.standard_normal(2 * Dd) * 0.2,
            "g_val": rng.standard_normal((B, S, Dd))}


def _fd_check(inp, tol=1e-6):
    f = adaln.forward(inp, "exact")
    b = adaln.backward(inp, f, "exact")
    G = inp["g_val"]
    grads = {"x_val": b["dx"], "temb_val": b["dtemb"], "W_val": b["dW"], "bias_val": b["db"]}
    worst = 0.0
    for key, ana in grads.items():
        base = inp[key]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            h = 1e-6 * max(1.0, abs(base[idx]))
            for sgn in (1, -1):
                p = dict(inp)
                arr = base.copy()
                arr[idx] += sgn * h
                p[key] = arr
                L = float((adaln.forward(p, "exact")["out"] * G).sum())
                fd[idx] += sgn * L / (2 * h)
        scale = max(np.abs(fd).max(), 1e-12)
        worst = max(worst, float(np.abs(fd - ana).max() / scale))
    return worst <= tol, worst


def test_finite_differences_all_gradients():
    """P-12: every gradient (dx, dtemb, dW, db) against central differences of
    L = sum(out * g) with the rounding points disabled."""
    ok, worst = _fd_check(_fd_inputs())
    assert ok, worst


def test_sgld_semantics_negative_control():
    """P-13: rounding the LayerNorm output to bf16 and modulating in bf16 (the
    semantics miles_diffusion pull request 108 found on the rollout side)
    differs from the autocast rounding points at relative size ~1e-3."""
    inp = _small_inputs(1, 64, seed=17)
    f = adaln.forward(inp)
    bad = adaln.sgld_forward_out(inp, f)
    ours = bits_to_f32(f["out_bits"]).astype(np.float64)
    rel = np.abs(bad - ours) / np.maximum(np.abs(ours), 1e-3)
    assert (bf16_ulp_diff(f32_to_bf16_bits(bad), f["out_bits"]) > 0).mean() > 0.2
    assert 2e-4 < rel.mean() < 1e-2


def test_twin_and_oracle_agree():
    """The fp32 oracle and the fp64 twin agree to 1 bf16 ulp except at outputs
    that cancel to near zero (where the fp32 rounding points decide)."""
    inp = _small_inputs(1, 64, seed=18)
    f = adaln.forward(inp)
    b = adaln.backward(inp, f)
    f6 = adaln.forward(inp, "fp64")
    b6 = adaln.backward(inp, f6, "fp64")
    for k, o, t in [("emb", f, f6), ("out", f, f6), ("dx", b, b6), ("dtemb", b, b6), ("dW", b, b6), ("db", b, b6)]:
        d = bf16_ulp_diff(o[k + "_bits"], t[k + "_bits"])
        assert (d > 1).mean() < 2e-3, k


# ------------------------------------------------------------ fp32 storage --
def _fp32_identity_case():
    inp = _small_inputs(2, 40, seed=31, outlier_frac=0.05, io="fp32")
    inp["W"] = np.concatenate([np.eye(D, dtype=np.float32), np.zeros((D, D), np.float32)])
    inp["bias"] = np.zeros(2 * D, np.float32)
    return inp


def _fp32_storage_checks(inp):
    """The facts P-16 checks, as booleans (the teeth test reuses them)."""
    f = adaln.forward(inp)
    ok = {}
    # identity projection: emb = (a | 0) exactly, a kept in fp32 (most values
    # are not bf16-representable)
    ok["emb_identity"] = (np.array_equal(f["emb"][:, :D], f["a"]) and np.all(f["emb"][:, D:] == 0))
    a_bf = bits_to_f32(f32_to_bf16_bits(f["a"]))
    ok["a_fp32"] = (a_bf != f["a"]).mean() > 0.9
    # W = 0, b = 0: out = LayerNorm(x) in fp32 against a float64 two-pass LayerNorm
    w0 = dict(inp, W=np.zeros_like(inp["W"]), bias=np.zeros_like(inp["bias"]))
    f0 = adaln.forward(w0)
    tb = _textbook_ln(inp["x"])
    ok["layernorm"] = bool(np.all(np.abs(f0["out"] - tb) <= 4e-7 * np.abs(tb) + 1e-7))
    # scale = 2^-12: 1 + scale stays in fp32 (a bf16 rounding would give m = 1)
    sh = np.random.default_rng(32).standard_normal(D).astype(np.float32)
    w1 = dict(w0, bias=np.concatenate([np.full(D, 2.0 ** -12, np.float32), sh]))
    f1 = adaln.forward(w1)
    ok["m_fp32"] = bool(np.all(f1["m"] == np.float32(1 + 2.0 ** -12)))
    # scale = -1: m = 0 and out = shift exactly
    w2 = dict(w0, bias=np.concatenate([np.full(D, -1.0, np.float32), sh]))
    f2 = adaln.forward(w2)
    ok["out_shift"] = bool(np.all(f2["m"] == 0) and np.array_equal(f2["out"], np.broadcast_to(sh, f2["out"].shape)))
    return ok


def test_fp32_storage_closed_forms():
    """P-16: fp32 storage.  W = [I; 0], b = 0 gives emb = (a | 0) exactly with a
    kept in fp32; W = 0, b = 0 gives out = LayerNorm(x) against a float64
    two-pass LayerNorm; 1 + scale is kept in fp32 (scale = 2^-12); scale = -1
    gives out = shift exactly."""
    ok = _fp32_storage_checks(_fp32_identity_case())
    assert all(ok.values()), ok


def test_fp32_storage_batch_sums_at_b1_s1():
    """P-17: fp32 storage, one sample of one token: d_shift = g and d_scale =
    g * n (one fp32 product), dW = d_emb * a (one fp32 product), db = d_emb,
    bit for bit."""
    inp = _small_inputs(1, 1, seed=33, io="fp32")
    f = adaln.forward(inp)
    b = adaln.backward(inp, f)
    g = inp["g"][:, 0, :]
    assert b["d_shift"].tobytes() == g.tobytes()
    assert b["d_scale"].tobytes() == (g * f["n"][:, 0, :]).astype(np.float32).tobytes()
    de, a = b["d_emb"][0], f["a"][0]
    assert b["dW"].tobytes() == (de[:, None] * a[None, :]).astype(np.float32).tobytes()
    assert b["db"].tobytes() == de.tobytes()


def test_projection_backward_fp32_operands_exact_rationals():
    """P-15b: da and dW with fp32 a and W (24-bit significands, products of up
    to 48 bits) against exact rational sums rounded once to fp32."""
    d, a, W, temb = _proj_bwd_cancelling_case(seed=34)
    rng = np.random.default_rng(35)
    a = (a * (1 + rng.random(a.shape) * 2.0 ** -9)).astype(np.float32)
    a[1] = -a[0]
    W = (W * (1 + rng.random(W.shape) * 2.0 ** -9)).astype(np.float32)
    W[1] = -W[0]
    r = adaln.proj_backward(d, a, W, temb, adaln.Arith("fp32", io="fp32"))
    dW_ex, da_ex = _exact_proj_bwd(d, a, W)
    assert np.array_equal(r["dW"].view(np.uint32), dW_ex.view(np.uint32))
    assert np.array_equal(r["da"].view(np.uint32), da_ex.view(np.uint32))


def test_teeth_bf16_rounding_in_fp32_storage_caught(monkeypatch):
    """A bf16 storage rounding left in the fp32 storage mode fails P-16."""
    monkeypatch.setattr(adaln.Arith, "store", lambda self, v: self.bf16(v))
    ok = _fp32_storage_checks(_fp32_identity_case())
    assert not all(ok.values())


# ---------------------------------------------------- residual norm site --
def test_residual_update_closed_forms():
    """P-18: gate = 0 gives h = residual; residual = 0 with gate = 1 gives h = x
    (bit for bit: the product and the add are exact there)."""
    inp = make_residual_inputs(2, 9, seed=51, D=D)
    Dd = D
    mod = bits_to_f32(inp["mod"]).copy()
    mod[:, 2 * Dd:] = 0.0
    f = residual.residual_forward(dict(inp, mod=f32_to_bf16_bits(mod)))
    assert np.array_equal(f["h_bits"], inp["residual"])
    mod[:, 2 * Dd:] = 1.0
    f = residual.residual_forward(dict(inp, mod=f32_to_bf16_bits(mod), residual=np.zeros_like(inp["residual"])))
    assert np.array_equal(f["h_bits"], inp["x"])


def test_residual_site_reduces_to_norm_out():
    """P-19: with one sample, the site's out, and with g_h = 0 its dh, d_scale and
    d_shift, are those of the (separately pinned) norm_out operator applied to
    h with emb = (scale | shift)."""
    rinp = make_residual_inputs(1, 21, seed=52, D=D)
    rinp["g_h"] = np.zeros_like(rinp["g_h"])
    f = residual.residual_forward(rinp)
    b = residual.residual_backward(rinp, f)
    mod = rinp["mod"][0]
    ninp = {"x": f["h_bits"], "temb": np.zeros((1, D), np.uint16), "W": np.zeros((2 * D, D), np.uint16),
            "bias": np.concatenate([mod[D:2 * D], mod[:D]]), "g": rinp["g_out"]}
    nf = adaln.forward(ninp)
    nb = adaln.backward(ninp, nf)
    assert np.array_equal(nf["emb_bits"][0], ninp["bias"])
    assert np.array_equal(f["out_bits"], nf["out_bits"])
    assert np.array_equal(b["dh_bits"], nb["dx_bits"])
    assert b["d_scale"].tobytes() == nb["d_scale"].tobytes()
    assert b["d_shift"].tobytes() == nb["d_shift"].tobytes()


def test_residual_site_gradient_closed_forms():
    """P-20: g_out = 0 gives dh = g_h and dx = bf16(g_h * gate) bit for bit, and
    with one token d_gate = g_h * x (one exact product), d_scale = d_shift = 0."""
    rinp = make_residual_inputs(2, 1, seed=53, D=D)
    rinp["g_out"] = np.zeros_like(rinp["g_out"])
    f = residual.residual_forward(rinp)
    b = residual.residual_backward(rinp, f)
    gh = bits_to_f32(rinp["g_h"])
    gate = bits_to_f32(rinp["mod"])[:, 2 * D:]
    assert np.array_equal(b["dh_bits"], rinp["g_h"])
    assert np.array_equal(b["dx_bits"], f32_to_bf16_bits(gh * gate[:, None, :]))
    xs = bits_to_f32(rinp["x"])
    assert b["d_gate"].tobytes() == (gh[:, 0, :] * xs[:, 0, :]).astype(np.float32).tobytes()
    assert np.all(b["d_scale"] == 0) and np.all(b["d_shift"] == 0)


def _residual_fd(seed=54, B=2, S=3, Dd=8, drop_gh=False):
    rng = np.random.default_rng(seed)
    inp = {"x_val": rng.standard_normal((B, S, Dd)), "residual_val": rng.standard_normal((B, S, Dd)),
           "mod_val": rng.standard_normal((B, 3 * Dd)) * 0.5, "g_out_val": rng.standard_normal((B, S, Dd)),
           "g_h_val": rng.standard_normal((B, S, Dd))}
    f = residual.residual_forward(inp, "exact")
    if drop_gh:
        inp_b = dict(inp, g_h_val=np.zeros_like(inp["g_h_val"]))
    else:
        inp_b = inp
    b = residual.residual_backward(inp_b, f, "exact")
    G, Gh = inp["g_out_val"], inp["g_h_val"]
    grads = {"x_val": b["dx"], "residual_val": b["d_residual"], "mod_val": b["d_mod"]}
    worst = 0.0
    for key, ana in grads.items():
        base = inp[key]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            hstep = 1e-6 * max(1.0, abs(base[idx]))
            for sgn in (1, -1):
                arr = base.copy()
                arr[idx] += sgn * hstep
                ff = residual.residual_forward(dict(inp, **{key: arr}), "exact")
                L = float((ff["out"] * G).sum() + (ff["h"] * Gh).sum())
                fd[idx] += sgn * L / (2 * hstep)
        sc = max(np.abs(fd).max(), 1e-12)
        worst = max(worst, float(np.abs(fd - ana).max() / sc))
    return worst


def test_residual_site_finite_differences():
    """P-21: dx, d_residual and d_mod = (d_shift | d_scale | d_gate) against
    central differences of L = sum(out * g_out) + sum(h * g_h), rounding points
    disabled."""
    assert _residual_fd() <= 1e-6


def test_teeth_residual_gradient_dropped_caught():
    """Leaving g_h out of dh fails P-21."""
    assert _residual_fd(drop_gh=True) > 1e-3


# ------------------------------------------------ 6-way modulation projection --
def test_mod6_projection_float64_and_chunks():
    """P-22: the 6-way projection (W6 [6K, K]) against numpy's float64 matmul;
    W6 = six scaled identities c_q I with b6 = 0 puts c_q * a in chunk q
    exactly, and site_chunks(., 2) returns chunks 3, 4, 5 as shift, scale, gate."""
    K = 64
    inp = make_mod6_inputs(3, seed=40, K=K)
    f = modulation.mod6_forward(inp)
    a = f["a"].astype(np.float64)
    W = bits_to_f32(inp["W"]).astype(np.float64)
    bias = bits_to_f32(inp["bias"]).astype(np.float64)
    d = bf16_ulp_diff(f["emb_bits"], fpmath.f64_to_bf16_bits(a @ W.T + bias))
    assert d.max() <= 1 and (d == 0).mean() > 0.99
    c = np.array([1.0, 2.0, -1.0, 0.5, 4.0, -2.0], np.float32)
    inp["W"] = f32_to_bf16_bits(np.concatenate([ci * np.eye(K, dtype=np.float32) for ci in c]))
    inp["bias"] = np.zeros_like(inp["bias"])
    f2 = modulation.mod6_forward(inp)
    av = f2["a"].astype(np.float32)
    for q in range(6):
        assert np.array_equal(f2["emb_bits"][:, q * K:(q + 1) * K], f32_to_bf16_bits(c[q] * av))
    ch = modulation.site_chunks(bits_to_f32(f2["emb_bits"]), 2)
    for name, q in (("shift", 3), ("scale", 4), ("gate", 5)):
        assert np.array_equal(ch[name], c[q] * av)


def _mod6_fd():
    """Largest relative error of dW6, db6 and dtemb against central differences
    of L = sum(emb6 * G), rounding points disabled (exact mode)."""
    rng = np.random.default_rng(41)
    B, K = 2, 4
    inp = {"temb_val": rng.standard_normal((B, K)), "W_val": rng.standard_normal((6 * K, K)) * 0.4,
           "bias_val": rng.standard_normal(6 * K) * 0.2}
    G = rng.standard_normal((B, 6 * K))
    f = modulation.mod6_forward(inp, "exact")
    b = modulation.mod6_backward(dict(inp, d_emb=G.astype(np.float32)), f, "exact")
    G = G.astype(np.float32).astype(np.float64)
    worst = 0.0
    for key, ana in (("W_val", b["dW"]), ("bias_val", b["db"]), ("temb_val", b["dtemb"])):
        base = inp[key]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            h = 1e-6 * max(1.0, abs(base[idx]))
            for sgn in (1, -1):
                arr = base.copy()
                arr[idx] += sgn * h
                L = float((modulation.mod6_forward(dict(inp, **{key: arr}), "exact")["emb"] * G).sum())
                fd[idx] += sgn * L / (2 * h)
        worst = max(worst, float(np.abs(fd - ana).max() / max(np.abs(fd).max(), 1e-12)))
    return worst


def test_mod6_backward_closed_forms_and_finite_differences():
    """P-23: one sample: dW6 = bf16(d_emb (x) a) (one fp32 product each), db6 =
    bf16(d_emb); every gradient against central differences."""
    inp = make_mod6_inputs(1, seed=42, K=32)
    f = modulation.mod6_forward(inp)
    b = modulation.mod6_backward(inp, f)
    de, a = inp["d_emb"][0], f["a"][0].astype(np.float32)
    assert np.array_equal(b["dW_bits"], f32_to_bf16_bits(de[:, None] * a[None, :]))
    assert np.array_equal(b["db_bits"], f32_to_bf16_bits(de))
    assert _mod6_fd() <= 1e-6


def test_teeth_mod6_second_site_dropped_caught(monkeypatch):
    """A backward that takes only the first site's half of d_emb (chunks 0..2)
    fails P-23."""
    orig = modulation.proj_backward

    def first_half(d_emb, a, W, temb, ar, want_abs=False):
        d = np.array(d_emb, copy=True)
        d[:, d.shape[1] // 2:] = 0
        return orig(d, a, W, temb, ar, want_abs)

    monkeypatch.setattr(modulation, "proj_backward", first_half)
    assert _mod6_fd() > 1e-3


# ----------------------------------------------------------------- proj_out --
def _proj_out_inputs(T, seed, K=D, O=64):
    rng = np.random.default_rng(seed)
    return {"out": f32_to_bf16_bits(rng.standard_normal((T, K), dtype=np.float32)),
            "W": f32_to_bf16_bits(rng.standard_normal((O, K), dtype=np.float32) * np.float32(0.02)),
            "bias": f32_to_bf16_bits(rng.standard_normal(O, dtype=np.float32) * np.float32(0.01)),
            "d_lat": f32_to_bf16_bits(rng.standard_normal((T, O), dtype=np.float32))}


def test_proj_out_float64_and_identity():
    """P-24: latent = bf16(out Wp^T + bp) against numpy's float64 matmul; Wp =
    [I | 0] with bp = 0 gives latent = out[:, :64] exactly."""
    inp = _proj_out_inputs(5, seed=60)
    f = proj_out.proj_out_forward(inp)
    x = bits_to_f32(inp["out"]).astype(np.float64)
    W = bits_to_f32(inp["W"]).astype(np.float64)
    b = bits_to_f32(inp["bias"]).astype(np.float64)
    d = bf16_ulp_diff(f["latent_bits"], fpmath.f64_to_bf16_bits(x @ W.T + b))
    assert d.max() <= 1 and (d == 0).mean() > 0.99
    inp["W"] = f32_to_bf16_bits(np.eye(64, D, dtype=np.float32))
    inp["bias"] = np.zeros_like(inp["bias"])
    assert np.array_equal(proj_out.proj_out_forward(inp)["latent_bits"], inp["out"][:, :64])


def _proj_out_fd():
    """Largest relative error of d_out, dWp and dbp against central differences
    of L = sum(latent * G), rounding points disabled (exact mode)."""
    rng = np.random.default_rng(61)
    T, K, O = 3, 5, 4
    inp = {"out_val": rng.standard_normal((T, K)), "W_val": rng.standard_normal((O, K)) * 0.4,
           "bias_val": rng.standard_normal(O) * 0.2, "d_lat_val": rng.standard_normal((T, O))}
    b = proj_out.proj_out_backward(inp, "exact")
    G = inp["d_lat_val"]
    worst = 0.0
    for key, ana in (("out_val", b["d_out"]), ("W_val", b["dW"]), ("bias_val", b["db"])):
        base = inp[key]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            h = 1e-6 * max(1.0, abs(base[idx]))
            for sgn in (1, -1):
                arr = base.copy()
                arr[idx] += sgn * h
                L = float((proj_out.proj_out_forward(dict(inp, **{key: arr}), "exact")["latent"] * G).sum())
                fd[idx] += sgn * L / (2 * h)
        worst = max(worst, float(np.abs(fd - ana).max() / max(np.abs(fd).max(), 1e-12)))
    return worst


def test_proj_out_backward_closed_forms_and_finite_differences():
    """P-25: one token: dWp = bf16(d_lat (x) out) (an exact product, one
    rounding), dbp = d_lat; d_out of Wp = [I | 0] is d_lat in the first 64
    columns and 0 elsewhere; every gradient against central differences."""
    inp = _proj_out_inputs(1, seed=62)
    b = proj_out.proj_out_backward(inp)
    dl, x = bits_to_f32(inp["d_lat"])[0], bits_to_f32(inp["out"])[0]
    assert np.array_equal(b["dW_bits"], f32_to_bf16_bits(dl[:, None] * x[None, :]))
    assert np.array_equal(b["db_bits"], inp["d_lat"][0])
    inp["W"] = f32_to_bf16_bits(np.eye(64, D, dtype=np.float32))
    b = proj_out.proj_out_backward(inp)
    assert np.array_equal(b["d_out_bits"][:, :64], inp["d_lat"])
    assert np.all(bits_to_f32(b["d_out_bits"][:, 64:]) == 0)
    assert _proj_out_fd() <= 1e-6


def test_teeth_proj_out_token_mixup_caught(monkeypatch):
    """A backward whose d_out rows land on the wrong tokens (a token index
    mix-up, here reversed) fails P-25's finite differences."""
    orig = proj_out.proj_out_backward

    def wrong(inp, mode="fp32", want_abs=False):
        r = orig(inp, mode, want_abs)
        return dict(r, d_out=r["d_out"][::-1].copy())

    monkeypatch.setattr(proj_out, "proj_out_backward", wrong)
    assert _proj_out_fd() > 1e-3


# ------------------------------------------------------------ planted mistakes --
def test_teeth_swapped_chunks_caught(monkeypatch):
    orig = adaln.projection

    def swapped(a, W, bias, ar, want_abs=False):
        e = orig(a, W, bias, ar, want_abs)
        Dd = e.shape[1] // 2
        return np.concatenate([e[:, Dd:], e[:, :Dd]], axis=1)

    monkeypatch.setattr(adaln, "projection", swapped)
    inp = _small_inputs(1, 16, seed=11)
    c1, c2 = 0.5, 0.25
    inp["W"] = np.zeros_like(inp["W"])
    inp["bias"] = np.concatenate([f32_to_bf16_bits(np.full(D, c1, np.float32)),
                                  f32_to_bf16_bits(np.full(D, c2, np.float32))])
    assert not _order_check(adaln.forward(inp), inp, c1, c2)


def test_teeth_logistic_derivative_caught(monkeypatch):
    """The derivative of the logistic in place of silu' fails the FD pin."""
    monkeypatch.setattr(adaln, "_dsilu64", lambda z: (1 / (1 + np.exp(-z))) * (1 - 1 / (1 + np.exp(-z))))
    ok, worst = _fd_check(_fd_inputs())
    assert not ok


def test_teeth_dropped_beta_term_caught(monkeypatch):
    """Dropping the n*beta term of the LayerNorm backward fails the FD pin."""
    orig_bwd = adaln.backward

    def bwd(inp, fwd, mode="fp32", want_abs=False, g=None):
        r = orig_bwd(inp, fwd, mode, want_abs, g)
        gy = inp["g_val"] * fwd["m"][:, None, :]
        alpha = gy.mean(-1, keepdims=True)
        r["dx"] = fwd["rstd"][..., None] * (gy - alpha)
        return r

    monkeypatch.setattr(adaln, "backward", bwd)
    ok, worst = _fd_check(_fd_inputs())
    assert not ok


def test_sampled_evaluation_matches_full_oracle():
    """The sampled helpers (used where the full oracle would be too slow) give
    the same bytes as the full backward on a small batch."""
    inp = _small_inputs(3, 40, seed=19)
    f = adaln.forward(inp)
    b = adaln.backward(inp, f)
    mean, rstd = adaln.ln_stats(inp)
    assert mean.tobytes() == f["mean"].tobytes() and rstd.tobytes() == f["rstd"].tobytes()
    cols = np.array([0, 5, 3071, 3072, 4000, 6143])
    assert adaln.d_emb_columns(inp, cols).tobytes() == b["d_emb"][:, cols].tobytes()
    dW, db, _ = adaln.param_grads_rows(inp, cols)
    assert np.array_equal(dW, b["dW_bits"][cols]) and np.array_equal(db, b["db_bits"][cols])
