"""Pins for the YaRN rotary encoding and the KV append step of the oracle (CPU only).

The source page ("GPT-OSS on Day 0", section "GPT-OSS on Hopper") names YaRN positional
encoding without a formula. The oracle follows the published method; these tests pin it by
what a rotary encoding must satisfy (a 2-D rotation in closed form, preserved pair norms,
scores that depend only on the distance between positions) and by the limits of YaRN's
frequency ramp and temperature, and pin the cache placement through an index route of
their own.
"""
import math

import numpy as np

import oracle
from workloads import CONFIGS, bf16_bits_to_f32, make_paged_prefill, scaled


def test_unscaled_frequencies_are_geometric():
    f, m = oracle.yarn_frequencies(64, 10000.0, 1.0, 4096, 1.0, 32.0)
    assert m == 1.0
    for i in (0, 1, 17, 31):
        assert math.isclose(f[i], math.exp(-(2 * i / 64) * math.log(10000.0)), rel_tol=1e-14)


def test_two_dimensional_rotation_closed_form():
    f = np.array([1.0])          # one pair, one radian per position
    x = np.array([[[0.6, -1.3]]] * 4)
    pos = np.array([0, 1, 2, 7])
    for m in (1.0, 1.25):
        out = oracle.rotate(x, pos, f, m)
        for t, p in enumerate(pos):
            c, s = math.cos(p), math.sin(p)
            assert math.isclose(out[t, 0, 0], m * (0.6 * c + 1.3 * s), abs_tol=1e-14)
            assert math.isclose(out[t, 0, 1], m * (0.6 * s - 1.3 * c), abs_tol=1e-14)


def test_pairs_keep_their_norm_and_position_zero_is_scaling():
    rng = np.random.default_rng(1)
    f, m = oracle.yarn_frequencies(64, 150000.0, 32.0, 4096, 1.0, 32.0)
    x = rng.standard_normal((5, 3, 64))
    pos = np.array([0, 1, 100, 4096, 131071])
    y = oracle.rotate(x, pos, f, m)
    nx = np.hypot(x[..., :32], x[..., 32:])
    ny = np.hypot(y[..., :32], y[..., 32:])
    np.testing.assert_allclose(ny, m * nx, rtol=1e-12)
    np.testing.assert_allclose(y[0], m * x[0], rtol=0, atol=1e-14)


def test_scores_depend_only_on_the_distance():
    rng = np.random.default_rng(2)
    f, m = oracle.yarn_frequencies(64, 150000.0, 32.0, 4096, 1.0, 32.0)
    q, k = rng.standard_normal((1, 1, 64)), rng.standard_normal((1, 1, 64))
    dot = lambda a, b: float((a * b).sum())
    base = dot(oracle.rotate(q, np.array([50]), f, m), oracle.rotate(k, np.array([20]), f, m))
    for shift in (1, 333, 9000):
        moved = dot(oracle.rotate(q, np.array([50 + shift]), f, m), oracle.rotate(k, np.array([20 + shift]), f, m))
        assert math.isclose(base, moved, rel_tol=1e-9, abs_tol=1e-9)
    # and it does change with the distance
    other = dot(oracle.rotate(q, np.array([51]), f, m), oracle.rotate(k, np.array([20]), f, m))
    assert abs(other - base) > 1e-6


def test_yarn_ramp_limits_and_temperature():
    theta, s, L0, a, b = 150000.0, 32.0, 4096, 1.0, 32.0
    f, m = oracle.yarn_frequencies(64, theta, s, L0, a, b)
    base, _ = oracle.yarn_frequencies(64, theta, 1.0, L0, a, b)
    turns = L0 / (2 * np.pi / base)              # turns over L0, through the wavelength
    fast, slow = turns >= b, turns <= a
    assert fast.any() and slow.any() and (~fast & ~slow).any()
    np.testing.assert_array_equal(f[fast], base[fast])                       # extrapolated: kept
    np.testing.assert_allclose(f[slow], base[slow] / s, rtol=1e-15)          # interpolated: / s
    mid = np.flatnonzero(~fast & ~slow)[0]
    g = (turns[mid] - a) / (b - a)
    assert math.isclose(f[mid], g * base[mid] + (1 - g) * base[mid] / s, rel_tol=1e-13)
    assert math.isclose(m, 0.1 * math.log(32.0) + 1.0, rel_tol=1e-15)
    assert oracle.yarn_frequencies(64, theta, math.e, L0, a, b)[1] == 1.1
    assert oracle.yarn_frequencies(64, theta, 0.5, L0, a, b)[1] == 1.0


def test_append_writes_each_new_token_at_its_page_slot():
    spec = scaled(CONFIGS["chunked_prefill"], batch=3, q_len=(1, 40), ctx_len=(0, 50), hq=8, hkv=2, seed=41)
    inp = make_paged_prefill(spec)
    f64 = lambda x: bf16_bits_to_f32(x).astype(np.float64)
    rng = np.random.default_rng(4)
    T = int(inp["cu_seqlens_q"][-1])
    k_new = rng.standard_normal((T, spec.hkv, 64))
    v_new = rng.standard_normal((T, spec.hkv, 64))
    kc0, vc0 = f64(inp["k_cache"]), f64(inp["v_cache"])
    freqs, m = oracle.yarn_frequencies(64, 150000.0, 32.0, 4096, 1.0, 32.0)
    q_rot, kc, vc = oracle.rope_append(f64(inp["q"]), k_new, v_new, inp["cu_seqlens_q"], inp["kv_lens"],
                                       inp["page_table"], kc0, vc0, freqs, m)
    touched = np.zeros(kc0.shape[:1] + kc0.shape[2:3], dtype=bool)   # [page, slot]
    P = spec.page_size
    for b, L in enumerate(inp["kv_lens"]):
        q0, q1 = int(inp["cu_seqlens_q"][b]), int(inp["cu_seqlens_q"][b + 1])
        for t, row in enumerate(range(q0, q1)):
            p = int(L) - (q1 - q0) + t
            page = int(inp["page_table"][b, p // P])
            touched[page, p % P] = True
            np.testing.assert_array_equal(vc[page, :, p % P], v_new[row])
            np.testing.assert_allclose(kc[page, :, p % P], oracle.rotate(k_new[row:row + 1], np.array([p]), freqs, m)[0],
                                       rtol=0, atol=1e-15)
            np.testing.assert_allclose(q_rot[row], oracle.rotate(f64(inp["q"])[row:row + 1], np.array([p]), freqs, m)[0],
                                       rtol=0, atol=1e-15)
    keep = ~touched
    np.testing.assert_array_equal(np.transpose(kc, (0, 2, 1, 3))[keep], np.transpose(kc0, (0, 2, 1, 3))[keep])
    np.testing.assert_array_equal(np.transpose(vc, (0, 2, 1, 3))[keep], np.transpose(vc0, (0, 2, 1, 3))[keep])


# ---------------------------------------------------------------------------------------
# The ramp's interior: hand-derived values (tests/golden/yarn_ramp.json)
# ---------------------------------------------------------------------------------------
import json  # noqa: E402
import os  # noqa: E402

import pytest  # noqa: E402

YARN_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "yarn_ramp.json")


def _yarn_cases():
    with open(YARN_GOLDEN) as fh:
        data = json.load(fh)
    return [dict(c, params=data["params"]) for c in data["cases"]]


def _ev(expr, **names):
    env = {"log": math.log, "exp": math.exp, "cos": math.cos, "sin": math.sin, "pi": math.pi, **names}
    return float(eval(expr, {"__builtins__": {}}, env))


@pytest.mark.parametrize("case", _yarn_cases(), ids=lambda c: c["name"])
def test_yarn_ramp_interior_hand_derived(case):
    p = case["params"]
    i = case["pair"]
    G = _ev(case["gamma_expr"])
    assert math.isclose(G, case["gamma_approx"], rel_tol=5e-4, abs_tol=5e-5)
    if "r_expr" in case:
        assert math.isclose(_ev(case["r_expr"]), case["r_approx"], rel_tol=5e-4)
    F = _ev(case["freq_expr"], G=G)
    if "freq_approx" in case:
        assert math.isclose(F, case["freq_approx"], rel_tol=5e-4)
    f, m = oracle.yarn_frequencies(p["head_dim"], p["theta"], p["factor"], p["orig_len"], p["alpha"], p["beta"],
                                   ramp=case["ramp"])
    assert math.isclose(f[i], F, rel_tol=1e-12), f"pair {i}: oracle {f[i]!r}, derived {F!r}"
    if "other_ramp_freq_expr" in case:
        # the pin separates the two ramp forms inside the band
        other = _ev(case["other_ramp_freq_expr"], G=G)
        assert abs(other - F) > 0.2 * F
        wrong = "index" if case["ramp"] == "turns" else "turns"
        fw, _ = oracle.yarn_frequencies(p["head_dim"], p["theta"], p["factor"], p["orig_len"], p["alpha"], p["beta"],
                                        ramp=wrong)
        assert abs(fw[i] - F) > 0.2 * F
    if "rotation" in case:
        rot = case["rotation"]
        x = np.zeros((1, 1, p["head_dim"]))
        x[0, 0, i], x[0, 0, i + p["head_dim"] // 2] = rot["x_pair"]
        y = oracle.rotate(x, np.array([rot["position"]]), f, m)
        exp_lo, exp_hi = (_ev(e, F=F) for e in rot["expect_expr"])
        assert math.isclose(y[0, 0, i], exp_lo, rel_tol=1e-9, abs_tol=1e-12)
        assert math.isclose(y[0, 0, i + p["head_dim"] // 2], exp_hi, rel_tol=1e-9, abs_tol=1e-12)
        others = np.delete(y[0, 0], [i, i + p["head_dim"] // 2])
        assert np.all(others == 0.0)


def test_yarn_index_ramp_is_linear_in_the_pair_index():
    """Inside the band the 'index' form's weight falls by the same step from pair to pair, and
    its ends sit where r = beta and r = alpha."""
    theta, s, L0, a, b = 150000.0, 32.0, 4096, 1.0, 32.0
    f, _ = oracle.yarn_frequencies(64, theta, s, L0, a, b, ramp="index")
    base, _ = oracle.yarn_frequencies(64, theta, 1.0, L0, a, b)
    g = (f / base - 1.0 / s) / (1.0 - 1.0 / s)
    inside = np.flatnonzero((g > 0) & (g < 1))
    assert len(inside) >= 5
    steps = np.diff(g[inside])
    np.testing.assert_allclose(steps, steps[0], rtol=1e-9)
    i_beta = 32 * math.log(L0 / (2 * math.pi * b)) / math.log(theta)
    i_alpha = 32 * math.log(L0 / (2 * math.pi * a)) / math.log(theta)
    assert math.isclose(steps[0], -1.0 / (i_alpha - i_beta), rel_tol=1e-9)
    with pytest.raises(ValueError):
        oracle.yarn_frequencies(64, theta, s, L0, a, b, ramp="linear")
