"""Pins for the CPU oracle: closed forms, invariants, printed values, brute force.

Each test checks the oracle against something other than itself, chosen so a
plausible mistake (a dropped term, a wrong sign or index, a transposed
operand, a wrong head mapping, an off-by-one in the cache) fails one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import synth
from oracle import oracle as O
from oracle.brute import brute_forward

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small(seed=0, **kw):
    shape = synth.small_shape(**kw)
    return shape, synth.make_weights(shape, seed)


# ---------------------------------------------------------------- P-a RMSNorm
def test_rmsnorm_constant_vector():
    g = np.linspace(0.5, 1.5, 16)
    for c in (3.0, -0.25, 1e-4):
        x = np.full(16, c)
        eps = 1e-6
        want = c / math.sqrt(c * c + eps) * g
        np.testing.assert_allclose(O.rms_norm(x, g, eps), want, rtol=1e-13, atol=0)
    np.testing.assert_array_equal(O.rms_norm(np.zeros(16), g, 1e-6), np.zeros(16))


def test_rmsnorm_scale_invariance_and_unit_rms():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(64)
    ones = np.ones(64)
    y = O.rms_norm(x, ones, 0.0)
    assert abs(np.sqrt(np.mean(y * y)) - 1.0) < 1e-12           # unit RMS
    np.testing.assert_allclose(O.rms_norm(7.0 * x, ones, 0.0), y, rtol=1e-12)
    # along the last axis only: rows are normalised independently
    m = np.stack([x, 2 * x + 1])
    np.testing.assert_allclose(O.rms_norm(m, ones, 0.0)[1], O.rms_norm(2 * x + 1, ones, 0.0), rtol=1e-13)


# ---------------------------------------------------------------- P-b RoPE
def test_rope_identity_at_zero_and_norm_preserving():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 3, 16))
    np.testing.assert_array_equal(O.rope(x, np.zeros(5, int), 1e6), x)
    y = O.rope(x, np.array([0, 1, 7, 100, 4000]), 1e6)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)


def test_rope_known_rotation():
    # d=2: the single pair has frequency theta^0 = 1, so unit vector e0 at
    # position p maps to (cos p, sin p) and e1 to (-sin p, cos p).
    for p in (1, 2, 5):
        e0 = np.array([[[1.0, 0.0]]])
        e1 = np.array([[[0.0, 1.0]]])
        np.testing.assert_allclose(O.rope(e0, np.array([p]), 10.0)[0, 0], [math.cos(p), math.sin(p)], atol=1e-15)
        np.testing.assert_allclose(O.rope(e1, np.array([p]), 10.0)[0, 0], [-math.sin(p), math.cos(p)], atol=1e-15)
    # d=4, theta=100: pair 0 = (x0, x2) at freq 1, pair 1 = (x1, x3) at freq 100^(-1/2) = 0.1
    x = np.array([[[0.0, 1.0, 0.0, 0.0]]])
    y = O.rope(x, np.array([3]), 100.0)[0, 0]
    np.testing.assert_allclose(y, [0.0, math.cos(0.3), 0.0, math.sin(0.3)], atol=1e-15)


def test_rope_relative_position():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, 32))
    k = rng.standard_normal((1, 1, 32))

    def dot(m, n):
        return float(np.sum(O.rope(q, np.array([m]), 1e4) * O.rope(k, np.array([n]), 1e4)))

    base = dot(10, 3)
    for m, n in ((7, 0), (107, 100), (2007, 2000)):
        assert abs(dot(m, n) - base) < 1e-9
    assert abs(dot(11, 3) - base) > 1e-6


# ---------------------------------------------------------------- P-l silu/softmax
def test_silu_softmax_closed_forms():
    assert O.silu(np.array(0.0)) == 0.0
    assert abs(float(O.silu(np.array(1.0))) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert abs(float(O.silu(np.array(40.0))) - 40.0) < 1e-12
    assert abs(float(O.silu(np.array(-40.0)))) < 1e-15
    rng = np.random.default_rng(4)
    s = rng.standard_normal((6, 9)) * 30
    s[:, 5:] = -np.inf
    p = O.softmax_rows(s)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=1e-14)
    assert np.all(p[:, 5:] == 0)
    # softmax of equal scores is uniform
    np.testing.assert_allclose(O.softmax_rows(np.zeros((1, 4))), 0.25)


# ---------------------------------------------------------------- P-c one token
def test_attention_single_key_returns_v():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 4, 8))
    k = rng.standard_normal((1, 2, 8))
    v = rng.standard_normal((1, 2, 8))
    out = O.gqa_attention(q, k, v, np.array([0]))
    for h in range(4):
        np.testing.assert_allclose(out[0, h], v[0, h // 2], rtol=1e-15)


def test_model_single_token_attention_is_v():
    shape, w = small(6)
    orc = O.Oracle(shape, w)
    dump = {}
    orc.forward([17], dump=dump)
    for li in range(shape.n_layers):
        a = dump[f"layer{li}.attn"].reshape(shape.n_heads, shape.head_dim)
        v = dump[f"layer{li}.v"][0]
        for h in range(shape.n_heads):
            np.testing.assert_allclose(a[h], v[h // (shape.n_heads // shape.n_kv_heads)], rtol=1e-13)


# ---------------------------------------------------------------- P-d GQA = MHA
def test_gqa_equals_mha_with_repeated_kv():
    shape, w = small(7)
    rep = shape.n_heads // shape.n_kv_heads
    d = shape.head_dim
    mha_shape = synth.small_shape(n_kv_heads=shape.n_heads)
    w2 = {"embed": w["embed"], "final_norm": w["final_norm"], "layers": []}
    for lw in w["layers"]:
        lw2 = dict(lw)
        for key in ("wk", "wv"):
            heads = lw[key].reshape(shape.n_kv_heads, d, shape.hidden)
            lw2[key] = np.repeat(heads, rep, axis=0).reshape(shape.n_heads * d, shape.hidden)
        w2["layers"].append(lw2)
    ids = [3, 9, 27, 1, 60, 44]
    a = O.Oracle(shape, w).forward(ids)
    b = O.Oracle(mha_shape, w2).forward(ids)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
    # a wrong mapping (h % nkv instead of h // rep) must differ
    w3 = {"embed": w["embed"], "final_norm": w["final_norm"], "layers": []}
    for lw in w["layers"]:
        lw3 = dict(lw)
        for key in ("wk", "wv"):
            heads = lw[key].reshape(shape.n_kv_heads, d, shape.hidden)
            lw3[key] = np.tile(heads, (rep, 1, 1)).reshape(shape.n_heads * d, shape.hidden)
        w3["layers"].append(lw3)
    c = O.Oracle(mha_shape, w3).forward(ids)
    assert np.max(np.abs(a - c)) > 1e-6


# ---------------------------------------------------------------- P-e cached = uncached
@pytest.mark.parametrize("dtype,tol", [(np.float64, 1e-12), (np.float32, 2e-5)])
def test_cached_equals_uncached(dtype, tol):
    shape, w = small(8)
    ids = np.array([5, 1, 63, 22, 8, 40, 40, 2, 19])
    orc = O.Oracle(shape, w, dtype=dtype)
    got = [orc.prefill(0, ids[:3])]
    for p in range(3, len(ids)):
        got.append(orc.decode_step(0, int(ids[p]), p))
    ref = O.Oracle(shape, w, dtype=dtype)
    for i, g in enumerate(got):
        want = ref.forward(ids[: 3 + i])
        scale = np.max(np.abs(want))
        assert np.max(np.abs(g - want)) <= tol * scale
    with pytest.raises(ValueError):
        orc.decode_step(0, 1, 3)              # position must equal the cached length


def test_cached_slots_are_independent():
    shape, w = small(9)
    orc = O.Oracle(shape, w)
    orc.prefill(0, [1, 2, 3])
    orc.prefill(1, [9, 8])
    a = orc.decode_step(1, 7, 2)
    ref = O.Oracle(shape, w)
    np.testing.assert_allclose(a, ref.forward([9, 8, 7]), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- P-f brute force
def test_brute_force_small():
    shape, w = small(10)
    ids = [4, 17, 33, 4, 60]
    want = np.array(brute_forward(shape, w, ids, all_rows=True))
    got = O.Oracle(shape, w).forward(ids, all_rows=True)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_brute_force_tiny_shape_head64():
    shape = synth.TINY
    w = synth.cached_weights(shape)
    ids = [7, 4095]
    want = np.array(brute_forward(shape, w, ids))
    got = O.Oracle(shape, w).forward(ids)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- P-g causality
def test_causality():
    shape, w = small(11)
    ids = np.array([1, 2, 3, 4, 5, 6, 7])
    orc = O.Oracle(shape, w)
    a = orc.forward(ids, all_rows=True)
    ids2 = ids.copy()
    ids2[4] = 50
    b = orc.forward(ids2, all_rows=True)
    np.testing.assert_array_equal(a[:4], b[:4])
    assert np.max(np.abs(a[4:] - b[4:])) > 1e-6


# ---------------------------------------------------------------- P-h printed values
def test_printed_shape_and_param_count():
    with open(os.path.join(GOLDEN, "qwen3_0p6b_shape.json")) as f:
        g = json.load(f)
    s = synth.QWEN3_0P6B
    assert (s.vocab, s.hidden, s.n_layers, s.n_heads, s.n_kv_heads, s.head_dim, s.ffn) == (
        g["vocab"], g["hidden"], g["n_layers"], g["n_heads"], g["n_kv_heads"], g["head_dim"], g["ffn"])
    assert s.q_width == g["q_width"] and s.q_width != s.hidden
    n = O.param_count(s)
    assert n == 596_049_920
    assert round(n / 1e6) == g["printed_logical_params_millions"]
    # 11 tensors per layer + embed + final norm = 310; the printed 311 has one more
    # stored tensor (read as a stored copy of the tied head), see the design notes.
    assert O.tensor_count(s) == g["printed_tensors"] - 1
    assert O.param_count(synth.TINY) == 2_622_976


# ---------------------------------------------------------------- P-i argmax rule
def test_argmax_rule_cases():
    with open(os.path.join(GOLDEN, "argmax_rule.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        row = np.array([float(v) for v in c["row"]], dtype=np.float32)
        assert O.greedy_argmax(row) == c["expect"], c
        assert O.greedy_argmax_fast(row) == c["expect"], c


def test_top_k_order():
    row = np.array([0.5, 3.0, 3.0, -1.0, np.nan, 2.0, np.inf])
    np.testing.assert_array_equal(O.top_k(row, 4), [1, 2, 5, 0])


# ---------------------------------------------------------------- P-j Wq = 0
def test_zero_query_gives_running_mean_of_v():
    shape, w = small(12)
    w["layers"][0]["wq"] = np.zeros_like(w["layers"][0]["wq"])
    ids = np.array([3, 14, 15, 9, 26, 53])
    dump = {}
    O.Oracle(shape, w).forward(ids, dump=dump)
    # layer-0 V computed here directly from the embedding
    x = w["embed"][ids].astype(np.float64)
    g = w["layers"][0]["attn_norm"].astype(np.float64)
    xn = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + shape.rms_eps) * g
    v = (xn @ w["layers"][0]["wv"].astype(np.float64).T).reshape(len(ids), shape.n_kv_heads, shape.head_dim)
    running = np.cumsum(v, axis=0) / np.arange(1, len(ids) + 1)[:, None, None]
    a = dump["layer0.attn"].reshape(len(ids), shape.n_heads, shape.head_dim)
    rep = shape.n_heads // shape.n_kv_heads
    for h in range(shape.n_heads):
        np.testing.assert_allclose(a[:, h], running[:, h // rep], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- P-k degenerate models
def test_zero_layer_model_is_plain_matvec():
    shape = synth.small_shape(n_layers=0)
    w = synth.make_weights(shape, 13)
    ids = [5, 6, 7]
    e = w["embed"].astype(np.float64)
    h = e[7] / np.sqrt(np.mean(e[7] ** 2) + shape.rms_eps) * w["final_norm"]
    np.testing.assert_allclose(O.Oracle(shape, w).forward(ids), e @ h, rtol=1e-13, atol=1e-15)


def test_zero_up_projection_adds_nothing():
    shape, w = small(14)
    for lw in w["layers"]:
        lw["w_up"] = np.zeros_like(lw["w_up"])
    dump = {}
    O.Oracle(shape, w).forward([1, 2, 3], dump=dump)
    for li in range(shape.n_layers):
        np.testing.assert_array_equal(dump[f"layer{li}.out"], dump[f"layer{li}.x_mid"])


def test_zero_output_projection_keeps_embedding():
    # Wo = 0 and W_down = 0: every block is the identity on the residual stream.
    shape, w = small(15)
    for lw in w["layers"]:
        lw["wo"] = np.zeros_like(lw["wo"])
        lw["w_down"] = np.zeros_like(lw["w_down"])
    dump = {}
    O.Oracle(shape, w).forward([9, 10], dump=dump)
    np.testing.assert_array_equal(dump["final"], w["embed"][[9, 10]].astype(np.float64))


# ---------------------------------------------------------------- attention scale (1/sqrt(head_dim))
# "Coming back to Failed Star", Second sitting: 16 query heads of width 128
# give 2048, not H, so head_dim is not hidden / n_heads and the two candidate
# scales differ.  Both brute-force shapes above have head_dim = hidden /
# n_heads; these cases do not.
def test_attention_scale_closed_form():
    d = 16
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = 4.0                   # score against k0: 4 / sqrt(16) = 1
    k = np.zeros((2, 1, d))
    k[0, 0, 0] = 1.0                   # k1 = 0: score 0
    v = np.zeros((2, 1, d))
    v[0, 0, 1] = 1.0
    v[1, 0, 2] = 1.0
    out = O.gqa_attention(q, k, v, np.array([1]))
    w0 = math.e / (math.e + 1.0)
    np.testing.assert_allclose(out[0, 0, 1:3], [w0, 1.0 - w0], rtol=1e-14)


def _wide_head_shape():
    # hidden 32, 4 query heads of width 16 (q width 64 = 2 x hidden, as the
    # 0.6B shape's 2048 = 2 x 1024), 2 KV heads
    return synth.small_shape(hidden=32, n_heads=4, n_kv_heads=2, head_dim=16, ffn=48, vocab=64)


def test_brute_force_head_dim_not_hidden_over_heads():
    shape = _wide_head_shape()
    assert shape.head_dim != shape.hidden // shape.n_heads
    w = synth.make_weights(shape, 16)
    ids = [5, 61, 0, 5, 33, 12]
    want = np.array(brute_forward(shape, w, ids, all_rows=True))
    got = O.Oracle(shape, w).forward(ids, all_rows=True)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_wrong_attention_scale_is_caught(monkeypatch):
    # A planted mistake in the oracle (scores scaled by 1/sqrt(hidden/n_heads)
    # instead of 1/sqrt(head_dim)) must fail the brute-force comparison.
    shape = _wide_head_shape()
    w = synth.make_weights(shape, 16)
    ids = [5, 61, 0, 5, 33, 12]
    want = np.array(brute_forward(shape, w, ids, all_rows=True))
    right = O.gqa_attention
    wrong = math.sqrt(shape.head_dim) / math.sqrt(shape.hidden / shape.n_heads)
    monkeypatch.setattr(O, "gqa_attention", lambda q, k, v, pos: right(q * wrong, k, v, pos))
    got = O.Oracle(shape, w).forward(ids, all_rows=True)
    assert np.max(np.abs(got - want)) > 1e-6


# ---------------------------------------------------------------- top2_gap (decides where argmax must match)
def test_top2_gap_closed_forms():
    nan, inf = float("nan"), float("inf")
    cases = [
        ([1.0, 3.0, 2.0], 1.0),
        ([3.0, 1.0, 3.0], 0.0),                 # exact tie: no gap
        ([-3.0, -1.0, -2.5], 1.5),              # all negative
        ([nan, 2.0, inf, 1.0], 1.0),            # +inf and NaN are not finite: excluded
        ([-inf, 0.25, nan, -0.5], 0.75),
        ([nan, 5.0, -inf], inf),                # one finite value: nothing to tie with
        ([nan, nan], inf),
        ([7.0], inf),
    ]
    for row, want in cases:
        got = O.top2_gap(np.array(row, dtype=np.float32))
        assert got == want, (row, got, want)


def test_top2_gap_matches_enumeration():
    rng = np.random.default_rng(17)
    for trial in range(50):
        row = rng.standard_normal(40).astype(np.float32)
        if trial % 3 == 0:
            row[rng.integers(40)] = row.max()           # planted tie at the top
        if trial % 4 == 1:
            row[rng.integers(40, size=3)] = np.nan
        if trial % 5 == 2:
            row[rng.integers(40)] = np.inf
        fin = [float(v) for v in row if math.isfinite(float(v))]
        best = max(fin)
        rest = list(fin)
        rest.remove(best)                                # one copy only: a tie leaves the same value
        want = best - max(rest)
        assert O.top2_gap(row) == pytest.approx(want, abs=0.0)
        assert O.greedy_argmax_fast(row) == O.greedy_argmax(row)
