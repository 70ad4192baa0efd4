"""Pins of the gated-attention variant in the oracle ("ferrite", section
"What it does": GQA with 8 query / 2 KV heads, a gated attention output,
rotate-half RoPE on 64 of 256 head dims, and the q/gate split taken per head).

Each check is a closed form or a relation to a case the base oracle already
pins; none retypes the variant's formulas.
"""
import math

import numpy as np

import synth
from oracle import oracle as O


def test_partial_rope_rotates_only_the_first_dims():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 3, 256))
    pos = np.array([0, 1, 7, 100, 4095])
    y = O.rope(x, pos, 1e6, 64)
    assert np.array_equal(y[..., 64:], x[..., 64:])                      # pass-through, exactly
    assert np.allclose(y[..., :64], O.rope(x[..., :64], pos, 1e6))       # a width-64 head's RoPE
    assert np.allclose(O.rope(x, pos, 1e6, 256), O.rope(x, pos, 1e6))
    # norms preserved and identity at position 0
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1))
    assert np.allclose(y[0], x[0])
    # first pair, position 1: angle 1 rad (theta^0)
    a = x[1, 0, 0] * math.cos(1.0) - x[1, 0, 32] * math.sin(1.0)
    assert np.isclose(y[1, 0, 0], a)


def _small_gated(**kw):
    return synth.small_shape(n_heads=4, n_kv_heads=2, head_dim=16, rope_dim=8, attn_gate=True, **kw)


def test_zero_gate_halves_the_attention_output():
    sh_g = _small_gated()
    sh_u = synth.small_shape(n_heads=4, n_kv_heads=2, head_dim=16, rope_dim=8)
    wg = synth.make_weights(sh_g, 5)
    wu = synth.make_weights(sh_u, 5)
    d = sh_g.head_dim
    for lg, lu in zip(wg["layers"], wu["layers"]):
        q = lu["wq"].reshape(sh_u.n_heads, d, -1)
        inter = np.stack([q, np.zeros_like(q)], axis=1)                  # [h, (q | gate), d, H]
        lg["wq"] = inter.reshape(sh_g.q_proj_width, -1)
        for k in ("wk", "wv", "wo", "w_gate", "w_up", "w_down", "attn_norm", "mlp_norm", "q_norm", "k_norm"):
            lg[k] = lu[k]
    wg["embed"], wg["final_norm"] = wu["embed"], wu["final_norm"]
    ids = synth.tokens(9, sh_g.vocab, 12)
    dg, du = {}, {}
    O.Oracle(sh_g, wg).forward(ids, dump=dg)
    O.Oracle(sh_u, wu).forward(ids, dump=du)
    # layer 0 sees identical inputs: sigmoid(0) = 1/2 exactly
    assert np.allclose(dg["layer0.attn"], 0.5 * du["layer0.attn"], rtol=1e-12, atol=1e-15)


def test_gate_split_is_per_head_interleaved():
    # head 0: zero query rows and zero gate rows.  With q = 0 every key gets
    # the same score, so head 0 outputs the running mean of V over positions
    # 0..s, times sigmoid(0) = 1/2.  A flat split (all queries, then all
    # gates) would read head 0's gate from another head's query rows.
    sh = _small_gated()
    w = synth.make_weights(sh, 6)
    d, H = sh.head_dim, sh.hidden
    lw = w["layers"][0]
    rows = lw["wq"].reshape(sh.n_heads, 2, d, H)
    rows[0] = 0.0
    lw["wq"] = rows.reshape(sh.q_proj_width, H)
    ids = synth.tokens(10, sh.vocab, 9)
    dump = {}
    O.Oracle(sh, w).forward(ids, dump=dump)
    attn = dump["layer0.attn"].reshape(len(ids), sh.n_heads, d)
    v = dump["layer0.v"][:, 0, :]                       # KV head 0 serves query heads 0 and 1
    running_mean = np.cumsum(v, axis=0) / np.arange(1, len(ids) + 1)[:, None]
    assert np.allclose(attn[:, 0, :], 0.5 * running_mean, rtol=1e-10, atol=1e-14)
    # head 1 shares KV head 0 but has a real query: not the running mean
    assert not np.allclose(attn[:, 1, :], 0.5 * running_mean, rtol=1e-3)
