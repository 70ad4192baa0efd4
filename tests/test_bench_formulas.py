"""The algorithmic work `bench.py` divides by, checked against independent counts.

The roofline figures are algorithmic bytes (decode) or flops (prefill) over a
measured time, so a wrong shape term would misstate every fraction.  Each
figure here is recomputed from the model shape by a different route: the
oracle's parameter count (itself pinned to the 596,049,920 of "596M"), the
per-matrix shapes, or the causal-attention closed form.
"""
import numpy as np

import bench
import synth
from oracle import oracle as O

S06 = synth.QWEN3_0P6B


def test_decode_step_bytes_are_the_parameters_plus_the_cache():
    # every parameter once in bf16 (the tied head once), the token's embedding
    # row, and K and V of every layer and KV head for each attended position
    kv_per_pos = S06.n_layers * 2 * S06.n_kv_heads * S06.head_dim * 2
    for ctx in (0, 1, 513, 768, 4096):
        want = 2 * O.param_count(S06) + 2 * S06.hidden + kv_per_pos * ctx
        assert bench.decode_bytes_per_step(S06, ctx) == want
    assert O.param_count(S06) == 596_049_920


def test_decode_launch_bytes_follow_the_matrix_shapes():
    H, d, I, V = S06.hidden, S06.head_dim, S06.ffn, S06.vocab
    qkv_rows = (S06.n_heads + 2 * S06.n_kv_heads) * d
    assert bench.decode_label_bytes(S06, "qkv", 640) == qkv_rows * H * 2 + 4 * H + 4 * qkv_rows
    assert bench.decode_label_bytes(S06, "o_proj", 640) == H * S06.n_heads * d * 2 + 4 * S06.n_heads * d + 8 * H
    assert bench.decode_label_bytes(S06, "gate_up", 640) == 2 * I * H * 2 + 4 * H + 4 * I
    assert bench.decode_label_bytes(S06, "down", 640) == H * I * 2 + 4 * I + 8 * H
    assert bench.decode_label_bytes(S06, "head", 640) == V * H * 2 + 4 * H
    # K and V rows of 640 positions of 8 KV heads, the new row written, q/k/v read
    kv = 2 * S06.n_kv_heads * d * 2
    assert bench.decode_label_bytes(S06, "attn", 640) == kv * 640 + kv + 4 * qkv_rows
    # the per-layer weight bytes add up to the layer's share of the parameters
    per_layer_w = sum(int(np.prod(s)) for k, s in S06.layer_shapes().items() if len(s) == 2) * 2
    got = sum(bench.decode_label_bytes(S06, k, 0) for k in ("qkv", "o_proj", "gate_up", "down"))
    acts = (4 * H + 4 * qkv_rows) + (4 * S06.n_heads * d + 8 * H) + (4 * H + 4 * I) + (4 * I + 8 * H)
    assert got - acts == per_layer_w


def test_prefill_flops_follow_the_shapes():
    # two flops per multiply-add: per token 2 x (every projection's weights)
    per_token = sum(bench.prefill_label_flops(S06, k, 1, 1) for k in ("qkv", "o_proj", "gate_up", "down"))
    w_layer = sum(int(np.prod(s)) for s in S06.layer_shapes().values() if len(s) == 2)
    assert per_token == 2 * w_layer == 2 * 15_728_640
    # causal attention: query t of a head attends to t + 1 keys, each costing
    # 2d flops for q.k and 2d for p.v, summed over t = 0..S-1: 2d S (S + 1)
    B, S = 4, 4096
    brute = 0
    for t in range(S):
        brute += 4 * S06.head_dim * (t + 1)
    assert bench.prefill_label_flops(S06, "attn", B, S) == B * S06.n_heads * brute
    total = bench.prefill_flops(S06, B, S)
    assert total == S06.n_layers * (B * S * per_token + bench.prefill_label_flops(S06, "attn", B, S)) \
        + 2 * B * S06.vocab * S06.hidden
    assert abs(S06.n_layers * bench.prefill_label_flops(S06, "attn", B, S) / 1e12 - 7.698) < 1e-3
