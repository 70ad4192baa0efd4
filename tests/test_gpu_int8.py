"""GPU parity of the int8 weight format (per-row codes and scales) against the
oracle ("Milestones", M7, the low-bit decision; the format reading is in
oracle/quant.py's header).

The library quantizes the same seeded bf16 / fp32 weights itself; the codes
and scales of its quantizer must equal the oracle's bit for bit, and the
forward pass must match the oracle run on the dequantized weights to the
usual tolerances: 1e-4 on the tiny fp32 model (GEMV path only), 2e-2 on the
0.6B shape with greedy IDs exact away from near-ties.  The 0.6B cases cover
the GEMV path (bs1 decode with the fused argmax, a 6-sequence decode step), the
MFMA GEMM path with the codes widened to bf16 and the scales applied per
column (the scorer's 6 tokens go through the 8-row GEMV; prefill of 130 and
1100 tokens, a 10-sequence decode step), and the 256x256 DMA GEMM
(2 x 4096 prefill, checked through its cached K/V against an oracle prefix).
"""
import functools

import numpy as np
import pytest
import torch

import synth
from oracle import oracle as O
from oracle import quant as Q

from gpu_common import GAP, TOL, check_argmax, check_logits, dev_tokens, make_model, need_gpu, weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _flush(msg):
    print(msg, flush=True)


@functools.lru_cache(maxsize=2)
def _dq(shape):
    return Q.dequantized_weights(weights(shape))


def q_oracle(shape):
    """A fresh oracle (empty cache) on the dequantized weights (shared, float64)."""
    return O.Oracle(shape, _dq(shape))


# ------------------------------------------------------------------ quantizer
def _tricky_rows(cols):
    rows = np.zeros((6, cols), dtype=np.float32)
    rows[1, :9] = [127, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5, 126.5]       # ties, scale 1
    rows[2, 5] = -0.75                                                      # one non-zero
    rows[3, :] = 0.25                                                       # all equal
    rows[4, ::2] = 1e-3
    rows[4, 1] = -3e-3
    rows[5, :] = np.linspace(-1, 1, cols, dtype=np.float32)
    return rows


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_quantizer_bit_exact(dt):
    from dense_gqa_transformer_amd.model import quantize_rows_i8
    rng = np.random.default_rng(61)
    cols = 1024
    w = (rng.standard_normal((300, cols)) * 0.02).astype(np.float32)
    w = np.concatenate([w, _tricky_rows(cols)])
    if dt == "bf16":
        w = synth.round_to_bf16(w)
        src = torch.from_numpy(synth.f32_to_bf16_bits(w).view(np.int16)).cuda().view(torch.bfloat16)
    else:
        src = torch.from_numpy(w).cuda()
    codes, scales = quantize_rows_i8(src)
    rc, rs = Q.quantize_rows(w)
    assert np.array_equal(scales.cpu().numpy(), rs)
    got = codes.cpu().numpy()
    bad = np.argwhere(got != rc)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:4].tolist()}"


def test_quantizer_ragged_width():
    from dense_gqa_transformer_amd.model import quantize_rows_i8
    rng = np.random.default_rng(62)
    w = (rng.standard_normal((7, 24)) * 3).astype(np.float32)      # cols not a multiple of 512
    codes, scales = quantize_rows_i8(torch.from_numpy(w).cuda())
    rc, rs = Q.quantize_rows(w)
    assert np.array_equal(codes.cpu().numpy(), rc) and np.array_equal(scales.cpu().numpy(), rs)


# ------------------------------------------------------------------ tiny fp32
def test_tiny_fp32_int8_prefill_and_decode():
    shape = synth.TINY_I8
    prompt = synth.workload("tiny_fp32").prompts[0]
    m = make_model(shape, max_seqs=2, max_ctx=64)
    orc = q_oracle(shape)
    try:
        lg = m.prefill(dev_tokens(prompt[None, :]), [0]).cpu().numpy()[0]
        ref = orc.prefill(0, prompt)
        check_logits(lg, ref, TOL["f32"], "int8 tiny prefill")
        out = torch.empty((1, shape.vocab), dtype=torch.float32, device="cuda")
        nxt = torch.empty((1,), dtype=torch.int32, device="cuda")
        for k in range(16):
            tok = O.greedy_argmax(ref)
            pos = len(prompt) + k
            m.decode_step(dev_tokens([tok]), [pos], [0], logits=out, next_ids=nxt)
            ref = orc.decode_step(0, tok, pos)
            check_logits(out.cpu().numpy()[0], ref, TOL["f32"], f"int8 tiny decode {k}")
            check_argmax(int(nxt.cpu()[0]), ref, f"int8 tiny decode {k}")
        # the quantized model differs from the unquantized one by more than the tolerance
        plain = O.Oracle(synth.TINY, weights(synth.TINY)).forward(prompt)
        assert np.max(np.abs(plain - orc.forward(prompt))) > 10 * TOL["f32"]
    finally:
        m.close()


# ------------------------------------------------------------------ 0.6B shape
@pytest.fixture(scope="module")
def big8():
    shape = synth.QWEN3_0P6B_I8
    _flush("building 0.6B int8 model")
    m = make_model(shape, max_seqs=10, max_ctx=1152)
    _flush("dequantized oracle")
    orc = q_oracle(shape)
    yield shape, m, orc
    m.close()


def test_0p6b_int8_scorer_and_short_prefills(big8):
    shape, m, orc = big8
    prompt = synth.workload("scorer_0p6b").prompts[0]
    ref = orc.forward(prompt)
    gpu = m.prefill(dev_tokens(prompt[None, :]), [0]).cpu().numpy()[0]
    check_logits(gpu, ref, TOL["bf16"], "int8 scorer")
    check_argmax(int(np.argmax(gpu)), ref, "int8 scorer argmax")
    for S in (130, 1100):
        _flush(f"int8 prefill S={S}")
        toks = synth.tokens(600 + S, shape.vocab, (1, S))
        ref = orc.forward(toks[0])
        gpu = m.prefill(dev_tokens(toks), [1]).cpu().numpy()[0]
        check_logits(gpu, ref, TOL["bf16"], f"int8 prefill S={S}")


def test_0p6b_int8_decode_bs1_and_bs6(big8):
    shape, m, _ = big8
    orc = q_oracle(shape)
    prompt = synth.tokens(611, shape.vocab, 64)
    ref = orc.prefill(0, prompt)
    m.prefill(dev_tokens(prompt[None, :]), [2])
    logits = torch.empty((1, shape.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty((1,), dtype=torch.int32, device="cuda")
    for k in range(8):
        tok = O.greedy_argmax_fast(ref)
        pos = len(prompt) + k
        m.decode_step(dev_tokens([tok]), [pos], [2], logits=logits, next_ids=nxt)
        ref = orc.decode_step(0, tok, pos)
        check_logits(logits.cpu().numpy()[0], ref, TOL["bf16"], f"int8 bs1 decode {k}")
        check_argmax(int(nxt.cpu()[0]), ref, f"int8 bs1 decode {k}")
    # six sequences in one step (the 8-row GEMV and the row-group GEMV head), then
    # ten (the GEMM path: codes widened to bf16, scales per column)
    prompts = synth.tokens(612, shape.vocab, (10, 20))
    toks = synth.tokens(613, shape.vocab, 10)
    refs = []
    for i in range(10):
        o = q_oracle(shape)
        o.prefill(0, prompts[i])
        refs.append(o.decode_step(0, int(toks[i]), 20))
    for B in (6, 10):
        slots = list(range(B))
        m.prefill(dev_tokens(prompts[:B]), slots)
        out = torch.empty((B, shape.vocab), dtype=torch.float32, device="cuda")
        nx = torch.empty((B,), dtype=torch.int32, device="cuda")
        m.decode_step(dev_tokens(toks[:B]), [20] * B, slots, logits=out, next_ids=nx)
        got = out.cpu().numpy()
        ids = nx.cpu().numpy()
        for i in range(B):
            check_logits(got[i], refs[i], TOL["bf16"], f"int8 B={B} row {i}")
            check_argmax(int(ids[i]), refs[i], f"int8 B={B} row {i}")


def test_0p6b_int8_prefill_2x4096_through_the_cache():
    shape = synth.QWEN3_0P6B_I8
    m = make_model(shape, max_seqs=2, max_ctx=4096)
    try:
        toks = synth.tokens(614, shape.vocab, (2, 4096))
        _flush("int8 prefill 2x4096")
        lg = m.prefill(dev_tokens(toks), [0, 1]).cpu().numpy()
        assert np.all(np.isfinite(lg))
        o = q_oracle(shape)
        o.prefill(0, toks[1, :24])
        for layer in (0, 13, 27):
            for j in (0, 7):
                kk, vv = m.kv_read(layer, 1, j, 0, 24)
                np.testing.assert_allclose(kk.float().cpu().numpy(), o.cache[0][layer][0][:, j], atol=3e-2, rtol=2e-2)
                np.testing.assert_allclose(vv.float().cpu().numpy(), o.cache[0][layer][1][:, j], atol=3e-2, rtol=2e-2)
    finally:
        m.close()
