"""GPU parity of the gated-attention variant ("ferrite", section "What it
does": 8 query / 2 KV heads of width 256, a sigmoid gate on each head's
output carried per head in the q projection, rotate-half RoPE on 64 of the 256
dims) against the oracle.

Shapes GATED_TINY (fp32, tolerance 1e-4) and GATED_BF16 (bf16, 2e-2), seeded
random-init weights and uniform-random tokens.  Covers the prefill (fp32 vector
path; bf16 GEMM path with the head_dim-256 vector attention), teacher-forced
decode at batch 2 (GEMV path) and batch 10 (GEMM path), and the cached K of
layer 0 (only its first 64 dims rotate).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import oracle as O

from gpu_common import TOL, check_argmax, check_logits, dev_tokens, make_model, need_gpu, weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def test_gated_tiny_fp32_prefill_and_decode():
    wl = synth.workload("gated_tiny_fp32")
    shape = wl.shape
    prompt = wl.prompts[0]
    m = make_model(shape, max_seqs=2, max_ctx=64)
    orc = O.Oracle(shape, weights(shape))
    try:
        lg = m.prefill(dev_tokens(prompt[None, :]), [0]).cpu().numpy()[0]
        ref = orc.prefill(0, prompt)
        check_logits(lg, ref, TOL["f32"], "gated fp32 prefill")
        tok = O.greedy_argmax(ref)
        out = torch.empty((1, shape.vocab), dtype=torch.float32, device="cuda")
        for k in range(wl.decode_steps):
            pos = len(prompt) + k
            m.decode_step(dev_tokens([tok]), [pos], [0], logits=out)
            ref = orc.decode_step(0, tok, pos)
            got = out.cpu().numpy()[0]
            check_logits(got, ref, TOL["f32"], f"gated fp32 decode step {k}")
            check_argmax(int(np.argmax(got)), ref, f"gated fp32 step {k}")
            tok = O.greedy_argmax(ref)
        # one-token prompt
        lg1 = m.prefill(dev_tokens(prompt[None, :1]), [1]).cpu().numpy()[0]
        check_logits(lg1, O.Oracle(shape, weights(shape)).prefill(0, prompt[:1]), TOL["f32"], "1-token prompt")
    finally:
        m.close()


def test_gated_bf16_prefill_decode_and_cache():
    wl = synth.workload("gated_bf16")
    shape = wl.shape
    m = make_model(shape, max_seqs=10, max_ctx=256)
    orc = O.Oracle(shape, weights(shape))
    try:
        toks = np.stack(wl.prompts)                                   # [2, 160]
        lg = m.prefill(dev_tokens(toks), [0, 1]).cpu().numpy()
        refs = [orc.prefill(i, toks[i]) for i in range(2)]
        for i in range(2):
            check_logits(lg[i], refs[i], TOL["bf16"], f"gated bf16 prefill row {i}")
        # layer-0 K of slot 0: normed, first 64 dims rotated, stored bf16
        dump = {}
        O.Oracle(shape, weights(shape)).forward(toks[0], dump=dump)
        k_ref = dump["layer0.k"][:, 0, :]                            # [160, 256], KV head 0
        k, v = m.kv_read(0, 0, 0, 0, toks.shape[1])
        k = k.float().cpu().numpy()
        assert np.max(np.abs(k - k_ref)) < 2e-2
        assert np.max(np.abs(v.float().cpu().numpy() - dump["layer0.v"][:, 0, :])) < 1e-2
        # teacher-forced decode, batch 2 (vector path)
        out = torch.empty((2, shape.vocab), dtype=torch.float32, device="cuda")
        nxt = [O.greedy_argmax(r) for r in refs]
        for k_ in range(wl.decode_steps):
            pos = toks.shape[1] + k_
            m.decode_step(dev_tokens(nxt), [pos, pos], [0, 1], logits=out)
            got = out.cpu().numpy()
            for i in range(2):
                ref = orc.decode_step(i, nxt[i], pos)
                check_logits(got[i], ref, TOL["bf16"], f"gated bf16 decode step {k_} row {i}")
                nxt[i] = O.greedy_argmax(ref)
        # batch 10 (GEMM path in the decode step): eight more sequences, short prompts
        more = synth.tokens(109, shape.vocab, (8, 24))
        m.prefill(dev_tokens(more), list(range(2, 10)))
        orcs = {}
        cur = {}
        for i in range(8):
            o = O.Oracle(shape, weights(shape))
            cur[2 + i] = O.greedy_argmax(o.prefill(0, more[i]))
            orcs[2 + i] = o
        slots = list(range(10))
        pos0 = toks.shape[1] + wl.decode_steps
        positions = [pos0, pos0] + [24] * 8
        tokens = nxt + [cur[s] for s in range(2, 10)]
        out10 = torch.empty((10, shape.vocab), dtype=torch.float32, device="cuda")
        m.decode_step(dev_tokens(tokens), positions, slots, logits=out10)
        got = out10.cpu().numpy()
        for i in range(2):
            check_logits(got[i], orc.decode_step(i, tokens[i], positions[i]), TOL["bf16"], f"B=10 row {i}")
        for s in range(2, 10):
            check_logits(got[s], orcs[s].decode_step(0, tokens[s], positions[s]), TOL["bf16"], f"B=10 row {s}")
    finally:
        m.close()
