"""GPU parity over the shapes the kernels are instantiated for, on small models.

The main parity suite runs the tiny fp32 model, the 0.6B shape and the gated
variant; these cases reach the remaining instantiations: grouped-query ratios
1, 4 and 8 (and 2 with one KV head per pair), head_dim 64, 128 and 256, partial
RoPE on the base model, hidden = ffn = 4096 (the widest rows the decode
GEMV takes), and both dtypes.  Each model (2 layers, seeded
random-init weights, uniform-random tokens) is checked against the oracle on
a batched prefill of two prompts (the MFMA GEMM and attention paths for bf16,
more than 64 rows), a one-token prompt, teacher-forced decode at batch 2 (GEMV)
and a decode step at batch 12 (the few-row MFMA GEMM for bf16).  Tolerances
as elsewhere: 1e-4 (fp32) and 2e-2 (bf16) on every logit, the bf16 bound
being the one set for the 0.6B shape's hidden width of 1024.  Its scaling to
wider models follows from the weight distribution, not from measured error:
a logit is E[v] . h with E ~ N(0, 0.02^2) and h the final RMSNorm output
(unit RMS times norm weights of mean 1), so logits spread with standard
deviation 0.02 * sqrt(hidden); rounding the activations to bf16 perturbs h by
a relative amount that does not depend on the width, so the logit error grows
with that spread, and the bound is 2e-2 * sqrt(hidden / 1024) for hidden
above 1024 (4e-2 at hidden 4096).
"""
import math
import numpy as np
import pytest
import torch

import synth
from oracle import oracle as O

from gpu_common import TOL, check_logits, dev_tokens, make_model, need_gpu, weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _shape(nq, nkv, d, dtype, rope_dim=0, hidden=512, ffn=768):
    return synth.ModelShape(n_layers=2, hidden=hidden, n_heads=nq, n_kv_heads=nkv, head_dim=d, ffn=ffn,
                            vocab=2048, dtype=dtype, rope_dim=rope_dim)



def bf16_tol(shape):
    """The 0.6B shape's 2e-2 bound scaled by the logit spread, sqrt(hidden / 1024)."""
    return TOL["bf16"] * max(1.0, math.sqrt(shape.hidden / 1024.0))


CASES = {
    "mha_d64_bf16": _shape(4, 4, 64, synth.BF16, hidden=256),      # ratio 1, odd group: one head per workgroup
    "gqa8_d64_bf16": _shape(8, 1, 64, synth.BF16),                 # ratio 8
    "gqa4_d128_bf16": _shape(8, 2, 128, synth.BF16),               # ratio 4: the DMA-fed attention kernel
    "mha_d128_bf16": _shape(4, 4, 128, synth.BF16),                # ratio 1 at d 128: MFMA kernel, one head
    "gqa2_d256_bf16": _shape(4, 2, 256, synth.BF16),               # d 256, full rotation
    "rope32_d128_bf16": _shape(8, 4, 128, synth.BF16, rope_dim=32),
    "wide_h4096_bf16": _shape(32, 8, 128, synth.BF16, hidden=4096, ffn=4096),   # the widest rows the GEMV takes
    "wide_h4096_f32": _shape(32, 8, 128, synth.F32, hidden=4096, ffn=4096),
    "gqa8_d64_f32": _shape(8, 1, 64, synth.F32),
    "gqa2_d256_f32": _shape(4, 2, 256, synth.F32, rope_dim=64),
}


@pytest.mark.parametrize("name", list(CASES))
def test_shape_parity(name):
    shape = CASES[name]
    tol = TOL["f32"] if shape.dtype == synth.F32 else bf16_tol(shape)
    seed = 700 + list(CASES).index(name)
    S = 96
    prompts = synth.tokens(seed, shape.vocab, (2, S))
    print(f"shape case {name} seed {seed}", flush=True)
    m = make_model(shape, max_seqs=12, max_ctx=160)
    errs = []

    def check(got, ref, tol, what):
        errs.append(check_logits(got, ref, tol, what))
    try:
        orcs = [O.Oracle(shape, weights(shape)) for _ in range(2)]
        lg = m.prefill(dev_tokens(prompts), [0, 1]).cpu().numpy()
        refs = [orcs[i].prefill(0, prompts[i]) for i in range(2)]
        for i in range(2):
            check(lg[i], refs[i], tol, f"{name} prefill row {i}")
        # teacher-forced decode at batch 2
        out = torch.empty((2, shape.vocab), dtype=torch.float32, device="cuda")
        for k in range(4):
            toks = [O.greedy_argmax(r) for r in refs]
            m.decode_step(dev_tokens(toks), [S + k, S + k], [0, 1], logits=out)
            got = out.cpu().numpy()
            refs = [orcs[i].decode_step(0, toks[i], S + k) for i in range(2)]
            for i in range(2):
                check(got[i], refs[i], tol, f"{name} decode {k} row {i}")
        # one-token prompts in ten more slots, then one step over all twelve
        singles = synth.tokens(seed + 50, shape.vocab, (10, 1))
        lg1 = m.prefill(dev_tokens(singles), list(range(2, 12))).cpu().numpy()
        o1 = []
        for i in range(10):
            o = O.Oracle(shape, weights(shape))
            r = o.prefill(0, singles[i])
            check(lg1[i], r, tol, f"{name} one-token prompt {i}")
            o1.append((o, O.greedy_argmax(r)))
        toks = [O.greedy_argmax(r) for r in refs] + [t for _, t in o1]
        pos = [S + 4, S + 4] + [1] * 10
        out12 = torch.empty((12, shape.vocab), dtype=torch.float32, device="cuda")
        m.decode_step(dev_tokens(toks), pos, list(range(12)), logits=out12)
        got = out12.cpu().numpy()
        for i in range(2):
            check(got[i], orcs[i].decode_step(0, toks[i], S + 4), tol, f"{name} B=12 row {i}")
        for i, (o, t) in enumerate(o1):
            check(got[2 + i], o.decode_step(0, t, 1), tol, f"{name} B=12 row {2 + i}")
        print(f"shape case {name}: max-abs logit error {max(errs):.3e} (bound {tol:.1e})", flush=True)
    finally:
        m.close()
