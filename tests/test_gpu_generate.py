"""GPU parity of the generation loop (fs_generate) with the oracle's loop.

The contract ("Coming back to Failed Star", section "Next: one complete
deterministic generation arc") is pinned on a scripted model in
test_generate_oracle.py; here the library's loop runs the real forward pass
and is compared with oracle.generate on the same model: generated IDs and
stop reasons for a zero budget, EOS on the first and on a later step (with and
without the stop ID), both sides of the context boundary, an over-long and an
empty prompt, a sampled run, and a greedy run on the 0.6B shape.  Greedy IDs
must agree until the first step where the oracle's top-2 logit gap is within
the numerical tolerance; from there either ID is acceptable and the comparison
ends.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import generate as G
from oracle import oracle as O
from oracle import sampling as smp

from gpu_common import GAP, fresh_oracle, make_model, need_gpu
from dense_gqa_transformer_amd import native

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def oracle_run(shape, prompt, budget, max_ctx, eos=(), inc=False, sampling=None, uniforms=None):
    """The oracle loop, recording the logits each token was selected from."""
    orc = fresh_oracle(shape)
    seen = []

    def select(lg, i):
        seen.append(lg)
        if sampling is None:
            return O.greedy_argmax(lg)
        T, k, p = sampling
        return smp.sample(lg, T, k, p, float(uniforms[i]))

    ids, why = G.generate_loop(lambda pr: orc.prefill(0, np.asarray(pr)),
                               lambda tok, pos: orc.decode_step(0, tok, pos),
                               prompt, budget, max_ctx, eos, inc, select)
    return ids, why, seen


def compare_greedy(gpu_ids, ref_ids, seen, gap):
    """Equal until the first near-tie of the oracle's logits."""
    for j, (a, b) in enumerate(zip(gpu_ids, ref_ids)):
        if a != b:
            lg = seen[j]
            assert O.top2_gap(lg) <= gap, f"step {j}: GPU {a} vs oracle {b} with top-2 gap {O.top2_gap(lg):.3g}"
            assert lg[a] >= np.max(lg) - gap
            return j
    assert len(gpu_ids) == len(ref_ids)
    return len(gpu_ids)


def test_generate_greedy_tiny():
    shape = synth.TINY
    prompt = synth.workload("tiny_fp32").prompts[0]
    m = make_model(shape, max_seqs=2, max_ctx=64)
    try:
        ids, why = m.generate(prompt, 16)
        ref, rwhy, seen = oracle_run(shape, prompt, 16, 64)
        compare_greedy(ids, ref, seen, 1e-3)
        assert why == rwhy == G.STOP_BUDGET
    finally:
        m.close()


def test_generate_stop_rules_tiny():
    shape = synth.TINY
    prompt = synth.workload("tiny_fp32").prompts[0]          # 16 tokens
    m = make_model(shape, max_seqs=3, max_ctx=24)
    try:
        # zero budget: nothing runs, the slot is untouched
        assert m.generate(prompt, 0, slot=1) == ([], G.STOP_BUDGET)
        assert m.slot_length(1) == 0
        base, _ = m.generate(prompt, 8)
        ref8, _, seen = oracle_run(shape, prompt, 8, 24)
        n_ok = compare_greedy(base, ref8, seen, 1e-3)
        assert n_ok == 8, "tiny greedy run met a near-tie; pick another prompt"
        t0 = base[0]
        # EOS on the first step, with and without the stop ID
        assert m.generate(prompt, 8, eos_ids=[t0]) == ([], G.STOP_EOS)
        assert m.generate(prompt, 8, eos_ids=[t0, 5], include_stop_id=True) == ([t0], G.STOP_EOS)
        # EOS on a later step: a seeded sampled run (deterministic given its
        # uniforms) gives a sequence with new IDs; the first occurrence of the
        # chosen ID stops the loop
        us = torch.from_numpy(synth.uniforms(72, 8)).cuda()
        sbase, _ = m.generate(prompt, 8, sampling=(1.0, 0, 1.0), uniforms=us)
        j = next((i for i in range(1, 8) if sbase[i] not in sbase[:i]), None)
        assert j is not None, f"sampled run repeats one ID: {sbase}"
        ids, why = m.generate(prompt, 8, eos_ids=[sbase[j]], sampling=(1.0, 0, 1.0), uniforms=us)
        assert (ids, why) == (sbase[:j], G.STOP_EOS)
        # context boundary: positions 16..23 can be forwarded, 24 cannot
        ids, why = m.generate(prompt, 100)
        ref, rwhy, seen = oracle_run(shape, prompt, 100, 24)
        compare_greedy(ids, ref, seen, 1e-3)
        assert (len(ids), why) == (9, G.STOP_CONTEXT) and rwhy == G.STOP_CONTEXT
        assert m.slot_length(0) == 24
        assert m.generate(prompt, 9) == (ids, G.STOP_BUDGET)
        # a prompt that fills the context returns one token
        full = np.concatenate([prompt, synth.tokens(77, shape.vocab, 8)]).astype(np.int32)
        ids, why = m.generate(full, 5)
        ref, rwhy, seen = oracle_run(shape, full, 5, 24)
        compare_greedy(ids, ref, seen, 1e-3)
        assert (len(ids), why) == (1, G.STOP_CONTEXT) and rwhy == G.STOP_CONTEXT
        # errors: over-long and empty prompts
        with pytest.raises(native.FsError) as e:
            m.generate(np.concatenate([full, [1]]).astype(np.int32), 5)
        assert e.value.status == native.FS_ERR_CAPACITY
        with pytest.raises(native.FsError) as e:
            m.generate(np.zeros(0, np.int32), 5)
        assert e.value.status == native.FS_ERR_INVALID_ARG
    finally:
        m.close()


def test_generate_sampled_tiny():
    shape = synth.TINY
    prompt = synth.workload("tiny_fp32").prompts[0]
    us = synth.uniforms(71, 20)
    m = make_model(shape, max_seqs=2, max_ctx=64)
    try:
        samp = (0.9, 20, 0.9)
        ids, why = m.generate(prompt, 20, sampling=samp, uniforms=torch.from_numpy(us).cuda())
        ref, rwhy, seen = oracle_run(shape, prompt, 20, 64, sampling=samp, uniforms=us)
        for j, (a, b) in enumerate(zip(ids, ref)):
            if a != b:       # a draw on a boundary: the GPU's token must still be valid there
                assert a in smp.acceptable(seen[j], *samp, float(us[j]), eps=1e-3), f"step {j}"
                break
        else:
            assert why == rwhy == G.STOP_BUDGET and len(ids) == 20
    finally:
        m.close()


def test_generate_greedy_0p6b():
    shape = synth.QWEN3_0P6B
    prompt = synth.workload("scorer_0p6b").prompts[0]         # 6 tokens
    m = make_model(shape, max_seqs=1, max_ctx=64)
    try:
        ids, why = m.generate(prompt, 24)
        ref, rwhy, seen = oracle_run(shape, prompt, 24, 64)
        n = compare_greedy(ids, ref, seen, GAP)
        print(f"0.6B greedy: {n} of 24 IDs identical before any near-tie", flush=True)
        if n == 24:
            assert why == rwhy == G.STOP_BUDGET
    finally:
        m.close()
