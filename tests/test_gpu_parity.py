"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Tolerances: max-abs logit error <= 1e-4 for the fp32 tiny model and <= 2e-2
for bf16 weights; greedy IDs bit-exact wherever the oracle's top-2 gap
exceeds 1e-2.  Full-size workloads are checked on sampled outputs the oracle
computes one by one (layer-0 K/V of single tokens, short prefixes, a few
teacher-forced decode rows) and on properties that hold at any size (batch
invariance, cached == uncached).
"""
import json
import os

import numpy as np
import pytest
import torch

import synth
from oracle import oracle as O
from tests.gpu_common import (GAP, TOL, check_argmax, check_logits, dev_tokens, fresh_oracle,
                              make_model, need_gpu, oracle_for, weights)

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _flush(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ argmax
def test_argmax_golden_rows():
    from dense_gqa_transformer_amd.model import argmax
    with open(os.path.join(GOLDEN, "argmax_rule.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        row = torch.tensor([[float(v) for v in c["row"]]], dtype=torch.float32).cuda()
        assert int(argmax(row).cpu()[0]) == c["expect"], c


def test_argmax_large_rows_with_ties_and_nonfinite():
    from dense_gqa_transformer_amd.model import argmax
    rng = np.random.default_rng(7)
    V = 151936
    a = rng.standard_normal((9, V)).astype(np.float32)
    a[0, [5, 70000, 151935]] = 9.0                       # exact tie: lowest ID
    a[1, :] = 1.0                                        # all equal -> 0
    a[2, 1000] = np.inf; a[2, 2000] = 50.0               # inf is not finite
    a[3, :] = np.nan; a[3, 123456] = -3.0                # one finite value
    a[4, :] = np.nan                                     # none finite -> -1
    a[5, :] = -np.inf
    a[6, 151935] = 100.0                                 # last element
    a[7, 0] = 100.0                                      # first element
    a[8, 77777] = a[8].max() + 1e-3
    got = argmax(torch.from_numpy(a).cuda()).cpu().numpy()
    want = [O.greedy_argmax_fast(r) for r in a]
    assert list(got) == want


# ------------------------------------------------------------------ tiny fp32 model
def test_tiny_fp32_prefill_and_teacher_forced_decode():
    shape = synth.TINY
    wl = synth.workload("tiny_fp32")
    model = make_model(shape, max_seqs=2, max_ctx=64)
    orc = fresh_oracle(shape)
    prompt = wl.prompts[0]
    ref = orc.prefill(0, prompt)
    gpu = model.prefill(dev_tokens(prompt[None, :]), [0]).cpu().numpy()[0]
    check_logits(gpu, ref, TOL["f32"], "tiny prefill")
    hist = list(prompt)
    logits = torch.empty((1, shape.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty((1,), dtype=torch.int32, device="cuda")
    for k in range(wl.decode_steps):
        tok = O.greedy_argmax_fast(ref)                   # teacher forcing: oracle's token
        pos = len(hist)
        model.decode_step(dev_tokens([tok]), [pos], [0], logits=logits, next_ids=nxt)
        ref = orc.decode_step(0, tok, pos)
        check_logits(logits.cpu().numpy()[0], ref, TOL["f32"], f"tiny decode step {k}")
        check_argmax(nxt.cpu().numpy()[0], ref, f"tiny decode step {k}")
        hist.append(tok)
    assert model.slot_length(0) == len(hist)
    # GPU cached == GPU uncached on the whole history
    full = model.prefill(dev_tokens(np.array(hist, dtype=np.int32)[None, :]), [1]).cpu().numpy()[0]
    check_logits(full, logits.cpu().numpy()[0], TOL["f32"], "tiny cached vs uncached")


def test_tiny_fp32_free_running_greedy_matches_oracle():
    shape = synth.TINY
    wl = synth.workload("tiny_fp32")
    model = make_model(shape, max_seqs=1, max_ctx=64)
    orc = fresh_oracle(shape)
    prompt = wl.prompts[0]
    ref = orc.prefill(0, prompt)
    gl = model.prefill(dev_tokens(prompt[None, :]), [0])
    nxt = torch.empty((1,), dtype=torch.int32, device="cuda")
    from dense_gqa_transformer_amd.model import argmax
    argmax(gl, out=nxt)
    pos = len(prompt)
    for k in range(wl.decode_steps):
        want = O.greedy_argmax_fast(ref)
        got = int(nxt.cpu()[0])
        if O.top2_gap(ref) <= GAP:
            break                                         # near-tie: sequences may part here
        assert got == want, f"greedy step {k}"
        model.decode_step(nxt, [pos], [0], next_ids=nxt)  # next fed back in place
        ref = orc.decode_step(0, want, pos)
        pos += 1


def test_tiny_single_token_and_batched_prefill():
    shape = synth.TINY
    model = make_model(shape, max_seqs=4, max_ctx=40)
    orc = oracle_for(shape)
    rng = np.random.default_rng(3)
    # S = 1 (attention over one token returns V)
    t1 = rng.integers(0, shape.vocab, size=(1, 1)).astype(np.int32)
    gpu = model.prefill(dev_tokens(t1), [2]).cpu().numpy()[0]
    check_logits(gpu, orc.forward(t1[0]), TOL["f32"], "S=1")
    # B = 3 rows of 37 tokens (ragged against every tile size)
    tb = rng.integers(0, shape.vocab, size=(3, 37)).astype(np.int32)
    gpu = model.prefill(dev_tokens(tb), [3, 0, 1]).cpu().numpy()
    for b in range(3):
        check_logits(gpu[b], orc.forward(tb[b]), TOL["f32"], f"B=3 row {b}")
    assert [model.slot_length(s) for s in (3, 0, 1, 2)] == [37, 37, 37, 1]


def test_decode_from_empty_slot_and_error_paths():
    from dense_gqa_transformer_amd import native
    shape = synth.TINY
    model = make_model(shape, max_seqs=2, max_ctx=8)
    orc = fresh_oracle(shape)
    logits = torch.empty((1, shape.vocab), dtype=torch.float32, device="cuda")
    # position 0 of an empty slot is a valid first step
    model.decode_step(dev_tokens([11]), [0], [1], logits=logits)
    check_logits(logits.cpu().numpy()[0], orc.decode_step(1, 11, 0), TOL["f32"], "decode at p=0")
    with pytest.raises(native.FsError) as e:
        model.decode_step(dev_tokens([1]), [5], [1], logits=logits)      # wrong position
    assert e.value.status == native.FS_ERR_INVALID_ARG
    with pytest.raises(native.FsError) as e:
        model.decode_step(dev_tokens([1, 2]), [1, 1], [1, 1], logits=None,
                          next_ids=torch.empty(2, dtype=torch.int32, device="cuda"))
    assert e.value.status == native.FS_ERR_INVALID_ARG                  # duplicate slot
    with pytest.raises(native.FsError) as e:
        model.prefill(dev_tokens(np.zeros((1, 9), np.int32)), [0])       # longer than max_ctx
    assert e.value.status == native.FS_ERR_CAPACITY
    model.prefill(dev_tokens(np.zeros((1, 8), np.int32)), [0])
    with pytest.raises(native.FsError) as e:
        model.decode_step(dev_tokens([1]), [8], [0], logits=logits)      # context exhausted
    assert e.value.status == native.FS_ERR_CAPACITY
    with pytest.raises(native.FsError) as e:
        model.decode_step(dev_tokens([1]), [0], [2], logits=logits)      # slot out of range
    assert e.value.status == native.FS_ERR_INVALID_ARG
    with pytest.raises(native.FsError) as e:
        model.decode_step(dev_tokens([1]), [1], [1])                     # no output requested
    assert e.value.status == native.FS_ERR_INVALID_ARG


# ------------------------------------------------------------------ 0.6B shape
@pytest.fixture(scope="module")
def big():
    shape = synth.QWEN3_0P6B
    _flush("building 0.6B model")
    return shape, make_model(shape, max_seqs=6, max_ctx=1152)


def test_scorer_6_tokens(big):
    shape, model = big
    wl = synth.workload("scorer_0p6b")
    prompt = wl.prompts[0]
    ref = oracle_for(shape).forward(prompt)
    gpu = model.prefill(dev_tokens(prompt[None, :]), [0]).cpu().numpy()[0]
    check_logits(gpu, ref, TOL["bf16"], "scorer")
    check_argmax(int(np.argmax(gpu)), ref, "scorer argmax")
    # top-10 by logit: same set except inside near-ties at the boundary
    want = O.top_k(ref, 10)
    got = O.top_k(gpu, 10)
    kth = np.sort(ref)[-10]
    for g in set(got) - set(want):
        assert ref[g] >= kth - 2 * TOL["bf16"]


@pytest.mark.parametrize("S", [1, 3, 5, 8, 9, 64, 65, 130, 1100])
def test_prefill_lengths_both_paths(big, S):
    # S <= 8 runs the GEMV path (1, 4 or 8 rows per workgroup); 9..64 the few-row
    # MFMA GEMM, whose O and down projections split K over workgroups and leave
    # partials for the next RMSNorm (the last layer's are added before the
    # head); larger S the tiled MFMA GEMMs (128-row tiles with ragged tails at
    # 65 and 130; 256-row tiles with a 76-row tail at 1100)
    shape, model = big
    toks = synth.tokens(500 + S, shape.vocab, (1, S))
    ref = oracle_for(shape).forward(toks[0])
    gpu = model.prefill(dev_tokens(toks), [1]).cpu().numpy()[0]
    check_logits(gpu, ref, TOL["bf16"], f"prefill S={S}")


def test_decode_bs1_teacher_forced(big):
    shape, model = big
    wl = synth.workload("decode_0p6b_bs1")
    prompt = wl.prompts[0]
    orc = fresh_oracle(shape)
    _flush("oracle prefill 512")
    ref = orc.prefill(0, prompt)
    gpu = model.prefill(dev_tokens(prompt[None, :]), [2]).cpu().numpy()[0]
    check_logits(gpu, ref, TOL["bf16"], "bs1 prefill 512")
    logits = torch.empty((1, shape.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty((1,), dtype=torch.int32, device="cuda")
    hist = list(prompt)
    errs = []
    for k in range(24):
        tok = O.greedy_argmax_fast(ref)
        pos = len(hist)
        model.decode_step(dev_tokens([tok]), [pos], [2], logits=logits, next_ids=nxt)
        ref = orc.decode_step(0, tok, pos)
        errs.append(check_logits(logits.cpu().numpy()[0], ref, TOL["bf16"], f"bs1 decode step {k}"))
        check_argmax(nxt.cpu().numpy()[0], ref, f"bs1 decode step {k}")
        hist.append(tok)
    _flush(f"bs1 teacher-forced max errors: {max(errs):.3e}")
    # the cached K/V of layer 0 equals the oracle's at sampled positions
    kk, vv = model.kv_read(0, 2, 3, 0, len(hist))
    ko = orc.cache[0][0][0][:, 3, :]
    vo = orc.cache[0][0][1][:, 3, :]
    np.testing.assert_allclose(kk.float().cpu().numpy(), ko, atol=2e-2, rtol=1e-2)
    np.testing.assert_allclose(vv.float().cpu().numpy(), vo, atol=2e-2, rtol=1e-2)


def test_decode_crosses_onepass_context(big):
    # batch-1 steps at 95..99 keys: the attention switches from the one-pass
    # form (up to 96 keys) to split-K chunks plus the merge launch (another
    # captured graph) in the middle of the sequence
    shape, model = big
    prompt = synth.tokens(4242, shape.vocab, 94)
    orc = fresh_oracle(shape)
    ref = orc.prefill(0, prompt)
    model.prefill(dev_tokens(prompt[None, :]), [5])
    logits = torch.empty((1, shape.vocab), dtype=torch.float32, device="cuda")
    for k in range(5):
        tok = O.greedy_argmax_fast(ref)
        pos = len(prompt) + k
        model.decode_step(dev_tokens([tok]), [pos], [5], logits=logits)
        ref = orc.decode_step(0, tok, pos)
        check_logits(logits.cpu().numpy()[0], ref, TOL["bf16"], f"decode at {pos + 1} keys")


def test_decode_bs1_free_running_then_uncached(big):
    # the timed configuration: 512 prompt + 256 greedy steps with next fed back
    shape, model = big
    wl = synth.workload("decode_0p6b_bs1")
    prompt = wl.prompts[0]
    from dense_gqa_transformer_amd.model import argmax
    gl = model.prefill(dev_tokens(prompt[None, :]), [3])
    nxt = torch.empty((1,), dtype=torch.int32, device="cuda")
    argmax(gl, out=nxt)
    toks = [int(nxt.cpu()[0])]
    logits = torch.empty((1, shape.vocab), dtype=torch.float32, device="cuda")
    for k in range(wl.decode_steps):
        model.decode_step(nxt, [len(prompt) + k], [3], logits=logits, next_ids=nxt)
        toks.append(int(nxt.cpu()[0]))
    assert model.slot_length(3) == len(prompt) + wl.decode_steps
    lg = logits.cpu().numpy()[0]
    assert toks[-1] == O.greedy_argmax_fast(lg)
    # uncached pass over the same 767 tokens gives the same last logits
    full = np.concatenate([prompt, np.array(toks[:-1], dtype=np.int32)])
    un = model.prefill(dev_tokens(full[None, :]), [4]).cpu().numpy()[0]
    check_logits(un, lg, TOL["bf16"], "bs1 cached vs uncached after 256 steps")


def test_layer0_kv_single_tokens_match_oracle(big):
    # layer-0 K and V at position p depend only on token p and p
    shape, model = big
    orc = oracle_for(shape)
    toks = synth.tokens(77, shape.vocab, (1, 900))
    model.prefill(dev_tokens(toks), [5])
    kk, vv = model.kv_read(0, 5, 6, 0, 900)
    for p in (0, 1, 255, 256, 511, 899):
        x = orc.embed[toks[0, p:p + 1].astype(np.int64)]
        _, k, v = orc._block(0, x, np.array([p]), None, None)
        np.testing.assert_allclose(kk[p].float().cpu().numpy(), k[0, 6], atol=1e-2, rtol=1e-2)
        np.testing.assert_allclose(vv[p].float().cpu().numpy(), v[0, 6], atol=1e-2, rtol=1e-2)


# ------------------------------------------------------------------ 4 x 4096 prefill
def test_prefill_4x4096_sampled():
    shape = synth.QWEN3_0P6B
    wl = synth.workload("prefill_0p6b_4x4096")
    model = make_model(shape, max_seqs=5, max_ctx=4096)
    orc = oracle_for(shape)
    toks = np.stack(wl.prompts)
    _flush("gpu prefill 4x4096")
    lg4 = model.prefill(dev_tokens(toks), [0, 1, 2, 3]).cpu().numpy()
    assert np.all(np.isfinite(lg4))
    # batch invariance: row 2 alone
    lg1 = model.prefill(dev_tokens(toks[2:3]), [4]).cpu().numpy()[0]
    check_logits(lg1, lg4[2], 1e-5, "4x4096 row 2 alone vs in batch")
    # all layers' K/V of the first 24 positions of row 1 == oracle prefix prefill
    o2 = fresh_oracle(shape)
    o2.prefill(0, toks[1, :24])
    for layer in (0, 13, 27):
        for j in (0, 7):
            kk, vv = model.kv_read(layer, 1, j, 0, 24)
            np.testing.assert_allclose(kk.float().cpu().numpy(), o2.cache[0][layer][0][:, j], atol=3e-2, rtol=2e-2)
            np.testing.assert_allclose(vv.float().cpu().numpy(), o2.cache[0][layer][1][:, j], atol=3e-2, rtol=2e-2)
    # layer-0 K/V at far positions, one token at a time
    kk, vv = model.kv_read(0, 3, 5, 0, 4096)
    for p in (0, 1000, 2047, 4095):
        x = orc.embed[toks[3, p:p + 1].astype(np.int64)]
        _, k, v = orc._block(0, x, np.array([p]), None, None)
        np.testing.assert_allclose(kk[p].float().cpu().numpy(), k[0, 5], atol=1e-2, rtol=1e-2)
        np.testing.assert_allclose(vv[p].float().cpu().numpy(), v[0, 5], atol=1e-2, rtol=1e-2)
    if os.environ.get("FS_FULL_ORACLE") == "1":
        _flush("oracle 4096-token forward (opt-in)")
        check_logits(lg4[0], orc.forward(toks[0]), TOL["bf16"], "4x4096 row 0 vs oracle")


@pytest.mark.parametrize("which,B,S", [("bf16", 2, 2048), ("bf16", 3, 1400), ("int8", 2, 2048)])
def test_prefill_fused_rope_epilogue_matches_separate_pass(monkeypatch, which, B, S):
    # On the large GEMM the per-head q/k norm + RoPE + K/V write run in the QKV
    # GEMM's epilogue; it must give the same bits as the GEMM storing q|k|v and
    # the separate rope_kv pass.  2 x 2048 tokens (16 x 16 tiles of 256) and
    # 3 x 1400 (a ragged last row tile, sequences starting inside tiles): the
    # logits and the K/V of every sequence in four layers, with the timing hook
    # confirming which path ran; int8 weights take the per-column scales
    # before the epilogue.
    shape = synth.QWEN3_0P6B if which == "bf16" else synth.QWEN3_0P6B_I8
    toks = synth.tokens(2055 + S, shape.vocab, (B, S))
    res = {}
    for mode in ("0", "1"):
        monkeypatch.setenv("FS_PREFILL_FUSE_ROPE", mode)
        model = make_model(shape, max_seqs=B, max_ctx=S)
        _flush(f"{which} {B} x {S} prefill, fused norm/RoPE epilogue {mode}")
        model.timing(True)
        lg = model.prefill(dev_tokens(toks), list(range(B))).cpu().numpy()
        torch.cuda.synchronize()
        n_rope = model.timing_read("rope_kv")[1]
        model.timing(False)
        assert n_rope == (0 if mode == "1" else shape.n_layers), (mode, n_rope)
        assert np.all(np.isfinite(lg))
        kv = []
        for layer in (0, 1, 14, 27):
            for slot in range(B):
                for j in (0, 3, 7):
                    kk, vv = model.kv_read(layer, slot, j, 0, S)
                    kv.append((kk.cpu(), vv.cpu()))
        res[mode] = (lg, kv)
        model.close()
    np.testing.assert_array_equal(res["0"][0], res["1"][0])
    for (k0, v0), (k1, v1) in zip(res["0"][1], res["1"][1]):
        assert torch.equal(k0, k1) and torch.equal(v0, v1)


# ------------------------------------------------------------------ 64-way ragged decode
def test_decode_bs64_ragged():
    shape = synth.QWEN3_0P6B
    wl = synth.workload("decode_0p6b_bs64")
    B = wl.batch
    model = make_model(shape, max_seqs=B + 1, max_ctx=wl.max_ctx)
    from dense_gqa_transformer_amd.model import argmax
    lens = [len(p) for p in wl.prompts]
    nxt = torch.empty((B,), dtype=torch.int32, device="cuda")
    _flush("gpu ragged prefill of 64 sequences")
    for i, p in enumerate(wl.prompts):
        lg = model.prefill(dev_tokens(p[None, :]), [i])
        argmax(lg, out=nxt[i:i + 1])
    # teacher-forced rows: the two shortest sequences
    order = np.argsort(lens)
    watch = [int(order[0]), int(order[1])]
    orcs = {}
    refs = {}
    for i in watch:
        o = fresh_oracle(shape)
        refs[i] = o.prefill(0, wl.prompts[i])
        orcs[i] = o
    logits = torch.empty((B, shape.vocab), dtype=torch.float32, device="cuda")
    slots = list(range(B))
    for k in range(4):
        host_next = nxt.cpu().numpy().copy()
        for i in watch:
            host_next[i] = O.greedy_argmax_fast(refs[i])
        toks = dev_tokens(host_next)
        positions = [lens[i] + k for i in range(B)]
        model.decode_step(toks, positions, slots, logits=logits, next_ids=nxt)
        lg = logits.cpu().numpy()
        ids = nxt.cpu().numpy()
        # every row's greedy ID is the rule applied to the logits it returned
        for i in range(B):
            assert int(ids[i]) == O.greedy_argmax_fast(lg[i]), f"bs64 row {i} step {k}: next ID"
        for i in watch:
            refs[i] = orcs[i].decode_step(0, int(host_next[i]), lens[i] + k)
            check_logits(lg[i], refs[i], TOL["bf16"], f"bs64 row {i} step {k}")
            check_argmax(nxt.cpu().numpy()[i], refs[i], f"bs64 row {i} step {k}")
    # batch invariance: replay row w alone in a spare slot up to the same point
    w = watch[0]
    hist = list(wl.prompts[w])
    # its teacher-forced tokens were the oracle's greedy picks
    o = fresh_oracle(shape)
    r = o.prefill(0, wl.prompts[w])
    for k in range(4):
        t = O.greedy_argmax_fast(r)
        r = o.decode_step(0, t, lens[w] + k)
        hist.append(t)
    solo = model.prefill(dev_tokens(np.array(hist[:-1], dtype=np.int32)[None, :]), [B])
    one = torch.empty((1, shape.vocab), dtype=torch.float32, device="cuda")
    model.decode_step(dev_tokens([hist[-1]]), [len(hist) - 1], [B], logits=one)
    check_logits(one.cpu().numpy()[0], lg[w], TOL["bf16"], "bs64 row vs B=1")
    # then the remaining free-running steps of the workload run and stay finite
    for k in range(4, wl.decode_steps):
        model.decode_step(nxt, [lens[i] + k for i in range(B)], slots, next_ids=nxt)
    ids = nxt.cpu().numpy()
    assert np.all((ids >= 0) & (ids < shape.vocab))
    assert [model.slot_length(i) for i in range(B)] == [lens[i] + wl.decode_steps for i in range(B)]


# ------------------------------------------------------------------ the two decode attention forms
@pytest.mark.parametrize("mode", ["split", "onepass"])
@pytest.mark.parametrize("which", ["tiny_fp32", "0p6b_bf16"])
def test_decode_attention_forms(monkeypatch, mode, which):
    # split-K chunks + merge launch, and the one-pass 16-wave workgroup, each
    # forced for every step: three ragged sequences (1, 37 and 300 tokens of
    # context on the tiny model, 1, 200 and 1100 on the 0.6B shape, the last
    # past the context up to which the one-pass form is chosen by itself),
    # teacher-forced decode at batch 3 and at batch 1, against the oracle
    shape = synth.TINY if which == "tiny_fp32" else synth.QWEN3_0P6B
    tol = TOL["f32"] if which == "tiny_fp32" else TOL["bf16"]
    lens = [1, 37, 300] if which == "tiny_fp32" else [1, 200, 1100]
    monkeypatch.setenv("FS_DECODE_ATTN", mode)
    _flush(f"decode attention form {mode} on {which}")
    model = make_model(shape, max_seqs=3, max_ctx=max(lens) + 8)
    try:
        orcs, refs = [], []
        for i, n in enumerate(lens):
            toks = synth.tokens(4100 + n, shape.vocab, (1, n))
            model.prefill(dev_tokens(toks), [i])
            o = fresh_oracle(shape)
            refs.append(o.prefill(0, toks[0]))
            orcs.append(o)
        out = torch.empty((3, shape.vocab), dtype=torch.float32, device="cuda")
        nxt = torch.empty((3,), dtype=torch.int32, device="cuda")
        for k in range(3):
            toks = [O.greedy_argmax_fast(r) for r in refs]
            pos = [n + k for n in lens]
            model.decode_step(dev_tokens(toks), pos, [0, 1, 2], logits=out, next_ids=nxt)
            got, ids = out.cpu().numpy(), nxt.cpu().numpy()
            refs = [orcs[i].decode_step(0, toks[i], pos[i]) for i in range(3)]
            for i in range(3):
                check_logits(got[i], refs[i], tol, f"{mode} {which} B=3 row {i} step {k}")
                check_argmax(int(ids[i]), refs[i], f"{mode} {which} B=3 row {i} step {k}")
        one = torch.empty((1, shape.vocab), dtype=torch.float32, device="cuda")
        for i in range(3):
            tok = O.greedy_argmax_fast(refs[i])
            pos = lens[i] + 3
            model.decode_step(dev_tokens([tok]), [pos], [i], logits=one)
            check_logits(one.cpu().numpy()[0], orcs[i].decode_step(0, tok, pos), tol, f"{mode} {which} B=1 row {i}")
    finally:
        model.close()


# ------------------------------------------------------------------ graph replay and timing hook
def test_graph_replay_matches_eager(monkeypatch):
    # decode steps replayed from captured graphs give the same bits as eager launches
    shape = synth.QWEN3_0P6B
    toks = synth.tokens(909, shape.vocab, (1, 40))
    res = {}
    for mode in ("1", "0"):
        monkeypatch.setenv("FS_DECODE_GRAPHS", mode)
        model = make_model(shape, max_seqs=1, max_ctx=128)
        lg = model.prefill(dev_tokens(toks), [0])
        nxt = torch.empty((1,), dtype=torch.int32, device="cuda")
        from dense_gqa_transformer_amd.model import argmax
        argmax(lg, out=nxt)
        logits = torch.empty((1, shape.vocab), dtype=torch.float32, device="cuda")
        outs = []
        for k in range(40):                    # crosses a chunk-count boundary (graph re-capture)
            model.decode_step(nxt, [40 + k], [0], logits=logits, next_ids=nxt)
            torch.cuda.synchronize()            # eager host work between replays
            outs.append(logits.cpu().numpy()[0].copy())
        res[mode] = np.stack(outs)
        model.close()
    np.testing.assert_array_equal(res["1"], res["0"])


def test_timing_hook_labels(big):
    shape, model = big
    toks = synth.tokens(31, shape.vocab, (1, 20))
    model.prefill(dev_tokens(toks), [0])
    model.timing(True)
    nxt = torch.tensor([5], dtype=torch.int32, device="cuda")
    for k in range(3):
        model.decode_step(nxt, [20 + k], [0], next_ids=nxt)
    torch.cuda.synchronize()
    for lab, per_step in (("qkv", 28), ("attn", 28), ("o_proj", 28), ("gate_up", 28), ("down", 28),
                          ("head", 1), ("argmax", 1), ("embed", 1)):
        ms, n = model.timing_read(lab)
        assert n == 3 * per_step and ms > 0, lab
    model.timing(False)


def test_kernel_bench_hook_leaves_decode_intact(big):
    shape, model = big
    toks = synth.tokens(57, shape.vocab, (1, 33))
    ref = model.prefill(dev_tokens(toks), [0]).cpu().numpy()[0]
    for lab in ("qkv", "attn", "attn_split", "attn_onepass", "combine", "o_proj", "gate_up", "down", "head",
                "empty", "mfma", "hbm"):
        us = model.kernel_bench(lab, reps=2, slot=5, position=100)
        assert 0.0 < us < 10000.0, lab
    from dense_gqa_transformer_amd import native
    with pytest.raises(native.FsError):
        model.kernel_bench("nope", reps=1)
    # the slot's state is untouched: decoding continues to match the uncached pass
    logits = torch.empty((1, shape.vocab), dtype=torch.float32, device="cuda")
    t = int(np.argmax(ref))
    model.decode_step(dev_tokens([t]), [33], [0], logits=logits)
    full = np.concatenate([toks[0], [t]]).astype(np.int32)
    un = model.prefill(dev_tokens(full[None, :]), [1]).cpu().numpy()[0]
    check_logits(logits.cpu().numpy()[0], un, TOL["bf16"], "decode after kernel_bench")
