"""The opt-in persistent batch-1 decode step (FS_DECODE_PERSIST=1: one launch
per step, 256 resident workgroups exchanging activations in memory) against
the oracle and against the default path of one kernel per product.

Teacher-forced batch-1 steps of the 0.6B shape after a 512-token prompt,
logits within 2e-2 of the oracle with greedy IDs exact where the top-2 gap
exceeds 1e-2 ("Milestones", M4/M5), and within 1e-4 of the default path
(same arithmetic, other summation order); then a free-running stretch with
the greedy ID fed back on the device, and the clock trace it records.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import oracle as O
from tests.gpu_common import TOL, check_argmax, check_logits, dev_tokens, make_model, need_gpu, weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def test_persistent_decode_matches_oracle_and_default_path(monkeypatch):
    shape = synth.QWEN3_0P6B
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the persistent step needs 256 CUs")
    prompt = synth.workload("decode_0p6b_bs1").prompts[0]
    monkeypatch.setenv("FS_DECODE_PERSIST", "1")
    monkeypatch.setenv("FS_DECODE_TRACE", "1")
    per = make_model(shape, max_seqs=1, max_ctx=640)
    monkeypatch.setenv("FS_DECODE_PERSIST", "0")
    ref = make_model(shape, max_seqs=1, max_ctx=640)
    try:
        tok = dev_tokens(prompt[None, :])
        per.prefill(tok, [0])
        ref.prefill(tok, [0])
        orc = O.Oracle(shape, weights(shape), dtype=np.float32)
        r = orc.prefill(0, prompt)
        la = torch.empty((1, shape.vocab), dtype=torch.float32, device="cuda")
        lb = torch.empty((1, shape.vocab), dtype=torch.float32, device="cuda")
        na = torch.empty((1,), dtype=torch.int32, device="cuda")
        P = len(prompt)
        for k in range(4):
            t = O.greedy_argmax_fast(r)
            per.decode_step(dev_tokens([t]), [P + k], [0], logits=la, next_ids=na)
            ref.decode_step(dev_tokens([t]), [P + k], [0], logits=lb)
            r = orc.decode_step(0, t, P + k)
            got = la.cpu().numpy()[0]
            err = check_logits(got, r, TOL["bf16"], f"persistent step {k}")
            check_argmax(int(na.cpu()[0]), r, f"persistent step {k} argmax")
            check_logits(got, lb.cpu().numpy()[0], 1e-4, f"persistent vs default path, step {k}")
            print(f"persistent step {k}: max-abs {err:.3e}", flush=True)
        # free-running: the greedy ID fed back on the device, both paths agree
        na2 = na.clone()
        for k in range(4, 36):
            per.decode_step(na, [P + k], [0], logits=la, next_ids=na)
            ref.decode_step(na2, [P + k], [0], logits=lb, next_ids=na2)
            check_logits(la.cpu().numpy()[0], lb.cpu().numpy()[0], 1e-4, f"free-running step {k}")
            if O.top2_gap(lb.cpu().numpy()[0]) > 1e-2:
                assert int(na.cpu()[0]) == int(na2.cpu()[0]), k
            na2.copy_(na)
        assert per.slot_length(0) == P + 36
        tr = per.decode_trace()
        assert tr[0] > 0 and tr[511] > tr[0] and tr[1023] > tr[0], "clock stamps of the last step"
    finally:
        per.close()
        ref.close()
