"""fs_sample_noalloc (the sampler on the library's static scratch, for callers
that cannot allocate) against fs_sample on the same rows and draws.

The draw is an integer decision made in fp32 by the same kernels on both
sides, so the IDs must be equal bit for bit.  Two calls in a row, the second
with fewer and shorter rows (the static scratch keeps the first call's
contents and must be cleared for the rows the second uses), then greedy and
the capacity error.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from dense_gqa_transformer_amd import native
    native.load()


def test_noalloc_sampler_matches_model_sampler():
    from dense_gqa_transformer_amd import native
    from dense_gqa_transformer_amd.model import Model, sample_noalloc
    shape = synth.TINY
    model = Model(shape, synth.make_weights(shape, 0), max_seqs=64, max_ctx=8)
    try:
        cases = [(64, 151936, 0.8, 50, 0.9, 1401), (5, 3000, 1.3, 0, 0.7, 1402)]
        for B, V, T, k, p, seed in cases:
            logits = torch.from_numpy(synth.logit_rows(seed, B, V)).cuda()
            u = torch.from_numpy(synth.uniforms(seed + 1, B)).cuda()
            want = model.sample(logits, T, k, p, u).cpu().numpy()
            got = sample_noalloc(logits, T, k, p, u).cpu().numpy()
            torch.cuda.synchronize()
            print(f"B={B} V={V} T={T} k={k} p={p}: {np.sum(got == want)} of {B} equal", flush=True)
            np.testing.assert_array_equal(got, want)
            assert np.all((got >= 0) & (got < V))
        # greedy path and a row with no finite value
        logits = torch.from_numpy(synth.logit_rows(1403, 3, 777)).cuda()
        logits[1] = float("nan")
        g0 = model.sample(logits, 0.0).cpu().numpy()
        g1 = sample_noalloc(logits, 0.0).cpu().numpy()
        np.testing.assert_array_equal(g0, g1)
        assert g1[1] == -1
        with pytest.raises(native.FsError) as e:
            sample_noalloc(torch.zeros((65, 16), device="cuda"), 1.0, 0, 1.0, torch.zeros(65, device="cuda"))
        assert e.value.status == native.FS_ERR_CAPACITY
    finally:
        model.close()
