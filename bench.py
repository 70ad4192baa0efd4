"""Benchmark of the forward pass on one MI355X.

Workload (a "step" is one pass of the whole hot path): the 0.6B-shape bf16
model decoding at batch 1 with a bf16 KV cache -- a 512-token uniform-random
prompt is prefilled (untimed), then each step is one fs_decode_step whose
greedy output is fed back on the device, at positions 512, 513, ...  The
prefill side is reported in the same line: one fs_prefill of 4 x 4096 tokens.

Prints one JSON line.  Inputs are seeded synthetic weights and tokens
(random-init, no checkpoint).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12           # bytes/s, MI355X
MFMA_BF16_PEAK = 2.5e15     # dense bf16 flop/s, MI355X


def decode_bytes(shape, ctx):
    """Algorithmic HBM bytes of one bs1 decode step at context length ctx (incl. new token)."""
    es = 2 if shape.dtype == "bf16" else 4
    H, L, I, V = shape.hidden, shape.n_layers, shape.ffn, shape.vocab
    qw, kvw = shape.q_width, shape.kv_width
    per_layer_w = ((qw + 2 * kvw) * H + H * qw + 2 * I * H + H * I) * es + (2 * H + 2 * shape.head_dim) * es
    weights = L * per_layer_w + V * H * es + H * es
    kv_read = L * 2 * kvw * es * (ctx - 1)
    kv_write = L * 2 * kvw * es
    return weights + kv_read + kv_write + H * es


def prefill_flops(shape, B, S):
    H, L, I = shape.hidden, shape.n_layers, shape.ffn
    qw, kvw, d = shape.q_width, shape.kv_width, shape.head_dim
    T = B * S
    gemm = 2 * T * L * ((qw + 2 * kvw) * H + H * qw + 2 * I * H + H * I)
    attn = B * L * shape.n_heads * 2 * d * S * (S + 1)
    head = 2 * B * shape.vocab * H
    return gemm, attn, head


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from dense_gqa_transformer_amd.model import Model, argmax

    wl = synth.workload("decode_0p6b_bs1")
    shape = wl.shape
    prompt = wl.prompts[0]
    steps = min(args.steps, wl.decode_steps)
    w = synth.make_weights(shape, 0)
    model = Model(shape, w, max_seqs=5, max_ctx=4096)
    dev = torch.device("cuda")
    tok = torch.from_numpy(prompt[None, :].astype(np.int32)).to(dev)
    nxt = torch.empty((1,), dtype=torch.int32, device=dev)

    # warmup on slot 1
    lg = model.prefill(tok, [1])
    argmax(lg, out=nxt)
    for k in range(args.warmup):
        model.decode_step(nxt, [len(prompt) + k], [1], next_ids=nxt)
    torch.cuda.synchronize()

    # timed: decode steps on slot 0 after an untimed prefill
    lg = model.prefill(tok, [0])
    argmax(lg, out=nxt)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        model.decode_step(nxt, [len(prompt) + k], [0], next_ids=nxt)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_step = dt * 1e3 / steps
    tok_s = steps / dt
    ctx_avg = len(prompt) + (steps + 1) / 2.0
    bytes_avg = decode_bytes(shape, ctx_avg)
    hbm_frac = bytes_avg / (dt / steps) / HBM_PEAK

    out = {
        "metric": "decode tok/s @bs1 (0.6B shape, bf16 weights + KV)",
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init weights, uniform-random tokens)",
        "config": {"workload": "decode_0p6b_bs1: 512-token prompt, greedy bs1 decode from position 512",
                   "global_batch": 1, "seq_len": len(prompt) + steps, "parallelism": "none"},
        "decode_hbm_frac_step": round(hbm_frac, 4),
    }

    if not args.no_prefill:
        pw = synth.workload("prefill_0p6b_4x4096")
        ptok = torch.from_numpy(np.stack(pw.prompts).astype(np.int32)).to(dev)
        logits = torch.empty((4, shape.vocab), dtype=torch.float32, device=dev)
        model.prefill(ptok, [0, 1, 2, 3], logits=logits)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        reps = 2
        for _ in range(reps):
            model.prefill(ptok, [0, 1, 2, 3], logits=logits)
        torch.cuda.synchronize()
        pdt = (time.perf_counter() - t0) / reps
        g, a, h = prefill_flops(shape, 4, 4096)
        out["prefill"] = {"workload": "prefill_0p6b_4x4096", "tok_s": round(4 * 4096 / pdt, 1),
                          "ms": round(pdt * 1e3, 3),
                          "mfma_frac_pass": round((g + a + h) / pdt / MFMA_BF16_PEAK, 4)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
