"""Benchmark of the forward pass on one MI355X.

Workload of `value` (a "step" is one pass of the whole hot path): the
0.6B-shape bf16 model decoding at batch 1 with a bf16 KV cache.  A 512-token
uniform-random prompt is prefilled (untimed); each step is one
fs_decode_step whose greedy output is fed back on the device, at positions
512, 513, ...  The prefill side is reported in the same line: fs_prefill of
4 x 4096 tokens.

Also reported:
  roofline     -- the dominant decode kernel (largest per-step time): its
                  algorithmic bytes per launch over its average launch time,
                  measured with HIP events on the library's stream while its
                  28 per-layer launches replay back to back in a graph,
                  against 8 TB/s HBM;
  prefill      -- prefill tok/s and the MFMA roofline of its dominant kernel;
  traffic      -- (in each roofline) HBM bytes per launch from the committed
                  counter summary, while the kernel sources are unchanged;
  cpu_baseline -- the float32 CPU oracle on a bounded sample of the same workload
                  (a 512-token prefill and decode steps), on the host's cores.

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

HBM_PEAK = 8.0e12           # bytes/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15     # dense bf16 flop/s, MI355X
MFMA_FP8_PEAK = 5.0e15      # dense fp8 flop/s, MI355X


# --------------------------------------------------------------------------- algorithmic work
def decode_bytes_per_step(shape, ctx):
    """HBM bytes one bs1 decode step must move at context length ctx (incl. the new token)."""
    es = 2
    H, L, I, V = shape.hidden, shape.n_layers, shape.ffn, shape.vocab
    qw, kvw = shape.q_width, shape.kv_width
    per_layer = ((qw + 2 * kvw) * H + H * qw + 2 * I * H + H * I) * es + (2 * H + 2 * shape.head_dim) * es
    return L * per_layer + V * H * es + H * es + L * 2 * kvw * es * ctx + H * es


def decode_label_bytes(shape, label, ctx):
    """Algorithmic bytes of ONE launch of a decode kernel (bs1), by step label."""
    es = 2
    H, I, V, d = shape.hidden, shape.ffn, shape.vocab, shape.head_dim
    qw, kvw = shape.q_width, shape.kv_width
    if label == "qkv":      # weights + fp32 x in + fp32 q/k/v out
        return (qw + 2 * kvw) * H * es + 4 * H + 4 * (qw + 2 * kvw)
    if label == "o_proj":   # weights + attention partials in + residual read/write
        return H * qw * es + 4 * qw + 8 * H
    if label == "gate_up":  # weights + x in + h out
        return 2 * I * H * es + 4 * H + 4 * I
    if label == "down":     # weights + h in + residual read/write
        return H * I * es + 4 * I + 8 * H
    if label == "head":     # tied embedding + x in
        return V * H * es + 4 * H
    if label == "attn":     # K and V of ctx positions of all KV heads + new k/v written
        return 2 * kvw * es * ctx + 2 * kvw * es + 4 * (qw + 2 * kvw)
    if label == "combine":  # one (o[d], m, l) partial per chunk and head, output row
        chunk = 32                                   # at most 32 chunks, up to 256 positions each
        while chunk < 256 and -(-ctx // chunk) > 32:
            chunk *= 2
        return 4 * shape.n_heads * (d + 2) * -(-ctx // chunk) + 4 * qw
    return None


def prefill_label_flops(shape, label, B, S):
    """Algorithmic flops of ONE launch of a prefill kernel, by step label."""
    H, I = shape.hidden, shape.ffn
    qw, kvw, d = shape.q_width, shape.kv_width, shape.head_dim
    T = B * S
    return {"qkv": 2 * T * (qw + 2 * kvw) * H, "o_proj": 2 * T * H * qw,
            "gate_up": 2 * T * 2 * I * H, "down": 2 * T * H * I,
            "attn": B * shape.n_heads * 2 * d * S * (S + 1)}.get(label)


def prefill_flops(shape, B, S):
    L = shape.n_layers
    total = sum(prefill_label_flops(shape, k, B, S) for k in ("qkv", "o_proj", "gate_up", "down", "attn"))
    return L * total + 2 * B * shape.vocab * shape.hidden


# --------------------------------------------------------------------------- CPU baseline
def cpu_baseline(wl, w, steps, prefill_tokens=512):
    """The CPU oracle in float32 (the precision of the pages' own CPU path) on a
    bounded sample of the same workload: one `prefill_tokens`-token prefill of
    the prompt (timed), then `steps` greedy decode steps (timed).  BLAS threads =
    the CPUs this process may run on; the CPU model and BLAS library are reported."""
    import numpy as np
    from oracle import oracle as O
    threads = len(os.sched_getaffinity(0))
    blas, cores = "unknown", threads
    limiter = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=threads, user_api="blas")
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            cores = int(info[0].get("num_threads", threads))
            blas = f"{info[0].get('internal_api')} {info[0].get('version')} ({info[0].get('architecture')})"
    except Exception:
        pass
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    orc = O.Oracle(wl.shape, w, dtype=np.float32)
    prompt = wl.prompts[0][:prefill_tokens]
    t0 = time.perf_counter()
    logits = orc.prefill(0, prompt)
    pdt = time.perf_counter() - t0
    t0 = time.perf_counter()
    for k in range(steps):
        tok = O.greedy_argmax_fast(logits)
        logits = orc.decode_step(0, tok, len(prompt) + k)
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.restore_original_limits()
    return {"value": round(steps / dt, 3), "unit": "tok/s", "cores": cores, "kind": "oracle",
            "sample": f"{steps} greedy bs1 decode steps from position {len(prompt)} after a {len(prompt)}-token "
                      f"prefill of the same prompt (float32 NumPy oracle)",
            "dtype": "float32", "cpu_model": cpu_model, "blas": blas,
            "prefill_tok_s": round(len(prompt) / pdt, 2), "prefill_tokens": len(prompt)}


def measured_traffic(key):
    """HBM bytes per launch of one kernel from the committed counter summary
    (profiles/traffic.json: rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a plain
    copy), or None when no figure exists or the kernel's sources changed since."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    try:
        with open(os.path.join(root, "profiles", "traffic.json")) as f:
            ent = json.load(f)["kernels"][key]
        h = hashlib.sha256()
        for src in ent["sources"]:
            with open(os.path.join(root, src), "rb") as f:
                h.update(f.read())
    except (OSError, KeyError, ValueError):
        return None
    return int(ent["traffic_bytes"]) if h.hexdigest() == ent["sources_sha256"] else None


def gated_variant_bench(dev, Model):
    """bs1 decode and a 1 x 1024 prefill of the gated-attention variant at the
    0.6B shape's widths (8 query / 2 KV heads of width 256, RoPE on 64 dims,
    sigmoid output gate), bf16 weights and KV."""
    import numpy as np
    import torch

    import synth
    gs = synth.GATED_0P6B
    gw = synth.make_weights(gs, 0)
    gm = Model(gs, gw, max_seqs=1, max_ctx=1024)
    del gw
    prompt = synth.tokens(110, gs.vocab, 512)
    tok = torch.from_numpy(prompt[None, :].astype(np.int32)).to(dev)
    lg = gm.prefill(tok, [0])
    nxt = torch.argmax(lg, dim=1).to(torch.int32)
    P, steps = len(prompt), 64
    for k in range(4):
        gm.decode_step(nxt, [P + k], [0], next_ids=nxt)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        gm.decode_step(nxt, [P + 4 + k], [0], next_ids=nxt)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    ctx = P + 4 + steps // 2
    wbytes = 2 * (gs.vocab * gs.hidden + gs.n_layers * (gs.q_proj_width * gs.hidden + 2 * gs.kv_width * gs.hidden +
                                                      gs.hidden * gs.q_width + 3 * gs.ffn * gs.hidden))
    kvbytes = gs.n_layers * 2 * gs.kv_width * 2 * ctx
    ptok = torch.from_numpy(synth.tokens(111, gs.vocab, (1, 1024)).astype(np.int32)).to(dev)
    gm.prefill(ptok, [0])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    gm.prefill(ptok, [0])
    torch.cuda.synchronize()
    pdt = time.perf_counter() - t0
    gm.close()
    return {"workload": "gated-attention variant, 28 layers, hidden 1024, 8 query / 2 KV heads x 256 "
                        "(RoPE on 64 dims), ffn 3072, vocab 151936, bf16; bs1 decode from a 512-token prompt",
            "decode_tok_s": round(1.0 / dt, 1), "ms_per_step": round(dt * 1e3, 4),
            "decode_hbm_frac_step": round((wbytes + kvbytes) / dt / 8e12, 4),
            "prefill_1x1024_tok_s": round(1024 / pdt, 1)}


def lowbit_weights_bench(dev, Model, shape, w, ref_model, prompt, fmt):
    """The low-bit decision's measurements ("Milestones", M7) for one weight
    format -- "i8_row" (int8 codes) or "f8_row" (e4m3 codes; norm outputs
    quantized per row, Q/K/V and gate/up on fp8 matrix instructions at prefill
    sizes) -- with one scale per output row, quantized by the library from the
    same bf16 weights, against the bf16 model: speed (bs1 decode, 4 x 4096
    prefill, per-kernel times), weight memory, and quality (logits of both
    models on one teacher-forced token stream, the bf16 model choosing the
    tokens)."""
    import dataclasses

    import numpy as np
    import torch

    import synth
    qs = dataclasses.replace(shape, weight_format=fmt)
    qm = Model(qs, w, max_seqs=4, max_ctx=4096)
    H, L, I, V = shape.hidden, shape.n_layers, shape.ffn, shape.vocab
    rows_cols = [(shape.q_width + 2 * shape.kv_width, H), (H, shape.q_width), (2 * I, H), (H, I)]
    bf16_w = 2 * (V * H + L * sum(r * c for r, c in rows_cols))
    code_w = V * H + 4 * V + L * sum(r * c + 4 * r for r, c in rows_cols)
    P = len(prompt)
    tok = torch.from_numpy(prompt[None, :].astype(np.int32)).to(dev)
    nxt = torch.empty((1,), dtype=torch.int32, device=dev)
    # speed: bs1 decode from the same 512-token prompt
    lg = qm.prefill(tok, [1])
    nxt.copy_(torch.argmax(lg, dim=1).to(torch.int32))
    for k in range(8):
        qm.decode_step(nxt, [P + k], [1], next_ids=nxt)
    qm.prefill(tok, [0])
    torch.cuda.synchronize()
    steps = 128
    t0 = time.perf_counter()
    for k in range(steps):
        qm.decode_step(nxt, [P + k], [0], next_ids=nxt)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    ctx = P + (steps + 1) / 2.0
    other = L * (2 * H + 2 * shape.head_dim) * 2 + 2 * H * 2       # norm weights, embedding row
    step_bytes = code_w + other + L * 2 * shape.kv_width * 2 * ctx
    per_launch = {lab: qm.kernel_bench(lab, reps=20, slot=2, position=P + steps // 2)
                  for lab in ("qkv", "o_proj", "gate_up", "down", "head")}
    # speed: 4 x 4096 prefill, and its GEMMs one by one
    pw = synth.workload("prefill_0p6b_4x4096")
    ptok = torch.from_numpy(np.stack(pw.prompts).astype(np.int32)).to(dev)
    plg = torch.empty((4, V), dtype=torch.float32, device=dev)
    qm.prefill(ptok, [0, 1, 2, 3], logits=plg)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    qm.prefill(ptok, [0, 1, 2, 3], logits=plg)
    torch.cuda.synchronize()
    pdt = time.perf_counter() - t0
    qm.timing(True)
    qm.prefill(ptok, [0, 1, 2, 3], logits=plg)
    torch.cuda.synchronize()
    gemms = {}
    for lab in ("wconv", "norm", "qkv", "o_proj", "gate_up", "down"):
        ms, n = qm.timing_read(lab)
        if n:
            gemms[lab] = round(ms, 3)
    qm.timing(False)
    fp8_mm = ("qkv", "gate_up") if fmt == "f8_row" else ()
    frac = {}
    for lab in ("qkv", "o_proj", "gate_up", "down"):
        if lab in gemms:
            peak = MFMA_FP8_PEAK if lab in fp8_mm else MFMA_BF16_PEAK
            fl = L * prefill_label_flops(shape, lab, 4, 4096)
            frac[lab] = {"tflop_s": round(fl / (gemms[lab] / 1e3) / 1e12, 1),
                         "peak": "fp8 5.0 PFLOP/s" if lab in fp8_mm else "bf16 2.5 PFLOP/s",
                         "frac": round(fl / (gemms[lab] / 1e3) / peak, 4)}
    # quality: one token stream through both models
    ql = qm.prefill(tok, [0])
    rl = ref_model.prefill(tok, [3])
    a, b = torch.empty((1, V), device=dev), torch.empty((1, V), device=dev)
    diffs, rel, agree = [], [], 0
    cur_q, cur_r = ql.clone(), rl.clone()
    n_q = 64
    for k in range(n_q):
        d = (cur_q - cur_r).abs().max().item()
        diffs.append(d)
        rel.append(((cur_q - cur_r).pow(2).mean().sqrt() / cur_r.pow(2).mean().sqrt()).item())
        ti = int(torch.argmax(cur_r[0]).item())
        agree += int(torch.argmax(cur_q[0]).item()) == ti
        t = torch.tensor([ti], dtype=torch.int32, device=dev)
        qm.decode_step(t, [P + k], [0], logits=a)
        ref_model.decode_step(t, [P + k], [3], logits=b)
        cur_q, cur_r = a.clone(), b.clone()
    qm.close()
    code = "int8" if fmt == "i8_row" else "e4m3"
    res = {"workload": f"0.6B shape, {code} codes + one fp32 scale per output row for every matrix (tied "
                       "embedding / head included), bf16 KV; bs1 decode from the same 512-token prompt; "
                       "4 x 4096 prefill",
           "decode_tok_s": round(1.0 / dt, 1), "ms_per_step": round(dt * 1e3, 4),
           "decode_hbm_frac_step": round(step_bytes / dt / HBM_PEAK, 4),
           "decode_us_per_launch": {k: round(v, 3) for k, v in per_launch.items()},
           "prefill_4x4096_tok_s": round(4 * 4096 / pdt, 1), "prefill_ms": round(pdt * 1e3, 2),
           "prefill_kernel_ms_per_pass": gemms, "prefill_gemm_mfma": frac,
           "weight_bytes": {code: int(code_w), "bf16": int(bf16_w)},
           "quality_vs_bf16": {"positions": n_q, "greedy_agree": agree,
                               "max_abs_logit_diff": round(max(diffs), 4),
                               "mean_max_abs_logit_diff": round(float(np.mean(diffs)), 4),
                               "mean_rel_rms_logit_diff": round(float(np.mean(rel)), 5)}}
    if fmt == "f8_row":
        # the same prefill with the fp8 products on widened (bf16) weights instead
        os.environ["FS_PREFILL_F8_MFMA"] = "0"
        try:
            wm = Model(qs, w, max_seqs=4, max_ctx=4096)
        finally:
            del os.environ["FS_PREFILL_F8_MFMA"]
        wm.prefill(ptok, [0, 1, 2, 3], logits=plg)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        wm.prefill(ptok, [0, 1, 2, 3], logits=plg)
        torch.cuda.synchronize()
        res["prefill_4x4096_tok_s_widened_bf16"] = round(4 * 4096 / (time.perf_counter() - t0), 1)
        wm.close()
    return res


def scorer_bench(dev, model, shape):
    """The 6-token scorer on the bs1 model: latency of one fs_prefill (last-token
    logits) and the weight bytes it must move over that time."""
    import numpy as np
    import torch

    import synth
    wl = synth.workload("scorer_0p6b")
    tok = torch.from_numpy(wl.prompts[0][None, :].astype(np.int32)).to(dev)
    lg = torch.empty((1, shape.vocab), dtype=torch.float32, device=dev)
    for _ in range(3):
        model.prefill(tok, [3], logits=lg)
    torch.cuda.synchronize()
    ts = []
    for _ in range(20):
        t0 = time.perf_counter()
        model.prefill(tok, [3], logits=lg)
        torch.cuda.synchronize()
        ts.append(time.perf_counter() - t0)
    t = float(np.median(ts))
    model.timing(True)
    model.prefill(tok, [3], logits=lg)
    torch.cuda.synchronize()
    per = {}
    for lab in ("embed", "norm", "qkv", "rope_kv", "attn", "o_proj", "gate_up", "down", "head"):
        ms, n = model.timing_read(lab)
        if n:
            per[lab] = round(ms, 4)
    model.timing(False)
    return {"workload": "scorer_0p6b: one 6-token prompt, last-token logits (fs_prefill)",
            "latency_ms_p50": round(t * 1e3, 4), "hbm_frac": round(decode_bytes_per_step(shape, 6) / t / HBM_PEAK, 4),
            "kernel_ms": per}


def batched_decode_bench(dev, Model, w, argmax):
    """64 sequences of ragged context (uniform in [256, 4096]), prefilled one by
    one (untimed), then decode steps with B = 64 and next IDs fed back on the
    device: 2 warmup steps, then the workload's 128 timed steps."""
    import numpy as np
    import torch

    import synth
    wl = synth.workload("decode_0p6b_bs64")
    shape = wl.shape
    B, steps, warm = wl.batch, wl.decode_steps, 2
    lens = np.array([len(p) for p in wl.prompts])
    m = Model(shape, w, max_seqs=B, max_ctx=int(lens.max()) + warm + steps + 1)
    nxt = torch.empty((B,), dtype=torch.int32, device=dev)
    for i, p in enumerate(wl.prompts):
        lg = m.prefill(torch.from_numpy(p[None, :].astype(np.int32)).to(dev), [i])
        argmax(lg, out=nxt[i:i + 1])
    slots = list(range(B))
    for k in range(warm):
        m.decode_step(nxt, [int(n) + k for n in lens], slots, next_ids=nxt)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(warm, warm + steps):
        m.decode_step(nxt, [int(n) + k for n in lens], slots, next_ids=nxt)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    # one more step under the per-launch event hook: time per kernel class
    m.timing(True)
    m.decode_step(nxt, [int(n) + warm + steps for n in lens], slots, next_ids=nxt)
    torch.cuda.synchronize()
    per = {}
    for lab in ("embed", "norm", "qkv", "attn", "combine", "o_proj", "gate_up", "down", "head", "argmax"):
        ms, n = m.timing_read(lab)
        if n:
            per[lab] = round(ms, 4)
    m.timing(False)
    m.close()
    kv_per_pos = shape.n_layers * 2 * shape.kv_width * 2
    wbytes = decode_bytes_per_step(shape, 0)
    ctx_sum = float(np.sum(lens)) * steps + B * sum(warm + k + 1 for k in range(steps))
    step_bytes = wbytes + kv_per_pos * ctx_sum / steps + B * kv_per_pos
    return {"workload": "decode_0p6b_bs64: 64 sequences, contexts uniform in [256, 4096], greedy, next IDs on "
                        "device; 2 warmup steps then 128 timed",
            "tok_s": round(B * steps / dt, 1), "ms_per_step": round(dt * 1e3 / steps, 3),
            "hbm_frac_step": round(step_bytes / (dt / steps) / HBM_PEAK, 4),
            "bytes_per_step": int(step_bytes), "kernel_ms_per_step": per}


def tiny_bench(dev, Model, argmax):
    """The tiny fp32 model: 16-token prompt, 16 greedy decode steps (launch-bound)."""
    import numpy as np
    import torch

    import synth
    wl = synth.workload("tiny_fp32")
    m = Model(wl.shape, synth.make_weights(wl.shape, 0), max_seqs=2, max_ctx=64)
    tok = torch.from_numpy(wl.prompts[0][None, :].astype(np.int32)).to(dev)
    nxt = torch.empty((1,), dtype=torch.int32, device=dev)
    P = tok.shape[1]
    for slot in (1, 0):
        argmax(m.prefill(tok, [slot]), out=nxt)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(wl.decode_steps):
            m.decode_step(nxt, [P + k], [slot], next_ids=nxt)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
    m.close()
    return {"workload": "tiny_fp32: 2 layers, hidden 256, 16-token prompt, 16 greedy decode steps (second run)",
            "decode_tok_s": round(wl.decode_steps / dt, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-steps", type=int, default=48)
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only one 4 x 4096 prefill (for hardware-counter passes) and exit")
    ap.add_argument("--decode-only", action="store_true",
                    help="run only the 512-token prefill and --steps bs1 decode steps (for hardware-counter "
                         "passes) and exit")
    ap.add_argument("--copy-cal", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-MiB device buffer 4 times and exit: the plain copy of known "
                         "size that calibrates the FETCH_SIZE / WRITE_SIZE byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: --gpus must be 1 "
                                   "(sharding across GPUs is not part of this library)"}))
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_cal > 0:
        n = args.copy_cal << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_cal_bytes": n, "copies": 4}), flush=True)
        return

    import synth
    from dense_gqa_transformer_amd.model import Model, argmax

    wl = synth.workload("decode_0p6b_bs1")
    shape = wl.shape
    prompt = wl.prompts[0]
    steps = max(1, min(args.steps, wl.decode_steps))
    w = synth.make_weights(shape, 0)
    model = Model(shape, w, max_seqs=5, max_ctx=4096)
    dev = torch.device("cuda")
    if args.prefill_only:
        pw = synth.workload("prefill_0p6b_4x4096")
        ptok = torch.from_numpy(np.stack(pw.prompts).astype(np.int32)).to(dev)
        logits = torch.empty((4, shape.vocab), dtype=torch.float32, device=dev)
        t0 = time.perf_counter()
        model.prefill(ptok, [0, 1, 2, 3], logits=logits)
        torch.cuda.synchronize()
        print(json.dumps({"prefill_only_ms": round((time.perf_counter() - t0) * 1e3, 3)}), flush=True)
        return
    tok = torch.from_numpy(prompt[None, :].astype(np.int32)).to(dev)
    nxt = torch.empty((1,), dtype=torch.int32, device=dev)
    P = len(prompt)
    if args.decode_only:
        argmax(model.prefill(tok, [0]), out=nxt)
        t0 = time.perf_counter()
        for k in range(steps):
            model.decode_step(nxt, [P + k], [0], next_ids=nxt)
        torch.cuda.synchronize()
        print(json.dumps({"decode_only_steps": steps, "ms": round((time.perf_counter() - t0) * 1e3, 3)}), flush=True)
        return

    # warmup on slot 1 (also captures the decode graphs used below)
    lg = model.prefill(tok, [1])
    argmax(lg, out=nxt)
    for k in range(min(args.warmup, wl.decode_steps)):
        model.decode_step(nxt, [P + k], [1], next_ids=nxt)
    torch.cuda.synchronize()

    # timed: `steps` decode steps on slot 0 after an untimed prefill
    lg = model.prefill(tok, [0])
    argmax(lg, out=nxt)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        model.decode_step(nxt, [P + k], [0], next_ids=nxt)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_step = dt * 1e3 / steps
    ctx_avg = P + (steps + 1) / 2.0
    hbm_frac = decode_bytes_per_step(shape, ctx_avg) / (dt / steps) / HBM_PEAK

    # per-step latency distribution: the same steps again on slot 2, with an
    # event after each step on the stream the steps run on
    lg = model.prefill(tok, [2])
    argmax(lg, out=nxt)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for k in range(steps):
        model.decode_step(nxt, [P + k], [2], next_ids=nxt)
        evs[k + 1].record()
    torch.cuda.synchronize()
    step_ms = np.array([evs[k].elapsed_time(evs[k + 1]) for k in range(steps)])

    # per-launch duration of each decode kernel class, replayed back to back in
    # a graph over the 28 layers' own weights (HIP events on the library's stream)
    # (the merge launch only where the step at this context runs the split form)
    model.timing(True)
    model.decode_step(nxt, [P + steps], [2], next_ids=nxt)
    torch.cuda.synchronize()
    merges = model.timing_read("combine")[1]
    model.timing(False)
    per_launch = {}
    for lab in ("qkv", "attn", "combine", "o_proj", "gate_up", "down", "head"):
        if lab == "combine" and not merges:
            continue
        per_launch[lab] = model.kernel_bench(lab, reps=20, slot=4, position=P + steps // 2)
    launches = {lab: (1 if lab == "head" else shape.n_layers) for lab in per_launch}
    dom = max(per_launch, key=lambda k: per_launch[k] * launches[k])
    avg_s = per_launch[dom] * 1e-6
    bytes_launch = decode_label_bytes(shape, dom, P + steps // 2 + 1)
    achieved = bytes_launch / avg_s
    out = {
        "metric": "decode tok/s @bs1 (0.6B shape, bf16 weights + bf16 KV cache)",
        "value": round(steps / dt, 2),
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
        "config": {"workload": "decode_0p6b_bs1: 28-layer 0.6B-shape bf16 model, 512-token prompt, "
                               "greedy batch-1 decode steps from position 512",
                   "global_batch": 1, "seq_len": P + steps, "parallelism": "none"},
        "decode_hbm_frac_step": round(hbm_frac, 4),
        "decode_step_ms_p50": round(float(np.percentile(step_ms, 50)), 4),
        "decode_step_ms_p99": round(float(np.percentile(step_ms, 99)), 4),
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved / 1e9, 1),
                     "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": round(achieved / HBM_PEAK, 4),
                     "traffic": measured_traffic("decode." + dom), "avg_launch_us": round(avg_s * 1e6, 3),
                     "bytes_per_launch": int(bytes_launch)},
        "decode_us_per_launch": {k: round(v, 3) for k, v in per_launch.items()},
        # the same graph-replayed chain with a kernel that does nothing: the
        # dispatch cost each of the step's dependent launches pays
        "decode_launch_floor_us": round(model.kernel_bench("empty", reps=20, slot=4, position=P + steps // 2), 3),
    }
    # the matrix unit on register operands only: the bf16 throughput the MFMA
    # kernels could reach at best (for context beside the published peak)
    mus = model.kernel_bench("mfma", reps=3, slot=4, position=P)
    mflops = 2 * 32 * 32 * 16 * 4 * 2048 * 256 * 8
    out["mfma_bf16_register_only"] = {"tflop_s": round(mflops / (mus * 1e-6) / 1e12, 1),
                                      "frac_of_peak": round(mflops / (mus * 1e-6) / MFMA_BF16_PEAK, 4),
                                      "us_per_launch": round(mus, 2)}
    # a plain streaming read of the stored matrices (bf16): the HBM rate a
    # read-only kernel reaches, beside the published 8 TB/s
    hus = model.kernel_bench("hbm", reps=3, slot=4, position=P)
    wbytes = 2 * (shape.vocab * shape.hidden +
                  shape.n_layers * sum(int(np.prod(s)) for s in shape.layer_shapes().values() if len(s) == 2))
    out["hbm_read_stream"] = {"gb_s": round(wbytes / (hus * 1e-6) / 1e9, 1),
                              "frac_of_peak": round(wbytes / (hus * 1e-6) / HBM_PEAK, 4),
                              "bytes_per_launch": int(wbytes), "us_per_launch": round(hus, 2)}

    if not args.no_prefill:
        pw = synth.workload("prefill_0p6b_4x4096")
        ptok = torch.from_numpy(np.stack(pw.prompts).astype(np.int32)).to(dev)
        logits = torch.empty((4, shape.vocab), dtype=torch.float32, device=dev)
        model.prefill(ptok, [0, 1, 2, 3], logits=logits)
        torch.cuda.synchronize()
        reps = 2
        t0 = time.perf_counter()
        for _ in range(reps):
            model.prefill(ptok, [0, 1, 2, 3], logits=logits)
        torch.cuda.synchronize()
        pdt = (time.perf_counter() - t0) / reps
        model.timing(True)
        model.prefill(ptok, [0, 1, 2, 3], logits=logits)
        torch.cuda.synchronize()
        pper = {}
        for lab in ("embed", "norm", "qkv", "rope_kv", "attn", "o_proj", "gate_up", "down", "head"):
            ms, n = model.timing_read(lab)
            if n:
                pper[lab] = (ms, n)
        model.timing(False)
        mf = {k: v for k, v in pper.items() if prefill_label_flops(shape, k, 4, 4096)}
        pdom = max(mf, key=lambda k: mf[k][0])
        pavg = mf[pdom][0] / mf[pdom][1] / 1e3
        pach = prefill_label_flops(shape, pdom, 4, 4096) / pavg
        gemm_time = sum(pper[k][0] for k in ("qkv", "o_proj", "gate_up", "down") if k in pper) / 1e3
        gemm_flops = shape.n_layers * sum(prefill_label_flops(shape, k, 4, 4096)
                                          for k in ("qkv", "o_proj", "gate_up", "down"))
        out["prefill"] = {
            "workload": "prefill_0p6b_4x4096: 4 x 4096 uniform-random tokens, KV for all positions, "
                        "last-token logits",
            "tok_s": round(4 * 4096 / pdt, 1), "ms": round(pdt * 1e3, 3),
            "mfma_frac_pass": round(prefill_flops(shape, 4, 4096) / pdt / MFMA_BF16_PEAK, 4),
            "mfma_frac_gemms": round(gemm_flops / gemm_time / MFMA_BF16_PEAK, 4),
            "roofline": {"bound": "mfma", "kernel": pdom, "achieved": round(pach / 1e12, 1),
                         "peak": MFMA_BF16_PEAK / 1e12, "unit": "TFLOP/s", "frac": round(pach / MFMA_BF16_PEAK, 4),
                         "traffic": measured_traffic("prefill." + pdom), "avg_launch_us": round(pavg * 1e6, 1)},
            "kernel_ms_per_pass": {k: round(v[0], 3) for k, v in pper.items()},
            # per projection: algorithmic flops over its time in the pass (Q/K/V and gate/up
            # also run the fp8 remainder pass and their fused epilogues inside that time)
            "gemm_mfma_frac": {k: round(shape.n_layers * prefill_label_flops(shape, k, 4, 4096)
                                        / (pper[k][0] / 1e3) / MFMA_BF16_PEAK, 4)
                               for k in ("qkv", "o_proj", "gate_up", "down") if k in pper},
        }

    # the library's generation loop on the same prompt (greedy, one host check per token)
    gen_n = 64
    model.generate(prompt, 4, slot=2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    gids, gwhy = model.generate(prompt, gen_n, slot=2)
    gdt = time.perf_counter() - t0
    out["generate"] = {"workload": f"fs_generate, greedy, {P}-token prompt, {gen_n} new tokens (prefill included)",
                       "tokens": len(gids), "stop_reason": gwhy, "ms": round(gdt * 1e3, 2),
                       "tok_s_incl_prefill": round(len(gids) / gdt, 1)}

    out["scorer"] = scorer_bench(dev, model, shape)
    out["batched_decode"] = batched_decode_bench(dev, Model, w, argmax)
    out["tiny"] = tiny_bench(dev, Model, argmax)
    out["gated_variant"] = gated_variant_bench(dev, Model)
    out["int8_weights"] = lowbit_weights_bench(dev, Model, shape, w, model, prompt, "i8_row")
    out["fp8_weights"] = lowbit_weights_bench(dev, Model, shape, w, model, prompt, "f8_row")

    # seeded sampling of one lm_head row (temperature -> top-k -> top-p -> draw)
    srow = torch.from_numpy(synth.logit_rows(900, 1, shape.vocab)).to(dev)
    su = torch.from_numpy(synth.uniforms(901, 1)).to(dev)
    sout = torch.empty((1,), dtype=torch.int32, device=dev)
    samp = {}
    for name, (T, k, p) in {"t0.8_k50_p0.9": (0.8, 50, 0.9), "t1.0_k0_p0.95": (1.0, 0, 0.95)}.items():
        for _ in range(5):
            model.sample(srow, T, k, p, su, out=sout)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(50):
            model.sample(srow, T, k, p, su, out=sout)
        e1.record()
        torch.cuda.synchronize()
        us_call = e0.elapsed_time(e1) / 50 * 1e3
        passes = 8 if p < 1.0 else 6          # row reads: 3 count + 1-3 mass + kept-sum passes, + final block
        samp[name] = {"us_per_call": round(us_call, 2), "row_bytes_read": passes * shape.vocab * 4}
    out["sampling"] = {"workload": f"one fp32 logits row of {shape.vocab}, batch 1", **samp}

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, w, args.cpu_steps)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
