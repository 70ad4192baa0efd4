"""CPU oracle for the dense GQA decoder forward pass (test infrastructure).

This file is test infrastructure.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import it; the GPU library never does,
and the two share no code.  It is plain NumPy, written for a reader to check
against the pages by eye, in float64 by default (``dtype`` may select float32,
the precision of the CPU oracle described in "Failed Star (fs)", section
"Status").

What it computes, and where the pages say so:

* the pipeline ``ids[S] -> embedding[S,H] -> N blocks[S,H] -> final norm ->
  last row -> logits[V]``: "Coming back to Failed Star", section "Second
  sitting: connect the story to the code" (the data-flow figure), and
  "Milestones", section M2 (embeddings, blocks of RMSNorm, RoPE, attention,
  SwiGLU, final norm, logits);
* a block is two residual halves, attention then FFN, and only the final row
  is projected to ``[V]``: "Coming back to Failed Star", section "First
  sitting" (checkpoint of item 4);
* a Linear weight is stored ``[out, in]`` and maps ``[S, in]`` to ``[S, out]``:
  same page, "First sitting", item 3;
* the head is tied to the embedding: "Failed Star (fs)", section "Status", and
  "Coming back to Failed Star", section "Where we actually are" (M1 row);
* grouped-query attention, RoPE, SwiGLU, RMSNorm: "Failed Star (fs)", section
  "How it's built"; 16 query heads of width 128 give 2048, not H: "Coming back
  to Failed Star", section "Second sitting";
* the KV-cached decode step does one-token work and agrees with the uncached
  pass: "Milestones", section M4;
* greedy selection is argmax over finite logits, lowest ID winning an exact
  tie: "Coming back to Failed Star", section "Next: one complete deterministic
  generation arc".

Readings where the pages are silent (each also listed in the design notes):
RMSNorm is ``x / sqrt(mean(x^2) + eps) * g``; each query and key head is
RMSNorm-ed over head_dim with one shared weight vector before RoPE (the Qwen3
layout); RoPE rotates the pairs (i, i + d/2) by ``p * theta^(-2i/d)``; the
attention scale is ``1/sqrt(head_dim)``; query head h reads KV head
``h // (n_heads / n_kv_heads)``; the mask is causal and includes the diagonal;
``silu(z) = z / (1 + exp(-z))``; a row with no finite logit selects -1.
The gated-attention variant ("ferrite", section "What it does": gated
attention output, partial rotate-half RoPE on 64 of 256 dims, and the fix of
its q/gate split to the per-head interleaved layout): wq rows hold, head by
head, the query then the gate; the head's attention output is multiplied by
``sigmoid(gate)`` before the output projection; only the first ``rope_dim``
dims of q and k rotate, with angles ``p * theta^(-2i/rope_dim)``.

Every function is pinned by tests in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import numpy as np


# --------------------------------------------------------------------------
# elementary operations
# --------------------------------------------------------------------------

def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * g.

    Named in "Failed Star (fs)", section "How it's built"; formula is the
    standard one (eps inside the square root, mean over the normalised axis).
    """
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope_cos_sin(positions: np.ndarray, head_dim: int, theta: float, dtype):
    """cos/sin of the rotary angles ``p * theta^(-2i/d)``, i < d/2.

    Angles are formed in float64 and the results cast to ``dtype``.
    """
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def rope(x: np.ndarray, positions: np.ndarray, theta: float, rot_dim: Optional[int] = None) -> np.ndarray:
    """Rotate-half RoPE on ``x[S, heads, d]`` at ``positions[S]``.

    The pair (x_i, x_{i+r/2}) is rotated by angle p*theta^(-2i/r):
    (x_i cos a - x_{i+r/2} sin a,  x_{i+r/2} cos a + x_i sin a), for the first
    ``r = rot_dim`` dims (default all of d); dims r..d-1 pass through.
    RoPE is named in "Failed Star (fs)", section "How it's built"; the
    rotate-half pairing, and rotating only 64 of 256 head dims, are what
    "ferrite", section "What it does", describes for its attention blocks.
    """
    d = x.shape[-1]
    if rot_dim is not None and rot_dim != d:
        return np.concatenate([rope(x[..., :rot_dim], positions, theta), x[..., rot_dim:]], axis=-1)
    half = d // 2
    cos, sin = rope_cos_sin(positions, d, theta, x.dtype)
    cos = cos[:, None, :]
    sin = sin[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def sigmoid(z: np.ndarray) -> np.ndarray:
    """Logistic function 1 / (1 + e^-z), the output gate of gated attention."""
    return 1.0 / (1.0 + np.exp(-z))


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU, the gate of SwiGLU: z / (1 + e^-z)."""
    return z / (1.0 + np.exp(-z))


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Max-subtracted softmax over the last axis; -inf entries get weight 0."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def gqa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                  q_pos: np.ndarray) -> np.ndarray:
    """Causal grouped-query attention.

    q: [S, nq, d] queries at absolute positions q_pos[S];
    k, v: [n, nkv, d] keys/values at positions 0..n-1.
    Query head h uses KV head h // (nq/nkv); query at position p sees keys
    0..p inclusive; scores are scaled by 1/sqrt(d).
    """
    S, nq, d = q.shape
    n, nkv, _ = k.shape
    rep = nq // nkv
    out = np.zeros((S, nq, d), dtype=q.dtype)
    key_pos = np.arange(n)
    masked = key_pos[None, :] > np.asarray(q_pos)[:, None]      # [S, n]
    scale = 1.0 / math.sqrt(d)
    for h in range(nq):
        j = h // rep
        scores = (q[:, h, :] @ k[:, j, :].T) * scale            # [S, n]
        scores = np.where(masked, -np.inf, scores)
        out[:, h, :] = softmax_rows(scores) @ v[:, j, :]
    return out


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = x W^T with W stored [out, in]: maps [S, in] to [S, out]."""
    return x @ w.T


# --------------------------------------------------------------------------
# the model
# --------------------------------------------------------------------------

class Oracle:
    """The forward pass of one model, uncached and KV-cached.

    ``weights`` is the dict from ``synth.make_weights`` (float32 arrays,
    ``[out, in]``); ``shape`` a ``synth.ModelShape``.  All arithmetic runs in
    ``dtype`` (float64 unless asked otherwise).  bf16 weights arrive already
    widened exactly to float32, so no rounding happens on this side.
    """

    def __init__(self, shape, weights: dict, dtype=np.float64, quantize_norm_outputs=None, kv_round=None):
        self.shape = shape
        self.dtype = np.dtype(dtype)
        # optional rule applied to every RMSNorm output that feeds a projection
        # (Q/K/V, gate/up, the head): the fp8 option's activation quantization
        # (oracle/fp8.py); None leaves them exact
        self.qn = quantize_norm_outputs
        # optional rounding of K (normed, rotated) and V as they enter the
        # cache, for a cache kept in a narrower type (a bf16 cache stores them
        # rounded to bf16); None keeps them exact
        self.kv_round = kv_round
        c = lambda a: np.asarray(a, dtype=self.dtype)
        self.embed = c(weights["embed"])
        self.final_norm = c(weights["final_norm"])
        self.layers = [{k: c(v) for k, v in lw.items()} for lw in weights["layers"]]
        # per-slot KV cache: slot -> list over layers of (K[n,nkv,d], V[n,nkv,d])
        self.cache: Dict[int, List[list]] = {}

    # one transformer block over new rows x[s, H] at positions pos[s],
    # attending to past keys/values (k_past, v_past) of positions 0..n0-1.
    def _block(self, li: int, x: np.ndarray, pos: np.ndarray,
               k_past: Optional[np.ndarray], v_past: Optional[np.ndarray],
               dump: Optional[dict] = None):
        sh = self.shape
        w = self.layers[li]
        s = x.shape[0]
        # attention half
        xn = rms_norm(x, w["attn_norm"], sh.rms_eps)
        if self.qn is not None:
            xn = np.asarray(self.qn(xn), dtype=self.dtype)
        qp = linear(xn, w["wq"])
        gate = None
        if getattr(sh, "attn_gate", False):
            # per-head interleaved [query | gate] rows ("ferrite", What it does)
            qg = qp.reshape(s, sh.n_heads, 2, sh.head_dim)
            q, gate = qg[:, :, 0, :], qg[:, :, 1, :]
        else:
            q = qp.reshape(s, sh.n_heads, sh.head_dim)
        k = linear(xn, w["wk"]).reshape(s, sh.n_kv_heads, sh.head_dim)
        v = linear(xn, w["wv"]).reshape(s, sh.n_kv_heads, sh.head_dim)
        rot = getattr(sh, "rope_dim", 0) or sh.head_dim
        q = rope(rms_norm(q, w["q_norm"], sh.rms_eps), pos, sh.rope_theta, rot)
        k = rope(rms_norm(k, w["k_norm"], sh.rms_eps), pos, sh.rope_theta, rot)
        if self.kv_round is not None:
            k = np.asarray(self.kv_round(k), dtype=self.dtype)
            v = np.asarray(self.kv_round(v), dtype=self.dtype)
        if k_past is not None and k_past.shape[0] > 0:
            k_all = np.concatenate([k_past, k], axis=0)
            v_all = np.concatenate([v_past, v], axis=0)
        else:
            k_all, v_all = k, v
        a = gqa_attention(q, k_all, v_all, pos)
        if gate is not None:
            a = a * sigmoid(gate)
        a = a.reshape(s, sh.q_width)
        x = x + linear(a, w["wo"])
        if dump is not None:
            dump[f"layer{li}.q"] = q
            dump[f"layer{li}.k"] = k
            dump[f"layer{li}.v"] = v
            dump[f"layer{li}.attn"] = a
            dump[f"layer{li}.x_mid"] = x
        # FFN half
        xn = rms_norm(x, w["mlp_norm"], sh.rms_eps)
        if self.qn is not None:
            xn = np.asarray(self.qn(xn), dtype=self.dtype)
        hmid = silu(linear(xn, w["w_gate"])) * linear(xn, w["w_up"])
        x = x + linear(hmid, w["w_down"])
        if dump is not None:
            dump[f"layer{li}.out"] = x
        return x, k_all, v_all

    def _head(self, x_last: np.ndarray) -> np.ndarray:
        """Final RMSNorm of the last row(s), then the tied head E . h."""
        hn = rms_norm(x_last, self.final_norm, self.shape.rms_eps)
        if self.qn is not None:
            hn = np.asarray(self.qn(hn), dtype=self.dtype)
        return hn @ self.embed.T

    # ---------------------------------------------------------------- uncached
    def forward(self, token_ids, dump: Optional[dict] = None,
                all_rows: bool = False) -> np.ndarray:
        """Uncached scorer: logits of the last row (or of every row).

        Positions start at 0 with no implicit BOS ("Coming back to Failed
        Star", section "Next": raw input, no automatic BOS).
        """
        ids = np.asarray(token_ids, dtype=np.int64)
        if ids.ndim != 1 or ids.size == 0:
            raise ValueError("need a non-empty 1-D token sequence")
        x = self.embed[ids]
        pos = np.arange(ids.size)
        if dump is not None:
            dump["embed"] = x
        for li in range(self.shape.n_layers):
            x, _, _ = self._block(li, x, pos, None, None, dump)
        if dump is not None:
            dump["final"] = x
        if all_rows:
            return self._head(x)
        return self._head(x[-1])

    # ------------------------------------------------------------------ cached
    def prefill(self, slot: int, token_ids) -> np.ndarray:
        """Uncached pass that also keeps each layer's K (normed, rotated) and V.

        Resets ``slot`` and returns the last-token logits.
        """
        ids = np.asarray(token_ids, dtype=np.int64)
        if ids.ndim != 1 or ids.size == 0:
            raise ValueError("need a non-empty 1-D token sequence")
        x = self.embed[ids]
        pos = np.arange(ids.size)
        kv = []
        for li in range(self.shape.n_layers):
            x, k_all, v_all = self._block(li, x, pos, None, None)
            kv.append([k_all, v_all])
        self.cache[slot] = kv
        return self._head(x[-1])

    def decode_step(self, slot: int, token_id: int, position: int,
                    dump: Optional[dict] = None) -> np.ndarray:
        """One-token step: append K/V at ``position`` and attend over 0..position."""
        kv = self.cache.setdefault(slot, [[None, None] for _ in range(self.shape.n_layers)])
        have = 0 if kv[0][0] is None else kv[0][0].shape[0]
        if position != have:
            raise ValueError(f"position {position} != cached length {have}")
        x = self.embed[np.array([token_id], dtype=np.int64)]
        pos = np.array([position])
        for li in range(self.shape.n_layers):
            x, k_all, v_all = self._block(li, x, pos, kv[li][0], kv[li][1], dump)
            kv[li][0], kv[li][1] = k_all, v_all
        return self._head(x[-1])

    def cached_len(self, slot: int) -> int:
        kv = self.cache.get(slot)
        return 0 if kv is None or kv[0][0] is None else kv[0][0].shape[0]


# --------------------------------------------------------------------------
# selection
# --------------------------------------------------------------------------

def greedy_argmax(logits: np.ndarray) -> int:
    """Argmax over finite entries; the lowest ID wins an exact tie; -1 if none.

    "Coming back to Failed Star", section "Next: one complete deterministic
    generation arc" (Selection); the -1 for a row with no finite entry is a
    reading, the pages leave that case open.
    """
    best = -1
    best_v = None
    for i, v in enumerate(np.asarray(logits).tolist()):
        if not math.isfinite(v):
            continue
        if best_v is None or v > best_v:
            best, best_v = i, v
    return best


def greedy_argmax_fast(logits: np.ndarray) -> int:
    """Vectorised form of ``greedy_argmax`` (same rule) for large rows."""
    a = np.asarray(logits)
    fin = np.isfinite(a)
    if not fin.any():
        return -1
    m = a[fin].max()
    return int(np.flatnonzero(fin & (a == m))[0])


def top_k(logits: np.ndarray, k: int) -> np.ndarray:
    """IDs of the k largest finite logits, by logit descending then ID ascending."""
    a = np.asarray(logits, dtype=np.float64)
    ids = np.flatnonzero(np.isfinite(a))
    order = np.lexsort((ids, -a[ids]))
    return ids[order[:k]]


def top2_gap(logits: np.ndarray) -> float:
    """Gap between the largest and second-largest finite logits."""
    a = np.sort(np.asarray(logits, dtype=np.float64)[np.isfinite(logits)])
    return float(a[-1] - a[-2]) if a.size >= 2 else math.inf


def param_count(shape) -> int:
    """Logical parameters with the tied head counted once."""
    per_layer = sum(int(np.prod(s)) for s in shape.layer_shapes().values())
    return shape.vocab * shape.hidden + shape.n_layers * per_layer + shape.hidden


def tensor_count(shape) -> int:
    """Tensors in the layout: embed + 11 per layer + final norm (tied head)."""
    return 2 + 11 * shape.n_layers
