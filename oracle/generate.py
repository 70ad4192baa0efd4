"""Generation-loop contract (test infrastructure; same rules of use as oracle.py).

The contract the pages ask to settle before the loop is written ("Coming back
to Failed Star", section "Next: one complete deterministic generation arc";
"Milestones", M3): raw token IDs with no implicit BOS and a defined empty
input; a ``max_new_tokens`` budget that may be zero; an explicit EOS ID set
and a record of whether the stop ID is returned; never forwarding beyond the
model's position limit; distinct stop reasons for EOS, budget and context
exhaustion; a defined outcome when the last allowed forward predicts one
more token that no forward can consume; generated IDs as the source of truth.

Readings adopted (each also in the design notes):

* an empty prompt is an error (nothing to condition on); a budget of zero
  returns no tokens, reason BUDGET, without running any forward pass;
* token i is selected from the logits of position S - 1 + i (S = prompt
  length); selection is greedy (the argmax rule) or the sampling chain with
  the i-th caller-supplied uniform;
* order of checks after selecting token i: EOS first (stop, reason EOS; the ID
  is appended only when ``include_stop_id``), then the token is appended and
  the budget checked (reason BUDGET when ``max_new_tokens`` tokens are out),
  then the context: the token would be forwarded at position S + i, which
  needs S + i < max_ctx; otherwise stop with reason CONTEXT, the token kept
  (it was predicted by an allowed forward, it just cannot be consumed);
* a prompt longer than max_ctx is an error; S == max_ctx returns the one
  token its logits predict, with reason CONTEXT.
"""
from __future__ import annotations

from typing import Callable, List, Optional, Sequence, Tuple

import numpy as np

from .oracle import greedy_argmax
from . import sampling as smp

STOP_NONE, STOP_EOS, STOP_BUDGET, STOP_CONTEXT = 0, 1, 2, 3


def generate_loop(prefill: Callable[[Sequence[int]], np.ndarray],
                  decode: Callable[[int, int], np.ndarray],
                  prompt: Sequence[int], max_new_tokens: int, max_ctx: int,
                  eos_ids: Sequence[int] = (), include_stop_id: bool = False,
                  select: Optional[Callable[[np.ndarray, int], int]] = None
                  ) -> Tuple[List[int], int]:
    """The loop with the model passed in as two callables:
    ``prefill(prompt) -> logits of the last prompt position`` and
    ``decode(token, position) -> logits of that position``.
    ``select(logits, i) -> token`` defaults to greedy.  Returns (ids, reason)."""
    S = len(prompt)
    if S == 0:
        raise ValueError("empty prompt")
    if S > max_ctx:
        raise ValueError("prompt longer than max_ctx")
    if max_new_tokens < 0:
        raise ValueError("negative budget")
    if max_new_tokens == 0:
        return [], STOP_BUDGET
    select = select or (lambda lg, i: greedy_argmax(lg))
    eos = set(int(e) for e in eos_ids)
    out: List[int] = []
    logits = prefill(prompt)
    i = 0
    while True:
        tok = int(select(logits, i))
        if tok in eos:
            if include_stop_id:
                out.append(tok)
            return out, STOP_EOS
        out.append(tok)
        if len(out) == max_new_tokens:
            return out, STOP_BUDGET
        pos = S + i
        if pos >= max_ctx:
            return out, STOP_CONTEXT
        logits = decode(tok, pos)
        i += 1


def generate(orc, prompt: Sequence[int], max_new_tokens: int, max_ctx: int,
             eos_ids: Sequence[int] = (), include_stop_id: bool = False, slot: int = 0,
             sampling: Optional[Tuple[float, int, float]] = None,
             uniforms: Optional[Sequence[float]] = None) -> Tuple[List[int], int]:
    """The loop on the oracle's cached forward pass (oracle.Oracle.prefill /
    decode_step).  ``sampling = (temperature, top_k, top_p)`` with one uniform
    per generated token, else greedy."""
    sel = None
    if sampling is not None and sampling[0] > 0.0:
        T, k, p = sampling
        sel = lambda lg, i: smp.sample(lg, T, k, p, float(uniforms[i]))
    return generate_loop(lambda pr: orc.prefill(slot, np.asarray(pr)),
                         lambda tok, pos: orc.decode_step(slot, tok, pos),
                         prompt, max_new_tokens, max_ctx, eos_ids, include_stop_id, sel)
