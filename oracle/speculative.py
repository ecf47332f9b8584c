"""Self-speculative greedy decoding, plain float64 (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path may import or call this module.

Method (the TinyLoop pages): the same weights draft at a shallow loop count
and verify at the full one ("Introduction" page, "What Makes It Different":
draft and verify share the weights, so self-speculative decode needs no
second model; "Current Status" page, speculative and adaptive decode table:
L=2 draft, L=8 verify, zero extra parameters; "Claims & Data Sources":
single-checkpoint decode with draft_loops and verify_loops).

The pages name the method but not its round structure; the reading taken
here is the standard greedy draft-then-verify loop over one shared cache:
  1. from the current token t0 at position p, draft k tokens t1..tk by cached
     greedy decode at draft_loops;
  2. run the verify depth over t0..tk at positions p..p+k in one call and
     take its greedy token v_i after each of them;
  3. accept t1..ta while t_(i+1) == v_i, emit them and then v_a (so every
     emitted token is the verify depth's greedy choice), keep positions
     p..p+a in the cache and continue from v_a.
The drafted positions are rewritten by the verify call at full depth, so the
cache left behind is exactly the one plain greedy decoding at verify_loops
would leave, and the emitted tokens equal plain greedy decoding's.
"""
from __future__ import annotations

import numpy as np

from .model import Cache, forward


def speculative_greedy(model, prompt, draft_loops, verify_loops, k_draft, n_new, max_seq,
                       kv_int8=False, casts=True):
    """Prefill `prompt` at verify_loops, then self-speculative greedy decode.

    Returns (tokens: the prefill's greedy token followed by n_new more,
    stats: dict with rounds, drafted and accepted counts).
    """
    if not 1 <= draft_loops <= verify_loops:
        raise ValueError("need 1 <= draft_loops <= verify_loops")
    cache = Cache(model.shape, max_seq, kv_int8)
    r = forward(model, prompt, verify_loops, cache=cache, casts=casts, logits="last")
    out = [int(np.argmax(r["logits"]))]
    stats = {"rounds": 0, "drafted": 0, "accepted": 0}
    while len(out) < n_new + 1:
        p = cache.length
        if p >= max_seq:
            raise ValueError("sequence reached max_seq")
        k = min(k_draft, max_seq - p - 1)
        depth_before = cache.depth.copy()
        # 1. draft: k cached greedy steps at draft_loops
        chain = [out[-1]]
        for _ in range(k):
            d = forward(model, [chain[-1]], draft_loops, cache=cache, casts=casts, logits="last")
            chain.append(int(np.argmax(d["logits"])))
        # 2. verify t0..tk at positions p..p+k (the drafted rows are rewritten)
        cache.length = p
        cache.depth[:] = depth_before
        v = forward(model, chain, verify_loops, cache=cache, casts=casts, logits="all")
        vt = [int(t) for t in np.argmax(v["logits"], axis=1)]
        # 3. accept the matching prefix, then the verifier's token
        a = 0
        while a < k and chain[a + 1] == vt[a]:
            a += 1
        emit = chain[1:a + 1] + [vt[a]]
        take = min(len(emit), n_new + 1 - len(out))
        out.extend(emit[:take])
        cache.length = p + take
        cache.depth[p + take:] = depth_before[p + take:]
        stats["rounds"] += 1
        stats["drafted"] += k
        stats["accepted"] += a
    return out, stats
