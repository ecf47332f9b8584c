"""Pins of the oracle's self-speculative decode.

The method's defining property ("Introduction" page, "What Makes It
Different"; "Current Status" page, speculative decode table): drafting at a
shallow loop count and verifying at the full one emits exactly the tokens
plain greedy decoding at the full loop count emits, whatever the drafts are.
So the pins compare against generate_greedy (an independent code path: one
cached decode call per token), and check the acceptance bookkeeping: with
the draft depth equal to the verify depth every draft is accepted; a round
emits its accepted drafts plus one token.
"""
import numpy as np
import pytest

import oracle
import synth


@pytest.fixture(scope="module")
def micro():
    s = synth.SHAPES["micro"]
    return s, oracle.OracleModel(synth.make_weights(s, seed=4))


@pytest.mark.parametrize("ld,lv,k", [(1, 3, 1), (1, 3, 4), (2, 3, 7), (2, 4, 3)])
def test_speculative_equals_plain_greedy(micro, ld, lv, k):
    s, om = micro
    prompt = synth.make_tokens(s.vocab, 9, seed=1)
    n = 20
    ref, _, _ = oracle.generate_greedy(om, prompt, lv, n, max_seq=64)
    got, st = oracle.speculative_greedy(om, prompt, ld, lv, k, n, max_seq=64)
    assert got == ref
    assert st["accepted"] <= st["drafted"] <= st["rounds"] * k
    # every round emits its accepted drafts and one more token
    assert st["accepted"] + st["rounds"] >= n


def test_same_depth_accepts_every_draft(micro):
    s, om = micro
    prompt = synth.make_tokens(s.vocab, 7, seed=2)
    got, st = oracle.speculative_greedy(om, prompt, 3, 3, 4, 15, max_seq=64)
    assert st["accepted"] == st["drafted"] > 0
    ref, _, _ = oracle.generate_greedy(om, prompt, 3, 15, max_seq=64)
    assert got == ref


def test_draft_length_shrinks_at_max_seq(micro):
    """The last rounds draft fewer tokens so positions p..p+k fit; the final
    position is reached with a draft-free verify call."""
    s, om = micro
    prompt = synth.make_tokens(s.vocab, 10, seed=3)
    max_seq = 24
    n = max_seq - len(prompt)          # every position gets used
    ref, _, _ = oracle.generate_greedy(om, prompt, 2, n, max_seq=max_seq + 1)
    got, st = oracle.speculative_greedy(om, prompt, 1, 2, 5, n, max_seq=max_seq)
    assert got == ref[:n + 1]
    with pytest.raises(ValueError):
        oracle.speculative_greedy(om, prompt, 1, 2, 5, n + 1, max_seq=max_seq)


def test_planted_acceptance_error_is_caught(micro, monkeypatch):
    """Accepting one draft too many (a plausible off-by-one) breaks the
    equality with plain greedy decoding on this input."""
    import oracle.speculative as sp
    s, om = micro
    prompt = synth.make_tokens(s.vocab, 9, seed=1)
    ref, _, _ = oracle.generate_greedy(om, prompt, 3, 20, max_seq=64)
    src = open(sp.__file__).read().replace("while a < k and chain[a + 1] == vt[a]:\n            a += 1",
                                           "while a < k and chain[a + 1] == vt[a]:\n            a += 1\n"
                                           "        a = min(a + 1, k)")
    ns = {}
    exec(compile(src, "planted", "exec"), sp.__dict__ | ns, ns)
    got, _ = ns["speculative_greedy"](om, prompt, 1, 3, 4, 20, max_seq=64)
    assert got != ref
