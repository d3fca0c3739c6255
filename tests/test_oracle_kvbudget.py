"""Pins of the oracle's Initial-Key KV budget (oracle/kvbudget.py, orc_attention_kept,
orc_step_kept) to things other than itself: torch's masked scaled_dot_product_attention and
softmax, the page's own guarantee (a budget at least the length is the full cache), closed
forms of the selection rule, and the invariant that a query's probabilities sum to one."""
import numpy as np
import pytest
import torch

import oracle
from oracle import kvbudget as KB
from decoder_only_transformer_decode_amd import synth


def test_kept_attention_matches_torch_masked_sdpa_and_softmax():
    rng = np.random.default_rng(0)
    hq, hkv, d, n = 8, 2, 16, 40
    q = rng.standard_normal((hq, d))
    K = rng.standard_normal((n, hkv, d))
    V = rng.standard_normal((n, hkv, d))
    keep = (rng.random(n) < 0.6).astype(np.uint8)
    keep[-1] = 1
    prob = np.zeros(n)
    got = oracle.attention_kept(q, hkv, K, V, keep, prob)
    G = hq // hkv
    Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, 0)       # [hq][n][d]
    Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, 0)
    mask = torch.from_numpy(keep.astype(bool))[None, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q)[:, None, :], Kt, Vt,
                                                           attn_mask=mask)[:, 0, :]
    assert np.allclose(got, ref.numpy(), rtol=1e-12, atol=1e-13)
    scores = (torch.from_numpy(q)[:, None, :] @ Kt.transpose(1, 2))[:, 0, :] / np.sqrt(d)
    p = torch.softmax(scores.masked_fill(~mask[0], float("-inf")), dim=-1)
    assert np.allclose(prob, p.sum(0).numpy(), rtol=1e-12, atol=1e-15)
    assert np.all(prob[keep == 0] == 0) and abs(prob.sum() - hq) < 1e-12
    # every position kept: the plain attention
    full = oracle.attention_kept(q, hkv, K, V, np.ones(n, np.uint8))
    assert np.allclose(full, oracle.attention(q, K, V), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("kw", [dict(), dict(act=synth.ACT_BF16, kvfmt=synth.KV_BF16)], ids=["f32", "bf16"])
def test_budget_at_least_the_length_is_the_full_cache(kw):
    s = synth.tiny_shape(**kw)
    w = synth.gen_weights(s, 3)
    m = oracle.Model(s, w, max_ctx=64, max_seqs=2)
    b = KB.BudgetedSeq(m, 0, budget=64, n_initial=4, n_recent=8, score_layers=2)
    prompt = synth.prompt_tokens(s.vocab, 20, seed=1)
    tb, lb = b.prefill(prompt)
    out = None
    for i, t in enumerate(prompt):
        out = m.step(1, int(t), i)
    assert tb == out[0] and np.array_equal(lb, out[1])
    tok = tb
    for step in range(20):
        tb, lb = b.step(tok)
        ta, la, _ = m.step(1, tok, 20 + step)
        assert tb == ta and np.array_equal(lb, la)
        tok = tb
    assert b.kept == list(range(40))


def test_selection_rule_closed_forms():
    pos = list(range(20))
    sc = np.zeros(64)
    sc[[5, 9, 12]] = [3.0, 2.0, 2.0]
    sc[7] = 2.0
    # budget 8 = 2 initial + 3 recent + 3 by score: 5 (3.0), then 7, 9 (2.0, earlier first); 12 loses the tie
    assert KB.select_kept(pos, sc, 8, 2, 3) == [0, 1, 5, 7, 9, 17, 18, 19]
    assert KB.select_kept(pos, sc, 20, 2, 3) == pos
    assert KB.select_kept(pos, sc, 5, 2, 3) == [0, 1, 17, 18, 19]
    # after earlier evictions the kept set has gaps; recent = the last kept positions
    kept = [0, 1, 4, 7, 11, 15, 16]
    assert KB.select_kept(kept, sc, 5, 1, 2) == [0, 1, 7, 15, 16]      # 7 (2.0) beats 1, 4, 11 (0)
    assert KB.select_kept(kept, sc, 4, 1, 2) == [0, 7, 15, 16]


def test_eviction_keeps_the_budget_and_the_rule():
    s = synth.tiny_shape()
    w = synth.gen_weights(s, 4)
    m = oracle.Model(s, w, max_ctx=96, max_seqs=1)
    budget, n_init, n_rec = 24, 3, 6
    b = KB.BudgetedSeq(m, 0, budget=budget, n_initial=n_init, n_recent=n_rec, score_layers=1)
    tok, _ = b.prefill(synth.prompt_tokens(s.vocab, 30, seed=2))
    assert len(b.kept) == budget and b.kept[:n_init] == [0, 1, 2] and b.kept[-n_rec:] == list(range(24, 30))
    for step in range(40):
        tok, logits = b._run(tok, score=True)
        cand, sc = list(b.kept), b.scores.copy()
        b._evict()
        assert len(b.kept) == budget
        assert b.kept[:n_init] == cand[:n_init] and b.kept[-n_rec:] == cand[-n_rec:]
        (g,) = sorted(set(cand) - set(b.kept))
        # the evicted position scored lowest among the middle ones (the later one on a tie)
        for p in b.kept[n_init:-n_rec]:
            assert sc[g] < sc[p] or (sc[g] == sc[p] and g > p), (g, p, sc[g], sc[p])
        assert b.scores[g] == 0.0 and np.isfinite(logits).all()
    # each scored query adds n_q_heads * score_layers in total over the positions it attends
    m2 = oracle.Model(s, w, max_ctx=96, max_seqs=1)
    b2 = KB.BudgetedSeq(m2, 0, budget=90, n_initial=3, n_recent=6, score_layers=2)
    t2, _ = b2.prefill(synth.prompt_tokens(s.vocab, 10, seed=3))
    assert abs(b2.scores.sum() - s.n_q_heads * 2) < 1e-9
    for k in range(5):
        t2, _ = b2.step(t2)
        assert abs(b2.scores.sum() - s.n_q_heads * 2 * (k + 2)) < 1e-9
