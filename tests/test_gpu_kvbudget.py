"""The Initial-Key KV budget on the GPU (dtd_set_kv_budget) against the oracle's
(oracle/kvbudget.py).

The oracle is stepped through the GPU's own tokens (teacher forcing), so both evict after
the same steps.  Each side ranks the middle entries by its own attention-score sums (fp32
recomputed dot products on the GPU, float64 in the oracle), so where two sums are within
rounding of each other the two may keep different entries; the comparison of kept entries
and logits ends at the first such near tie, and everything before it must agree: the kept
token positions exactly, the score sums of the kept entries within 1e-3, the logits within
the tolerance, or with bf16 activations within the oracle's own sensitivity (ENV_FACTOR x the
distance from an oracle with perturbed norm gains, run through the same tokens).  A budget at least the sequence's length must give the full cache's outputs.
"""
import numpy as np
import pytest

import oracle
from oracle import kvbudget as KB
from decoder_only_transformer_decode_amd import dtd, synth
from _pair import ENV_FACTOR, TOL, Pair, need_gpu, normwise, top2_margin

pytestmark = pytest.mark.gpu

_GRID = synth.ModelShape("grid", 320, 2, 10, 2, 32, 608, 1000, synth.W_INT8_ROW, synth.ACT_F32, synth.KV_F32)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _say(*a):
    print(*a, flush=True)


def test_budget_at_least_the_length_is_the_full_cache():
    s = _GRID.replace(act=synth.ACT_BF16, kvfmt=synth.KV_BF16)
    P = Pair(s, max_ctx=96, max_seqs=2, seed=5, path=dtd.PATH_PER_KERNEL)
    P.eng.set_kv_budget(0, 96, n_initial=4, n_recent=8, score_layers=2)
    prompt = synth.prompt_tokens(s.vocab, 40, seed=1)
    a_tok, a_log = P.gpu_prefill(0, prompt)
    b_tok, b_log = P.gpu_prefill(1, prompt)
    assert np.array_equal(a_log, b_log) and a_tok == b_tok
    ta, tb = a_tok, b_tok
    for step in range(30):
        na, la, _ = P.gpu_step([0], [ta])
        nb, lb, _ = P.gpu_step([1], [tb])
        assert np.array_equal(la, lb), f"step {step}"
        ta, tb = int(na[0]), int(nb[0])
    assert P.eng.kv_positions(0) == list(range(70))
    P.close()


def _oracle_run(ob, token, score=True):
    """one oracle step; returns (token, logits, score sums before the eviction)"""
    tok, log = ob._run(int(token), score=score)
    pre = ob.scores.copy()
    ob._evict()
    return tok, log, pre


def _run_budgeted(s, kw_budget, prompt_len, steps, seed, batch_with_plain=False, path=dtd.PATH_AUTO):
    """GPU sequence 0 under the budget (free-running greedy), the oracle's BudgetedSeq
    teacher-forced through its tokens.  Returns the number of steps compared before the first
    near tie (or all of them)."""
    budget, n_init, n_rec, layers = kw_budget
    P = Pair(s, max_ctx=128, max_seqs=3, max_batch=2, seed=seed, path=path)
    if path == dtd.PATH_PERSISTENT:
        assert dtd.dtd_debug_uses_persistent(P.eng.h, 1)
    O = oracle.Model(s, P.w, max_ctx=128, max_seqs=2)
    P.eng.set_kv_budget(0, budget, n_initial=n_init, n_recent=n_rec, score_layers=layers)
    ob = KB.BudgetedSeq(O, 0, budget, n_init, n_rec, layers)
    ob2 = KB.BudgetedSeq(P.perturbed_oracle(seed, max_ctx=128), 0, budget, n_init, n_rec, layers)
    prompt = synth.prompt_tokens(s.vocab, prompt_len, seed=seed + 1)
    g_tok, g_log = P.gpu_prefill(0, prompt)
    for i, t in enumerate(prompt[:-1]):
        ob._run(int(t), score=False)
        ob2._run(int(t), score=False)
    o_tok, o_log, pre = _oracle_run(ob, prompt[-1])
    o2_log = _oracle_run(ob2, prompt[-1])[1]
    plain_tok = None
    if batch_with_plain:
        plain_tok, _ = P.gpu_prefill(1, prompt)
        for i, t in enumerate(prompt):
            O.step(1, int(t), i)
    compared = 0
    for step in range(steps + 1):
        gpos = P.eng.kv_positions(0)
        assert len(gpos) <= budget
        if gpos != ob.kept:
            # only a near tie of the oracle's score sums (at that eviction) may part the two
            extra = sorted(set(gpos) ^ set(ob.kept))
            spread = float(np.ptp(pre[extra]))
            _say(f"step {step}: kept entries part at positions {extra}, oracle sums {pre[extra]}")
            assert spread <= 1e-3 * max(1.0, float(np.abs(pre[extra]).max())), "kept entries differ without a near tie"
            break
        gsc = P.eng.kv_scores(0)
        assert np.allclose(gsc, ob.scores[gpos], rtol=1e-3, atol=1e-5), f"step {step}: score sums"
        err = normwise(g_log, o_log)
        bound = max(TOL, ENV_FACTOR * normwise(o2_log, o_log))
        assert err <= bound, f"step {step}: logits {err:.2e} > {bound:.2e}"
        if top2_margin(o_log) > 2 * float(np.abs(g_log.astype(np.float64) - o_log).max()):
            assert g_tok == o_tok, f"step {step}: greedy token"
        compared += 1
        if step == steps:
            break
        if batch_with_plain:
            ng, lg, _ = P.gpu_step([0, 1], [g_tok, plain_tok])
            g_log, g_next, plain_next = lg[0], int(ng[0]), int(ng[1])
            op = O.step(1, plain_tok, prompt_len + step)
            assert normwise(lg[1], op[1]) <= TOL
            if top2_margin(op[1]) > 2 * float(np.abs(lg[1].astype(np.float64) - op[1]).max()):
                assert plain_next == op[0], f"step {step}: the unbudgeted sequence"
            plain_tok = plain_next
        else:
            ng, lg, _ = P.gpu_step([0], [g_tok])
            g_log, g_next = lg[0], int(ng[0])
        o_tok, o_log, pre = _oracle_run(ob, g_tok)
        o2_log = _oracle_run(ob2, g_tok)[1]
        g_tok = g_next
    P.close()
    return compared


@pytest.mark.parametrize("path", [dtd.PATH_PERSISTENT, dtd.PATH_PER_KERNEL], ids=["step-kernel", "per-kernel"])
@pytest.mark.parametrize("kw", [dict(), dict(act=synth.ACT_BF16, kvfmt=synth.KV_I8),
                                dict(n_q_heads=8, n_kv_heads=2, head_dim=128, act=synth.ACT_BF16,
                                     kvfmt=synth.KV_BF16)],
                         ids=["f32", "bf16-int8kv", "hd128"])
def test_budget_evicts_like_the_oracle(kw, path):
    # batch 1: the step kernel (scores from its kept queries and softmax statistics) or the
    # per-sub-step kernels
    s = _GRID.replace(**kw)
    n = _run_budgeted(s, (24, 3, 6, 1), prompt_len=30, steps=40, seed=7, path=path)
    _say(f"{kw}: {n} steps with the same kept entries, scores and outputs as the oracle")
    assert n >= 20


@pytest.mark.parametrize("kw", [dict(), dict(act=synth.ACT_BF16, kvfmt=synth.KV_I8)], ids=["f32", "bf16-int8kv"])
def test_budget_scores_every_scored_layer_in_one_launch(kw):
    # batch 1 on the step kernel with both layers scored: the score sums of the two layers
    # come from one launch, layer by layer
    s = _GRID.replace(**kw)
    n = _run_budgeted(s, (24, 3, 6, 2), prompt_len=30, steps=30, seed=11, path=dtd.PATH_PERSISTENT)
    _say(f"{kw}, 2 scored layers: {n} steps with the same kept entries, scores and outputs as the oracle")
    assert n >= 15


def test_budgeted_and_plain_sequences_share_a_batch():
    n = _run_budgeted(_GRID, (32, 4, 8, 2), prompt_len=20, steps=40, seed=9, batch_with_plain=True)
    _say(f"batch of a budgeted and a plain sequence: {n} steps compared")
    assert n >= 20


def test_budget_bounds_the_blocks_held():
    s = _GRID
    P = Pair(s, max_ctx=128, max_seqs=2, seed=3)
    total = P.eng.kv_blocks_free()
    P.eng.set_kv_budget(0, 40, n_initial=4, n_recent=8, score_layers=1)
    tok, _ = P.gpu_prefill(0, synth.prompt_tokens(s.vocab, 60, seed=4))
    held = []
    for _ in range(50):
        ng, _, _ = P.gpu_step([0], [tok])
        tok = int(ng[0])
        held.append(total - P.eng.kv_blocks_free())
    assert max(held) <= (40 + 1 + 15) // 16 and P.eng.seq_len(0) == 40
    assert P.eng.kv_positions(0)[:4] == [0, 1, 2, 3] and P.eng.kv_positions(0)[-1] == 109
    with pytest.raises(dtd.DtdError):
        P.eng.set_kv_budget(1, 10, n_initial=4, n_recent=8)      # budget below 4 + 8 + 1
    P.eng.reset_seq(0)
    assert P.eng.kv_blocks_free() == total
    P.close()
