"""Continuous batching (dtd_sched_*) and the prefix cache (dtd_set_prefix_cache) on the GPU.

Parity: every request's tokens from a mixed, changing batch equal its tokens when it runs
alone, and both follow the oracle: the oracle is stepped through the request's own tokens
(teacher forcing), and each greedy token must be the oracle's argmax wherever the oracle's
top-1/top-2 margin is clear of the logit error (MARGIN of the largest logit).  A prefix-cache
hit must give what recomputing the prefix gives.
"""
import numpy as np
import pytest

import oracle
from decoder_only_transformer_decode_amd import dtd, synth
from _pair import TOL, Pair, need_gpu, normwise, top2_margin

pytestmark = pytest.mark.gpu

_GRID = synth.ModelShape("grid", 320, 2, 10, 2, 32, 608, 1000, synth.W_INT8_ROW, synth.ACT_F32, synth.KV_F32)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _say(*a):
    print(*a, flush=True)


def _requests(vocab, seed=5):
    lens = [5, 17, 32, 9, 40, 3, 23, 12]
    news = [12, 8, 20, 5, 16, 10, 7, 14]
    return [(synth.prompt_tokens(vocab, n, seed=seed + i), m) for i, (n, m) in enumerate(zip(lens, news))]


def _oracle_check(O, prompt, toks, margin_rel, tag):
    """Teacher-forces oracle model O (slot 0, overwritten from position 0) through prompt +
    toks; each token must be the oracle's argmax where the margin is clear.  Returns the number
    of tokens checked."""
    out = None
    for i, t in enumerate(prompt):
        out = O.step(0, int(t), i)
    o_tok, o_log = out[0], out[1]
    checked = 0
    for i, t in enumerate(toks):
        if top2_margin(o_log) > margin_rel * float(np.abs(o_log).max()):
            assert t == o_tok, f"{tag}: token {i} is {t}, the oracle's argmax is {o_tok}"
            checked += 1
        if i + 1 < len(toks):
            o_tok, o_log, _ = O.step(0, int(t), len(prompt) + i)
    return checked


@pytest.mark.parametrize("kw,margin_rel", [(dict(), 1e-4), (dict(act=synth.ACT_BF16, kvfmt=synth.KV_BF16), 8e-3)],
                         ids=["f32", "bf16"])
def test_continuous_batching_each_request_as_if_alone(kw, margin_rel):
    """Eight requests of different prompt lengths and budgets arrive in three waves into a
    batch of at most four: admissions wait for room, departures let the next ones in.  Each
    request's tokens equal those it gets alone, and follow the oracle."""
    s = _GRID.replace(**kw)
    P = Pair(s, max_ctx=96, max_seqs=8, max_batch=4, seed=3)
    total_blocks = P.eng.kv_blocks_free()
    reqs = _requests(s.vocab)
    sch = dtd.Scheduler(P.eng)
    ids = [sch.submit(p, m) for p, m in reqs[:3]]
    sch.step()
    sch.step()
    ids += [sch.submit(p, m) for p, m in reqs[3:6]]
    for _ in range(3):
        sch.step()
    ids += [sch.submit(p, m) for p, m in reqs[6:]]
    steps = 5 + sch.run()
    together = []
    for rid, (p, m) in zip(ids, reqs):
        toks, done = sch.result(rid)
        assert done and len(toks) == m
        together.append(toks)
    assert P.eng.kv_blocks_free() == total_blocks     # every departure freed its KV
    # each request alone, one after the other
    alone = []
    for p, m in reqs:
        rid = sch.submit(p, m)
        sch.run()
        alone.append(sch.result(rid)[0])
    O = oracle.Model(s, P.w, max_ctx=96, max_seqs=1)
    checked = 0
    for i, ((p, m), a, b) in enumerate(zip(reqs, together, alone)):
        if a != b:
            # only where the two runs met a near tie: the first difference must be one
            k = next(j for j in range(m) if a[j] != b[j])
            _say(f"request {i}: batched and alone part at token {k}")
            checked += _oracle_check(O, p, a[:k + 1], margin_rel, f"request {i} batched")
            checked += _oracle_check(O, p, b[:k + 1], margin_rel, f"request {i} alone")
        else:
            checked += _oracle_check(O, p, a, margin_rel, f"request {i}")
    _say(f"{s.name} {kw}: {len(reqs)} requests in {steps} steps; {checked} tokens checked against the oracle")
    assert checked >= sum(m for _, m in reqs) * 0.8
    sch.close()
    P.close()


def test_stop_token_and_background_loop():
    s = _GRID
    P = Pair(s, max_ctx=96, max_seqs=8, max_batch=4, seed=3)
    reqs = _requests(s.vocab, seed=40)
    sch = dtd.Scheduler(P.eng)
    ref_ids = [sch.submit(p, m) for p, m in reqs]
    sch.run()
    ref = [sch.result(r)[0] for r in ref_ids]
    # stop at the third token of request 2
    stop = ref[2][2]
    rid = sch.submit(reqs[2][0], reqs[2][1], stop_token=stop)
    sch.run()
    toks, done = sch.result(rid)
    assert done and toks == ref[2][:ref[2].index(stop) + 1]
    # the scheduler's own thread: submissions while it runs, waits from this thread
    sch.start()
    with pytest.raises(dtd.DtdError):
        sch.step()
    ids = [sch.submit(p, m) for p, m in reqs]
    for rid in ids:
        assert sch.wait(rid, 60000) == dtd.DTD_OK
    got = [sch.result(r)[0] for r in ids]
    sch.stop()
    O = oracle.Model(s, P.w, max_ctx=96, max_seqs=1)
    for i, (a, b) in enumerate(zip(got, ref)):
        k = next((j for j in range(len(a)) if a[j] != b[j]), len(a))
        if k < len(a):     # batches form differently in the loop; only a near tie may part them
            _oracle_check(O, reqs[i][0], a[:k + 1], 1e-4, f"loop request {i}")
            _oracle_check(O, reqs[i][0], b[:k + 1], 1e-4, f"stepped request {i}")
    for r in ids:
        sch.release(r)
    with pytest.raises(dtd.DtdError):
        sch.release(ids[0])
    sch.close()
    P.close()


def test_sampled_and_greedy_requests_share_batches():
    """Two sampled requests (counter = position) and two greedy ones: each sampled draw is in
    the oracle's acceptable set for the oracle's logits after the same tokens, and equal to
    the oracle's own draw until the first draw where the two picked different members."""
    import test_gpu_sampling as TS
    w = synth.TINY
    s = w.shape
    P = Pair(s, max_ctx=96, max_seqs=4, max_batch=4, seed=synth.weights_seed(w))
    sch = dtd.Scheduler(P.eng)
    samps = [dtd.sampler(temperature=0.9, top_k=64, top_p=0.95, seed=11),
             dtd.sampler(temperature=1.2, min_p=0.02, seed=12)]
    prompts = [synth.prompt_tokens(s.vocab, n, seed=60 + n) for n in (12, 30, 7, 21)]
    ids = [sch.submit(prompts[0], 24, sampler=samps[0]), sch.submit(prompts[1], 24),
           sch.submit(prompts[2], 24, sampler=samps[1]), sch.submit(prompts[3], 24)]
    sch.run()
    outs = [sch.result(r)[0] for r in ids]
    O = oracle.Model(s, P.w, max_ctx=96, max_seqs=1)
    for i, (p, toks) in enumerate(zip(prompts, outs)):
        samp = samps[i // 2] if i % 2 == 0 else None
        out = None
        for j, t in enumerate(p):
            out = O.step(0, int(t), j)
        ol = out[1]
        same = 0
        for j, t in enumerate(toks):
            pos = len(p) - 1 + j
            if j > 0:
                _, ol, _ = O.step(0, toks[j - 1], pos)
            if samp is None:
                if top2_margin(ol) > 1e-4 * float(np.abs(ol).max()):
                    assert t == int(np.argmax(ol)), f"greedy request {i} token {j}"
                continue
            want, ok = TS._oracle(ol, samp, pos, eps=1e-4)
            assert t in ok, f"sampled request {i} draw {j}: {t} not in {sorted(ok)}"
            if t != want:
                break
            same += 1
        if samp is not None:
            _say(f"sampled request {i}: {same} draws equal to the oracle's")
            assert same >= 12
    sch.close()
    P.close()


# ---------------------------------------------------------------------------------------
# prefix cache
# ---------------------------------------------------------------------------------------

def _kv(P, seq, layer, n):
    s = P.shape
    dt = {synth.KV_F32: np.float32, synth.KV_BF16: np.uint16, synth.KV_I8: np.int8}[s.kvfmt]
    k = np.empty((n, s.n_kv_heads, s.head_dim), dt)
    v = np.empty_like(k)
    ks = vs = None
    if s.kvfmt == synth.KV_I8:
        ks, vs = np.empty((n, s.n_kv_heads), np.uint16), np.empty((n, s.n_kv_heads), np.uint16)
    dtd.dtd_debug_kv_read(P.eng.h, seq, layer, 0, n, k, v, ks, vs)
    return k, v, ks, vs


@pytest.mark.parametrize("kw", [dict(), dict(act=synth.ACT_BF16, kvfmt=synth.KV_I8)], ids=["f32", "bf16-int8kv"])
def test_prefix_hit_equals_recompute(kw):
    s = _GRID.replace(**kw)
    P = Pair(s, max_ctx=128, max_seqs=6, seed=8)          # a cache-free engine with the same weights:
    R = Pair(s, max_ctx=128, max_seqs=6, seed=8, weights=P.w)
    P.eng.set_prefix_cache(8)
    base = synth.prompt_tokens(s.vocab, 60, seed=1)
    tail = synth.prompt_tokens(s.vocab, 20, seed=2)
    a_tok, a_log = P.gpu_prefill(1, base)
    assert P.eng.prefix_reused(1) == 0 and P.eng.prefix_entries() == 1
    for reuse in (45, 32):                                 # a partial last block, then whole blocks
        seq = 10 + reuse
        prompt = np.concatenate([base[:reuse], tail])
        g_tok, g_log = P.gpu_prefill(seq, prompt)
        assert P.eng.prefix_reused(seq) == reuse
        r_tok, r_log = R.gpu_prefill(seq, prompt)
        err = normwise(g_log, r_log)
        _say(f"{kw} reuse {reuse}: logits {err:.2e} from recomputing the prefix")
        assert err <= TOL
        if top2_margin(r_log) > 2 * np.abs(g_log - r_log).max():
            assert g_tok == r_tok
        for layer in range(s.n_layers):                    # the reused positions hold the owner's KV
            for x, y in zip(_kv(P, seq, layer, reuse), _kv(P, 1, layer, reuse)):
                assert x is None or np.array_equal(x, y)
    # the whole prompt again: every position but the last is reused
    c_tok, c_log = P.gpu_prefill(2, base)
    assert P.eng.prefix_reused(2) == 59
    assert normwise(c_log, a_log) <= TOL
    # the owner leaves; a sharer keeps decoding on the shared blocks, like a recomputed twin
    P.eng.reset_seq(1)
    seq = 10 + 45
    tok_p, tok_r = [int(P.gpu_step([seq], [7])[0][0])], [int(R.gpu_step([seq], [7])[0][0])]
    for _ in range(6):
        ng, lg, _ = P.gpu_step([seq], [tok_p[-1]])
        nr, lr, _ = R.gpu_step([seq], [tok_r[-1]])
        assert normwise(lg[0], lr[0]) <= TOL
        tok_p.append(int(ng[0]))
        tok_r.append(int(nr[0]))
    assert tok_p == tok_r
    # no common prefix: nothing reused
    P.gpu_prefill(3, synth.prompt_tokens(s.vocab, 30, seed=99))
    assert P.eng.prefix_reused(3) == 0
    P.close()
    R.close()


def test_prefix_cache_eviction_and_block_accounting():
    s = _GRID
    # 8 blocks of 16 positions: two 40-token prompts (3 blocks each) fit, a third evicts
    P = Pair(s, max_ctx=64, max_seqs=4, kv_num_blocks=8, seed=8)
    P.eng.set_prefix_cache(4)
    prompts = [synth.prompt_tokens(s.vocab, 40, seed=80 + i) for i in range(4)]
    P.gpu_prefill(1, prompts[0])
    P.eng.reset_seq(1)                       # its blocks stay with the cache entry
    assert P.eng.kv_blocks_free() == 5 and P.eng.prefix_entries() == 1
    P.gpu_prefill(2, prompts[1])
    P.eng.reset_seq(2)
    assert P.eng.kv_blocks_free() == 2 and P.eng.prefix_entries() == 2
    P.gpu_prefill(3, prompts[2])             # needs 3 blocks: the oldest entry goes
    assert P.eng.prefix_entries() == 2 and P.eng.kv_blocks_free() == 2
    P.gpu_prefill(4, prompts[1])             # still cached
    assert P.eng.prefix_reused(4) == 39
    for sid in (3, 4):
        P.eng.reset_seq(sid)
    P.eng.set_prefix_cache(0)
    assert P.eng.prefix_entries() == 0 and P.eng.kv_blocks_free() == 8
    P.close()


def test_scheduler_records_finished_requests_for_follow_ups():
    """A follow-up that repeats a finished request's prompt and answer skips their prefill."""
    s = _GRID
    P = Pair(s, max_ctx=96, max_seqs=4, max_batch=2, seed=3)
    P.eng.set_prefix_cache(4)
    sch = dtd.Scheduler(P.eng)
    p = synth.prompt_tokens(s.vocab, 20, seed=4)
    r1 = sch.submit(p, 10)
    sch.run()
    ans = sch.result(r1)[0]
    follow = np.concatenate([p, ans, synth.prompt_tokens(s.vocab, 6, seed=5)]).astype(np.int32)
    r2 = sch.submit(follow, 5)
    sch.run()
    assert P.eng.prefix_entries() >= 1
    # the engine reports the reuse of the follow-up's sequence only while it exists; check the
    # tokens instead: equal to the follow-up run on a cache-free engine
    R = Pair(s, max_ctx=96, max_seqs=4, max_batch=2, seed=3, weights=P.w)
    sr = dtd.Scheduler(R.eng)
    r3 = sr.submit(follow, 5)
    sr.run()
    a, b = sch.result(r2)[0], sr.result(r3)[0]
    k = next((j for j in range(len(a)) if a[j] != b[j]), len(a))
    if k < len(a):
        O = oracle.Model(s, P.w, max_ctx=96, max_seqs=1)
        _oracle_check(O, follow, a[:k + 1], 1e-4, "cached follow-up")
        _oracle_check(O, follow, b[:k + 1], 1e-4, "recomputed follow-up")
    sch.close()
    sr.close()
    P.close()
    R.close()
