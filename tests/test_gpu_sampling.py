"""The device sampler (dtd_sample, dtd_set_sampler) against the oracle's sampler.

Both sides read the same fp32 logits.  The oracle works in float64; the device sums
fixed-point weights built from fp32 exponentials, whose relative error is a few 1e-7 per
token weight, so its cumulative distribution can sit up to about 3e-6 (of the total) from
the oracle's.  Where u falls that close to the boundary between two tokens, or a top-p
running sum or a probability sits that close to p or min-p, the two may pick different
tokens.  So each device token must lie in the oracle's acceptable set: the tokens whose
cumulative-probability interval meets [u - EPS, u + EPS], under the oracle's filters and, when
a filter's cut is within DELTA (relative) of a tie, under the same filters with p and min-p
moved by DELTA either way.  And the device token must equal the oracle's own in nearly every
row.  Top-k and greedy order fp32 logits exactly on both sides.
"""
import numpy as np
import pytest

from decoder_only_transformer_decode_amd import dtd, synth
from oracle import sampling as S
from _pair import Pair, need_gpu

pytestmark = pytest.mark.gpu

EPS = 1e-5     # cumulative-probability slack of the draw (absolute, of the total)
DELTA = 1e-5   # relative slack of the top-p and min-p cuts


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _say(*a):
    print(*a, flush=True)


def _f32(x):
    return float(np.float32(x))


def _oracle(l32, s: "dtd.dtd_sampler", counter, eps=EPS):
    """(the oracle's token, the acceptable set) for one row, NaN read as -inf."""
    l = np.where(np.isnan(l32), -np.inf, np.asarray(l32, np.float64))
    o = S.Sampler(_f32(s.temperature), int(s.top_k), _f32(s.top_p), _f32(s.min_p), int(s.seed))
    d = S.sample(l, o, counter)
    if d.u != d.u:                      # greedy
        return d.token, {d.token}
    variants = [o]
    if d.cut_margins and min(d.cut_margins) < DELTA:
        for fp in (1 - DELTA, 1.0, 1 + DELTA):
            for fm in (1 - DELTA, 1.0, 1 + DELTA):
                variants.append(S.Sampler(o.temperature, o.top_k, min(1.0, o.top_p * fp) if o.top_p < 1 else 1.0,
                                          o.min_p * fm, o.seed))
    ok = set()
    for v in variants:
        p, _ = S.filtered_probs(l, v)
        cdf = np.cumsum(p)
        lo = cdf - p
        ok |= set(int(x) for x in np.flatnonzero((p > 0) & (lo <= d.u + eps) & (cdf > d.u - eps)))
    ok.add(d.token)
    return d.token, ok


def _gpu_sample(logits_dev, samplers, counters):
    t = pytest.importorskip("torch")
    B, V = logits_dev.shape
    out = t.full((B,), -1, dtype=t.int32, device=logits_dev.device)
    dtd.dtd_sample(logits_dev.data_ptr(), V, B, V, samplers, counters, out.data_ptr(),
                   t.cuda.current_stream().cuda_stream)
    t.cuda.synchronize()
    return out.cpu().numpy()


SETTINGS = [
    dict(temperature=0.0),
    dict(temperature=1.0),
    dict(temperature=0.7, top_k=40),
    dict(temperature=1.0, top_p=0.9),
    dict(temperature=0.8, top_k=50, top_p=0.95),
    dict(temperature=1.3, min_p=0.05),
    dict(temperature=0.6, top_k=200, top_p=0.8, min_p=0.02),
    dict(temperature=1.0, top_k=1),
    dict(temperature=2.0, top_p=0.5),
    dict(temperature=0.3, top_k=5, min_p=0.2),
    dict(temperature=1.0, top_k=1000, top_p=0.99),
    dict(temperature=0.05),
]


@pytest.mark.parametrize("vocab", [1000, 151936, 37])
def test_sample_rows_match_oracle(vocab):
    t = pytest.importorskip("torch")
    B = 64
    logits = synth.sampling_logits(B, vocab, seed=vocab)
    dev = t.from_numpy(logits).cuda()
    equal = other = 0
    for rnd in range(3):
        samplers = [dtd.sampler(seed=1000 * rnd + b, **SETTINGS[(b + rnd) % len(SETTINGS)]) for b in range(B)]
        counters = [rnd * 7919 + 13 * b for b in range(B)]
        got = _gpu_sample(dev, samplers, counters)
        for b in range(B):
            want, ok = _oracle(logits[b], samplers[b], counters[b])
            assert 0 <= got[b] < vocab and not np.isnan(logits[b, got[b]])
            assert int(got[b]) in ok, (f"row {b} round {rnd} {SETTINGS[(b + rnd) % len(SETTINGS)]}: "
                                       f"gpu {got[b]} oracle {want}, acceptable {sorted(ok)[:8]}")
            if got[b] == want:
                equal += 1
            else:
                other += 1
    _say(f"V={vocab}: {equal} rows equal to the oracle's token, {other} another token of its acceptable set")
    assert other <= 0.05 * (equal + other)


def test_draws_are_per_row_and_repeatable():
    # a row's token depends only on its logits, settings and counter: the same row in other
    # batch slots, next to other rows, draws the same token; the same call twice is identical
    t = pytest.importorskip("torch")
    V = 5000
    base = synth.sampling_logits(8, V, seed=3)
    s0 = dtd.sampler(temperature=0.9, top_k=100, top_p=0.9, seed=42)
    rows = np.stack([base[1]] * 64)
    rows[::3] = base[2]
    dev = t.from_numpy(rows).cuda()
    samplers = [s0 if b % 3 else dtd.sampler(temperature=1.5, seed=b) for b in range(64)]
    counters = [77 if b % 3 else b for b in range(64)]
    a = _gpu_sample(dev, samplers, counters)
    b2 = _gpu_sample(dev, samplers, counters)
    assert np.array_equal(a, b2)
    same = [a[b] for b in range(64) if b % 3]
    assert len(set(same)) == 1
    alone = _gpu_sample(t.from_numpy(base[1:2].copy()).cuda(), [s0], [77])
    assert alone[0] == same[0]


def test_greedy_limits_on_the_device():
    t = pytest.importorskip("torch")
    B, V = 64, 32000
    logits = synth.sampling_logits(B, V, seed=11)
    dev = t.from_numpy(logits).cuda()
    clean = np.where(np.isnan(logits), -np.inf, logits)
    top = np.array([int(np.flatnonzero(r == r.max())[0]) for r in clean])
    for s in (dict(temperature=0.0), dict(temperature=1.0, top_k=1), dict(temperature=1.0, top_p=1e-7),
              dict(temperature=1.5, min_p=1.0)):
        got = _gpu_sample(dev, [dtd.sampler(seed=b, **s) for b in range(B)], list(range(B)))
        for b in range(B):
            assert got[b] == top[b], (s, b)


@pytest.mark.parametrize("s", [dict(temperature=1.0), dict(temperature=0.7, top_k=6),
                               dict(temperature=1.0, top_p=0.8, min_p=0.03)])
def test_chi_square_of_device_draws(s):
    stats = pytest.importorskip("scipy.stats")
    t = pytest.importorskip("torch")
    V, B, rounds = 16, 64, 400
    l = np.linspace(-3, 1.5, V).astype(np.float32)[np.random.default_rng(5).permutation(V)]
    dev = t.from_numpy(np.stack([l] * B)).cuda()
    samplers = [dtd.sampler(seed=9, **s)] * B
    counts = np.zeros(V, np.int64)
    for r in range(rounds):
        got = _gpu_sample(dev, samplers, [r * B + b for b in range(B)])
        counts += np.bincount(got, minlength=V)
    o = S.Sampler(_f32(s["temperature"]), s.get("top_k", 0), _f32(s.get("top_p", 1.0)), _f32(s.get("min_p", 0.0)))
    p, _ = S.filtered_probs(l.astype(np.float64), o)
    n = B * rounds
    assert np.all(counts[p == 0] == 0)
    live = p > 0
    res = stats.chisquare(counts[live], p[live] * n)
    _say(f"chi-square {s}: p-value {res.pvalue:.3f} over {n} draws, {int(live.sum())} tokens kept")
    assert res.pvalue > 1e-4


def test_sample_rejects_bad_arguments():
    t = pytest.importorskip("torch")
    dev = t.zeros((2, 10), dtype=t.float32, device="cuda")
    out = t.zeros(2, dtype=t.int32, device="cuda")
    ok = dtd.sampler(temperature=1.0)
    for bad in (dtd.sampler(temperature=-1.0), dtd.sampler(temperature=float("nan")),
                dtd.sampler(temperature=1.0, top_p=0.0), dtd.sampler(temperature=1.0, top_p=1.5),
                dtd.sampler(temperature=1.0, min_p=-0.1), dtd.sampler(temperature=1.0, top_k=-2)):
        with pytest.raises(dtd.DtdError):
            dtd.dtd_sample(dev.data_ptr(), 10, 2, 10, [ok, bad], [0, 1], out.data_ptr(), 0)
    with pytest.raises(dtd.DtdError):
        dtd.dtd_sample(dev.data_ptr(), 9, 2, 10, [ok, ok], [0, 1], out.data_ptr(), 0)


def _run_pair(P, samp, prompt, steps, together):
    """Sequence 0 samples with samp, sequence 1 stays greedy; both prefill the prompt and
    run free for `steps` decode steps (one batch of two, or one batch-1 step each).
    Returns the two token lists."""
    w = synth.TINY
    P.eng.set_sampler(0, samp)
    g0, _ = P.gpu_prefill(0, prompt)
    g1, _ = P.gpu_prefill(1, prompt)
    toks0, toks1 = [g0], [g1]
    for step in range(steps):
        if together:
            ng, _, _ = P.gpu_step([0, 1], [toks0[-1], toks1[-1]])
            a, b = int(ng[0]), int(ng[1])
        else:
            a = int(P.gpu_step([0], [toks0[-1]])[0][0])
            b = int(P.gpu_step([1], [toks1[-1]])[0][0])
        toks0.append(a)
        toks1.append(b)
    return toks0, toks1


@pytest.mark.parametrize("together", [False, True], ids=["batch-1-steps", "batch-2-steps"])
def test_engine_sampling_follows_the_oracle(together):
    """Sequence 0 samples (counter = position), sequence 1 stays greedy.  Each sampled token
    is compared with the oracle's draw from the oracle's own logits after the same tokens: it
    must be in the oracle's acceptable set, and the comparison ends at the first draw where
    the two picked different members of it (the runs part there).
    Batch-1 steps run the persistent step kernel, batches of two the per-sub-step kernels."""
    w = synth.TINY
    s = w.shape
    P = Pair(s, max_ctx=w.context, max_seqs=2, max_batch=2, seed=synth.weights_seed(w))
    assert dtd.dtd_debug_uses_persistent(P.eng.h, 1) == 1
    samp = dtd.sampler(temperature=0.9, top_k=64, top_p=0.95, min_p=0.01, seed=1234)
    prompt = synth.prompt_tokens(s.vocab, w.prompt_len)
    steps = w.context - w.prompt_len
    toks0, toks1 = _run_pair(P, samp, prompt, steps, together)
    # the oracle after the same tokens
    _, ol = P.orc_prefill(0, prompt)
    o1, _ = P.orc_prefill(1, prompt)
    assert toks1[0] == o1
    compared = 0
    for i in range(steps + 1):
        pos = w.prompt_len - 1 + i
        if i > 0:
            _, ol, _ = P.orc_step(0, toks0[i - 1], pos)
            n1, _, _ = P.orc_step(1, toks1[i - 1], pos)
            assert toks1[i] == n1, f"greedy sequence differs at step {i}"
        # the logits differ by rounding too (about 1e-6 of their range): a wider draw slack
        want, ok = _oracle(ol, samp, pos, eps=1e-4)
        assert toks0[i] in ok, f"draw {i}: gpu {toks0[i]} oracle {want}, acceptable {sorted(ok)}"
        if toks0[i] != want:
            _say(f"draw {i}: gpu {toks0[i]}, oracle {want}, both within the rounding slack; comparison ends")
            break
        compared += 1
    _say(f"sampled sequence ({'batch 2' if together else 'batch 1'}): {compared} draws equal to the oracle; "
         f"tokens {toks0}")
    assert compared >= 16 and len(set(toks0)) > 3
    # the same seeds after a reset reproduce both runs bit for bit
    P.eng.reset_seq(0)
    P.eng.reset_seq(1)
    a0, a1 = _run_pair(P, samp, prompt, steps, together)
    assert a0 == toks0 and a1 == toks1
    # reset drops the setting: greedy again
    P.eng.reset_seq(0)
    rg, _ = P.gpu_prefill(0, prompt)
    assert rg == o1
    P.close()
