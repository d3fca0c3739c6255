"""Parity of the HIP decode step (through the C ABI) with the CPU oracle.

Bar: bit-exact for dequantisation, block-table indexing and greedy tokens on the tiny
config; logits and hidden states within max|gpu - oracle| / max|oracle| <= 2e-3.  Where a
test is teacher-forced, the GPU's greedy token must equal the oracle's whenever the
oracle's top-1/top-2 margin exceeds twice the observed logit error (then no rounding
difference of that size can reorder them).
"""
import numpy as np
import pytest

from decoder_only_transformer_decode_amd import dtd, synth
from _pair import (ENV_FACTOR, TOL, Pair, need_gpu, normwise, probe_step, stored_kv_error, stored_kv_reference,
                   top2_margin)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _say(*a):
    print(*a, flush=True)


def _check_logits(tag, g_log, o_log, g_tok, o_tok):
    err = normwise(g_log, o_log)
    delta = np.abs(np.asarray(g_log, np.float64) - np.asarray(o_log, np.float64)).max()
    margin = top2_margin(o_log)
    _say(f"{tag}: logits err {err:.2e} margin {margin:.3e} tok gpu {g_tok} oracle {o_tok}")
    assert err <= TOL, f"{tag}: logits normwise error {err:.3e}"
    if margin > 2 * delta:
        assert g_tok == o_tok, f"{tag}: greedy token differs with margin {margin} > 2*{delta}"


# ---------------------------------------------------------------------------------------
# the tiny configuration, end to end, free-running greedy
# ---------------------------------------------------------------------------------------

PATHS = [dtd.PATH_PERSISTENT, dtd.PATH_PER_KERNEL]
PATH_IDS = ["persistent", "per-kernel"]


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_tiny_config_end_to_end_identical_greedy_tokens(path):
    w = synth.TINY
    s = w.shape
    P = Pair(s, max_ctx=w.context, seed=synth.weights_seed(w), path=path)
    assert dtd.dtd_debug_uses_persistent(P.eng.h, 1) == (path == dtd.PATH_PERSISTENT)
    prompt = synth.prompt_tokens(s.vocab, w.prompt_len)
    g_tok, g_log = P.gpu_prefill(0, prompt)
    o_tok, o_log = P.orc_prefill(0, prompt)
    _check_logits("prefill", g_log, o_log, g_tok, o_tok)
    toks_g, toks_o = [g_tok], [o_tok]
    worst_h = 0.0
    capture = path == dtd.PATH_PER_KERNEL      # hidden-state capture runs the per-kernel schedule
    for step in range(w.context - w.prompt_len):
        pos = w.prompt_len + step
        ng, lg, hid = P.gpu_step([0], [toks_g[-1]], capture=capture)
        no, lo, ho = P.orc_step(0, toks_o[-1], pos, hidden=True)
        if capture:
            for layer in range(s.n_layers + 1):
                e = normwise(hid[layer, 0], ho[layer])
                worst_h = max(worst_h, e)
                assert e <= TOL, f"step {step} layer {layer} hidden error {e:.3e}"
        _check_logits(f"step {step}", lg[0], lo, int(ng[0]), no)
        toks_g.append(int(ng[0]))
        toks_o.append(no)
    _say(f"tiny ({PATH_IDS[PATHS.index(path)]}): tokens {toks_g}, worst hidden err {worst_h:.2e}")
    assert toks_g == toks_o
    assert len(toks_g) == 33
    P.close()


def test_persistent_and_per_kernel_schedules_agree():
    s = _GRID.replace(act=synth.ACT_BF16, kvfmt=synth.KV_BF16)
    A = Pair(s, max_ctx=64, seed=6, path=dtd.PATH_PERSISTENT)
    B = Pair(s, max_ctx=64, seed=6, weights=A.w, path=dtd.PATH_PER_KERNEL)
    prompt = synth.prompt_tokens(s.vocab, 24, seed=2)
    _, la = A.gpu_prefill(0, prompt)
    _, lb = B.gpu_prefill(0, prompt)
    assert normwise(la, lb) <= TOL
    assert dtd.dtd_debug_uses_persistent(A.eng.h, 1) and not dtd.dtd_debug_uses_persistent(A.eng.h, 2)
    A.close()
    B.close()


# ---------------------------------------------------------------------------------------
# every storage format, multi-tile and ragged shapes
#
# Two comparisons per step.  (1) Kernel by kernel (dtd_debug_decode_probe): every GPU
# kernel of every layer reads the oracle's own input for it.  fp32 outputs (q, k, v, the
# residual stream, logits) must be within 2e-3; outputs rounded to bf16 (the norm outputs,
# attention output, SwiGLU output) must equal the oracle's rounding of its unrounded value
# wherever that rounding is unique, i.e. outside a band of 2e-5 x rms around a rounding
# midpoint, and be one of the two neighbours inside it.  (2) Free-running: the GPU's own
# trajectory against the oracle's.  With bf16 rounding points the method itself is
# ill-conditioned: fp32-rounding-sized noise flips a few roundings, each moving the outputs
# by up to ~1e-3.  The free-running bound is max(2e-3, 4 x the distance between the oracle
# and an oracle whose norm gains carry 1e-6 relative noise), on the same tokens.
# ---------------------------------------------------------------------------------------

_GRID = synth.ModelShape("grid", 320, 2, 10, 2, 32, 608, 1000, synth.W_INT8_ROW, synth.ACT_F32, synth.KV_F32)
_FORMATS = [
    dict(),
    dict(act=synth.ACT_BF16, kvfmt=synth.KV_BF16),
    dict(wfmt=synth.W_Q8_0, act=synth.ACT_BF16, kvfmt=synth.KV_BF16, tied=True),
    dict(wfmt=synth.W_BF16, act=synth.ACT_BF16, kvfmt=synth.KV_BF16),
    dict(act=synth.ACT_BF16, kvfmt=synth.KV_I8),
    dict(wfmt=synth.W_Q8_0, kvfmt=synth.KV_I8),
    dict(n_q_heads=8, n_kv_heads=4, head_dim=64, act=synth.ACT_BF16, kvfmt=synth.KV_BF16),
    dict(n_q_heads=4, n_kv_heads=4, head_dim=16, wfmt=synth.W_BF16),   # MHA, q_dim != D
    dict(wfmt=synth.W_Q8_0),                                            # Q8_0 with fp32 KV
    dict(wfmt=synth.W_BF16, act=synth.ACT_BF16, kvfmt=synth.KV_I8),
    # head size 128 with 4 query heads per KV head (and the default 16-position KV blocks),
    # the shape the batch-1 step kernel is also built for with those sizes fixed at compile
    # time: each activation type and each weight and KV encoding at least once
    dict(n_q_heads=8, n_kv_heads=2, head_dim=128),
    dict(n_q_heads=8, n_kv_heads=2, head_dim=128, wfmt=synth.W_Q8_0, act=synth.ACT_BF16, kvfmt=synth.KV_I8),
    dict(n_q_heads=8, n_kv_heads=2, head_dim=128, wfmt=synth.W_BF16, act=synth.ACT_BF16, kvfmt=synth.KV_BF16),
    # int8-row weights, bf16 activations and bf16 KV at that shape: the instantiation the
    # benchmark times on the SmolLM3-3B shape (its probe variant has the same parameters)
    dict(n_q_heads=8, n_kv_heads=2, head_dim=128, act=synth.ACT_BF16, kvfmt=synth.KV_BF16),
    # Q4_0 weights; the last one is the instantiation the benchmark's Q4_0 workload times
    dict(wfmt=synth.W_Q4_0),
    dict(wfmt=synth.W_Q4_0, act=synth.ACT_BF16, kvfmt=synth.KV_BF16, tied=True),
    dict(n_q_heads=8, n_kv_heads=2, head_dim=128, wfmt=synth.W_Q4_0, act=synth.ACT_BF16, kvfmt=synth.KV_I8),
    dict(n_q_heads=8, n_kv_heads=2, head_dim=128, wfmt=synth.W_Q4_0, act=synth.ACT_BF16, kvfmt=synth.KV_BF16),
    # head size 64 with G 4 and bf16 activations: the fixed-shape instantiation the Llama-3.2-1B
    # workload runs (Q8_0, bf16 KV, tied head), and one with int8 KV
    dict(n_q_heads=8, n_kv_heads=2, head_dim=64, wfmt=synth.W_Q8_0, act=synth.ACT_BF16, kvfmt=synth.KV_BF16, tied=True),
    dict(n_q_heads=8, n_kv_heads=2, head_dim=64, act=synth.ACT_BF16, kvfmt=synth.KV_I8),
]


class Tracker:
    """Free-running errors and the oracle's own sensitivity over a whole run."""

    def __init__(self):
        self.gpu = 0.0
        self.env = 0.0

    def add(self, g, r, rp):
        self.gpu = max(self.gpu, normwise(g, r))
        self.env = max(self.env, normwise(rp, r))

    def check(self, tag):
        bound = max(TOL, ENV_FACTOR * self.env)
        _say(f"{tag}: free-running max err {self.gpu:.2e}, oracle sensitivity {self.env:.2e}, bound {bound:.2e}")
        assert self.gpu <= bound, f"{tag}: free-running error {self.gpu:.3e} > {bound:.3e}"


def teacher_forced(P, gpu_ids, orc_ids, toks, poss, tag):
    """One probed step: every GPU kernel fed the oracle's inputs and compared with it."""
    return probe_step(P, gpu_ids, orc_ids, toks, poss, tag)


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("kw", _FORMATS, ids=lambda kw: "-".join(f"{k}={v}" for k, v in kw.items()) or "base")
def test_formats(kw, path):
    s = _GRID.replace(**kw)
    P = Pair(s, max_ctx=96, max_seqs=2, seed=21, path=path)
    g4 = s.n_q_heads == 4 * s.n_kv_heads
    fixed = 128 if g4 and s.head_dim == 128 else (64 if g4 and s.head_dim == 64 and s.act == synth.ACT_BF16 else 0)
    assert dtd.dtd_debug_step_kernel_shape(P.eng.h) == fixed
    _say(f"formats {kw}: step kernel shape {f'fixed hd {fixed}, G 4, bs 16' if fixed else 'run time'}, "
         f"{PATH_IDS[PATHS.index(path)]} schedule")
    O2 = P.perturbed_oracle(1, max_ctx=96)
    prompt = synth.prompt_tokens(s.vocab, 70, seed=3)
    tr = Tracker()
    # sequence 0 (GPU) is teacher-forced position by position; sequence 1 (GPU) runs free
    for i, t in enumerate(prompt[:-1]):
        teacher_forced(P, [0], [0], [int(t)], [i], f"prefill {i}")
        O2.step(0, int(t), i)
    _, g_log = P.gpu_prefill(1, prompt)
    outs = teacher_forced(P, [0], [0], [int(prompt[-1])], [69], "prefill 69")
    tr.add(g_log, outs[0][1], O2.step(0, int(prompt[-1]), 69)[1])
    tok = outs[0][0]
    for step in range(8):
        ng, lg, _ = P.gpu_step([1], [tok])
        outs = teacher_forced(P, [0], [0], [tok], [70 + step], f"step {step}")
        o2 = O2.step(0, tok, 70 + step)
        tr.add(lg[0], outs[0][1], o2[1])
        tok = outs[0][0]
    tr.check("formats " + s.name)
    P.close()


def test_dequant_rows_bit_exact_all_formats():
    for kw in _FORMATS[:4] + [dict(wfmt=synth.W_Q4_0)]:
        s = _GRID.replace(**kw)
        P = Pair(s, max_ctx=32, seed=5)
        t = P.torch
        for name, (rows, cols) in synth.matrix_shapes(s).items():
            out = t.empty((rows, cols), dtype=t.float32, device=P.dev)
            dtd.dtd_debug_dequant_rows(P.eng.h, name, 0, rows, out.data_ptr())
            got = out.cpu().numpy()
            parts = P.w[name]
            import oracle
            w = parts.get("w", parts.get("q"))
            sc = parts.get("s")
            for r in range(rows):
                ref = oracle.dequant_row(s.wfmt, w, sc, r)
                assert np.array_equal(got[r].view(np.uint32), ref.view(np.uint32)), (name, r)
        P.close()


# ---------------------------------------------------------------------------------------
# batched decode over paged KV: sequences of different lengths in one step
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("kw", [dict(), dict(wfmt=synth.W_BF16, act=synth.ACT_BF16, kvfmt=synth.KV_BF16),
                                dict(act=synth.ACT_BF16, kvfmt=synth.KV_I8)], ids=["f32", "bf16", "i8kv"])
def test_batched_decode_mixed_lengths(kw):
    s = _GRID.replace(**kw)
    lens = [3, 17, 40, 64, 65]
    ids = [7, 3, 11, 5, 9]
    P = Pair(s, max_ctx=80, max_seqs=12, max_batch=6, seed=8)
    O2 = P.perturbed_oracle(2, max_ctx=80, max_seqs=6)
    toks = {}
    tr = Tracker()
    # free-running sequences use the ids; teacher-forced copies use id + 100
    for sid, n in zip(ids, lens):
        prompt = synth.prompt_tokens(s.vocab, n, seed=sid)
        P.gpu_prefill(sid, prompt)
        for i, t in enumerate(prompt):
            outs = teacher_forced(P, [sid + 100], [sid], [int(t)], [i], f"prefill seq {sid} pos {i}")
            O2.step(P.oslot(sid), int(t), i)
        toks[sid] = outs[0][0]
    order = [9, 7, 5, 11, 3]          # batch order differs from creation order
    pos = {sid: n for sid, n in zip(ids, lens)}
    for step in range(4):
        ng, lg, hid = P.gpu_step(order, [toks[i] for i in order])
        outs = teacher_forced(P, [i + 100 for i in order], order, [toks[i] for i in order],
                              [pos[i] for i in order], f"step {step}")
        for b, sid in enumerate(order):
            tr.add(lg[b], outs[b][1], O2.step(P.oslot(sid), toks[sid], pos[sid])[1])
            toks[sid] = outs[b][0]
            pos[sid] += 1
    for sid in ids:
        assert P.eng.seq_len(sid) == pos[sid] == P.eng.seq_len(sid + 100)
    tr.check("batched " + s.name)
    P.close()


# ---------------------------------------------------------------------------------------
# batched steps: projections on the matrix cores (bf16 activations, int8-row or bf16 weights)
# ---------------------------------------------------------------------------------------

def _write_kv_ids(P, sid, gpu_ids, n, seed):
    s = P.shape
    for layer in range(s.n_layers):
        k, v, ks, vs = synth.synthetic_kv(s, n, seed=seed, layer=layer)
        ks16 = None if ks is None else ks.view(np.uint16)
        vs16 = None if vs is None else vs.view(np.uint16)
        for g in gpu_ids:
            dtd.dtd_debug_kv_write(P.eng.h, g, layer, 0, k, v, ks16, vs16)
        P.orc.kv_write(P.oslot(sid), layer, 0, k, v, ks, vs)


@pytest.mark.parametrize("kw", [dict(act=synth.ACT_BF16, kvfmt=synth.KV_BF16),
                                dict(wfmt=synth.W_BF16, act=synth.ACT_BF16, kvfmt=synth.KV_BF16),
                                dict(act=synth.ACT_BF16, kvfmt=synth.KV_I8)],
                         ids=["int8row", "bf16w", "int8row-i8kv"])
def test_batched_steps_matrix_core_projections(kw):
    """64 sequences of mixed lengths, stepped in batches of 64, 40, 17 and 2 (one to four
    16-sequence column blocks, ragged ones included); the grid shape's matrices have fewer
    row tiles than compute units, so every projection also takes the split-K path.  Each
    batch is checked kernel by kernel (probe) and free-running against the oracle."""
    s = _GRID.replace(**kw)
    P = Pair(s, max_ctx=64, max_seqs=160, max_batch=64, seed=31)
    O2 = P.perturbed_oracle(5, max_ctx=64, max_seqs=64)
    rng = np.random.default_rng(44)
    ids = list(range(64))
    lens = [int(n) for n in rng.integers(1, 48, size=64)]
    for sid, n in zip(ids, lens):
        _write_kv_ids(P, sid, [sid, sid + 100], n, seed=200 + sid)
        for layer in range(s.n_layers):
            k, v, ks, vs = synth.synthetic_kv(s, n, seed=200 + sid, layer=layer)
            O2.kv_write(P.oslot(sid), layer, 0, k, v, ks, vs)
    toks = {sid: int(t) for sid, t in zip(ids, rng.integers(0, s.vocab, size=64))}
    pos = dict(zip(ids, lens))
    tr = Tracker()
    for sub in (ids, ids[5:45], ids[30:47], [63, 0]):
        ng, lg, _ = P.gpu_step(sub, [toks[i] for i in sub])
        outs = teacher_forced(P, [i + 100 for i in sub], sub, [toks[i] for i in sub], [pos[i] for i in sub],
                              f"batch {len(sub)}")
        for b, sid in enumerate(sub):
            tr.add(lg[b], outs[b][1], O2.step(P.oslot(sid), toks[sid], pos[sid])[1])
            toks[sid] = outs[b][0]
            pos[sid] += 1
        _say(f"batch {len(sub)}: probe ok (bf16 flips so far {P.probe_stats[0]})")
    tr.check("matrix-core batched " + s.name)
    P.close()


# ---------------------------------------------------------------------------------------
# the KV append's rounding to the cache type, on fresh float32 vectors with constructed ties
# ---------------------------------------------------------------------------------------

def _kv_cases(hd, rng):
    """float32 head vectors that put the KV rounding on its edge cases."""
    m = 1 + 2.0 ** -11                       # fp16 midpoint between 1 and 1 + 2^-10
    c = []
    v = rng.standard_normal(hd) * 0.3
    v[3] = 127 * m                           # int8 scale exactly on an fp16 midpoint (ties even)
    c.append(v)
    v = rng.standard_normal(hd) * 0.3
    v[0] = 127 * (1 + 3 * 2.0 ** -11)        # midpoint between odd and even fp16 neighbours
    c.append(v)
    s = 2.0 ** -6                            # int8 codes exactly on half integers
    v = (rng.integers(-126, 126, hd) + 0.5) * s
    v[0] = 127 * s
    c.append(v)
    v = rng.standard_normal(hd)              # bf16 ties and their float32 neighbours
    v[:6] = [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1 + 2.0 ** -8 + 2.0 ** -23,
             1 + 2.0 ** -8 - 2.0 ** -23, 2.0 ** -130]
    c.append(v)
    v = rng.standard_normal(hd) * 1e-6       # a subnormal fp16 scale that rounds down: clamps
    v[1] = 127 * 1.4 * 2.0 ** -24
    v[2] = -127 * 1.4 * 2.0 ** -24
    c.append(v)
    c.append(np.zeros(hd))                   # zero scale
    c.append(rng.standard_normal(hd) * 40.0)
    return [np.asarray(x, dtype=np.float32) for x in c]


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("kvfmt", [synth.KV_F32, synth.KV_BF16, synth.KV_I8], ids=["f32", "bf16", "i8"])
@pytest.mark.parametrize("hd", [32, 128], ids=["hd32", "hd128"])
def test_kv_append_rounding_bit_exact(kvfmt, path, hd):
    """Probe steps inject fresh float32 k/v (not already rounded) for the new position; the
    entry the GPU appends must equal the oracle's KV rounding of those same values, bit for
    bit: scale and codes for int8, bits for bf16 and fp32."""
    kw = dict(kvfmt=kvfmt, act=synth.ACT_BF16)
    if hd == 128:
        kw.update(n_q_heads=8, n_kv_heads=2, head_dim=128)
    s = _GRID.replace(**kw)
    P = Pair(s, max_ctx=32, max_seqs=1, seed=3, path=path)
    rng = np.random.default_rng(5 + hd + kvfmt)
    cases = _kv_cases(s.head_dim, rng)
    n_steps = (len(cases) + s.n_kv_heads - 1) // s.n_kv_heads * 2
    for step in range(n_steps):
        inj = {}
        for layer in range(s.n_layers):
            vec = []
            for which in range(2):          # k, v
                heads = [cases[(step * s.n_kv_heads + j + which + layer) % len(cases)]
                         for j in range(s.n_kv_heads)]
                vec.append(np.concatenate(heads)[None, :])
            inj[layer] = tuple(vec)
        probe_step(P, [0], [0], [3 + step], [step], f"kv rounding step {step}", check=False, kv_inject=inj)
        for layer in range(s.n_layers):
            kr, ksr = stored_kv_reference(s, inj[layer][0])
            vr, vsr = stored_kv_reference(s, inj[layer][1])
            kg, vg = np.empty_like(kr), np.empty_like(vr)
            ksg = vsg = None
            if ksr is not None:
                ksg, vsg = np.empty_like(ksr), np.empty_like(vsr)
            dtd.dtd_debug_kv_read(P.eng.h, 0, layer, step, 1, kg, vg, ksg, vsg)
            where = f"step {step} layer {layer}"
            assert np.array_equal(kg.view(np.uint8), kr.view(np.uint8)), f"{where}: stored k"
            assert np.array_equal(vg.view(np.uint8), vr.view(np.uint8)), f"{where}: stored v"
            if ksr is not None:
                assert np.array_equal(ksg, ksr) and np.array_equal(vsg, vsr), f"{where}: scales"
    _say(f"kv rounding {synth.KV_NAMES[kvfmt]} hd {hd} ({PATH_IDS[PATHS.index(path)]}): "
         f"{n_steps} positions x {s.n_layers} layers bit-exact")
    P.close()


# ---------------------------------------------------------------------------------------
# KV cache: block-table indexing, long contexts from identical stored KV
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("kvfmt", [synth.KV_F32, synth.KV_BF16, synth.KV_I8])
def test_kv_block_table_roundtrip_bit_exact(kvfmt):
    s = _GRID.replace(kvfmt=kvfmt)
    P = Pair(s, max_ctx=200, max_seqs=2, seed=1)
    n, hk, hd = 150, s.n_kv_heads, s.head_dim
    t, j, i = np.meshgrid(np.arange(n), np.arange(hk), np.arange(hd), indexing="ij")
    code = (t * 7 + j * 3 + i) % 251 - 125            # exactly representable in every format
    if kvfmt == synth.KV_F32:
        k = code.astype(np.float32); v = (-code).astype(np.float32)
    elif kvfmt == synth.KV_BF16:
        k = synth.f32_to_bf16_bits(code.astype(np.float32)); v = synth.f32_to_bf16_bits((-code).astype(np.float32))
    else:
        k = code.clip(-127, 127).astype(np.int8); v = (-code).clip(-127, 127).astype(np.int8)
    ks = vs = None
    if kvfmt == synth.KV_I8:
        ks = (np.arange(n * hk).reshape(n, hk) % 97 + 1).astype(np.float16).view(np.uint16)
        vs = (np.arange(n * hk).reshape(n, hk) % 89 + 2).astype(np.float16).view(np.uint16)
    for layer in range(s.n_layers):
        dtd.dtd_debug_kv_write(P.eng.h, 4, layer, 0, k, v, ks, vs)
        # a second sequence interleaves its blocks with the first one's
        dtd.dtd_debug_kv_write(P.eng.h, 6, layer, 0, v, k, vs, ks)
    for layer in range(s.n_layers):
        for sid, (ek, ev, eks, evs) in ((4, (k, v, ks, vs)), (6, (v, k, vs, ks))):
            ko, vo = np.empty_like(k), np.empty_like(v)
            kso = vso = None
            if kvfmt == synth.KV_I8:
                kso, vso = np.empty_like(ks), np.empty_like(vs)
            dtd.dtd_debug_kv_read(P.eng.h, sid, layer, 0, n, ko, vo, kso, vso)
            assert np.array_equal(ko, ek) and np.array_equal(vo, ev)
            if kvfmt == synth.KV_I8:
                assert np.array_equal(kso, eks) and np.array_equal(vso, evs)
    P.close()


def _splitmix_final(z):
    z = z.astype(np.uint64)
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xbf58476d1ce4e5b9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94d049bb133111eb)
    return z ^ (z >> np.uint64(31))


def _kv_fill_values(s, layer, n, seed):
    """dtd_debug_kv_fill's contents as its declaration defines them: (u, a) with u of shape
    [2][n][Hkv][hd] (K, V) and the fp32 amplitude a."""
    t, j, i, w = np.meshgrid(np.arange(n, dtype=np.uint64), np.arange(s.n_kv_heads, dtype=np.uint64),
                             np.arange(s.head_dim, dtype=np.uint64), np.arange(2, dtype=np.uint64), indexing="ij")
    key = (np.uint64(layer) << np.uint64(40)) ^ (t << np.uint64(20)) ^ (j << np.uint64(12)) ^ (i << np.uint64(1)) ^ w
    h = _splitmix_final(np.uint64(seed) ^ _splitmix_final(key))
    u = (h >> np.uint64(40)).astype(np.float32) * np.float32(2.0 ** -23) - np.float32(1.0)
    a = np.float32(0.02) * np.float32(np.sqrt(np.float32(s.dim))) * np.float32(1.7320508)
    return np.moveaxis(u, 3, 0), a


@pytest.mark.parametrize("kvfmt", [synth.KV_F32, synth.KV_BF16, synth.KV_I8])
def test_kv_fill_is_its_definition(kvfmt):
    # the long-context timing fill: every stored element against the declared hash, through
    # the block table of two interleaved sequences; the length it sets; a step on top of it
    s = _GRID.replace(kvfmt=kvfmt)
    P = Pair(s, max_ctx=160, max_seqs=3, max_batch=2, seed=1)
    n_a, n_b = 150, 37
    dtd.dtd_debug_kv_fill(P.eng.h, 2, 20, 11)
    dtd.dtd_debug_kv_fill(P.eng.h, 1, n_a, 9)
    dtd.dtd_debug_kv_fill(P.eng.h, 2, n_b, 11)       # grows into a block after sequence 1's
    assert P.eng.seq_len(1) == n_a and P.eng.seq_len(2) == n_b
    for sid, n, seed in ((1, n_a, 9), (2, n_b, 11)):
        for layer in range(s.n_layers):
            u, a = _kv_fill_values(s, layer, n, seed)
            dt = {synth.KV_F32: np.float32, synth.KV_BF16: np.uint16, synth.KV_I8: np.int8}[kvfmt]
            ko = np.empty((n, s.n_kv_heads, s.head_dim), dt)
            vo = np.empty_like(ko)
            kso = vso = None
            if kvfmt == synth.KV_I8:
                kso, vso = np.empty((n, s.n_kv_heads), np.uint16), np.empty((n, s.n_kv_heads), np.uint16)
            dtd.dtd_debug_kv_read(P.eng.h, sid, layer, 0, n, ko, vo, kso, vso)
            for w, got in ((0, ko), (1, vo)):
                where = f"seq {sid} layer {layer} {'KV'[w]}"
                if kvfmt == synth.KV_I8:
                    # the codes depend on u alone: exact
                    assert np.array_equal(got, np.rint(u[w] * np.float32(127.0)).astype(np.int8)), where
                    sc = (kso if w == 0 else vso).view(np.float16).astype(np.float64)
                    assert np.allclose(sc, float(a) / 127.0, rtol=1e-3, atol=0), where
                    continue
                ref = u[w] * a                       # fp32 product, as stored for fp32
                g = got.astype(np.float64) if kvfmt == synth.KV_F32 else synth.bf16_bits_to_f32(got).astype(np.float64)
                # a comes from the device's sqrtf: allow a few fp32 ulps of it, then bf16's step
                rel = 2.0 ** -21 if kvfmt == synth.KV_F32 else 2.0 ** -8
                assert np.all(np.abs(g - ref) <= rel * np.abs(ref) + 1e-30), where
                if kvfmt == synth.KV_BF16:
                    exact = np.mean(got == synth.f32_to_bf16_bits(ref.astype(np.float32)))
                    assert exact > 0.999, f"{where}: {exact:.4f} of elements round like the definition"
    # a shorter fill of a longer sequence overwrites positions and keeps its length
    dtd.dtd_debug_kv_fill(P.eng.h, 1, 20, 10)
    assert P.eng.seq_len(1) == n_a
    free = P.eng.kv_blocks_free()
    for bad in (0, -3, 161):
        with pytest.raises(dtd.DtdError):
            dtd.dtd_debug_kv_fill(P.eng.h, 2, bad, 1)
    assert P.eng.seq_len(2) == n_b and P.eng.kv_blocks_free() == free
    # decoding continues at position len
    ng, lg, _ = P.gpu_step([1, 2], [3, 4])
    assert np.isfinite(lg).all() and P.eng.seq_len(1) == n_a + 1 and P.eng.seq_len(2) == n_b + 1
    P.close()


@pytest.mark.parametrize("kw,n_pos", [(dict(act=synth.ACT_BF16, kvfmt=synth.KV_BF16), 700),
                                      (dict(act=synth.ACT_BF16, kvfmt=synth.KV_I8), 1000),
                                      (dict(), 333)], ids=["bf16-700", "i8-1000", "f32-333"])
def test_long_context_from_identical_stored_kv(kw, n_pos):
    s = _GRID.replace(**kw)
    P = Pair(s, max_ctx=n_pos + 4, max_seqs=2, seed=2)
    O2 = P.perturbed_oracle(3, max_ctx=n_pos + 4)
    P.write_kv_both(0, n_pos, seed=77, extra=[(O2, 0)])
    for layer in range(s.n_layers):          # the free-running GPU copy gets the same KV
        k, v, ks, vs = synth.synthetic_kv(s, n_pos, 77, layer)
        dtd.dtd_debug_kv_write(P.eng.h, 1, layer, 0, k, v, None if ks is None else ks.view(np.uint16),
                               None if vs is None else vs.view(np.uint16))
    tr = Tracker()
    tok = 5
    for step in range(3):
        ng, lg, _ = P.gpu_step([1], [tok])
        outs = teacher_forced(P, [0], [0], [tok], [n_pos + step], f"T={n_pos + step + 1}")
        tr.add(lg[0], outs[0][1], O2.step(0, tok, n_pos + step)[1])
        tok = outs[0][0]
    tr.check(f"long context {n_pos}")
    # the KV the GPU appended (teacher-forced copy) matches the oracle's stored KV
    for layer in range(s.n_layers):
        excess, flipped = stored_kv_error(P, 0, layer, n_pos, 3)
        assert excess <= TOL, f"layer {layer} stored KV beyond one encoding step: {excess:.3e}"
    P.close()


# ---------------------------------------------------------------------------------------
# engine semantics
# ---------------------------------------------------------------------------------------

def test_prefill_equals_sequential_steps_and_is_deterministic():
    # batched prefill (chunks of positions as one step) against the same tokens stepped one
    # at a time: the same method, different kernels, so equal within the tolerance; and
    # repeatable bit for bit
    s = _GRID.replace(act=synth.ACT_BF16, kvfmt=synth.KV_BF16)
    P = Pair(s, max_ctx=160, max_seqs=3, seed=4)
    prompt = synth.prompt_tokens(s.vocab, 90, seed=9)
    gp, lp = P.gpu_prefill(1, prompt)
    P.gpu_prefill(2, prompt[:1])
    for t in prompt[1:]:
        ns, ls, _ = P.gpu_step([2], [t])
    err = normwise(lp, ls[0])
    _say(f"batched prefill vs sequential steps: logits err {err:.2e}")
    assert err <= TOL
    delta = float(np.abs(lp.astype(np.float64) - ls[0]).max())
    if top2_margin(ls[0]) > 2 * delta:
        assert gp == int(ns[0])
    P.eng.reset_seq(1)
    _, lp2 = P.gpu_prefill(1, prompt)
    assert np.array_equal(lp, lp2)
    P.close()


@pytest.mark.parametrize("kw", [dict(act=synth.ACT_BF16, kvfmt=synth.KV_BF16),
                                dict(act=synth.ACT_BF16, kvfmt=synth.KV_I8),
                                dict(wfmt=synth.W_BF16, act=synth.ACT_BF16, kvfmt=synth.KV_BF16),
                                dict(n_q_heads=8, n_kv_heads=2, head_dim=128, act=synth.ACT_BF16, kvfmt=synth.KV_BF16),
                                dict(wfmt=synth.W_Q8_0, kvfmt=synth.KV_F32)],
                         ids=["int8row-bf16kv", "int8kv", "bf16w", "hd128", "q8_0-f32"])
def test_batched_prefill_matches_oracle(kw):
    """A 100-token prompt prefilled as chunks of 64 and 36 positions (NEXT-1): logits of the
    last position and every stored K/V against the oracle's position-by-position run, then
    free-running decode steps."""
    s = _GRID.replace(**kw)
    P = Pair(s, max_ctx=128, max_seqs=2, seed=17)
    O2 = P.perturbed_oracle(6, max_ctx=128)
    prompt = synth.prompt_tokens(s.vocab, 100, seed=12)
    tr = Tracker()
    g_tok, g_log = P.gpu_prefill(0, prompt)
    o_tok, o_log = P.orc_prefill(0, prompt)
    for i, t in enumerate(prompt):
        o2 = O2.step(0, int(t), i)
    tr.add(g_log, o_log, o2[1])
    # every stored position: each side rounded its own k/v to the KV encoding, so an
    # element may sit one encoding step from the oracle's where a rounding boundary fell
    # between the two unrounded values.  Beyond that step, layer 0 is within the tolerance;
    # deeper layers carry the rounding of the activations before them, so they are held to
    # the free-running bound, from the perturbed oracle's KV measured the same way
    for layer in range(s.n_layers):
        excess, flipped, env = stored_kv_error(P, 0, layer, 0, 100, other=O2)
        bound = TOL if layer == 0 else max(TOL, ENV_FACTOR * env)
        _say(f"layer {layer} stored KV: excess {excess:.2e} (bound {bound:.2e}, oracle sensitivity {env:.2e}), "
             f"elements one step apart {flipped:.2%}")
        assert excess <= bound, f"layer {layer} stored KV beyond one encoding step: {excess:.3e} > {bound:.3e}"
    toks_g, toks_o = [g_tok], [o_tok]
    for step in range(4):
        ng, lg, _ = P.gpu_step([0], [toks_g[-1]])
        no, lo, _ = P.orc_step(0, toks_o[-1], 100 + step)
        tr.add(lg[0], lo, O2.step(0, toks_o[-1], 100 + step)[1])
        toks_g.append(int(ng[0]))
        toks_o.append(no)
    _say(f"batched prefill {kw}: tokens {toks_g} / oracle {toks_o}")
    tr.check("batched prefill " + s.name)
    P.close()


def test_error_paths_leave_state_unchanged():
    t = pytest.importorskip("torch")
    s = _GRID
    P = Pair(s, max_ctx=40, max_seqs=2, max_batch=2, kv_num_blocks=3, seed=4)
    h = P.eng.h
    dev = P.dev
    tok = t.zeros(4, dtype=t.int32, device=dev)
    out = t.zeros(4, dtype=t.int32, device=dev)
    lib = dtd.load()
    ids = (dtd.C.c_int64 * 2)(1, 2)
    assert lib.dtd_decode_step(h, 1, ids, tok.data_ptr(), out.data_ptr(), None) == dtd.DTD_E_NOSEQ
    P.gpu_prefill(1, [1, 2, 3])
    same = (dtd.C.c_int64 * 2)(1, 1)
    assert lib.dtd_decode_step(h, 2, same, tok.data_ptr(), out.data_ptr(), None) == dtd.DTD_E_ARG
    assert lib.dtd_decode_step(h, 3, ids, tok.data_ptr(), out.data_ptr(), None) == dtd.DTD_E_ARG
    big = t.zeros(60, dtype=t.int32, device=dev)
    assert lib.dtd_prefill(h, 1, big.data_ptr(), 60, out.data_ptr(), None) == dtd.DTD_E_CTX
    # 3 blocks of 16: seq 1 holds one; 40 positions of a new sequence need 3 -> KV full
    assert lib.dtd_prefill(h, 2, big.data_ptr(), 40, out.data_ptr(), None) == dtd.DTD_E_KVFULL
    assert P.eng.seq_len(1) == 3 and P.eng.seq_len(2) == dtd.DTD_E_NOSEQ
    assert lib.dtd_reset_seq(h, 99) == dtd.DTD_E_NOSEQ
    bad = t.tensor([5, s.vocab + 3], dtype=t.int32, device=dev)
    assert lib.dtd_prefill(h, 2, bad.data_ptr(), 2, out.data_ptr(), None) == dtd.DTD_OK
    assert lib.dtd_check_device_errors(h) == dtd.DTD_E_ARG
    assert lib.dtd_check_device_errors(h) == dtd.DTD_OK
    P.close()


def test_load_weights_fail_closed():
    s = _GRID
    w = synth.flat_tensors(synth.gen_weights(s, 1))
    eng = dtd.Engine(s, max_ctx=16)
    missing = dict(w)
    missing.pop("L1.w_down.q")
    with pytest.raises(dtd.DtdError) as ei:
        eng.load_weights(missing)
    assert ei.value.status == dtd.DTD_E_ARG and "missing" in str(ei.value)
    wrong = dict(w)
    wrong["L0.wq.s"] = wrong["L0.wq.s"][:-1]
    with pytest.raises(dtd.DtdError):
        eng.load_weights(wrong)
    extra = dict(w)
    extra["L9.wq.q"] = w["L0.wq.q"]
    with pytest.raises(dtd.DtdError):
        eng.load_weights(extra)
    t = eng.torch
    tok = t.zeros(1, dtype=t.int32, device=eng.device)
    with pytest.raises(dtd.DtdError) as ei:
        eng.prefill(0, tok)
    assert ei.value.status == dtd.DTD_E_STATE
    eng.load_weights(w)
    eng.prefill(0, tok)
    eng.close()
