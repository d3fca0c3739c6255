"""Runs the HIP engine (through the C ABI) and the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np

import oracle
from decoder_only_transformer_decode_amd import dtd, synth

TOL = 2e-3   # max |gpu - oracle| / max |oracle| per tensor (fp32 accumulation)
ENV_EPS = 1e-6     # relative noise used to measure the oracle's own sensitivity
ENV_FACTOR = 4.0   # free-running bound: max(TOL, ENV_FACTOR x the oracle's sensitivity)


def normwise(g, r) -> float:
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    den = np.abs(r).max()
    return float(np.abs(g - r).max() / (den if den > 0 else 1.0))


def top2_margin(logits) -> float:
    s = np.sort(np.asarray(logits, dtype=np.float64))
    return float(s[-1] - s[-2])


def need_gpu():
    import pytest
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; none is visible")
    dtd.load()   # raises if libdtd.so was not built: no fallback


class Pair:
    """An engine and an oracle model holding the same weights."""

    def __init__(self, shape, *, max_ctx, max_seqs=1, max_batch=1, seed=11, weights=None,
                 kv_block_size=16, kv_num_blocks=None, path=dtd.PATH_AUTO):
        import torch
        self.torch = torch
        self.shape = shape
        self.w = weights if weights is not None else synth.gen_weights(shape, seed)
        self.eng = dtd.Engine(shape, max_ctx=max_ctx, max_seqs=max_seqs, max_batch=max_batch,
                              kv_block_size=kv_block_size, kv_num_blocks=kv_num_blocks)
        self.eng.load_weights(synth.flat_tensors(self.w))
        dtd.dtd_debug_set_path(self.eng.h, path)
        self.orc = oracle.Model(shape, self.w, max_ctx=max_ctx, max_seqs=max_seqs)
        self.dev = self.eng.device
        self.slot_of = {}

    def close(self):
        self.eng.close()

    def oslot(self, seq_id):
        if seq_id not in self.slot_of:
            self.slot_of[seq_id] = len(self.slot_of)
        return self.slot_of[seq_id]

    # ---- GPU side ----
    def gpu_prefill(self, seq_id, tokens):
        nxt, logits = self.eng.prefill(seq_id, tokens, want_logits=True)
        self.torch.cuda.synchronize()
        return int(nxt.item()), logits.cpu().numpy()

    def gpu_step(self, seq_ids, tokens, capture=False):
        t = self.torch
        B = len(seq_ids)
        hid = None
        if capture:
            hid = t.empty((self.shape.n_layers + 1, B, self.shape.dim), dtype=t.float32, device=self.dev)
            dtd.dtd_debug_capture_hidden(self.eng.h, True, hid.data_ptr())
        nxt, logits = self.eng.decode_step(seq_ids, tokens, want_logits=True)
        t.cuda.synchronize()
        if capture:
            dtd.dtd_debug_capture_hidden(self.eng.h, False)
        return (nxt.cpu().numpy().astype(np.int64), logits.cpu().numpy(),
                None if hid is None else hid.cpu().numpy())

    # ---- oracle side ----
    def orc_prefill(self, seq_id, tokens, start=0):
        s = self.oslot(seq_id)
        out = None
        for i, tok in enumerate(tokens):
            out = self.orc.step(s, int(tok), start + i)
        return out[0], out[1]

    def orc_step(self, seq_id, token, pos, hidden=False):
        return self.orc.step(self.oslot(seq_id), int(token), pos, want_hidden=hidden)

    def perturbed_oracle(self, seed, max_ctx, max_seqs=1):
        """An oracle whose norm gains are scaled by (1 + ENV_EPS * N(0,1)): its distance from
        the plain oracle measures how far rounding-sized noise moves the method's outputs."""
        rng = np.random.default_rng(seed)
        w2 = {}
        for n, parts in self.w.items():
            if "g" in parts:
                g = parts["g"].astype(np.float64)
                w2[n] = {"g": (g * (1 + ENV_EPS * rng.standard_normal(g.shape))).astype(np.float32)}
            else:
                w2[n] = parts
        return oracle.Model(self.shape, w2, max_ctx=max_ctx, max_seqs=max_seqs)

    def write_kv_both(self, seq_id, n_pos, seed, extra=()):
        """Identical synthetic stored KV for positions [0, n_pos) of every layer."""
        for layer in range(self.shape.n_layers):
            k, v, ks, vs = synth.synthetic_kv(self.shape, n_pos, seed, layer)
            dtd.dtd_debug_kv_write(self.eng.h, seq_id, layer, 0, k, v,
                                   None if ks is None else ks.view(np.uint16),
                                   None if vs is None else vs.view(np.uint16))
            self.orc.kv_write(self.oslot(seq_id), layer, 0, k, v, ks, vs)
            for om, slot in extra:
                om.kv_write(slot, layer, 0, k, v, ks, vs)


# ---------------------------------------------------------------------------------------
# per-kernel probe: the GPU's kernels fed the oracle's own intermediate values
# ---------------------------------------------------------------------------------------

BAND = 2e-5   # half-width of the "near a rounding midpoint" band, x rms of the vector


def check_rounded(tag, g, r, act):
    """g: GPU values after the activation rounding (float64 array); r: the oracle's values
    before it.  Rounding is monotone, so g is a correct rounding of some value within `band`
    of r exactly when round(r - band) <= g <= round(r + band), band = BAND * rms(r).  Where
    that interval holds one bf16 value (r is not near a rounding midpoint) this demands g
    == round(r) bit for bit."""
    r = np.asarray(r, dtype=np.float64)
    if act == synth.ACT_F32:
        e = normwise(g, r)
        assert e <= TOL, f"{tag}: {e:.3e}"
        return 0
    band = BAND * np.sqrt(np.mean(r * r))
    lo = oracle.round_act_n(r - band, act)
    hi = oracle.round_act_n(r + band, act)
    ok = (g >= lo) & (g <= hi)
    if not ok.all():
        i = int(np.flatnonzero(~ok)[0])
        raise AssertionError(f"{tag}: {int((~ok).sum())} of {r.size} roundings outside "
                             f"[round(r-band), round(r+band)]; first at {i}: gpu {g[i]!r}, "
                             f"oracle unrounded {r[i]!r}, band {band:.3e}")
    return int((g != oracle.round_act_n(r, act)).sum())


def _to_act(x, act):
    if act == synth.ACT_BF16:
        return synth.f32_to_bf16_bits(x.astype(np.float32))   # x already holds bf16 values
    return x.astype(np.float32)


def _from_act(raw, act):
    if act == synth.ACT_BF16:
        return synth.bf16_bits_to_f32(raw.view(np.uint16)).astype(np.float64)
    return raw.view(np.float32).astype(np.float64)


def probe_step(P, gpu_ids, orc_ids, toks, poss, tag, check=True, kv_inject=None):
    """Oracle step (with its per-layer trace) for each sequence, then one GPU probe step in
    which every kernel reads the oracle's own inputs; every kernel's output is compared
    with the oracle's.  Returns the oracle outputs [(next, logits, hidden, trace)].
    kv_inject (layer -> (k, v), float32 [B][kv_dim]) replaces the new position's injected
    k and v, which the GPU then rounds to the KV type as it appends them."""
    t = P.torch
    s = P.shape
    B = len(gpu_ids)
    act = s.act
    outs = [P.orc.step(P.oslot(o), int(toks[b]), int(poss[b]), want_trace=True)
            for b, o in enumerate(orc_ids)]
    fields = {name: (off, n) for name, off, n in P.orc.trace_fields()}
    layout, rec = dtd.probe_fields(s, B)
    inj = np.zeros((s.n_layers, rec), dtype=np.uint8)
    # k and v are injected as the oracle's stored (already rounded) cache entries: the GPU
    # stores round_kv of what it is given, which reproduces them exactly in every KV format
    stored = [[P.orc.kv_read(P.oslot(o), l, int(poss[b]), 1) for l in range(s.n_layers)]
              for b, o in enumerate(orc_ids)]
    for l in range(s.n_layers):
        for name, off, n, is_act in layout:
            o0, _ = fields[name]
            if name in ("k", "v") and kv_inject is not None:
                vals = np.asarray(kv_inject[l][0 if name == "k" else 1], dtype=np.float64).reshape(B, n)
            elif name in ("k", "v"):
                vals = np.stack([stored[b][l][0 if name == "k" else 1].reshape(-1) for b in range(B)])
            else:
                vals = np.stack([outs[b][3][l, o0:o0 + n] for b in range(B)])   # [B][n] float64
            if is_act:
                vals = oracle.round_act_n(vals, act).reshape(B, n)
                raw = _to_act(vals, act)
            else:
                raw = vals.astype(np.float32)
            inj[l, off:off + raw.nbytes] = raw.view(np.uint8).reshape(-1)
    inj_d = t.as_tensor(inj).to(P.dev)
    cap_d = t.zeros_like(inj_d)
    tok = t.as_tensor(np.asarray(toks, dtype=np.int32)).to(P.dev)
    nxt = t.empty(B, dtype=t.int32, device=P.dev)
    logits = t.empty((B, s.vocab), dtype=t.float32, device=P.dev)
    dtd.dtd_debug_decode_probe(P.eng.h, list(gpu_ids), tok.data_ptr(), inj_d.data_ptr(), cap_d.data_ptr(),
                               nxt.data_ptr(), logits.data_ptr())
    t.cuda.synchronize()
    if not check:
        return outs
    cap = cap_d.cpu().numpy()
    lg = logits.cpu().numpy()
    ng = nxt.cpu().numpy()
    flips = 0
    worst = 0.0
    for l in range(s.n_layers):
        for name, off, n, is_act in layout:
            if name == "x_in":
                continue
            o0, _ = fields[name]
            for b in range(B):
                raw = cap[l, off + b * n * (2 if (is_act and act == synth.ACT_BF16) else 4):][
                    : n * (2 if (is_act and act == synth.ACT_BF16) else 4)]
                r = outs[b][3][l, o0:o0 + n]
                where = f"{tag} seq {gpu_ids[b]} layer {l} {name}"
                if is_act:
                    flips += check_rounded(where, _from_act(raw.copy(), act), r, act)
                else:
                    e = normwise(raw.copy().view(np.float32), r)
                    worst = max(worst, e)
                    assert e <= TOL, f"{where}: {e:.3e}"
    # the KV the GPU appended at the new position equals the oracle's, bit for bit
    for b, o in enumerate(orc_ids):
        for l in range(s.n_layers):
            kr, vr, ksr, vsr = P.orc.kv_read_raw(P.oslot(o), l, int(poss[b]), 1)
            kg, vg = np.empty_like(kr), np.empty_like(vr)
            ksg = vsg = None
            if ksr is not None:
                ksg, vsg = np.empty_like(ksr), np.empty_like(vsr)
            dtd.dtd_debug_kv_read(P.eng.h, gpu_ids[b], l, int(poss[b]), 1, kg, vg, ksg, vsg)
            assert np.array_equal(kg, kr) and np.array_equal(vg, vr), f"{tag} seq {gpu_ids[b]} layer {l} KV"
            if ksr is not None:
                assert np.array_equal(ksg, ksr) and np.array_equal(vsg, vsr), f"{tag} KV scales"
    for b in range(B):
        no, lo = outs[b][0], outs[b][1]
        e = normwise(lg[b], lo)
        delta = np.abs(lg[b].astype(np.float64) - lo).max()
        assert e <= TOL, f"{tag} seq {gpu_ids[b]} logits {e:.3e}"
        if top2_margin(lo) > 2 * delta:
            assert int(ng[b]) == no, f"{tag} seq {gpu_ids[b]}: token {int(ng[b])} vs {no}"
    P.probe_stats = getattr(P, "probe_stats", [0, 0.0])
    P.probe_stats[0] += flips
    P.probe_stats[1] = max(P.probe_stats[1], worst)
    return outs


def stored_kv_reference(shape, x32):
    """The cache entry the KV rounding of the int8-KV, bf16 and fp32 readings makes of
    float32 vectors x32 [..., n_kv_heads * head_dim], from the oracle's own rounding
    functions: (codes or bits [..., Hkv, hd], fp16 scale bits [..., Hkv] or None)."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    x = x.reshape(x.shape[:-1] + (shape.n_kv_heads, shape.head_dim))
    if shape.kvfmt == synth.KV_F32:
        return x.astype(np.float32), None
    if shape.kvfmt == synth.KV_BF16:
        return np.vectorize(oracle.double_to_bf16, otypes=[np.uint16])(x), None
    q = np.empty(x.shape, dtype=np.int8)
    sc = np.empty(x.shape[:-1], dtype=np.uint16)
    for idx in np.ndindex(*x.shape[:-1]):
        q[idx], sc[idx] = oracle.kv_quant_i8(x[idx])
    return q, sc


def kv_encoding_step(shape, ref, ref_scales):
    """One step of the stored KV encoding at each of the oracle's decoded values `ref`
    (fp32 or bf16: one unit in the last place; int8: one code at the row's fp16 scale, plus
    the scale itself landing one fp16 step the other way)."""
    mag = np.abs(np.asarray(ref, np.float64))
    if shape.kvfmt == synth.KV_F32:
        return np.ldexp(1.0, np.frexp(np.maximum(mag, 1e-30))[1] - 24)
    if shape.kvfmt == synth.KV_BF16:
        return np.ldexp(1.0, np.frexp(np.maximum(mag, 1e-30))[1] - 8)
    return ref_scales.view(np.float16).astype(np.float64)[..., None] + mag * 2.0 ** -10


def kv_excess(g, ref, step):
    """(largest |g - ref| beyond one encoding step, relative to max |ref|; the fraction of
    elements more than half a step apart)"""
    ref = np.asarray(ref, np.float64)
    diff = np.abs(np.asarray(g, np.float64) - ref)
    den = np.abs(ref).max()
    den = den if den > 0 else 1.0
    return float(np.maximum(diff - step, 0.0).max() / den), float(np.mean(diff > 0.5 * step))


def stored_kv_error(P, seq_id, layer, start, n, other=None):
    """The GPU's stored K/V of positions [start, start + n) against the oracle's.

    Each side rounds its own fp32 k/v to the KV encoding, and the two unrounded values differ
    by accumulation-order error, so a stored element may sit one encoding step away from the
    oracle's (a rounding boundary fell between them).  Returns (excess, flipped): the largest
    difference beyond that one step, relative to max |oracle|, and the fraction of elements
    that differ by more than half a step.  With `other` (a second oracle model that ran the
    same tokens in slot 0) also returns that model's excess over the oracle, measured the
    same way.
    """
    s = P.shape
    k0, v0, ks0, vs0 = P.orc.kv_read_raw(P.oslot(seq_id), layer, start, n)
    ko, vo = np.empty_like(k0), np.empty_like(v0)
    kso = vso = None
    if ks0 is not None:
        kso, vso = np.empty_like(ks0), np.empty_like(vs0)
    dtd.dtd_debug_kv_read(P.eng.h, seq_id, layer, start, n, ko, vo, kso, vso)
    kd, vd = P.orc.kv_read(P.oslot(seq_id), layer, start, n)
    o2 = other.kv_read(0, layer, start, n) if other is not None else (None, None)
    worst, flip, env = 0.0, 0.0, 0.0
    for raw, sc, ref, osc, alt in ((ko, kso, kd, ks0, o2[0]), (vo, vso, vd, vs0, o2[1])):
        if s.kvfmt == synth.KV_F32:
            g = raw.astype(np.float64)
        elif s.kvfmt == synth.KV_BF16:
            g = synth.bf16_bits_to_f32(raw).astype(np.float64)
        else:
            g = raw.astype(np.float64) * sc.view(np.float16).astype(np.float64)[..., None]
        step = kv_encoding_step(s, ref, osc)
        e, f = kv_excess(g, ref, step)
        worst, flip = max(worst, e), max(flip, f)
        if alt is not None:
            env = max(env, kv_excess(alt, ref, step)[0])
    return (worst, flip, env) if other is not None else (worst, flip)
