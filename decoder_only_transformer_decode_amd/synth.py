"""Seeded synthetic inputs for the decode step: model shapes, random weights, prompts,
context lengths and KV contents.

This module holds no arithmetic of the decode step itself.  It draws random numbers and
encodes them into the stored weight formats that the step consumes (the offline export
step that the pages describe before inference starts):

* int8 weight-only, one fp32 scale per output row, ``scale = max|row| / 127``
  ("从 smollm3.go 看 LLM inference", section "int8 weight-only quantization").
* Q8_0: blocks of 32 int8 weights sharing one fp16 scale ("Go 语言原本" 20.2.4, the int8
  figure of one f16 scale per 32 weights).
* bf16: round-to-nearest-even of the float32 draw.

Both the HIP path and the CPU oracle receive the same bytes from here; neither imports
the other.  Everything is a pure function of (shape, seed).
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Dict, List, Optional

import numpy as np

W_INT8_ROW, W_Q8_0, W_BF16, W_Q4_0 = 0, 1, 2, 3
ACT_F32, ACT_BF16 = 0, 1
KV_F32, KV_BF16, KV_I8 = 0, 1, 2

WFMT_NAMES = {W_INT8_ROW: "int8-row", W_Q8_0: "q8_0", W_BF16: "bf16", W_Q4_0: "q4_0"}
ACT_NAMES = {ACT_F32: "f32", ACT_BF16: "bf16"}
KV_NAMES = {KV_F32: "f32", KV_BF16: "bf16", KV_I8: "int8+fp16 scale per token and head"}

Q8_BLOCK = 32


@dataclasses.dataclass(frozen=True)
class ModelShape:
    """Shape and storage formats of one Llama-family decoder."""
    name: str
    dim: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    wfmt: int
    act: int
    kvfmt: int
    tied: bool = False
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def replace(self, **kw) -> "ModelShape":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class Workload:
    """A decode workload on one model shape."""
    shape: ModelShape
    batch: int
    prompt_len: int          # tokens prefilled per sequence before decoding
    context: int             # attended context the workload decodes up to / at
    block_size: int = 16     # KV block size (tokens per block)
    seed_index: int = 0      # weights use seed 1234 + seed_index
    note: str = ""
    # the context before the decoded steps is synthetic stored KV (the workload names a
    # context to decode at, not a prompt to prefill)
    synthetic_prefix: bool = False
    # batched: each sequence's context drawn by context_lengths() (else all at `context`)
    mixed_contexts: bool = False


# The five model shapes and workloads this library is measured and checked on.
TINY = Workload(
    ModelShape("tiny-llama", 256, 4, 8, 2, 32, 688, 4096, W_INT8_ROW, ACT_F32, KV_F32),
    batch=1, prompt_len=32, context=64, seed_index=0,
    note="32-token random prompt, then 32 greedy decode steps")
SMOLLM3_3B = Workload(
    ModelShape("smollm3-3b-shaped", 2048, 36, 16, 4, 128, 11008, 128256,
               W_INT8_ROW, ACT_BF16, KV_BF16),
    batch=1, prompt_len=512, context=2048, seed_index=1,
    note="prefill 512 random tokens, then decode to context 2048")
LLAMA32_1B = Workload(
    ModelShape("llama-3.2-1b-shaped", 2048, 16, 32, 8, 64, 8192, 128256,
               W_Q8_0, ACT_BF16, KV_BF16, tied=True),
    batch=1, prompt_len=4032, context=4096, seed_index=2,
    note="decode at context 4096 (tied embeddings)", synthetic_prefix=True)
QWEN3_8B = Workload(
    ModelShape("qwen3-8b-shaped", 4096, 36, 32, 8, 128, 12288, 151936,
               W_BF16, ACT_BF16, KV_BF16),
    batch=64, prompt_len=0, context=4096, block_size=16, seed_index=3,
    note="batch 64, paged KV block 16, per-sequence context uniform in [512, 4096]",
    synthetic_prefix=True, mixed_contexts=True)
LLAMA3_8B = Workload(
    ModelShape("llama-3-8b-shaped", 4096, 32, 32, 8, 128, 14336, 128256,
               W_INT8_ROW, ACT_BF16, KV_I8),
    batch=32, prompt_len=16384 - 16, context=16384, seed_index=4,
    note="batch 32 at context 16384, int8 KV with an fp16 scale per token and head", synthetic_prefix=True)

WORKLOADS = [TINY, SMOLLM3_3B, LLAMA32_1B, QWEN3_8B, LLAMA3_8B]
BY_NAME = {w.shape.name: w for w in WORKLOADS}


def weights_seed(w: Workload) -> int:
    return 1234 + w.seed_index


# ---------------------------------------------------------------------------------------
# tensor inventory
# ---------------------------------------------------------------------------------------

def matrix_shapes(s: ModelShape) -> Dict[str, tuple]:
    """Every weight matrix by name, as [rows (outputs), cols (inputs)], row-major."""
    out = {"tok_emb": (s.vocab, s.dim)}
    for i in range(s.n_layers):
        out[f"L{i}.wq"] = (s.q_dim, s.dim)
        out[f"L{i}.wk"] = (s.kv_dim, s.dim)
        out[f"L{i}.wv"] = (s.kv_dim, s.dim)
        out[f"L{i}.wo"] = (s.dim, s.q_dim)
        out[f"L{i}.w_gate"] = (s.ffn_dim, s.dim)
        out[f"L{i}.w_up"] = (s.ffn_dim, s.dim)
        out[f"L{i}.w_down"] = (s.dim, s.ffn_dim)
    if not s.tied:
        out["lm_head"] = (s.vocab, s.dim)
    return out


def norm_names(s: ModelShape) -> List[str]:
    return ([f"L{i}.attn_norm" for i in range(s.n_layers)]
            + [f"L{i}.ffn_norm" for i in range(s.n_layers)] + ["final_norm"])


def tensor_order(s: ModelShape) -> List[str]:
    """Fixed order used to derive one independent random stream per tensor."""
    names = ["tok_emb"]
    for i in range(s.n_layers):
        names += [f"L{i}.attn_norm", f"L{i}.wq", f"L{i}.wk", f"L{i}.wv", f"L{i}.wo",
                  f"L{i}.ffn_norm", f"L{i}.w_gate", f"L{i}.w_up", f"L{i}.w_down"]
    names.append("final_norm")
    if not s.tied:
        names.append("lm_head")
    return names


# ---------------------------------------------------------------------------------------
# storage encodings (offline export; the decode step only ever reads their output)
# ---------------------------------------------------------------------------------------

def _round_half_away(x32: np.ndarray) -> np.ndarray:
    """C ``roundf`` semantics (ties away from zero) of float32 values |x| < 2^22, in place.

    x + copysign(0.5, x) is exact in float32 unless it crosses into the next binade, and
    there any rounding lands on the same integer after truncation, so no float64 needed."""
    x32 += np.copysign(np.float32(0.5), x32)
    return np.trunc(x32, out=x32)


def f32_to_bf16_bits(w: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(w, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


_CHUNK_ROWS = 512


def encode_int8_row(w: np.ndarray):
    """Per-output-row symmetric int8: scale = max|row|/127 (fp32), q = roundf(w/scale)
    clamped to [-127, 127]; an all-zero row gets scale 0 and codes 0."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    r, c = w.shape
    q = np.empty((r, c), dtype=np.int8)
    s = np.empty(r, dtype=np.float32)
    for r0 in range(0, r, _CHUNK_ROWS):
        blk = w[r0:r0 + _CHUNK_ROWS]
        amax = np.abs(blk).max(axis=1)
        sc = (amax / np.float32(127.0)).astype(np.float32)
        safe = np.where(sc > 0, sc, np.float32(1.0)).astype(np.float32)
        y = blk / safe[:, None]
        _round_half_away(y)
        np.clip(y, -127, 127, out=y)
        y[sc == 0, :] = 0
        q[r0:r0 + _CHUNK_ROWS] = y
        s[r0:r0 + _CHUNK_ROWS] = sc
    return q, s


def encode_q8_0(w: np.ndarray):
    """Q8_0: each run of 32 columns shares one fp16 scale d = fp16(max|blk|/127);
    q = roundf(w / float(d)) clamped to [-127, 127]; d == 0 gives q == 0."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    r, c = w.shape
    assert c % Q8_BLOCK == 0
    q = np.empty((r, c), dtype=np.int8)
    d = np.empty((r, c // Q8_BLOCK), dtype=np.float16)
    for r0 in range(0, r, _CHUNK_ROWS):
        wb = w[r0:r0 + _CHUNK_ROWS].reshape(-1, c // Q8_BLOCK, Q8_BLOCK)
        amax = np.abs(wb).max(axis=2)
        d16 = (amax / np.float32(127.0)).astype(np.float32).astype(np.float16)
        d32 = d16.astype(np.float32)
        safe = np.where(d32 > 0, d32, np.float32(1.0)).astype(np.float32)
        y = wb / safe[:, :, None]
        _round_half_away(y)
        np.clip(y, -127, 127, out=y)
        y[d32 == 0] = 0
        q[r0:r0 + _CHUNK_ROWS] = y.reshape(-1, c)
        d[r0:r0 + _CHUNK_ROWS] = d16
    return q, d


def encode_q4_0(w: np.ndarray):
    """Q4_0 ("Go 语言原本" 20.2.4): blocks of 32 columns; d = fp16(m / -8) where m is the
    block's element of largest magnitude (the first one on ties); q = roundf(w / float(d))
    + 8 clamped to [0, 15] (d == 0 gives q == 8); byte j of a block's 16 holds q[j] in its
    low 4 bits and q[j + 16] in its high 4 bits.  Returns codes [rows][cols/2] uint8 and
    scales [rows][cols/32] fp16."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    r, c = w.shape
    assert c % Q8_BLOCK == 0
    nb = c // Q8_BLOCK
    codes = np.empty((r, c // 2), dtype=np.uint8)
    d = np.empty((r, nb), dtype=np.float16)
    for r0 in range(0, r, _CHUNK_ROWS):
        wb = w[r0:r0 + _CHUNK_ROWS].reshape(-1, nb, Q8_BLOCK)
        m = np.take_along_axis(wb, np.abs(wb).argmax(axis=2)[:, :, None], axis=2)[:, :, 0]
        d16 = (m / np.float32(-8.0)).astype(np.float32).astype(np.float16)
        d32 = d16.astype(np.float32)
        safe = np.where(d32 != 0, d32, np.float32(1.0)).astype(np.float32)
        y = wb / safe[:, :, None]
        _round_half_away(y)
        y += np.float32(8.0)
        np.clip(y, 0, 15, out=y)
        y[d32 == 0] = 8
        q = y.astype(np.uint8)
        packed = q[:, :, :16] | (q[:, :, 16:] << np.uint8(4))
        codes[r0:r0 + _CHUNK_ROWS] = packed.reshape(-1, c // 2)
        d[r0:r0 + _CHUNK_ROWS] = d16
    return codes, d


def encode_matrix(w: np.ndarray, wfmt: int) -> Dict[str, np.ndarray]:
    """Planar parts as handed to load_weights: '.q' + '.s' (int8-row / Q8_0 / Q4_0) or '.w'
    (bf16)."""
    if wfmt == W_INT8_ROW:
        q, s = encode_int8_row(w)
        return {"q": q, "s": s}
    if wfmt == W_Q8_0:
        q, d = encode_q8_0(w)
        return {"q": q, "s": d}
    if wfmt == W_Q4_0:
        q, d = encode_q4_0(w)
        return {"q": q, "s": d}
    if wfmt == W_BF16:
        return {"w": f32_to_bf16_bits(w)}
    raise ValueError(f"unknown weight format {wfmt}")


# ---------------------------------------------------------------------------------------
# generation
# ---------------------------------------------------------------------------------------

def _stream(seed: int, index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, index])))


def _gen_one(s: ModelShape, seed: int, idx: int, name: str, shapes: Dict[str, tuple]):
    g = _stream(seed, idx)
    if name.endswith("_norm"):
        gain = (1.0 + 0.02 * g.standard_normal(s.dim, dtype=np.float32)).astype(np.float32)
        return name, {"g": gain}
    r, c = shapes[name]
    # drawn in row chunks from the one stream: the same values as one (r, c) draw
    parts = None
    for r0 in range(0, r, _CHUNK_ROWS):
        n = min(_CHUNK_ROWS, r - r0)
        w = g.standard_normal((n, c), dtype=np.float32)
        w *= np.float32(0.02)
        enc = encode_matrix(w, s.wfmt)
        if parts is None:
            parts = {k: np.empty((r,) + v.shape[1:], dtype=v.dtype) for k, v in enc.items()}
        for k, v in enc.items():
            parts[k][r0:r0 + n] = v
    return name, parts


def gen_weights(s: ModelShape, seed: int, threads: Optional[int] = None) -> Dict[str, Dict[str, np.ndarray]]:
    """All weights of a model: matrices ~ N(0, 0.02^2) then encoded in ``s.wfmt``;
    norm gains 1 + N(0, 0.02^2) in fp32.  One independent PCG64 stream per tensor."""
    shapes = matrix_shapes(s)
    order = tensor_order(s)
    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    out: Dict[str, Dict[str, np.ndarray]] = {}
    with _cf.ThreadPoolExecutor(max_workers=threads) as ex:
        futs = [ex.submit(_gen_one, s, seed, i, n, shapes) for i, n in enumerate(order)]
        for f in futs:
            name, parts = f.result()
            out[name] = parts
    return out


def flat_tensors(weights: Dict[str, Dict[str, np.ndarray]]) -> Dict[str, np.ndarray]:
    """'name.part' -> array, the naming the C ABI's load_weights expects."""
    return {f"{n}.{p}": a for n, parts in weights.items() for p, a in parts.items()}


def prompt_tokens(vocab: int, n: int, seed: int = 42) -> np.ndarray:
    return _stream(seed, 0).integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def context_lengths(batch: int, lo: int = 512, hi: int = 4096, seed: int = 7) -> np.ndarray:
    """Per-sequence context lengths, uniform on the integers lo..hi inclusive."""
    return _stream(seed, 0).integers(lo, hi + 1, size=batch, dtype=np.int64).astype(np.int32)


def synthetic_kv(s: ModelShape, n_pos: int, seed: int, layer: int, seq: int = 0):
    """K and V rows for n_pos positions, [n_pos, n_kv_heads, head_dim], values
    N(0, (0.02*sqrt(dim))^2) (the spread a k/v projection of a unit-RMS input with
    N(0, 0.02^2) weights has), encoded in the model's KV format:
    f32 -> float32 arrays; bf16 -> uint16 bit arrays; int8 -> (int8 q, fp16 scale per
    position and head) built with the same per-(token, head) symmetric rule the cache uses.
    Returns (k, v, k_scale, v_scale); scales are None unless the format is int8."""
    g = _stream(seed, 1 + layer * 65536 + seq)
    sd = np.float32(0.02 * np.sqrt(s.dim))
    shp = (n_pos, s.n_kv_heads, s.head_dim)
    k = (g.standard_normal(shp, dtype=np.float32) * sd).astype(np.float32)
    v = (g.standard_normal(shp, dtype=np.float32) * sd).astype(np.float32)
    if s.kvfmt == KV_F32:
        return k, v, None, None
    if s.kvfmt == KV_BF16:
        return f32_to_bf16_bits(k), f32_to_bf16_bits(v), None, None
    if s.kvfmt == KV_I8:
        # Synthetic stored bytes: a random int8 code with a random positive fp16 scale is
        # a valid cache entry whatever rule produced it.
        kq = g.integers(-127, 128, size=shp, dtype=np.int64).astype(np.int8)
        vq = g.integers(-127, 128, size=shp, dtype=np.int64).astype(np.int8)
        ks = (np.abs(k).max(axis=2) / np.float32(127.0)).astype(np.float16)
        vs = (np.abs(v).max(axis=2) / np.float32(127.0)).astype(np.float16)
        return kq, vq, ks, vs
    raise ValueError(s.kvfmt)


def tiny_shape(**kw) -> ModelShape:
    """A very small shape for brute-force oracle checks."""
    base = ModelShape("micro", 64, 2, 4, 2, 16, 96, 97, W_INT8_ROW, ACT_F32, KV_F32)
    return base.replace(**kw)


def sampling_logits(rows: int, vocab: int, seed: int = 0) -> np.ndarray:
    """fp32 logit rows [rows][vocab] for sampler tests: Gaussian with a spread that varies by
    row (0.5 to 8), plus rows with many exact ties (multiples of 0.25), rows with a few -inf
    and NaN entries, a row with one dominant logit and a row of equal logits."""
    rng = np.random.default_rng(seed)
    spreads = [0.5, 1.0, 2.0, 4.0, 8.0]
    out = np.empty((rows, vocab), np.float32)
    for r in range(rows):
        x = rng.standard_normal(vocab) * spreads[r % len(spreads)]
        if r % 7 == 3:
            x = np.round(x * 4) / 4
        if r % 11 == 5 and vocab > 8:
            bad = rng.choice(vocab, size=max(2, vocab // 100), replace=False)
            x[bad[: len(bad) // 2]] = -np.inf
            x[bad[len(bad) // 2:]] = np.nan
        if r % 13 == 8:
            x[rng.integers(vocab)] = x.max() + 20.0
        if r % 17 == 9:
            x[:] = 1.5
        out[r] = x.astype(np.float32)
    return out


def bench_logits(rows: int, vocab: int, seed: int = 0) -> np.ndarray:
    """fp32 logit rows [rows][vocab], N(0, 3^2): the sampler's timing input."""
    return (_stream(seed, 1).standard_normal((rows, vocab)) * 3.0).astype(np.float32)
