"""ctypes wrapper of the plain CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by ``__graft_entry__.smoke()`` and by the
CPU-baseline leg of ``bench.py``.  The GPU library never imports, links or runs it.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

W_INT8_ROW, W_Q8_0, W_BF16, W_Q4_0 = 0, 1, 2, 3
ACT_F32, ACT_BF16 = 0, 1
KV_F32, KV_BF16, KV_I8 = 0, 1, 2


def build(verbose: bool = False) -> str:
    """Compile oracle.c with gcc (plain C11, OpenMP, no FMA contraction, no fast-math)."""
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", LIB_PATH + ".tmp",
           os.path.join(_HERE, "oracle.c"), "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


class _Cfg(C.Structure):
    _fields_ = [("dim", C.c_int32), ("n_layers", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn_dim", C.c_int32),
                ("vocab", C.c_int32), ("rms_eps", C.c_double), ("rope_theta", C.c_double),
                ("tied", C.c_int32), ("wfmt", C.c_int32), ("act", C.c_int32),
                ("kvfmt", C.c_int32), ("max_ctx", C.c_int32), ("max_seqs", C.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = C.CDLL(LIB_PATH)
        P, I32, D, U16 = C.c_void_p, C.c_int32, C.c_double, C.c_uint16
        L.orc_bf16_to_double.argtypes, L.orc_bf16_to_double.restype = [U16], D
        L.orc_double_to_bf16.argtypes, L.orc_double_to_bf16.restype = [D], U16
        L.orc_fp16_to_double.argtypes, L.orc_fp16_to_double.restype = [U16], D
        L.orc_double_to_fp16.argtypes, L.orc_double_to_fp16.restype = [D], U16
        L.orc_round_act.argtypes, L.orc_round_act.restype = [D, I32], D
        L.orc_round_act_n.argtypes, L.orc_round_act_n.restype = [P, I32, I32, P], None
        L.orc_rmsnorm.argtypes, L.orc_rmsnorm.restype = [P, P, I32, D, P], None
        L.orc_dequant_row.argtypes, L.orc_dequant_row.restype = [I32, P, P, I32, I32, P], None
        L.orc_gemv.argtypes, L.orc_gemv.restype = [I32, P, P, I32, I32, P, P], None
        L.orc_rope.argtypes, L.orc_rope.restype = [P, I32, I32, D], None
        L.orc_attention.argtypes, L.orc_attention.restype = [P, I32, I32, I32, I32, P, P, P], None
        L.orc_silu.argtypes, L.orc_silu.restype = [D], D
        L.orc_argmax_f32.argtypes, L.orc_argmax_f32.restype = [P, I32], I32
        L.orc_kv_quant_i8.argtypes, L.orc_kv_quant_i8.restype = [P, I32, P, P], None
        L.orc_create.argtypes, L.orc_create.restype = [C.POINTER(_Cfg)], P
        L.orc_destroy.argtypes, L.orc_destroy.restype = [P], None
        L.orc_set_tensor.argtypes, L.orc_set_tensor.restype = [P, C.c_char_p, P, P], I32
        L.orc_ready.argtypes, L.orc_ready.restype = [P], I32
        L.orc_step.argtypes, L.orc_step.restype = [P, I32, I32, I32, P, P, P], I32
        L.orc_step_kept.argtypes, L.orc_step_kept.restype = [P, I32, I32, I32, P, I32, P, P], I32
        L.orc_attention_kept.argtypes, L.orc_attention_kept.restype = [P, I32, I32, I32, I32, P, P, P, P, P], None
        L.orc_trace_len.argtypes, L.orc_trace_len.restype = [P], I32
        L.orc_kv_write.argtypes, L.orc_kv_write.restype = [P, I32, I32, I32, I32, P, P, P, P], I32
        L.orc_kv_read.argtypes, L.orc_kv_read.restype = [P, I32, I32, I32, I32, P, P], I32
        L.orc_kv_read_raw.argtypes, L.orc_kv_read_raw.restype = [P, I32, I32, I32, I32, P, P, P, P], I32
        L.orc_full_forward.argtypes, L.orc_full_forward.restype = [P, P, I32, P, P], I32
        L.orc_num_threads.argtypes, L.orc_num_threads.restype = [], I32
        L.orc_set_num_threads.argtypes, L.orc_set_num_threads.restype = [I32], None
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---- single operations -------------------------------------------------------------

def bf16_to_double(b: int) -> float:
    return lib().orc_bf16_to_double(int(b))


def double_to_bf16(x: float) -> int:
    return int(lib().orc_double_to_bf16(float(x)))


def fp16_to_double(h: int) -> float:
    return lib().orc_fp16_to_double(int(h))


def double_to_fp16(x: float) -> int:
    return int(lib().orc_double_to_fp16(float(x)))


def round_act(x: float, act: int) -> float:
    return lib().orc_round_act(float(x), int(act))


def round_act_n(x, act: int):
    x = _c(x, np.float64)
    out = np.empty_like(x)
    lib().orc_round_act_n(_p(x), x.size, int(act), _p(out))
    return out


def rmsnorm(x, g, eps):
    x = _c(x, np.float64); g = _c(g, np.float32)
    out = np.empty_like(x)
    lib().orc_rmsnorm(_p(x), _p(g), x.size, float(eps), _p(out))
    return out


def _cols(wfmt, w):
    """matrix width: Q4_0 codes pack two columns per byte"""
    return w.shape[1] * 2 if wfmt == W_Q4_0 else w.shape[1]


def dequant_row(wfmt, w, s, r):
    w = np.ascontiguousarray(w)
    s = None if s is None else np.ascontiguousarray(s)
    out = np.empty(_cols(wfmt, w), dtype=np.float32)
    lib().orc_dequant_row(wfmt, _p(w), _p(s), _cols(wfmt, w), int(r), _p(out))
    return out


def attention_kept(q, hkv, K, V, keep, prob=None):
    """q [hq][d]; K, V [n][hkv][d]; keep [n] -> out [hq][d] (prob [n] accumulated in place)"""
    q = _c(q, np.float64); K = _c(K, np.float64); V = _c(V, np.float64)
    keep = np.ascontiguousarray(keep, dtype=np.uint8)
    hq, d = q.shape
    out = np.empty((hq, d), dtype=np.float64)
    lib().orc_attention_kept(_p(q), hq, hkv, d, K.shape[0], _p(K), _p(V), _p(keep), _p(out),
                             _p(prob) if prob is not None else None)
    return out


def gemv(wfmt, w, s, x):
    w = np.ascontiguousarray(w)
    s = None if s is None else np.ascontiguousarray(s)
    x = _c(x, np.float64)
    out = np.empty(w.shape[0], dtype=np.float64)
    lib().orc_gemv(wfmt, _p(w), _p(s), w.shape[0], _cols(wfmt, w), _p(x), _p(out))
    return out


def rope(v, pos, theta):
    v = _c(v, np.float64).copy()
    lib().orc_rope(_p(v), v.size, int(pos), float(theta))
    return v


def attention(q, K, V):
    """q [hq, d]; K, V [n_pos, hkv, d] -> [hq, d]"""
    q = _c(q, np.float64); K = _c(K, np.float64); V = _c(V, np.float64)
    hq, d = q.shape
    n_pos, hkv, _ = K.shape
    out = np.empty_like(q)
    lib().orc_attention(_p(q), hq, hkv, d, n_pos, _p(K), _p(V), _p(out))
    return out


def silu(z):
    return lib().orc_silu(float(z))


def argmax_f32(v):
    v = _c(v, np.float32)
    return int(lib().orc_argmax_f32(_p(v), v.size))


def kv_quant_i8(x):
    x = _c(x, np.float64)
    q = np.empty(x.size, dtype=np.int8)
    s = np.empty(1, dtype=np.uint16)
    lib().orc_kv_quant_i8(_p(x), x.size, _p(q), _p(s))
    return q, int(s[0])


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    lib().orc_set_num_threads(int(n))


# ---- whole model ---------------------------------------------------------------------

class Model:
    """The oracle model bound to host weight arrays (kept alive here)."""

    def __init__(self, shape, weights: Dict[str, Dict[str, np.ndarray]], max_ctx: int,
                 max_seqs: int = 1):
        self.shape = shape
        cfg = _Cfg(shape.dim, shape.n_layers, shape.n_q_heads, shape.n_kv_heads,
                   shape.head_dim, shape.ffn_dim, shape.vocab, float(shape.rms_eps),
                   float(shape.rope_theta), int(bool(shape.tied)), shape.wfmt, shape.act,
                   shape.kvfmt, int(max_ctx), int(max_seqs))
        self._h = lib().orc_create(C.byref(cfg))
        if not self._h:
            raise ValueError("oracle rejected the configuration")
        self._keep = []
        for name, parts in weights.items():
            if "g" in parts:
                p0, p1 = _c(parts["g"], np.float32), None
            elif "w" in parts:
                p0, p1 = np.ascontiguousarray(parts["w"]), None
            else:
                p0, p1 = np.ascontiguousarray(parts["q"]), np.ascontiguousarray(parts["s"])
            self._keep += [p0, p1]
            rc = lib().orc_set_tensor(self._h, name.encode(), _p(p0), _p(p1))
            if rc != 0:
                raise ValueError(f"oracle does not know tensor {name}")
        if not lib().orc_ready(self._h):
            raise ValueError("oracle: weights incomplete")
        self.max_ctx = max_ctx

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            lib().orc_destroy(h)
            self._h = None

    def step(self, seq: int, token: int, pos: int, want_logits=True, want_hidden=False,
             want_trace=False):
        """Returns (next token, logits, hidden) or, with want_trace, (next, logits, hidden,
        trace [L][record]) -- see trace_fields for the record layout."""
        s = self.shape
        logits = np.empty(s.vocab, dtype=np.float32) if want_logits else None
        hidden = np.empty((s.n_layers + 1, s.dim), dtype=np.float64) if (want_hidden or want_trace) else None
        trace = None
        if want_trace:
            trace = np.empty((s.n_layers, lib().orc_trace_len(self._h)), dtype=np.float64)
        nxt = lib().orc_step(self._h, int(seq), int(token), int(pos), _p(logits), _p(hidden), _p(trace))
        if nxt < 0:
            raise RuntimeError(f"orc_step failed: {nxt}")
        if want_trace:
            return nxt, logits, hidden, trace
        return nxt, logits, hidden

    def step_kept(self, seq: int, token: int, pos: int, keep, score_layers: int, scores):
        """orc_step over the kept positions (keep: bool/uint8 [pos + 1]); adds the attention
        probabilities of the last score_layers layers to scores (float64 [pos + 1], in place).
        Returns (next token, logits)."""
        keep = np.ascontiguousarray(keep, dtype=np.uint8)
        assert keep.size == pos + 1 and scores.dtype == np.float64 and scores.size >= pos + 1
        logits = np.empty(self.shape.vocab, dtype=np.float32)
        nxt = lib().orc_step_kept(self._h, int(seq), int(token), int(pos), _p(keep), int(score_layers),
                                  _p(scores), _p(logits))
        if nxt < 0:
            raise RuntimeError(f"orc_step_kept failed: {nxt}")
        return nxt, logits

    def trace_fields(self):
        """(name, offset, length) of each field of a trace record."""
        s = self.shape
        out, off = [], 0
        for name, n in (("x_in", s.dim), ("xn", s.dim), ("q", s.q_dim), ("k", s.kv_dim),
                        ("v", s.kv_dim), ("o", s.q_dim), ("x_mid", s.dim), ("xn2", s.dim),
                        ("h", s.ffn_dim), ("x_out", s.dim)):
            out.append((name, off, n))
            off += n
        return out

    def kv_write(self, seq, layer, pos0, k, v, ks=None, vs=None):
        k = np.ascontiguousarray(k); v = np.ascontiguousarray(v)
        ks = None if ks is None else _c(ks, np.float16).view(np.uint16)
        vs = None if vs is None else _c(vs, np.float16).view(np.uint16)
        rc = lib().orc_kv_write(self._h, seq, layer, pos0, k.shape[0], _p(k), _p(v), _p(ks), _p(vs))
        if rc != 0:
            raise RuntimeError(f"orc_kv_write failed: {rc}")

    def kv_read(self, seq, layer, pos0, n):
        s = self.shape
        k = np.empty((n, s.n_kv_heads, s.head_dim), dtype=np.float64)
        v = np.empty_like(k)
        rc = lib().orc_kv_read(self._h, seq, layer, pos0, n, _p(k), _p(v))
        if rc != 0:
            raise RuntimeError(f"orc_kv_read failed: {rc}")
        return k, v

    def kv_read_raw(self, seq, layer, pos0, n):
        s = self.shape
        dt = {KV_F32: np.float32, KV_BF16: np.uint16, KV_I8: np.int8}[s.kvfmt]
        k = np.empty((n, s.n_kv_heads, s.head_dim), dtype=dt)
        v = np.empty_like(k)
        ks = vs = None
        if s.kvfmt == KV_I8:
            ks = np.empty((n, s.n_kv_heads), dtype=np.uint16)
            vs = np.empty_like(ks)
        rc = lib().orc_kv_read_raw(self._h, seq, layer, pos0, n, _p(k), _p(v), _p(ks), _p(vs))
        if rc != 0:
            raise RuntimeError(f"orc_kv_read_raw failed: {rc}")
        return k, v, ks, vs

    def full_forward(self, tokens, want_hidden=False):
        s = self.shape
        t = _c(tokens, np.int32)
        logits = np.empty(s.vocab, dtype=np.float32)
        hidden = np.empty((s.n_layers + 1, s.dim), dtype=np.float64) if want_hidden else None
        nxt = lib().orc_full_forward(self._h, _p(t), t.size, _p(logits), _p(hidden))
        if nxt < 0:
            raise RuntimeError(f"orc_full_forward failed: {nxt}")
        return nxt, logits, hidden
