"""Thin ctypes binding of libdtd.so (include/dtd.h), with the same names.

Argument marshalling only: every step of the decode path runs in the HIP library.
PyTorch supplies device memory and the stream.  The library must be built
(``python -m decoder_only_transformer_decode_amd.build`` or ``__graft_entry__.build()``);
``load()`` raises if it is missing -- there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
import re
from typing import Dict, List, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdtd.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "dtd.h")

ABI_VERSION = 1
DTD_OK, DTD_E_ARG, DTD_E_STATE, DTD_E_NOSEQ, DTD_E_CTX, DTD_E_KVFULL, DTD_E_OOM, DTD_E_HIP, \
    DTD_E_UNSUPPORTED = 0, -1, -2, -3, -4, -5, -6, -7, -8
STATUS_NAMES = {0: "DTD_OK", -1: "DTD_E_ARG", -2: "DTD_E_STATE", -3: "DTD_E_NOSEQ", -4: "DTD_E_CTX",
                -5: "DTD_E_KVFULL", -6: "DTD_E_OOM", -7: "DTD_E_HIP", -8: "DTD_E_UNSUPPORTED"}
KERNEL_GATE_UP, KERNEL_DOWN, KERNEL_QKV, KERNEL_O, KERNEL_ATTN, KERNEL_HEAD, KERNEL_STEP = range(7)
PATH_AUTO, PATH_PER_KERNEL, PATH_PERSISTENT = 0, 1, 2


class dtd_config(C.Structure):
    _fields_ = [("abi_version", C.c_int32), ("dim", C.c_int32), ("n_layers", C.c_int32),
                ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("ffn_dim", C.c_int32), ("vocab", C.c_int32), ("rms_eps", C.c_float),
                ("rope_theta", C.c_float), ("tied_embeddings", C.c_int32), ("wfmt", C.c_int32),
                ("act", C.c_int32), ("kvfmt", C.c_int32), ("kv_block_size", C.c_int32),
                ("kv_num_blocks", C.c_int32), ("max_seqs", C.c_int32), ("max_ctx", C.c_int32),
                ("max_batch", C.c_int32)]


class dtd_tensor(C.Structure):
    _fields_ = [("name", C.c_char_p), ("data", C.c_void_p), ("nbytes", C.c_int64),
                ("on_device", C.c_int32)]


class dtd_tensor_spec(C.Structure):
    _fields_ = [("name", C.c_char * 48), ("nbytes", C.c_int64), ("rows", C.c_int32),
                ("cols", C.c_int32), ("elem", C.c_int32)]


class dtd_sampler(C.Structure):
    _fields_ = [("temperature", C.c_float), ("top_k", C.c_int32), ("top_p", C.c_float),
                ("min_p", C.c_float), ("seed", C.c_uint64)]


class DtdError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None

_P, _I32, _I64, _U64 = C.c_void_p, C.c_int32, C.c_int64, C.c_uint64
_SIGS = {
    "dtd_validate_config": ([C.POINTER(dtd_config), C.c_char_p, _I32], _I32),
    "dtd_expected_tensors": ([C.POINTER(dtd_config), C.POINTER(dtd_tensor_spec), _I32], _I32),
    "dtd_create": ([C.POINTER(dtd_config), _P, C.POINTER(_P)], _I32),
    "dtd_load_weights": ([_P, C.POINTER(dtd_tensor), _I32], _I32),
    "dtd_prefill": ([_P, _I64, _P, _I32, _P, _P], _I32),
    "dtd_decode_step": ([_P, _I32, C.POINTER(_I64), _P, _P, _P], _I32),
    "dtd_decode_step_noalloc": ([_P, _I32, C.POINTER(_I64), _P, _P, _P], _I32),
    "dtd_reset_seq": ([_P, _I64], _I32),
    "dtd_sample": ([_P, _I64, _I32, _I32, C.POINTER(dtd_sampler), C.POINTER(_I64), _P, _P], _I32),
    "dtd_set_sampler": ([_P, _I64, C.POINTER(dtd_sampler)], _I32),
    "dtd_set_prefix_cache": ([_P, _I32], _I32),
    "dtd_prefix_cache_add": ([_P, _I64, C.POINTER(_I32), _I32], _I32),
    "dtd_get_config": ([_P, C.POINTER(dtd_config)], _I32),
    "dtd_get_stream": ([_P], _P),
    "dtd_debug_prefix_reused": ([_P, _I64], _I32),
    "dtd_debug_kv_blocks_free": ([_P], _I32),
    "dtd_debug_prefix_entries": ([_P], _I32),
    "dtd_set_kv_budget": ([_P, _I64, _I32, _I32, _I32, _I32], _I32),
    "dtd_debug_kv_positions": ([_P, _I64, C.POINTER(_I32), _I32], _I32),
    "dtd_debug_kv_scores": ([_P, _I64, C.POINTER(C.c_float), _I32], _I32),
    "dtd_sched_create": ([_P, _I32, C.POINTER(_P)], _I32),
    "dtd_sched_destroy": ([_P], None),
    "dtd_sched_submit": ([_P, C.POINTER(_I32), _I32, _I32, _I32, C.POINTER(dtd_sampler), C.POINTER(_I64)], _I32),
    "dtd_sched_step": ([_P, C.POINTER(_I32)], _I32),
    "dtd_sched_start": ([_P], _I32),
    "dtd_sched_stop": ([_P], _I32),
    "dtd_sched_wait": ([_P, _I64, _I32], _I32),
    "dtd_sched_result": ([_P, _I64, C.POINTER(_I32), _I32, C.POINTER(_I32)], _I32),
    "dtd_sched_release": ([_P, _I64], _I32),
    "dtd_sched_last_error": ([_P], C.c_char_p),
    "dtd_seq_len": ([_P, _I64], _I32),
    "dtd_check_device_errors": ([_P], _I32),
    "dtd_destroy": ([_P], None),
    "dtd_last_error": ([_P], C.c_char_p),
    "dtd_debug_dequant_rows": ([_P, C.c_char_p, _I32, _I32, _P], _I32),
    "dtd_debug_capture_hidden": ([_P, _I32, _P], _I32),
    "dtd_debug_kv_write": ([_P, _I64, _I32, _I32, _I32, _P, _P, _P, _P], _I32),
    "dtd_debug_kv_read": ([_P, _I64, _I32, _I32, _I32, _P, _P, _P, _P], _I32),
    "dtd_debug_kv_fill": ([_P, _I64, _I32, _U64], _I32),
    "dtd_debug_kernel_timing": ([_P, _I32, _I32, C.POINTER(C.c_double), C.POINTER(_I64)], _I32),
    "dtd_debug_decode_probe": ([_P, _I32, C.POINTER(_I64), _P, _P, _P, _P, _P], _I32),
    "dtd_debug_probe_record_bytes": ([C.POINTER(dtd_config), _I32], _I64),
    "dtd_debug_set_path": ([_P, _I32], _I32),
    "dtd_debug_uses_persistent": ([_P, _I32], _I32),
    "dtd_debug_step_kernel_shape": ([_P], _I32),
    "dtd_debug_plan_attention_chunks": ([_I32, C.POINTER(_I32), _I32, _I32, _I32, C.POINTER(_I32), C.POINTER(_I32)],
                                        _I32),
    "dtd_debug_stream_read": ([_P, _I64, _I32, _P, C.POINTER(C.c_double)], _I32),
}


def load(path: str = LIB_PATH):
    """Opens libdtd.so.  Raises FileNotFoundError if it has not been built."""
    global _lib
    if _lib is None:
        # torch ships its own HIP runtime under the same soname; it has to be in the process
        # first, so that the library binds to that one runtime (two runtimes in one process
        # do not share devices or streams)
        import torch  # noqa: F401
        if not os.path.exists(path):
            raise FileNotFoundError(f"{path} is missing: build it with __graft_entry__.build()")
        L = C.CDLL(path)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes, f.restype = args, res
        _lib = L
    return _lib


def declared_functions(header: str = HEADER) -> List[str]:
    """Names of the functions include/dtd.h declares."""
    with open(header) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return sorted(set(re.findall(r"\b(dtd_[a-z_]+)\s*\(", text)))


# ---------------------------------------------------------------------------------------
# plain wrappers with the C names (raise DtdError on failure)
# ---------------------------------------------------------------------------------------

def _check(eng, st):
    if st != DTD_OK:
        msg = load().dtd_last_error(eng).decode() if eng else ""
        raise DtdError(st, msg)


def config_from_shape(shape, *, max_ctx: int, max_seqs: int = 1, max_batch: int = 1,
                      kv_block_size: int = 16, kv_num_blocks: Optional[int] = None) -> dtd_config:
    if kv_num_blocks is None:
        kv_num_blocks = max_seqs * ((max_ctx + kv_block_size - 1) // kv_block_size)
    return dtd_config(ABI_VERSION, shape.dim, shape.n_layers, shape.n_q_heads, shape.n_kv_heads,
                      shape.head_dim, shape.ffn_dim, shape.vocab, shape.rms_eps, shape.rope_theta,
                      int(bool(shape.tied)), shape.wfmt, shape.act, shape.kvfmt, kv_block_size,
                      kv_num_blocks, max_seqs, max_ctx, max_batch)


def dtd_validate_config(cfg: dtd_config):
    buf = C.create_string_buffer(256)
    st = load().dtd_validate_config(C.byref(cfg), buf, 256)
    return st, buf.value.decode()


def dtd_expected_tensors(cfg: dtd_config) -> List[dtd_tensor_spec]:
    n = load().dtd_expected_tensors(C.byref(cfg), None, 0)
    if n < 0:
        raise DtdError(n, "invalid configuration")
    arr = (dtd_tensor_spec * n)()
    load().dtd_expected_tensors(C.byref(cfg), arr, n)
    return list(arr)


def dtd_create(cfg: dtd_config, stream: int):
    h = C.c_void_p()
    st = load().dtd_create(C.byref(cfg), C.c_void_p(stream), C.byref(h))
    if st != DTD_OK:
        raise DtdError(st, load().dtd_last_error(None).decode() or "dtd_create failed")
    return h


def dtd_load_weights(eng, tensors: Dict[str, np.ndarray]):
    arrs = []
    t = (dtd_tensor * len(tensors))()
    for i, (name, a) in enumerate(tensors.items()):
        if hasattr(a, "data_ptr"):   # torch tensor on the device
            t[i] = dtd_tensor(name.encode(), a.data_ptr(), a.numel() * a.element_size(), 1)
        else:
            a = np.ascontiguousarray(a)
            arrs.append(a)
            t[i] = dtd_tensor(name.encode(), a.ctypes.data, a.nbytes, 0)
    _check(eng, load().dtd_load_weights(eng, t, len(tensors)))


def dtd_prefill(eng, seq_id: int, tokens_dev: int, n: int, next_token_dev: int, logits_dev: int = 0):
    _check(eng, load().dtd_prefill(eng, seq_id, C.c_void_p(tokens_dev), n, C.c_void_p(next_token_dev),
                                   C.c_void_p(logits_dev or None)))


def dtd_decode_step(eng, seq_ids: Sequence[int], tokens_dev: int, next_tokens_dev: int,
                    logits_dev: int = 0):
    ids = (C.c_int64 * len(seq_ids))(*seq_ids)
    _check(eng, load().dtd_decode_step(eng, len(seq_ids), ids, C.c_void_p(tokens_dev),
                                       C.c_void_p(next_tokens_dev), C.c_void_p(logits_dev or None)))


def dtd_reset_seq(eng, seq_id: int):
    _check(eng, load().dtd_reset_seq(eng, seq_id))


def dtd_seq_len(eng, seq_id: int) -> int:
    return int(load().dtd_seq_len(eng, seq_id))


def dtd_decode_step_noalloc(eng, seq_ids: Sequence[int], tokens_dev: int, next_tokens_dev: int,
                            logits_dev: int = 0):
    ids = (C.c_int64 * len(seq_ids))(*seq_ids)
    _check(eng, load().dtd_decode_step_noalloc(eng, len(seq_ids), ids, C.c_void_p(tokens_dev),
                                               C.c_void_p(next_tokens_dev), C.c_void_p(logits_dev or None)))


def dtd_check_device_errors(eng):
    _check(eng, load().dtd_check_device_errors(eng))


def dtd_destroy(eng):
    load().dtd_destroy(eng)


def dtd_last_error(eng) -> str:
    return load().dtd_last_error(eng).decode()


def dtd_debug_dequant_rows(eng, matrix: str, r0: int, nrows: int, out_dev: int):
    _check(eng, load().dtd_debug_dequant_rows(eng, matrix.encode(), r0, nrows, C.c_void_p(out_dev)))


def dtd_debug_capture_hidden(eng, enable: bool, out_dev: int = 0):
    _check(eng, load().dtd_debug_capture_hidden(eng, int(enable), C.c_void_p(out_dev or None)))


def _np_ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def dtd_debug_kv_write(eng, seq_id, layer, pos0, k, v, ks=None, vs=None):
    k, v = np.ascontiguousarray(k), np.ascontiguousarray(v)
    ks = None if ks is None else np.ascontiguousarray(ks)
    vs = None if vs is None else np.ascontiguousarray(vs)
    _check(eng, load().dtd_debug_kv_write(eng, seq_id, layer, pos0, k.shape[0], _np_ptr(k), _np_ptr(v),
                                          _np_ptr(ks), _np_ptr(vs)))


def dtd_debug_kv_read(eng, seq_id, layer, pos0, n, k_out, v_out, ks_out=None, vs_out=None):
    _check(eng, load().dtd_debug_kv_read(eng, seq_id, layer, pos0, n, _np_ptr(k_out), _np_ptr(v_out),
                                         _np_ptr(ks_out), _np_ptr(vs_out)))


PROBE_FIELDS = ("x_in", "xn", "q", "k", "v", "o", "x_mid", "xn2", "h", "x_out")
PROBE_ACT_FIELDS = ("xn", "o", "xn2", "h")


def probe_fields(shape, batch: int):
    """(name, byte offset, n, is_act) of each field of a probe record."""
    ab = 2 if shape.act == 1 else 4
    sizes = dict(x_in=shape.dim, xn=shape.dim, q=shape.q_dim, k=shape.kv_dim, v=shape.kv_dim,
                 o=shape.q_dim, x_mid=shape.dim, xn2=shape.dim, h=shape.ffn_dim, x_out=shape.dim)
    out, off = [], 0
    for f in PROBE_FIELDS:
        act = f in PROBE_ACT_FIELDS
        out.append((f, off, sizes[f], act))
        off += batch * sizes[f] * (ab if act else 4)
    return out, off


def dtd_debug_probe_record_bytes(cfg: dtd_config, batch: int) -> int:
    return int(load().dtd_debug_probe_record_bytes(C.byref(cfg), batch))


def dtd_debug_decode_probe(eng, seq_ids: Sequence[int], tokens_dev: int, inject_dev: int,
                           capture_dev: int, next_tokens_dev: int, logits_dev: int = 0):
    ids = (C.c_int64 * len(seq_ids))(*seq_ids)
    _check(eng, load().dtd_debug_decode_probe(
        eng, len(seq_ids), ids, C.c_void_p(tokens_dev), C.c_void_p(inject_dev),
        C.c_void_p(capture_dev), C.c_void_p(next_tokens_dev), C.c_void_p(logits_dev or None)))


def dtd_debug_set_path(eng, path: int):
    _check(eng, load().dtd_debug_set_path(eng, path))


def dtd_debug_uses_persistent(eng, batch: int) -> bool:
    return bool(load().dtd_debug_uses_persistent(eng, batch))


def dtd_debug_step_kernel_shape(eng) -> int:
    return int(load().dtd_debug_step_kernel_shape(eng))


def dtd_debug_kv_fill(eng, seq_id: int, length: int, seed: int):
    _check(eng, load().dtd_debug_kv_fill(eng, seq_id, length, seed))


def dtd_debug_kernel_timing(eng, kind: int, enable: bool):
    ms, cnt = C.c_double(), C.c_int64()
    _check(eng, load().dtd_debug_kernel_timing(eng, kind, int(enable), C.byref(ms), C.byref(cnt)))
    return ms.value, cnt.value


# ---------------------------------------------------------------------------------------
# convenience object over the same calls (torch tensors for device buffers)
# ---------------------------------------------------------------------------------------

class Engine:
    """Owns one dtd_engine on the current torch device and stream."""

    def __init__(self, shape, *, max_ctx: int, max_seqs: int = 1, max_batch: int = 1,
                 kv_block_size: int = 16, kv_num_blocks: Optional[int] = None, stream=None):
        import torch
        self.torch = torch
        self.shape = shape
        self.cfg = config_from_shape(shape, max_ctx=max_ctx, max_seqs=max_seqs, max_batch=max_batch,
                                     kv_block_size=kv_block_size, kv_num_blocks=kv_num_blocks)
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        self.h = dtd_create(self.cfg, self.stream.cuda_stream)
        self.device = torch.device("cuda", torch.cuda.current_device())

    def close(self):
        if getattr(self, "h", None):
            dtd_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def load_weights(self, weights_flat: Dict[str, np.ndarray]):
        dtd_load_weights(self.h, weights_flat)

    def prefill(self, seq_id: int, tokens, want_logits: bool = False):
        t = self.torch
        tok = tokens if isinstance(tokens, t.Tensor) else t.as_tensor(np.asarray(tokens, dtype=np.int32))
        tok = tok.to(device=self.device, dtype=t.int32).contiguous()
        nxt = t.empty(1, dtype=t.int32, device=self.device)
        logits = t.empty(self.shape.vocab, dtype=t.float32, device=self.device) if want_logits else None
        dtd_prefill(self.h, seq_id, tok.data_ptr(), tok.numel(), nxt.data_ptr(),
                    logits.data_ptr() if logits is not None else 0)
        self._inflight = (tok, nxt, logits)   # alive until the next call
        return nxt, logits

    def decode_step(self, seq_ids: Sequence[int], tokens, want_logits: bool = False, out=None):
        t = self.torch
        tok = tokens if isinstance(tokens, t.Tensor) else t.as_tensor(np.asarray(tokens, dtype=np.int32))
        tok = tok.to(device=self.device, dtype=t.int32).contiguous()
        nxt = out if out is not None else t.empty(len(seq_ids), dtype=t.int32, device=self.device)
        logits = (t.empty((len(seq_ids), self.shape.vocab), dtype=t.float32, device=self.device)
                  if want_logits else None)
        dtd_decode_step(self.h, list(seq_ids), tok.data_ptr(), nxt.data_ptr(),
                        logits.data_ptr() if logits is not None else 0)
        self._inflight = (tok, nxt, logits)   # alive until the next call
        return nxt, logits

    def reset_seq(self, seq_id: int):
        dtd_reset_seq(self.h, seq_id)

    def set_sampler(self, seq_id: int, s: Optional["dtd_sampler"]):
        dtd_set_sampler(self.h, seq_id, s)

    def set_prefix_cache(self, max_entries: int):
        _check(self.h, load().dtd_set_prefix_cache(self.h, max_entries))

    def prefix_cache_add(self, seq_id: int, tokens):
        arr = np.ascontiguousarray(tokens, dtype=np.int32)
        _check(self.h, load().dtd_prefix_cache_add(self.h, seq_id, arr.ctypes.data_as(C.POINTER(C.c_int32)),
                                                   arr.size))

    def prefix_reused(self, seq_id: int) -> int:
        return load().dtd_debug_prefix_reused(self.h, seq_id)

    def kv_blocks_free(self) -> int:
        return load().dtd_debug_kv_blocks_free(self.h)

    def prefix_entries(self) -> int:
        return load().dtd_debug_prefix_entries(self.h)

    def set_kv_budget(self, seq_id: int, budget: int, n_initial: int = 4, n_recent: int = 16,
                      score_layers: int = 1):
        _check(self.h, load().dtd_set_kv_budget(self.h, seq_id, budget, n_initial, n_recent, score_layers))

    def kv_positions(self, seq_id: int):
        cap = self.cfg.max_ctx
        buf = (C.c_int32 * cap)()
        n = load().dtd_debug_kv_positions(self.h, seq_id, buf, cap)
        if n < 0:
            raise DtdError(n, "dtd_debug_kv_positions")
        return [int(buf[i]) for i in range(n)]

    def kv_scores(self, seq_id: int):
        cap = self.cfg.max_ctx
        buf = (C.c_float * cap)()
        n = load().dtd_debug_kv_scores(self.h, seq_id, buf, cap)
        if n < 0:
            raise DtdError(n, load().dtd_last_error(self.h).decode())
        return np.array(buf[:n], dtype=np.float32)

    def seq_len(self, seq_id: int) -> int:
        return dtd_seq_len(self.h, seq_id)


def dtd_debug_stream_read(buf_ptr: int, nbytes: int, reps: int, stream: int) -> float:
    """Streaming-read bandwidth (GB/s) over a device buffer."""
    out = C.c_double()
    st = load().dtd_debug_stream_read(C.c_void_p(buf_ptr), nbytes, reps, C.c_void_p(stream), C.byref(out))
    if st != DTD_OK:
        raise DtdError(st, load().dtd_last_error(None).decode())
    return out.value


def sampler(temperature: float = 0.0, top_k: int = 0, top_p: float = 1.0, min_p: float = 0.0,
            seed: int = 0) -> dtd_sampler:
    return dtd_sampler(temperature, top_k, top_p, min_p, seed)


def dtd_sample(logits_ptr: int, row_stride: int, batch: int, vocab: int, samplers: Sequence[dtd_sampler],
               counters: Sequence[int], tokens_ptr: int, stream: int = 0):
    """One sampled token per row into tokens_ptr (device int32 [batch]); asynchronous."""
    arr = (dtd_sampler * batch)(*samplers)
    ctr = (C.c_int64 * batch)(*[int(c) for c in counters])
    st = load().dtd_sample(C.c_void_p(logits_ptr), row_stride, batch, vocab, arr, ctr, C.c_void_p(tokens_ptr),
                           C.c_void_p(stream))
    if st != DTD_OK:
        raise DtdError(st, load().dtd_last_error(None).decode())


def dtd_set_sampler(h, seq_id: int, s: Optional[dtd_sampler]):
    _check(h, load().dtd_set_sampler(h, seq_id, C.byref(s) if s is not None else None))


class Scheduler:
    """Continuous batching over an Engine (dtd_sched_*): submit requests, then step, or run
    the scheduler's own loop with start() and wait()."""

    def __init__(self, eng: "Engine", prompt_budget: int = 0):
        self.eng = eng
        h = C.c_void_p()
        st = load().dtd_sched_create(eng.h, prompt_budget, C.byref(h))
        if st != DTD_OK:
            raise DtdError(st, "dtd_sched_create")
        self.h = h

    def _check(self, st):
        if st != DTD_OK:
            raise DtdError(st, load().dtd_sched_last_error(self.h).decode())

    def submit(self, prompt, max_new_tokens: int, stop_token: int = -1,
               sampler: Optional[dtd_sampler] = None) -> int:
        arr = np.ascontiguousarray(prompt, dtype=np.int32)
        rid = C.c_int64()
        st = load().dtd_sched_submit(self.h, arr.ctypes.data_as(C.POINTER(C.c_int32)), arr.size, max_new_tokens,
                                     stop_token, C.byref(sampler) if sampler is not None else None, C.byref(rid))
        if st != DTD_OK:
            raise DtdError(st, "dtd_sched_submit")
        return rid.value

    def step(self) -> int:
        pending = C.c_int32()
        self._check(load().dtd_sched_step(self.h, C.byref(pending)))
        return pending.value

    def run(self, max_steps: int = 1 << 20) -> int:
        """Steps until nothing is queued or running; returns the number of steps."""
        for i in range(max_steps):
            if self.step() == 0:
                return i + 1
        raise RuntimeError("scheduler did not drain")

    def start(self):
        self._check(load().dtd_sched_start(self.h))

    def stop(self):
        self._check(load().dtd_sched_stop(self.h))

    def wait(self, rid: int, timeout_ms: int = -1) -> int:
        return load().dtd_sched_wait(self.h, rid, timeout_ms)

    def result(self, rid: int):
        done = C.c_int32()
        cap = 1 << 16
        buf = (C.c_int32 * cap)()
        n = load().dtd_sched_result(self.h, rid, buf, cap, C.byref(done))
        if n < 0:
            raise DtdError(n, load().dtd_sched_last_error(self.h).decode())
        return [int(buf[i]) for i in range(min(n, cap))], bool(done.value)

    def release(self, rid: int):
        self._check(load().dtd_sched_release(self.h, rid))

    def close(self):
        if getattr(self, "h", None):
            load().dtd_sched_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def plan_attention_chunks(pos, n_kv_heads: int, max_chunks: int, slots: int):
    """the batched decode attention's per-sequence chunk lengths and running chunk counts
    for contexts pos[b] + 1 (host only); returns (ct, cend)"""
    import numpy as np
    p = np.ascontiguousarray(pos, dtype=np.int32)
    ct = np.zeros(len(p), np.int32)
    cend = np.zeros(len(p), np.int32)
    ip = C.POINTER(_I32)
    n = load().dtd_debug_plan_attention_chunks(len(p), p.ctypes.data_as(ip), n_kv_heads, max_chunks, slots,
                                               ct.ctypes.data_as(ip), cend.ctypes.data_as(ip))
    if n < 0:
        raise DtdError(n, "dtd_debug_plan_attention_chunks")
    return ct, cend
