"""The C-ABI library: loads without a GPU, exports every declared symbol, and its host-only
entry points (configuration checks, weight manifest) agree with the input recipe."""
import ctypes as C

import numpy as np
import pytest

from decoder_only_transformer_decode_amd import dtd, synth


def test_library_exports_every_declared_function():
    lib = dtd.load()
    names = dtd.declared_functions()
    assert len(names) >= 17
    for n in names:
        assert hasattr(lib, n), n
        assert n in dtd._SIGS, f"binding lacks {n}"


@pytest.mark.parametrize("w", synth.WORKLOADS, ids=lambda w: w.shape.name)
def test_expected_tensors_match_input_recipe(w):
    s = w.shape.replace(n_layers=2)
    cfg = dtd.config_from_shape(s, max_ctx=256, max_batch=min(w.batch, 64))
    st, msg = dtd.dtd_validate_config(cfg)
    assert st == dtd.DTD_OK, msg
    specs = {sp.name.decode(): sp for sp in dtd.dtd_expected_tensors(cfg)}
    shapes = synth.matrix_shapes(s)
    # sizes implied by the recipe's encodings, without generating the weights
    want = {}
    for name, (r, c) in shapes.items():
        if s.wfmt == synth.W_BF16:
            want[name + ".w"] = r * c * 2
        else:
            want[name + ".q"] = r * c
            want[name + ".s"] = r * 4 if s.wfmt == synth.W_INT8_ROW else r * (c // 32) * 2
    for n in synth.norm_names(s):
        want[n + ".g"] = s.dim * 4
    assert {k: v.nbytes for k, v in specs.items()} == want


def test_expected_tensors_match_generated_bytes():
    s = synth.tiny_shape(wfmt=synth.W_Q8_0, tied=True)
    flat = synth.flat_tensors(synth.gen_weights(s, 3))
    cfg = dtd.config_from_shape(s, max_ctx=64)
    specs = {sp.name.decode(): sp.nbytes for sp in dtd.dtd_expected_tensors(cfg)}
    assert specs == {k: v.nbytes for k, v in flat.items()}


def _cfg(**kw):
    c = dtd.config_from_shape(synth.TINY.shape, max_ctx=64)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("kw,status", [
    (dict(), dtd.DTD_OK),
    (dict(abi_version=2), dtd.DTD_E_ARG),
    (dict(n_kv_heads=3), dtd.DTD_E_ARG),
    (dict(head_dim=50), dtd.DTD_E_UNSUPPORTED),
    (dict(head_dim=256, dim=512), dtd.DTD_E_UNSUPPORTED),
    (dict(dim=0), dtd.DTD_E_ARG),
    (dict(wfmt=7), dtd.DTD_E_ARG),
    (dict(max_batch=65), dtd.DTD_E_UNSUPPORTED),
    (dict(max_batch=0), dtd.DTD_E_ARG),
    (dict(kv_block_size=0), dtd.DTD_E_ARG),
    (dict(dim=264), dtd.DTD_E_UNSUPPORTED),            # not a multiple of 16
    (dict(wfmt=1, dim=272), dtd.DTD_E_ARG),            # Q8_0 needs multiples of 32
    (dict(rope_theta=0.0), dtd.DTD_E_ARG),
    (dict(n_q_heads=128, n_kv_heads=1, head_dim=32, dim=4096), dtd.DTD_E_UNSUPPORTED),  # G*hd > 2048
])
def test_validate_config(kw, status):
    st, msg = dtd.dtd_validate_config(_cfg(**kw))
    assert st == status, msg
    if status != dtd.DTD_OK:
        assert msg


def test_expected_tensors_rejects_bad_config():
    lib = dtd.load()
    bad = _cfg(n_kv_heads=3)
    assert lib.dtd_expected_tensors(C.byref(bad), None, 0) == dtd.DTD_E_ARG


def test_null_engine_calls_are_errors_not_crashes():
    lib = dtd.load()
    assert lib.dtd_reset_seq(None, 1) == dtd.DTD_E_ARG
    assert lib.dtd_seq_len(None, 1) == dtd.DTD_E_ARG
    assert lib.dtd_decode_step(None, 1, None, None, None, None) == dtd.DTD_E_ARG
    assert lib.dtd_set_sampler(None, 1, None) == dtd.DTD_E_ARG
    assert lib.dtd_last_error(None) == b"null engine"
    lib.dtd_destroy(None)


def test_rejected_create_leaves_its_reason_for_last_error():
    # the config is checked before any device call, so this runs without a GPU
    lib = dtd.load()
    bad = _cfg(n_kv_heads=3)
    h = C.c_void_p(1)
    assert lib.dtd_create(C.byref(bad), None, C.byref(h)) == dtd.DTD_E_ARG
    assert not h.value
    assert b"n_kv_heads 3" in lib.dtd_last_error(None)
    with pytest.raises(dtd.DtdError, match="n_kv_heads 3"):
        dtd.dtd_create(bad, 0)


def test_sample_checks_its_arguments_before_any_device_call():
    # null pointers and out-of-range sizes are rejected on the host (no GPU needed)
    lib = dtd.load()
    s = (dtd.dtd_sampler * 1)(dtd.sampler(temperature=1.0))
    c = (C.c_int64 * 1)(0)
    assert lib.dtd_sample(None, 10, 1, 10, s, c, None, None) == dtd.DTD_E_ARG
    assert b"sample:" in lib.dtd_last_error(None)
    assert lib.dtd_sample(None, 10, 0, 10, None, None, None, None) == dtd.DTD_E_ARG
    assert lib.dtd_sample(None, 10, 65, 10, None, None, None, None) == dtd.DTD_E_ARG


def test_prefix_cache_and_scheduler_calls_check_their_arguments():
    lib = dtd.load()
    assert lib.dtd_set_prefix_cache(None, 4) == dtd.DTD_E_ARG
    assert lib.dtd_prefix_cache_add(None, 1, None, 1) == dtd.DTD_E_ARG
    cfg = dtd.dtd_config()
    assert lib.dtd_get_config(None, C.byref(cfg)) == dtd.DTD_E_ARG
    assert lib.dtd_get_stream(None) is None
    h = C.c_void_p(1)
    assert lib.dtd_sched_create(None, 0, C.byref(h)) == dtd.DTD_E_ARG and not h.value
    rid = C.c_int64()
    assert lib.dtd_sched_submit(None, None, 1, 1, -1, None, C.byref(rid)) == dtd.DTD_E_ARG
    assert lib.dtd_sched_step(None, None) == dtd.DTD_E_ARG
    assert lib.dtd_sched_result(None, 0, None, 0, None) == dtd.DTD_E_ARG
    assert lib.dtd_sched_wait(None, 0, 0) == dtd.DTD_E_ARG
    assert lib.dtd_sched_last_error(None) == b"null scheduler"
    lib.dtd_sched_destroy(None)


def test_attention_chunk_plan_worked_example():
    # contexts 600, 1000 and 4096, 8 KV heads, 8 chunks at most, 64 resident waves: the
    # shortest bound T (multiples of 16 from max(64, 5696 * 8 / 64 = 712 -> 720, 4096 / 8 =
    # 512)) whose chunks fit 64 waves is 832: 4096 -> 5 chunks of 832 (T = 720 .. 816 still
    # needs 6), 1000 -> 2 of 512, 600 -> 1 of 608; 8 chunks x 8 heads = 64 waves
    ct, cend = dtd.plan_attention_chunks([599, 999, 4095], 8, 8, 64)
    assert list(ct) == [608, 512, 832] and list(cend) == [1, 3, 8]
    # equal contexts 16384 at batch 32, 2048 slots: chunks of 2048, 8 per sequence, one wave
    # per slot
    ct, cend = dtd.plan_attention_chunks([16383] * 32, 8, 16, 2048)
    assert set(ct) == {2048} and cend[-1] * 8 == 2048
    # a short context alone: at least 64 positions per chunk
    ct, cend = dtd.plan_attention_chunks([99], 8, 64, 2048)
    assert list(ct) == [64] and list(cend) == [2]


@pytest.mark.parametrize("seed", range(6))
def test_attention_chunk_plan_invariants(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 65))
    max_ctx = int(rng.choice([256, 4096, 16384, 32768]))
    hkv = int(rng.choice([1, 2, 8]))
    nch = -(-max_ctx // int(rng.choice([64, 512, 1024, 2048])))
    slots = int(rng.choice([64, 1024, 2048]))
    pos = rng.integers(0, max_ctx, B).astype(np.int32)
    ct, cend = dtd.plan_attention_chunks(pos, hkv, nch, slots)
    ln = pos.astype(np.int64) + 1
    n = -(-ln // ct)
    assert np.all(ct % 16 == 0) and np.all(ct >= 16) and np.all(ct <= 2048)
    assert np.all(n <= nch) and np.array_equal(np.cumsum(n), cend)
    # the chunks of a sequence are equal but for the last, which is never empty
    assert np.all((n - 1) * ct < ln) and np.all(ln <= n * ct)
    # they fit the slots whenever chunks of 2048 would
    if int(np.sum(-(-ln // 2048))) * hkv <= slots:
        assert int(cend[-1]) * hkv <= slots
    with pytest.raises(dtd.DtdError):
        dtd.plan_attention_chunks(np.array([max_ctx], np.int32) * 0 + nch * 2048, hkv, nch, slots)
