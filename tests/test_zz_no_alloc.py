"""dtd_decode_step_noalloc (the entry point that allocates nothing, for callers that cannot:
code under HIP graph capture, tight serving loops) against dtd_decode_step: the same greedy
tokens and logits on calls in a row, each with a smaller batch than the one before, and a
clear error for a call whose work memory would not fit its static scratch."""
import numpy as np
import pytest

from decoder_only_transformer_decode_amd import dtd, synth
from _pair import TOL, need_gpu, normwise, top2_margin

pytestmark = pytest.mark.gpu

_GRID = synth.ModelShape("grid", 320, 2, 10, 2, 32, 608, 1000, synth.W_INT8_ROW, synth.ACT_BF16, synth.KV_BF16)


def _engine(s, w, **kw):
    eng = dtd.Engine(s, **kw)
    eng.load_weights(synth.flat_tensors(w))
    return eng


@pytest.mark.parametrize("kw", [dict(), dict(kvfmt=synth.KV_I8), dict(wfmt=synth.W_BF16, act=synth.ACT_F32)],
                         ids=["int8row-bf16kv", "int8kv", "bf16w-f32act"])
def test_noalloc_step_matches_decode_step(kw):
    need_gpu()
    import torch
    s = _GRID.replace(**kw)
    w = synth.gen_weights(s, 12)
    A = _engine(s, w, max_ctx=96, max_seqs=4, max_batch=4)
    B = _engine(s, w, max_ctx=96, max_seqs=4, max_batch=4)
    toks = {}
    for sid, n in ((0, 5), (1, 40), (2, 71)):
        prompt = synth.prompt_tokens(s.vocab, n, seed=sid + 1)
        na, _ = A.prefill(sid, prompt)
        nb, _ = B.prefill(sid, prompt)
        torch.cuda.synchronize()
        assert int(na.item()) == int(nb.item())
        toks[sid] = int(na.item())
    dev = A.device
    for call, ids in enumerate(([0, 1, 2], [2, 0], [1])):     # each call smaller than the last
        t = torch.tensor([toks[i] for i in ids], dtype=torch.int32, device=dev)
        na = torch.empty(len(ids), dtype=torch.int32, device=dev)
        nb = torch.empty_like(na)
        la = torch.empty((len(ids), s.vocab), dtype=torch.float32, device=dev)
        lb = torch.empty_like(la)
        dtd.dtd_decode_step(A.h, ids, t.data_ptr(), na.data_ptr(), la.data_ptr())
        dtd.dtd_decode_step_noalloc(B.h, ids, t.data_ptr(), nb.data_ptr(), lb.data_ptr())
        torch.cuda.synchronize()
        ga, gb = la.cpu().numpy(), lb.cpu().numpy()
        ta, tb = na.cpu().numpy(), nb.cpu().numpy()
        for b, sid in enumerate(ids):
            err = normwise(gb[b], ga[b])
            delta = float(np.abs(gb[b].astype(np.float64) - ga[b]).max())
            print(f"call {call} batch {len(ids)} seq {sid}: logits err {err:.2e}, tokens {tb[b]}/{ta[b]}", flush=True)
            assert err <= TOL
            if top2_margin(ga[b]) > 2 * delta:
                assert tb[b] == ta[b]
            if len(ids) > 1:
                # both run the one-kernel-per-sub-step schedule: identical arithmetic
                assert np.array_equal(gb[b], ga[b]) and tb[b] == ta[b]
            toks[sid] = int(ta[b])
        assert A.seq_len(ids[0]) == B.seq_len(ids[0])
    A.close()
    B.close()


def test_noalloc_rejects_work_beyond_its_scratch():
    need_gpu()
    import torch
    s = _GRID
    w = synth.gen_weights(s, 13)
    # 64 sequences at a very long max_ctx need more attention partials than the scratch holds
    eng = _engine(s, w, max_ctx=1_000_000, max_seqs=64, max_batch=64, kv_num_blocks=64)
    ids = list(range(64))
    t = torch.zeros(64, dtype=torch.int32, device=eng.device)
    lib = dtd.load()
    arr = (dtd.C.c_int64 * 64)(*ids)
    st = lib.dtd_decode_step_noalloc(eng.h, 64, arr, t.data_ptr(), t.data_ptr(), None)
    assert st == dtd.DTD_E_UNSUPPORTED
    assert "static scratch" in lib.dtd_last_error(eng.h).decode()
    # a batch that fits is accepted (here: an unknown sequence, reported as such)
    st = lib.dtd_decode_step_noalloc(eng.h, 1, arr, t.data_ptr(), t.data_ptr(), None)
    assert st == dtd.DTD_E_NOSEQ
    eng.close()
