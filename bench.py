"""Decode-step benchmark: tokens/s and achieved HBM bandwidth of the MI355X decode step.

Workload (default): the SmolLM3-3B-shaped decoder with random weights (dim 2048, 36 layers,
16 q / 4 kv heads, head_dim 128, ffn 11008, vocab 128256; int8 weight-only with per-row
fp32 scales, bf16 activations and KV cache), batch 1: prefill 512 random tokens, then
greedy decode toward context 2048.  One step = one pass of the whole decode step (embed,
36 x [RMSNorm, QKV+RoPE, KV append + GQA attention, O + residual, RMSNorm, gate/up +
SwiGLU, down + residual], final RMSNorm, LM head, argmax) for one token.

Prints one JSON line (rank 0).  Runs on one GPU only.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from decoder_only_transformer_decode_amd import dtd, synth  # noqa: E402

PEAK_HBM_GBS = 8000.0   # MI355X HBM3E, 8 TB/s


def weight_bytes(s: synth.ModelShape) -> dict:
    """Stored bytes of every matrix read by one decode step (the embedding row gather and
    the norm gains are left out), by projection."""
    def mat(r, c):
        if s.wfmt == synth.W_BF16:
            return r * c * 2
        if s.wfmt == synth.W_INT8_ROW:
            return r * c + r * 4
        if s.wfmt == synth.W_Q4_0:
            return r * c // 2 + r * (c // 32) * 2
        return r * c + r * (c // 32) * 2
    per_layer = {
        "qkv": mat(s.q_dim + 2 * s.kv_dim, s.dim),
        "o": mat(s.dim, s.q_dim),
        "gate_up": mat(2 * s.ffn_dim, s.dim),
        "down": mat(s.dim, s.ffn_dim),
    }
    out = {k: v * s.n_layers for k, v in per_layer.items()}
    out["lm_head"] = mat(s.vocab, s.dim)
    out["per_layer"] = per_layer
    return out


def kv_bytes_per_position(s: synth.ModelShape) -> int:
    """Stored K and V bytes of one position across all layers (+ fp16 scales for int8)."""
    el = {synth.KV_F32: 4, synth.KV_BF16: 2, synth.KV_I8: 1}[s.kvfmt]
    per = 2 * s.n_layers * s.n_kv_heads * s.head_dim * el
    if s.kvfmt == synth.KV_I8:
        per += 2 * s.n_layers * s.n_kv_heads * 2
    return per


KERNEL_SOURCES = ["decoder_only_transformer_decode_amd/csrc/dtd_persistent.hip",
                  "decoder_only_transformer_decode_amd/csrc/dtd_device.h",
                  "decoder_only_transformer_decode_amd/csrc/dtd_internal.h"]


def kernel_source_hash() -> str:
    """sha256 over the step kernel's sources (of the shared internal header, the part before
    its launcher declarations), to tell whether recorded counters still apply"""
    import hashlib
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for rel in KERNEL_SOURCES:
        with open(os.path.join(root, rel), "rb") as f:
            data = f.read()
        if rel.endswith("dtd_internal.h"):
            data = data.split(b"// ---- launchers")[0]
        h.update(data)
    return h.hexdigest()


def recorded_traffic(workload: str, attended: str, weights: str, kv_budget: int):
    """HBM bytes per step-kernel launch from the committed FETCH_SIZE / WRITE_SIZE readings of
    this workload (same weight format and KV budget) over the same attended contexts (each
    counter scaled by what it reads for a plain copy of known size), or None when there are
    none, they cover other contexts or another variant of the workload, or the kernel's
    sources have changed since they were taken."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", f"k_step_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        doc = json.load(f)
    for r in doc.get("records", []):
        if (r.get("kernel_source_sha256") == kernel_source_hash() and r.get("attended") == attended
                and r.get("weights") == weights and r.get("kv_budget", 0) == kv_budget):
            return (r["fetch_kib_per_launch"] * r["fetch_scale"] + r["write_kib_per_launch"] * r["write_scale"]) * 1024.0
    return None


def sampler_timing(vocab: int, batch: int, step_ms: float) -> dict:
    """Average duration of one k_sample launch (dtd_sample) over `batch` rows of the
    workload's vocabulary, HIP events on the launch stream: temperature only, and every
    filter on.  The logits are Gaussian with spread 3 (synth.bench_logits)."""
    import torch
    st = torch.cuda.current_stream()
    logits = torch.from_numpy(synth.bench_logits(batch, vocab, seed=3)).cuda()
    out = torch.zeros(batch, dtype=torch.int32, device="cuda")
    res = {"kernel": "k_sample (one workgroup per row)", "vocab": vocab, "batch": batch}
    for name, kw in (("temperature_only", dict(temperature=0.8)),
                     ("all_filters", dict(temperature=0.8, top_k=40, top_p=0.95, min_p=0.05))):
        samp = [dtd.sampler(seed=b, **kw) for b in range(batch)]
        ctr = list(range(batch))
        for _ in range(3):
            dtd.dtd_sample(logits.data_ptr(), vocab, batch, vocab, samp, ctr, out.data_ptr(), st.cuda_stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 20
        a.record(st)
        for _ in range(n):
            dtd.dtd_sample(logits.data_ptr(), vocab, batch, vocab, samp, ctr, out.data_ptr(), st.cuda_stream)
        b.record(st)
        b.synchronize()
        us = a.elapsed_time(b) / n * 1e3
        res[f"{name}_us"] = round(us, 1)
        res[f"{name}_share_of_step"] = round(us / (step_ms * 1e3), 4)
    res["all_filters_settings"] = "temperature 0.8, top_k 40, top_p 0.95, min_p 0.05"
    return res


def cpu_baseline(w: synth.Workload, weights, n_steps: int) -> dict:
    """The oracle, as it stands, on this host: n_steps decode steps ending at the workload's
    context (synthetic stored KV before them), with every core OpenMP offers, then with one."""
    import oracle
    s = w.shape
    pos0 = w.context - n_steps
    out = {}
    for label, threads in (("all", oracle.num_threads()), ("one", 1)):
        oracle.set_num_threads(threads)
        m = oracle.Model(s, weights, max_ctx=w.context, max_seqs=1)
        for layer in range(s.n_layers):
            k, v, ks, vs = synth.synthetic_kv(s, pos0, seed=5, layer=layer)
            m.kv_write(0, layer, 0, k, v, ks, vs)
        tok = 17
        t0 = time.perf_counter()
        for i in range(n_steps):
            tok, _, _ = m.step(0, tok, pos0 + i)
        out[label] = (n_steps / (time.perf_counter() - t0), threads)
        del m
    oracle.set_num_threads(out["all"][1])
    return {"value": round(out["all"][0], 4), "unit": "tokens/s", "cores": out["all"][1], "kind": "oracle",
            "value_1_thread": round(out["one"][0], 4),
            "sample": f"{n_steps} batch-1 decode steps at attended context {pos0 + 1}..{w.context} "
                      f"(synthetic stored KV before them), fp64 oracle, with {out['all'][1]} OpenMP threads "
                      f"and again with 1"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1536)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default=synth.SMOLLM3_3B.shape.name, choices=sorted(synth.BY_NAME))
    ap.add_argument("--cpu-steps", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--no-read-ceiling", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device to device 3 times and exit: the plain copy whose "
                         "FETCH_SIZE / WRITE_SIZE counter readings scale the step kernel's")
    ap.add_argument("--weights", choices=sorted(synth.WFMT_NAMES.values()), default=None,
                    help="store the workload's matrices in this format instead of its own")
    ap.add_argument("--path", choices=["auto", "per-kernel", "persistent"], default="auto",
                    help="schedule: auto (persistent step kernel at batch 1), or force one")
    ap.add_argument("--kv-budget", type=int, default=0, metavar="B",
                    help="batch-1 workloads: decode under an Initial-Key KV budget of B entries "
                         "(4 initial, 64 recent, the last 2 layers scored)")
    ap.add_argument("--serve", type=int, default=0, metavar="N",
                    help="instead of the decode step: N requests through the continuous-batching "
                         "scheduler (qwen3-8b-shaped unless --workload names another batched shape), "
                         "with the prefix cache off and then on; prints one JSON line")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this decode step runs on a single MI355X and has no "
              "multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 3}), flush=True)
        return
    w = synth.BY_NAME[args.workload]
    if args.weights:
        fmt = {v: k for k, v in synth.WFMT_NAMES.items()}[args.weights]
        w = dataclasses.replace(w, shape=w.shape.replace(wfmt=fmt))
    s = w.shape
    if args.serve:
        bench_serve(args, w if w.batch != 1 else synth.QWEN3_8B)
        return
    if w.batch != 1:
        bench_batched(args, w)
        return
    K, W = args.steps, args.warmup
    # The K timed steps end at the workload's context: the first takes position start.
    start = w.context - K
    if K < 1 or start < 1:
        print(f"--steps {K} does not fit below context {w.context}", file=sys.stderr)
        sys.exit(2)
    # prefill the workload's prompt and decode up to start, or synthetic KV up to start
    real_prompt = not w.synthetic_prefix and w.prompt_len <= start
    attended = f"{start + 1}..{w.context}"

    t0 = time.perf_counter()
    weights = synth.gen_weights(s, synth.weights_seed(w))
    t_gen = time.perf_counter() - t0
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    eng = dtd.Engine(s, max_ctx=w.context, max_seqs=2, max_batch=1)
    eng.load_weights(synth.flat_tensors(weights))
    dtd.dtd_debug_set_path(eng.h, {"auto": dtd.PATH_AUTO, "per-kernel": dtd.PATH_PER_KERNEL,
                                   "persistent": dtd.PATH_PERSISTENT}[args.path])
    persistent = dtd.dtd_debug_uses_persistent(eng.h, 1)
    print(f"[bench] weights generated in {t_gen:.1f} s and loaded; "
          f"{'persistent step kernel' if persistent else 'one kernel per sub-step'}", file=sys.stderr, flush=True)

    prompt = torch.as_tensor(synth.prompt_tokens(s.vocab, w.prompt_len)).to(dev)
    hist = torch.zeros(K + 1, dtype=torch.int32, device=dev)     # tokens of the timed steps

    def decode_on(seq, buf, n):
        """n greedy steps of seq: step i reads buf[i] and writes its next token to buf[i + 1]."""
        base = buf.data_ptr()
        for i in range(n):
            dtd.dtd_decode_step(eng.h, [seq], base + 4 * i, base + 4 * (i + 1))

    def build_sequence(seq, length):
        """seq at `length` positions, its next token in hist[0]: the workload's prompt then
        greedy decode steps, or synthetic KV (workloads that decode at a fixed context)."""
        if eng.seq_len(seq) >= 0:
            eng.reset_seq(seq)
        if args.kv_budget:
            eng.set_kv_budget(seq, args.kv_budget, n_initial=4, n_recent=64, score_layers=2)
        if real_prompt:
            nxt, _ = eng.prefill(seq, prompt)
            fill = torch.zeros(length - w.prompt_len + 1, dtype=torch.int32, device=dev)
            fill[0] = nxt[0]
            decode_on(seq, fill, length - w.prompt_len)
            hist[0] = fill[-1]
        else:
            dtd.dtd_debug_kv_fill(eng.h, seq, length, 5)
            hist[0] = 17
        torch.cuda.synchronize()

    # warmup: W steps on another sequence at the same contexts
    build_sequence(1, start)
    warm = torch.zeros(W + 1, dtype=torch.int32, device=dev)
    warm[0] = hist[0]
    decode_on(1, warm, W)
    torch.cuda.synchronize()
    dtd.dtd_check_device_errors(eng.h)
    eng.reset_seq(1)

    # timed region: K greedy steps, the token fed back on the device
    build_sequence(0, start)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    decode_on(0, hist, K)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    dtd.dtd_check_device_errors(eng.h)     # a device-side wait that gave up, or a bad token id
    assert eng.seq_len(0) == (min(w.context, args.kv_budget) if args.kv_budget else w.context)
    tokens = hist.cpu().numpy().copy()

    wb = weight_bytes(s)
    wtot = sum(v for k, v in wb.items() if k != "per_layer")
    kvpp = kv_bytes_per_position(s)
    attended_t = np.arange(start + 1, w.context + 1, dtype=np.float64)
    if args.kv_budget:      # the kept entries and the new one
        attended_t = np.minimum(attended_t, args.kv_budget + 1)
    kv_total = float(kvpp * attended_t.sum())
    bytes_total = wtot * K + kv_total
    gbs = bytes_total / dt / 1e9

    roofline = None
    if not args.no_kernel_timing:
        # the same workload again with HIP events around every launch of the kernel that
        # moves the most bytes, on the engine's stream: the persistent step kernel (weights
        # + KV of one step per launch) or, per sub-step, the gate/up projection; the greedy
        # tokens must repeat those of the timed run
        build_sequence(0, start)
        kind = dtd.KERNEL_STEP if persistent else dtd.KERNEL_GATE_UP
        dtd.dtd_debug_kernel_timing(eng.h, kind, True)
        decode_on(0, hist, K)
        ms, cnt = dtd.dtd_debug_kernel_timing(eng.h, kind, False)
        dtd.dtd_check_device_errors(eng.h)
        again = hist.cpu().numpy()
        if not np.array_equal(again, tokens):
            print(f"[bench] the rerun's greedy tokens differ from the timed run's "
                  f"(first at step {int(np.flatnonzero(again != tokens)[0])})", file=sys.stderr)
            sys.exit(1)
        if persistent:
            per_launch = wtot + kv_total / K
            name = (f"k_step (persistent batch-1 decode step, {synth.WFMT_NAMES[s.wfmt]} weights, "
                    f"{synth.KV_NAMES[s.kvfmt]} KV)")
        else:
            per_launch = wb["per_layer"]["gate_up"]
            name = "k_gemv (gate/up projection, SwiGLU epilogue)"
        avg_s = ms / 1e3 / max(cnt, 1)
        ach = per_launch / avg_s / 1e9 if cnt else 0.0
        traffic = (recorded_traffic(s.name, attended, synth.WFMT_NAMES[s.wfmt], args.kv_budget)
                   if persistent else None)
        roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(ach / PEAK_HBM_GBS, 4),
                    "traffic": None if traffic is None else round(traffic), "kernel": name,
                    "bytes_per_launch": round(per_launch), "avg_launch_us": round(avg_s * 1e6, 2),
                    "launches": cnt}

    ceiling = None
    if not args.no_read_ceiling:
        buf = torch.empty(8 << 30, dtype=torch.uint8, device=dev)
        ceiling = dtd.dtd_debug_stream_read(buf.data_ptr(), buf.numel(), 10, torch.cuda.current_stream().cuda_stream)
        del buf
        torch.cuda.empty_cache()
        if roofline is not None:
            roofline["measured_read_ceiling_gbs"] = round(ceiling, 1)
            roofline["frac_of_measured_ceiling"] = round(roofline["achieved"] / ceiling, 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, weights, args.cpu_steps)
    sampling = sampler_timing(s.vocab, 1, dt / K * 1e3)

    if real_prompt:
        how = f"prefill {w.prompt_len} random tokens, greedy decode to position {start}, then {K} timed steps"
    else:
        how = f"synthetic KV for {start} positions, then {K} timed greedy steps"
    rec = {
        "metric": "decode tokens/s and achieved HBM GB/s (% of peak) per decode step, 1 GPU",
        "value": round(K / dt, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(dt / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{synth.WFMT_NAMES[s.wfmt]} weights x {synth.ACT_NAMES[s.act]} activations, "
                 f"{synth.KV_NAMES[s.kvfmt]} KV, fp32 accumulation",
        "data": "synthetic",
        "config": {"workload": f"{s.name} batch-1 greedy decode to context {w.context}: {how} "
                               f"(attended context {attended})",
                   "dim": s.dim, "layers": s.n_layers, "q_heads": s.n_q_heads, "kv_heads": s.n_kv_heads,
                   "head_dim": s.head_dim, "ffn": s.ffn_dim, "vocab": s.vocab,
                   "weights": synth.WFMT_NAMES[s.wfmt], "activations": synth.ACT_NAMES[s.act],
                   "kv_cache": synth.KV_NAMES[s.kvfmt], "tied": bool(s.tied), "batch": 1,
                   **({"kv_budget": {"entries": args.kv_budget, "initial": 4, "recent": 64, "scored_layers": 2}}
                      if args.kv_budget else {})},
        "hbm_gbs": round(gbs, 1),
        "hbm_frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
        "bytes_per_step": round(bytes_total / K),
        "greedy_tokens_checked": "timed run == kernel-timing rerun; device error word clear",
        "roofline": roofline,
        "cpu_baseline": cpu,
        "sampling": sampling,
    }
    eng.close()
    print(json.dumps(rec), flush=True)


def bench_serve(args, w: synth.Workload):
    """Continuous batching: N requests, all sharing a 256-token system prefix, each with its
    own user part (32..480 tokens) and answer budget (32..256 tokens), submitted at once to
    the scheduler (batches of up to 64); greedy decoding.  Runs twice, prefix cache off and
    on; value = generated tokens/s with the cache on.  Both runs must produce the same tokens
    wherever no near tie parts them (counted, reported)."""
    import torch
    s = w.shape
    N, B, ctx = args.serve, 64, 2048
    rng = np.random.default_rng(11)
    system = synth.prompt_tokens(s.vocab, 256, seed=500)
    reqs = []
    for i in range(N):
        user = synth.prompt_tokens(s.vocab, int(rng.integers(32, 481)), seed=1000 + i)
        reqs.append((np.concatenate([system, user]).astype(np.int32), int(rng.integers(32, 257))))
    t0 = time.perf_counter()
    weights = synth.gen_weights(s, synth.weights_seed(w))
    print(f"[bench] weights generated in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    torch.cuda.set_device(0)
    eng = dtd.Engine(s, max_ctx=ctx, max_seqs=B, max_batch=B, kv_block_size=16,
                     kv_num_blocks=B * (ctx // 16))
    eng.load_weights(synth.flat_tensors(weights))
    runs = {}
    outs = {}
    for cache in (0, B):
        eng.set_prefix_cache(cache)
        sch = dtd.Scheduler(eng)
        # warmup: a few requests through the same paths, then a clean cache
        for p, m in reqs[:4]:
            sch.submit(p[:300], 8)
        sch.run()
        eng.set_prefix_cache(0)
        eng.set_prefix_cache(cache)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ids = [sch.submit(p, m) for p, m in reqs]
        steps = sch.run()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        toks = [sch.result(r)[0] for r in ids]
        gen = sum(len(t) for t in toks)
        runs[cache] = {"seconds": round(dt, 3), "generated_tokens": gen,
                       "generated_tokens_per_s": round(gen / dt, 1),
                       "prompt_tokens": int(sum(len(p) for p, _ in reqs)), "scheduling_steps": steps,
                       "mean_decode_batch": round((gen - N) / max(steps, 1), 2)}
        outs[cache] = toks
        sch.close()
        print(f"[bench] prefix cache {'on' if cache else 'off'}: {runs[cache]}", file=sys.stderr, flush=True)
    same = sum(int(a == b) for a, b in zip(outs[0], outs[B]))
    on, off = runs[B], runs[0]
    rec = {
        "metric": "continuous-batching serving throughput (generated tokens/s), 1 GPU",
        "value": on["generated_tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "higher_is_better": True,
        "vs_baseline": None,
        "dtype": f"{synth.WFMT_NAMES[s.wfmt]} weights x {synth.ACT_NAMES[s.act]} activations, "
                 f"{synth.KV_NAMES[s.kvfmt]} KV, fp32 accumulation",
        "data": "synthetic",
        "config": {"workload": f"{s.name} serving: {N} requests submitted at once, a shared 256-token system "
                               f"prefix + a 32..480-token user part each, 32..256 greedy tokens each, "
                               f"batches of up to {B}, max context {ctx}",
                   "requests": N, "max_batch": B},
        "prefix_cache_on": on,
        "prefix_cache_off": off,
        "requests_with_identical_tokens_both_runs": same,
    }
    eng.close()
    print(json.dumps(rec), flush=True)


def cpu_baseline_batched(w: synth.Workload, weights, ctxs, n_seqs: int) -> dict:
    """The oracle on this host: one decode step for each of the first n_seqs sequences of the
    batch at its context (synthetic stored KV before it), every OpenMP thread.  The oracle
    steps sequences one at a time, so its tokens/s over the sample is its batch rate."""
    import oracle
    s = w.shape
    m = oracle.Model(s, weights, max_ctx=w.context, max_seqs=n_seqs)
    for b in range(n_seqs):
        for layer in range(s.n_layers):
            k, v, ks, vs = synth.synthetic_kv(s, int(ctxs[b]) - 1, seed=5 + b, layer=layer)
            m.kv_write(b, layer, 0, k, v, ks, vs)
    t0 = time.perf_counter()
    for b in range(n_seqs):
        m.step(b, 17 + b, int(ctxs[b]) - 1)
    dt = time.perf_counter() - t0
    return {"value": round(n_seqs / dt, 4), "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"one decode step of {n_seqs} of the batch's sequences (attended contexts "
                      f"{', '.join(str(int(c)) for c in ctxs[:n_seqs])}), synthetic stored KV, fp64 oracle, "
                      f"{dt:.1f} s"}


def bench_batched(args, w: synth.Workload):
    """Batched decode: every step advances all B sequences by one token (continuous-batch
    decode at the workload's contexts); the K timed steps end at each sequence's context."""
    import torch
    s = w.shape
    B, K, W = w.batch, args.steps, args.warmup
    ctxs = synth.context_lengths(B) if w.mixed_contexts else np.full(B, w.context, dtype=np.int32)
    if int(ctxs.min()) - K - W < 1:
        print(f"--steps {K} + --warmup {W} do not fit below the shortest context {int(ctxs.min())}", file=sys.stderr)
        sys.exit(2)
    t0 = time.perf_counter()
    print(f"[bench] generating {s.name} weights", file=sys.stderr, flush=True)
    weights = synth.gen_weights(s, synth.weights_seed(w))
    t_gen = time.perf_counter() - t0
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    eng = dtd.Engine(s, max_ctx=w.context, max_seqs=B, max_batch=B, kv_block_size=w.block_size)
    eng.load_weights(synth.flat_tensors(weights))
    print(f"[bench] weights generated in {t_gen:.1f} s and loaded; batch {B}", file=sys.stderr, flush=True)
    ids = list(range(B))
    hist = torch.zeros((K + 1, B), dtype=torch.int32, device=dev)
    row = B * 4

    def prepare():
        """every sequence at context - K - W positions of synthetic KV, then W warmup steps"""
        for b in ids:
            if eng.seq_len(b) >= 0:
                eng.reset_seq(b)
            dtd.dtd_debug_kv_fill(eng.h, b, int(ctxs[b]) - K - W, 7 + b)
        warm = torch.zeros((W + 1, B), dtype=torch.int32, device=dev)
        warm[0] = torch.as_tensor(synth.prompt_tokens(s.vocab, B, seed=3)).to(dev)
        for i in range(W):
            dtd.dtd_decode_step(eng.h, ids, warm.data_ptr() + i * row, warm.data_ptr() + (i + 1) * row)
        hist[0] = warm[W]
        torch.cuda.synchronize()
        dtd.dtd_check_device_errors(eng.h)

    def run():
        for i in range(K):
            dtd.dtd_decode_step(eng.h, ids, hist.data_ptr() + i * row, hist.data_ptr() + (i + 1) * row)

    prepare()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    dtd.dtd_check_device_errors(eng.h)
    tokens = hist.cpu().numpy().copy()

    wb = weight_bytes(s)
    wtot = sum(v for k, v in wb.items() if k != "per_layer")
    kvpp = kv_bytes_per_position(s)
    # attended contexts of the timed steps: step i attends ctx_b - K + 1 + i positions
    att = sum(float(c - K + 1 + i) for c in ctxs for i in range(K))
    kv_total = kvpp * att
    bytes_total = wtot * K + kv_total
    gbs = bytes_total / dt / 1e9

    def timed(kind):
        prepare()
        dtd.dtd_debug_kernel_timing(eng.h, kind, True)
        run()
        ms, cnt = dtd.dtd_debug_kernel_timing(eng.h, kind, False)
        dtd.dtd_check_device_errors(eng.h)
        again = hist.cpu().numpy()
        if not np.array_equal(again, tokens):
            print("[bench] a rerun's greedy tokens differ from the timed run's", file=sys.stderr)
            sys.exit(1)
        return ms / 1e3 / max(cnt, 1), cnt

    roofline = None
    if not args.no_kernel_timing:
        a_s, a_n = timed(dtd.KERNEL_ATTN)
        per_attn = kv_total / K / s.n_layers            # one layer's KV read, all sequences
        g_s, g_n = timed(dtd.KERNEL_GATE_UP)
        per_gu = wb["per_layer"]["gate_up"]
        roofline = {"bound": "hbm", "achieved": round(per_attn / a_s / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(per_attn / a_s / 1e9 / PEAK_HBM_GBS, 4), "traffic": None,
                    "kernel": f"k_attn (split-K GQA decode attention over paged {synth.KV_NAMES[s.kvfmt]} KV, "
                              f"{B} sequences, one layer)",
                    "bytes_per_launch": round(per_attn), "avg_launch_us": round(a_s * 1e6, 2), "launches": a_n,
                    "gemm_gate_up": {"kernel": f"k_gemm (gate/up projection on the matrix cores, "
                                               f"{synth.WFMT_NAMES[s.wfmt]} weights, batch {B})",
                                     "achieved": round(per_gu / g_s / 1e9, 1),
                                     "frac": round(per_gu / g_s / 1e9 / PEAK_HBM_GBS, 4),
                                     "bytes_per_launch": per_gu, "avg_launch_us": round(g_s * 1e6, 2),
                                     "launches": g_n,
                                     "mfma_tflops": round(2.0 * s.dim * 2 * s.ffn_dim * B / g_s / 1e12, 2)}}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_batched(w, weights, ctxs, 2)
    sampling = sampler_timing(s.vocab, B, dt / K * 1e3)
    ctx_desc = (f"per-sequence contexts uniform in [512, 4096] (seed 7; mean {float(ctxs.mean()):.0f})"
                if w.mixed_contexts else f"every sequence at context {w.context}")
    rec = {
        "metric": "decode tokens/s and achieved HBM GB/s (% of peak) per decode step, 1 GPU",
        "value": round(B * K / dt, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(dt / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{synth.WFMT_NAMES[s.wfmt]} weights x {synth.ACT_NAMES[s.act]} activations, "
                 f"{synth.KV_NAMES[s.kvfmt]} KV, fp32 accumulation",
        "data": "synthetic",
        "config": {"workload": f"{s.name} batched greedy decode, batch {B}, paged KV blocks of {w.block_size}, "
                               f"{ctx_desc}; synthetic KV, then {W} warmup and {K} timed steps ending at each "
                               f"sequence's context",
                   "dim": s.dim, "layers": s.n_layers, "q_heads": s.n_q_heads, "kv_heads": s.n_kv_heads,
                   "head_dim": s.head_dim, "ffn": s.ffn_dim, "vocab": s.vocab,
                   "weights": synth.WFMT_NAMES[s.wfmt], "activations": synth.ACT_NAMES[s.act],
                   "kv_cache": synth.KV_NAMES[s.kvfmt], "batch": B},
        "hbm_gbs": round(gbs, 1),
        "hbm_frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
        "bytes_per_step": round(bytes_total / K),
        "greedy_tokens_checked": "timed run == kernel-timing reruns; device error word clear",
        "roofline": roofline,
        "cpu_baseline": cpu,
        "sampling": sampling,
        "sampling": sampling,
    }
    eng.close()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
