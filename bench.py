"""Benchmark of one MTP speculative-decoding step on one MI355X.

A step is one round of the whole path on synthetic inputs resident in HBM:
  mtp_draft_loop (catch-up rows + D-1 serial draft steps: dual RMSNorm + eh_proj, decoder
  block with RoPE over the head's KV cache, final norm, lm_head + argmax)
  -> synthetic target logits (draft logits + seeded noise, standing in for the main model)
  -> [mtp_state_snapshot of a recurrent state, for workloads that carry one]
  -> spec_verify -> [mtp_state_restore where a draft was rejected] -> kv_crop.
The default workload is the largest single-GPU one: the DeepSeek-V3-scale single-module head
(H 7168, eh_proj 14336 -> 7168, 56/8 heads of 128, FFN 18432, vocab 129280, bf16), the same
layer reused for D = 3 serial drafts, B = 32 sequences at an 8192-position KV context, greedy
verification over 4 positions with target logits = draft logits + N(0, 0.7).

Prints one JSON line: accepted tokens/s (sum over rounds and sequences of accepted drafts + 1,
divided by the timed wall time), the lm_head kernel's HBM roofline and the CPU oracle timed on
a bounded sample of the same workload.  --config names another head workload (qwen: the
single-layer 2048-hidden head at B 1, D 1; drafter4: the 4-layer 1024-hidden drafter with
sampling verification) or, with --config stress, the verifier alone (B=256, D=4, vocab 151936,
sampling).
--target-layers L times the target's verify pass instead: a dense stand-in with the head's
dimensions and L blocks, scoring 1, 2 or 7 positions per call.  --prefill-rows N times one MTP
prefill call over N prompt rows.  --shared-kv T runs the same rounds with a head that keeps no
cache of its own and reads a T-layer main-model cache (head layer l reads layer l mod T) through
mtp_draft_loop_shared_kv; the main model's cache length then follows the verifier's crop length.
--modules M drafts with M MTP modules (step k by module (k-1) mod M, each with its own cache,
re-prefilled by every catch-up) through mtp_draft_loop_multi.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

METRIC = "accepted tokens/s per MTP draft+verify step; kernel HBM GB/s vs MI355X peak"
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="dsv3")
    ap.add_argument("--state-bytes", type=int, default=None, help="recurrent state bytes per sequence")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle baseline sample budget (0: skip)")
    ap.add_argument("--traffic", default=os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                                                      "lm_head_counters.json"),
                    help="counter-measured lm_head bytes per launch (ignored when the kernel sources changed)")
    ap.add_argument("--graph", type=int, default=0, help="capture this many rounds per HIP graph (0: eager)")
    ap.add_argument("--prefill-rows", type=int, default=0,
                    help="time one MTP prefill of this many rows per sequence instead (from an empty cache)")
    ap.add_argument("--target-layers", type=int, default=0,
                    help="time the target's verify pass instead (a dense stand-in with this many layers)")
    ap.add_argument("--modules", type=int, default=1,
                    help="draft with this many MTP modules, step k by module (k-1) mod M (mtp_draft_loop_multi)")
    ap.add_argument("--shared-kv", type=int, default=0,
                    help="the head keeps no cache and reads a main-model cache of this many layers instead")
    ap.add_argument("--sigma", type=float, default=1.0,
                    help="verifier-only workloads: std of the target-logit noise around the draft logits")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="run one plain device copy of this many MiB first (counter calibration)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    import torch
    import speculative_decoding_mtp_amd as M
    from synth import CONFIGS, make_first_round, make_kv_prefix, make_round_hiddens, make_round_noise, \
        make_round_uniforms, make_state, make_weights
    from tests.gpu_util import config, f32, i32, kv_from_numpy, upload_weights

    from synth import VERIFY_CONFIGS
    if args.config in VERIFY_CONFIGS:
        return bench_verify(args, VERIFY_CONFIGS[args.config], args.sigma)
    cfg = CONFIGS[args.config]
    if args.target_layers > 0:
        return bench_target(args, cfg, args.target_layers)
    if args.prefill_rows > 0:
        return bench_prefill(args, cfg, args.prefill_rows)
    B, D, H, V = cfg.batch, cfg.D, cfg.hidden, cfg.vocab
    state_bytes = cfg.state_bytes_per_seq if args.state_bytes is None else args.state_bytes
    rounds_total = args.warmup + args.steps
    max_len = M.round_max_len(cfg.ctx + 1 + (rounds_total + args.graph) * (D + 1) + 64)
    t0 = time.time()
    w = make_weights(cfg)
    c = config(cfg)
    gw = upload_weights(cfg, w)
    T = args.shared_kv
    if T:
        # the main model's cache: seeded N(0,1) keys and values in every slot, ctx + 1 positions
        # cached at the start (the settled token's predecessor included)
        kv = M.KVCache(c, B, max_len, n_layers=T)
        gen = torch.Generator(device="cuda")
        gen.manual_seed(1000 * cfg.index + 3)
        kv.k.copy_(torch.randn(kv.k.shape, generator=gen, device="cuda"))
        kv.v.copy_(torch.randn(kv.v.shape, generator=gen, device="cuda"))
        kv.len.fill_(cfg.ctx + 1)
        kv_layer = [l % T for l in range(cfg.n_layers)]
        K = Vv = None
    else:
        K, Vv = make_kv_prefix(cfg)
        kv = kv_from_numpy(cfg, K, Vv, cfg.ctx, max_len)
    MODS = max(1, args.modules)
    gws, kvs = [gw], [kv]
    if MODS > 1:
        # modules 1.. : seeded on the device (same init as make_weights: N(0, 0.02) matrices, unit
        # gains), sharing module 0's embedding and lm_head; their caches hold seeded N(0,1) K/V
        gen = torch.Generator(device="cuda")
        dt = c.torch_dtype
        for m in range(1, MODS):
            gen.manual_seed(1000 * cfg.index + 7 + m)
            rnd = lambda *shape: (torch.randn(shape, generator=gen, device="cuda") * 0.02).to(dt)
            ones = lambda n: torch.ones(n, device="cuda", dtype=dt)
            t = dict(embed=gw.t["embed"], lm_head=gw.t["lm_head"], enorm=ones(H), hnorm=ones(H),
                     final_norm=ones(H), eh_proj=rnd(H, 2 * H), layers=[])
            for _ in range(cfg.n_layers):
                t["layers"].append(dict(in_norm=ones(H), wq=rnd(cfg.q_dim, H), wk=rnd(cfg.kv_dim, H),
                                        wv=rnd(cfg.kv_dim, H), wo=rnd(H, cfg.q_dim), post_norm=ones(H),
                                        wgate=rnd(cfg.ffn, H), wup=rnd(cfg.ffn, H), wdown=rnd(H, cfg.ffn)))
            gws.append(M.Weights(c, t))
            km = M.KVCache(c, B, max_len)
            km.k.copy_(torch.randn(km.k.shape, generator=gen, device="cuda"))
            km.v.copy_(torch.randn(km.v.shape, generator=gen, device="cuda"))
            km.len.fill_(cfg.ctx)
            kvs.append(km)
    print(f"[bench] inputs ready in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    if args.calib_copy_mb:
        src = torch.ones(args.calib_copy_mb * 1024 * 1024 // 4, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    rps = D + 1
    toks0, hid0 = make_first_round(cfg)
    tok_pad = np.full((B, rps), -1, np.int32)
    tok_pad[:, :1] = toks0
    hid_pad = np.zeros((B, rps, H), np.float32)
    hid_pad[:, :1] = hid0
    NBUF = 16
    hid_bufs = [f32(make_round_hiddens(cfg, r)) for r in range(NBUF)]
    noise_bufs = [f32(make_round_noise(cfg, r)) for r in range(NBUF)]
    tokens = i32(tok_pad)
    hidden0 = f32(hid_pad)
    ws = M.new_workspace(M.mtp_draft_workspace_size(c, B, 1 if T else max(rps, D - 1), D, max_len))
    if T:  # one settled token and one main-model hidden per sequence and round
        tok_shared = i32(toks0[:, 0])
        hid_shared = [f32(np.ascontiguousarray(make_round_hiddens(cfg, r)[:, 0])) for r in range(NBUF)]
        hid_shared0 = f32(np.ascontiguousarray(hid0[:, 0]))
    sp = cfg.sampling
    csp = None if sp is None else M.sampling(sp.temperature, sp.top_k, sp.top_p, sp.q_mode)
    vws = M.new_workspace(M.spec_verify_workspace_size(B, D, V, csp))
    unif = [tuple(f32(u) for u in make_round_uniforms(cfg.index, B, D, r)) for r in range(NBUF)] if sp else None
    drafts = torch.zeros(B, D, dtype=torch.int32, device="cuda")
    hiddens = torch.zeros(B, D, H, device="cuda")
    dlog = torch.zeros(B, D, V, device="cuda")
    tl = torch.zeros(B, D + 1, V, device="cuda")
    out_tok = [torch.zeros(B, D + 1, dtype=torch.int32, device="cuda") for _ in range(2)]
    ctx = [torch.full((B,), cfg.ctx + 1, dtype=torch.int32, device="cuda"),
           torch.zeros(B, dtype=torch.int32, device="cuda")]
    hist = torch.zeros(rounds_total + max(args.graph, 0), B, dtype=torch.int32, device="cuda")
    state = snap = None
    if state_bytes:
        state = torch.from_numpy(make_state(B, state_bytes)).cuda()
        snap = torch.empty_like(state)

    def step(r):
        cur, nxt = r % 2, (r + 1) % 2
        if T:
            if r > 0:  # the last emitted token of the previous round is the settled one
                torch.gather(out_tok[cur], 1, hist[r - 1].long().unsqueeze(1), out=tok_shared.view(B, 1))
            hin = hid_shared0 if r == 0 else hid_shared[r % NBUF]
            M.mtp_draft_loop_shared_kv(c, gw, kv, kv_layer, D, tok_shared, hin, drafts, hiddens, dlog, ws)
        else:
            tk = tokens if r == 0 else out_tok[cur]
            hin = hidden0 if r == 0 else hid_bufs[r % NBUF]
            if MODS > 1:
                M.mtp_draft_loop_multi(c, gws, kvs, D, rps, tk, hin, drafts, hiddens, dlog, ws)
            else:
                M.mtp_draft_loop(c, gw, kv, D, rps, tk, hin, drafts, hiddens, dlog, ws)
        # stand-in target forward: target row j = draft logits of step j+1 + noise (row D
        # reuses step D's logits), one elementwise kernel for D = 1
        noise = noise_bufs[r % NBUF]
        if D == 1:
            torch.add(noise, dlog.expand(B, 2, V), out=tl)
        else:
            torch.add(noise[:, :D], dlog, out=tl[:, :D])
            torch.add(noise[:, D], dlog[:, D - 1], out=tl[:, D])
        if state is not None:
            M.mtp_state_snapshot(state, snap, state_bytes, B)
        n_acc = hist[r]
        ua, us = unif[r % NBUF] if unif else (None, None)
        M.spec_verify(B, D, V, tl, drafts, None, csp, ua, us, ctx[cur], n_acc, out_tok[nxt], ctx[nxt], vws)
        if state is not None:
            M.mtp_state_restore(state, snap, state_bytes, B, n_acc, D)
        if T:  # stand-in for the main model's verify pass + crop: its cache now ends at crop_len
            kv.len.copy_(ctx[nxt])
        else:
            for km in kvs:
                M.kv_crop(km, ctx[cur])

    for r in range(args.warmup):
        step(r)
    torch.cuda.synchronize()
    M.mtp_check(ws)
    graph = None
    G = args.graph
    if G:
        # rounds warmup .. warmup+G-1 captured once (their buffers cycle with r), replayed
        assert G % 2 == 0 and args.steps % G == 0 and args.warmup % 2 == 0
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for r in range(args.warmup, args.warmup + G):
                step(r)
        torch.cuda.synchronize()   # capture ran nothing: the state after warmup is still current
    else:
        M.mtp_timer_start(M.MTP_KERNEL_LM_HEAD, args.steps * D)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ctx0 = int(ctx[args.warmup % 2].sum())
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0.record()
    if graph is not None:
        for _ in range(args.steps // G):
            graph.replay()
    else:
        for r in range(args.warmup, rounds_total):
            step(r)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    gpu_ms = ev0.elapsed_time(ev1)
    if graph is not None:
        # kernel events cannot be timed inside a graph: time the same rounds eagerly right after
        M.mtp_timer_start(M.MTP_KERNEL_LM_HEAD, G * D)
        for r in range(rounds_total, rounds_total + G):
            step(r)
        torch.cuda.synchronize()
    lm_ms, lm_n = M.mtp_timer_read(M.MTP_KERNEL_LM_HEAD)
    M.mtp_check(ws)
    # every round grows the target length by the accepted drafts + 1
    tokens_out = int(ctx[rounds_total % 2].sum()) - ctx0
    acc = hist[args.warmup:].cpu().numpy() if graph is None else hist[args.warmup:args.warmup + G].cpu().numpy()
    value = tokens_out / wall
    ms_per_step = wall * 1e3 / args.steps

    # the lm_head kernel's algorithmic bytes per launch: the weights once, each sequence's
    # (normalised, fp32-equivalent) activation row in, its logits row out
    lm_bytes = V * H * cfg.wbytes + B * H * 4 + B * V * 4
    lm_avg_s = lm_ms / 1e3 / max(lm_n, 1)
    achieved = lm_bytes / lm_avg_s / 1e9
    traffic = None
    workload = cfg.name + (f"-sharedkv{T}" if T else "") + (f"-modules{MODS}" if MODS > 1 else "")
    if args.traffic and os.path.exists(args.traffic):
        rec = json.load(open(args.traffic))
    else:
        rec = {}
    # the counters were taken on one workload's lm_head, with the kernel sources of that time
    if rec.get("workload") == workload:
        root = os.path.dirname(os.path.abspath(__file__))
        h = hashlib.sha256()
        for p in rec.get("source_files", []):
            h.update(open(os.path.join(root, p), "rb").read())
        if h.hexdigest() == rec.get("source_sha256"):
            traffic = rec.get("bytes_per_launch")

    cpu = None
    if args.cpu_seconds > 0 and not T and MODS == 1:
        cpu = cpu_baseline(cfg, w, K, Vv, args.cpu_seconds)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "accepted tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded random-init weights, KV prefix, hiddens and target-logit noise)",
        "config": {"workload": workload,
                   "batch": B, "draft_tokens": D, "mtp_modules": MODS,
                   "kv_context": cfg.ctx,
                   "head_kv": f"reads a {T}-layer main-model cache (layer l mod {T})" if T else "own cache",
                   "target_noise_std": cfg.noise_std,
                   "verify": "greedy" if sp is None else
                   f"sampling T={sp.temperature} top_k={sp.top_k} top_p={sp.top_p} q_mode={sp.q_mode}",
                   "recurrent_state_bytes_per_seq": state_bytes},
        "steps_per_s": round(args.steps / wall, 2),
        "accepted_drafts_per_s": round(float(acc.sum()) * (args.steps / max(len(acc), 1)) / wall, 2),
        "acceptance": round(float(acc.mean()) / D, 4),
        "gpu_event_ms_per_step": round(gpu_ms / args.steps, 4),
        "roofline": {"bound": "hbm", "kernel": M.mtp_timer_kernel_name(M.MTP_KERNEL_LM_HEAD),
                     "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "bytes_per_launch": lm_bytes,
                     "avg_launch_us": round(lm_avg_s * 1e6, 2), "launches": lm_n},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_verify(args, vc, sigma=1.0):
    """The verifier on its own (--config stress): spec_verify over B sequences of D drafts with
    fp32 target logits resident in HBM, sampling with the workload's settings (q_mode 0, greedy
    drafts = argmax of the draft logits).  Reports verified sequences/s and the logits scan rate."""
    import torch
    import speculative_decoding_mtp_amd as M
    from synth import gen, make_verify_inputs
    from tests.gpu_util import f32, i32

    B, D, V, sp = vc.batch, vc.D, vc.vocab, vc.sampling
    dl, tl_np, ctx_np = make_verify_inputs(vc, sigma)
    drafts = i32(np.argmax(dl, axis=-1))
    del dl
    g = gen(vc.index, 6, int(sigma * 10))
    ua, us = f32(g.random((B, D), dtype=np.float32)), f32(g.random(B, dtype=np.float32))
    tl, ctx = f32(tl_np), i32(ctx_np)
    del tl_np
    csp = M.sampling(sp.temperature, sp.top_k, sp.top_p, sp.q_mode)
    vws = M.new_workspace(M.spec_verify_workspace_size(B, D, V, csp))
    n_acc = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = torch.zeros(B, D + 1, dtype=torch.int32, device="cuda")
    crop = torch.zeros(B, dtype=torch.int32, device="cuda")

    def step():
        M.spec_verify(B, D, V, tl, drafts, None, csp, ua, us, ctx, n_acc, out, crop, vws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    M.mtp_timer_start(M.MTP_KERNEL_VERIFY, args.steps)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    v_ms, v_n = M.mtp_timer_read(M.MTP_KERNEL_VERIFY)
    logits_bytes = B * (D + 1) * V * 4
    cpu = None
    if args.cpu_seconds > 0:
        tl_h, ctx_h, d_h = tl.cpu().numpy(), ctx.cpu().numpy(), drafts.cpu().numpy()
        ua_h, us_h = ua.cpu().numpy(), us.cpu().numpy()
        cpu = cpu_baseline_verify(tl_h, d_h, ctx_h, sp, ua_h, us_h, args.cpu_seconds)
    achieved = logits_bytes / (v_ms / v_n * 1e-3) / 1e9
    line = {
        "metric": "spec_verify sequences/s; target-logits scan HBM GB/s vs MI355X peak",
        "value": round(B * args.steps / wall, 1), "unit": "verified sequences/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded draft logits N(0,3), target = draft + N(0,1), uniforms)",
        "config": {"workload": vc.name, "batch": B, "draft_tokens": D, "vocab": V,
                   "verify": f"sampling T={sp.temperature} top_k={sp.top_k} top_p={sp.top_p} q_mode={sp.q_mode}",
                   "target_noise_std": sigma},
        "acceptance": round(float(n_acc.float().mean()) / D, 4),
        "roofline": {"bound": "hbm", "kernel": "spec_verify (top-k scan, merge, decide)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": logits_bytes, "avg_launch_us": round(v_ms / v_n * 1e3, 2),
                     "launches": v_n},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_prefill(args, cfg, rows):
    """One MTP prefill call (mtp_draft_step over ``rows`` rows per sequence, B = cfg.batch) from an
    empty head cache, timed with HIP events; the cache length is reset between calls."""
    import torch
    import speculative_decoding_mtp_amd as M
    from synth import make_prefill, make_weights
    from tests.gpu_util import config, f32, i32, upload_weights

    B, H, V = cfg.batch, cfg.hidden, cfg.vocab
    w = make_weights(cfg)
    c, gw = config(cfg), upload_weights(cfg, w)
    del w
    toks, hid = make_prefill(cfg, rows)
    max_len = M.round_max_len(rows + 8)
    kv = M.KVCache(c, B, max_len)
    ws = M.new_workspace(M.mtp_draft_workspace_size(c, B, rows, 1, max_len))
    t, h = i32(toks), f32(hid)
    hout = torch.zeros(B, rows, H, device="cuda")
    draft = torch.zeros(B, dtype=torch.int32, device="cuda")
    zero = torch.zeros(B, dtype=torch.int32, device="cuda")

    def call():
        M.mtp_draft_step(c, gw, kv, rows, t, h, hout, draft, None, ws)
        M.kv_crop(kv, zero)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    M.mtp_check(ws)
    ms = e0.elapsed_time(e1) / args.steps
    # algorithmic work: every row through eh_proj, the blocks and the final norm; causal
    # attention; lm_head for each sequence's last row
    per_row = 2 * H * H + cfg.n_layers * ((cfg.q_dim + 2 * cfg.kv_dim) * H + H * cfg.q_dim + 3 * cfg.ffn * H)
    flops = 2.0 * B * rows * per_row + 2.0 * B * V * H
    flops += cfg.n_layers * B * 4.0 * cfg.q_dim * rows * (rows + 1) / 2
    tflops = flops / (ms * 1e-3) / 1e12
    line = {
        "metric": "MTP prefill rows/s (one call over the prompt)", "value": round(B * rows / (ms * 1e-3), 1),
        "unit": "rows/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.wdtype,
        "data": "synthetic (seeded random-init head, uniform tokens, N(0,1) hiddens)",
        "config": {"workload": f"{cfg.name}-prefill{rows}", "batch": B, "rows": rows},
        "roofline": {"bound": "mfma", "kernel": "mtp_draft_step over the prompt (all kernels)",
                     "achieved": round(tflops, 2), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(tflops / 2500.0, 4), "traffic": None, "flops_per_launch": flops},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def bench_target(args, cfg, layers, row_counts=(1, 2, 7)):
    """The target's verify pass (mtp_target_forward) on a dense stand-in with the head's
    dimensions and ``layers`` blocks over a KV context of cfg.ctx positions (B = cfg.batch):
    time per call when it scores 1, 2 or 7 positions per sequence ([DLM "MTP speculative
    decoding"]: seven positions cost little more than one, because the pass is bound by reading
    the weights)."""
    import dataclasses
    import torch
    import speculative_decoding_mtp_amd as M
    from synth import gen, make_kv_prefix, make_target_weights, make_weights
    from tests.gpu_util import config, i32, kv_from_numpy, upload_target_weights

    B, H, V = cfg.batch, cfg.hidden, cfg.vocab
    tcfg = dataclasses.replace(cfg, n_layers=layers)
    w = make_weights(cfg)
    tw = make_target_weights(cfg, layers, w)
    c, gw = config(tcfg), upload_target_weights(tcfg, tw)
    del w, tw
    K, Vv = make_kv_prefix(tcfg)
    max_len = M.round_max_len(cfg.ctx + max(row_counts) + 8)
    kv = kv_from_numpy(tcfg, K, Vv, cfg.ctx, max_len)
    del K, Vv
    ctx = i32(np.full(B, cfg.ctx))
    R = max(row_counts)
    ws = M.new_workspace(M.mtp_target_workspace_size(c, B, R, max_len))
    hid = torch.zeros(B, R, H, device="cuda")
    lg = torch.zeros(B, R, V, device="cuda")
    toks = i32(gen(cfg.index, 4, 77).integers(0, V, size=(B, R)))
    ms = {}
    for rows in row_counts:
        t = toks[:, :rows].contiguous()
        for _ in range(args.warmup):
            M.mtp_target_forward(c, gw, kv, rows, t, hid, lg, ws)
            M.kv_crop(kv, ctx)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            M.mtp_target_forward(c, gw, kv, rows, t, hid, lg, ws)
            M.kv_crop(kv, ctx)
        e1.record()
        torch.cuda.synchronize()
        ms[rows] = e0.elapsed_time(e1) / args.steps
    M.mtp_check(ws)
    wb = 2 if cfg.wdtype == "bf16" else 4
    per_layer = ((cfg.q_dim + 2 * cfg.kv_dim) * H + H * cfg.q_dim + 3 * cfg.ffn * H) * wb
    weight_bytes = layers * per_layer + V * H * wb
    kv_bytes = layers * B * 2 * cfg.kv_dim * cfg.ctx * wb
    r7 = max(row_counts)
    achieved = (weight_bytes + kv_bytes) / (ms[r7] * 1e-3) / 1e9
    line = {
        "metric": "target verify pass: time for 7 scored positions relative to 1",
        "value": round(ms[r7] / ms[min(row_counts)], 4), "unit": "ratio", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms[r7], 4), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.wdtype,
        "data": "synthetic (seeded random-init dense target sharing the head's embedding and lm_head, random KV)",
        "config": {"workload": f"target-{layers}layer-h{H}-v{V}-{cfg.wdtype}-b{B}-ctx{cfg.ctx}", "batch": B,
                   "layers": layers, "kv_context": cfg.ctx},
        "ms_per_call": {str(k): round(v, 4) for k, v in ms.items()},
        "roofline": {"bound": "hbm", "kernel": f"mtp_target_forward at {r7} rows (all kernels)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": weight_bytes + kv_bytes},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def host_cores():
    """Host cores this process may run on, and the BLAS thread pool size NumPy uses."""
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = cores
    return cores, blas


def _timed_split(run, budget_s):
    """run(budget) -> (units, seconds, sample text); two thirds of the budget with NumPy's BLAS
    threads as configured, one third single-threaded (reported as single_thread_value)."""
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    cores, blas = host_cores()
    units, dt, what = run(budget_s * 2 / 3)
    line = {"value": round(units / dt, 4), "cores": cores, "blas_threads": blas, "kind": "oracle",
            "sample": f"{what}; {dt:.1f} s"}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            u1, dt1, what1 = run(budget_s / 3)
        line["single_thread_value"] = round(u1 / dt1, 4)
        line["single_thread_sample"] = f"{what1}; {dt1:.1f} s"
    return line


def cpu_baseline_verify(tl, drafts, ctx, sp, ua, us, budget_s):
    """The oracle's verification on the same resident inputs, one sequence at a time (sequences
    0, 1, 2, ... until the time budget is spent): verified sequences/s."""
    import oracle as O
    B = tl.shape[0]

    def run(budget):
        n, spent = 0, 0.0
        while n < 1 or spent < budget:
            b = n % B
            t0 = time.perf_counter()
            O.spec_verify(tl[b:b + 1], drafts[b:b + 1], ctx[b:b + 1], sp, None, ua[b:b + 1], us[b:b + 1])
            spent += time.perf_counter() - t0
            n += 1
        return n, spent, f"{n} sequences of the same batch (the oracle verifies one at a time)"

    line = _timed_split(run, budget_s)
    line["unit"] = "verified sequences/s"
    return line


def cpu_baseline(cfg, w, K, Vv, budget_s):
    """The float64 oracle as it stands, on a bounded sample of the same workload and inputs.

    The oracle runs one row of one sequence at a time, so a sequence's round costs it the same
    inside or outside the batch: the sample is round 0 of sequences 0, 1, 2, ... (batched
    workloads) or rounds 0, 1, 2, ... of the one sequence (B = 1), each with the same catch-up
    rows, draft steps, target-logit recipe and verification as the device rounds, until the time
    budget is spent.  Building the float64 weights and loading each sequence's KV prefix are
    set-up, outside the timed part."""
    import oracle as O
    from synth import make_first_round, make_round_hiddens, make_round_noise, make_round_uniforms
    model = O.OracleModel(cfg, w)
    B, D = cfg.batch, cfg.D
    toks0, hid0 = make_first_round(cfg)
    noise0 = make_round_noise(cfg, 0)
    sp = cfg.sampling

    def run(budget):
        tokens_out = units = 0
        spent = 0.0
        b = r = 0
        cache = None
        toks = hid = None
        while units < 1 or spent < budget:
            if cache is None:   # a fresh sequence: its KV prefix and first catch-up row
                cache = O.KVCache(cfg, 1, cfg.ctx + 64 * (D + 1))
                cache.load_prefix(K[:, b:b + 1], Vv[:, b:b + 1], cfg.ctx)
                toks, hid = toks0[b:b + 1], hid0[b:b + 1]
            noise = noise0[b:b + 1] if r == 0 else make_round_noise(cfg, r)[b:b + 1]
            ua, us = make_round_uniforms(cfg.index, B, D, r)
            t0 = time.perf_counter()
            drafts, _, logits, _ = O.draft_loop(model, cache, toks, hid, D)
            ctx = cache.len.copy() - (D - 1)
            tl = np.concatenate([logits, logits[:, D - 1:D]], axis=1).astype(np.float32) + noise
            res = O.spec_verify(tl, drafts, ctx, sp, None, ua[b:b + 1], us[b:b + 1])
            O.kv_crop(cache, ctx)
            spent += time.perf_counter() - t0
            tokens_out += int(res.n_accept[0]) + 1
            units += 1
            if B > 1 or r + 1 >= 64:   # batched: the next sequence's round 0
                b, r, cache = (b + 1) % B, 0, None
            else:                      # one sequence: its next round
                r += 1
                toks, hid = res.out_tokens, make_round_hiddens(cfg, r)[:1]
        what = (f"round 0 of {units} of the {B} sequences" if B > 1 else f"{units} rounds of the one sequence")
        return tokens_out, spent, what + " (float64 NumPy, row by row)"

    line = _timed_split(run, budget_s)
    line["unit"] = "accepted tokens/s"
    return line


if __name__ == "__main__":
    main()
