#!/usr/bin/env python3
"""Throughput of the speculative-decoding verify step on one MI355X.

One step = spec_verify_attn (one attention layer over the paged KV cache)
followed by spec_reject_sample (full-vocabulary verifier + KV commit) for one
batch; with --tree SHAPE, spec_verify_attn_tree + spec_reject_sample_tree
over a draft tree of that shape instead.  Default workload: the Llama-3-8B-shaped serving batch (B=64, K=7,
V=128256, 32 q / 8 kv heads, D=128, contexts U[2048, 8192], bf16, T=1,
draft noise giving alpha ~ 0.8).

Inputs are resident in device memory before the timed region.  Three logit
sets rotate between steps (the logits of one set, 246 MB, are about the size
of the 256 MB Infinity Cache); every step gets its own pre-copied kv_len
buffer, because the verifier commits into it.

Prints one JSON line.  ``value`` = committed tokens per second: the sum over
sequences of (accepted drafts + 1) per step, divided by the time of the timed
steps (HIP events around the whole loop; nothing else is in the stream).
``roofline`` is for the dominant call (attention), timed afterwards over the
same number of back-to-back launches with HIP events on the launch stream;
``kernels`` gives the same for the reject call; ``cpu_baseline`` times the
float64 oracle on a bounded sample of the same workload on the host cores.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified tokens/sec at batch 64, K=7, V=128256; % of peak HBM GB/s"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0          # dense bf16 MFMA


def _files_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic():
    """HBM bytes per attention call from the committed rocprofv3 counter runs
    (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy of known size), if they
    were taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "attn_llama8b_b64_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    try:
        if rec.get("source_sha256_16") != _files_hash(rec["source_files"]):
            return None
    except (KeyError, OSError):
        return None
    return rec.get("bytes_per_launch")


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="llama8b_b64")
    p.add_argument("--batch", type=int, default=0,
                   help="batch size instead of the workload's (e.g. the low-concurrency sweep "
                        "1, 2, 4, 8); 0: the workload's")
    p.add_argument("--temp", type=float, default=1.0)
    p.add_argument("--seed", type=int, default=2024)
    p.add_argument("--cpu-sample", type=int, default=64,
                   help="sequences in the oracle's timed sample (0 disables)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="repeat the oracle over the sample until this much CPU time has passed")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="instead of the bench: copy MIB MiB device to device 8 times (the "
                        "known-size kernel that scales the HBM byte counters), then exit")
    p.add_argument("--peak-probe", action="store_true",
                   help="instead of the bench: time the streaming-read probe (spec_read_probe) "
                        "over a 2 GiB buffer and print its bandwidth, then exit")
    p.add_argument("--k-layout-ab", default="", metavar="LIB",
                   help="instead of the bench: time spec_verify_attn with the in-tree library "
                        "(K pages [D/8,16,8]) against LIB, a build with SV_K_TOKEN_MAJOR=1 "
                        "(token-major K pages [16,D]) given the same cache permuted; the "
                        "outputs must agree bit for bit")
    p.add_argument("--lib", default="", metavar="LIB",
                   help="load LIB instead of the in-tree library (another build of it)")
    p.add_argument("--wg-timeline", action="store_true",
                   help="after the bench, one more attention call with a library built with "
                        "SV_ATTN_TIMESTAMPS=1 (--lib): add the per-workgroup timeline of "
                        "k_attn_stream to the line as wg_timeline")
    p.add_argument("--traffic-record", nargs=4, default=None,
                   metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                   help="instead of the bench (no GPU needed): write "
                        "profiles/attn_llama8b_b64_traffic.json from four rocprofv3 --pmc output "
                        "folders: FETCH_SIZE and WRITE_SIZE of this bench at its defaults, then of "
                        "--copy-calibration 1024")
    p.add_argument("--no-probe", action="store_true",
                   help="skip the streaming-read probe in the bench line (measured_peak null)")
    p.add_argument("--sets", type=int, default=3, help="rotating logit sets")
    p.add_argument("--window", default="none", choices=["none", "append", "scratch", "separate"],
                   help="where the window's K/V come from: already in the cache (none); from "
                        "the projection output, stored into the cache by the attention kernel "
                        "(append) or committed afterwards by spec_kv_commit (scratch); or a "
                        "separate copy pass before the plain attention (separate)")
    p.add_argument("--top-k", type=int, default=0,
                   help="top-k filter for every sequence (spec_reject_sample_filtered, or "
                        "spec_reject_sample_tree_filtered with --tree; 0: off)")
    p.add_argument("--top-p", type=float, default=1.0,
                   help="top-p filter for every sequence (1: off)")
    p.add_argument("--tree-mix", type=int, default=0, metavar="N",
                   help="verify one draft tree of N nodes per sequence (a mix of chains, stars, "
                        "two-level and random trees): spec_verify_attn_tree with per-sequence "
                        "ancestor sets + spec_reject_sample_trees")
    p.add_argument("--tree", default="", metavar="SHAPE",
                   help="verify a draft tree instead of a chain: branching factors per level, "
                        "e.g. 2,2,2 (15 nodes); times spec_verify_attn_tree + "
                        "spec_reject_sample_tree on the same serving batch")
    return p.parse_args()


def main():
    args = parse()
    if args.traffic_record:
        traffic_record(*args.traffic_record)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the verify step here runs on a single "
              "MI355X (no collectives); --gpus %d is not supported." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import speculative_decoding_verification_verify_amd as sv
    from synth import CONFIGS, gen
    from synth.device import to_device, from_device, make_attn_inputs_device

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.lib:
        lib = os.path.abspath(args.lib)
        sv.lib_path = lambda: lib
    sv.load()
    if args.peak_probe:
        print(json.dumps(read_peak(sv)), flush=True)
        return
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.k_layout_ab:
        k_layout_ab(args, args.k_layout_ab)
        return
    cfg = CONFIGS[args.config]
    B, K, V = (args.batch or cfg.B), cfg.K, cfg.V
    parent = None
    if args.tree and args.tree_mix:
        raise SystemExit("--tree and --tree-mix exclude each other")
    if args.tree:
        from synth.tree import tree_parents
        shape = tuple(int(x) for x in args.tree.split(","))
        parent = tree_parents(shape)
        K = len(parent) - 1                       # window of N = K + 1 tree nodes
    elif args.tree_mix:
        from synth.tree import mixed_parents
        if not 1 <= args.tree_mix <= 17:
            raise SystemExit("--tree-mix takes 1..17 nodes")
        parent = mixed_parents(args.seed, B, args.tree_mix)     # [B, N]: one tree per sequence
        K = args.tree_mix - 1
    K1 = K + 1
    print("bench: %s B=%d K=%d V=%d T=%.2f steps=%d warmup=%d" %
          (cfg.name, B, K, V, args.temp, args.steps, args.warmup), file=sys.stderr, flush=True)

    # ---- inputs, resident before timing ---------------------------------
    attn = make_attn_inputs_device(args.seed, B, K, cfg.Hq, cfg.Hkv, cfg.D, cfg.ctx, dev)
    kv0 = attn["kv_len"]
    max_kv = int(from_device(kv0).max())
    rsets = []
    for j in range(args.sets):
        if parent is None:
            inp = gen.make_reject_inputs(seed=args.seed + 1 + j, B=B, K=K, V=V,
                                         dtype=cfg.logit_dtype, logit_std=cfg.logit_std,
                                         draft_sigma=cfg.draft_sigma, temperature=args.temp)
        else:
            inp = gen.make_tree_reject_inputs(seed=args.seed + 1 + j, B=B, parent=parent, V=V,
                                              dtype=cfg.logit_dtype, logit_std=cfg.logit_std,
                                              draft_sigma=cfg.draft_sigma,
                                              temperature=args.temp)
        rsets.append({"host": inp, "dev": {k: to_device(v, dev) for k, v in inp.items()
                                           if k != "parent"}})
    kn = vn = None
    if args.window != "none":
        kn_h, vn_h = gen.make_window_kv(args.seed + 99, B, K1, cfg.Hkv, cfg.D)
        kn, vn = to_device(kn_h, dev), to_device(vn_h, dev)
    anc = par_dev = None
    if parent is not None:
        from synth.tree import ancestor_bits
        bits = (np.stack([ancestor_bits(p) for p in parent]) if parent.ndim == 2
                else np.broadcast_to(ancestor_bits(parent), (B, K1)))
        anc = to_device(bits.astype(np.uint32).copy().view(np.int32), dev)
        if parent.ndim == 2:
            par_dev = to_device(parent.astype(np.int32), dev)
    n_total = args.warmup + args.steps
    kv_bufs = [kv0.clone() for _ in range(n_total)]
    attn_out = torch.empty_like(attn["q"])
    attn_ws = torch.empty(max(256, sv.verify_attn_workspace_bytes(B, K, cfg.Hq, cfg.Hkv, cfg.D,
                                                                  max_kv)),
                          dtype=torch.uint8, device=dev)
    filtered = args.top_k > 0 or args.top_p < 1.0
    if parent is None:
        rej_bytes = (sv.reject_sample_filtered_workspace_bytes(B, K, V) if filtered else
                     sv.reject_sample_workspace_bytes(B, K, V))
    else:
        rej_bytes = (sv.reject_sample_tree_filtered_workspace_bytes(B, K1, V) if filtered else
                     sv.reject_sample_tree_workspace_bytes(B, K1, V))
    rej_ws = torch.empty(rej_bytes,
                         dtype=torch.uint8, device=dev)
    out_tok = [torch.empty((B, K1), dtype=torch.int32, device=dev) for _ in range(args.sets)]
    out_node = [torch.empty((B, K1), dtype=torch.int32, device=dev) for _ in range(args.sets)]
    n_acc = [torch.empty((B,), dtype=torch.int32, device=dev) for _ in range(args.sets)]
    torch.cuda.synchronize()
    print("bench: inputs resident", file=sys.stderr, flush=True)

    filt_k = filt_p = None
    if args.top_k > 0 or args.top_p < 1.0:
        # The drafts stay the generator's (unfiltered) draws: the filter's
        # cost does not depend on them.
        filt_k = torch.full((B,), args.top_k, dtype=torch.int32, device=dev)
        filt_p = torch.full((B,), args.top_p, dtype=torch.float32, device=dev)
    all_acc = torch.full((B,), K, dtype=torch.int32, device=dev)
    kv_full = kv0 + K1                                   # lengths as if every row survived

    def attn_call():
        if args.window in ("append", "scratch"):
            sv.verify_attn_window(attn["q"], kn, vn, attn["k_cache"], attn["v_cache"],
                                  attn["block_table"], kv0, anc=anc,
                                  mode=sv.SV_WINDOW_APPEND if args.window == "append"
                                  else sv.SV_WINDOW_READ,
                                  out=attn_out, max_kv_len=max_kv, workspace=attn_ws)
            return
        if args.window == "separate":
            # The window copied into its slots by its own pass (every row kept).
            sv.kv_commit(attn["k_cache"], attn["v_cache"], attn["block_table"], kv_full, all_acc,
                         k_src=kn, v_src=vn, N=K1)
        if parent is None:
            sv.verify_attn(attn["q"], attn["k_cache"], attn["v_cache"], attn["block_table"], kv0,
                           out=attn_out, max_kv_len=max_kv, workspace=attn_ws)
        else:
            sv.verify_attn_tree(attn["q"], attn["k_cache"], attn["v_cache"], attn["block_table"],
                                kv0, anc, out=attn_out, max_kv_len=max_kv, workspace=attn_ws)

    # Greedy verification reads no draft logits: at T <= 0 none are passed (the
    # library then knows every sequence is greedy and sizes its grids to it).
    greedy_only = args.temp <= 0

    def reject_call(s, kv):
        r = rsets[s % args.sets]["dev"]
        drf = None if greedy_only else r["draft"]
        if parent is None:
            sv.reject_sample(r["target"], drf, r["draft_tokens"], r["uniforms"],
                             r["temperature"], kv, out_tokens=out_tok[s % args.sets],
                             num_accepted=n_acc[s % args.sets], workspace=rej_ws,
                             top_k=filt_k, top_p=filt_p)
        elif par_dev is not None:
            sv.reject_sample_trees(r["target"], drf, par_dev, r["tokens"], r["uniforms"],
                                   r["temperature"], kv, out_tokens=out_tok[s % args.sets],
                                   out_nodes=out_node[s % args.sets],
                                   num_accepted=n_acc[s % args.sets], workspace=rej_ws,
                                   top_k=filt_k, top_p=filt_p)
        else:
            sv.reject_sample_tree(r["target"], drf, parent, r["tokens"], r["uniforms"],
                                  r["temperature"], kv, out_tokens=out_tok[s % args.sets],
                                  out_nodes=out_node[s % args.sets],
                                  num_accepted=n_acc[s % args.sets], workspace=rej_ws,
                                  top_k=filt_k, top_p=filt_p)

    def commit_call(s, kv):
        # Scratch window: the surviving rows into the cache; a tree appended in
        # place: its path compacted.  A chain appended in place has nothing to move.
        if args.window == "scratch" or (args.window == "append" and parent is not None):
            sv.kv_commit(attn["k_cache"], attn["v_cache"], attn["block_table"], kv,
                         n_acc[s % args.sets],
                         nodes=out_node[s % args.sets] if parent is not None else None,
                         k_src=kn if args.window == "scratch" else None,
                         v_src=vn if args.window == "scratch" else None, N=K1)

    def step(s):
        attn_call()
        reject_call(s, kv_bufs[s])
        commit_call(s, kv_bufs[s])

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    emitted = [int(from_device(n_acc[j]).astype(np.int64).sum()) + B for j in range(args.sets)]

    # ---- timed region: whole verify steps, nothing else in the stream -----
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for s in range(args.warmup, n_total):
        step(s)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    tokens = sum(emitted[s % args.sets] for s in range(args.warmup, n_total))
    value = tokens / (total_ms / 1e3)

    # Committed lengths must be L0 + n + 1 for the last step's set.
    last = n_total - 1
    assert np.array_equal(from_device(kv_bufs[last]),
                          from_device(kv0) + from_device(n_acc[last % args.sets]) + 1)

    # ---- each call alone: the same number of back-to-back launches, bracketed
    # by HIP events on the launch stream (torch's current stream) -------------
    timing_mode = []

    def timed(fn):
        """Mean GPU time of one call: the same number of back-to-back calls,
        captured in one HIP graph and replayed between HIP events on the
        launch stream, so the host's per-call launch cost (Python argument
        checks, ctypes) is not in the figure; a short call is otherwise
        limited by how fast the host enqueues it.  Falls back to eager
        launches if the capture fails."""
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        try:
            g = torch.cuda.CUDAGraph()
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                for s in range(args.steps):
                    fn(s)
            g.replay()                                  # warm-up replay
            torch.cuda.synchronize()
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            timing_mode.append("graph")
            del g
        except Exception as exc:                        # pragma: no cover - device dependent
            print("bench: graph capture failed (%s); timing eager launches" % exc,
                  file=sys.stderr, flush=True)
            torch.cuda.synchronize()
            e0.record()
            for s in range(args.steps):
                fn(s)
            e1.record()
            torch.cuda.synchronize()
            timing_mode.append("eager")
        return e0.elapsed_time(e1) / args.steps

    attn_ms = timed(lambda s: attn_call())
    kv_scratch = kv0.clone()
    rej_ms = timed(lambda s: reject_call(s, kv_scratch))
    commits = args.window == "scratch" or (args.window == "append" and parent is not None)
    commit_ms = (timed(lambda s: commit_call(n_total - 1, kv_bufs[n_total - 1]))
                 if commits else None)

    # ---- roofline of the attention call (dominant kernel) ----------------
    kvl = from_device(kv0).astype(np.int64)
    kv_bytes = int((kvl + K1).sum()) * cfg.Hkv * cfg.D * 2 * 2
    qo_bytes = B * K1 * cfg.Hq * cfg.D * 2 * 2
    # The window's K/V are read once whatever their source; append also
    # writes them into the cache.
    win_write = B * K1 * cfg.Hkv * cfg.D * 2 * 2 if args.window == "append" else 0
    attn_bytes = kv_bytes + qo_bytes + win_write
    attn_us = float(attn_ms * 1e3)
    achieved = attn_bytes / (attn_us * 1e-6) / 1e9
    # Algorithmic MFMA work: QK^T and PV, 2 D flops each per (query row,
    # visible key); a chain's row i sees L0 + i + 1 keys, a tree node L0 plus
    # its path.
    if parent is None:
        vis = int(sum(int(l) * K1 + K1 * (K1 + 1) // 2 for l in kvl))
    else:
        pars = parent if parent.ndim == 2 else np.broadcast_to(parent, (B, K1))
        depth = [sum(bin(int(a)).count("1") for a in ancestor_bits(pp)) for pp in pars]
        vis = int(sum(int(l) * K1 + dep for l, dep in zip(kvl, depth)))
    attn_flops = 4 * cfg.D * cfg.Hq * vis
    attn_tflops = attn_flops / (attn_us * 1e-6) / 1e12
    # The sweep reads every target row and the draft rows of the nodes with
    # children (all K draft rows of a chain); greedy reads target rows only.
    # The exact passes after rejections come on top and are not counted.
    if parent is None:
        n_draft_rows = B * K
    else:
        pars = parent if parent.ndim == 2 else np.broadcast_to(parent, (B, K1))
        n_draft_rows = sum(len(set(int(x) for x in pp[1:])) for pp in pars)
    rej_bytes = (B * K1 + (n_draft_rows if args.temp > 0 else 0)) * V * 2
    probe = None if args.no_probe else read_peak(sv, sizes={"attn": attn_bytes,
                                                            "reject": rej_bytes})
    measured_peak = None if probe is None else probe["gbs"]
    same = {} if probe is None else probe["same_size"]

    def vs_probe(name, us):
        # Time of the probe over the call's bytes / time of the call.
        return None if name not in same else round(same[name]["avg_us"] / us, 4)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": (_traffic() if parent is None and args.window == "none"
                            and cfg.name == "llama8b_b64" and B == cfg.B and args.seed == 2024
                            else None),
                "kernel": "%s call = k_attn_stream + k_attn_stream_combine" %
                          ("spec_verify_attn_window (%s)" % args.window
                           if args.window in ("append", "scratch") else
                           "spec_verify_attn" if parent is None else "spec_verify_attn_tree"),
                "algorithmic_bytes": attn_bytes, "avg_us": round(attn_us, 2),
                "measured_peak": measured_peak,
                "frac_of_measured_peak": (None if not measured_peak
                                          else round(achieved / measured_peak, 4)),
                "frac_of_same_size_probe": vs_probe("attn", attn_us),
                "mfma": {"tflops": round(attn_tflops, 1), "algorithmic_flops": attn_flops,
                         "peak_tflops": PEAK_BF16_TFLOPS,
                         "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4)}}
    rej_us = float(rej_ms * 1e3)
    rej_gbs = rej_bytes / (rej_us * 1e-6) / 1e9
    # Both calls of the step against the HBM peak, and the smaller of the two.
    by_call = {"attn": round(achieved / PEAK_HBM_GBS, 4), "reject": round(rej_gbs / PEAK_HBM_GBS, 4)}
    roofline["frac_by_call"] = by_call
    roofline["min_frac_by_call"] = min(by_call.values())
    # The rows the method itself needs: drafts after the first rejection are
    # discarded, so a chain needs target rows 0..n and draft rows
    # 0..min(n, K-1) (greedy: target rows 0..n), averaged over the sets the
    # timed calls rotate through.
    min_rows = None
    if parent is None:
        tot = 0
        for j in range(args.sets):
            n = from_device(n_acc[j]).astype(np.int64)
            tot += int((n + 1).sum()) + (int(np.minimum(n + 1, K).sum()) if args.temp > 0 else 0)
        min_rows = tot / args.sets
    rej_min_bytes = None if min_rows is None else int(round(min_rows * V * 2))

    # ---- CPU baseline: the oracle on a bounded sample ---------------------
    cpu = None
    if args.cpu_sample > 0:
        cpu = cpu_baseline(args, cfg, attn, rsets[0]["host"], from_device, parent)

    if parent is None:
        window_desc = "K=%d" % K
    elif parent.ndim == 1:
        window_desc = "draft tree [%s] (%d nodes)" % (args.tree, K1)
    else:
        window_desc = "one draft tree of %d nodes per sequence (mixed shapes)" % K1
    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s: B=%d %s V=%d, %dq/%dkv heads D=%d, ctx U[%d,%d], "
                               "bf16 logits N(0,2), draft sigma %.2f, T=%.2f" %
                               (cfg.name, B, window_desc,
                                V, cfg.Hq, cfg.Hkv, cfg.D, cfg.ctx[0], cfg.ctx[1],
                                cfg.draft_sigma, args.temp),
                   "global_batch": B, "K": K, "V": V, "parallelism": "single GPU",
                   "window": args.window, "top_k": args.top_k, "top_p": args.top_p},
        "roofline": roofline,
        "roofline_reject": {"bound": "hbm", "achieved": round(rej_gbs, 1), "peak": PEAK_HBM_GBS,
                            "unit": "GB/s", "frac": round(rej_gbs / PEAK_HBM_GBS, 4),
                            "traffic": None,
                            "kernel": "spec_reject_sample%s call" % (
                                "" if parent is None else "_tree" if parent.ndim == 1
                                else "_trees"),
                            "algorithmic_bytes": rej_bytes, "avg_us": round(rej_us, 2),
                            "frac_of_same_size_probe": vs_probe("reject", rej_us)},
        "read_probe": probe,
        "cpu_baseline": cpu,
        "kernels": {
            "attn": {"avg_us": round(attn_us, 2), "gbs": round(achieved, 1),
                     "frac_hbm": round(achieved / PEAK_HBM_GBS, 4), "bytes": attn_bytes},
            "reject": {"avg_us": round(rej_us, 2), "gbs": round(rej_gbs, 1),
                       "frac_hbm": round(rej_gbs / PEAK_HBM_GBS, 4), "bytes": rej_bytes,
                       "frac_of_measured_peak": (None if not measured_peak
                                                 else round(rej_gbs / measured_peak, 4)),
                       "frac_of_same_size_probe": vs_probe("reject", rej_us),
                       "min_rows_bytes": rej_min_bytes,
                       "min_rows_per_seq": (None if min_rows is None
                                            else round(min_rows / B, 3)),
                       "frac_hbm_min_rows": (None if rej_min_bytes is None else round(
                           rej_min_bytes / (rej_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4))},
            "commit": None if commit_ms is None else {"avg_us": round(float(commit_ms * 1e3), 2)},
        },
        "per_call_timing": "/".join(sorted(set(timing_mode))),
        "tokens_per_step": round(tokens / args.steps, 2),
        "positions_per_s": round(B * K1 * args.steps / (total_ms / 1e3), 1),
        "mean_accept_len": round(tokens / args.steps / B, 4),
        "wall_s": round(wall, 3),
    }
    if args.wg_timeline:
        attn_call()
        torch.cuda.synchronize()
        rec["wg_timeline"] = wg_timeline(sv.load())
    print(json.dumps(rec), flush=True)


def wg_timeline(lib):
    """Summary of the per-wave stamps of the last k_attn_stream launch (a
    build with SV_ATTN_TIMESTAMPS=1; the device clock runs at 100 MHz).  Per
    workgroup: its end (last merge end, from the earliest start of any
    workgroup), the prologue (start to segment loop), the waves' wait at the
    end-of-segment barrier (for each segment, the mean over waves of the
    slowest wave's pair-loop end minus their own) and the merges (slowest
    pair-loop end to merge end), summed over its segments.  Workgroup w is
    counted on XCD w mod 8 (round-robin dispatch)."""
    import ctypes
    import heapq
    if not hasattr(lib, "spec_attn_timestamps"):
        raise SystemExit("--wg-timeline needs a library built with SV_ATTN_TIMESTAMPS=1 (--lib)")
    fn = lib.spec_attn_timestamps
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    fn.restype = ctypes.c_size_t
    n = fn(None, 0)
    buf = np.zeros(n // 8, dtype=np.uint64)
    if fn(buf.ctypes.data_as(ctypes.c_void_p), n) != n:
        raise SystemExit("spec_attn_timestamps failed")
    ev = 24
    nw = int(buf[ev - 2])
    a = buf.reshape(-1, nw, ev).astype(np.int64)
    wgs = [w for w in range(a.shape[0]) if a[w, 0, ev - 1] > 0]
    t0 = min(int(a[w, :, 0].min()) for w in wgs)
    end, pro, wait, merge, segs = [], [], [], [], []
    for w in wgs:
        k = min(int(a[w, 0, ev - 1]), (ev - 4) // 2)
        le = np.array([a[w, :, 2 + 2 * j] for j in range(k)])     # [segment, wave]
        me = np.array([a[w, :, 3 + 2 * j] for j in range(k)])
        end.append((me[-1].max() - t0) / 100.0)
        pro.append((a[w, :, 1].max() - a[w, :, 0].min()) / 100.0)
        wait.append(float((le.max(1)[:, None] - le).mean(1).sum()) / 100.0)
        merge.append(float((me.max(1) - le.max(1)).sum()) / 100.0)
        segs.append(int(a[w, 0, ev - 1]))
    end = np.array(end)
    xcd = np.array(wgs) % 8
    r = lambda v: round(float(v), 1)
    # Replay with balancing: each workgroup keeps its own measured rate; the
    # last fraction f of the work is cut into chunks of `pairs` (in units of
    # a share's pairs per workgroup: the shares are equal), each taken by the
    # workgroup that is free first, at a fixed cost `cost_us` per chunk.
    share = 1.0 / len(end)
    rate = share / end                       # work fraction per microsecond
    replay = {}
    for f, nchunk, cost in ((0.1, 512, 1.0), (0.1, 512, 2.0), (0.1, 512, 4.0), (0.2, 256, 2.0)):
        heap = [((1.0 - f) * share / rate[i], i) for i in range(len(end))]
        heapq.heapify(heap)
        for _ in range(nchunk):
            t, i = heapq.heappop(heap)
            heapq.heappush(heap, (t + f / nchunk / rate[i] + cost, i))
        replay["f%.1f_chunks%d_cost%.0fus" % (f, nchunk, cost)] = r(max(t for t, _ in heap))
    return {"workgroups": len(wgs), "waves_per_workgroup": nw, "kernel_span_us": r(end.max()),
            "wg_end_us": {"mean": r(end.mean()), "min": r(end.min()), "max": r(end.max()),
                          "p10": r(np.percentile(end, 10)), "p90": r(np.percentile(end, 90))},
            "wg_end_mean_by_xcd_us": [r(end[xcd == x].mean()) for x in range(8) if (xcd == x).any()],
            "prologue_mean_us": r(np.mean(pro)), "barrier_wait_mean_us": r(np.mean(wait)),
            "merge_mean_us": r(np.mean(merge)), "segments_mean": r(np.mean(segs)),
            "balanced_end_us_replay": replay}


def read_peak(sv, mib=2048, reps=5, sizes=None):
    """Streaming-read bandwidth of this GPU: spec_read_probe over a 2 GiB
    buffer (8x the last-level cache), best of a few grid sizes, each timed
    over ``reps`` back-to-back launches with HIP events on the launch stream;
    then, per entry of ``sizes`` (name -> bytes), the probe over that many
    bytes."""
    import torch
    buf = torch.zeros(mib << 20, dtype=torch.uint8, device="cuda:0")
    best = None
    for grid in (2048, 4096, 8192, 16384):
        sink = torch.empty(grid, dtype=torch.int32, device="cuda:0")
        sv.read_probe(buf, sink, grid)                  # warm-up
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            sv.read_probe(buf, sink, grid)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        gbs = buf.numel() / (us * 1e-6) / 1e9
        if best is None or gbs > best["gbs"]:
            best = {"gbs": round(gbs, 1), "grid": grid, "bytes": buf.numel(), "avg_us": round(us, 1)}
    best["kernel"] = "spec_read_probe (16-byte nontemporal loads, 8 KB per wave step)"
    # The same probe over exactly the bytes of each timed call: short reads
    # pay the launch ramp and drain too, so this is the ceiling a call of that
    # size can reach.  Consecutive launches read consecutive windows of the
    # buffer (2 GiB, 8x the last-level cache), so no window is still cached;
    # timed like the calls, as one HIP graph of back-to-back launches.
    best["same_size"] = {}
    for name, nbytes in (sizes or {}).items():
        n = (int(nbytes) + 8191) // 8192 * 8192
        if n > buf.numel():
            continue
        launches = 16
        span = buf.numel() - n
        wins = [buf[(k * n) % (span + 1) // 8192 * 8192:][:n] for k in range(launches)]
        res = None
        for grid in (1024, 2048, 4096, 8192):
            sink = torch.empty(grid, dtype=torch.int32, device="cuda:0")
            g = torch.cuda.CUDAGraph()
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                for w in wins:
                    sv.read_probe(w, sink, grid)
            g.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / launches
            del g
            if res is None or us < res["avg_us"]:
                res = {"bytes": n, "grid": grid, "avg_us": round(us, 2),
                       "gbs": round(n / (us * 1e-6) / 1e9, 1)}
        best["same_size"][name] = res
    del buf
    torch.cuda.empty_cache()
    return best


def k_layout_ab(args, other_lib):
    """Attention call time with each K page layout, same inputs: the in-tree
    library reads [D/8, 16, 8] pages, ``other_lib`` (built with
    SV_K_TOKEN_MAJOR=1) reads the same cache permuted to token-major
    [16, D].  Each timed as a graph of ``args.steps`` calls, twice in
    alternation; one JSON line."""
    import torch
    import speculative_decoding_verification_verify_amd as sv
    from synth import CONFIGS
    from synth.device import from_device, make_attn_inputs_device
    cfg = CONFIGS[args.config]
    B, K = (args.batch or cfg.B), cfg.K
    dev = "cuda:0"
    attn = make_attn_inputs_device(args.seed, B, K, cfg.Hq, cfg.Hkv, cfg.D, cfg.ctx, dev)
    kv0 = attn["kv_len"]
    max_kv = int(from_device(kv0).max())
    kc = attn["k_cache"]
    kc_tok = kc.permute(0, 1, 3, 2, 4).contiguous().view(kc.shape)   # [NB, Hkv, 16, D] bytes
    out = torch.empty_like(attn["q"])
    libs = (("chunked [D/8,16,8]", sv.lib_path(), kc), ("token-major [16,D]", other_lib, kc_tok))
    ref, times = None, {}
    for _ in range(2):
        for name, path, k in libs:
            sv._LIB = None
            sv.lib_path = (lambda p=path: p)
            sv.load()
            ws = torch.empty(max(256, sv.verify_attn_workspace_bytes(B, K, cfg.Hq, cfg.Hkv, cfg.D,
                                                                      max_kv)),
                             dtype=torch.uint8, device=dev)

            def call():
                sv.verify_attn(attn["q"], k, attn["v_cache"], attn["block_table"], kv0, out=out,
                               max_kv_len=max_kv, workspace=ws)
            call()
            torch.cuda.synchronize()
            o = from_device(out)
            if ref is None:
                ref = o
            elif not np.array_equal(o, ref):
                raise SystemExit("k-layout A/B: outputs differ between the layouts")
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(args.steps):
                    call()
            g.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            times.setdefault(name, []).append(round(e0.elapsed_time(e1) * 1e3 / args.steps, 2))
            del g
    print(json.dumps({"k_layout_ab": {"workload": cfg.name, "B": B, "K": K,
                                      "call_us": times, "outputs_identical": True}}), flush=True)


def _counter_means(folder):
    """Mean value per kernel name of the one counter in a rocprofv3 --pmc
    output folder (its counter_collection CSV)."""
    import csv
    import glob
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection CSV under %s" % folder)
    acc = {}
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def traffic_record(fetch_dir, write_dir, cfetch_dir, cwrite_dir):
    """HBM bytes per attention call from the FETCH_SIZE / WRITE_SIZE counter
    runs, each scaled by the same counter on a 1 GiB device copy (reads and
    writes 1 GiB per dispatch), with a hash of the attention sources: bench.py
    reports the figure only while the sources still hash to it."""
    copy_bytes = 1 << 30
    cf = [v for k, v in _counter_means(cfetch_dir).items() if "copyBuffer" in k]
    cw = [v for k, v in _counter_means(cwrite_dir).items() if "copyBuffer" in k]
    if not cf or not cw:
        raise SystemExit("no copy kernel in the calibration folders")
    fscale = copy_bytes / (cf[0] * 1024.0)
    wscale = copy_bytes / (cw[0] * 1024.0)
    fetch, write = _counter_means(fetch_dir), _counter_means(write_dir)
    per = {}
    for name, fv in fetch.items():
        if "sv::" not in name:
            continue
        short = name.split("(")[0].replace("void ", "")
        wv = write.get(name, 0.0)
        per[short] = {"fetch_kib": round(fv, 3), "write_kib": round(wv, 3),
                      "fetch_bytes": int(round(fv * 1024 * fscale)),
                      "write_bytes": int(round(wv * 1024 * wscale))}
    attn = [k for k in per if k.startswith("sv::k_attn_stream")]
    if not attn:
        raise SystemExit("no attention kernel in %s" % fetch_dir)
    files = ["speculative_decoding_verification_verify_amd/csrc/verify_attn.hip",
             "speculative_decoding_verification_verify_amd/csrc/common.h"]
    rec = {"workload": "llama8b_b64 (B=64 K=7, 32q/8kv, D=128, ctx U[2048,8192], seed 2024)",
           "call": "spec_verify_attn = k_attn_stream + k_attn_stream_combine",
           "source_files": files, "source_sha256_16": _files_hash(files),
           "fetch_scale": fscale, "write_scale": wscale,
           "bytes_per_launch": sum(per[k]["fetch_bytes"] + per[k]["write_bytes"] for k in attn),
           "summary": "profiles/verify_step_llama8b_b64_counters.md", "per_kernel": per}
    out = os.path.join(ROOT, "profiles", "attn_llama8b_b64_traffic.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps({k: rec[k] for k in ("bytes_per_launch", "fetch_scale", "write_scale")}))


def copy_calibration(mib):
    """A plain device-to-device copy of known size: its FETCH_SIZE / WRITE_SIZE
    counters give the scale from counter units to bytes."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(8):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 8}), flush=True)


def cpu_baseline(args, cfg, attn, host_rej, from_device, parent=None):
    """Time the oracle (as it stands) on the first ``cpu_sample`` sequences of
    the same workload, repeated until ``cpu_seconds`` have passed."""
    import torch
    from oracle import attention as oat
    from oracle import reject as orj
    from oracle import tree as otr
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    K1 = cfg.K + 1 if parent is None else parent.shape[-1]
    # The tree oracle's attention masks every node separately: a smaller sample.
    B = args.batch or cfg.B
    n = min(args.cpu_sample if parent is None else max(1, args.cpu_sample // 8), B)
    idx = np.arange(n)
    kvl = from_device(attn["kv_len"])[:n]
    bt = from_device(attn["block_table"])[:n]
    pages = np.unique(np.concatenate([bt[b, :(kvl[b] + K1 + 15) // 16] for b in range(n)]))
    remap = np.zeros(int(pages.max()) + 1, dtype=np.int32)
    remap[pages] = np.arange(len(pages), dtype=np.int32)
    sel = torch.from_numpy(pages).long().to(attn["k_cache"].device)
    kc = from_device(attn["k_cache"][sel])
    vc = from_device(attn["v_cache"][sel])
    q = from_device(attn["q"][:n])
    bt_local = np.zeros_like(bt)
    for b in range(n):
        m = (kvl[b] + K1 + 15) // 16
        bt_local[b, :m] = remap[bt[b, :m]]
    h = host_rej
    if parent is not None and parent.ndim == 2:
        parent = parent[:n]                       # one tree per sequence: the sample's
    t_attn = t_rej = 0.0
    passes = tokens = 0
    while passes == 0 or t_attn + t_rej < args.cpu_seconds:
        t0 = time.perf_counter()
        if parent is None:
            oat.verify_attention(q, kc, vc, bt_local, kvl)
        else:
            otr.tree_attention(q, kc, vc, bt_local, kvl, parent)
        t_attn += time.perf_counter() - t0
        t0 = time.perf_counter()
        if parent is None:
            res = orj.reject_sample(h["target"][idx], h["draft"][idx], h["draft_tokens"][idx],
                                    h["uniforms"][idx], h["temperature"][idx])
        else:
            res = otr.reject_sample_tree(h["target"][idx], h["draft"][idx], parent,
                                         h["tokens"][idx], h["uniforms"][idx],
                                         h["temperature"][idx])
        t_rej += time.perf_counter() - t0
        tokens += int(res["num_accepted"].astype(np.int64).sum()) + n
        passes += 1
    return {"value": round(tokens / (t_attn + t_rej), 2), "unit": "tokens/s",
            "cores": int(blas_threads), "kind": "oracle",
            "sample": "first %d of %d sequences of the same workload (attention + reject), %d "
                      "pass(es): float64 numpy oracle, attention %.2f s + reject %.2f s" %
                      (n, B, passes, t_attn, t_rej),
            "host_cores_available": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()
