"""Decode-step benchmark: coarse-to-fine hash retrieval + sparse attention.

One step = one hhr_decode call (query encode, page bounds, top-P page pruning,
Hamming scan, exact top-k, split-K sparse attention) for one sequence's
one-token decode through one attention layer, all 32 query heads, on the
Llama-3.1-8B-shaped 128K workload (8 KV heads, d = 128, bf16 K/V, keep 1/8
of the pages, top-k 4096).  Inputs are seeded synthetic data resident in HBM
before timing starts; keys are encoded (the prefill-time encoder) before
timing too, and that encoder is timed separately.

To keep the 256 MB Infinity Cache from serving repeated steps, the step
rotates through --layers independent copies of every per-layer buffer
(K, V, codes, page metadata, R, W), about 4.8 GB at 8 layers.

Prints one JSON line.  `roofline` is for k_score_topp (query rotation, page
bounds and top-P in one launch), the step's longest kernel and the one that
moves most of its bytes; its average launch duration is measured with one pair
of HIP events on its stream around a pass of back-to-back hhr_select_pages
calls (which launch it alone) over the same rotating layers; `traffic` is its
counter-measured HBM bytes per launch from the committed profile, while the
kernel's sources are unchanged since.  `--meta bf16` runs the same step on
bfloat16 page metadata rounded outward (half the metadata bytes).
`cpu_baseline` times the CPU oracle (numpy fp64) on whole decode steps of the
same workload for a bounded number of seconds, once with the KV heads spread
over the host's cores and once on one core.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_FP8_PEAK_TFLOPS = 5000.0

# Measured HBM traffic of a roofline kernel comes from a committed counter profile
# (a JSON record in a fenced block of the named file under profiles/); it is reported
# only while the kernel sources that the record lists are unchanged since the counters
# were taken.
TRAFFIC_PROFILES = {
    "llama8b_128k": "score_topp_llama8b_128k_hbm_traffic.md",
    "llama8b_ragged_b16": "select_pages_ragged_b16_hbm_traffic.md",
    "hisa_128k": "hisa_token_topk_128k_hbm_traffic.md",
}


def source_digest(sources) -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str, meta_dtype: str = "f32"):
    """Calibrated HBM bytes per launch of `kernel` on `workload` from its counter profile,
    or None if there is none for this workload, kernel and metadata format, or if the
    sources listed in the record changed since."""
    name = TRAFFIC_PROFILES.get(workload)
    if name is None:
        return None
    try:
        with open(os.path.join(ROOT, "profiles", name)) as f:
            text = f.read()
        rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, IndexError, ValueError):
        return None
    for r in rec if isinstance(rec, list) else [rec]:
        if (r.get("workload") == workload and r.get("kernel") == kernel
                and r.get("meta_dtype", "f32") == meta_dtype
                and r.get("source_sha256") == source_digest(r.get("sources", []))):
            return int(r["traffic_bytes_per_launch"])
    return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="llama8b_128k")
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", type=int, default=1, help="replay the rotation as one HIP graph")
    ap.add_argument("--path", choices=("decode", "staged", "append", "append_then_decode"),
                    default="decode",
                    help="decode: one hhr_decode call per step; staged: hhr_select then "
                         "hhr_sparse_decode; append: hhr_decode_append (the step also encodes "
                         "the sequence's last key, idempotent when replayed); "
                         "append_then_decode: hhr_append_keys of that key, then hhr_decode")
    ap.add_argument("--meta", choices=("f32", "bf16"), default="f32",
                    help="page metadata format: f32 min/max, or bfloat16 rounded outward")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this size (counter calibration)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    from hash_hierarchical_top_amd import hhr, quality, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    hhr.load()
    dev = torch.device("cuda", 0)
    if args.workload in synth.HISA_WORKLOADS:
        return main_hisa(args, torch, hhr, synth, dev)
    if args.workload in synth.HISA_PREFILL_WORKLOADS:
        return main_hisa_prefill(args, torch, hhr, synth, dev)
    w = synth.WORKLOADS[args.workload]
    B, Hq, Hkv, Lcap, top_k = w.batch, w.n_q_heads, w.n_kv_heads, w.max_ctx, w.top_k
    keep = (w.keep_num, w.keep_den, w.keep_pages_abs)
    G = Hq // Hkv
    t_gen = time.time()
    inp = synth.make_workload_inputs(args.workload)
    t_gen = time.time() - t_gen
    seq_np = inp["seq_len"]
    shape = hhr.make_shape(B, Hq, Hkv, Lcap, w.kv_dtype, meta_dtype=args.meta)
    meta_dt = torch.float32 if args.meta == "f32" else torch.int32
    meta_page_bytes = 1024 if args.meta == "f32" else 512
    NpCap = Lcap // 16
    scale = 1.0 / math.sqrt(128.0)

    def kv(a):
        t = torch.from_numpy(a)
        return (t.view(torch.bfloat16) if w.kv_dtype == "bf16" else t).to(dev)

    seq = torch.from_numpy(seq_np).to(dev)
    zero = torch.zeros(B, dtype=torch.int32, device=dev)
    K0, V0 = kv(inp["K"]), kv(inp["V"])
    q = torch.from_numpy(inp["q"]).to(dev)
    R0 = torch.from_numpy(inp["R"]).to(dev)
    W0 = torch.from_numpy(inp["W"]).to(dev)
    layers = []
    for i in range(args.layers):
        lay = dict(K=K0 if i == 0 else K0.clone(), V=V0 if i == 0 else V0.clone(),
                   R=R0 if i == 0 else R0.clone(), W=W0 if i == 0 else W0.clone(),
                   codes=torch.zeros((B, Hkv, Lcap, 4), dtype=torch.int32, device=dev),
                   meta=torch.zeros(hhr.meta_shape(shape), dtype=meta_dt, device=dev))
        layers.append(lay)
    ws_bytes = hhr.hhr_workspace_size(shape, *keep, top_k)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    sel = torch.zeros((B, Hkv, top_k), dtype=torch.int32, device=dev)
    cnt = torch.zeros((B, Hkv), dtype=torch.int32, device=dev)
    out = torch.zeros((B, Hq, 128), dtype=torch.float32, device=dev)
    max_len = int(seq_np.max())

    # ---- prefill-time encoder (S1), timed per layer
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.layers)]
    for i, lay in enumerate(layers):
        ev[2 * i].record(stream)
        hhr.hhr_append_keys(shape, lay["K"], zero, seq, max_len, lay["R"], lay["W"],
                            lay["codes"], lay["meta"], ws)
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    enc_ms = float(np.median([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(1, args.layers)]
                             if args.layers > 1 else [ev[0].elapsed_time(ev[1])]))
    n_keys = int(seq_np.sum()) * Hkv
    kv_bytes = 2 if w.kv_dtype == "bf16" else 4
    enc_bytes = n_keys * (128 * kv_bytes + 16) + sum(
        -(-int(L) // 16) for L in seq_np) * Hkv * meta_page_bytes + Hkv * 2 * 128 * 128 * 4
    enc_flops = 2.0 * n_keys * 128 * 256
    passes = 2 if w.kv_dtype == "bf16" else 3
    enc = {"ms": round(enc_ms, 4), "hbm_gbs": round(enc_bytes / enc_ms / 1e6, 1),
           "tflops": round(enc_flops / enc_ms / 1e9, 2),
           "mfma_bf16_tflops_issued": round(passes * enc_flops / enc_ms / 1e9, 2),
           "mfma_util_vs_bf16_peak": round(passes * enc_flops / enc_ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4),
           "bytes": enc_bytes, "flops": enc_flops}

    last = (seq - 1).clamp(min=0)
    one = (seq > 0).to(torch.int32)

    def step(i):
        lay = layers[i % args.layers]
        if args.path == "decode":
            hhr.hhr_decode(shape, q, seq, lay["R"], lay["W"], lay["codes"], lay["meta"],
                           lay["K"], lay["V"], *keep, top_k, scale, sel, cnt, out, ws)
        elif args.path == "append":
            hhr.hhr_decode_append(shape, q, seq, lay["R"], lay["W"], lay["codes"], lay["meta"],
                                  lay["K"], lay["V"], *keep, top_k, scale, sel, cnt, out, ws)
        elif args.path == "append_then_decode":
            hhr.hhr_append_keys(shape, lay["K"], last, one, 1, lay["R"], lay["W"], lay["codes"],
                                lay["meta"], ws)
            hhr.hhr_decode(shape, q, seq, lay["R"], lay["W"], lay["codes"], lay["meta"],
                           lay["K"], lay["V"], *keep, top_k, scale, sel, cnt, out, ws)
        else:
            hhr.hhr_select(shape, q, seq, lay["R"], lay["W"], lay["codes"], lay["meta"], *keep,
                           top_k, sel, cnt, ws)
            hhr.hhr_sparse_decode(shape, q, lay["K"], lay["V"], sel, cnt, top_k, scale, out, ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    assert hhr.hhr_read_device_status(ws) == 0

    graph, graph_rem = None, None
    n_rep, rem = divmod(args.steps, args.layers)
    if args.graph:
        # one graph holding one step per layer (and one with the remaining steps, so that
        # exactly --steps steps are timed); the library enqueues only kernels
        gs = torch.cuda.Stream()
        gs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(gs):
            for i in range(args.layers):
                step(i)
        torch.cuda.current_stream().wait_stream(gs)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.layers):
                step(i)
        if rem:
            graph_rem = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph_rem):
                for i in range(rem):
                    step(i)
        torch.cuda.synchronize()
        for _ in range(max(1, args.warmup // args.layers)):
            graph.replay()
        torch.cuda.synchronize()

    # ---- timed region: exactly args.steps steps, one event pair around all of them and
    # one event per graph replay (each replay = one step of every rotated layer)
    steps = args.steps
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    rep_ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_rep + 1)] if graph else []
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    if graph is not None:
        for r in range(n_rep):
            rep_ev[r].record()
            graph.replay()
        rep_ev[n_rep].record()
        if graph_rem is not None:
            graph_rem.replay()
    else:
        for i in range(steps):
            step(i)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / steps
    value = B * steps / (total_ms / 1e3)
    per_step_us = [rep_ev[r].elapsed_time(rep_ev[r + 1]) * 1e3 / args.layers
                   for r in range(n_rep)] if graph is not None else []
    dist = None
    if per_step_us:
        pq = np.percentile(per_step_us, [10, 50, 90])
        dist = {"p10": round(float(pq[0]), 3), "p50": round(float(pq[1]), 3),
                "p90": round(float(pq[2]), 3), "unit": "us per step",
                "samples": len(per_step_us),
                "sample": f"mean step time of each graph replay of {args.layers} steps"}
    assert hhr.hhr_read_device_status(ws) == 0

    # ---- algorithmic bytes per step
    Np = np.array([-(-int(L) // 16) for L in seq_np])
    P = np.array([hhr.hhr_keep_count(int(n), *keep) for n in Np])
    cand = int(P.sum()) * 16 * Hkv
    meta_bytes = int(Np.sum()) * Hkv * meta_page_bytes
    sel_rows = int(cnt.sum().item())
    step_bytes = (meta_bytes + cand * 16 + sel_rows * 2 * 128 * kv_bytes
                  + Hkv * 2 * 128 * 128 * 4 + B * Hq * 128 * 4 * 2)
    step_gbs = step_bytes / (ms_per_step * 1e6)

    # ---- dominant kernel: k_score_topp (query rotation, page bounds, top-P), which
    # hhr_select_pages launches alone; back to back on its stream between one pair of
    # HIP events, rotating layers as the step does
    nk = min(args.steps, 400)
    p_max = hhr.hhr_keep_count(NpCap, *keep)
    kept_b = torch.zeros((B, Hkv, p_max), dtype=torch.int32, device=dev)
    kc_b = torch.zeros((B, Hkv), dtype=torch.int32, device=dev)
    ws_p = torch.zeros(hhr.hhr_workspace_size(shape, *keep, 1), dtype=torch.uint8, device=dev)

    def select_pages(i):
        lay = layers[i % args.layers]
        hhr.hhr_select_pages(shape, q, seq, lay["R"], lay["W"], lay["meta"], *keep, kept_b, kc_b,
                             None, ws_p)

    def time_launches(fn):
        for i in range(args.layers):
            fn(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(nk):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / nk

    k_ms = time_launches(select_pages)
    assert hhr.hhr_read_device_status(ws_p) == 0
    n_pages_all = int(Np.sum()) * Hkv
    # metadata, queries, R and W once per KV head, the bounds written and read back by the
    # last workgroup, kept pages and query codes written
    k_bytes = (meta_bytes + B * Hq * 128 * 4 + Hkv * 128 * 256 * 4 + n_pages_all * 8
               + int(P.sum()) * Hkv * 4 + B * Hq * 16)
    # the library runs k_score_topp while the scoring grid is at most two rounds of
    # one 1024-thread workgroup per CU, else the staged coarse launches
    one_launch = -(-NpCap // 256) * B * Hkv <= 512
    k_name = ("k_score_topp" if one_launch
              else "hhr_select_pages (k_encode_queries + k_page_scores + k_top_pages)")
    roofline = {"bound": "hbm", "achieved": round(k_bytes / (k_ms * 1e6), 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(k_bytes / (k_ms * 1e6) / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(args.workload, k_name, args.meta),
                "kernel": k_name,
                "bytes_per_launch": k_bytes, "avg_launch_us": round(k_ms * 1e3, 3)}

    # the bound computation alone (staged k_page_scores, S3 only), for context
    q_rot = torch.zeros((B, Hq, 128), dtype=torch.float32, device=dev)
    q_codes = torch.zeros((B, Hq, 4), dtype=torch.int32, device=dev)
    scores = torch.zeros((B, Hkv, NpCap), dtype=torch.float32, device=dev)
    hhr.hhr_encode_queries(shape, q, R0, W0, q_rot, q_codes)
    s_ms = time_launches(lambda i: hhr.hhr_page_scores(shape, q_rot, seq,
                                                       layers[i % args.layers]["meta"], scores,
                                                       ws))
    s_bytes = meta_bytes + B * Hq * 128 * 4 + n_pages_all * 4
    scorer_only = {"kernel": "k_page_scores", "bytes_per_launch": s_bytes,
                   "avg_launch_us": round(s_ms * 1e3, 3),
                   "achieved_gbs": round(s_bytes / (s_ms * 1e6), 1),
                   "frac": round(s_bytes / (s_ms * 1e6) / HBM_PEAK_GBS, 4)}

    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    # ---- top-k recall against the exact q.k top-k, per KV head (HHR Figure 4's form), on
    # every (b, g) of the first sequence, and the planted-key hit rate
    sel_h = sel.cpu().numpy()
    cnt_h = cnt.cpu().numpy()
    recalls, planted_hits = [], []
    L0 = int(seq_np[0])
    for g in range(Hkv):
        exact = quality.exact_topk(q[0, g * G:(g + 1) * G], K0[0, g, :L0], top_k)
        recalls.append(quality.overlap(sel_h[0, g, :int(cnt_h[0, g])], exact.cpu().numpy()))
        planted_hits.append(np.isin(inp["planted"][0, g], sel_h[0, g]).mean())

    # ---- CPU baseline: the oracle's decode step (encoded keys prepared beforehand), on all
    # host cores and on one; the same leg compares the oracle's selection from raw inputs
    # with this step's GPU selection (excused mismatches, IoU)
    cpu = agreement = None
    if not args.no_cpu_baseline:
        select_pages(0)  # the kept pages of layer 0 (every layer holds the same data)
        torch.cuda.synchronize()
        cpu, agreement = cpu_baseline(inp, w, seq_np, keep, top_k, scale, args.cpu_seconds,
                                      gpu_sel=sel_h, gpu_cnt=cnt_h,
                                      gpu_codes=layers[0]["codes"].cpu().numpy().view(np.uint32),
                                      gpu_kept=kept_b.cpu().numpy())

    step_roofline = {"bound": "hbm", "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(step_gbs / HBM_PEAK_GBS, 4),
                     "bytes_per_step": step_bytes, "us_per_step": round(ms_per_step * 1e3, 3),
                     "us_at_60pct_of_peak": round(step_bytes / (0.6 * HBM_PEAK_GBS * 1e3), 3)}
    line = {
        "metric": "decode queries/s (all heads) at 128K ctx",
        "value": round(value, 1), "unit": "queries/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 K/V, f32 accumulate",
        "data": "synthetic (seeded; Llama-3.1-8B shape, planted-key queries)",
        "config": {"workload": args.workload, "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv,
                   "ctx": int(seq_np.max()), "max_ctx": Lcap, "page_size": 16, "code_bits": 128,
                   "keep": f"{keep[0]}/{keep[1]}" if keep[2] == 0 else keep[2], "top_k": top_k,
                   "meta_dtype": args.meta,
                   "layers_rotated": args.layers, "hip_graph": bool(graph is not None),
                   "entry": {"decode": "hhr_decode", "staged": "hhr_select+hhr_sparse_decode",
                             "append": "hhr_decode_append",
                             "append_then_decode": "hhr_append_keys+hhr_decode"}[args.path]},
        "roofline": roofline,
        "step_roofline": step_roofline,
        "cpu_baseline": cpu,
        "step_time_distribution": dist,
        "kernels": {"k_score_topp": {k: roofline[k] for k in ("bytes_per_launch",
                                                            "avg_launch_us")},
                    "k_page_scores": scorer_only},
        "step_algorithmic_bytes": step_bytes,
        "step_hbm_gbs": round(step_gbs, 1),
        "step_frac_of_hbm_peak": round(step_gbs / HBM_PEAK_GBS, 4),
        "recall_topk_vs_exact": {"per_kv_head": [round(r, 4) for r in recalls],
                                 "mean": round(float(np.mean(recalls)), 4)},
        "planted_hit_rate": {"per_kv_head": [round(float(x), 3) for x in planted_hits],
                             "mean": round(float(np.mean(planted_hits)), 4)},
        "oracle_agreement": agreement,
        "encoder_prefill": enc,
        "wall_s_timed": round(wall, 3),
        "input_gen_s": round(t_gen, 1),
    }
    print(json.dumps(line), flush=True)


def main_hisa(args, torch, hhr, synth, dev):
    from hash_hierarchical_top_amd import quality

    """HISA decode step: hhr_hisa_select (block scores, top blocks, fp8 token scores,
    token top-k) then hhr_sparse_decode with the attention heads on one KV head."""
    w = synth.HISA_WORKLOADS[args.workload]
    t_gen = time.time()
    inp = synth.make_hisa_workload_inputs(args.workload)
    t_gen = time.time() - t_gen
    L, Hi, Ha, blk = w.ctx, w.n_index_heads, w.n_attn_heads, w.block
    hs = hhr.make_hisa_shape(1, Hi, blk, L)
    ashape = hhr.make_shape(1, Ha, 1, L, "bf16")
    scale = 1.0 / math.sqrt(128.0)

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    q8, q_scale, wt = t(inp["q8"][None]), t(inp["q_scale"][None]), t(inp["w"][None])
    qa = t(inp["q_attn"][None])
    seq = t(inp["seq_len"])
    zero = torch.zeros(1, dtype=torch.int32, device=dev)
    k80, ks0 = t(inp["k8"][None]), t(inp["k_scale"][None])
    K0, V0 = t(inp["K"]).view(torch.bfloat16), t(inp["V"]).view(torch.bfloat16)
    layers = []
    for i in range(args.layers):
        lay = dict(k8=k80 if i == 0 else k80.clone(), ks=ks0 if i == 0 else ks0.clone(),
                   K=K0 if i == 0 else K0.clone(), V=V0 if i == 0 else V0.clone(),
                   reps=torch.zeros((1, L // blk, 128), dtype=torch.float32, device=dev))
        layers.append(lay)
    ws_h = torch.zeros(hhr.hhr_hisa_workspace_size(hs, w.keep_blocks, w.top_k), dtype=torch.uint8,
                       device=dev)
    ws_a = torch.zeros(hhr.hhr_workspace_size(ashape, 0, 1, 1, w.top_k), dtype=torch.uint8,
                       device=dev)  # attention only: the keep count does not matter
    sel = torch.zeros((1, 1, w.top_k), dtype=torch.int32, device=dev)
    cnt = torch.zeros((1, 1), dtype=torch.int32, device=dev)
    out = torch.zeros((1, Ha, 128), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    # ---- prefill-time pooling (H1), timed per layer
    pe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    pool_ms = []
    for lay in layers:
        pe[0].record(stream)
        hhr.hhr_hisa_pool_keys(hs, lay["k8"], lay["ks"], zero, seq, L, lay["reps"], ws_h)
        pe[1].record(stream)
        torch.cuda.synchronize()
        pool_ms.append(pe[0].elapsed_time(pe[1]))

    if args.copy_probe_mib:  # a plain copy of known size, to calibrate HBM byte counters
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    def step(i):
        lay = layers[i % args.layers]
        hhr.hhr_hisa_select(hs, q8, q_scale, wt, lay["k8"], lay["ks"], lay["reps"], seq,
                            w.keep_blocks, w.top_k, sel.view(1, w.top_k), cnt.view(1), ws_h)
        hhr.hhr_sparse_decode(ashape, qa, lay["K"], lay["V"], sel, cnt, w.top_k, scale, out, ws_a)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    graph = None
    if args.graph:
        gs = torch.cuda.Stream()
        gs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(gs):
            for i in range(args.layers):
                step(i)
        torch.cuda.current_stream().wait_stream(gs)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.layers):
                step(i)
        torch.cuda.synchronize()
        for _ in range(max(1, args.warmup // args.layers)):
            graph.replay()
        torch.cuda.synchronize()
    n_rep, rem = divmod(args.steps, args.layers)
    steps = args.steps
    graph_rem = None
    if graph is not None and rem:
        graph_rem = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph_rem):
            for i in range(rem):
                step(i)
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record()
    if graph is not None:
        for _ in range(n_rep):
            graph.replay()
        if graph_rem is not None:
            graph_rem.replay()
    else:
        for i in range(steps):
            step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = e0.elapsed_time(e1) / steps
    assert hhr.hhr_read_device_status(ws_h) == 0 and hhr.hhr_read_device_status(ws_a) == 0

    # algorithmic bytes per step: pooled reps, kept fp8 keys + scales, K/V rows, q and o
    n_sel = int(cnt.item())
    step_bytes = ((L // blk) * 128 * 4 + w.keep_blocks * blk * (128 + 4) + n_sel * 2 * 128 * 2
                  + Hi * (128 + 8) + Ha * 128 * 4 * 2)
    # dominant kernel by bytes: the fp8 token scorer with the token top-k in its last
    # workgroup (hhr_hisa_token_topk, one launch at one row), timed back to back on its
    # stream over the rotating layers
    kept = torch.zeros((1, w.keep_blocks), dtype=torch.int32, device=dev)
    kc = torch.zeros((1,), dtype=torch.int32, device=dev)
    bs = torch.zeros((1, L // blk), dtype=torch.float32, device=dev)
    hhr.hhr_hisa_block_scores(hs, q8, q_scale, wt, layers[0]["reps"], seq, bs, ws_h)
    hhr.hhr_hisa_top_blocks(hs, bs, seq, w.keep_blocks, kept, kc, ws_h)
    nk = min(args.steps, 400)
    ke0, ke1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ke0.record(stream)
    for i in range(nk):
        lay = layers[i % args.layers]
        hhr.hhr_hisa_token_topk(hs, q8, q_scale, wt, lay["k8"], lay["ks"], seq, kept, kc,
                                w.keep_blocks, w.top_k, sel.view(1, w.top_k), cnt.view(1), None,
                                ws_h)
    ke1.record(stream)
    torch.cuda.synchronize()
    k_ms = ke0.elapsed_time(ke1) / nk
    k_bytes = w.keep_blocks * blk * (128 + 4) + Hi * (128 + 8) + w.keep_blocks * 4 + w.top_k * 4
    roofline = {"bound": "hbm", "achieved": round(k_bytes / (k_ms * 1e6), 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(k_bytes / (k_ms * 1e6) / HBM_PEAK_GBS, 5),
                "traffic": measured_traffic(args.workload, "k_hisa_token_scores<16, true>"),
                "kernel": "k_hisa_token_scores<16, true> (hhr_hisa_token_topk)",
                "bytes_per_launch": k_bytes, "avg_launch_us": round(k_ms * 1e3, 3),
                "note": "latency-bound: ~1 MB per launch"}

    # ---- selection quality, then the CPU baseline (oracle select + attention, 1 thread)
    sel_h = sel.cpu().numpy()[0, 0, :n_sel]
    flat = quality.flat_indexer_topk(inp["q8"], inp["q_scale"], inp["w"], inp["k8"],
                                     inp["k_scale"], L, w.top_k, dev)
    iou_flat = quality.iou(sel_h, flat)
    # the same on the planted-block variant: 16 blocks whose keys lean towards the index
    # queries' mean direction, i.e. data with block structure for the coarse stage to find
    pin = synth.make_hisa_workload_inputs(args.workload, planted_blocks=16, make_kv=False)
    pk8, pks = t(pin["k8"][None]), t(pin["k_scale"][None])
    preps = torch.zeros((1, L // blk, 128), dtype=torch.float32, device=dev)
    hhr.hhr_hisa_pool_keys(hs, pk8, pks, zero, seq, L, preps, ws_h)
    hhr.hhr_hisa_select(hs, t(pin["q8"][None]), t(pin["q_scale"][None]), t(pin["w"][None]), pk8,
                        pks, preps, seq, w.keep_blocks, w.top_k, sel.view(1, w.top_k),
                        cnt.view(1), ws_h)
    torch.cuda.synchronize()
    iou_planted = quality.iou(sel.cpu().numpy()[0, 0, :int(cnt.item())],
                              quality.flat_indexer_topk(pin["q8"], pin["q_scale"], pin["w"],
                                                        pin["k8"], pin["k_scale"], L, w.top_k,
                                                        dev))
    cpu = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits

        from oracle import hhr as OH
        from oracle import hisa as OS

        Kf = synth.bf16_bits_to_f32(inp["K"][0, 0])
        Vf = synth.bf16_bits_to_f32(inp["V"][0, 0])

        def oracle_step():
            r = OS.select(inp["q8"], inp["q_scale"], inp["w"], inp["k8"], inp["k_scale"], L,
                          blk, w.keep_blocks, w.top_k)
            OH.attend(inp["q_attn"], Kf[r["sel"]], Vf[r["sel"]], scale)

        nt = _host_threads()
        with threadpool_limits(limits=nt):
            n, el = _timed_loop(oracle_step, args.cpu_seconds)
        with threadpool_limits(limits=1):
            n1, el1 = _timed_loop(oracle_step, args.cpu_seconds * 0.5)
        cpu = {"value": round(n / el, 3), "unit": "queries/s", "cores": nt, "kind": "oracle",
               "sample": f"{n} whole HISA decode steps of {w.name} (pooling included, "
                         f"attention on {Ha} heads), {el:.1f} s, numpy fp64, BLAS {nt} threads",
               "host_cpus": os.cpu_count(), "host_cpus_usable": nt,
               "single_thread": {"value": round(n1 / el1, 3), "unit": "queries/s", "cores": 1,
                                 "sample": f"{n1} steps, {el1:.1f} s"}}
    line = {
        "metric": "HISA decode queries/s (64 fp8 index heads + 16 attention heads) at 128K ctx",
        "value": round(steps / (ms_per_step * steps / 1e3), 1), "unit": "queries/s",
        "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8 e4m3 index, bf16 K/V, f32 accumulate",
        "data": "synthetic (seeded; N(0,1) index queries and keys quantised to e4m3)",
        "config": {"workload": w.name, "ctx": L, "index_heads": Hi, "block": blk,
                   "keep_blocks": w.keep_blocks, "top_k": w.top_k, "attn_heads": Ha,
                   "layers_rotated": args.layers, "hip_graph": bool(graph is not None),
                   "entry": "hhr_hisa_select+hhr_sparse_decode"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "step_algorithmic_bytes": step_bytes,
        "step_hbm_gbs": round(step_bytes / (ms_per_step * 1e6), 1),
        "iou_vs_flat_indexer": round(float(iou_flat), 4),
        "iou_vs_flat_indexer_planted_blocks": round(float(iou_planted), 4),
        "pool_prefill_ms": round(float(np.median(pool_ms[1:] if len(pool_ms) > 1 else pool_ms)), 4),
        "wall_s_timed": round(wall, 3),
        "input_gen_s": round(t_gen, 1),
    }
    print(json.dumps(line), flush=True)


def main_hisa_prefill(args, torch, hhr, synth, dev):
    """HISA prefill indexer: M query rows spread over a 128K prompt against one shared fp8
    index-key cache (hhr_hisa_prefill_select), plus hierarchical against flat (every block
    kept) at 16K, the largest context whose flat candidate set fits one token top-k."""
    base, M = synth.HISA_PREFILL_WORKLOADS[args.workload]
    w = synth.HISA_WORKLOADS[base]
    Hi, blk, L = w.n_index_heads, w.block, w.ctx
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    src = synth.make_hisa_workload_inputs(base, make_kv=False)
    k8, ks = t(src["k8"]), t(src["k_scale"])

    def pool(Lc):
        shape1 = hhr.make_hisa_shape(1, Hi, blk, Lc)
        reps = torch.zeros((1, Lc // blk, 128), dtype=torch.float32, device=dev)
        ws1 = torch.zeros(hhr.hhr_hisa_workspace_size(shape1, 1, 1), dtype=torch.uint8,
                          device=dev)
        hhr.hhr_hisa_pool_keys(shape1, k8[None, :Lc].contiguous(), ks[None, :Lc].contiguous(),
                               torch.zeros(1, dtype=torch.int32, device=dev),
                               t(np.array([Lc], np.int32)), Lc, reps, ws1[:4].view(torch.int32))
        return reps

    def timed(Lc, keep, rows, reps):
        shape = hhr.make_hisa_shape(M, Hi, blk, Lc)
        ws = torch.zeros(hhr.hhr_hisa_workspace_size(shape, keep, w.top_k), dtype=torch.uint8,
                         device=dev)
        sel = torch.zeros((M, w.top_k), dtype=torch.int32, device=dev)
        cnt = torch.zeros((M,), dtype=torch.int32, device=dev)
        args_ = (shape, t(rows["q8"]), t(rows["q_scale"]), t(rows["w"]), k8[:Lc].contiguous(),
                 ks[:Lc].contiguous(), reps, t(rows["q_len"]), keep, w.top_k, sel, cnt, ws)
        for _ in range(max(2, min(args.warmup, 10))):
            hhr.hhr_hisa_prefill_select(*args_)
        torch.cuda.synchronize()
        assert hhr.hhr_read_device_status(ws) == 0
        n = args.steps
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            hhr.hhr_hisa_prefill_select(*args_)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, sel, cnt

    rows = synth.make_hisa_prefill_rows(args.workload)
    reps = pool(L)
    ms, sel, cnt = timed(L, w.keep_blocks, rows, reps)
    # hierarchical against flat at 16K (same rows' queries, positions over 16K)
    L16 = 16384
    rows16 = synth.make_hisa_prefill_rows(args.workload, ctx=L16)
    reps16 = pool(L16)
    ms_flat, sel_f, cnt_f = timed(L16, L16 // blk, rows16, reps16)
    ms_hier, sel_h, cnt_h = timed(L16, 16, rows16, reps16)
    sf, ch, sh = sel_f.cpu().numpy(), cnt_f.cpu().numpy(), sel_h.cpu().numpy()
    from hash_hierarchical_top_amd import quality

    iou16 = float(np.mean([quality.iou(sh[r, :cnt_h[r].item()], sf[r, :ch[r]])
                           for r in range(M)]))
    q_len = rows["q_len"].astype(np.int64)
    # flops: block scores (f32) over each row's blocks, fp8 token scores over kept tokens
    nb = -(-q_len // blk)
    flops = float((nb * Hi * 128 * 2).sum() + (np.minimum(nb, w.keep_blocks) * blk * Hi * 128 * 2)
                  .sum())
    # the call is dominated by its fp8 token scorer (a contraction on MFMA): its roofline is
    # the call's indexer flops against the fp8 dense MFMA peak, timed with one event pair
    # around back-to-back calls on the stream (per-kernel durations: the committed trace)
    roofline = {"bound": "mfma", "achieved": round(flops / (ms * 1e9), 2),
                "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(flops / (ms * 1e9) / MFMA_FP8_PEAK_TFLOPS, 5), "traffic": None,
                "kernel": "hhr_hisa_prefill_select (k_hisa_pool_tail, k_hisa_block_scores, "
                          "k_hisa_top_blocks, k_hisa_token_scores, k_hisa_topk)",
                "flops_per_launch": flops, "avg_launch_us": round(ms * 1e3, 3),
                "note": "each row re-reads its 64 kept blocks (1 MiB of fp8 keys), mostly from "
                        "L2 and the last-level cache: bound by on-chip cache work and latency, "
                        "not HBM"}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_prefill(rows, src, w, L, args.cpu_seconds)
    line = {
        "metric": "HISA prefill indexer query rows/s at 128K ctx",
        "value": round(M / (ms / 1e3), 1), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": max(2, min(args.warmup, 10)), "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8 e4m3 index, f32 block scores",
        "data": "synthetic (seeded; N(0,1) index queries and keys quantised to e4m3)",
        "config": {"workload": args.workload, "ctx": L, "rows": M, "index_heads": Hi,
                   "block": blk, "keep_blocks": w.keep_blocks, "top_k": w.top_k,
                   "row_positions": "drawn uniformly over the context (seeded)",
                   "entry": "hhr_hisa_prefill_select"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "indexer_tflops": round(flops / (ms * 1e9), 2),
        "flat_vs_hierarchical_16k": {
            "ctx": L16, "flat_ms": round(ms_flat, 4), "hierarchical_ms": round(ms_hier, 4),
            "speedup": round(ms_flat / ms_hier, 2), "keep_blocks": 16,
            "mean_iou_with_flat": round(iou16, 4)},
    }
    print(json.dumps(line), flush=True)


def cpu_baseline_prefill(rows, src, w, L, budget_s):
    """The oracle's causal prefill selection of query rows (cycling over the chunk's rows)
    against the same shared 131072-key cache, on the host's cores (one worker thread per
    row, BLAS 1 thread each) and on one thread, for a bounded time; rows/s."""
    import concurrent.futures

    from threadpoolctl import threadpool_limits

    from oracle import hisa as OS

    def row(r):
        OS.prefill_select(rows["q8"][r], rows["q_scale"][r], rows["w"][r], src["k8"],
                          src["k_scale"], L, int(rows["q_len"][r]), w.block, w.keep_blocks,
                          w.top_k)

    M = rows["q_len"].size
    nt = _host_threads()
    cursor = [0]

    def batch():
        rs = [(cursor[0] + i) % M for i in range(nt)]
        cursor[0] += nt
        list(ex.map(row, rs))

    with threadpool_limits(limits=1):
        with concurrent.futures.ThreadPoolExecutor(max_workers=nt) as ex:
            n, el = _timed_loop(batch, budget_s)
        n1, el1 = _timed_loop(lambda: row(0), budget_s * 0.5)
    return {"value": round(n * nt / el, 3), "unit": "rows/s", "cores": nt, "kind": "oracle",
            "sample": f"{n * nt} prefill rows (oracle.hisa.prefill_select, {nt} at once, "
                      f"cycling over the chunk's {M} rows) on the 131072-key cache, {el:.1f} s, "
                      f"numpy fp64, BLAS 1 thread each",
            "host_cpus": os.cpu_count(), "host_cpus_usable": nt,
            "single_thread": {"value": round(n1 / el1, 3), "unit": "rows/s", "cores": 1,
                              "sample": f"{n1} rows, {el1:.1f} s"}}


def _host_threads() -> int:
    """The CPUs this process may run on (the box's share), capped at 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _timed_loop(fn, budget_s):
    """Calls fn() until budget_s seconds have passed; returns (calls, seconds)."""
    n = 0
    t0 = time.perf_counter()
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            return n, el


def cpu_baseline(inp, w, seq_np, keep, top_k, scale, budget_s, gpu_sel=None, gpu_cnt=None,
                 gpu_codes=None, gpu_kept=None):
    """The oracle's decode step (query encode .. attention, all KV heads of the first
    sequence) on the host, keys pre-encoded (prefill, untimed), repeated for budget_s
    seconds: once with the KV heads run concurrently on the host's cores (one worker thread
    per head, at most the CPUs this process may use, BLAS one thread each), once on one
    thread.  Returns (baseline, agreement): agreement compares the oracle's selection
    from raw inputs with the GPU's (gpu_sel / gpu_cnt [B][Hkv][top_k], gpu_codes [B][Hkv]
    [Lcap][4]): per KV head the IoU of the two selections, the key code bits that differ
    (each inside the rounding band |y| <= 1e-4 sum|k W| or not), and the kept pages that
    differ (inside the band |s - s_P| <= 1e-4 |s_P| of the P-th bound, or not)."""
    import concurrent.futures

    from threadpoolctl import threadpool_limits

    from hash_hierarchical_top_amd import synth
    from oracle import hhr as O

    G = w.n_q_heads // w.n_kv_heads
    b = 0
    L = int(seq_np[b])
    heads = []
    for g in range(w.n_kv_heads):
        K = synth.kv_values(inp["K"][b, g, :L], w.kv_dtype)
        V = synth.kv_values(inp["V"][b, g, :L], w.kv_dtype)
        enc = O.encode_keys(K, inp["R"][g], inp["W"][g], 16)  # prefill: not timed
        heads.append((K, V, enc, inp["q"][b, g * G:(g + 1) * G], inp["R"][g], inp["W"][g]))
    P = O.keep_count(O.n_pages(L, 16), *keep)

    def head_step(h):
        K, V, enc, qg, R, W = h
        qe = O.encode_query(qg, R, W)
        s = O.page_scores(qe["qrot"], enc["meta"])
        kept = O.top_pages(s, P)
        cand = O.candidates(kept, L, 16)
        H = O.hamming(qe["qcodes"], enc["codes"][cand])
        sel = O.topk_smallest(H, cand, top_k)
        O.attend(qg, K[sel], V[sel], scale)
        return s, kept, sel, qe

    n_workers = min(_host_threads(), len(heads))
    with threadpool_limits(limits=1):
        with concurrent.futures.ThreadPoolExecutor(max_workers=n_workers) as ex:
            n_all, el_all = _timed_loop(lambda: list(ex.map(head_step, heads)), budget_s)
        n_one, el_one = _timed_loop(lambda: [head_step(h) for h in heads], budget_s * 0.5)
    baseline = {
        "value": round(n_all / el_all, 3), "unit": "queries/s", "cores": n_workers,
        "kind": "oracle",
        "sample": f"{n_all} whole decode steps of {w.name} (all {w.n_kv_heads} KV heads of one "
                  f"sequence, keys pre-encoded), {el_all:.1f} s, numpy fp64, one worker thread "
                  f"per KV head ({n_workers} at once), BLAS 1 thread each",
        "host_cpus": os.cpu_count(), "host_cpus_usable": _host_threads(),
        "single_thread": {"value": round(n_one / el_one, 3), "unit": "queries/s", "cores": 1,
                          "sample": f"{n_one} steps, {el_one:.1f} s"}}
    agreement = None
    if gpu_sel is not None:
        per = []
        for g, (K, V, enc, qg, R, W) in enumerate(heads):
            s, kept, sel, qe = head_step(heads[g])
            n = int(gpu_cnt[b, g])
            gs = gpu_sel[b, g, :n]
            union = np.union1d(gs, sel).size
            iou = 1.0 if union == 0 else np.intersect1d(gs, sel).size / union
            Y = K @ np.asarray(W, np.float64)
            band = 1e-4 * (np.abs(K) @ np.abs(np.asarray(W, np.float64)))
            mism = O.unpack_bits(gpu_codes[b, g, :L]) != (Y >= 0)
            rec = {"kv_head": g, "iou_vs_oracle_from_raw_inputs": round(float(iou), 4),
                   "code_bits_differing": int(mism.sum()),
                   "code_bits_outside_band": int((mism & ~(np.abs(Y) <= band)).sum())}
            if gpu_kept is not None:
                dk = np.setxor1d(gpu_kept[b, g, :P], kept)
                sP = np.sort(s)[::-1][P - 1]
                rec["pages_differing"] = int(dk.size)
                rec["pages_outside_band"] = int((np.abs(s[dk] - sP) > 1e-4 * abs(sP)).sum())
            per.append(rec)
        agreement = {"per_kv_head": per,
                     "mean_iou": round(float(np.mean([r["iou_vs_oracle_from_raw_inputs"]
                                                      for r in per])), 4),
                     "code_bits_differing": int(sum(r["code_bits_differing"] for r in per)),
                     "code_bits_outside_band": int(sum(r["code_bits_outside_band"] for r in per)),
                     "note": "the oracle selects from raw inputs in fp64; the GPU in fp32: a "
                             "code bit or kept page may differ only inside its 1e-4 band"}
        if gpu_kept is not None:
            agreement["pages_differing"] = int(sum(r["pages_differing"] for r in per))
            agreement["pages_outside_band"] = int(sum(r["pages_outside_band"] for r in per))
    return baseline, agreement


if __name__ == "__main__":
    main()
