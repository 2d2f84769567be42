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

Prints one JSON line.  `roofline` is for the page-bound scorer, the kernel
that moves most of the step's bytes; its duration is measured with HIP events
around each launch on the stream it runs on, in a pass of its own over the
same rotating layers.  `cpu_baseline` times the CPU oracle (numpy, 1 thread)
on whole decode steps of the same workload for a bounded number of seconds.
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
    ap.add_argument("--path", choices=("decode", "staged"), default="decode",
                    help="decode: one hhr_decode call per step; staged: hhr_select then "
                         "hhr_sparse_decode")
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

    from hash_hierarchical_top_amd import hhr, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    hhr.load()
    dev = torch.device("cuda", 0)
    w = synth.WORKLOADS[args.workload]
    B, Hq, Hkv, Lcap, top_k = w.batch, w.n_q_heads, w.n_kv_heads, w.max_ctx, w.top_k
    keep = (w.keep_num, w.keep_den, w.keep_pages_abs)
    G = Hq // Hkv
    t_gen = time.time()
    inp = synth.make_workload_inputs(args.workload)
    t_gen = time.time() - t_gen
    seq_np = inp["seq_len"]
    shape = hhr.make_shape(B, Hq, Hkv, Lcap, w.kv_dtype)
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
                   meta=torch.zeros((B, Hkv, NpCap, 128, 2), dtype=torch.float32, device=dev))
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
        -(-int(L) // 16) for L in seq_np) * Hkv * 1024 + Hkv * 2 * 128 * 128 * 4
    enc_flops = 2.0 * n_keys * 128 * 256
    passes = 2 if w.kv_dtype == "bf16" else 3
    enc = {"ms": round(enc_ms, 4), "hbm_gbs": round(enc_bytes / enc_ms / 1e6, 1),
           "tflops": round(enc_flops / enc_ms / 1e9, 2),
           "mfma_bf16_tflops_issued": round(passes * enc_flops / enc_ms / 1e9, 2),
           "mfma_util_vs_bf16_peak": round(passes * enc_flops / enc_ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4),
           "bytes": enc_bytes, "flops": enc_flops}

    def step(i):
        lay = layers[i % args.layers]
        if args.path == "decode":
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

    graph = None
    if args.graph:
        # one graph holding one step per layer; the library enqueues only kernels
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

    # ---- timed region
    n_rep = -(-args.steps // args.layers) if graph is not None else 0
    steps = n_rep * args.layers if graph is not None else args.steps
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    if graph is not None:
        for _ in range(n_rep):
            graph.replay()
    else:
        for i in range(steps):
            step(i)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / steps
    value = B * steps / (total_ms / 1e3)
    assert hhr.hhr_read_device_status(ws) == 0

    # ---- algorithmic bytes per step
    Np = np.array([-(-int(L) // 16) for L in seq_np])
    P = np.array([hhr.hhr_keep_count(int(n), *keep) for n in Np])
    cand = int(P.sum()) * 16 * Hkv
    meta_bytes = int(Np.sum()) * Hkv * 1024
    sel_rows = int(cnt.sum().item())
    step_bytes = (meta_bytes + cand * 16 + sel_rows * 2 * 128 * kv_bytes
                  + Hkv * 2 * 128 * 128 * 4 + B * Hq * 128 * 4 * 2)
    step_gbs = step_bytes / (ms_per_step * 1e6)

    # ---- dominant kernel: page-bound scorer, per-launch HIP events on its stream
    q_rot = torch.zeros((B, Hq, 128), dtype=torch.float32, device=dev)
    q_codes = torch.zeros((B, Hq, 4), dtype=torch.int32, device=dev)
    scores = torch.zeros((B, Hkv, NpCap), dtype=torch.float32, device=dev)
    hhr.hhr_encode_queries(shape, q, R0, W0, q_rot, q_codes)
    nk = min(args.steps, 400)
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(nk)]
    for i in range(args.layers):
        hhr.hhr_page_scores(shape, q_rot, seq, layers[i]["meta"], scores, ws)
    torch.cuda.synchronize()
    for i in range(nk):
        lay = layers[i % args.layers]
        kev[i][0].record(stream)
        hhr.hhr_page_scores(shape, q_rot, seq, lay["meta"], scores, ws)
        kev[i][1].record(stream)
    torch.cuda.synchronize()
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in kev]))
    k_bytes = meta_bytes + B * Hq * 128 * 4 + int(Np.sum()) * Hkv * 4
    roofline = {"bound": "hbm", "achieved": round(k_bytes / (k_ms * 1e6), 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(k_bytes / (k_ms * 1e6) / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "k_page_scores", "bytes_per_launch": k_bytes,
                "avg_launch_us": round(k_ms * 1e3, 3)}

    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    # ---- top-k recall against exact q.k top-k (per KV head, as in HHR Figure 4) on 2 heads
    from oracle import hhr as O

    sel_h = sel.cpu().numpy()
    recalls, planted_hits = [], []
    for g in (0, Hkv - 1):
        L = int(seq_np[0])
        Kg = synth.kv_values(inp["K"][0, g, :L], w.kv_dtype)
        qg = inp["q"][0, g * G:(g + 1) * G]
        exact = O.exact_topk(qg, Kg, top_k)
        recalls.append(O.recall(sel_h[0, g, :int(cnt[0, g])], exact))
        planted_hits.append(np.isin(inp["planted"][0, g], sel_h[0, g]).mean())

    # ---- CPU baseline: the oracle's decode step (encoded keys prepared beforehand)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, w, seq_np, keep, top_k, scale, args.cpu_seconds)

    line = {
        "metric": "decode queries/s (all heads) at 128K ctx",
        "value": round(value, 1), "unit": "queries/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 K/V, f32 accumulate",
        "data": "synthetic (seeded; Llama-3.1-8B shape, planted-key queries)",
        "config": {"workload": args.workload, "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv,
                   "ctx": int(seq_np.max()), "page_size": 16, "code_bits": 128,
                   "keep": f"{keep[0]}/{keep[1]}" if keep[2] == 0 else keep[2], "top_k": top_k,
                   "layers_rotated": args.layers, "hip_graph": bool(graph is not None),
                   "entry": "hhr_decode" if args.path == "decode"
                   else "hhr_select+hhr_sparse_decode"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "step_algorithmic_bytes": step_bytes,
        "step_hbm_gbs": round(step_gbs, 1),
        "step_frac_of_hbm_peak": round(step_gbs / HBM_PEAK_GBS, 4),
        "recall_topk_vs_exact": [round(r, 4) for r in recalls],
        "planted_hit_rate": [round(float(x), 3) for x in planted_hits],
        "encoder_prefill": enc,
        "wall_s_timed": round(wall, 3),
        "input_gen_s": round(t_gen, 1),
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(inp, w, seq_np, keep, top_k, scale, budget_s):
    """Oracle decode steps (query encode .. attention, all KV heads of one sequence) on the
    host, single-threaded BLAS, repeated until the time budget is used."""
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
        heads.append((K, V, enc["codes"], enc["meta"], inp["q"][b, g * G:(g + 1) * G],
                      inp["R"][g], inp["W"][g]))
    P = O.keep_count(O.n_pages(L, 16), *keep)
    with threadpool_limits(limits=1):
        n = 0
        t0 = time.perf_counter()
        while True:
            for K, V, codes, meta, qg, R, W in heads:
                qe = O.encode_query(qg, R, W)
                s = O.page_scores(qe["qrot"], meta)
                kept = O.top_pages(s, P)
                cand = O.candidates(kept, L, 16)
                H = O.hamming(qe["qcodes"], codes[cand])
                sel = O.topk_smallest(H, cand, top_k)
                O.attend(qg, K[sel], V[sel], scale)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    return {"value": round(n / el, 3), "unit": "queries/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} whole decode steps of {w.name} (all {w.n_kv_heads} KV heads of one "
                      f"sequence, keys pre-encoded), {el:.1f} s, numpy fp64, BLAS 1 thread"}


if __name__ == "__main__":
    main()
