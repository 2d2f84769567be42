"""Recall sweeps on synthetic data, run through hhr_decode on the GPU.

    python -m hash_hierarchical_top_amd.sweep [--workload llama8b_32k] [--steps 40]

For each candidate ratio r (keys attended / context, the axis of HHR appendix Figure 9)
three selections with the same attention budget k = r L are compared, as in the
stage-wise ablation of HHR appendix Table 8:

  - HHR: the coarse stage keeps `coarse` x r of the pages (GKR page bounds), the fine
    stage takes the k keys with the smallest summed Hamming distance among them (LHP);
  - GKR-only: keep r of the pages and attend every key in them (top_k = 16 P);
  - LHP-only: keep every page and take the k smallest Hamming distances over all keys.

Each line reports the mean recall of the exact top-k (per KV head, by summed group
logit), the planted-key hit rate and the step time (HIP graph of one step per rotated
layer copy).  With untrained random R and W these numbers describe the synthetic data
and the mechanism, not the pages' accuracy results.  LHP-only keeps every page, so the
context is limited to 32768 / 16 = 2048 pages (32K keys).
"""
from __future__ import annotations

import argparse
import json
import math

import numpy as np


def _variants(Np: int, L: int, r: float, coarse: int):
    k = max(1, int(round(r * L)))
    P_hhr = min(Np, max(1, int(math.ceil(coarse * r * Np))))
    P_gkr = min(Np, max(1, int(math.ceil(r * Np))))
    return [
        ("HHR", (0, 1, P_hhr), k),
        ("GKR-only", (0, 1, P_gkr), P_gkr * 16),
        ("LHP-only", (1, 1, 0), k),
    ]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="llama8b_32k")
    ap.add_argument("--ratios", default="0.015625,0.03125,0.0625,0.125")
    ap.add_argument("--coarse", type=int, default=4, help="HHR keeps coarse x r of the pages")
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--steps", type=int, default=40)
    args = ap.parse_args()

    import torch

    from hash_hierarchical_top_amd import hhr, quality, synth

    assert torch.cuda.is_available(), "the sweep runs on a GPU"
    dev = torch.device("cuda", 0)
    w = synth.WORKLOADS[args.workload]
    B, Hq, Hkv, Lcap = w.batch, w.n_q_heads, w.n_kv_heads, w.max_ctx
    G = Hq // Hkv
    inp = synth.make_workload_inputs(args.workload)
    seq_np = inp["seq_len"]
    assert B == 1, "one sequence per sweep point"
    L = int(seq_np[0])
    Np = -(-L // 16)
    shape = hhr.make_shape(B, Hq, Hkv, Lcap, w.kv_dtype)

    def kv(a):
        t = torch.from_numpy(a)
        return (t.view(torch.bfloat16) if w.kv_dtype == "bf16" else t).to(dev)

    seq = torch.from_numpy(seq_np).to(dev)
    q = torch.from_numpy(inp["q"]).to(dev)
    K0, V0 = kv(inp["K"]), kv(inp["V"])
    R0, W0 = torch.from_numpy(inp["R"]).to(dev), torch.from_numpy(inp["W"]).to(dev)
    layers = []
    zero = torch.zeros(B, dtype=torch.int32, device=dev)
    ws0 = torch.zeros(hhr.hhr_workspace_size(shape, 1, 1, 0, 1), dtype=torch.uint8, device=dev)
    for i in range(args.layers):
        lay = dict(K=K0 if i == 0 else K0.clone(), V=V0 if i == 0 else V0.clone(),
                   R=R0, W=W0,
                   codes=torch.zeros((B, Hkv, Lcap, 4), dtype=torch.int32, device=dev),
                   meta=torch.zeros(hhr.meta_shape(shape), dtype=torch.float32, device=dev))
        hhr.hhr_append_keys(shape, lay["K"], zero, seq, L, lay["R"], lay["W"], lay["codes"],
                            lay["meta"], ws0)
        layers.append(lay)
    torch.cuda.synchronize()
    # exact top-k per KV head for every budget, from layer 0's keys (all copies are equal)
    ks = sorted({max(1, int(round(float(r) * L))) for r in args.ratios.split(",")})
    exact = {k: [quality.exact_topk(q[0, g * G:(g + 1) * G], K0[0, g, :L], k).cpu().numpy()
                 for g in range(Hkv)] for k in ks}
    scale = 1.0 / math.sqrt(128.0)
    rows = []
    for r in map(float, args.ratios.split(",")):
        budget = max(1, int(round(r * L)))
        for name, keep, top_k in _variants(Np, L, r, args.coarse):
            ws = torch.zeros(hhr.hhr_workspace_size(shape, *keep, top_k), dtype=torch.uint8,
                             device=dev)
            sel = torch.zeros((B, Hkv, top_k), dtype=torch.int32, device=dev)
            cnt = torch.zeros((B, Hkv), dtype=torch.int32, device=dev)
            out = torch.zeros((B, Hq, 128), dtype=torch.float32, device=dev)

            def step(i):
                lay = layers[i % len(layers)]
                hhr.hhr_decode(shape, q, seq, lay["R"], lay["W"], lay["codes"], lay["meta"],
                               lay["K"], lay["V"], *keep, top_k, scale, sel, cnt, out, ws)

            for i in range(len(layers)):
                step(i)
            torch.cuda.synchronize()
            assert hhr.hhr_read_device_status(ws) == 0
            s_h, c_h = sel.cpu().numpy(), cnt.cpu().numpy()
            rec = float(np.mean([quality.overlap(s_h[0, g, :c_h[0, g]], exact[budget][g])
                                 for g in range(Hkv)]))
            hit = float(np.mean([np.isin(inp["planted"][0, g], s_h[0, g, :c_h[0, g]]).mean()
                                 for g in range(Hkv)]))
            gs = torch.cuda.Stream()
            gs.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(gs):
                for i in range(len(layers)):
                    step(i)
            torch.cuda.current_stream().wait_stream(gs)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(len(layers)):
                    step(i)
            graph.replay()
            torch.cuda.synchronize()
            reps = max(1, args.steps // len(layers))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (reps * len(layers))
            row = {"workload": args.workload, "candidate_ratio": r, "variant": name,
                   "kept_pages": keep[2] if keep[2] else Np, "top_k": top_k,
                   "attended_keys": int(c_h[0].mean()),
                   "recall_vs_exact_topk": round(rec, 4), "planted_hit_rate": round(hit, 4),
                   "us_per_step": round(us, 2)}
            rows.append(row)
            print(json.dumps(row), flush=True)
            del graph
    print("\n| ratio | variant | kept pages | attended keys | recall | planted hits | us/step |")
    print("|---|---|---|---|---|---|---|")
    for x in rows:
        print(f"| {x['candidate_ratio']:.4g} | {x['variant']} | {x['kept_pages']} | "
              f"{x['attended_keys']} | {x['recall_vs_exact_topk']:.3f} | "
              f"{x['planted_hit_rate']:.3f} | {x['us_per_step']:.1f} |")


if __name__ == "__main__":
    main()
