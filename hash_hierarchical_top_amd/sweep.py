"""Recall sweeps on synthetic data, run through hhr_decode on the GPU.

    python -m hash_hierarchical_top_amd.sweep [--workload llama8b_32k] [--steps 40]
                                              [--code-bits 64,128,256]

For each candidate ratio r (keys attended / context, the axis of HHR appendix Figure 9)
three selections with the same attention budget k = r L are compared, as in the
stage-wise ablation of HHR appendix Table 8:

  - HHR: the coarse stage keeps `coarse` x r of the pages (GKR page bounds), the fine
    stage takes the k keys with the smallest summed Hamming distance among them (LHP);
  - GKR-only: keep r of the pages and attend every key in them (top_k = 16 P);
  - LHP-only: keep every page and take the k smallest Hamming distances over all keys.

With several --code-bits widths, every point is repeated per width (the axis of
HHR appendix Figure 10, the number of hash bits); GKR-only ignores the codes.
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
    ap.add_argument("--code-bits", default="128", help="comma-separated code widths")
    args = ap.parse_args()
    widths = [int(x) for x in args.code_bits.split(",")]

    import torch

    from hash_hierarchical_top_amd import hhr, quality, synth

    assert torch.cuda.is_available(), "the sweep runs on a GPU"
    dev = torch.device("cuda", 0)
    w = synth.WORKLOADS[args.workload]
    B, Hq, Hkv, Lcap = w.batch, w.n_q_heads, w.n_kv_heads, w.max_ctx
    G = Hq // Hkv
    inp = synth.make_workload_inputs(args.workload)
    seq_np = inp["seq_len"]
    # the workload's own 128-bit projection; other widths drawn from seeds of their own
    Ws = {bits: inp["W"] if bits == inp["W"].shape[-1] else
          np.random.Generator(np.random.PCG64(w.seed + bits)).standard_normal(
              (Hkv, 128, bits)).astype(np.float32) for bits in widths}
    assert B == 1, "one sequence per sweep point"
    L = int(seq_np[0])
    Np = -(-L // 16)

    def kv(a):
        t = torch.from_numpy(a)
        return (t.view(torch.bfloat16) if w.kv_dtype == "bf16" else t).to(dev)

    seq = torch.from_numpy(seq_np).to(dev)
    q = torch.from_numpy(inp["q"]).to(dev)
    K0, V0 = kv(inp["K"]), kv(inp["V"])
    R0 = torch.from_numpy(inp["R"]).to(dev)
    zero = torch.zeros(B, dtype=torch.int32, device=dev)
    Ks = [K0] + [K0.clone() for _ in range(args.layers - 1)]
    Vs = [V0] + [V0.clone() for _ in range(args.layers - 1)]

    def build_layers(bits):
        """Rotated layer copies with their codes and metadata at one code width."""
        shape = hhr.make_shape(B, Hq, Hkv, Lcap, w.kv_dtype, code_bits=bits)
        W0 = torch.from_numpy(Ws[bits]).to(dev)
        ws0 = torch.zeros(hhr.hhr_workspace_size(shape, 1, 1, 0, 1), dtype=torch.uint8,
                          device=dev)
        layers = []
        for i in range(args.layers):
            lay = dict(K=Ks[i], V=Vs[i], R=R0, W=W0,
                       codes=torch.zeros((B, Hkv, Lcap, bits // 32), dtype=torch.int32,
                                         device=dev),
                       meta=torch.zeros(hhr.meta_shape(shape), dtype=torch.float32,
                                        device=dev))
            hhr.hhr_append_keys(shape, lay["K"], zero, seq, L, lay["R"], lay["W"],
                                lay["codes"], lay["meta"], ws0)
            layers.append(lay)
        torch.cuda.synchronize()
        return shape, layers

    # exact top-k per KV head for every budget, from layer 0's keys (all copies are equal)
    ks = sorted({max(1, int(round(float(r) * L))) for r in args.ratios.split(",")})
    exact = {k: [quality.exact_topk(q[0, g * G:(g + 1) * G], K0[0, g, :L], k).cpu().numpy()
                 for g in range(Hkv)] for k in ks}
    scale = 1.0 / math.sqrt(128.0)
    rows = []
    points = []
    for bits in widths:
        shape, layers = build_layers(bits)
        for r in map(float, args.ratios.split(",")):
            for name, keep, top_k in _variants(Np, L, r, args.coarse):
                if name == "GKR-only" and bits != widths[0]:
                    continue  # no codes involved: once is enough
                points.append((bits, shape, layers, r, name, keep, top_k))
    for bits, shape, layers, r, name, keep, top_k in points:
        budget = max(1, int(round(r * L)))
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
        row = {"workload": args.workload, "code_bits": bits, "candidate_ratio": r,
               "variant": name,
               "kept_pages": keep[2] if keep[2] else Np, "top_k": top_k,
               "attended_keys": int(c_h[0].mean()),
               "recall_vs_exact_topk": round(rec, 4), "planted_hit_rate": round(hit, 4),
               "us_per_step": round(us, 2)}
        rows.append(row)
        print(json.dumps(row), flush=True)
        del graph
    print("\n| bits | ratio | variant | kept pages | attended keys | recall | planted hits "
          "| us/step |")
    print("|---|---|---|---|---|---|---|---|")
    for x in rows:
        print(f"| {x['code_bits']} | {x['candidate_ratio']:.4g} | {x['variant']} | "
              f"{x['kept_pages']} | "
              f"{x['attended_keys']} | {x['recall_vs_exact_topk']:.3f} | "
              f"{x['planted_hit_rate']:.3f} | {x['us_per_step']:.1f} |")


if __name__ == "__main__":
    main()
