"""Reference selections for the quality figures that bench.py and sweep.py report
(recall against the exact top-k, IoU against the flat indexer).  These are reported,
never used to decide anything: plain definitions in torch fp64 on the GPU.

  - exact top-k of a KV head: the k positions with the largest summed group logit
    sum_h q_h . k_t over the group's query heads (HHR Figure 4 measures the recall of
    this set per KV head), ties to the lower position;
  - the flat indexer: s_t = sum_h w_h ReLU(q_h . k_t) over every valid token, on
    e4m3-decoded codes times their row scales (the DSA indexer that the HISA abstract
    makes hierarchical), top-k with ties to the lower position.
"""
from __future__ import annotations

import numpy as np
import torch


def exact_topk(q_group: torch.Tensor, K_valid: torch.Tensor, k: int) -> torch.Tensor:
    """Positions (ascending) of the k largest summed group logits."""
    logits = (K_valid.double() @ q_group.double().T).sum(dim=-1)
    order = torch.sort(-logits, stable=True).indices[:k]
    return torch.sort(order).values


def flat_indexer_topk(q8, q_scale, w, k8, k_scale, L: int, k: int, device) -> np.ndarray:
    """The flat indexer's exact top-k (ascending positions) over tokens [0, L)."""
    def deq(codes, scale):
        f = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(device)
        return f.double() * torch.from_numpy(np.ascontiguousarray(scale)).to(device).double()[:, None]

    q = deq(q8, q_scale)
    keys = deq(k8[:L], k_scale[:L])
    wt = torch.from_numpy(np.ascontiguousarray(w)).to(device).double()
    s = (torch.relu(keys @ q.T) * wt[None, :]).sum(dim=-1)
    order = torch.sort(-s, stable=True).indices[:k]
    return torch.sort(order).values.cpu().numpy()


def overlap(selected, exact) -> float:
    """|selected & exact| / |exact|."""
    exact = np.asarray(exact)
    return 1.0 if exact.size == 0 else np.intersect1d(np.asarray(selected), exact).size / exact.size


def iou(a, b) -> float:
    union = np.union1d(a, b).size
    return 1.0 if union == 0 else np.intersect1d(a, b).size / union
