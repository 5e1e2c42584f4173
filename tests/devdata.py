"""Upload seeded workloads to GPU tensors and compare against the oracle (test helper)."""
from __future__ import annotations

import numpy as np
import torch

from tree_verification_amd.workloads import Workload, bf16_bits


def to_dev_kv(x: np.ndarray, dtype: str, device) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(bf16_bits(x)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def i32(x, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(device)


def f32(x, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


class DevWorkload:
    """GPU copies of a Workload's arrays (logits optional)."""

    def __init__(self, wl: Workload, device="cuda:0", logits=True):
        self.wl = wl
        self.q = to_dev_kv(wl.q, wl.dtype, device)
        self.k = to_dev_kv(wl.k_cache, wl.dtype, device)
        self.v = to_dev_kv(wl.v_cache, wl.dtype, device)
        self.table = i32(wl.block_table, device)
        self.prefix_len = i32(wl.prefix_len, device)
        self.n_nodes = i32(wl.n_nodes, device)
        self.parent = i32(wl.parent, device)
        self.tokens = i32(wl.tokens, device)
        self.u_accept = f32(wl.u_accept, device)
        self.u_sample = f32(wl.u_sample, device)
        if logits and wl.target_logits is not None:
            self.target = f32(wl.target_logits, device)
            self.draft = f32(wl.draft_logits, device)


def attn_rel_errors(out_np: np.ndarray, ref_rows: dict) -> float:
    """Max over (b, u, h) rows of ||o - ref|| / ||ref||."""
    worst = 0.0
    for (b, u, h), ref in ref_rows.items():
        o = out_np[b, u, h].astype(np.float64)
        den = max(np.linalg.norm(ref), 1e-30)
        worst = max(worst, float(np.linalg.norm(o - ref) / den))
    return worst


def out_to_np(out: torch.Tensor) -> np.ndarray:
    return out.float().cpu().numpy()
