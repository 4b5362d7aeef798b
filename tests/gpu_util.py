"""Helpers for the GPU tests: device copies of generated layers and the
comparison metrics.  Inputs come from the seeded generator; expected values
come from the oracle only."""
from __future__ import annotations

import functools

import numpy as np

import block_scaled_fp4_router_amd as ft
import synth

DEV = "cuda"


def say(msg: str) -> None:
    print(msg, flush=True)


@functools.lru_cache(maxsize=4)
def layer_pair(name: str, packed: bool = False):
    """(host layer, device layer) for a named configuration, cached; with
    ``packed`` the device layer also holds the prefill tile layout."""
    lay = synth.make_layer(name)
    dlay = ft.DeviceLayer.from_host(lay, DEV)
    return lay, dlay.pack() if packed else dlay


def to_dev_bf16(x_bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(DEV)


def bf16_dev_to_f64(t) -> np.ndarray:
    u = t.cpu().numpy().view(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def run_forward(dlay: ft.DeviceLayer, x_bits: np.ndarray, path: str = "auto"):
    """ftmoe_forward through the C ABI; returns (y f64, ids, w)."""
    import torch
    T = x_bits.shape[0]
    lay = dlay.with_path(path)
    x = to_dev_bf16(x_bits)
    ws = ft.alloc_workspace(lay, T)
    y = torch.empty((T, dlay.hidden), dtype=torch.int16, device=DEV)
    ids = torch.empty((T, dlay.top_k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, dlay.top_k), dtype=torch.float32, device=DEV)
    ft.forward(lay, x, T, ws, y, ids, w)
    torch.cuda.synchronize()
    return bf16_dev_to_f64(y), ids.cpu().numpy(), w.cpu().numpy()


def rel_fro(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def sample_tokens(T: int, n: int, seed: int = 0) -> np.ndarray:
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    s = np.sort(rng.choice(T, n - 2, replace=False))
    return np.unique(np.concatenate([[0], s, [T - 1]]))  # include both ends
