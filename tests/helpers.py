"""Shared test helpers: device transfers and the parity tolerance."""
import sys

import numpy as np


def log(msg: str):
    """Name the case on stdout before a GPU step (flushed, so a fault still shows it)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(a).cuda()


def host(t) -> np.ndarray:
    import torch
    a = t.detach().cpu()
    if a.dtype == torch.int16:
        return a.numpy().view(np.uint16)
    return a.numpy()


def vb_from_rows(v: np.ndarray) -> np.ndarray:
    """Values [nkv][Lmax][hd] -> the blocked value cache the kernels use,
    [nkv][Lmax / 32][hd][32] (position p, dimension d at [p / 32][d][p % 32])."""
    nkv, lmax, hd = v.shape
    return np.ascontiguousarray(v.reshape(nkv, lmax // 32, 32, hd).transpose(0, 1, 3, 2))


def rows_from_vb(vb: np.ndarray) -> np.ndarray:
    """The blocked value cache [nkv][Lmax / 32][hd][32] -> values [nkv][Lmax][hd]."""
    nkv, nb, hd, _ = vb.shape
    return np.ascontiguousarray(vb.transpose(0, 1, 3, 2).reshape(nkv, nb * 32, hd))


def gemm_rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    """max |y - ref| / max(|ref|, rms of ref's row): the fp32-logit parity metric
    (the floor keeps near-zero outputs from dominating)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt((ref ** 2).mean(axis=-1, keepdims=True)) + 1e-300
    den = np.maximum(np.abs(ref), rms)
    return float((np.abs(y - ref) / den).max())


GEMM_RTOL = 1e-3  # relative tolerance for fp32 logits / GEMM outputs
