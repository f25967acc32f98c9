"""Helpers shared by the GPU parity tests: widen device tensors to float64
numpy, gather logical K/V through the oracle's paged gather, and compare."""
import sys

import numpy as np
import torch

import oracle as O


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a bf16 / fp32 tensor to float64 numpy (on the CPU)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def logical_kv(k_pages, v_pages, block_table, b: int, L: int):
    """Logical ``[H_kv][L][d]`` K (and V) of sequence b, via the oracle."""
    bt = block_table[b].cpu().numpy()
    kp = f64(k_pages)
    K = O.gather_paged(kp, bt, L)
    V = None if v_pages is None else O.gather_paged(f64(v_pages), bt, L)
    return K, V


def logical_kv_rows(k_pages, v_pages, block_table, b: int, kvh: int, L: int):
    """Like ``logical_kv`` for one KV head, copying only the pages it needs
    (for multi-gigabyte caches)."""
    P = k_pages.shape[2]
    n_pg = -(-L // P)
    pages = block_table[b, :n_pg].long()
    kp = k_pages[pages.to(k_pages.device), kvh:kvh + 1]
    vp = None if v_pages is None else v_pages[pages.to(v_pages.device), kvh:kvh + 1]
    ident = np.arange(n_pg)
    K = O.gather_paged(f64(kp), ident, L)
    V = None if vp is None else O.gather_paged(f64(vp), ident, L)
    return K, V


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def max_rel(a: np.ndarray, b: np.ndarray, floor: float = 1e-30) -> float:
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), floor))) if a.size else 0.0


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def keep_swap_gap(got, want, scores, n: int, sinks: int = 0, window: int = 0, tol: float = 1e-6) -> float:
    """End-to-end keep-set check: the GPU's set ``got`` (chosen from the GPU's
    own scores) against the oracle's set ``want`` (chosen from the oracle's
    float64 scores ``scores``).  They must have the same size and keep the same
    forced positions; every position in which they differ must be a middle
    position whose oracle score lies within tol * max(1, |tau|) of the cut tau
    (the lowest oracle score the oracle kept in the middle): a swap between
    near-equal scores, which fp32 rounding may decide either way.  Returns the
    worst |score - tau| / max(1, |tau|) over the differences (0 when equal)."""
    got = set(int(x) for x in np.asarray(got).ravel())
    want = set(int(x) for x in np.asarray(want).ravel())
    assert len(got) == len(want), f"keep sets differ in size: {len(got)} vs {len(want)}"
    diff = sorted(got ^ want)
    if not diff:
        return 0.0
    lo, hi = min(sinks, n), max(n - window, 0)
    assert all(lo <= j < hi for j in diff), f"a forced position differs: {[j for j in diff if not lo <= j < hi]}"
    kept_mid = [j for j in want if lo <= j < hi]
    tau = min(scores[j] for j in kept_mid)
    scale = max(1.0, abs(tau))
    gaps = [abs(scores[j] - tau) / scale for j in diff]
    worst = max(gaps)
    assert worst <= tol, (f"{len(diff)} differing positions, worst gap {worst:.3e} > {tol:g} "
                          f"(tau {tau:.9g}; positions {diff[:8]})")
    return worst
