"""Seeded synthetic inputs for score-guided KV selection.

This module only draws and lays out inputs: queries, a paged K/V cache with a
shuffled block table, ragged lengths, planted attention sinks and "hot"
regions.  It holds none of the method's arithmetic (no softmax, no scoring, no
selection), so both the float64 oracle checks and the GPU path may consume
what it returns.

Every draw comes from ``torch.Generator`` seeded explicitly; float32 draws are
rounded to bfloat16 with round-to-nearest-even where a workload is bf16.
Generation runs on whatever device the caller names (CPU for tests, the GPU
for the multi-gigabyte caches).

Planted structure (the pages describe the mechanism, not a recipe):
* attention sinks: a seeded unit direction u0 is projected out of every key and
  query; every query gets sqrt(d)*u0 and sink key j gets b_j*u0, so that with
  the softmax scale d^-1/2 the logit of sink key j rises by exactly b_j before
  rounding ("KV-cache eviction strategies" §3: early tokens soak up surplus
  attention);
* hot regions: 8 disjoint Gaussian bumps of 512 positions, each along its own
  direction orthogonal to u0, amplitude 4*exp(-t^2 / (2*(512/6)^2)) at offset t
  from the centre; queries carry sqrt(d) times the sum of the bump directions.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import torch

__all__ = [
    "PagedKV", "generator", "shuffled_block_table", "normal", "write_positions",
    "orthonormal_directions", "plant_sinks_and_bumps",
    "tiny_case", "qwen_like_layer", "llama3_8b_layer", "llama70b_layer", "long_context_128k",
]


@dataclass
class PagedKV:
    """One layer's paged cache.  Pages are ``[num_pages][H_kv][P][d]``."""
    k_pages: torch.Tensor
    v_pages: Optional[torch.Tensor]
    block_table: torch.Tensor          # int32 [B][max_pages]
    seq_lens: torch.Tensor             # int32 [B]
    page_size: int

    @property
    def num_seqs(self) -> int:
        return int(self.block_table.shape[0])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k_pages.shape[1])

    @property
    def head_dim(self) -> int:
        return int(self.k_pages.shape[3])

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    def to(self, device) -> "PagedKV":
        return PagedKV(self.k_pages.to(device),
                       None if self.v_pages is None else self.v_pages.to(device),
                       self.block_table.to(device), self.seq_lens.to(device), self.page_size)


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, gen: torch.Generator, dtype=torch.float32, device="cpu") -> torch.Tensor:
    """N(0,1) float32 draws, rounded (RNE) to ``dtype``."""
    x = torch.randn(*shape, generator=gen, dtype=torch.float32, device=device)
    return x if dtype == torch.float32 else x.to(dtype)


def shuffled_block_table(num_seqs: int, capacity: int, page_size: int, gen: torch.Generator,
                         device="cpu", extra_pages: int = 0):
    """Give every sequence ceil(capacity / P) physical pages drawn from a
    random permutation of the pool (plus ``extra_pages`` never referenced).
    Returns (block_table int32 [B][max_pages], num_pages)."""
    max_pages = -(-capacity // page_size)
    num_pages = num_seqs * max_pages + extra_pages
    perm = torch.randperm(num_pages, generator=gen, device=device)
    bt = perm[:num_seqs * max_pages].view(num_seqs, max_pages).to(torch.int32)
    return bt.contiguous(), num_pages


def write_positions(pages: torch.Tensor, block_table_row: torch.Tensor, start: int,
                    values: torch.Tensor) -> None:
    """Store ``values`` ``[H_kv][n][d]`` at logical positions start..start+n-1
    of one sequence (slot j lives in page block_table_row[j // P], row j % P)."""
    P = pages.shape[2]
    n = values.shape[1]
    pos = torch.arange(start, start + n, device=pages.device)
    pg = block_table_row.to(pages.device).long()[pos // P]
    pages[pg, :, pos % P, :] = values.permute(1, 0, 2).to(pages.dtype)


def orthonormal_directions(n: int, d: int, gen: torch.Generator, device="cpu") -> torch.Tensor:
    """``n`` seeded orthonormal directions in R^d (rows), float32."""
    a = torch.randn(d, n, generator=gen, dtype=torch.float64, device=gen.device).cpu()
    qm, _ = torch.linalg.qr(a)
    return qm.T.contiguous().to(torch.float32).to(device)


def plant_sinks_and_bumps(keys: torch.Tensor, queries: torch.Tensor, dirs: torch.Tensor,
                          sink_bias: torch.Tensor, bump_amp: Optional[torch.Tensor]):
    """Plant sinks (and optionally bumps) into float32 logical data.

    keys ``[H_kv][L][d]`` and queries ``[..., d]`` are modified in place.
    ``dirs`` rows: u0 first, then one direction per bump.  ``sink_bias``
    ``[H_kv][n_sink]`` is added along u0 to keys 0..n_sink-1.  ``bump_amp``
    ``[n_bump][L]`` (or None) is the per-position amplitude along each bump
    direction.  Queries get sqrt(d) times every direction used.
    """
    d = keys.shape[-1]
    used = dirs if bump_amp is not None else dirs[:1]
    # project the planted directions out of the random data
    keys -= (keys @ used.T) @ used
    queries -= (queries @ used.T) @ used
    n_sink = sink_bias.shape[1]
    keys[:, :n_sink, :] += sink_bias[:, :, None] * used[0]
    if bump_amp is not None:
        keys += (bump_amp.T @ used[1:])[None, :, :]
    queries += math.sqrt(d) * used.sum(0)


def _bump_amplitude(L: int, centres, device="cpu") -> torch.Tensor:
    """Gaussian bump amplitude per position for each centre: 4 exp(-t^2/(2
    sigma^2)), sigma = 512/6, over the 511 positions with |t| < 256."""
    pos = torch.arange(L, dtype=torch.float32, device=device)
    sigma = 512.0 / 6.0
    amps = []
    for c in centres:
        t = pos - float(c)
        a = 4.0 * torch.exp(-(t * t) / (2.0 * sigma * sigma))
        a[t.abs() >= 256] = 0.0
        amps.append(a)
    return torch.stack(amps)


def _bump_centres(L_prefix: int, n: int, gen: torch.Generator):
    """``n`` centres in [1024, L_prefix - 1024) at least 512 apart (disjoint)."""
    lo, hi = 1024, L_prefix - 1024
    assert hi - lo > n * 512, "sequence too short for disjoint bumps"
    centres = []
    while len(centres) < n:
        c = int(torch.randint(lo, hi, (1,), generator=gen, device=gen.device))
        if all(abs(c - x) >= 512 for x in centres):
            centres.append(c)
    return sorted(centres)


# --------------------------------------------------------------------------
# workload builders
# --------------------------------------------------------------------------
def tiny_case(seed: int = 1, prompt: int = 512, steps: int = 16, device="cpu"):
    """Tiny case: 1 sequence, 4 query heads on 1 KV head, d=64, fp32, P=16,
    a 512-token prompt, +4 logit on keys 0-3, then ``steps`` decode steps each
    appending one N(0,1) key/value and drawing a fresh query."""
    g = generator(seed)
    Hq, Hkv, d, P = 4, 1, 64, 16
    cap = prompt + steps
    K = normal((Hkv, cap, d), g)
    V = normal((Hkv, cap, d), g)
    q = normal((steps, 1, Hq, d), g)
    dirs = orthonormal_directions(1, d, g)
    sink = torch.full((Hkv, 4), 4.0)
    plant_sinks_and_bumps(K, q, dirs, sink, None)
    bt, num_pages = shuffled_block_table(1, cap, P, g)
    kp = normal((num_pages, Hkv, P, d), g)
    vp = normal((num_pages, Hkv, P, d), g)
    write_positions(kp, bt[0], 0, K)
    write_positions(vp, bt[0], 0, V)
    kv = PagedKV(kp, vp, bt, torch.tensor([prompt], dtype=torch.int32), P)
    return {"kv": kv.to(device), "q_steps": q.to(device), "num_q_heads": Hq,
            "scale": 1.0 / math.sqrt(d), "prompt": prompt, "steps": steps,
            "block_size": 16, "sinks": 4, "window": 64, "budget": 128}


def qwen_like_layer(seed: int = 2, n_tokens: int = 1600, device="cpu"):
    """Qwen3-0.6B-like layer: 16 query / 8 KV heads, d=128, bf16; one
    sequence of ``n_tokens`` whose keys carry sink boosts U[3,5] on positions
    0-3.  Returns logical K, V, Q (queries for every position), bf16."""
    g = generator(seed)
    Hq, Hkv, d = 16, 8, 128
    K = normal((Hkv, n_tokens, d), g)
    V = normal((Hkv, n_tokens, d), g)
    Q = normal((Hq, n_tokens, d), g)
    dirs = orthonormal_directions(1, d, g)
    sink = 3.0 + 2.0 * torch.rand(Hkv, 4, generator=g)
    plant_sinks_and_bumps(K, Q.view(-1, d), dirs, sink, None)
    return {"K": K.to(torch.bfloat16).to(device), "V": V.to(torch.bfloat16).to(device),
            "Q": Q.to(torch.bfloat16).to(device), "num_q_heads": Hq,
            "scale": 1.0 / math.sqrt(d), "chunk": 64, "budget": 256, "sinks": 4,
            "page_size": 16}


def llama3_8b_layer(seed: int = 3, num_seqs: int = 16, min_len: int = 8192, max_len: int = 32768,
                  steps: int = 256, device="cpu"):
    """Llama-3-8B-shape layer: 32 query / 8 KV heads, d=128, bf16, P=16,
    ragged L_b ~ U{min_len..max_len}, shuffled block table, N(0,1) data, and a
    per-sequence temperature T_b ~ U[0.5, 2] folded into the queries (q/T_b).
    The cache has room for ``steps`` appended tokens; ``q_steps`` holds one
    query per step, ``new_kv`` the appended K/V per step."""
    g = generator(seed, device)
    Hq, Hkv, d, P = 32, 8, 128, 16
    lens = torch.randint(min_len, max_len + 1, (num_seqs,), generator=g, device=device)
    cap = int(lens.max()) + steps
    bt, num_pages = shuffled_block_table(num_seqs, cap, P, g, device)
    kp = normal((num_pages, Hkv, P, d), g, torch.bfloat16, device)
    vp = normal((num_pages, Hkv, P, d), g, torch.bfloat16, device)
    temp = 0.5 + 1.5 * torch.rand(num_seqs, generator=g, device=device)
    q = normal((steps, num_seqs, Hq, d), g, torch.float32, device)
    q = (q / temp[None, :, None, None]).to(torch.bfloat16)
    kv = PagedKV(kp, vp, bt, lens.to(torch.int32), P)
    return {"kv": kv, "q_steps": q, "num_q_heads": Hq, "scale": 1.0 / math.sqrt(d),
            "temperature": temp, "block_size": 16, "sinks": 4, "window": 512,
            "budget_frac": 0.2}


def llama70b_layer(layer: int, seed: int = 4, num_seqs: int = 8, seq_len: int = 32768,
                  device="cpu", block_table: Optional[torch.Tensor] = None):
    """One layer of the LLaMA-70B-shape step: 64 query / 8 KV heads, d=128,
    bf16, P=64, B=8 at L=32768, N(0,1) data.  Each layer draws from its own
    seed (seed * 1000 + layer); all layers share one block table."""
    Hq, Hkv, d, P = 64, 8, 128, 64
    g = generator(seed * 1000 + layer, device)
    if block_table is None:
        bt, num_pages = shuffled_block_table(num_seqs, seq_len, P, generator(seed, device), device)
    else:
        bt, num_pages = block_table, int(block_table.numel())
    kp = normal((num_pages, Hkv, P, d), g, torch.bfloat16, device)
    vp = normal((num_pages, Hkv, P, d), g, torch.bfloat16, device)
    q = normal((num_seqs, Hq, d), g, torch.bfloat16, device)
    lens = torch.full((num_seqs,), seq_len, dtype=torch.int32, device=device)
    return {"kv": PagedKV(kp, vp, bt, lens, P), "q": q, "num_q_heads": Hq,
            "scale": 1.0 / math.sqrt(d), "block_size": 64, "budget_frac": 0.25}


def long_context_128k(seed: int = 5, num_seqs: int = 4, seq_len: int = 131072, window: int = 32,
            sparse_steps: int = 64, device="cpu"):
    """128K long-context case: 32 query / 8 KV heads, d=128, bf16, P=16,
    planted sinks (U[3,5]) and 8 Gaussian hot regions per sequence; a
    one-head d=64 indexer cache with the same planted positions; window
    queries for the vote and per-step decode queries (model and indexer) for
    ``sparse_steps`` decode steps whose K/V are appended after position L."""
    Hq, Hkv, d, dI, P = 32, 8, 128, 64, 16
    g = generator(seed, device)
    cap = seq_len + sparse_steps
    bt, num_pages = shuffled_block_table(num_seqs, cap, P, g, device)
    kp = torch.empty((num_pages, Hkv, P, d), dtype=torch.bfloat16, device=device)
    vp = normal((num_pages, Hkv, P, d), g, torch.bfloat16, device)
    kip = torch.empty((num_pages, 1, P, dI), dtype=torch.bfloat16, device=device)
    dirs = orthonormal_directions(9, d, g, device)
    dirs_i = orthonormal_directions(9, dI, g, device)
    q_win = torch.empty((num_seqs, Hq, window, d), dtype=torch.bfloat16, device=device)
    q_dec = torch.empty((sparse_steps, num_seqs, Hq, d), dtype=torch.bfloat16, device=device)
    qi_dec = torch.empty((sparse_steps, num_seqs, Hq, dI), dtype=torch.bfloat16, device=device)
    centres_all = []
    for b in range(num_seqs):
        centres = _bump_centres(seq_len - window, 8, g)
        centres_all.append(centres)
        amp = _bump_amplitude(cap, centres, device)
        sink = 3.0 + 2.0 * torch.rand(Hkv, 4, generator=g, device=device)
        K = normal((Hkv, cap, d), g, torch.float32, device)
        qw = normal((Hq, window + sparse_steps, d), g, torch.float32, device)
        plant_sinks_and_bumps(K, qw, dirs, sink, amp)
        KI = normal((1, cap, dI), g, torch.float32, device)
        qi = normal((Hq, sparse_steps, dI), g, torch.float32, device)
        plant_sinks_and_bumps(KI, qi, dirs_i, sink[:1], amp)
        write_positions(kp, bt[b], 0, K)
        write_positions(kip, bt[b], 0, KI)
        q_win[b] = qw[:, :window].to(torch.bfloat16)
        q_dec[:, b] = qw[:, window:].permute(1, 0, 2).to(torch.bfloat16)
        qi_dec[:, b] = qi.permute(1, 0, 2).to(torch.bfloat16)
    lens = torch.full((num_seqs,), seq_len, dtype=torch.int32, device=device)
    return {"kv": PagedKV(kp, vp, bt, lens, P),
            "kv_index": PagedKV(kip, None, bt, lens.clone(), P),
            "q_win": q_win, "q_dec": q_dec, "qi_dec": qi_dec, "centres": centres_all,
            "num_q_heads": Hq, "scale": 1.0 / math.sqrt(d), "window": window,
            "pool_kernel": 7, "vote_k": 4096, "index_k": 2048}
