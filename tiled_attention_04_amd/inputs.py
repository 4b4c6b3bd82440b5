"""Seeded synthetic inputs shared by the tests, the bench and the smoke run.

This module holds no attention arithmetic: it only draws random numbers and
rounds them to the storage dtype, so that the HIP path and the fp64 oracle
receive bit-identical inputs.

Recipe (one ``numpy.random.default_rng(seed)`` per workload, seed 0 unless a
test says otherwise):

* dense attention: Q, then K, then V (then dO for the backward), each drawn
  as ``standard_normal(shape, dtype=float32)`` with shape [B, H, N, d] and
  rounded to bf16 (or fp16) with round-to-nearest-even (torch's
  conversion) when the workload is 16-bit;
* decode: the cache lengths first (``integers(lo, hi, endpoint=True)``), then
  the new queries [S, H, d], then for every sequence s in order its K rows
  [H, n_s, d] and its V rows [H, n_s, d].  Cache rows at or past n_s are not
  drawn: the caller fills them with NaN so that any read of them shows.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

# The workloads, by what they are.  Sizes follow the five measured settings:
# the worked example (n=8, d=4, block 4, fp32), a small bf16 forward, a
# LLaMA-7B-like bf16 layer (causal, and causal with a 1024-token window), a
# ragged KV-cache decode batch, and a causal backward.
WORKLOADS = {
    "tiny_n8_d4_fp32": dict(B=1, H=1, N=8, d=4, dtype="fp32", block=4),
    "fwd_b1_h8_n1024_d64_bf16": dict(B=1, H=8, N=1024, d=64, dtype="bf16", block=64),
    "fwd_b4_h32_n4096_d128_bf16": dict(B=4, H=32, N=4096, d=128, dtype="bf16", window=1024),
    "decode_s64_h32_d128_len512to8192_bf16": dict(S=64, H=32, d=128, Lmax=8192,
                                                  len_lo=512, len_hi=8192, dtype="bf16"),
    "bwd_b2_h16_n4096_d128_bf16": dict(B=2, H=16, N=4096, d=128, dtype="bf16"),
}

_TORCH_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPE[name]


def normal(rng: np.random.Generator, shape, dtype: str) -> torch.Tensor:
    """N(0,1) float32 draws, stored in ``dtype`` (CPU tensor, contiguous)."""
    x = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32))
    return x.to(_TORCH_DTYPE[dtype]).contiguous()


def attention_inputs(B: int, H: int, N: int, d: int, dtype: str = "bf16",
                     seed: int = 0, with_grad: bool = False):
    """q, k, v (and dO) as [B, H, N, d] CPU tensors in ``dtype``."""
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    q = normal(rng, shape, dtype)
    k = normal(rng, shape, dtype)
    v = normal(rng, shape, dtype)
    if with_grad:
        return q, k, v, normal(rng, shape, dtype)
    return q, k, v


@dataclass
class DecodeInputs:
    seqlens: np.ndarray          # [S] int32, each in [lo, hi]
    q: torch.Tensor              # [S, H, d] CPU
    k_rows: list                 # per sequence: [H, n_s, d] CPU tensor
    v_rows: list                 # per sequence: [H, n_s, d] CPU tensor

    def valid_bytes(self, elem_bytes: int) -> int:
        """Bytes of K and V rows a decode step must read."""
        H, d = self.q.shape[1], self.q.shape[2]
        return int(self.seqlens.astype(np.int64).sum()) * H * d * elem_bytes * 2


def decode_inputs(S: int, H: int, d: int, len_lo: int, len_hi: int,
                  dtype: str = "bf16", seed: int = 0, seqlens=None) -> DecodeInputs:
    """Ragged KV-cache decode batch; lengths drawn first (unless given)."""
    rng = np.random.default_rng(seed)
    if seqlens is None:
        seqlens = rng.integers(len_lo, len_hi, endpoint=True, size=S)
    seqlens = np.asarray(seqlens, dtype=np.int32)
    q = normal(rng, (S, H, d), dtype)
    k_rows, v_rows = [], []
    for s in range(S):
        n = int(seqlens[s])
        k_rows.append(normal(rng, (H, n, d), dtype))
        v_rows.append(normal(rng, (H, n, d), dtype))
    return DecodeInputs(seqlens, q, k_rows, v_rows)


def dense_cache(inp: DecodeInputs, Lmax: int, device="cpu", fill=float("nan")):
    """[S, H, Lmax, d] K and V caches holding the drawn rows; other rows = ``fill``."""
    S, H, d = inp.q.shape
    kc = torch.full((S, H, Lmax, d), fill, dtype=inp.q.dtype, device=device)
    vc = torch.full((S, H, Lmax, d), fill, dtype=inp.q.dtype, device=device)
    for s in range(S):
        n = int(inp.seqlens[s])
        kc[s, :, :n].copy_(inp.k_rows[s])
        vc[s, :, :n].copy_(inp.v_rows[s])
    return kc, vc


def paged_cache(inp: DecodeInputs, page_size: int, device="cpu", seed: int = 0,
                spare_pages: int = 0, fill=float("nan")):
    """The same rows in a page pool: ([P_total, H, page_size, d] K and V pools,
    [S, max_pages] int32 page table).

    Sequence s takes ceil(n_s / page_size) pages; the pages of all sequences
    (plus ``spare_pages`` that belong to nobody) are a random permutation of
    the pool drawn from ``default_rng(seed)``, so neighbouring tokens of one
    sequence are scattered over the pool.  Rows of a page past the sequence's
    end, spare pages and unused table entries (-1) hold ``fill``.
    """
    S, H, d = inp.q.shape
    slots = [-(-int(n) // page_size) for n in inp.seqlens]
    num_pages = sum(slots) + spare_pages
    perm = np.random.default_rng(seed).permutation(num_pages)
    max_pages = max(slots)
    table = np.full((S, max_pages), -1, dtype=np.int32)
    kp = torch.full((num_pages, H, page_size, d), fill, dtype=inp.q.dtype, device=device)
    vp = torch.full((num_pages, H, page_size, d), fill, dtype=inp.q.dtype, device=device)
    nxt = 0
    for s in range(S):
        n, m = int(inp.seqlens[s]), slots[s]
        ids = perm[nxt:nxt + m]
        nxt += m
        table[s, :m] = ids
        idx = torch.from_numpy(ids.astype(np.int64)).to(device)
        for pool, rows in ((kp, inp.k_rows[s]), (vp, inp.v_rows[s])):
            pad = torch.full((H, m * page_size, d), fill, dtype=rows.dtype)
            pad[:, :n] = rows
            pages = pad.view(H, m, page_size, d).transpose(0, 1).contiguous().to(device)
            pool.index_copy_(0, idx, pages)
    return kp, vp, torch.from_numpy(table).to(device)
