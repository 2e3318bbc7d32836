"""Seeded synthetic inputs for the K4V2 KV-cache workloads.

This module holds no arithmetic of the method: it only draws keys, values,
queries, page tables and lengths.  Both the GPU path and the CPU oracle are fed
from it.  Every array is a deterministic function of (workload, seed, index)
and of the torch device whose generator draws it (CPU and GPU generators give
different streams for the same seed; a test uses one of them for both sides).

Workloads (attention shapes of the models named; the models' weights and
evaluation sets are not used, these tensors stand in for them):

* ``tiny``           1 seq, 1 q head, 1 KV head, 1024 tokens; 4 key channels x20.
* ``qwen3_32b_16k``  8 seqs x 16384 tokens (+1 appended), 64 q / 8 KV heads;
                     3 key channels (2% of 128) x15 per KV head.
* ``qwen3_4b_64k``   32 seqs, ragged lengths U{32768..65536}, 32 q / 8 KV heads.
* ``qwen3_30b_a3b_128k`` 4 seqs x 131072 tokens, 32 q / 4 KV heads.
* ``llama31_70b_128k``   1 seq, 131072-token prompt with Student-t(3) keys,
                     then 64 decode steps appending one token each; 64 q / 8 KV.

Values and queries are N(0, 1); keys are N(0, 1) with fixed outlier channels
(drawn once per KV head from the seed), or raw Student-t(3).  All cast to fp16
with round-to-nearest-even.  Pages hold 16 tokens; the block table is a random
permutation of all pages of the batch.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np
import torch

HEAD_DIM = 128
PAGE = 16
BASE_SEED = 20260605


@dataclass(frozen=True)
class Workload:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    context: int                 # tokens cached before the step (max for ragged)
    new_tokens: int = 0          # tokens appended per sequence (one per step)
    ragged_min: int = 0          # >0: lengths uniform in [ragged_min, context]
    outlier_channels: int = 0    # key channels scaled per KV head
    outlier_scale: float = 1.0
    key_dist: str = "normal"     # "normal" | "student_t3"
    seed_index: int = 0
    notes: str = ""

    @property
    def gqa(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def seed(self) -> int:
        return BASE_SEED + self.seed_index


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1, 1024, new_tokens=0, outlier_channels=4,
                     outlier_scale=20.0, seed_index=0),
    "qwen3_32b_16k": Workload("qwen3_32b_16k", 8, 64, 8, 16384, new_tokens=1,
                              outlier_channels=3, outlier_scale=15.0, seed_index=1),
    "qwen3_4b_64k": Workload("qwen3_4b_64k", 32, 32, 8, 65536, ragged_min=32768,
                             outlier_channels=3, outlier_scale=15.0, seed_index=2),
    "qwen3_30b_a3b_128k": Workload("qwen3_30b_a3b_128k", 4, 32, 4, 131072,
                                   outlier_channels=3, outlier_scale=15.0, seed_index=3),
    "llama31_70b_128k": Workload("llama31_70b_128k", 1, 64, 8, 131072, new_tokens=64,
                                 key_dist="student_t3", seed_index=4),
}


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    if overrides:
        d = dict(w.__dict__)
        d.update(overrides)
        w = Workload(**d)
    return w


def _gen(seed: int, stream: int, index: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    # a fixed, documented mixing of (seed, stream, index) into one 63-bit seed
    s = (seed * 1_000_003 + stream * 7_919 + index * 104_729) & ((1 << 63) - 1)
    g.manual_seed(s)
    return g


_K, _V, _Q, _OUT, _PERM, _LEN, _EXTRA = range(7)


def seq_lens(w: Workload) -> np.ndarray:
    """Cached lengths before the step (int64 [num_seqs])."""
    if w.ragged_min:
        g = _gen(w.seed, _LEN, 0, "cpu")
        n = torch.randint(w.ragged_min, w.context + 1, (w.num_seqs,), generator=g)
        return n.numpy().astype(np.int64)
    return np.full(w.num_seqs, w.context, np.int64)


def final_lens(w: Workload) -> np.ndarray:
    """Lengths once every new token of the workload has been appended."""
    return seq_lens(w) + w.new_tokens


def outlier_channels(w: Workload) -> np.ndarray:
    """int64 [num_kv_heads][outlier_channels], distinct channels per KV head."""
    g = _gen(w.seed, _OUT, 0, "cpu")
    rows = [torch.randperm(HEAD_DIM, generator=g)[: w.outlier_channels] for _ in range(w.num_kv_heads)]
    if w.outlier_channels == 0:
        return np.zeros((w.num_kv_heads, 0), np.int64)
    return torch.stack(rows).numpy().astype(np.int64)


def page_table(w: Workload):
    """(block_tables int32 [num_seqs][max_pages], num_pages).  Sequence b owns
    ceil(final_len_b / 16) pages, taken in order from one random permutation
    of all pages; unused entries are -1."""
    lens = final_lens(w)
    pages = [int(math.ceil(n / PAGE)) for n in lens]
    total = sum(pages)
    max_pages = max(pages)
    g = _gen(w.seed, _PERM, 0, "cpu")
    perm = torch.randperm(total, generator=g).numpy().astype(np.int32)
    bt = np.full((w.num_seqs, max_pages), -1, np.int32)
    o = 0
    for b, p in enumerate(pages):
        bt[b, :p] = perm[o:o + p]
        o += p
    return bt, total


def slot_mapping(block_tables: np.ndarray, b: int, start: int, count: int) -> np.ndarray:
    """Slots of token positions [start, start+count) of sequence b (int64)."""
    t = np.arange(start, start + count, dtype=np.int64)
    return block_tables[b, t // PAGE].astype(np.int64) * PAGE + t % PAGE


def sequence_kv(w: Workload, b: int, start: int = 0, count: int | None = None,
                device="cpu"):
    """Keys and values of sequence b, token positions [start, start+count):
    fp16 torch tensors [count][num_kv_heads][128] on `device`.  Draws are made
    per block of 4096 positions, so any sub-range reproduces the same values."""
    n = int(final_lens(w)[b])
    if count is None:
        count = n - start
    assert 0 <= start and start + count <= n
    out_k = torch.empty((count, w.num_kv_heads, HEAD_DIM), dtype=torch.float16, device=device)
    out_v = torch.empty_like(out_k)
    blk = 4096
    och = torch.as_tensor(outlier_channels(w), device=device)
    for b0 in range(start - start % blk, start + count, blk):
        k, v = _kv_block(w, b, b0 // blk, blk, device, och)
        lo = max(start, b0)
        hi = min(start + count, b0 + blk)
        out_k[lo - start:hi - start] = k[lo - b0:hi - b0]
        out_v[lo - start:hi - start] = v[lo - b0:hi - b0]
    return out_k, out_v


def _kv_block(w: Workload, b: int, blk_idx: int, blk: int, device, och):
    shape = (blk, w.num_kv_heads, HEAD_DIM)
    gk = _gen(w.seed, _K, b * 1_000_000 + blk_idx, device)
    gv = _gen(w.seed, _V, b * 1_000_000 + blk_idx, device)
    if w.key_dist == "student_t3":
        z = torch.randn(shape, generator=gk, device=device, dtype=torch.float32)
        c = torch.randn((3,) + shape, generator=gk, device=device, dtype=torch.float32)
        k = z / torch.sqrt((c * c).sum(0) / 3.0)
    else:
        k = torch.randn(shape, generator=gk, device=device, dtype=torch.float32)
    if och.numel():
        scale = torch.ones((w.num_kv_heads, HEAD_DIM), device=device)
        scale.scatter_(1, och, w.outlier_scale)
        k = k * scale
    v = torch.randn(shape, generator=gv, device=device, dtype=torch.float32)
    return k.half(), v.half()


def queries(w: Workload, step: int = 0, device="cpu") -> torch.Tensor:
    """fp16 [num_seqs][num_q_heads][128] query of decode step `step`."""
    g = _gen(w.seed, _Q, step, device)
    q = torch.randn((w.num_seqs, w.num_q_heads, HEAD_DIM), generator=g, device=device,
                    dtype=torch.float32)
    return q.half()


def extra_normal(seed: int, index: int, shape, device="cpu") -> torch.Tensor:
    """Plain seeded N(0,1) fp16 draws for ad-hoc test shapes."""
    g = _gen(seed, _EXTRA, index, device)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).half()
