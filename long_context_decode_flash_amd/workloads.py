"""Seeded synthetic workloads for the paged K8/V4 decode-attention path.

This module only draws inputs: fp32 K/V rows, fp16 queries, page tables, slot numbers and
sequence lengths.  It holds none of the method's arithmetic (no quantization, no attention),
so both the HIP path and the CPU oracle can be fed from it.

The shapes stand in for the workloads of the three pages, which measure on private prompts
rather than a public suite:
  * a 65,536-token single-request decode (blog page "標籤: vLLM", opening summary);
  * a 256K context on one card with MTP (video notes "影片筆記：NInfer + 千问3.8 27b = 1.5倍速
    @256K上下文(单张4090 24GB)", 核心重點);
  * a 184,320-token KV pool shared by two concurrent requests, MTP with 3 drafts, prefill in
    1,024-token chunks (forum post "3090 单卡跑 Qwen3.8-27B：NInfer 上机实测（180K 上下文 / C2
    并发 / 4bit KV）", 一、部署 launch-flag table and 二、测评).
Values are N(0, 1) unless a workload says otherwise.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

TILE = 16  # tokens per tile of the page format


@dataclass(frozen=True)
class Workload:
    name: str
    n_seq: int            # concurrent sequences sharing one pool
    seq_len: int          # tokens attended by the last query row of each sequence
    num_kv_heads: int
    n_q_heads: int
    head_dim: int
    page_size: int
    pool_pages: int       # pages in the pool
    page_order: str       # "identity" | "random" | "interleaved"
    n_rows: int           # query rows per sequence (1 = decode, 4 = MTP 1 + 3 drafts)
    n_new: int            # tokens appended per sequence in the step (already counted in seq_len)
    k_outliers: bool      # multiply 4 random K channels per KV head by 8
    seed: int
    q_scale: float = 1.0  # queries are N(0, q_scale^2): > 1 makes attention peaked

    @property
    def group(self) -> int:
        return self.n_q_heads // self.num_kv_heads

    @property
    def pages_per_seq(self) -> int:
        return -(-self.seq_len // self.page_size)


WORKLOADS = {
    "tiny_512": Workload("tiny_512", 1, 512, 1, 4, 64, 16, 32, "identity", 1, 1, False, 1000),
    "ctx8k": Workload("ctx8k", 1, 8192, 4, 24, 256, 64, 128, "identity", 1, 1, False, 1001),
    "ctx64k_outlier": Workload("ctx64k_outlier", 1, 65536, 4, 24, 256, 64, 1024, "random", 1,
                               0, True, 1002),
    "ctx184k_c2": Workload("ctx184k_c2", 2, 92160, 4, 24, 256, 64, 2880, "interleaved", 1, 1,
                           False, 1003),
    "ctx256k_mtp": Workload("ctx256k_mtp", 1, 262144, 4, 24, 256, 64, 4096, "random", 4, 4,
                            False, 1004),
}

# the workload the throughput metric is quoted on: 184,320-token pool, two sequences
HEADLINE = "ctx184k_c2"


def scaled(wl: Workload, seq_len: int, name: str | None = None, **kw) -> Workload:
    """Same structure (heads, dims, page size, order, rows) at another context length; the
    pool keeps its slack over what the sequences need."""
    pages = -(-seq_len // wl.page_size)
    slack = max(wl.pool_pages - wl.n_seq * wl.pages_per_seq, 0)
    pool = wl.n_seq * pages + min(slack, 8)
    return replace(wl, name=name or f"{wl.name}@{seq_len}", seq_len=seq_len, pool_pages=pool,
                   **kw)


def page_tables(wl: Workload, rng: np.random.Generator) -> np.ndarray:
    """int32 [n_seq][pages_per_seq] logical -> physical page."""
    npp = wl.pages_per_seq
    need = wl.n_seq * npp
    assert wl.pool_pages >= need, "pool too small for the sequences"
    if wl.page_order == "identity":
        order = np.arange(wl.pool_pages)
        table = order[:need].reshape(wl.n_seq, npp)
    elif wl.page_order == "random":
        order = rng.permutation(wl.pool_pages)
        table = order[:need].reshape(wl.n_seq, npp)
    elif wl.page_order == "interleaved":
        # one seeded permutation of the pool dealt alternately to the sequences
        order = rng.permutation(wl.pool_pages)[:need]
        table = np.stack([order[s::wl.n_seq] for s in range(wl.n_seq)])
    else:
        raise ValueError(wl.page_order)
    return np.ascontiguousarray(table, dtype=np.int32)


def slots_for(table: np.ndarray, page_size: int, seq: int, t0: int, t1: int) -> np.ndarray:
    """Cache slots of logical tokens [t0, t1) of sequence ``seq``."""
    t = np.arange(t0, t1, dtype=np.int64)
    return (table[seq, t // page_size].astype(np.int64) * page_size + t % page_size).astype(
        np.int32)


@dataclass
class Inputs:
    wl: Workload
    k: np.ndarray          # fp32 [n_seq][seq_len][Hkv][D]
    v: np.ndarray          # fp32 [n_seq][seq_len][Hkv][D]
    q_bits: np.ndarray     # uint16 (fp16 bits) [n_seq][n_rows][Hq][D]
    page_table: np.ndarray  # int32 [n_seq][pages_per_seq]
    seq_lens: np.ndarray   # int32 [n_seq]
    outlier_dims: np.ndarray | None  # int64 [Hkv][4] when k_outliers

    def token_range(self, t0: int, t1: int):
        """(k, v, slots) of tokens [t0, t1) of every sequence, sequence-major, flattened to
        [n][Hkv][D] as kvq_append takes them."""
        wl = self.wl
        ks, vs, ss = [], [], []
        for s in range(wl.n_seq):
            ks.append(self.k[s, t0:t1])
            vs.append(self.v[s, t0:t1])
            ss.append(slots_for(self.page_table, wl.page_size, s, t0, t1))
        return (np.ascontiguousarray(np.concatenate(ks)), np.ascontiguousarray(np.concatenate(vs)),
                np.concatenate(ss))

    def all_tokens(self):
        """Every sequence's tokens [0, seq_lens[s]) (ragged lengths respected)."""
        wl = self.wl
        ks, vs, ss = [], [], []
        for s in range(wl.n_seq):
            n = int(self.seq_lens[s])
            ks.append(self.k[s, :n])
            vs.append(self.v[s, :n])
            ss.append(slots_for(self.page_table, wl.page_size, s, 0, n))
        return (np.ascontiguousarray(np.concatenate(ks)), np.ascontiguousarray(np.concatenate(vs)),
                np.concatenate(ss))

    def ring(self, ring_pages: int, extra_cols: int = 2, lens=None):
        """The same tokens on ring pages: sequence s owns pool pages [s * ring_pages, (s + 1) *
        ring_pages) in a seeded order, and logical page n of it sits in table entry
        n % ring_pages.  Returns (table [n_seq][ring_pages + extra_cols] int32, (k, v, slots) of
        the tokens a ring that size still holds: each sequence's last ring_pages logical pages,
        below its length, flattened as token_range does).  The extra columns name pages of
        another sequence, so a lookup that ignores the ring reads the wrong tokens.  ``lens``
        (default seq_lens) are the lengths whose resident tokens are returned."""
        wl = self.wl
        P = wl.page_size
        assert wl.n_seq * ring_pages <= wl.pool_pages
        rng = np.random.default_rng(wl.seed + 77)
        table = np.zeros((wl.n_seq, ring_pages + extra_cols), np.int32)
        for s in range(wl.n_seq):
            table[s, :ring_pages] = s * ring_pages + rng.permutation(ring_pages)
            other = (s + 1) % wl.n_seq
            table[s, ring_pages:] = other * ring_pages + (np.arange(extra_cols) % ring_pages)
        ks, vs, ss = [], [], []
        lens = self.seq_lens if lens is None else lens
        for s in range(wl.n_seq):
            n = int(lens[s])
            t0 = max(0, (n - 1) // P - ring_pages + 1) * P
            t = np.arange(t0, n, dtype=np.int64)
            ks.append(self.k[s, t0:n])
            vs.append(self.v[s, t0:n])
            ss.append((table[s, (t // P) % ring_pages].astype(np.int64) * P + t % P).astype(np.int32))
        return table, (np.ascontiguousarray(np.concatenate(ks)),
                       np.ascontiguousarray(np.concatenate(vs)), np.concatenate(ss))

    def ring_slots(self, table: np.ndarray, ring_pages: int, seq: int, t0: int, t1: int):
        """Slots of logical tokens [t0, t1) of ``seq`` on the ring ``table``."""
        P = self.wl.page_size
        t = np.arange(t0, t1, dtype=np.int64)
        return (table[seq, (t // P) % ring_pages].astype(np.int64) * P + t % P).astype(np.int32)

    def ragged_split(self, n_new: int):
        """For ragged lengths: the tokens cached before a step that appends each sequence's last
        n_new tokens, as (k, v, slots) flattened like token_range; and those new tokens, both as
        the same flattened triple and as (k_new, v_new) fp32 [n_seq][n_new][Hkv][D]."""
        wl = self.wl
        pre = ([], [], [])
        new = ([], [], [])
        k_new = np.zeros((wl.n_seq, n_new, wl.num_kv_heads, wl.head_dim), np.float32)
        v_new = np.zeros_like(k_new)
        for s in range(wl.n_seq):
            n = int(self.seq_lens[s])
            t0 = max(n - n_new, 0)
            for dst, a, b in ((pre, 0, t0), (new, t0, n)):
                dst[0].append(self.k[s, a:b])
                dst[1].append(self.v[s, a:b])
                dst[2].append(slots_for(self.page_table, wl.page_size, s, a, b))
            k_new[s, n_new - (n - t0):] = self.k[s, t0:n]
            v_new[s, n_new - (n - t0):] = self.v[s, t0:n]
        flat = lambda t: (np.ascontiguousarray(np.concatenate(t[0])),
                          np.ascontiguousarray(np.concatenate(t[1])), np.concatenate(t[2]))
        return flat(pre), flat(new), k_new, v_new

    def prefill(self):
        """Tokens already in the cache before the step: [0, seq_len - n_new)."""
        return self.token_range(0, self.wl.seq_len - self.wl.n_new)

    def step_tokens(self):
        """Tokens the step appends: [seq_len - n_new, seq_len)."""
        return self.token_range(self.wl.seq_len - self.wl.n_new, self.wl.seq_len)


def generate(wl: Workload) -> Inputs:
    """Draw a workload's inputs from ``numpy.random.default_rng(wl.seed)`` in a fixed order:
    K, V, Q, page permutation, outlier channels."""
    rng = np.random.default_rng(wl.seed)
    shape = (wl.n_seq, wl.seq_len, wl.num_kv_heads, wl.head_dim)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    q = rng.standard_normal((wl.n_seq, wl.n_rows, wl.n_q_heads, wl.head_dim), dtype=np.float32)
    if wl.q_scale != 1.0:
        q *= np.float32(wl.q_scale)
    q_bits = q.astype(np.float16).view(np.uint16)
    table = page_tables(wl, rng)
    outliers = None
    if wl.k_outliers:
        outliers = np.stack([rng.choice(wl.head_dim, 4, replace=False)
                             for _ in range(wl.num_kv_heads)])
        for h in range(wl.num_kv_heads):
            k[:, :, h, outliers[h]] *= np.float32(8.0)
    seq_lens = np.full(wl.n_seq, wl.seq_len, np.int32)
    return Inputs(wl, k, v, q_bits, table, seq_lens, outliers)


def custom(n_seq=1, seq_lens=(100,), num_kv_heads=1, n_q_heads=4, head_dim=64, page_size=16,
           n_rows=1, page_order="random", extra_pages=3, seed=7, q_scale=1.0,
           k_outliers=False, name="custom"):
    """A small case with per-sequence lengths (ragged allowed) for parity tests. Returns
    Inputs whose ``seq_lens`` hold the given lengths; K/V are drawn to the longest."""
    seq_lens = tuple(int(x) for x in seq_lens)
    assert len(seq_lens) == n_seq
    L = max(seq_lens)
    npp = -(-L // page_size)
    wl = Workload(name, n_seq, L, num_kv_heads, n_q_heads, head_dim, page_size,
                  n_seq * npp + extra_pages, page_order, n_rows, 0, k_outliers, seed, q_scale)
    inp = generate(wl)
    inp.seq_lens = np.asarray(seq_lens, np.int32)
    return inp
