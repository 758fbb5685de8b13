"""Seeded synthetic inputs for the NVFP4 paged-KV decode workloads.

Shared by the tests (both the oracle side and the GPU side), ``__graft_entry__.smoke`` and
``bench.py``.  This module only draws random numbers, rounds them to bf16 (torch's cast) and
builds page tables; it holds none of the method's arithmetic.

Every random stream but one is an SFC64 generator keyed by (seed, tag, layer, sequence, 8192-token
chunk) through numpy's SeedSequence, so any one sequence of any layer can be regenerated on its own
(the oracle checks sampled outputs of the largest workloads without generating the rest) and chunks
are drawn in parallel threads.  The ragged lengths are the first draw of numpy's default generator
seeded with the workload's seed.

Workload recipes (the pages measure end-to-end serving of real models, which is not available;
these synthetic shapes stand in for it):
  tiny      1 x 256 tokens, 1/4 heads, identity page table; K/V ~ N(0,1) with 2 channels x20.
  batch32   32 x 4096, 8/32 heads, pages permuted in a shared 8192-page pool; K/V ~ N(0,1) times a
            per-(head, channel) scale log-uniform in [0.1, 10] (separate for K and V).
  long      4 x 131072, 8/64 heads, random page table; same K/V distribution.
  ragged    64 sequences, lengths clip(rint(exp(U(ln 512, ln 32768))), 512, 32768) (seed 1004: total
            512,723), 8/64 heads, permuted pages, one appended bf16 token per sequence (same distribution).
  mixed     28 layers (FP8 at 0, 25, 26, 27), 44 x 8192, 8/32 heads; per layer K/V ~ N(0,1) (drawn
            per layer) with 2 outlier channels x20 per head; extend: a 16384-token prefix + a 2048-token chunk.
q ~ N(0,1) everywhere.  softmax scale 1/sqrt(128).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

HEAD_DIM = 128
PAGE = 16

_TAG = {"k": 1, "v": 2, "q": 3, "chan_k": 4, "chan_v": 5, "perm": 6, "lens": 7, "new_k": 8, "new_v": 9,
        "chunk_k": 10, "chunk_v": 11}


CHUNK = 8192   # tokens per independent random stream of a sequence


def _rng(seed: int, tag: str, layer: int = 0, seq: int = 0, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.SFC64(np.random.SeedSequence([seed, _TAG[tag], layer, seq, chunk])))


def _threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """fp32 numpy -> bf16 torch (CPU), round to nearest even."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def bf16_to_f32(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.float32).numpy()


@dataclass
class Workload:
    name: str
    seed: int
    batch: int
    h_kv: int
    h_q: int
    seq_lens: np.ndarray                 # cached tokens per sequence (before any append)
    chan: str = "logu"                   # "logu" or "outlier2"
    append: bool = False                 # one new token per sequence is appended by the step
    layers: int = 1
    fp8_layers: tuple = ()
    page_mode: str = "permuted"          # "identity" or "permuted"
    extra_pages: int = 0                 # unused pages in the pool (pool size = used + extra)
    sm_scale: float = 1.0 / math.sqrt(HEAD_DIM)
    extend_prefix: int = 0
    extend_chunk: int = 0
    page_table: np.ndarray = field(init=False)
    num_pages: int = field(init=False)

    def __post_init__(self):
        self.seq_lens = np.asarray(self.seq_lens, dtype=np.int64)
        assert self.seq_lens.shape == (self.batch,) and (self.seq_lens >= 1).all()
        need = (self.seq_lens + (1 if self.append else 0) + PAGE - 1) // PAGE
        self.num_pages = int(need.sum()) + self.extra_pages
        maxp = int(need.max())
        if self.page_mode == "identity":
            ids = np.arange(self.num_pages)
        else:
            ids = _rng(self.seed, "perm").permutation(self.num_pages)
        pt = np.zeros((self.batch, maxp), dtype=np.int32)
        pos = 0
        for b in range(self.batch):
            pt[b, :need[b]] = ids[pos:pos + need[b]]
            pos += need[b]
        self.page_table = pt

    # ---- shapes -------------------------------------------------------------------------------
    @property
    def group(self) -> int:
        return self.h_q // self.h_kv

    @property
    def total_lens(self) -> np.ndarray:
        """Tokens attended by the step (cached + appended)."""
        return self.seq_lens + (1 if self.append else 0)

    def is_fp8(self, layer: int) -> bool:
        return layer in self.fp8_layers

    def slots(self, b: int, start: int = 0, stop: int | None = None) -> np.ndarray:
        stop = int(self.seq_lens[b]) if stop is None else stop
        t = np.arange(start, stop, dtype=np.int64)
        return (self.page_table[b, t // PAGE].astype(np.int64) * PAGE + t % PAGE).astype(np.int32)

    # ---- random tensors -------------------------------------------------------------------------
    def channel_scale(self, which: str, layer: int = 0) -> np.ndarray:
        """fp32 [H_kv][128] per-channel multiplier of K ('k') or V ('v'), fixed over tokens."""
        r = _rng(self.seed, "chan_" + which, layer)
        if self.chan == "logu":
            return np.exp(r.uniform(math.log(0.1), math.log(10.0), size=(self.h_kv, HEAD_DIM))).astype(np.float32)
        s = np.ones((self.h_kv, HEAD_DIM), dtype=np.float32)
        for h in range(self.h_kv):
            s[h, r.choice(HEAD_DIM, size=2, replace=False)] = 20.0
        return s

    def kv_base(self, which: str, b: int, length: int | None = None, layer: int = 0) -> np.ndarray:
        """fp32 [L_b][H_kv][128] standard normals of sequence b in layer `layer` (each layer draws its own)."""
        n = int(self.seq_lens[b]) if length is None else length
        out = np.empty((n, self.h_kv, HEAD_DIM), dtype=np.float32)

        def fill(c):
            lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
            _rng(self.seed, which, layer, b, c).standard_normal(out=out[lo:hi], dtype=np.float32)

        nchunks = (n + CHUNK - 1) // CHUNK
        if nchunks == 1:
            fill(0)
        else:
            with ThreadPoolExecutor(_threads()) as ex:
                list(ex.map(fill, range(nchunks)))
        return out

    def kv(self, which: str, b: int, layer: int = 0, length: int | None = None) -> torch.Tensor:
        """bf16 [L_b][H_kv][128] cached K ('k') or V ('v') of sequence b, layer `layer` (CPU tensor):
        bf16(fp32(base normal * channel scale of the layer))."""
        x = self.kv_base(which, b, length, layer)
        x *= self.channel_scale(which, layer)[None]
        return to_bf16(x)

    def new_token(self, which: str, layer: int = 0) -> torch.Tensor:
        """bf16 [B][H_kv][128] token appended by the step (same distribution as the cache)."""
        x = _rng(self.seed, "new_" + which, layer).standard_normal((self.batch, self.h_kv, HEAD_DIM), dtype=np.float32)
        x *= self.channel_scale(which, layer)[None]
        return to_bf16(x)

    def chunk(self, which: str, layer: int = 0) -> torch.Tensor:
        """bf16 [chunk][H_kv][128] extend-chunk K or V (sequence 0)."""
        x = _rng(self.seed, "chunk_" + which, layer).standard_normal((self.extend_chunk, self.h_kv, HEAD_DIM),
                                                                     dtype=np.float32)
        x *= self.channel_scale(which, layer)[None]
        return to_bf16(x)

    def q(self, layer: int = 0) -> torch.Tensor:
        """bf16 [B][H_q][128] queries."""
        return to_bf16(_rng(self.seed, "q", layer).standard_normal((self.batch, self.h_q, HEAD_DIM), dtype=np.float32))

    def kv_bytes_nvfp4(self) -> int:
        """NVFP4 K+V bytes one decode step reads: 144 B per (token, kv head)."""
        return int(self.total_lens.sum()) * self.h_kv * 144

    def kv_bytes_fp8(self) -> int:
        return int(self.total_lens.sum()) * self.h_kv * 256


def ragged_lengths(seed: int, batch: int, lo: int = 512, hi: int = 32768) -> np.ndarray:
    """Log-uniform lengths: the first draw of numpy's default generator seeded with `seed`
    (seed 1004, 64 sequences: total 512,723 tokens, from 514 to 32,330)."""
    r = np.random.default_rng(seed)
    return np.clip(np.rint(np.exp(r.uniform(math.log(lo), math.log(hi), size=batch))), lo, hi).astype(np.int64)


def config(index: int, **override) -> Workload:
    """The five workloads by index (0-based): 0 tiny, 1 batch32, 2 long, 3 ragged, 4 mixed."""
    seed = 1001 + index
    if index == 0:
        kw = dict(name="tiny", batch=1, h_kv=1, h_q=4, seq_lens=[256], chan="outlier2", page_mode="identity")
    elif index == 1:
        kw = dict(name="batch32", batch=32, h_kv=8, h_q=32, seq_lens=[4096] * 32)
    elif index == 2:
        kw = dict(name="long", batch=4, h_kv=8, h_q=64, seq_lens=[131072] * 4)
    elif index == 3:
        kw = dict(name="ragged", batch=64, h_kv=8, h_q=64, seq_lens=ragged_lengths(seed, 64), append=True)
    elif index == 4:
        kw = dict(name="mixed", batch=44, h_kv=8, h_q=32, seq_lens=[8192] * 44, chan="outlier2", layers=28,
                  fp8_layers=(0, 25, 26, 27), extend_prefix=16384, extend_chunk=2048)
    else:
        raise ValueError(index)
    seed = override.pop("seed", seed)
    kw.update(override)
    return Workload(seed=seed, **kw)
