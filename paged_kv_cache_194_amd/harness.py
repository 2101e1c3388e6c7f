"""Bucketed paged decode cache and a captured decode step per bucket.

vLLM-Omni paged_decode (SenseNova-U1): PagedDecodeCache keeps one set of
per-layer K/V buffers sized to a bucket behind an identity block table; the
live length sits in a device tensor, so a captured graph is replayed unchanged
for every length in the bucket; crossing a bucket edge reallocates (`grow`,
built in locals and published in one step) and bumps `generation`, which keys
the captures of DecodeGraphRunner.

load_prefix / from_dynamic_cache bring a prefill cache in and
to_dynamic_cache hands the decoded prefix back out, each layer one library
copy (pkv.prefix_import / pkv.prefix_export).

Here the whole step of a layer -- append this token's K/V at position
length-1 and attend over the live prefix -- is one library call
(pkv.paged_decode_attn with k_new/v_new): the write slot is derived on the
device from seqused_k and the block table, so seqused_k is the only tensor a
step changes.
"""
from __future__ import annotations

from typing import Callable, Dict, List, Optional, Sequence, Tuple

import torch

from . import BLOCK_SIZE, attn_workspace_bytes, paged_decode_attn, prefix_export, prefix_import

BUCKETS = (512, 1024, 2048, 4096, 8192)
TAIL_STEP = 2048

_GRAPH_POOL = None


def shared_graph_pool():
    """One memory pool for every capture.  A private pool per capture table is
    never handed back, and tables are rebuilt whenever the cache reallocates
    (the pages measured about 40 MiB of growth per request that way)."""
    global _GRAPH_POOL
    if _GRAPH_POOL is None:
        _GRAPH_POOL = torch.cuda.graph_pool_handle()
    return _GRAPH_POOL


def bucket_for(length: int) -> int:
    """Smallest bucket that holds ``length`` tokens; past the list, whole
    TAIL_STEP increments (each bucket costs a capture, so no per-block steps)."""
    for b in BUCKETS:
        if length <= b:
            return b
    over = length - BUCKETS[-1]
    return BUCKETS[-1] + ((over + TAIL_STEP - 1) // TAIL_STEP) * TAIL_STEP


class PagedDecodeCache:
    """Per-layer paged K/V ``[bucket/16, 16, Hkv, D]`` for single-sequence decode."""

    def __init__(self, num_layers: int, q_heads: int, kv_heads: int, head_dim: int, length: int,
                 device, dtype, num_splits: int = 0,
                 alloc: Callable[..., torch.Tensor] = torch.zeros):
        self.num_layers = num_layers
        self.q_heads = q_heads
        self.kv_heads = kv_heads
        self.head_dim = head_dim
        self.device = torch.device(device)
        self.dtype = dtype
        self.num_splits = num_splits
        self._alloc = alloc
        self.bucket = bucket_for(length)
        self.k, self.v, self.block_table, self.workspace = self._buffers(self.bucket)
        self.seqused = torch.zeros(1, dtype=torch.int32, device=self.device)
        self._length = 0
        self.generation = 0

    def _buffers(self, bucket: int):
        nblocks = bucket // BLOCK_SIZE
        shape = (nblocks, BLOCK_SIZE, self.kv_heads, self.head_dim)
        k = [self._alloc(shape, device=self.device, dtype=self.dtype) for _ in range(self.num_layers)]
        v = [self._alloc(shape, device=self.device, dtype=self.dtype) for _ in range(self.num_layers)]
        table = torch.arange(nblocks, device=self.device, dtype=torch.int32).unsqueeze(0)
        ws_bytes = attn_workspace_bytes(1, 1, bucket, self.q_heads, self.kv_heads, self.head_dim,
                                        self.num_splits)
        ws = self._alloc((max(ws_bytes, 1),), device=self.device, dtype=torch.uint8)
        return k, v, table, ws

    @property
    def length(self) -> int:
        return self._length

    def set_length(self, n: int) -> None:
        """The step about to run holds ``n`` live keys, its own included."""
        if n > self.bucket:
            raise ValueError(f"length {n} exceeds bucket {self.bucket}; grow first")
        self._length = n
        self.seqused.fill_(n)

    def reusable_for(self, num_layers, kv_heads, head_dim, dtype, length) -> bool:
        return (len(self.k) == num_layers and self.kv_heads == kv_heads
                and self.head_dim == head_dim and self.dtype == dtype
                and bucket_for(length) <= self.bucket)

    def grow(self, length: int) -> bool:
        """Move to the bucket for ``length`` keeping the stored prefix.  New
        buffers are built in locals and published together with generation+1,
        so a failure part way leaves the old buffers and generation in place."""
        new_bucket = bucket_for(length)
        if new_bucket == self.bucket:
            return False
        k, v, table, ws = self._buffers(new_bucket)
        n = self._length
        H, D = self.kv_heads, self.head_dim
        for i in range(self.num_layers):
            k[i].view(-1, H, D)[:n].copy_(self.k[i].view(-1, H, D)[:n])
            v[i].view(-1, H, D)[:n].copy_(self.v[i].view(-1, H, D)[:n])
        self.k, self.v, self.block_table, self.workspace, self.bucket = k, v, table, ws, new_bucket
        self.generation += 1
        self.set_length(n)
        return True

    def load_prefix(self, keys: Sequence[Optional[torch.Tensor]],
                    values: Sequence[Optional[torch.Tensor]]) -> bool:
        """Copy a prefill cache (per layer ``[1, Hkv, S, D]``) into slots
        ``[:S]`` and make S the live length; the tail keeps stale data.
        Returns False when the prefill cache is empty."""
        if not keys or keys[0] is None:
            return False
        if len(keys) != self.num_layers or len(values) != self.num_layers:
            raise ValueError("one prefill K and V per layer expected")
        prefix = keys[0].shape[2]
        if prefix > self.bucket:
            raise ValueError(f"prefix {prefix} exceeds bucket {self.bucket}; grow first")
        for i in range(self.num_layers):
            # The last layer's launch also publishes the live length.
            prefix_import(self.k[i], self.v[i], keys[i], values[i], self.block_table, prefix,
                          seqused_k=self.seqused if i == self.num_layers - 1 else None)
        self._length = prefix
        return True

    @classmethod
    def from_dynamic_cache(cls, keys, values, q_heads: int, device, dtype, min_length: int = 0,
                           **kw) -> Optional["PagedDecodeCache"]:
        """A cache whose bucket holds the prefill prefix plus the next token
        (at least ``min_length``), loaded with that prefix; None if empty."""
        if not keys or keys[0] is None:
            return None
        _, kv_heads, prefix, head_dim = keys[0].shape
        obj = cls(len(keys), q_heads, kv_heads, head_dim, max(prefix + 1, min_length), device, dtype,
                  **kw)
        obj.load_prefix(keys, values)
        return obj

    def to_dynamic_cache(self) -> List[Tuple[torch.Tensor, torch.Tensor]]:
        """Per layer, slots ``[:length]`` copied out as contiguous
        ``[1, Hkv, length, D]`` K and V (the hand-off to an ordinary cache)."""
        n, H, D = self._length, self.kv_heads, self.head_dim
        out = []
        for i in range(self.num_layers):
            k = torch.empty((1, H, n, D), device=self.device, dtype=self.dtype)
            v = torch.empty((1, H, n, D), device=self.device, dtype=self.dtype)
            prefix_export(k, v, self.k[i], self.v[i], self.block_table)
            out.append((k, v))
        return out

    def attend(self, layer: int, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
               out: torch.Tensor) -> torch.Tensor:
        """Append this step's ``k_new``/``v_new`` ``[1, Hkv, D]`` at position
        length-1 and attend ``q`` ``[1, Hq, D]`` over the live prefix."""
        return paged_decode_attn(out, q, self.k[layer], self.v[layer], self.block_table,
                                 self.seqused, max_seqlen_k=self.bucket, num_splits=self.num_splits,
                                 workspace=self.workspace, k_new=k_new, v_new=v_new)


class DecodeStepGraph:
    """One captured decode step (all layers) per (bucket, generation).

    ``inputs`` ``[layers, Hq + 2 Hkv, D]`` holds each layer's q, k_new, v_new
    for the step; ``out`` ``[layers, Hq, D]`` receives the attention outputs.
    """

    def __init__(self, cache: PagedDecodeCache, inputs: torch.Tensor, out: torch.Tensor):
        self.cache = cache
        self.inputs = inputs
        self.out = out
        self._graphs: Dict[Tuple[int, int], torch.cuda.CUDAGraph] = {}
        self.captures = 0

    def forward(self) -> None:
        c = self.cache
        hq, hkv = c.q_heads, c.kv_heads
        for layer in range(c.num_layers):
            x = self.inputs[layer]
            c.attend(layer, x[:hq].unsqueeze(0), x[hq:hq + hkv].unsqueeze(0),
                     x[hq + hkv:hq + 2 * hkv].unsqueeze(0), self.out[layer].unsqueeze(0))

    def _capture(self, key) -> torch.cuda.CUDAGraph:
        # Warm-ups on a side stream rewrite the same slot with the same values.
        side = torch.cuda.Stream(device=self.cache.device)
        side.wait_stream(torch.cuda.current_stream(self.cache.device))
        with torch.cuda.stream(side):
            for _ in range(3):
                self.forward()
        torch.cuda.current_stream(self.cache.device).wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, pool=shared_graph_pool()):
            self.forward()
        self.captures += 1
        self._graphs = {k: g for k, g in self._graphs.items() if k[1] == self.cache.generation}
        self._graphs[key] = graph
        return graph

    def step(self) -> torch.Tensor:
        key = (self.cache.bucket, self.cache.generation)
        graph = self._graphs.get(key) or self._capture(key)
        graph.replay()
        return self.out


class DecodeSession:
    """Decode requests served one after another over one reusable paged cache.

    vLLM-Omni paged_decode: one set of buffers behind an identity block table,
    reused by whichever request fits them (``reusable_for``), so the captures
    bound to those buffers survive from request to request.  Per request:
    ``begin`` brings the prefill cache in -- ``load_prefix`` into the current
    cache when it fits, else a new cache (``from_dynamic_cache``) with a new
    capture table; each ``step`` advances the length by one token (growing at
    a bucket edge, which bumps the generation and so the capture key), stages
    the token's per-layer q / k_new / v_new and replays; ``end`` hands the K/V
    back (``to_dynamic_cache``).  ``release`` drops buffers and captures.
    """

    def __init__(self, num_layers: int, q_heads: int, kv_heads: int, head_dim: int, device,
                 dtype, num_splits: int = 0):
        self.num_layers = num_layers
        self.q_heads = q_heads
        self.kv_heads = kv_heads
        self.head_dim = head_dim
        self.device = torch.device(device)
        self.dtype = dtype
        self.num_splits = num_splits
        self.inputs = torch.zeros((num_layers, q_heads + 2 * kv_heads, head_dim), device=self.device,
                                  dtype=dtype)
        self.out = torch.zeros((num_layers, q_heads, head_dim), device=self.device, dtype=dtype)
        self.cache: Optional[PagedDecodeCache] = None
        self.runner: Optional[DecodeStepGraph] = None
        self.requests = 0
        self.reused = 0

    def begin(self, keys: Sequence[Optional[torch.Tensor]],
              values: Sequence[Optional[torch.Tensor]]) -> PagedDecodeCache:
        """Start a request from its prefill cache (per layer ``[1, Hkv, S, D]``;
        an empty one starts from length 0)."""
        prefix = keys[0].shape[2] if keys and keys[0] is not None else 0
        c = self.cache
        if c is not None and c.reusable_for(self.num_layers, self.kv_heads, self.head_dim, self.dtype,
                                            prefix + 1):
            if not c.load_prefix(keys, values):
                c.set_length(0)
            self.reused += 1
        else:
            self.release()
            c = PagedDecodeCache.from_dynamic_cache(keys, values, self.q_heads, self.device, self.dtype,
                                                    num_splits=self.num_splits)
            if c is None:
                c = PagedDecodeCache(self.num_layers, self.q_heads, self.kv_heads, self.head_dim, 1,
                                     self.device, self.dtype, num_splits=self.num_splits)
            self.cache = c
            self.runner = DecodeStepGraph(c, self.inputs, self.out)
        self.requests += 1
        return c

    def step(self, token_inputs: torch.Tensor) -> torch.Tensor:
        """One token: ``token_inputs`` ``[layers, Hq + 2 Hkv, D]`` (q, k_new,
        v_new of every layer).  Returns the static ``[layers, Hq, D]`` output."""
        c = self.cache
        if c is None or self.runner is None:
            raise RuntimeError("begin a request first")
        n = c.length + 1
        if n > c.bucket:
            c.grow(n)
        c.set_length(n)
        self.inputs.copy_(token_inputs)
        return self.runner.step()

    def end(self) -> List[Tuple[torch.Tensor, torch.Tensor]]:
        if self.cache is None:
            raise RuntimeError("no request in progress")
        return self.cache.to_dynamic_cache()

    def release(self) -> None:
        """Drop the buffers and every capture bound to them."""
        self.runner = None
        self.cache = None
