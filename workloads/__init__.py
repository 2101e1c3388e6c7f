"""Seeded synthetic inputs for paged and column-store decode attention.

This module draws random numbers and lays out workload *structure*: sequence
lengths, block tables dealt from a random permutation of pool blocks, segment
tables, which storage holds garbage (NaN).  It holds no attention arithmetic
and no slot addressing: where a new token goes is given as its logical
position inside its sequence, and each consumer (the HIP path's caller, the
CPU oracle) turns that into a physical slot its own way.

Every tensor is drawn with a ``torch.Generator`` seeded from the caller's
seed: fp32 N(0, 1), then rounded to nearest-even into the workload dtype.
Large pools are drawn on the device they are going to live on; the oracle
always receives the exact bits by copying back.

The shapes follow the five workloads of the hot path: a tiny fp32 paged decode,
a 42-layer bucketed single-sequence decode, a 64-sequence batched paged decode
over a 40000-block pool, a 32-column ring store with mixed decode and chunked
prefill segments, and a long-context (32K/64K) head_dim-256 pass with 16-token
draft blocks.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

BLOCK = 16
GARBAGE_BLOCK_ID = 0x7FFFFFFF  # filler for block-table entries past a sequence's blocks


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def randn(shape, dtype, seed: int, device="cpu") -> torch.Tensor:
    """fp32 N(0,1) from the seed, rounded to nearest-even into ``dtype``."""
    g = _gen(seed, device)
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    return x.to(dtype)


def _rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(int(seed))


@dataclass
class PagedInputs:
    """One call's inputs over a paged pool ``[num_blocks, 16, Hkv, D]``.

    Sequence ``b`` owns query rows ``cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1``
    and has ``seqused_k[b]`` keys, the new ones included.  ``new_pos[t]`` /
    ``new_seq[t]`` say which logical position of which sequence the ``t``-th
    row of ``k_new``/``v_new`` belongs to (the last ``q_len`` positions).
    """
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    block_table: torch.Tensor      # int32 [num_seqs, max_blocks]
    seqused_k: torch.Tensor        # int32 [num_seqs]
    cu_seqlens_q: torch.Tensor     # int32 [num_seqs + 1]
    new_pos: torch.Tensor          # int64 [total_q]
    new_seq: torch.Tensor          # int32 [total_q]
    q_heads: int
    kv_heads: int
    head_dim: int
    scale: float
    causal: bool
    window: int
    max_seqlen_q: int
    max_seqlen_k: int
    name: str = ""

    @property
    def num_seqs(self) -> int:
        return int(self.seqused_k.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])


@dataclass
class ColumnInputs:
    """One call's inputs over a column store ``[rows, cols, Hkv, D]``.

    ``seq_info[s] = (q_start, q_len, col, kv_end)``.  Query rows that no
    segment covers have ``new_pos == -1`` (nothing to append).
    """
    q: torch.Tensor
    k_store: torch.Tensor
    v_store: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    seq_info: torch.Tensor         # int32 [S, 4]
    new_pos: torch.Tensor          # int64 [total_q], -1 where uncovered
    new_col: torch.Tensor          # int32 [total_q], -1 where uncovered
    q_heads: int
    kv_heads: int
    head_dim: int
    scale: float
    causal: bool
    window: int
    max_seqlen_q: int
    name: str = ""

    @property
    def rows(self) -> int:
        return int(self.k_store.shape[0])

    @property
    def cols(self) -> int:
        return int(self.k_store.shape[1])

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_segments(self) -> int:
        return int(self.seq_info.shape[0])


def _nan_like(dtype):
    return float("nan")


def deal_block_tables(lengths, num_blocks: int, max_blocks: int, seed: int,
                      identity: bool = False):
    """Deal distinct pool blocks to sequences in order from one random permutation.

    Sequence ``b`` needs ``ceil(lengths[b] / 16)`` blocks.  Returns the int32
    table (tails filled with ``GARBAGE_BLOCK_ID``) and the bool mask of pool
    blocks that were dealt.
    """
    need = [(int(n) + BLOCK - 1) // BLOCK for n in lengths]
    if sum(need) > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {sum(need)}")
    if max(need + [0]) > max_blocks:
        raise ValueError("a sequence needs more blocks than the table width")
    perm = np.arange(num_blocks) if identity else _rng(seed).permutation(num_blocks)
    table = np.full((len(lengths), max_blocks), GARBAGE_BLOCK_ID, dtype=np.int64)
    used = np.zeros(num_blocks, dtype=bool)
    k = 0
    for b, nb in enumerate(need):
        table[b, :nb] = perm[k:k + nb]
        used[perm[k:k + nb]] = True
        k += nb
    return torch.from_numpy(table.astype(np.int32)), torch.from_numpy(used)


def paged_inputs(*, seed: int, lengths, q_lens, q_heads: int, kv_heads: int,
                 head_dim: int, dtype, num_blocks: int, max_blocks: int,
                 causal: bool = False, window: int = 0, identity: bool = False,
                 nan_unused: bool = True, scale: Optional[float] = None,
                 device="cpu", max_seqlen_k: Optional[int] = None,
                 name: str = "") -> PagedInputs:
    lengths = [int(x) for x in lengths]
    q_lens = [int(x) for x in q_lens]
    assert len(lengths) == len(q_lens)
    table, used = deal_block_tables(lengths, num_blocks, max_blocks, seed + 1, identity)
    total_q = sum(q_lens)
    q = randn((total_q, q_heads, head_dim), dtype, seed + 2, device)
    k_cache = randn((num_blocks, BLOCK, kv_heads, head_dim), dtype, seed + 3, device)
    v_cache = randn((num_blocks, BLOCK, kv_heads, head_dim), dtype, seed + 4, device)
    if nan_unused:
        unused = (~used).to(device)
        k_cache[unused] = float("nan")
        v_cache[unused] = float("nan")
    k_new = randn((total_q, kv_heads, head_dim), dtype, seed + 5, device)
    v_new = randn((total_q, kv_heads, head_dim), dtype, seed + 6, device)
    cu = np.zeros(len(q_lens) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(q_lens)
    new_pos = np.concatenate([np.arange(n - L, n) for n, L in zip(lengths, q_lens)] or [np.zeros(0)])
    new_seq = np.concatenate([np.full(L, b) for b, L in enumerate(q_lens)] or [np.zeros(0)])
    return PagedInputs(
        q=q, k_cache=k_cache, v_cache=v_cache, k_new=k_new, v_new=v_new,
        block_table=table.to(device),
        seqused_k=torch.tensor(lengths, dtype=torch.int32, device=device),
        cu_seqlens_q=torch.from_numpy(cu.astype(np.int32)).to(device),
        new_pos=torch.from_numpy(new_pos.astype(np.int64)).to(device),
        new_seq=torch.from_numpy(new_seq.astype(np.int32)).to(device),
        q_heads=q_heads, kv_heads=kv_heads, head_dim=head_dim,
        scale=(1.0 / float(np.sqrt(head_dim))) if scale is None else float(scale),
        causal=bool(causal), window=int(window),
        max_seqlen_q=max(q_lens + [1]),
        max_seqlen_k=int(max_seqlen_k) if max_seqlen_k is not None else max_blocks * BLOCK,
        name=name)


@dataclass
class PrefixInputs:
    """A dense prefill cache ``[B, Hkv, S, D]`` and a paged pool to copy it into.

    ``block_table`` deals each sequence the blocks of its first ``n`` positions
    from a random permutation of the pool (or in order with ``identity``);
    pool blocks no sequence owns hold NaN.  ``bad_entries`` lists
    ``(sequence, table column, value)`` entries overwritten with ids outside the
    pool.
    """
    k_src: torch.Tensor
    v_src: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    n: int


def prefix_inputs(*, seed: int, batch: int, kv_heads: int, head_dim: int, src_len: int, n: int,
                  num_blocks: int, max_blocks: int, dtype, device="cpu", identity: bool = False,
                  bad_entries=()) -> PrefixInputs:
    table, used = deal_block_tables([n] * batch, num_blocks, max_blocks, seed + 1, identity)
    for b, col, val in bad_entries:
        table[b, col] = int(val)
    k_src = randn((batch, kv_heads, src_len, head_dim), dtype, seed + 2, device)
    v_src = randn((batch, kv_heads, src_len, head_dim), dtype, seed + 3, device)
    k_cache = randn((num_blocks, BLOCK, kv_heads, head_dim), dtype, seed + 4, device)
    v_cache = randn((num_blocks, BLOCK, kv_heads, head_dim), dtype, seed + 5, device)
    unused = (~used).to(device)
    k_cache[unused] = float("nan")
    v_cache[unused] = float("nan")
    return PrefixInputs(k_src=k_src, v_src=v_src, k_cache=k_cache, v_cache=v_cache,
                        block_table=table.to(device), n=int(n))


def column_inputs(*, seed: int, rows: int, cols: int, q_lens, kv_ends, total_q: int,
                  q_heads: int, kv_heads: int, head_dim: int, dtype, causal: bool,
                  window: int, scale: Optional[float] = None, device="cpu",
                  nan_unwritten: bool = True, name: str = "") -> ColumnInputs:
    """Segments get distinct columns (a random permutation) and are packed into
    ``total_q`` query rows in random order with random gaps."""
    q_lens = [int(x) for x in q_lens]
    kv_ends = [int(x) for x in kv_ends]
    S = len(q_lens)
    assert S == len(kv_ends) and S <= cols and sum(q_lens) <= total_q
    r = _rng(seed + 11)
    col_of = r.permutation(cols)[:S]
    order = r.permutation(S)
    spare = total_q - sum(q_lens)
    cuts = np.sort(r.integers(0, spare + 1, size=S))
    gaps = np.diff(np.concatenate([[0], cuts]))          # S gaps, the rest is tail
    info = np.zeros((S, 4), dtype=np.int64)
    new_pos = np.full(total_q, -1, dtype=np.int64)
    new_col = np.full(total_q, -1, dtype=np.int64)
    at = 0
    for k, s in enumerate(order):
        at += int(gaps[k])
        L, E = q_lens[s], kv_ends[s]
        info[s] = (at, L, col_of[s], E)
        new_pos[at:at + L] = np.arange(E - L, E)
        new_col[at:at + L] = col_of[s]
        at += L
    q = randn((total_q, q_heads, head_dim), dtype, seed + 12, device)
    k_store = randn((rows, cols, kv_heads, head_dim), dtype, seed + 13, device)
    v_store = randn((rows, cols, kv_heads, head_dim), dtype, seed + 14, device)
    if nan_unwritten:
        # A column that has taken E < rows writes holds data in its first E rows only.
        for s in range(S):
            E = kv_ends[s]
            if E < rows:
                k_store[max(E, 0):, col_of[s]] = float("nan")
                v_store[max(E, 0):, col_of[s]] = float("nan")
        for c in range(cols):
            if c not in set(int(x) for x in col_of):
                k_store[:, c] = float("nan")
                v_store[:, c] = float("nan")
    k_new = randn((total_q, kv_heads, head_dim), dtype, seed + 15, device)
    v_new = randn((total_q, kv_heads, head_dim), dtype, seed + 16, device)
    return ColumnInputs(
        q=q, k_store=k_store, v_store=v_store, k_new=k_new, v_new=v_new,
        seq_info=torch.from_numpy(info.astype(np.int32)).to(device),
        new_pos=torch.from_numpy(new_pos).to(device),
        new_col=torch.from_numpy(new_col.astype(np.int32)).to(device),
        q_heads=q_heads, kv_heads=kv_heads, head_dim=head_dim,
        scale=(1.0 / float(np.sqrt(head_dim))) if scale is None else float(scale),
        causal=bool(causal), window=int(window), max_seqlen_q=max(q_lens + [1]),
        name=name)


# --------------------------------------------------------------------------
# The five workloads.  Seeds are 194000 + k for workload k.
# --------------------------------------------------------------------------

SEED_BASE = 194000
C2_BUCKETS = (512, 1024, 2048, 4096, 8192)


def c1_tiny(device="cpu") -> PagedInputs:
    """1 sequence, Hq 4 / Hkv 2, D 64, fp32, 512-token bucket (32 blocks),
    identity table, 100 live keys, the new token is key 99; slots 100.. NaN."""
    seed = SEED_BASE + 1
    inp = paged_inputs(seed=seed, lengths=[100], q_lens=[1], q_heads=4, kv_heads=2,
                       head_dim=64, dtype=torch.float32, num_blocks=32, max_blocks=32,
                       identity=True, nan_unused=False, device=device, scale=1.0 / 8.0,
                       max_seqlen_k=512, name="tiny fp32 paged decode")
    # Under the identity table flat slot s holds logical key s: the tail past
    # the 100 live keys is stale storage.
    inp.k_cache.view(-1, 2, 64)[100:] = float("nan")
    inp.v_cache.view(-1, 2, 64)[100:] = float("nan")
    return inp


@dataclass
class DecodeModel:
    """Shapes of the 42-layer single-sequence bucketed decode."""
    layers: int = 42
    q_heads: int = 32
    kv_heads: int = 8
    head_dim: int = 128
    dtype: torch.dtype = torch.bfloat16
    buckets: tuple = C2_BUCKETS


def c2_step_inputs(steps: int, model: DecodeModel = DecodeModel(), device="cpu",
                   seed: int = SEED_BASE + 2) -> torch.Tensor:
    """Per-step q, k_new, v_new for every layer: ``[steps, layers, Hq + 2 Hkv, D]``."""
    m = model
    return randn((steps, m.layers, m.q_heads + 2 * m.kv_heads, m.head_dim), m.dtype, seed, device)


def c3_lengths(seed: int = SEED_BASE + 3, num_seqs: int = 64, max_len: int = 8192):
    return [int(x) for x in _rng(seed).integers(1, max_len + 1, size=num_seqs)]


def c3_batched(device="cpu", num_seqs: int = 64, max_len: int = 8192,
               num_blocks: int = 40000, seed: int = SEED_BASE + 3) -> PagedInputs:
    lengths = c3_lengths(seed, num_seqs, max_len)
    return paged_inputs(seed=seed, lengths=lengths, q_lens=[1] * num_seqs, q_heads=32,
                        kv_heads=8, head_dim=128, dtype=torch.bfloat16,
                        num_blocks=num_blocks, max_blocks=max_len // BLOCK,
                        device=device, max_seqlen_k=max_len, name="batched paged decode")


def c4_segments(seed: int = SEED_BASE + 4, n_decode: int = 24, n_prefill: int = 8,
                total_q: int = 4096, rows: int = 8192, lo: int = 64, hi: int = 512):
    """q_len 1 for the decode segments and U[lo, hi] for the chunked-prefill ones
    (redrawn until they fit ``total_q``); kv_end U[1, 2*rows] for decode and
    start + q_len with start U[0, 2*rows - q_len] for prefill, so rings wrap."""
    r = _rng(seed)
    while True:
        pre = [int(x) for x in r.integers(lo, hi + 1, size=n_prefill)]
        if sum(pre) + n_decode <= total_q:
            break
    q_lens = [1] * n_decode + pre
    ends = [int(x) for x in r.integers(1, 2 * rows + 1, size=n_decode)]
    for L in pre:
        start = int(r.integers(0, 2 * rows - L + 1))
        ends.append(start + L)
    return q_lens, ends


def c4_column(device="cpu", rows: int = 8192, cols: int = 32, total_q: int = 4096,
              window: int = 4096, n_decode: int = 24, n_prefill: int = 8,
              lo: int = 64, hi: int = 512, seed: int = SEED_BASE + 4) -> ColumnInputs:
    q_lens, ends = c4_segments(seed, n_decode, n_prefill, total_q, rows, lo, hi)
    return column_inputs(seed=seed, rows=rows, cols=cols, q_lens=q_lens, kv_ends=ends,
                         total_q=total_q, q_heads=32, kv_heads=8, head_dim=128,
                         dtype=torch.bfloat16, causal=True, window=window, device=device,
                         name="column store, decode + chunked prefill")


def c5_long(device="cpu", lengths=(32768, 65536, 32768, 65536), draft: int = 16,
            num_blocks: int = 16384, seed: int = SEED_BASE + 5, decode: bool = False,
            q_heads: int = 64, kv_heads: int = 8, head_dim: int = 256) -> PagedInputs:
    """Draft verify (non-causal 16-token blocks) or, with ``decode``, the
    single-token causal pass over the same keys (no new tokens)."""
    mb = max(lengths) // BLOCK
    inp = paged_inputs(seed=seed, lengths=list(lengths),
                       q_lens=[1 if decode else draft] * len(lengths),
                       q_heads=q_heads, kv_heads=kv_heads, head_dim=head_dim,
                       dtype=torch.bfloat16, num_blocks=num_blocks, max_blocks=mb,
                       causal=decode, device=device, max_seqlen_k=max(lengths),
                       name="long-context decode" if decode else "long-context draft verify")
    return inp
