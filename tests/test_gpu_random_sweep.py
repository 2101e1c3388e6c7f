"""GPU parity over seeded random call shapes: head_dim 64/128/256, GQA groups
1..16, bf16 and fp32, paged varlen (2..16 sequences, up to 9000 keys and 100
query rows in the wide set) and column-store calls,
causal or not, windows, left-padding bounds and split counts drawn per case.
Each case picks its own kernels through the library's routing (vector path,
matrix-core shapes, fp32 row mode) and is compared, every output element,
with the fp64 oracle; rows no unit covers must come back exactly 0."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_cache_194_amd as pkv
import workloads
from helpers import check_close, oracle_column, oracle_paged

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N_CASES = 40
N_WIDE = 60


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pkv.lib()


def _draw(case: int, wide: bool = False) -> dict:
    """Small shapes, or (wide) up to 16 units of up to 9000 keys and 100 query rows."""
    r = np.random.default_rng((15000 if wide else 5000) + case)
    D = int(r.choice([64, 128, 256]))
    fp32 = bool(r.random() < 0.25)
    groups = [1, 2, 4, 8] if fp32 else [1, 2, 4, 8, 16]
    G = int(r.choice(groups))
    hkv = int(r.choice([1, 2, 4, 8]))
    n = int(r.integers(2, 17 if wide else 7))         # sequences or segments (never one)
    lq_max = int(r.choice([1, 1, 4, 16, 40, 100] if wide else [1, 1, 4, 16, 40]))
    q_lens = [int(x) for x in r.integers(1, lq_max + 1, size=n)]
    lengths = [int(x) for x in r.integers(0, 9000 if wide else 1500, size=n)]
    lengths = [max(E, L) for E, L in zip(lengths, q_lens)]
    return dict(D=D, dtype=torch.float32 if fp32 else torch.bfloat16, G=G, hkv=hkv, n=n, q_lens=q_lens,
                lengths=lengths, causal=bool(r.random() < 0.7), window=int(r.choice([0, 0, 100, 700])),
                splits=int(r.choice([0, 0, 1, 3, 7])), column=bool(r.random() < 0.35),
                pad=bool(r.random() < 0.3), wrap=int(r.choice([0, 2500])),
                rows=4096 if wide else 2048, cols=16 if wide else 8,
                seed=(16000 if wide else 6000) + 17 * case)


def _pads(c: dict, ends):
    """Left-padding bounds anywhere in [0, E) per unit, or none."""
    if not c["pad"]:
        return None, None
    r = np.random.default_rng(c["seed"] + 1)
    ks_np = np.array([int(r.integers(0, max(1, E))) for E in ends], dtype=np.int64)
    return torch.tensor(ks_np, dtype=torch.int32, device=DEV), ks_np


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_call_shape(case):
    _run(_draw(case), case)


@pytest.mark.parametrize("case", range(N_WIDE))
def test_random_call_shape_wide(case):
    _run(_draw(case, wide=True), case)


def _run(c: dict, case: int):
    name = "f32" if c["dtype"] == torch.float32 else "bf16"
    what = f"case {case}: {c}"
    hq = c["G"] * c["hkv"]
    if c["column"]:
        # A window lets a segment's keys run past the ring (rows >= window +
        # max_seqlen_q - 1 keeps every visible key stored); without one the
        # ring holds every key, E <= rows.
        rows = c["rows"]
        ends = [E + c["wrap"] if c["window"] > 0 else min(E, rows) for E in c["lengths"]]
        inp = workloads.column_inputs(seed=c["seed"], rows=rows, cols=c["cols"], q_lens=c["q_lens"], kv_ends=ends,
                                      total_q=sum(c["q_lens"]) + 13, q_heads=hq, kv_heads=c["hkv"],
                                      head_dim=c["D"], dtype=c["dtype"], causal=c["causal"], window=c["window"],
                                      device=DEV)
        max_k = (c["window"] + inp.max_seqlen_q - 1) if c["window"] > 0 else max(ends)
        ks, ks_np = _pads(c, ends)
        out = torch.full_like(inp.q, float("nan"))
        pkv.varlen_attn(out, inp.q, inp.k_store, inp.v_store, seq_info=inp.seq_info,
                        max_seqlen_q=inp.max_seqlen_q, max_seqlen_k=max_k, softmax_scale=inp.scale,
                        causal=c["causal"], window=c["window"], num_splits=c["splits"], kv_start=ks)
        torch.cuda.synchronize()
        ref = oracle_column(inp, **({} if ks_np is None else dict(kv_start=ks_np)))
        covered = torch.from_numpy(inp.new_pos.cpu().numpy() >= 0).to(DEV)
        assert (out[~covered] == 0).all(), what
    else:
        nb = sum((E + 15) // 16 for E in c["lengths"]) + 8
        mb = max((E + 15) // 16 for E in c["lengths"]) + 2
        inp = workloads.paged_inputs(seed=c["seed"], lengths=c["lengths"], q_lens=c["q_lens"], q_heads=hq,
                                     kv_heads=c["hkv"], head_dim=c["D"], dtype=c["dtype"], num_blocks=nb,
                                     max_blocks=mb, causal=c["causal"], window=c["window"], device=DEV)
        ks, ks_np = _pads(c, c["lengths"])
        out = torch.full_like(inp.q, float("nan"))
        pkv.varlen_attn(out, inp.q, inp.k_cache, inp.v_cache, cu_seqlens_q=inp.cu_seqlens_q,
                        seqused_k=inp.seqused_k, block_table=inp.block_table, max_seqlen_q=inp.max_seqlen_q,
                        max_seqlen_k=inp.max_seqlen_k, softmax_scale=inp.scale, causal=c["causal"],
                        window=c["window"], num_splits=c["splits"], kv_start=ks)
        torch.cuda.synchronize()
        ref = oracle_paged(inp, **({} if ks_np is None else dict(kv_start=ks_np)))
    check_close(out, ref, name, what)
