"""GPU parity of the balanced split-K deal of the vector path.

With several single-row units and several splits, the work groups of a kv head
share one blocks-per-split figure computed on the device from every unit's live
length, so a long unit takes many work groups and a short or empty one takes
one.  These cases exercise the deal where it can go wrong: more units than a
wave has lanes (each lane then sums several units), empty units beside long
ones, spare slots, multi-row units mixed in (they are not the vector path's),
the fused append, and a window.  Every output row is compared with the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_194_amd as pkv
import workloads
from helpers import check_close, oracle_paged, raw

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pkv.lib()


def _lengths(seed, n, zeros, long_len, n_long, short_max):
    rng = np.random.default_rng(seed)
    lengths = rng.integers(1, short_max + 1, size=n)
    lengths[rng.choice(n, zeros, replace=False)] = 0
    longs = rng.choice(np.flatnonzero(lengths > 0), n_long, replace=False)
    lengths[longs] = long_len
    return [int(x) for x in lengths]


def _decode(inp, splits, **kw):
    out = torch.full_like(inp.q, float("nan"))
    pkv.paged_decode_attn(out, inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.seqused_k,
                          max_seqlen_k=inp.max_seqlen_k, softmax_scale=inp.scale, causal=inp.causal,
                          window=inp.window, num_splits=splits, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("splits", [2, 5, 16])
def test_many_units_with_empties_and_long_ones(splits):
    """200 units (three or four per lane of the dealing wave), 30 empty, 3 of
    3000 keys among short ones of 1..200 keys; G 4, D 128, bf16."""
    lengths = _lengths(700 + splits, 200, 30, 3000, 3, 200)
    inp = workloads.paged_inputs(seed=710, lengths=lengths, q_lens=[1] * 200, q_heads=32, kv_heads=8,
                                 head_dim=128, dtype=torch.bfloat16, num_blocks=4000, max_blocks=200,
                                 device=DEV)
    out = _decode(inp, splits)
    ref = oracle_paged(inp)
    check_close(out, ref, "bf16", f"200 units splits={splits}")
    empty = torch.tensor([x == 0 for x in lengths], device=DEV)
    assert (out[empty] == 0).all()


def test_one_long_unit_takes_most_work_groups():
    """Units of 0, 0, 5000, 0, 1 keys at 16 splits: the long unit is dealt
    nearly all 80 work groups; fp32, G 2, D 64."""
    lengths = [0, 0, 5000, 0, 1]
    inp = workloads.paged_inputs(seed=720, lengths=lengths, q_lens=[1] * 5, q_heads=4, kv_heads=2,
                                 head_dim=64, dtype=torch.float32, num_blocks=330, max_blocks=320,
                                 device=DEV)
    for splits in (16, 3):
        out = _decode(inp, splits)
        check_close(out, oracle_paged(inp), "f32", f"one long unit splits={splits}")
        assert (out[[0, 1, 3]] == 0).all()


def test_window_with_balanced_deal():
    lengths = _lengths(730, 90, 10, 2500, 4, 200)
    inp = workloads.paged_inputs(seed=731, lengths=lengths, q_lens=[1] * 90, q_heads=16, kv_heads=4,
                                 head_dim=256, dtype=torch.bfloat16, num_blocks=2000, max_blocks=160,
                                 window=300, causal=True, device=DEV)
    check_close(_decode(inp, 4), oracle_paged(inp), "bf16", "window 300, 90 units")


def test_fused_append_with_balanced_deal():
    """70 units, the new token of each appended through its block table inside
    the attention call; append bit-exact, attention within tolerance."""
    lengths = _lengths(740, 70, 0, 2000, 2, 300)
    H, D = 8, 128
    inp = workloads.paged_inputs(seed=741, lengths=lengths, q_lens=[1] * 70, q_heads=32, kv_heads=H,
                                 head_dim=D, dtype=torch.bfloat16, num_blocks=2000, max_blocks=128,
                                 device=DEV)
    bt = inp.block_table.cpu().numpy()
    used = inp.seqused_k.cpu().numpy()
    slots = np.array([oracle.paged_slot(bt[b], int(used[b]) - 1) for b in range(70)])
    k_ref, v_ref = oracle.kv_append(raw(inp.k_cache).reshape(-1, H, D), raw(inp.v_cache).reshape(-1, H, D),
                                    raw(inp.k_new), raw(inp.v_new), slots)
    out = _decode(inp, 3, k_new=inp.k_new, v_new=inp.v_new)
    assert np.array_equal(raw(inp.k_cache).reshape(-1, H, D), k_ref)
    assert np.array_equal(raw(inp.v_cache).reshape(-1, H, D), v_ref)
    ref = oracle.paged_attention(raw(inp.q), k_ref, v_ref, bt, np.arange(71), used, dtype="bf16",
                                 scale=inp.scale, max_seqlen_k=inp.max_seqlen_k)
    check_close(out, ref, "bf16", "fused append, 70 units")


def test_varlen_single_and_multi_row_units_mixed():
    """Paged varlen units of 1, 4, 1, 1, 7, 1, 16 query rows: the one-row units
    are dealt over the vector path's work groups, the others go to the matrix
    cores; bf16, G 4, D 128."""
    q_lens = [1, 4, 1, 1, 7, 1, 16]
    lengths = [900, 40, 0, 3000, 300, 17, 1200]
    inp = workloads.paged_inputs(seed=750, lengths=lengths, q_lens=q_lens, q_heads=32, kv_heads=8,
                                 head_dim=128, dtype=torch.bfloat16, num_blocks=400, max_blocks=200,
                                 causal=True, device=DEV)
    for splits in (0, 6):
        out = torch.full_like(inp.q, float("nan"))
        pkv.varlen_attn(out, inp.q, inp.k_cache, inp.v_cache, cu_seqlens_q=inp.cu_seqlens_q,
                        seqused_k=inp.seqused_k, block_table=inp.block_table, max_seqlen_q=16,
                        max_seqlen_k=inp.max_seqlen_k, softmax_scale=inp.scale, causal=True,
                        num_splits=splits)
        torch.cuda.synchronize()
        check_close(out, oracle_paged(inp), "bf16", f"mixed varlen splits={splits}")


def _mixed_call(inp, out, ws, splits=0):
    pkv.varlen_attn(out, inp.q, inp.k_cache, inp.v_cache, cu_seqlens_q=inp.cu_seqlens_q,
                    seqused_k=inp.seqused_k, block_table=inp.block_table, max_seqlen_q=16,
                    max_seqlen_k=inp.max_seqlen_k, softmax_scale=inp.scale, causal=True,
                    num_splits=splits, workspace=ws)


def _mixed_inputs():
    return workloads.paged_inputs(seed=760, lengths=[900, 40, 0, 3000, 300, 17, 1200], q_lens=[1, 4, 1, 1, 7, 1, 16],
                                  q_heads=32, kv_heads=8, head_dim=128, dtype=torch.bfloat16, num_blocks=400,
                                  max_blocks=200, causal=True, device=DEV)


def _capture_and_replay(inp, label):
    """Capture one mixed call, replay it three times with eager work between
    the replays; every replay must equal the eager result bit for bit."""
    ws = torch.zeros(pkv.attn_workspace_bytes(7, 16, inp.max_seqlen_k, 32, 8, 128, 0), dtype=torch.uint8,
                     device=DEV)
    eager = torch.full_like(inp.q, float("nan"))
    _mixed_call(inp, eager, ws)
    torch.cuda.synchronize()
    out = torch.full_like(inp.q, float("nan"))
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            _mixed_call(inp, out, ws)
    for k in range(3):
        out.fill_(float("nan"))
        scratch = torch.full_like(inp.q, float("nan"))
        _mixed_call(inp, scratch, ws)                 # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"{label}: replay {k} != eager"
    check_close(out, oracle_paged(inp), "bf16", label)


def test_graph_of_mixed_call_replays_like_eager():
    """One-row and multi-row units in one call (vector and matrix-core kernels,
    zeroed rows) captured once and replayed with eager work in between."""
    _capture_and_replay(_mixed_inputs(), "mixed call in a graph")
