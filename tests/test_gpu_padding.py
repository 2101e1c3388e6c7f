"""GPU parity of the left-padding bound ``kv_start`` on both attention calls.

tiny-llm kv_cache.py, padded_causal_mask: keys before a row's first valid
position are hidden and a pad query keeps its own key.  Each case mixes units
with no bound, a negative bound, a bound inside the prefix, bounds that make
some or all of a unit's query rows pad rows, and bounds past the live length.
Keys below every row's range are overwritten with NaN first: they must never
reach the output.  Outputs are compared with the oracle on every row.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_194_amd as pkv
import workloads
from helpers import check_close, oracle_column, oracle_paged, raw, ring_slots

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pkv.lib()


def _bounds(seed, lengths, q_lens):
    """One bound per unit, cycling through the interesting kinds."""
    rng = np.random.default_rng(seed)
    out = []
    for b, (E, L) in enumerate(zip(lengths, q_lens)):
        kind = b % 5
        if kind == 0:
            out.append(0)
        elif kind == 1:
            out.append(-int(rng.integers(1, 6)))
        elif kind == 2:
            out.append(int(rng.integers(1, max(2, E - L + 1))))
        elif kind == 3:
            out.append(max(1, E - L + int(rng.integers(0, L + 1))))       # some rows are pad rows
        else:
            out.append(E + int(rng.integers(0, 10)))                       # every row is a pad row
    return out


def _nan_below(inp, bounds, q_lens):
    """NaN into the keys of each paged sequence that no row can see: below
    min(bound, first row's position)."""
    bt = inp.block_table.cpu().numpy()
    H, D = inp.kv_heads, inp.head_dim
    kf = inp.k_cache.view(-1, H, D)
    vf = inp.v_cache.view(-1, H, D)
    used = inp.seqused_k.cpu().numpy()
    for b, (s, L) in enumerate(zip(bounds, q_lens)):
        stop = min(s, int(used[b]) - L) if s > 0 else 0
        if stop <= 0:
            continue
        slots = torch.tensor([oracle.paged_slot(bt[b], j) for j in range(stop)], device=DEV)
        kf[slots] = float("nan")
        vf[slots] = float("nan")


def _ks(bounds):
    return torch.tensor(bounds, dtype=torch.int32, device=DEV)


@pytest.mark.parametrize("splits", [0, 5])
def test_decode_bf16_with_padding(splits):
    """50 sequences of 1..2500 keys, one query each (vector path), G 4, D 128."""
    rng = np.random.default_rng(900)
    lengths = [int(x) for x in rng.integers(1, 2501, size=50)]
    inp = workloads.paged_inputs(seed=901, lengths=lengths, q_lens=[1] * 50, q_heads=32, kv_heads=8,
                                 head_dim=128, dtype=torch.bfloat16, num_blocks=8200, max_blocks=160,
                                 device=DEV)
    bounds = _bounds(902, lengths, [1] * 50)
    _nan_below(inp, bounds, [1] * 50)
    out = torch.full_like(inp.q, float("nan"))
    pkv.paged_decode_attn(out, inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.seqused_k,
                          max_seqlen_k=inp.max_seqlen_k, softmax_scale=inp.scale, num_splits=splits,
                          kv_start=_ks(bounds))
    torch.cuda.synchronize()
    ref = oracle_paged(inp, kv_start=np.array(bounds))
    check_close(out, ref, "bf16", f"decode with padding, splits={splits}")
    # a pad query sees only its own key: the output is that key's V row
    v = raw(inp.v_cache).reshape(-1, 8, 128)
    bt = inp.block_table.cpu().numpy()
    for b in range(4, 50, 5):
        if lengths[b] > 0:
            vrow = oracle.to_f64(v[oracle.paged_slot(bt[b], lengths[b] - 1)], "bf16")
            got = out[b].float().cpu().numpy().reshape(8, 4, 128)
            assert np.array_equal(got, np.repeat(vrow[:, None, :], 4, axis=1)), b


def test_decode_fp32_window_and_fused_append_with_padding():
    """fp32, G 2, D 64, a 300-key window, the new token appended in the call."""
    rng = np.random.default_rng(910)
    lengths = [int(x) for x in rng.integers(1, 1200, size=23)]
    inp = workloads.paged_inputs(seed=911, lengths=lengths, q_lens=[1] * 23, q_heads=4, kv_heads=2,
                                 head_dim=64, dtype=torch.float32, num_blocks=2000, max_blocks=80,
                                 window=300, device=DEV)
    bounds = _bounds(912, lengths, [1] * 23)
    _nan_below(inp, bounds, [1] * 23)
    bt = inp.block_table.cpu().numpy()
    slots = np.array([oracle.paged_slot(bt[b], lengths[b] - 1) for b in range(23)])
    k_ref, v_ref = oracle.kv_append(raw(inp.k_cache).reshape(-1, 2, 64), raw(inp.v_cache).reshape(-1, 2, 64),
                                    raw(inp.k_new), raw(inp.v_new), slots)
    out = torch.full_like(inp.q, float("nan"))
    pkv.paged_decode_attn(out, inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.seqused_k,
                          max_seqlen_k=inp.max_seqlen_k, softmax_scale=inp.scale, window=300,
                          num_splits=3, k_new=inp.k_new, v_new=inp.v_new, kv_start=_ks(bounds))
    torch.cuda.synchronize()
    ref = oracle.paged_attention(raw(inp.q), k_ref, v_ref, bt, np.arange(24), inp.seqused_k.cpu().numpy(),
                                 dtype="f32", scale=inp.scale, window=300, max_seqlen_k=inp.max_seqlen_k,
                                 kv_start=np.array(bounds))
    check_close(out, ref, "f32", "fp32 window + append + padding")


@pytest.mark.parametrize("causal", [True, False])
def test_varlen_multi_row_with_padding(causal):
    """Paged units of 1..16 query rows (matrix-core path for the multi-row
    ones), bounds that turn some rows into pad rows; bf16, G 4, D 128."""
    q_lens = [1, 4, 7, 16, 1, 9, 3, 12, 16, 2]
    lengths = [900, 40, 3000, 300, 17, 1200, 3, 2000, 16, 60]
    inp = workloads.paged_inputs(seed=920, lengths=lengths, q_lens=q_lens, q_heads=32, kv_heads=8,
                                 head_dim=128, dtype=torch.bfloat16, num_blocks=600, max_blocks=200,
                                 causal=causal, device=DEV)
    bounds = _bounds(921, lengths, q_lens)
    _nan_below(inp, bounds, q_lens)
    ref = oracle_paged(inp, kv_start=np.array(bounds))
    for splits in (0, 4):
        out = torch.full_like(inp.q, float("nan"))
        pkv.varlen_attn(out, inp.q, inp.k_cache, inp.v_cache, cu_seqlens_q=inp.cu_seqlens_q,
                        seqused_k=inp.seqused_k, block_table=inp.block_table, max_seqlen_q=16,
                        max_seqlen_k=inp.max_seqlen_k, softmax_scale=inp.scale, causal=causal,
                        num_splits=splits, kv_start=_ks(bounds))
        torch.cuda.synchronize()
        check_close(out, ref, "bf16", f"varlen padding causal={causal} splits={splits}")


def test_column_store_with_window_and_padding():
    """Ring store, causal, window 300, decode and chunked-prefill segments,
    one bound per segment; uncovered rows stay 0."""
    q_lens = [1, 1, 37, 1, 90, 16, 1, 20]
    ends = [5, 700, 900, 1500, 3000, 40, 64, 380]
    inp = workloads.column_inputs(seed=930, rows=512, cols=8, q_lens=q_lens, kv_ends=ends, total_q=260,
                                  q_heads=32, kv_heads=8, head_dim=128, dtype=torch.bfloat16, causal=True,
                                  window=300, device=DEV)
    pkv.kv_append(inp.k_store, inp.v_store, inp.k_new, inp.v_new, ring_slots(inp))
    bounds = _bounds(931, ends, q_lens)
    ref = oracle_column(inp, kv_start=np.array(bounds))
    covered = torch.from_numpy(inp.new_pos.cpu().numpy() >= 0).to(DEV)
    for s in (0, 3):
        out = torch.full_like(inp.q, float("nan"))
        pkv.varlen_attn(out, inp.q, inp.k_store, inp.v_store, seq_info=inp.seq_info,
                        max_seqlen_q=inp.max_seqlen_q, max_seqlen_k=300 + inp.max_seqlen_q - 1,
                        softmax_scale=inp.scale, causal=True, window=300, num_splits=s,
                        kv_start=_ks(bounds))
        torch.cuda.synchronize()
        assert (out[~covered] == 0).all()
        check_close(out, ref, "bf16", f"column padding splits={s}")


def test_zero_bounds_equal_no_bounds_bitwise():
    """kv_start of zeros and negatives gives the same bits as no kv_start."""
    rng = np.random.default_rng(940)
    lengths = [int(x) for x in rng.integers(1, 3000, size=12)]
    q_lens = [1, 5, 1, 16, 1, 3, 1, 1, 8, 1, 2, 1]
    inp = workloads.paged_inputs(seed=941, lengths=lengths, q_lens=q_lens, q_heads=32, kv_heads=8,
                                 head_dim=128, dtype=torch.bfloat16, num_blocks=2400, max_blocks=200,
                                 causal=True, device=DEV)
    outs = []
    for ks in (None, _ks([0] * 12), _ks([-7] * 12)):
        out = torch.full_like(inp.q, float("nan"))
        pkv.varlen_attn(out, inp.q, inp.k_cache, inp.v_cache, cu_seqlens_q=inp.cu_seqlens_q,
                        seqused_k=inp.seqused_k, block_table=inp.block_table, max_seqlen_q=16,
                        max_seqlen_k=inp.max_seqlen_k, softmax_scale=inp.scale, causal=True,
                        num_splits=4, kv_start=ks)
        torch.cuda.synchronize()
        outs.append(out.view(torch.int16))
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
