"""GPU parity of the prefix import and export copies (bit-exact).

A dense prefill cache ``[B, Hkv, S, D]`` goes into the slots its block table
names and comes back out; every byte of the pool and of the exported tensors is
compared with the oracle.  Cases: a ragged prefix over permuted tables with
entries outside the pool, the identity table of a single sequence (the pages'
flat copy), fp32, head_dim 64/128/256, a 4096-token 8-head prefix, 64
sequences over a permuted pool, n = 0, and the harness flow -- import, decode
steps that append, export.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_194_amd as pkv
import workloads
from helpers import bits, raw
from paged_kv_cache_194_amd.harness import PagedDecodeCache

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pkv.lib()


def _b(t: torch.Tensor) -> np.ndarray:
    """Integer bit view on the host (NaN-safe equality, the oracle's input form)."""
    return bits(t).cpu().numpy()


def _flat(t: torch.Tensor) -> np.ndarray:
    return _b(t).reshape(-1, t.shape[2], t.shape[3])


def _check_import_export(inp: workloads.PrefixInputs, label: str):
    B, H, S, D = inp.k_src.shape
    n = inp.n
    bt = inp.block_table.cpu().numpy()
    k_ref, v_ref = oracle.prefix_import(_flat(inp.k_cache), _flat(inp.v_cache), _b(inp.k_src),
                                        _b(inp.v_src), bt, n)
    used = torch.full((B,), -5, dtype=torch.int32, device=DEV)
    print(f"[prefix] {label}: B={B} H={H} S={S} D={D} n={n} {inp.k_src.dtype}", flush=True)
    pkv.prefix_import(inp.k_cache, inp.v_cache, inp.k_src, inp.v_src, inp.block_table, n,
                      seqused_k=used)
    torch.cuda.synchronize()
    assert np.array_equal(_flat(inp.k_cache), k_ref), f"{label}: K pool differs from the oracle"
    assert np.array_equal(_flat(inp.v_cache), v_ref), f"{label}: V pool differs from the oracle"
    assert (used == n).all(), f"{label}: seqused_k not set to n"

    ke_ref, ve_ref = oracle.prefix_export(k_ref, v_ref, bt, B, n)
    k_out = torch.full((B, H, n, D), float("nan"), dtype=inp.k_src.dtype, device=DEV)
    v_out = torch.full((B, H, n, D), float("nan"), dtype=inp.k_src.dtype, device=DEV)
    pkv.prefix_export(k_out, v_out, inp.k_cache, inp.v_cache, inp.block_table)
    torch.cuda.synchronize()
    assert np.array_equal(_b(k_out), ke_ref), f"{label}: exported K differs from the oracle"
    assert np.array_equal(_b(v_out), ve_ref), f"{label}: exported V differs from the oracle"
    return k_out, v_out


def test_ragged_prefix_permuted_tables_with_entries_outside_the_pool():
    """Three sequences, n = 37 of 45 (a ragged last block); sequence 1's
    second entry is -1 and sequence 2's third is num_blocks: those positions
    are skipped on import and read as zero on export."""
    inp = workloads.prefix_inputs(seed=800, batch=3, kv_heads=2, head_dim=64, src_len=45, n=37,
                                  num_blocks=20, max_blocks=4, dtype=torch.bfloat16, device=DEV,
                                  bad_entries=[(1, 1, -1), (2, 2, 20)])
    k_out, _ = _check_import_export(inp, "ragged, bad entries")
    assert (bits(k_out[1, :, 16:32]) == 0).all() and (bits(k_out[2, :, 32:37]) == 0).all()


def test_identity_table_single_sequence_is_the_flat_copy():
    """The pages' case: one sequence, identity table, slots [:n] of the flat
    view get the [S, H, D] transpose; fp32, 8 heads, head_dim 128."""
    inp = workloads.prefix_inputs(seed=810, batch=1, kv_heads=8, head_dim=128, src_len=128, n=100,
                                  num_blocks=32, max_blocks=32, dtype=torch.float32, device=DEV,
                                  identity=True)
    before = inp.k_cache.clone()
    _check_import_export(inp, "identity fp32")
    flat = inp.k_cache.view(-1, 8, 128)
    assert torch.equal(bits(flat[:100]), bits(inp.k_src[0].transpose(0, 1)[:100]))
    assert torch.equal(bits(flat[100:]), bits(before.view(-1, 8, 128)[100:]))


@pytest.mark.parametrize("head_dim,heads,dtype", [(64, 4, torch.float32), (256, 8, torch.bfloat16),
                                                  (8, 3, torch.bfloat16), (40, 5, torch.float32)])
def test_head_geometries(head_dim, heads, dtype):
    """Rows of one 16-byte chunk (head_dim 8, bf16) up to 32 chunks, odd head
    counts and chunk counts that leave a partial work group."""
    inp = workloads.prefix_inputs(seed=820 + head_dim, batch=2, kv_heads=heads, head_dim=head_dim,
                                  src_len=70, n=70, num_blocks=16, max_blocks=6, dtype=dtype,
                                  device=DEV)
    _check_import_export(inp, f"D={head_dim} H={heads}")


def test_4k_prefix_of_the_42_layer_model_shape():
    """One layer of the 42-layer decode model: 4096-token prefix, 8 kv heads,
    head_dim 128, bf16, imported into an 8192 bucket (prefix + 1 crosses 4096)."""
    inp = workloads.prefix_inputs(seed=830, batch=1, kv_heads=8, head_dim=128, src_len=4096, n=4096,
                                  num_blocks=512, max_blocks=512, dtype=torch.bfloat16, device=DEV,
                                  identity=True)
    _check_import_export(inp, "4k prefix")


def test_64_sequences_over_a_permuted_pool():
    """64 sequences of 1000 positions each over a permuted 5000-block pool."""
    inp = workloads.prefix_inputs(seed=840, batch=64, kv_heads=8, head_dim=128, src_len=1000,
                                  n=1000, num_blocks=5000, max_blocks=64, dtype=torch.bfloat16,
                                  device=DEV)
    _check_import_export(inp, "64 sequences")


def test_zero_length_only_sets_the_length():
    inp = workloads.prefix_inputs(seed=850, batch=2, kv_heads=2, head_dim=64, src_len=8, n=0,
                                  num_blocks=4, max_blocks=2, dtype=torch.bfloat16, device=DEV)
    before = inp.k_cache.clone()
    used = torch.full((2,), 9, dtype=torch.int32, device=DEV)
    pkv.prefix_import(inp.k_cache, inp.v_cache, inp.k_src, inp.v_src, inp.block_table, 0,
                      seqused_k=used)
    torch.cuda.synchronize()
    assert (used == 0).all()
    assert torch.equal(bits(inp.k_cache), bits(before))


def test_harness_import_decode_export_round_trip():
    """from_dynamic_cache with a 300-token prefix over 3 layers, 5 decode steps
    that append through the fused path, then to_dynamic_cache: each layer's
    export is the prefix followed by the 5 appended rows, bit for bit."""
    layers, hq, hkv, d, prefix, steps = 3, 8, 2, 128, 300, 5
    keys = [workloads.randn((1, hkv, prefix, d), torch.bfloat16, 860 + i, DEV) for i in range(layers)]
    vals = [workloads.randn((1, hkv, prefix, d), torch.bfloat16, 870 + i, DEV) for i in range(layers)]
    cache = PagedDecodeCache.from_dynamic_cache(keys, vals, hq, DEV, torch.bfloat16)
    assert cache.length == prefix and cache.bucket == 512
    assert int(cache.seqused.item()) == prefix
    new = workloads.randn((steps, layers, hq + 2 * hkv, d), torch.bfloat16, 880, DEV)
    out = torch.empty((1, hq, d), dtype=torch.bfloat16, device=DEV)
    for t in range(steps):
        cache.set_length(cache.length + 1)
        for i in range(layers):
            x = new[t, i]
            cache.attend(i, x[:hq].unsqueeze(0), x[hq:hq + hkv].unsqueeze(0),
                         x[hq + hkv:].unsqueeze(0), out)
    torch.cuda.synchronize()
    exported = cache.to_dynamic_cache()
    for i, (k, v) in enumerate(exported):
        assert k.shape == (1, hkv, prefix + steps, d)
        want_k = np.concatenate([raw(keys[i]), raw(new[:, i, hq:hq + hkv]).transpose(1, 0, 2)[None]], axis=2)
        want_v = np.concatenate([raw(vals[i]), raw(new[:, i, hq + hkv:]).transpose(1, 0, 2)[None]], axis=2)
        assert np.array_equal(raw(k), want_k), f"layer {i}: K hand-off differs"
        assert np.array_equal(raw(v), want_v), f"layer {i}: V hand-off differs"
    assert PagedDecodeCache.from_dynamic_cache([None], [None], hq, DEV, torch.bfloat16) is None
