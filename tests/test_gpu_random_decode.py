"""GPU parity of ``paged_decode_attn`` over seeded random call shapes: head_dim
64/128/256, GQA groups 1..16, bf16 and fp32, 2..12 sequences of 1..3000 keys,
windows, left-padding bounds, split counts, the fused append of the new token
and the no-workspace entry point.  The caches after the call must equal the
oracle's append bit for bit and every output element must match the fp64
oracle on the appended caches."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_194_amd as pkv
import workloads
from helpers import check_close, raw

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N_CASES = 32


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pkv.lib()


def _draw(case: int) -> dict:
    r = np.random.default_rng(7000 + case)
    fp32 = bool(r.random() < 0.25)
    G = int(r.choice([1, 2, 4, 8] if fp32 else [1, 2, 4, 8, 16]))
    B = int(r.integers(2, 13))                           # several sequences
    lengths = [int(x) for x in r.integers(1, 3001, size=B)]
    lengths[int(r.integers(0, B))] = int(r.choice([1, 16, 17]))
    return dict(D=int(r.choice([64, 128, 256])), dtype=torch.float32 if fp32 else torch.bfloat16, G=G,
                hkv=int(r.choice([1, 2, 4, 8])), lengths=lengths, window=int(r.choice([0, 0, 64, 1000])),
                splits=int(r.choice([0, 0, 1, 2, 5])), append=bool(r.random() < 0.5),
                pad=bool(r.random() < 0.3), causal=bool(r.random() < 0.5), noalloc=bool(r.random() < 0.25),
                seed=8000 + 13 * case)


def _same_bits(a: np.ndarray, b: np.ndarray) -> bool:
    """Equal bytes (NaN payloads included; fp32 caches come back as floats)."""
    return a.shape == b.shape and np.array_equal(np.ascontiguousarray(a).view(np.uint8),
                                                 np.ascontiguousarray(b).view(np.uint8))


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_decode_call(case):
    c = _draw(case)
    name = "f32" if c["dtype"] == torch.float32 else "bf16"
    D, H, B = c["D"], c["hkv"], len(c["lengths"])
    Hq = c["G"] * H
    nb = sum((E + 15) // 16 for E in c["lengths"]) + 8
    mb = max((E + 15) // 16 for E in c["lengths"]) + 3
    inp = workloads.paged_inputs(seed=c["seed"], lengths=c["lengths"], q_lens=[1] * B, q_heads=Hq, kv_heads=H,
                                 head_dim=D, dtype=c["dtype"], num_blocks=nb, max_blocks=mb, causal=c["causal"],
                                 window=c["window"], device=DEV)
    bt = inp.block_table.cpu().numpy()
    used = inp.seqused_k.cpu().numpy().astype(np.int64)
    k_flat, v_flat = raw(inp.k_cache).reshape(-1, H, D), raw(inp.v_cache).reshape(-1, H, D)
    kw = {}
    if c["append"]:
        kn = workloads.randn((B, H, D), c["dtype"], c["seed"] + 7, DEV)
        vn = workloads.randn((B, H, D), c["dtype"], c["seed"] + 8, DEV)
        slots = np.array([oracle.paged_slot(bt[b], int(used[b]) - 1) for b in range(B)])
        k_flat, v_flat = oracle.kv_append(k_flat, v_flat, raw(kn), raw(vn), slots)
        kw.update(k_new=kn, v_new=vn)
    ks_np = None
    if c["pad"]:
        r = np.random.default_rng(c["seed"] + 9)
        ks_np = np.array([int(r.integers(0, E)) for E in c["lengths"]], dtype=np.int64)
        kw["kv_start"] = torch.tensor(ks_np, dtype=torch.int32, device=DEV)
    ref = oracle.paged_attention(raw(inp.q), k_flat, v_flat, bt, np.arange(B + 1), used, dtype=name,
                                 scale=inp.scale, causal=c["causal"], window=c["window"],
                                 max_seqlen_k=inp.max_seqlen_k, kv_start=ks_np)
    out = torch.full_like(inp.q, float("nan"))
    need = pkv.attn_workspace_bytes(B, 1, inp.max_seqlen_k, Hq, H, D, c["splits"])
    entry = pkv.paged_decode_attn
    if c["noalloc"] and need <= pkv.NOALLOC_SCRATCH_BYTES:
        entry = pkv.paged_decode_attn_noalloc
    entry(out, inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.seqused_k, max_seqlen_k=inp.max_seqlen_k,
          softmax_scale=inp.scale, causal=c["causal"], window=c["window"], num_splits=c["splits"], **kw)
    torch.cuda.synchronize()
    what = f"case {case} ({entry.__name__}): {c}"
    assert _same_bits(raw(inp.k_cache).reshape(-1, H, D), k_flat), what
    assert _same_bits(raw(inp.v_cache).reshape(-1, H, D), v_flat), what
    check_close(out, ref, name, what)
