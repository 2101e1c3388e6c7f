"""GPU parity of kv_append and single-query (decode) attention against the oracle.

Every case is generated from a seed, run through the C ABI (via the binding),
copied back, and compared with the fp64 oracle on the same bits: append and
indexing bit-exactly, attention within 2e-2 (bf16) / 1e-4 (fp32) max abs plus
an RMS bound.  Invariants that must hold bit-for-bit (block-table permutation,
garbage past the live prefix, one key, window 1) are checked directly.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_194_amd as pkv
import workloads
from helpers import bits, check_close, dname, oracle_column, oracle_paged, paged_slots, raw, ring_slots

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pkv.lib()
    return torch.device("cuda:0")


DEV = "cuda:0"


# ---------------------------------------------------------------------------
# kv_append
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_kv_append_bit_exact(dtype):
    g = torch.Generator().manual_seed(11)
    H, D, NB = 3, 64, 6
    esz = 2 if dtype == torch.bfloat16 else 4
    itype = torch.int16 if esz == 2 else torch.int32
    lo, hi = (-2 ** 15, 2 ** 15) if esz == 2 else (-2 ** 31, 2 ** 31 - 1)
    cache_bits = torch.randint(lo, hi, (NB, 16, H, D), generator=g, dtype=torch.int64).to(itype)
    new_bits = torch.randint(lo, hi, (7, H, D), generator=g, dtype=torch.int64).to(itype)
    # NaN payloads and signalling patterns must survive the copy
    specials = [0x7FC1, -1, 0x7F81, -32768, 1, -128] if esz == 2 else [0x7FA00001, -4194304, 0x7F800001, 1]
    new_bits.view(-1)[:len(specials)] = torch.tensor(specials, dtype=itype)
    k = cache_bits.clone().to(DEV).view(dtype)
    v = (cache_bits.flip(0)).clone().to(DEV).view(dtype)
    kn = new_bits.to(DEV).view(dtype)
    vn = new_bits.flip(0).contiguous().to(DEV).view(dtype)
    slots = torch.tensor([5, -1, 95, 96, 40, 1000, 0], dtype=torch.int64, device=DEV)
    ut = np.uint16 if esz == 2 else np.uint32       # compare bit patterns, not float values
    k_ref, v_ref = oracle.kv_append(raw(k).reshape(-1, H, D).view(ut), raw(v).reshape(-1, H, D).view(ut),
                                    raw(kn).view(ut), raw(vn).view(ut), slots.cpu().numpy())
    pkv.kv_append(k, v, kn, vn, slots)
    torch.cuda.synchronize()
    assert np.array_equal(raw(k).reshape(-1, H, D).view(ut), k_ref)
    assert np.array_equal(raw(v).reshape(-1, H, D).view(ut), v_ref)


def test_kv_append_ring_column_store():
    inp = workloads.column_inputs(seed=5, rows=64, cols=5, q_lens=[1, 3, 7, 1], kv_ends=[70, 5, 200, 64],
                                  total_q=20, q_heads=8, kv_heads=2, head_dim=128,
                                  dtype=torch.bfloat16, causal=True, window=16, device=DEV)
    slots = ring_slots(inp)
    H, D = inp.kv_heads, inp.head_dim
    k_ref, v_ref = oracle.kv_append(raw(inp.k_store).reshape(-1, H, D), raw(inp.v_store).reshape(-1, H, D),
                                    raw(inp.k_new), raw(inp.v_new), slots.cpu().numpy())
    pkv.kv_append(inp.k_store, inp.v_store, inp.k_new, inp.v_new, slots)
    torch.cuda.synchronize()
    assert np.array_equal(raw(inp.k_store).reshape(-1, H, D), k_ref)
    assert np.array_equal(raw(inp.v_store).reshape(-1, H, D), v_ref)


def test_fused_decode_append_writes_block_table_slot():
    inp = workloads.paged_inputs(seed=21, lengths=[1, 16, 17, 100, 0], q_lens=[1, 1, 1, 1, 0],
                                 q_heads=8, kv_heads=2, head_dim=128, dtype=torch.bfloat16,
                                 num_blocks=20, max_blocks=8, device=DEV)
    # sequence 4 has no keys: give it a query row anyway so every row is a unit
    B = 5
    q = workloads.randn((B, 8, 128), torch.bfloat16, 3, DEV)
    kn = workloads.randn((B, 2, 128), torch.bfloat16, 4, DEV)
    vn = workloads.randn((B, 2, 128), torch.bfloat16, 5, DEV)
    H, D = 2, 128
    bt = inp.block_table.cpu().numpy()
    used = inp.seqused_k.cpu().numpy()
    slots = np.array([oracle.paged_slot(bt[b], int(used[b]) - 1) if used[b] > 0 else -1 for b in range(B)])
    k_ref, v_ref = oracle.kv_append(raw(inp.k_cache).reshape(-1, H, D), raw(inp.v_cache).reshape(-1, H, D),
                                    raw(kn), raw(vn), slots)
    out = torch.full_like(q, float("nan"))
    pkv.paged_decode_attn(out, q, inp.k_cache, inp.v_cache, inp.block_table, inp.seqused_k,
                          max_seqlen_k=128, k_new=kn, v_new=vn)
    torch.cuda.synchronize()
    assert np.array_equal(raw(inp.k_cache).reshape(-1, H, D), k_ref)
    assert np.array_equal(raw(inp.v_cache).reshape(-1, H, D), v_ref)
    ref = oracle.paged_attention(raw(q), k_ref, v_ref, bt, np.arange(B + 1), used, dtype="bf16",
                                 scale=inp.scale, max_seqlen_k=128)
    check_close(out, ref, "bf16", "fused append + decode")
    assert (out[4] == 0).all()


# ---------------------------------------------------------------------------
# decode attention parity
# ---------------------------------------------------------------------------

FUSED_ONE_WAVE = [
    # (head_dim, q_heads, kv_heads, dtype): shapes held to one wave per SIMD,
    # whose fused append stores the new row before the block loop
    (256, 64, 8, torch.bfloat16),
    (128, 64, 8, torch.bfloat16),
    (128, 16, 4, torch.float32),
]


@pytest.mark.parametrize("D,hq,hkv,dtype", FUSED_ONE_WAVE,
                         ids=[f"D{c[0]}-{c[1]}x{c[2]}-{str(c[3])[6:]}" for c in FUSED_ONE_WAVE])
def test_fused_append_one_wave_shapes(D, hq, hkv, dtype):
    lengths = [1, 16, 17, 300, 1000, 2049]
    B = len(lengths)
    inp = workloads.paged_inputs(seed=300 + D + hq, lengths=lengths, q_lens=[1] * B, q_heads=hq, kv_heads=hkv,
                                 head_dim=D, dtype=dtype, num_blocks=400, max_blocks=160, device=DEV)
    kn = workloads.randn((B, hkv, D), dtype, 301 + D, DEV)
    vn = workloads.randn((B, hkv, D), dtype, 302 + D, DEV)
    bt = inp.block_table.cpu().numpy()
    used = inp.seqused_k.cpu().numpy()
    slots = np.array([oracle.paged_slot(bt[b], int(used[b]) - 1) for b in range(B)])

    def cache_bits(t):      # bit patterns: the unused pool blocks hold NaN
        a = raw(t).reshape(-1, hkv, D)
        return a.view(np.uint32) if a.dtype == np.float32 else a

    def row_bits(t):
        a = raw(t)
        return a.view(np.uint32) if a.dtype == np.float32 else a

    k_ref, v_ref = oracle.kv_append(cache_bits(inp.k_cache), cache_bits(inp.v_cache), row_bits(kn), row_bits(vn),
                                    slots)
    as_vals = (lambda a: a.view(np.float32)) if dtype == torch.float32 else (lambda a: a)
    ref = oracle.paged_attention(raw(inp.q), as_vals(k_ref), as_vals(v_ref), bt, np.arange(B + 1), used,
                                 dtype=dname(inp.q), scale=inp.scale, max_seqlen_k=inp.max_seqlen_k)
    for splits in (1, 3, 0):
        out = torch.full_like(inp.q, float("nan"))
        pkv.paged_decode_attn(out, inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.seqused_k,
                              max_seqlen_k=inp.max_seqlen_k, softmax_scale=inp.scale, num_splits=splits,
                              k_new=kn, v_new=vn)
        torch.cuda.synchronize()
        assert np.array_equal(cache_bits(inp.k_cache), k_ref)
        assert np.array_equal(cache_bits(inp.v_cache), v_ref)
        check_close(out, ref, dname(inp.q), f"splits={splits}")


def test_long_ranges_past_one_id_group_with_fused_append():
    """A split of more than 256 blocks gives each of the 4 waves more than 64
    blocks, so block ids are read again for each further group of 64: 8192 and
    4500 keys in one or two splits, permuted tables, with the fused append, and
    again with a window of 3000 keys."""
    lengths = [8192, 4500, 100]
    H, D, B = 8, 128, len(lengths)
    inp = workloads.paged_inputs(seed=91, lengths=lengths, q_lens=[1] * B, q_heads=32, kv_heads=H,
                                 head_dim=D, dtype=torch.bfloat16, num_blocks=1000, max_blocks=512,
                                 device=DEV)
    kn = workloads.randn((B, H, D), torch.bfloat16, 92, DEV)
    vn = workloads.randn((B, H, D), torch.bfloat16, 93, DEV)
    bt = inp.block_table.cpu().numpy()
    used = inp.seqused_k.cpu().numpy()
    slots = np.array([oracle.paged_slot(bt[b], int(used[b]) - 1) for b in range(B)])
    k_ref, v_ref = oracle.kv_append(raw(inp.k_cache).reshape(-1, H, D), raw(inp.v_cache).reshape(-1, H, D),
                                    raw(kn), raw(vn), slots)
    for window in (0, 3000):
        ref = oracle.paged_attention(raw(inp.q), k_ref, v_ref, bt, np.arange(B + 1), used, dtype="bf16",
                                     scale=inp.scale, max_seqlen_k=inp.max_seqlen_k, window=window)
        for splits in (1, 2):
            out = torch.full_like(inp.q, float("nan"))
            pkv.paged_decode_attn(out, inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.seqused_k,
                                  max_seqlen_k=inp.max_seqlen_k, softmax_scale=inp.scale, window=window,
                                  num_splits=splits, k_new=kn, v_new=vn)
            torch.cuda.synchronize()
            assert np.array_equal(raw(inp.k_cache).reshape(-1, H, D), k_ref)
            assert np.array_equal(raw(inp.v_cache).reshape(-1, H, D), v_ref)
            check_close(out, ref, "bf16", f"window={window} splits={splits}")


def run_decode(inp, num_splits=0, out=None, **kw):
    out = torch.full_like(inp.q, float("nan")) if out is None else out
    pkv.paged_decode_attn(out, inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.seqused_k,
                          max_seqlen_k=inp.max_seqlen_k, softmax_scale=inp.scale,
                          causal=inp.causal, window=inp.window, num_splits=num_splits, **kw)
    torch.cuda.synchronize()
    return out


def test_tiny_fp32_config():
    """1 seq, Hq 4 / Hkv 2, D 64, fp32, 512-token bucket, 100 live keys, NaN tail;
    the new token is appended at key 99, then attended, one split."""
    inp = workloads.c1_tiny(device=DEV)
    H, D = inp.kv_heads, inp.head_dim
    k0 = raw(inp.k_cache).reshape(-1, H, D).view(np.uint32)
    v0 = raw(inp.v_cache).reshape(-1, H, D).view(np.uint32)
    slots = paged_slots(inp)
    assert slots.tolist() == [99]
    pkv.kv_append(inp.k_cache, inp.v_cache, inp.k_new, inp.v_new, slots)
    out = run_decode(inp, num_splits=1)
    k1, v1 = oracle.kv_append(k0, v0, raw(inp.k_new).view(np.uint32), raw(inp.v_new).view(np.uint32),
                              slots.cpu().numpy())
    assert np.array_equal(raw(inp.k_cache).reshape(-1, H, D).view(np.uint32), k1)
    ref = oracle_paged(inp)
    check_close(out, ref, "f32", "tiny")
    for s in (2, 7, 0):
        check_close(run_decode(inp, num_splits=s), ref, "f32", f"tiny splits={s}")


CASES = [
    # (head_dim, q_heads, kv_heads, dtype)
    (128, 32, 8, torch.bfloat16),
    (128, 8, 8, torch.bfloat16),
    (128, 16, 8, torch.bfloat16),
    (128, 24, 8, torch.bfloat16),
    (128, 64, 8, torch.bfloat16),
    (64, 8, 2, torch.bfloat16),
    (64, 16, 2, torch.bfloat16),
    (256, 64, 8, torch.bfloat16),
    (256, 16, 4, torch.bfloat16),
    (256, 8, 8, torch.bfloat16),
    (64, 4, 2, torch.float32),
    (128, 32, 8, torch.float32),
    (256, 16, 2, torch.float32),
    (64, 8, 1, torch.float32),
    # K layouts of 8 and 16 lanes per token with 2..8 chunks per lane
    (256, 4, 2, torch.float32),
    (256, 8, 2, torch.float32),
    (128, 64, 8, torch.float32),
    (64, 16, 16, torch.bfloat16),
]


@pytest.mark.parametrize("D,hq,hkv,dtype", CASES, ids=[f"D{c[0]}-{c[1]}x{c[2]}-{str(c[3])[6:]}" for c in CASES])
def test_decode_parity(D, hq, hkv, dtype):
    lengths = [1, 15, 16, 17, 100, 255, 256, 257, 700, 33]
    inp = workloads.paged_inputs(seed=100 + D + hq + hkv, lengths=lengths, q_lens=[1] * len(lengths),
                                 q_heads=hq, kv_heads=hkv, head_dim=D, dtype=dtype, num_blocks=160,
                                 max_blocks=48, device=DEV)
    ref = oracle_paged(inp)
    for s in (0, 1, 3, 16):
        check_close(run_decode(inp, num_splits=s), ref, dname(inp.q), f"splits={s}")
    # peaked scores (q x 4) make outputs O(1)
    q4 = (inp.q.float() * 4).to(dtype)
    ref4 = oracle_paged(inp, q=q4)
    out4 = torch.full_like(q4, float("nan"))
    pkv.paged_decode_attn(out4, q4, inp.k_cache, inp.v_cache, inp.block_table, inp.seqused_k,
                          max_seqlen_k=inp.max_seqlen_k, softmax_scale=inp.scale)
    torch.cuda.synchronize()
    check_close(out4, ref4, dname(q4), "peaked")


def test_window_and_causal_decode():
    inp = workloads.paged_inputs(seed=7, lengths=[300, 20, 1, 64], q_lens=[1] * 4, q_heads=32,
                                 kv_heads=8, head_dim=128, dtype=torch.bfloat16, num_blocks=40,
                                 max_blocks=24, device=DEV, window=37, causal=True)
    ref = oracle_paged(inp)
    for s in (0, 1, 5):
        check_close(run_decode(inp, num_splits=s), ref, "bf16", f"window splits={s}")


def test_batched_decode_64_sequences_full_size():
    """64 sequences, lengths U[1, 8192], 40000-block pool of distinct random blocks,
    32 q / 8 kv heads, D 128, bf16; the new tokens are appended first.  Every
    output of every sequence and head against the oracle, with the library's
    split choice (the launch the bench times) and with q scaled by 4 (peaked
    scores, outputs O(1))."""
    inp = workloads.c3_batched(device=DEV)
    slots = paged_slots(inp)
    pkv.kv_append(inp.k_cache, inp.v_cache, inp.k_new, inp.v_new, slots)
    out = run_decode(inp)
    check_close(out, oracle_paged(inp), "bf16", "batched, every sequence")
    q4 = (inp.q.float() * 4).to(torch.bfloat16)
    out4 = torch.full_like(q4, float("nan"))
    pkv.paged_decode_attn(out4, q4, inp.k_cache, inp.v_cache, inp.block_table, inp.seqused_k,
                          max_seqlen_k=inp.max_seqlen_k, softmax_scale=inp.scale)
    torch.cuda.synchronize()
    check_close(out4, oracle_paged(inp, q=q4), "bf16", "batched, peaked")


# ---------------------------------------------------------------------------
# invariants that hold bit for bit
# ---------------------------------------------------------------------------

def _logical_pair(seed, lengths, H, D, dtype, nb, mb):
    """The same logical keys placed through an identity and a permuted table."""
    ident = workloads.paged_inputs(seed=seed, lengths=lengths, q_lens=[1] * len(lengths), q_heads=4 * H,
                                   kv_heads=H, head_dim=D, dtype=dtype, num_blocks=nb, max_blocks=mb,
                                   identity=True, device=DEV)
    perm = workloads.paged_inputs(seed=seed, lengths=lengths, q_lens=[1] * len(lengths), q_heads=4 * H,
                                  kv_heads=H, head_dim=D, dtype=dtype, num_blocks=nb, max_blocks=mb,
                                  device=DEV)
    # copy each logical block of the identity layout into the permuted table's block
    bt_i = ident.block_table.cpu()
    bt_p = perm.block_table.cpu()
    for b, E in enumerate(lengths):
        n = (E + 15) // 16
        perm.k_cache[bt_p[b, :n].long().to(DEV)] = ident.k_cache[bt_i[b, :n].long().to(DEV)]
        perm.v_cache[bt_p[b, :n].long().to(DEV)] = ident.v_cache[bt_i[b, :n].long().to(DEV)]
    perm.q.copy_(ident.q)
    return ident, perm


def test_permuted_block_table_is_bit_identical():
    ident, perm = _logical_pair(31, [5, 300, 64, 1000], 8, 128, torch.bfloat16, 200, 64)
    for s in (1, 4, 0):
        a = run_decode(ident, num_splits=s)
        b = run_decode(perm, num_splits=s)
        assert torch.equal(bits(a), bits(b)), f"splits={s}"


def test_garbage_past_live_prefix_changes_nothing():
    inp = workloads.paged_inputs(seed=41, lengths=[37, 290, 3], q_lens=[1, 1, 1], q_heads=16,
                                 kv_heads=4, head_dim=128, dtype=torch.bfloat16, num_blocks=40,
                                 max_blocks=32, device=DEV, nan_unused=False)
    base = run_decode(inp, num_splits=4)
    k, v = inp.k_cache.clone(), inp.v_cache.clone()
    bt = inp.block_table.cpu()
    used = inp.seqused_k.cpu()
    # poison every slot past each live prefix, unused blocks, and the table tails
    kf, vf = k.view(-1, 4, 128), v.view(-1, 4, 128)
    live = torch.zeros(kf.shape[0], dtype=torch.bool)
    for b in range(3):
        for j in range(int(used[b])):
            live[int(bt[b, j // 16]) * 16 + j % 16] = True
    for fill in (float("nan"), float("inf")):
        kf[~live.to(DEV)] = fill
        vf[~live.to(DEV)] = fill
        bt2 = inp.block_table.clone()
        for b in range(3):
            bt2[b, (int(used[b]) + 15) // 16:] = -7
        out = torch.full_like(inp.q, float("nan"))
        pkv.paged_decode_attn(out, inp.q, k, v, bt2, inp.seqused_k, max_seqlen_k=inp.max_seqlen_k,
                              softmax_scale=inp.scale, num_splits=4)
        torch.cuda.synchronize()
        assert torch.equal(bits(out), bits(base)), f"fill={fill}"


def test_single_key_returns_v_exactly():
    inp = workloads.paged_inputs(seed=51, lengths=[1, 1, 1], q_lens=[1, 1, 1], q_heads=32, kv_heads=8,
                                 head_dim=128, dtype=torch.bfloat16, num_blocks=8, max_blocks=4, device=DEV)
    out = run_decode(inp)
    bt = inp.block_table.cpu()
    for b in range(3):
        vb = inp.v_cache[int(bt[b, 0]), 0]           # [Hkv, D], key 0
        want = vb.repeat_interleave(4, dim=0)
        assert torch.equal(bits(out[b]), bits(want))


def test_window_one_returns_last_key_exactly():
    inp = workloads.paged_inputs(seed=52, lengths=[77, 16, 1000], q_lens=[1, 1, 1], q_heads=16, kv_heads=8,
                                 head_dim=128, dtype=torch.bfloat16, num_blocks=80, max_blocks=64,
                                 device=DEV, window=1)
    out = run_decode(inp)
    bt = inp.block_table.cpu()
    used = inp.seqused_k.cpu()
    for b in range(3):
        j = int(used[b]) - 1
        vb = inp.v_cache[int(bt[b, j // 16]), j % 16]
        assert torch.equal(bits(out[b]), bits(vb.repeat_interleave(2, dim=0)))


def test_constant_v_and_empty_sequences():
    inp = workloads.paged_inputs(seed=53, lengths=[500, 0, 3], q_lens=[1, 1, 1], q_heads=32, kv_heads=8,
                                 head_dim=128, dtype=torch.bfloat16, num_blocks=40, max_blocks=32, device=DEV)
    inp.v_cache.fill_(0.8125)
    out = run_decode(inp, num_splits=8)
    assert (out[0].float() == 0.8125).all() and (out[2].float() == 0.8125).all()
    assert (out[1] == 0).all()


def test_out_of_range_block_id_skips_those_keys():
    inp = workloads.paged_inputs(seed=54, lengths=[100, 60], q_lens=[1, 1], q_heads=8, kv_heads=2,
                                 head_dim=64, dtype=torch.bfloat16, num_blocks=16, max_blocks=8,
                                 device=DEV, nan_unused=False)
    inp.block_table[0, 2] = 999999
    inp.block_table[1, 0] = -3
    ref = oracle_paged(inp)
    check_close(run_decode(inp, num_splits=2), ref, "bf16", "bad block ids")


def test_repeat_runs_are_bit_identical():
    inp = workloads.paged_inputs(seed=55, lengths=[4000, 3, 1234], q_lens=[1, 1, 1], q_heads=32, kv_heads=8,
                                 head_dim=128, dtype=torch.bfloat16, num_blocks=400, max_blocks=256, device=DEV)
    a = run_decode(inp)
    b = run_decode(inp)
    assert torch.equal(bits(a), bits(b))


# ---------------------------------------------------------------------------
# column store, decode segments
# ---------------------------------------------------------------------------

def test_column_store_decode_segments():
    """Ring columns (rows 512) with wrap, window 200, q_len 1 segments scattered in
    the packed rows; uncovered rows must come back exactly 0 (output prefilled NaN)."""
    ends = [1, 17, 511, 512, 513, 900, 5000, 64]
    inp = workloads.column_inputs(seed=61, rows=512, cols=8, q_lens=[1] * 8, kv_ends=ends, total_q=40,
                                  q_heads=32, kv_heads=8, head_dim=128, dtype=torch.bfloat16,
                                  causal=True, window=200, device=DEV)
    pkv.kv_append(inp.k_store, inp.v_store, inp.k_new, inp.v_new, ring_slots(inp))
    ref = oracle_column(inp)
    covered = inp.new_pos.cpu().numpy() >= 0
    for s in (0, 1, 4):
        out = torch.full_like(inp.q, float("nan"))
        pkv.varlen_attn(out, inp.q, inp.k_store, inp.v_store, seq_info=inp.seq_info, max_seqlen_q=1,
                        max_seqlen_k=200, softmax_scale=inp.scale, causal=True, window=200,
                        num_splits=s)
        torch.cuda.synchronize()
        assert (out[torch.from_numpy(~covered).to(DEV)] == 0).all()
        check_close(out, ref, "bf16", f"column splits={s}")


def test_max_seqlen_q_one_computes_row_zero_of_longer_units():
    """With max_seqlen_q = 1 each unit's first row is computed (at position E - L,
    causal bound included) and its later rows count as uncovered (zero), for
    units of several rows too."""
    inp = workloads.paged_inputs(seed=63, lengths=[50, 300, 2, 40], q_lens=[3, 1, 4, 2], q_heads=16,
                                 kv_heads=4, head_dim=128, dtype=torch.bfloat16, num_blocks=40,
                                 max_blocks=24, causal=True, window=0, device=DEV)
    for causal, window in ((True, 0), (False, 0), (True, 20)):
        out = torch.full_like(inp.q, float("nan"))
        pkv.varlen_attn(out, inp.q, inp.k_cache, inp.v_cache, cu_seqlens_q=inp.cu_seqlens_q,
                        seqused_k=inp.seqused_k, block_table=inp.block_table, max_seqlen_q=1,
                        max_seqlen_k=inp.max_seqlen_k, softmax_scale=inp.scale, causal=causal,
                        window=window, num_splits=2)
        torch.cuda.synchronize()
        ref = oracle_paged(inp, causal=causal, window=window, max_seqlen_q=1)
        first = inp.cu_seqlens_q.cpu().numpy()[:-1]
        rest = np.setdiff1d(np.arange(inp.q.shape[0]), first)
        assert (out[torch.from_numpy(rest).to(DEV)] == 0).all(), (causal, window)
        check_close(out, ref, "bf16", f"max_seqlen_q=1 causal={causal} window={window}")


def test_paged_varlen_single_rows_and_uncovered_tail():
    inp = workloads.paged_inputs(seed=62, lengths=[40, 1, 333], q_lens=[1, 1, 1], q_heads=16, kv_heads=4,
                                 head_dim=64, dtype=torch.bfloat16, num_blocks=40, max_blocks=24, device=DEV)
    q = torch.cat([inp.q, workloads.randn((5, 16, 64), torch.bfloat16, 9, DEV)])
    out = torch.full_like(q, float("nan"))
    pkv.varlen_attn(out, q, inp.k_cache, inp.v_cache, cu_seqlens_q=inp.cu_seqlens_q,
                    seqused_k=inp.seqused_k, block_table=inp.block_table, max_seqlen_q=1,
                    max_seqlen_k=inp.max_seqlen_k, softmax_scale=inp.scale)
    torch.cuda.synchronize()
    ref = oracle_paged(inp, q=q)
    assert (out[3:] == 0).all()
    check_close(out, ref, "bf16", "paged varlen")


# ---------------------------------------------------------------------------
# graph capture: one capture serves every length
# ---------------------------------------------------------------------------

def test_graph_replay_matches_eager_across_lengths():
    H, D, hq, bucket = 8, 128, 32, 1024
    nb = bucket // 16
    dev = torch.device(DEV)
    k = workloads.randn((nb, 16, H, D), torch.bfloat16, 71, dev)
    v = workloads.randn((nb, 16, H, D), torch.bfloat16, 72, dev)
    bt = torch.arange(nb, dtype=torch.int32, device=dev)[None]
    used = torch.zeros(1, dtype=torch.int32, device=dev)
    q = torch.zeros(1, hq, D, dtype=torch.bfloat16, device=dev)
    kn = torch.zeros(1, H, D, dtype=torch.bfloat16, device=dev)
    vn = torch.zeros(1, H, D, dtype=torch.bfloat16, device=dev)
    out = torch.zeros(1, hq, D, dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(pkv.attn_workspace_bytes(1, 1, bucket, hq, H, D), dtype=torch.uint8, device=dev)
    steps = workloads.randn((40, hq + 2 * H, D), torch.bfloat16, 73, dev)

    def step():
        pkv.paged_decode_attn(out, q, k, v, bt, used, max_seqlen_k=bucket, workspace=ws, k_new=kn, v_new=vn)

    lengths = [1, 2, 15, 16, 17, 300, 511, 512, 513, 1000, 1023, 1024]
    used.fill_(lengths[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    k_eager, v_eager = k.clone(), v.clone()
    for i, L in enumerate(lengths):
        src = steps[i]
        q.copy_(src[:hq][None]); kn.copy_(src[hq:hq + H][None]); vn.copy_(src[hq + H:][None])
        used.fill_(L)
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        # eager on copies of the cache state before this step
        out_e = torch.empty_like(out)
        pkv.paged_decode_attn(out_e, q, k_eager, v_eager, bt, used, max_seqlen_k=bucket, workspace=ws,
                              k_new=kn, v_new=vn)
        torch.cuda.synchronize()
        assert torch.equal(bits(got), bits(out_e)), f"length {L}"
        assert torch.equal(bits(k), bits(k_eager)) and torch.equal(bits(v), bits(v_eager))
        ref = oracle.paged_attention(raw(q), raw(k), raw(v), bt.cpu().numpy(), np.array([0, 1]),
                                     np.array([L]), dtype="bf16", scale=1 / D ** 0.5, max_seqlen_k=bucket)
        check_close(got, ref, "bf16", f"graph length {L}")


def test_split_tickets_reset_and_workspace_reuse():
    """Split-K arrival counters come back to zero after every call, so one
    zero-filled workspace serves many calls and split counts in a row."""
    inp = workloads.paged_inputs(seed=81, lengths=[3000, 17, 900, 1], q_lens=[1] * 4, q_heads=32, kv_heads=8,
                                 head_dim=128, dtype=torch.bfloat16, num_blocks=300, max_blocks=192, device=DEV)
    ref = oracle_paged(inp)
    ws = torch.zeros(pkv.attn_workspace_bytes(4, 1, inp.max_seqlen_k, 32, 8, 128, 64), dtype=torch.uint8,
                     device=DEV)
    first = None
    tickets = ws[:4 * 8 * 256].view(torch.int32)[::64]     # one counter per 256 bytes
    assert tickets.numel() == 4 * 8
    for s in (64, 2, 7, 64, 33):
        out = run_decode(inp, num_splits=s, workspace=ws)
        check_close(out, ref, "bf16", f"splits={s}")
        assert int(tickets.abs().sum()) == 0, f"splits={s}: {tickets.tolist()}"
        if s == 64:
            if first is None:
                first = out.clone()
            else:
                assert torch.equal(bits(out), bits(first))


def test_single_sequence_split_counts_share_one_workspace():
    """One sequence, one zero-filled workspace, a run of calls with different
    split counts (empty splits included): every kv head's arrival counter is
    back at zero after each call, and equal split counts give equal bits."""
    H = 8
    inp = workloads.paged_inputs(seed=82, lengths=[1000], q_lens=[1], q_heads=32, kv_heads=H, head_dim=128,
                                 dtype=torch.bfloat16, num_blocks=70, max_blocks=64, device=DEV)
    ref = oracle_paged(inp)
    ws = torch.zeros(pkv.attn_workspace_bytes(1, 1, inp.max_seqlen_k, 32, H, 128, 256), dtype=torch.uint8,
                     device=DEV)
    tickets = ws[:H * 256].view(torch.int32)[::64]
    seen = {}
    for s in (64, 2, 7, 256, 64, 1, 33, 2, 256):
        out = run_decode(inp, num_splits=s, workspace=ws)
        check_close(out, ref, "bf16", f"splits={s}")
        assert int(tickets.abs().sum()) == 0, f"splits={s}: {tickets.tolist()}"
        if s in seen:
            assert torch.equal(bits(out), bits(seen[s])), f"splits={s} repeat"
        seen[s] = out.clone()
    short = workloads.paged_inputs(seed=83, lengths=[5], q_lens=[1], q_heads=32, kv_heads=H, head_dim=128,
                                   dtype=torch.bfloat16, num_blocks=8, max_blocks=64, device=DEV)
    for s in (32, 256):
        check_close(run_decode(short, num_splits=s, workspace=ws), oracle_paged(short), "bf16", f"E=5 splits={s}")
