"""Pins for the CPU fp64 oracle (no GPU).

Each check ties the oracle to something other than itself: values worked by
hand from the pages' stated rules (``tests/golden/``), a pure-Python brute
force on tiny inputs, torch's CPU SDPA with explicit masks, closed forms, and
invariants the method must satisfy (block-table permutation, garbage past the
live prefix, ring vs unrolled storage, GQA vs repeated heads).  The last test
plants mistakes in the oracle and checks that some pin catches each one.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Test-side construction of storage (independent of the oracle's gathers).
# ---------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def raw(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


def garbage(shape, dtype, kind="nan", rng=None):
    if kind == "zero":
        return raw(np.zeros(shape, np.float32), dtype)
    if kind == "nan":
        return raw(np.full(shape, np.nan, np.float32), dtype)
    if kind == "inf":
        return raw(np.full(shape, np.inf, np.float32), dtype)
    g = np.random.default_rng(99)   # its own stream: garbage never shifts the real values
    return raw(g.standard_normal(shape).astype(np.float32) * 1e4, dtype)


def place_paged(pool, table_row, logical):
    """Put logical keys 0..E-1 into the pool block by block: table entry k
    names the pool block that holds tokens 16k .. 16k+15."""
    E = logical.shape[0]
    nb = (E + 15) // 16
    for k in range(nb):
        n = min(16, E - 16 * k)
        pool[table_row[k], :n] = logical[16 * k:16 * k + n]


def place_ring(store, col, logical):
    """Append logical keys 0..E-1 one at a time into a ring column: each new
    key goes to the row after the previous one, wrapping at the end."""
    rows = store.shape[0]
    r = 0
    for j in range(logical.shape[0]):
        store[r, col] = logical[j]
        r = r + 1 if r + 1 < rows else 0


# ---------------------------------------------------------------------------
# Pure-Python brute force (the definition with nested loops and math.exp).
# ---------------------------------------------------------------------------

def brute_unit(q, K, V, E, scale, causal, window, ok=None):
    """q [L][Hq][D], K/V [E][Hkv][D] logical float lists -> out [L][Hq][D].
    ``ok[j]`` False: key j has no storage and is left out of every row."""
    L, Hq, D = len(q), len(q[0]), len(q[0][0])
    Hkv = len(K[0]) if E else 1
    G = Hq // Hkv
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(L)]
    for i in range(L):
        p = E - L + i
        vis = []
        for j in range(E):
            if causal and j > p:
                continue
            if window > 0 and j < p - window + 1:
                continue
            if ok is not None and not ok[j]:
                continue
            vis.append(j)
        if not vis:
            continue
        for h in range(Hq):
            g = h // G
            s = [scale * sum(q[i][h][d] * K[j][g][d] for d in range(D)) for j in vis]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            tot = sum(w)
            out[i][h] = [sum(w[k] * V[vis[k]][g][d] for k in range(len(vis))) / tot
                         for d in range(D)]
    return out


def f64(a, dtype):
    """Test-side widening through torch (independent of the oracle's decoder)."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
        return t.to(torch.float64).numpy()
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def make_paged_case(rng, *, lengths, q_lens, hq, hkv, d, dtype, num_blocks, max_blocks,
                    tail="nan", identity=False):
    """Random logical K/V per sequence placed through a random (or identity) table."""
    nbs = [(E + 15) // 16 for E in lengths]
    perm = rng.permutation(num_blocks)
    if identity:
        perm = np.arange(num_blocks)
    table = np.full((len(lengths), max_blocks), 0x7FFFFFFF, dtype=np.int64)
    k = 0
    for b, nb in enumerate(nbs):
        table[b, :nb] = perm[k:k + nb]
        k += nb
    pool_k = garbage((num_blocks, 16, hkv, d), dtype, tail, rng)
    pool_v = garbage((num_blocks, 16, hkv, d), dtype, tail, rng)
    logical = []
    for b, E in enumerate(lengths):
        Kl = raw(rng.standard_normal((E, hkv, d)).astype(np.float32), dtype)
        Vl = raw(rng.standard_normal((E, hkv, d)).astype(np.float32), dtype)
        place_paged(pool_k, table[b], Kl)
        place_paged(pool_v, table[b], Vl)
        logical.append((Kl, Vl))
    total_q = sum(q_lens)
    q = raw(rng.standard_normal((total_q, hq, d)).astype(np.float32), dtype)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    return dict(q=q, k=pool_k, v=pool_v, table=table, cu=cu,
                used=np.array(lengths, dtype=np.int64), logical=logical)


# ---------------------------------------------------------------------------
# Pins as plain functions (so the mutation test can re-run them).
# ---------------------------------------------------------------------------

def pin_golden_causal_rule():
    fx = _load("causal_rule.json")
    for c in fx["cases"]:
        E, L = c["start"] + c["T"], c["T"]
        for i, want in enumerate(c["visible"]):
            lo, hi = oracle.visible_range(E, L, i, True, 0)
            assert list(range(lo, hi)) == want, (c, i)


def pin_golden_slots():
    fx = _load("slots.json")
    bt = fx["paged"]["block_table"]
    for j, s in fx["paged"]["cases"]:
        assert oracle.paged_slot(bt, j) == s
    slots, ok = oracle.gather_slots_paged(np.array(bt), 41, 8)
    assert ok.all()
    for j, s in fx["paged"]["cases"]:
        assert int(slots[j]) == s
    r = fx["ring"]
    for pos, col, s in r["cases"]:
        assert oracle.ring_slot(pos, r["rows"], r["cols"], col) == s
    for n, s in fx["decode_append"]["cases"]:
        ident = np.arange((n + 15) // 16 + 1)
        assert int(oracle.paged_slots_for(ident[None, :], [0], [n - 1])[0]) == s
    r = fx["ring_unwritten"]
    pos, col, want = zip(*r["cases"])
    got = oracle.ring_slots_for(list(pos), list(col), r["rows"], r["cols"])
    assert got.tolist() == list(want)


def _golden_column(case, causal, window):
    q = np.array(case["q"], dtype=np.float32)[:, None, :]
    k = np.array(case["k"], dtype=np.float32)
    v = np.array(case["v"], dtype=np.float32)
    E, L = k.shape[0], q.shape[0]
    store_k = np.full((16, 1, 1, k.shape[1]), np.nan, np.float32)
    store_v = np.full((16, 1, 1, k.shape[1]), np.nan, np.float32)
    store_k[:E, 0, 0] = k
    store_v[:E, 0, 0] = v
    info = np.array([[0, L, 0, E]])
    return oracle.column_attention(q, store_k, store_v, info, dtype="f32", scale=case["scale"],
                                   causal=causal, window=window)[:, 0, :]


def pin_golden_closed_forms():
    fx = _load("closed_forms.json")
    c = fx["two_key"]
    np.testing.assert_allclose(_golden_column(c, False, 0), c["out"], atol=1e-12)
    c = fx["causal_offset"]
    np.testing.assert_allclose(_golden_column(c, True, 0), c["out"], atol=1e-12)
    c = fx["window_two"]
    np.testing.assert_allclose(_golden_column(c, True, c["window"]), c["out"], atol=1e-12)


def pin_window_span():
    """Ring of window + max_write - 1 rows holds exactly what a causal step sees."""
    for W in (1, 2, 5, 16):
        for T in (1, 2, 3, 7):
            start = 40
            E = start + T
            lows, highs = zip(*(oracle.visible_range(E, T, i, True, W) for i in range(T)))
            assert max(highs) - min(lows) == W + T - 1
            for i in range(T):
                lo, hi = oracle.visible_range(E, T, i, True, W)
                assert hi - lo == W


def pin_brute_force(seed=0):
    rng = np.random.default_rng(seed)
    for causal in (False, True):
        for window in (0, 1, 3, 17):
            for hq, hkv in ((2, 1), (4, 2), (2, 2)):
                lengths = [int(x) for x in rng.integers(1, 41, size=3)]
                q_lens = [int(rng.integers(1, min(4, E) + 1)) for E in lengths]
                d = 4
                case = make_paged_case(rng, lengths=lengths, q_lens=q_lens, hq=hq, hkv=hkv,
                                       d=d, dtype="f32", num_blocks=12, max_blocks=4)
                got = oracle.paged_attention(case["q"], case["k"], case["v"], case["table"],
                                             case["cu"], case["used"], dtype="f32", scale=0.7,
                                             causal=causal, window=window)
                for b, E in enumerate(lengths):
                    Kl, Vl = case["logical"][b]
                    qb = case["q"][case["cu"][b]:case["cu"][b + 1]]
                    ref = brute_unit(qb.astype(np.float64).tolist(), Kl.astype(np.float64).tolist(),
                                     Vl.astype(np.float64).tolist(), E, 0.7, causal, window)
                    np.testing.assert_allclose(got[case["cu"][b]:case["cu"][b + 1]], ref,
                                               atol=1e-12, rtol=0)


def pin_brute_force_column(seed=1):
    rng = np.random.default_rng(seed)
    rows, cols, hq, hkv, d = 12, 3, 4, 2, 4
    for causal in (False, True):
        for window in (0, 2, 5):
            q_lens = [1, 3, 2]
            ends = [9, 20, 30] if window else [9, 11, 7]   # ring wraps only under a window
            ks = garbage((rows, cols, hkv, d), "f32", "nan")
            vs = garbage((rows, cols, hkv, d), "f32", "nan")
            logical = []
            for s, E in enumerate(ends):
                Kl = rng.standard_normal((E, hkv, d)).astype(np.float32)
                Vl = rng.standard_normal((E, hkv, d)).astype(np.float32)
                place_ring(ks, s, Kl)
                place_ring(vs, s, Vl)
                logical.append((Kl, Vl))
            total_q = 10
            q = rng.standard_normal((total_q, hq, d)).astype(np.float32)
            info = np.array([[0, 1, 0, ends[0]], [2, 3, 1, ends[1]], [6, 2, 2, ends[2]]])
            got = oracle.column_attention(q, ks, vs, info, dtype="f32", scale=0.9,
                                          causal=causal, window=window)
            covered = set()
            for s, (q0, L, c, E) in enumerate(info.tolist()):
                Kl, Vl = logical[s]
                ref = brute_unit(q[q0:q0 + L].astype(np.float64).tolist(),
                                 Kl.astype(np.float64).tolist(), Vl.astype(np.float64).tolist(),
                                 E, 0.9, causal, window)
                np.testing.assert_allclose(got[q0:q0 + L], ref, atol=1e-12, rtol=0)
                covered.update(range(q0, q0 + L))
            for r in range(total_q):
                if r not in covered:
                    assert (got[r] == 0).all()


def pin_sdpa_noncausal_decode(seed=2):
    rng = np.random.default_rng(seed)
    hq, hkv, d, E = 8, 2, 16, 77
    case = make_paged_case(rng, lengths=[E], q_lens=[1], hq=hq, hkv=hkv, d=d, dtype="bf16",
                           num_blocks=8, max_blocks=8, identity=True)
    got = oracle.paged_attention(case["q"], case["k"], case["v"], case["table"], case["cu"],
                                 case["used"], dtype="bf16", scale=0.25)
    Kl, Vl = case["logical"][0]
    qt = torch.from_numpy(f64(case["q"], "bf16")).permute(1, 0, 2)[None]          # [1,Hq,1,D]
    kt = torch.from_numpy(f64(Kl, "bf16")).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)[None]
    vt = torch.from_numpy(f64(Vl, "bf16")).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.25)
    np.testing.assert_allclose(got, ref[0].permute(1, 0, 2).numpy(), atol=1e-12, rtol=0)


def pin_sdpa_causal_offset(seed=3):
    rng = np.random.default_rng(seed)
    hq, hkv, d = 4, 4, 8
    for start, T in ((5, 4), (17, 3), (0, 6)):
        E = start + T
        case = make_paged_case(rng, lengths=[E], q_lens=[T], hq=hq, hkv=hkv, d=d, dtype="f32",
                               num_blocks=4, max_blocks=4)
        got = oracle.paged_attention(case["q"], case["k"], case["v"], case["table"], case["cu"],
                                     case["used"], dtype="f32", scale=0.5, causal=True)
        Kl, Vl = case["logical"][0]
        qt = torch.from_numpy(case["q"].astype(np.float64)).permute(1, 0, 2)[None]
        kt = torch.from_numpy(Kl.astype(np.float64)).permute(1, 0, 2)[None]
        vt = torch.from_numpy(Vl.astype(np.float64)).permute(1, 0, 2)[None]
        q_pos = torch.arange(start, start + T)[:, None]
        k_pos = torch.arange(E)[None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=k_pos <= q_pos,
                                                               scale=0.5)
        np.testing.assert_allclose(got, ref[0].permute(1, 0, 2).numpy(), atol=1e-12, rtol=0)
        if start > 0 and T > 1:
            top_left = torch.nn.functional.scaled_dot_product_attention(
                qt, kt[:, :, :T], vt[:, :, :T], is_causal=True, scale=0.5)
            assert not np.allclose(got, top_left[0].permute(1, 0, 2).numpy(), atol=1e-6)


def pin_window1_gather(seed=4):
    """Causal window 1 with q_len = E: row i sees only key i, so out[i] is V[i] exactly."""
    rng = np.random.default_rng(seed)
    for dtype in ("bf16", "f32"):
        E = 45
        case = make_paged_case(rng, lengths=[E, 20], q_lens=[E, 20], hq=4, hkv=2, d=8,
                               dtype=dtype, num_blocks=12, max_blocks=4)
        got = oracle.paged_attention(case["q"], case["k"], case["v"], case["table"], case["cu"],
                                     case["used"], dtype=dtype, scale=1.3, causal=True, window=1)
        for b in range(2):
            Vl = f64(case["logical"][b][1], dtype)
            o = got[case["cu"][b]:case["cu"][b + 1]]
            for h in range(4):
                assert np.array_equal(o[:, h, :], Vl[:, h // 2, :])
    # the same through a wrapped ring column
    rows, E = 16, 50
    ks = garbage((rows, 2, 1, 4), "f32")
    vs = garbage((rows, 2, 1, 4), "f32")
    Vl = rng.standard_normal((E, 1, 4)).astype(np.float32)
    place_ring(ks, 1, rng.standard_normal((E, 1, 4)).astype(np.float32))
    place_ring(vs, 1, Vl)
    L = 16
    q = rng.standard_normal((L, 1, 4)).astype(np.float32)
    got = oracle.column_attention(q, ks, vs, np.array([[0, L, 1, E]]), dtype="f32", scale=1.0,
                                  causal=True, window=1)
    assert np.array_equal(got[:, 0, :], Vl[E - L:, 0, :].astype(np.float64))


def pin_single_key(seed=5):
    rng = np.random.default_rng(seed)
    case = make_paged_case(rng, lengths=[1, 1], q_lens=[1, 1], hq=4, hkv=1, d=8, dtype="bf16",
                           num_blocks=6, max_blocks=2)
    got = oracle.paged_attention(case["q"], case["k"], case["v"], case["table"], case["cu"],
                                 case["used"], dtype="bf16", scale=10.0)
    for b in range(2):
        Vl = f64(case["logical"][b][1], "bf16")
        for h in range(4):
            assert np.array_equal(got[b, h], Vl[0, 0])


def pin_permutation_invariance(seed=6):
    rng = np.random.default_rng(seed)
    lengths = [37, 5, 64]
    a = make_paged_case(np.random.default_rng(seed), lengths=lengths, q_lens=[1, 2, 3], hq=4,
                        hkv=2, d=8, dtype="bf16", num_blocks=10, max_blocks=4, identity=True)
    b = make_paged_case(np.random.default_rng(seed), lengths=lengths, q_lens=[1, 2, 3], hq=4,
                        hkv=2, d=8, dtype="bf16", num_blocks=10, max_blocks=4)
    for causal in (False, True):
        ra = oracle.paged_attention(a["q"], a["k"], a["v"], a["table"], a["cu"], a["used"],
                                    dtype="bf16", scale=0.4, causal=causal, window=9)
        rb = oracle.paged_attention(b["q"], b["k"], b["v"], b["table"], b["cu"], b["used"],
                                    dtype="bf16", scale=0.4, causal=causal, window=9)
        assert np.array_equal(ra, rb)
    del rng


def pin_garbage_invariance(seed=7):
    outs = []
    for kind in ("zero", "nan", "inf", "big"):
        c = make_paged_case(np.random.default_rng(seed), lengths=[23, 40], q_lens=[2, 1], hq=2,
                            hkv=1, d=4, dtype="bf16", num_blocks=9, max_blocks=5, tail=kind)
        if kind == "nan":
            c["table"][0, 2:] = -1
        outs.append(oracle.paged_attention(c["q"], c["k"], c["v"], c["table"], c["cu"],
                                           c["used"], dtype="bf16", scale=0.5, causal=True))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    assert np.isfinite(outs[0]).all()


def pin_uncovered_rows_zero(seed=8):
    rng = np.random.default_rng(seed)
    c = make_paged_case(rng, lengths=[30], q_lens=[2], hq=2, hkv=1, d=4, dtype="f32",
                        num_blocks=3, max_blocks=2)
    q = np.concatenate([c["q"], raw(rng.standard_normal((3, 2, 4)), "f32")])
    got = oracle.paged_attention(q, c["k"], c["v"], c["table"], c["cu"], c["used"], dtype="f32",
                                 scale=1.0)
    assert (got[2:] == 0).all() and (got[:2] != 0).any()
    # q_len beyond the static bound: rows past it are uncovered
    got2 = oracle.paged_attention(c["q"], c["k"], c["v"], c["table"], c["cu"], c["used"],
                                  dtype="f32", scale=1.0, max_seqlen_q=1)
    assert (got2[1] == 0).all() and np.array_equal(got2[0], got[0])
    # empty sequence, causal row before the first key
    got3 = oracle.paged_attention(c["q"], c["k"], c["v"], c["table"], c["cu"],
                                  np.array([0]), dtype="f32", scale=1.0)
    assert (got3 == 0).all()
    got4 = oracle.paged_attention(c["q"], c["k"], c["v"], c["table"], c["cu"],
                                  np.array([1]), dtype="f32", scale=1.0, causal=True)
    assert (got4[0] == 0).all() and (got4[1] != 0).any()


def pin_window_large_is_none(seed=9):
    c = make_paged_case(np.random.default_rng(seed), lengths=[50, 7], q_lens=[5, 3], hq=4, hkv=2,
                        d=8, dtype="bf16", num_blocks=8, max_blocks=4)
    for causal in (False, True):
        a = oracle.paged_attention(c["q"], c["k"], c["v"], c["table"], c["cu"], c["used"],
                                   dtype="bf16", scale=0.3, causal=causal)
        b = oracle.paged_attention(c["q"], c["k"], c["v"], c["table"], c["cu"], c["used"],
                                   dtype="bf16", scale=0.3, causal=causal, window=55)
        assert np.array_equal(a, b)


def pin_ring_equals_unrolled(seed=10):
    rng = np.random.default_rng(seed)
    rows, E, L, W = 10, 37, 3, 6
    Kl = rng.standard_normal((E, 2, 4)).astype(np.float32)
    Vl = rng.standard_normal((E, 2, 4)).astype(np.float32)
    ring_k = garbage((rows, 1, 2, 4), "f32")
    ring_v = garbage((rows, 1, 2, 4), "f32")
    place_ring(ring_k, 0, Kl)
    place_ring(ring_v, 0, Vl)
    flat_k = garbage((64, 1, 2, 4), "f32")
    flat_v = garbage((64, 1, 2, 4), "f32")
    flat_k[:E, 0] = Kl
    flat_v[:E, 0] = Vl
    q = rng.standard_normal((L, 4, 4)).astype(np.float32)
    info = np.array([[0, L, 0, E]])
    a = oracle.column_attention(q, ring_k, ring_v, info, dtype="f32", scale=0.6, causal=True,
                                window=W)
    b = oracle.column_attention(q, flat_k, flat_v, info, dtype="f32", scale=0.6, causal=True,
                                window=W)
    assert np.array_equal(a, b)


def pin_gqa_repeat(seed=11):
    rng = np.random.default_rng(seed)
    c = make_paged_case(rng, lengths=[33], q_lens=[2], hq=6, hkv=2, d=8, dtype="f32",
                        num_blocks=3, max_blocks=3)
    a = oracle.paged_attention(c["q"], c["k"], c["v"], c["table"], c["cu"], c["used"],
                               dtype="f32", scale=0.5, causal=True)
    kr = np.repeat(c["k"], 3, axis=2)
    vr = np.repeat(c["v"], 3, axis=2)
    b = oracle.paged_attention(c["q"], kr, vr, c["table"], c["cu"], c["used"], dtype="f32",
                               scale=0.5, causal=True)
    np.testing.assert_allclose(a, b, atol=1e-12, rtol=0)


def pin_closed_form_means(seed=12):
    rng = np.random.default_rng(seed)
    c = make_paged_case(rng, lengths=[29], q_lens=[1], hq=2, hkv=1, d=4, dtype="f32",
                        num_blocks=2, max_blocks=2, identity=True)
    # constant V -> that constant
    v = c["v"].copy()
    v[:, :, :, :] = np.float32(0.375)
    o = oracle.paged_attention(c["q"], c["k"], v, c["table"], c["cu"], c["used"], dtype="f32",
                               scale=2.0)
    np.testing.assert_allclose(o, 0.375, atol=1e-15, rtol=0)
    # q = 0 -> mean of visible V
    q0 = np.zeros_like(c["q"])
    o = oracle.paged_attention(q0, c["k"], c["v"], c["table"], c["cu"], c["used"], dtype="f32",
                               scale=2.0)
    mean = c["logical"][0][1].astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(o[0, 0], mean[0], atol=1e-12, rtol=0)
    # all keys equal -> mean of visible V
    k = c["k"].copy()
    k[:, :, :, :] = np.float32(-1.25)
    o = oracle.paged_attention(c["q"], k, c["v"], c["table"], c["cu"], c["used"], dtype="f32",
                               scale=2.0)
    np.testing.assert_allclose(o[0, 1], mean[0], atol=1e-12, rtol=0)


def pin_kv_append_bits():
    n, h, d = 6, 2, 3
    k = np.arange(n * h * d, dtype=np.uint16).reshape(n, h, d)
    v = (np.arange(n * h * d, dtype=np.uint16) + 1000).reshape(n, h, d)
    specials = np.array([0x7FC1, 0xFFFF, 0x7F81, 0x8000, 0x0001, 0xFF80], dtype=np.uint16)
    kn = np.stack([specials.reshape(h, d), specials[::-1].reshape(h, d), specials.reshape(h, d)])
    vn = kn[::-1].copy()
    ko, vo = oracle.kv_append(k, v, kn, vn, [4, -1, 6])
    assert np.array_equal(ko[4], kn[0]) and np.array_equal(vo[4], vn[0])
    untouched = [0, 1, 2, 3, 5]
    assert np.array_equal(ko[untouched], k[untouched]) and np.array_equal(vo[untouched], v[untouched])
    k32 = np.zeros((3, 1, 2), dtype=np.uint32)
    kn32 = np.array([[[0x7FA00001, 0xFFC00000]]], dtype=np.uint32)
    ko32, _ = oracle.kv_append(k32, k32, kn32, kn32, [2])
    assert ko32[2, 0, 0] == 0x7FA00001 and ko32[2, 0, 1] == 0xFFC00000


def pin_bf16_decode():
    """bfloat16 bit patterns with known values (IEEE binary32 upper halves)."""
    known = {0x3F80: 1.0, 0xC000: -2.0, 0x3FC0: 1.5, 0x0000: 0.0, 0x4049: 3.140625,
             0x7F80: np.inf, 0xFF80: -np.inf, 0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126}
    bits = np.array(list(known), dtype=np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    assert np.array_equal(got, np.array(list(known.values())))
    assert np.isnan(oracle.bf16_bits_to_f64(np.array([0x7FC0, 0xFFC1], dtype=np.uint16))).all()
    rnd = np.random.default_rng(13).integers(0, 0x7F80, size=4096).astype(np.uint16)
    assert np.array_equal(oracle.to_f64(rnd, "bf16"), f64(rnd, "bf16"))


def pin_golden_prefix_copy():
    """Hand-worked import through a permuted table, a block edge crossed at
    position 16, a tail past n left alone, and a sequence whose table names no
    pool block; the export reads the same values back (zero for that one)."""
    fx = _load("prefix_copy.json")
    H, D, S, n, nb = fx["kv_heads"], fx["head_dim"], fx["src_len"], fx["n"], fx["num_blocks"]
    bt = np.array(fx["block_table"], dtype=np.int32)
    B = bt.shape[0]
    b, h, j, d = np.meshgrid(np.arange(B), np.arange(H), np.arange(S), np.arange(D), indexing="ij")
    k_src = (1000 * b + 100 * h + 10 * j + d).astype(np.uint32)
    v_src = k_src + np.uint32(fx["v_offset"])
    fill = np.uint32(0xDEADBEEF)
    k_flat = np.full((nb * 16, H, D), fill, dtype=np.uint32)
    v_flat = np.full((nb * 16, H, D), fill, dtype=np.uint32)
    ko, vo = oracle.prefix_import(k_flat, v_flat, k_src, v_src, bt, n)
    hh, dd = np.meshgrid(np.arange(H), np.arange(D), indexing="ij")
    for sb, sj, slot in fx["written"]:
        want = 1000 * sb + 100 * hh + 10 * sj + dd
        assert np.array_equal(ko[slot], want) and np.array_equal(vo[slot], want + fx["v_offset"])
    for slot in fx["untouched_slots"]:
        assert (ko[slot] == fill).all() and (vo[slot] == fill).all()
    written = {slot for _, _, slot in fx["written"]}
    assert len(written) == len(fx["written"])
    ke, ve = oracle.prefix_export(ko, vo, bt, B, n)
    assert ke.shape == (B, H, n, D)
    for sb in range(B):
        if sb in fx["skipped_sequences"]:
            assert (ke[sb] == 0).all() and (ve[sb] == 0).all()
        else:
            assert np.array_equal(ke[sb], k_src[sb, :, :n]) and np.array_equal(ve[sb], v_src[sb, :, :n])


def pin_prefix_identity_is_transpose():
    """With one sequence and the identity table the import is the pages' flat
    copy of the [S, H, D] transpose into slots [:n], and the export the
    transpose back of slots [:n]; bf16 bit patterns including NaN payloads."""
    rng = np.random.default_rng(31)
    H, D, S, n = 3, 16, 45, 37
    k_src = rng.integers(0, 1 << 16, size=(1, H, S, D)).astype(np.uint16)
    v_src = rng.integers(0, 1 << 16, size=(1, H, S, D)).astype(np.uint16)
    k_src[0, 1, 3, :4] = [0x7FC1, 0xFF81, 0x7F80, 0x8000]
    k_flat = rng.integers(0, 1 << 16, size=(64, H, D)).astype(np.uint16)
    v_flat = rng.integers(0, 1 << 16, size=(64, H, D)).astype(np.uint16)
    ident = np.arange(4, dtype=np.int32)[None, :]
    ko, vo = oracle.prefix_import(k_flat, v_flat, k_src, v_src, ident, n)
    assert np.array_equal(ko[:n], np.transpose(k_src[0], (1, 0, 2))[:n])
    assert np.array_equal(vo[:n], np.transpose(v_src[0], (1, 0, 2))[:n])
    assert np.array_equal(ko[n:], k_flat[n:]) and np.array_equal(vo[n:], v_flat[n:])
    ke, ve = oracle.prefix_export(ko, vo, ident, 1, n)
    assert np.array_equal(ke, np.ascontiguousarray(np.transpose(ko[:n], (1, 0, 2)))[None])
    assert np.array_equal(ve, np.ascontiguousarray(np.transpose(vo[:n], (1, 0, 2)))[None])


def pin_prefix_roundtrip_permuted():
    """Three sequences on disjoint permuted pool blocks: export after import
    gives back the first n source positions, and exactly the slots the tables
    name for positions < n changed (the test finds them by comparing)."""
    rng = np.random.default_rng(32)
    B, H, D, S, n, nb = 3, 2, 8, 50, 41, 20
    perm = rng.permutation(nb).astype(np.int32)
    bt = perm[:B * 4].reshape(B, 4)
    k_src = rng.integers(0, 1 << 32, size=(B, H, S, D), dtype=np.uint64).astype(np.uint32)
    v_src = rng.integers(0, 1 << 32, size=(B, H, S, D), dtype=np.uint64).astype(np.uint32)
    k_flat = np.zeros((nb * 16, H, D), dtype=np.uint32) + np.uint32(7)
    v_flat = k_flat.copy()
    ko, vo = oracle.prefix_import(k_flat, v_flat, k_src, v_src, bt, n)
    ke, ve = oracle.prefix_export(ko, vo, bt, B, n)
    assert np.array_equal(ke, k_src[:, :, :n]) and np.array_equal(ve, v_src[:, :, :n])
    changed = np.flatnonzero((ko != 7).any(axis=(1, 2)))
    expect = sorted(int(bt[b, j // 16]) * 16 + j % 16 for b in range(B) for j in range(n))
    assert changed.tolist() == expect


def pin_golden_padded_mask():
    """The pages' left-padded causal rule, worked by hand, as key ranges; and
    through the paged oracle: a pad row's output is its own value row exactly."""
    fx = _load("padded_mask.json")
    for c in fx["cases"]:
        E, L, fv = c["start"] + c["T"], c["T"], c["first_valid"]
        for i, want in enumerate(c["visible"]):
            lo, hi = oracle.visible_range(E, L, i, True, 0, fv)
            assert list(range(lo, hi)) == want, (c, i)
    rng = np.random.default_rng(41)
    E, L, fv, D = 8, 4, 7, 8                     # rows at 4, 5, 6 are pad rows
    k = rng.standard_normal((16, 1, 1, D)).astype(np.float32)
    v = rng.standard_normal((16, 1, 1, D)).astype(np.float32)
    q = rng.standard_normal((L, 1, D)).astype(np.float32)
    out = oracle.paged_attention(q, k, v, np.array([[0]]), np.array([0, L]), np.array([E]),
                                 dtype="f32", scale=0.3, causal=True, kv_start=np.array([fv]))
    for i in range(3):
        assert np.array_equal(out[i, 0], v[4 + i, 0, 0].astype(np.float64))


def pin_left_padding_is_translation():
    """Valid rows over a left-padded prefix equal the same rows over the
    prefix with the pad keys cut off (no padding), causal and non-causal, with
    a window, through a permuted table; kv_start <= 0 is no padding."""
    rng = np.random.default_rng(42)
    Hq, Hkv, D, E, L, pad = 4, 2, 16, 45, 5, 13
    q = rng.standard_normal((L, Hq, D)).astype(np.float32)
    keys = rng.standard_normal((E, Hkv, D)).astype(np.float32)
    vals = rng.standard_normal((E, Hkv, D)).astype(np.float32)

    def paged(kk, vv, n, seed):
        nb = (n + 15) // 16 + 2
        perm = np.random.default_rng(seed).permutation(nb)
        kc = np.full((nb * 16, Hkv, D), np.nan, np.float32)
        vc = np.full((nb * 16, Hkv, D), np.nan, np.float32)
        for j in range(n):
            kc[perm[j // 16] * 16 + j % 16] = kk[j]
            vc[perm[j // 16] * 16 + j % 16] = vv[j]
        return kc, vc, perm[None, :]

    kc, vc, bt = paged(keys, vals, E, 1)
    kt, vt, btt = paged(keys[pad:], vals[pad:], E - pad, 2)
    for causal, window in ((True, 0), (False, 0), (True, 30), (False, 30)):
        a = oracle.paged_attention(q, kc, vc, bt, np.array([0, L]), np.array([E]), dtype="f32",
                                   scale=0.25, causal=causal, window=window, kv_start=np.array([pad]))
        b = oracle.paged_attention(q, kt, vt, btt, np.array([0, L]), np.array([E - pad]), dtype="f32",
                                   scale=0.25, causal=causal, window=window)
        assert np.allclose(a, b, rtol=0, atol=1e-12), (causal, window)
        none = oracle.paged_attention(q, kc, vc, bt, np.array([0, L]), np.array([E]), dtype="f32",
                                      scale=0.25, causal=causal, window=window)
        for ks in (0, -3):
            z = oracle.paged_attention(q, kc, vc, bt, np.array([0, L]), np.array([E]), dtype="f32",
                                       scale=0.25, causal=causal, window=window, kv_start=np.array([ks]))
            assert np.array_equal(z, none)


def _brute_rows(q, K, V, E, scale, causal, window, ok=None):
    return np.array(brute_unit(q.tolist(), K.tolist(), V.tolist(), E, scale, causal, window, ok))


def pin_multichunk_rows(seed=13):
    """Units of up to 130 rows, taken 1, 3, 7 or 64 rows at a time by the
    oracle, against the brute force: every row, across chunk edges."""
    rng = np.random.default_rng(seed)
    for L, E, causal, window, chunk in ((130, 150, True, 0, 64), (130, 140, True, 9, 7),
                                        (67, 67, False, 0, 3), (65, 90, True, 40, 64),
                                        (20, 31, False, 5, 1), (129, 129, True, 0, 64)):
        Hq, Hkv, D = 2, 1, 3
        q = rng.standard_normal((L, Hq, D))
        K = rng.standard_normal((E, Hkv, D))
        V = rng.standard_normal((E, Hkv, D))
        want = _brute_rows(q, K, V, E, 0.7, causal, window)
        got = oracle.attend_unit(q, K, V, np.ones(E, bool), E, 0.7, causal, window, chunk=chunk)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12, err_msg=f"L={L} chunk={chunk}")


def pin_hidden_nonfinite(seed=14):
    """A NaN (or Inf) in a live key that some rows cannot see.  The oracle
    computes each row from the keys it sees (brute force selects exactly
    those): rows that cannot see it come out finite and equal to the brute
    force, a row that sees a NaN V comes out NaN.  The unspecified mask flags
    exactly the rows that cannot see a non-finite V another row sees, for the
    kv head that holds it; a non-finite key no row sees flags nothing."""
    rng = np.random.default_rng(seed)
    L, E, Hq, Hkv, D = 6, 20, 4, 2, 3
    q = rng.standard_normal((L, Hq, D))
    for what, bad_key, bad_head, causal, window, val in (
            ("V", E - 1, 1, True, 0, np.nan), ("K", E - 2, 0, True, 0, np.nan),
            ("V", E - 3, 0, True, 0, np.inf), ("V", 0, 1, True, 8, np.nan)):
        K = rng.standard_normal((E, Hkv, D))
        V = rng.standard_normal((E, Hkv, D))
        (V if what == "V" else K)[bad_key, bad_head, 1] = val
        want = _brute_rows(q, K, V, E, 0.5, causal, window)
        got = oracle.attend_unit(q, K, V, np.ones(E, bool), E, 0.5, causal, window)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12, equal_nan=True)
        flags = oracle.hidden_nonfinite(V, np.ones(E, bool), E, L, causal, window)
        expect = np.zeros((L, Hkv), bool)
        seen_by = [oracle.visible_range(E, L, i, causal, window) for i in range(L)]
        some_row_sees = any(lo <= bad_key < hi for lo, hi in seen_by)
        if what == "V" and some_row_sees:
            for i, (lo, hi) in enumerate(seen_by):
                expect[i, bad_head] = not (lo <= bad_key < hi)
        assert np.array_equal(flags, expect), (what, bad_key, flags, expect)
        for i, (lo, hi) in enumerate(seen_by):
            g = slice(bad_head * (Hq // Hkv), (bad_head + 1) * (Hq // Hkv))
            sees = lo <= bad_key < hi
            assert np.isnan(got[i, g]).any() == (sees and np.isnan(val) or (sees and what == "K")), (what, i)
    # through the paged entry point: the mask lands on the unit's rows and the kv head's q heads
    K = rng.standard_normal((32, 1, Hkv, D)).astype(np.float32)
    V = rng.standard_normal((32, 1, Hkv, D)).astype(np.float32)
    pool_k = np.full((2, 16, Hkv, D), 7.0, np.float32)
    pool_v = np.full((2, 16, Hkv, D), 7.0, np.float32)
    pool_k.reshape(32, Hkv, D)[:E] = K[:E, 0]
    pool_v.reshape(32, Hkv, D)[:E] = V[:E, 0]
    pool_v.reshape(32, Hkv, D)[E - 1, 1, 0] = np.nan
    qq = rng.standard_normal((L + 1, Hq, D)).astype(np.float32)
    out, unspec = oracle.paged_attention(qq, pool_k, pool_v, np.array([[0, 1]]), np.array([1, L + 1]),
                                         np.array([E]), dtype="f32", scale=0.5, causal=True,
                                         with_unspecified=True)
    assert unspec.shape == (L + 1, Hq)
    assert not unspec[0].any() and not unspec[L].any()
    assert unspec[1:L, 2:].all() and not unspec[1:L, :2].any()
    assert np.isnan(out[L, 2:, 0]).all() and np.isfinite(out[:L]).all()


def pin_compare_known_answer():
    """compare() on values worked by hand: errors over finite references only,
    NaN placement, the skip mask."""
    got = np.array([1.0, 2.0, np.nan, 4.0])
    ref = np.array([1.0, 2.5, np.nan, 3.0])
    c = oracle.compare(got, ref)
    # |d| over the finite references = (0, 0.5, 1); RMS ratio sqrt(1.25 / 16.25) = sqrt(1/13)
    assert c["max_abs"] == 1.0 and abs(c["rms_rel"] - (1 / 13) ** 0.5) < 1e-15
    assert c["finite"] and c["nan_match"]
    c = oracle.compare(np.array([1.0, np.nan, 3.0]), np.array([1.0, 2.0, 3.0]))
    assert not c["finite"] and not c["nan_match"] and np.isnan(c["max_abs"])
    c = oracle.compare(np.array([1.0, 2.0, 3.0]), np.array([1.0, np.nan, 3.0]))
    assert c["finite"] and not c["nan_match"] and c["max_abs"] == 0.0
    g2 = np.array([[[0.0, 9.0]], [[np.nan, 1.0]]])      # [rows, heads, d]
    r2 = np.array([[[0.0, 1.0]], [[5.0, 1.0]]])
    c = oracle.compare(g2, r2, skip=np.array([[False], [True]]))
    assert c["max_abs"] == 8.0 and c["finite"] and c["nan_match"]
    c = oracle.compare(g2, r2, skip=np.array([[True], [True]]))
    assert c["max_abs"] == 0.0 and c["rms_rel"] == 0.0


def pin_storage_missing_in_live_range(seed=15):
    """Block-table entries outside the pool inside the live range: those 16
    keys drop out of every row (brute force with the keys left out), and a
    row whose visible keys all lack storage is 0."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, E, L = 2, 1, 4, 60, 12
    K = rng.standard_normal((E, Hkv, D)).astype(np.float32)
    V = rng.standard_normal((E, Hkv, D)).astype(np.float32)
    table = np.array([[3, -1, 0, 0x7FFFFFFF]])           # keys 16..31 and 48..59 without storage
    table[0, 2] = 1
    pool_k = np.full((4, 16, Hkv, D), np.nan, np.float32)
    pool_v = np.full((4, 16, Hkv, D), np.nan, np.float32)
    pool_k[3, :] = K[:16]
    pool_v[3, :] = V[:16]
    pool_k[1, :] = K[32:48]
    pool_v[1, :] = V[32:48]
    ok = np.array([(j < 16) or (32 <= j < 48) for j in range(E)])
    q = rng.standard_normal((L, Hq, D)).astype(np.float32)
    for causal, window in ((True, 0), (False, 0), (True, 10)):
        got = oracle.paged_attention(q, pool_k, pool_v, table, np.array([0, L]), np.array([E]), dtype="f32",
                                     scale=0.3, causal=causal, window=window)
        want = _brute_rows(q.astype(np.float64), K.astype(np.float64), V.astype(np.float64), E, 0.3,
                           causal, window, ok)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
        if window == 10:           # the last rows see keys 50..59 only: all without storage
            assert np.array_equal(got[-1], np.zeros((Hq, D)))


ALL_PINS = [
    pin_bf16_decode,
    pin_golden_causal_rule, pin_golden_slots, pin_golden_closed_forms, pin_window_span,
    pin_brute_force, pin_brute_force_column, pin_sdpa_noncausal_decode, pin_sdpa_causal_offset,
    pin_window1_gather, pin_single_key, pin_permutation_invariance, pin_garbage_invariance,
    pin_uncovered_rows_zero, pin_window_large_is_none, pin_ring_equals_unrolled, pin_gqa_repeat,
    pin_closed_form_means, pin_kv_append_bits,
    pin_golden_prefix_copy, pin_prefix_identity_is_transpose, pin_prefix_roundtrip_permuted,
    pin_golden_padded_mask, pin_left_padding_is_translation,
    pin_multichunk_rows, pin_hidden_nonfinite, pin_compare_known_answer,
    pin_storage_missing_in_live_range,
]


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    pin()


# ---------------------------------------------------------------------------
# Planted mistakes: each must make at least one pin fail.
# ---------------------------------------------------------------------------

def _top_left_causal(E, L, i, causal, window, kv_start=0):
    p = i
    hi = min(E, p + 1) if causal else E
    lo = max(0, p - window + 1) if window > 0 else 0
    return lo, max(lo, hi)


def _window_off_by_one(E, L, i, causal, window, kv_start=0):
    p = E - L + i
    hi = min(E, p + 1) if causal else E
    lo = max(0, p - window) if window > 0 else 0
    return lo, max(lo, hi)


def _causal_excludes_self(E, L, i, causal, window, kv_start=0):
    p = E - L + i
    hi = min(E, p) if causal else E
    lo = max(0, p - window + 1) if window > 0 else 0
    return lo, max(lo, hi)


_real_gather = oracle.gather_slots_paged


def _gather_transposed(row, E, nb):
    slots, ok = _real_gather(row, E, nb)
    jj = np.arange(E)
    blk = np.asarray(row).astype(np.int64)[jj // 16]
    return np.where(ok, blk * 16 + (15 - jj % 16), 0), ok


def _gather_no_table(row, E, nb):
    jj = np.arange(E)
    return jj.astype(np.int64), np.ones(E, dtype=bool)


_real_attend = oracle.attend_unit


def _attend_no_scale(q, keys, vals, ok, E, scale, causal, window, chunk=64, kv_start=0):
    return _real_attend(q, keys, vals, ok, E, 1.0, causal, window, chunk, kv_start)


def _attend_swapped_kv(q, keys, vals, ok, E, scale, causal, window, chunk=64, kv_start=0):
    return _real_attend(q, vals, keys, ok, E, scale, causal, window, chunk, kv_start)


def _attend_last_kv_head(q, keys, vals, ok, E, scale, causal, window, chunk=64, kv_start=0):
    return _real_attend(q, keys[:, ::-1], vals[:, ::-1], ok, E, scale, causal, window, chunk, kv_start)


_real_ring = oracle.ring_slot


_real_import = oracle.prefix_import
_real_export = oracle.prefix_export


def _import_heads_reversed(kf, vf, ks, vs, bt, n):
    return _real_import(kf, vf, ks[:, ::-1], vs[:, ::-1], bt, n)


def _import_kv_swapped(kf, vf, ks, vs, bt, n):
    return _real_import(kf, vf, vs, ks, bt, n)


def _import_one_extra(kf, vf, ks, vs, bt, n):
    return _real_import(kf, vf, ks, vs, bt, min(n + 1, ks.shape[2]))


def _import_s_h_mixed(kf, vf, ks, vs, bt, n):
    B, H, S, D = ks.shape
    return _real_import(kf, vf, ks.reshape(B, S, H, D).transpose(0, 2, 1, 3),
                        vs.reshape(B, S, H, D).transpose(0, 2, 1, 3), bt, n)


def _export_shifted(kf, vf, bt, B, n):
    ke, ve = _real_export(kf, vf, bt, B, n + 1)
    return ke[:, :, 1:], ve[:, :, 1:]


_real_visible = oracle.visible_range


def _padding_ignored(E, L, i, causal, window, kv_start=0):
    return _real_visible(E, L, i, causal, window, 0)


def _pad_rows_see_nothing(E, L, i, causal, window, kv_start=0):
    if kv_start > 0 and E - L + i < kv_start:
        return 0, 0
    return _real_visible(E, L, i, causal, window, kv_start)


def _padding_off_by_one(E, L, i, causal, window, kv_start=0):
    return _real_visible(E, L, i, causal, window, kv_start + 1 if kv_start > 0 else 0)


_real_chunks = oracle._attend_chunks


def _chunk_drops_last_row(q, keys, vals, key_ok, ranges, scale, G, Hkv, D, L, chunk, out):
    """Each chunk of rows stops one row short (an off-by-one at the chunk edge)."""
    for c0 in range(0, L, chunk):
        sub = [r if c0 <= i < min(L, c0 + chunk - 1) else (0, 0) for i, r in enumerate(ranges)]
        _real_chunks(q, keys, vals, key_ok, sub, scale, G, Hkv, D, L, chunk, out)


def _chunk_no_fallback(q, keys, vals, key_ok, ranges, scale, G, Hkv, D, L, chunk, out):
    """Hidden non-finite keys not special-cased (0 * NaN leaks into rows)."""
    with np.errstate(invalid="ignore"):
        for c0 in range(0, L, chunk):
            rows = [i for i in range(c0, min(L, c0 + chunk)) if ranges[i][1] > ranges[i][0]]
            if not rows:
                continue
            lo_c = min(ranges[i][0] for i in rows)
            hi_c = max(ranges[i][1] for i in rows)
            j = np.arange(lo_c, hi_c)
            mask = np.stack([(j >= ranges[i][0]) & (j < ranges[i][1]) for i in rows]) & key_ok[lo_c:hi_c][None, :]
            for g in range(Hkv):
                hs = slice(g * G, (g + 1) * G)
                s = scale * np.einsum("rgd,kd->rgk", q[rows][:, hs, :], keys[lo_c:hi_c, g, :])
                s = np.where(mask[:, None, :], s, -np.inf)
                m = s.max(axis=2, keepdims=True)
                w = np.exp(s - m)
                out[rows, hs, :] = (w @ vals[lo_c:hi_c, g, :]) / w.sum(axis=2, keepdims=True)


def _flags_never(vals, key_ok, E, L, causal, window, kv_start=0):
    return np.zeros((L, vals.shape[1] if vals.ndim == 3 else 0), dtype=bool)


_real_compare = oracle.compare


def _compare_all_elements(got, ref, skip=None):
    c = _real_compare(got, ref, skip)
    d = np.abs(np.asarray(got, float) - np.asarray(ref, float))
    c["max_abs"] = float(np.nanmax(d)) if d.size else 0.0
    return c


def _compare_ignores_nan(got, ref, skip=None):
    c = _real_compare(got, ref, skip)
    c["nan_match"] = True
    return c


def _ring_slots_no_skip(pos, col, rows, cols):
    return np.array([(p % rows) * cols + c for p, c in zip(pos, col)], dtype=np.int64)


def _storage_ignored(row, E, nb):
    slots, ok = _real_gather(row, E, nb)
    return slots, np.ones_like(ok)


MUTANTS = [
    ("visible_range", _top_left_causal),
    ("visible_range", _window_off_by_one),
    ("visible_range", _causal_excludes_self),
    ("gather_slots_paged", _gather_transposed),
    ("gather_slots_paged", _gather_no_table),
    ("attend_unit", _attend_no_scale),
    ("attend_unit", _attend_swapped_kv),
    ("attend_unit", _attend_last_kv_head),
    ("ring_slot", lambda p, rows, cols, col: (p % rows) + col * rows),
    ("bf16_bits_to_f64", lambda b: (np.asarray(b).astype(np.uint32) << 15).view(np.float32)
     .astype(np.float64)),
    ("prefix_import", _import_heads_reversed),
    ("prefix_import", _import_kv_swapped),
    ("prefix_import", _import_one_extra),
    ("prefix_import", _import_s_h_mixed),
    ("prefix_export", _export_shifted),
    ("paged_slot", lambda row, j: int(row[j // 16]) * 16 + 15 - j % 16),
    ("visible_range", _padding_ignored),
    ("visible_range", _pad_rows_see_nothing),
    ("visible_range", _padding_off_by_one),
    ("_attend_chunks", _chunk_drops_last_row),
    ("_attend_chunks", _chunk_no_fallback),
    ("hidden_nonfinite", _flags_never),
    ("compare", _compare_all_elements),
    ("compare", _compare_ignores_nan),
    ("ring_slots_for", _ring_slots_no_skip),
    ("gather_slots_paged", _storage_ignored),
]


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=[f"{n}-{i}" for i, (n, _) in enumerate(MUTANTS)])
def test_planted_mistake_is_caught(monkeypatch, name, mutant):
    monkeypatch.setattr(oracle, name, mutant)
    failed = []
    for pin in ALL_PINS:
        try:
            pin()
        except (AssertionError, IndexError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake in {name}"
