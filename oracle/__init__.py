"""CPU fp64 oracle for paged / column-store decode attention.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library and imports nothing from it.

What it computes is the plain definition the pages describe, written out
without blocking, splitting or fusion:

* append -- vLLM-Omni ``paged_decode.py``, ``PagedDecodeCache.attend``: this
  step's K and V rows are copied into the flat slot view of the per-layer
  paged K/V before attention; ExecuTorch PR #24073 (the #24074 part): the
  in-graph write goes to slot ``(position % rows) * columns + column``.
* addressing -- ``PagedDecodeCache`` class docstring: the cache is laid out
  ``(num_blocks, BLOCK_SIZE, kv_heads, head_dim)`` and read through a block
  table, BLOCK_SIZE 16; only the first ``seqused`` keys are live.
* attention -- ``flash_attn_varlen_func`` as called from ``attend``:
  ``softmax(q K^T * softmax_scale) V`` over the live prefix; the causal rule
  of tiny-llm ``kv_cache.py`` ``causal_kwargs`` (query i of T new tokens over
  start+T keys sees keys 0..start+i); the ``sdpa_varlen`` segment table,
  sliding window, ring storage and zeroed uncovered rows of ExecuTorch PR
  #24073 (the #24072 part).
* prefix import / export -- ``PagedDecodeCache.load_prefix``,
  ``_write_prefix`` and ``to_dynamic_cache``: a dense prefill cache
  ``[B, Hkv, S, D]`` to and from the slots of the paged cache, raw bits.

Readings taken where the pages are silent (each is also listed with its
support in the design notes):
* the live length counts this step's new tokens (append comes first);
* causal alignment is bottom-right: row i of a unit with L rows and E keys
  sits at position ``p = E - L + i``;
* a window W shows keys ``p - W + 1 .. p`` (W keys including the query);
* a left-padding bound ``kv_start > 0`` (per sequence or segment) hides the
  keys before it; a row at a position before it sees only its own key (the
  diagonal the pages always keep), also without ``causal``; ``kv_start <= 0``
  is no padding;
* GQA: q head h reads kv head ``h // (Hq // Hkv)``;
* a row with no visible key, and a row no unit covers, is 0;
* paged ``seqused_k`` is clamped to ``[0, min(max_seqlen_k, 16*max_blocks)]``;
  column ``kv_end`` below 0 counts as 0;
* a live key whose block-table entry lies outside ``[0, num_blocks)``, or a
  segment whose column lies outside ``[0, cols)``, contributes no keys;
* a non-finite V value in a live key that one row of a unit sees and another
  row of the same unit does not (causal, window or padding rule) leaves the
  output of the row that does not see it unspecified: a dense masked product
  multiplies it by a zero weight.  The oracle computes that row from its
  visible keys and, when asked, reports it in an ``unspecified`` mask
  ``[total_q, Hq]`` that comparisons skip;
* query rows of a unit past ``max_seqlen_q`` are treated as uncovered (0);
* ``kv_append`` skips slots outside ``[0, num_slots)`` and copies raw bits;
* prefix import takes the same rule; prefix export writes zero bits for a
  position whose slot lies outside the cache.
"""
from __future__ import annotations

import numpy as np

BLOCK_SIZE = 16

# --------------------------------------------------------------------------
# Element decoding: raw storage bits -> exact float64.
# --------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the upper half of an IEEE binary32: widen exactly."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """``dtype`` 'bf16': ``arr`` holds uint16 bit patterns; 'f32': float32 values."""
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# Append: raw-bit scatter into the flat slot view.
# --------------------------------------------------------------------------


def kv_append(k_flat: np.ndarray, v_flat: np.ndarray, k_new: np.ndarray,
              v_new: np.ndarray, slots) -> tuple[np.ndarray, np.ndarray]:
    """Return copies of the flat caches ``[num_slots, Hkv, D]`` after writing
    row ``t`` of ``k_new``/``v_new`` to slot ``slots[t]``, in order.

    The arrays are integer bit views (uint16 for bf16, uint32 for fp32), so
    NaN payloads and signalling bits are moved untouched.  Slots outside
    ``[0, num_slots)`` are skipped.
    """
    k_out = np.array(k_flat, copy=True)
    v_out = np.array(v_flat, copy=True)
    n = k_out.shape[0]
    for t, s in enumerate(np.asarray(slots).tolist()):
        if 0 <= s < n:
            k_out[s] = k_new[t]
            v_out[s] = v_new[t]
    return k_out, v_out


# --------------------------------------------------------------------------
# Addressing.
# --------------------------------------------------------------------------


def paged_slot(block_table_row, j: int) -> int:
    """Flat slot of logical key ``j``: block ``table[j // 16]``, row ``j % 16``."""
    return int(block_table_row[j // BLOCK_SIZE]) * BLOCK_SIZE + (j % BLOCK_SIZE)


def ring_slot(position: int, rows: int, cols: int, col: int) -> int:
    """Flat slot of ``position`` in column ``col`` of a ``[rows, cols]`` ring store."""
    return (position % rows) * cols + col


def paged_slots_for(block_table: np.ndarray, seq_of_token, pos_of_token) -> np.ndarray:
    """Append slots for new tokens given (sequence, logical position)."""
    out = np.empty(len(pos_of_token), dtype=np.int64)
    for t, (b, p) in enumerate(zip(np.asarray(seq_of_token).tolist(),
                                   np.asarray(pos_of_token).tolist())):
        out[t] = paged_slot(block_table[b], p)
    return out


def ring_slots_for(pos_of_token, col_of_token, rows: int, cols: int) -> np.ndarray:
    out = np.empty(len(pos_of_token), dtype=np.int64)
    for t, (p, c) in enumerate(zip(np.asarray(pos_of_token).tolist(),
                                   np.asarray(col_of_token).tolist())):
        out[t] = ring_slot(p, rows, cols, c) if p >= 0 and c >= 0 else -1
    return out


def gather_slots_paged(block_table_row, E: int, num_blocks: int):
    """Flat slots of logical keys ``0..E-1`` through one block-table row, and
    whether each key's block id is a real pool block (only the first
    ``ceil(E / 16)`` entries are read)."""
    jj = np.arange(E)
    if E == 0:
        return np.zeros(0, dtype=np.int64), np.zeros(0, dtype=bool)
    blk = np.asarray(block_table_row).astype(np.int64)[jj // BLOCK_SIZE]
    ok = (blk >= 0) & (blk < num_blocks)
    return np.where(ok, blk * BLOCK_SIZE + jj % BLOCK_SIZE, 0), ok


# --------------------------------------------------------------------------
# Masks.
# --------------------------------------------------------------------------


def visible_range(E: int, L: int, i: int, causal: bool, window: int,
                  kv_start: int = 0) -> tuple[int, int]:
    """Half-open key range ``[lo, hi)`` that row ``i`` of ``L`` new queries sees
    over ``E`` keys.  The row sits at position ``p = E - L + i``.

    ``kv_start > 0`` is a left-padding bound (tiny-llm ``kv_cache.py``,
    ``padded_causal_mask`` and the module docstring): keys before it are
    hidden, and a query before it (a pad query) still sees its own key, so no
    row is left without keys.
    """
    p = E - L + i
    if kv_start > 0 and p < kv_start:
        lo, hi = max(p, 0), min(p + 1, E)
        return lo, max(lo, hi)
    hi = min(E, p + 1) if causal else E
    lo = max(0, p - window + 1) if window > 0 else 0
    lo = max(lo, kv_start)
    return lo, max(lo, hi)


# --------------------------------------------------------------------------
# Attention over one unit (a sequence, or a segment) with its keys gathered.
# --------------------------------------------------------------------------


def hidden_nonfinite(vals: np.ndarray, key_ok: np.ndarray, E: int, L: int, causal: bool,
                     window: int, kv_start: int = 0) -> np.ndarray:
    """bool [L, Hkv]: row ``i`` and kv head ``g`` have a live key with storage
    whose V row (head ``g``) holds a non-finite value, that row ``i`` does not
    see while some other row of the unit does.  Such a row's output is
    unspecified (see the module docstring)."""
    Hkv = vals.shape[1] if vals.ndim == 3 else 0
    flags = np.zeros((L, Hkv), dtype=bool)
    if L == 0 or E <= 0:
        return flags
    ranges = [visible_range(E, L, i, causal, window, kv_start) for i in range(L)]
    seen = np.zeros(E, dtype=bool)
    for lo, hi in ranges:
        seen[lo:hi] = True
    seen &= np.asarray(key_ok, dtype=bool)
    bad = seen[:, None] & ~np.isfinite(vals).all(axis=2)          # [E, Hkv]
    if not bad.any():
        return flags
    for i, (lo, hi) in enumerate(ranges):
        hidden = np.ones(E, dtype=bool)
        hidden[lo:hi] = False
        flags[i] = (bad & hidden[:, None]).any(axis=0)
    return flags


def attend_unit(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, key_ok: np.ndarray,
                E: int, scale: float, causal: bool, window: int,
                chunk: int = 64, kv_start: int = 0) -> np.ndarray:
    """softmax(q K^T * scale) V for the ``L`` query rows of one unit.

    q      float64 [L, Hq, D]
    keys   float64 [E, Hkv, D]  logical keys 0..E-1 (entries outside ``key_ok`` unused)
    vals   float64 [E, Hkv, D]
    key_ok bool [E]  keys that have storage (see the block-id rule above)
    kv_start  left-padding bound of the unit (see ``visible_range``)
    Returns float64 [L, Hq, D]; a row with no visible key is 0.

    Rows are taken ``chunk`` at a time over the union of their key ranges with
    a per-row visibility mask: a hidden key gets score -inf and weight exactly
    0.  Where a hidden key holds a non-finite value (0 * NaN would leak), the
    chunk falls back to selecting each row's visible keys one row at a time.
    """
    L, Hq, D = q.shape
    Hkv = keys.shape[1]
    G = Hq // Hkv
    out = np.zeros((L, Hq, D), dtype=np.float64)
    if L == 0 or E <= 0:
        return out
    key_ok = np.asarray(key_ok, dtype=bool)
    ranges = [visible_range(E, L, i, causal, window, kv_start) for i in range(L)]
    with np.errstate(invalid="ignore", over="ignore"):
        _attend_chunks(q, keys, vals, key_ok, ranges, scale, G, Hkv, D, L, chunk, out)
    return out


def _attend_chunks(q, keys, vals, key_ok, ranges, scale, G, Hkv, D, L, chunk, out):
    for c0 in range(0, L, chunk):
        rows = [i for i in range(c0, min(L, c0 + chunk)) if ranges[i][1] > ranges[i][0]]
        if not rows:
            continue
        lo_c = min(ranges[i][0] for i in rows)
        hi_c = max(ranges[i][1] for i in rows)
        j = np.arange(lo_c, hi_c)
        mask = np.stack([(j >= ranges[i][0]) & (j < ranges[i][1]) for i in rows])
        mask &= key_ok[lo_c:hi_c][None, :]
        Kc = keys[lo_c:hi_c]
        Vc = vals[lo_c:hi_c]
        seen_by_all = mask.all(axis=0)
        seen_by_some = mask.any(axis=0)
        finite = np.isfinite(Kc).all(axis=(1, 2)) & np.isfinite(Vc).all(axis=(1, 2))
        if (seen_by_some & ~seen_by_all & ~finite).any():
            for i in rows:
                idx = lo_c + np.nonzero(mask[rows.index(i)])[0]
                if idx.size == 0:
                    continue
                for g in range(Hkv):
                    hs = slice(g * G, (g + 1) * G)
                    s = scale * (q[i, hs, :] @ keys[idx, g, :].T)
                    w = np.exp(s - s.max(axis=1, keepdims=True))
                    out[i, hs, :] = (w @ vals[idx, g, :]) / w.sum(axis=1, keepdims=True)
            continue
        any_vis = mask.any(axis=1)
        for g in range(Hkv):
            hs = slice(g * G, (g + 1) * G)
            qg = q[rows][:, hs, :]                                  # [r, G, D]
            nr = len(rows)
            s = scale * (qg.reshape(nr * G, D) @ Kc[:, g, :].T).reshape(nr, G, -1)
            s = np.where(mask[:, None, :], s, -np.inf)
            m = s.max(axis=2, keepdims=True)
            m = np.where(any_vis[:, None, None], m, 0.0)
            w = np.exp(s - m)                                        # hidden -> 0
            Vg = np.where(seen_by_some[:, None], Vc[:, g, :], 0.0)
            num = (w.reshape(nr * G, -1) @ Vg).reshape(nr, G, D)
            den = w.sum(axis=2, keepdims=True)
            res = np.where(any_vis[:, None, None], num / np.where(den > 0, den, 1.0), 0.0)
            out[rows, hs, :] = res


# --------------------------------------------------------------------------
# Paged mode: cu_seqlens_q + seqused_k + block_table.
# --------------------------------------------------------------------------


def paged_attention(q, k_cache, v_cache, block_table, cu_seqlens_q, seqused_k, *,
                    dtype: str, scale: float, causal: bool = False, window: int = 0,
                    max_seqlen_q: int | None = None, max_seqlen_k: int | None = None,
                    seqs=None, kv_start=None, with_unspecified: bool = False):
    """Oracle for varlen attention over a paged cache.

    q        raw [total_q, Hq, D]          (bits for bf16, float32 for f32)
    k_cache  raw [num_blocks, 16, Hkv, D]  (or any view with a flat slot axis)
    block_table int [num_seqs, max_blocks]; cu_seqlens_q int [num_seqs+1];
    seqused_k int [num_seqs].  ``seqs`` restricts the work to some sequences
    (the other rows are left 0, as uncovered rows are).  ``kv_start`` int
    [num_seqs] or None: each sequence's left-padding bound.
    Returns float64 [total_q, Hq, D]; with ``with_unspecified`` also the bool
    mask [total_q, Hq] of outputs the module docstring leaves unspecified.
    """
    q = np.asarray(q)
    total_q, Hq, D = q.shape
    k_flat = np.asarray(k_cache).reshape(-1, np.asarray(k_cache).shape[-2], D)
    v_flat = np.asarray(v_cache).reshape(-1, np.asarray(v_cache).shape[-2], D)
    num_slots = k_flat.shape[0]
    num_blocks = num_slots // BLOCK_SIZE
    block_table = np.asarray(block_table).astype(np.int64)
    cu = np.asarray(cu_seqlens_q).astype(np.int64)
    used = np.asarray(seqused_k).astype(np.int64)
    num_seqs, max_blocks = block_table.shape
    cap = max_blocks * BLOCK_SIZE
    if max_seqlen_k is not None:
        cap = min(cap, int(max_seqlen_k))
    out = np.zeros((total_q, Hq, D), dtype=np.float64)
    unspec = np.zeros((total_q, Hq), dtype=bool)
    for b in (range(num_seqs) if seqs is None else seqs):
        start, stop = int(cu[b]), int(cu[b + 1])
        L = stop - start
        if L <= 0:
            continue
        E = int(min(max(used[b], 0), cap))
        n_rows = L if max_seqlen_q is None else min(L, int(max_seqlen_q))
        # Gather the logical prefix 0..E-1 through the block table.
        slots, ok = gather_slots_paged(block_table[b], E, num_blocks)
        keys = to_f64(k_flat[slots], dtype)
        vals = to_f64(v_flat[slots], dtype)
        qq = to_f64(q[start:stop], dtype)
        ks = 0 if kv_start is None else int(kv_start[b])
        res = attend_unit(qq, keys, vals, ok, E, scale, causal, window, kv_start=ks)
        flags = (hidden_nonfinite(vals, ok, E, L, causal, window, ks) if with_unspecified
                 else np.zeros((L, keys.shape[1]), dtype=bool))
        G = Hq // keys.shape[1]
        for i in range(n_rows):
            r = start + i
            if 0 <= r < total_q:
                out[r] = res[i]
                unspec[r] = np.repeat(flags[i], G)
    return (out, unspec) if with_unspecified else out


# --------------------------------------------------------------------------
# Column mode: seq_info = (q_start, q_len, col, kv_end) over [rows, cols, Hkv, D].
# --------------------------------------------------------------------------


def column_attention(q, k_store, v_store, seq_info, *, dtype: str, scale: float,
                     causal: bool, window: int, max_seqlen_q: int | None = None,
                     segments=None, kv_start=None, with_unspecified: bool = False):
    """Oracle for ``sdpa_varlen`` over a column (ring) store.  Key ``j`` of the
    segment's column sits in store row ``j % rows``.  ``kv_start`` int
    [num_segments] or None: each segment's left-padding bound.  Returns
    float64 [total_q, Hq, D] with uncovered rows 0; with ``with_unspecified``
    also the bool mask [total_q, Hq] of unspecified outputs."""
    q = np.asarray(q)
    total_q, Hq, D = q.shape
    ks = np.asarray(k_store)
    vs = np.asarray(v_store)
    rows, cols = ks.shape[0], ks.shape[1]
    info = np.asarray(seq_info).astype(np.int64)
    out = np.zeros((total_q, Hq, D), dtype=np.float64)
    unspec = np.zeros((total_q, Hq), dtype=bool)
    for s in (range(info.shape[0]) if segments is None else segments):
        q_start, L, col, E = (int(x) for x in info[s])
        if L <= 0:
            continue
        E = max(E, 0)
        pad = 0 if kv_start is None else int(kv_start[s])
        n_rows = L if max_seqlen_q is None else min(L, int(max_seqlen_q))
        # Only the keys some row can see are gathered (the rest may be
        # overwritten ring rows); unseen keys are zero placeholders.
        lo_all = E
        for i in range(n_rows):
            lo, hi = visible_range(E, L, i, causal, window, pad)
            if hi > lo:
                lo_all = min(lo_all, lo)
        keys = np.zeros((E, ks.shape[2], D), dtype=np.float64)
        vals = np.zeros((E, ks.shape[2], D), dtype=np.float64)
        ok = np.zeros(E, dtype=bool)
        if 0 <= col < cols and lo_all < E:
            j = np.arange(lo_all, E)
            keys[lo_all:] = to_f64(ks[j % rows, col], dtype)
            vals[lo_all:] = to_f64(vs[j % rows, col], dtype)
            ok[lo_all:] = True
        qq = np.zeros((L, Hq, D), dtype=np.float64)
        lo_r, hi_r = max(q_start, 0), min(q_start + L, total_q)
        if hi_r > lo_r:
            qq[lo_r - q_start:hi_r - q_start] = to_f64(q[lo_r:hi_r], dtype)
        res = attend_unit(qq, keys, vals, ok, E, scale, causal, window, kv_start=pad)
        flags = (hidden_nonfinite(vals, ok, E, L, causal, window, pad) if with_unspecified
                 else np.zeros((L, ks.shape[2]), dtype=bool))
        G = Hq // ks.shape[2]
        for i in range(n_rows):
            r = q_start + i
            if 0 <= r < total_q:
                out[r] = res[i]
                unspec[r] = np.repeat(flags[i], G)
    return (out, unspec) if with_unspecified else out


# --------------------------------------------------------------------------
# Prefix import / export between a dense prefill cache and paged slots.
# --------------------------------------------------------------------------


def prefix_import(k_flat: np.ndarray, v_flat: np.ndarray, k_src: np.ndarray,
                  v_src: np.ndarray, block_table: np.ndarray,
                  n: int) -> tuple[np.ndarray, np.ndarray]:
    """vLLM-Omni ``paged_decode.py``, ``PagedDecodeCache.load_prefix`` and
    ``_write_prefix``: a prefill cache holds, per sequence, one ``[S, D]`` plane
    per kv head (``[B, Hkv, S, D]``); its first ``n`` positions are written into
    the paged cache position by position, position ``j`` of sequence ``b``
    (all heads: ``src[b, :, j, :]``) going to the slot its block-table row
    names.  The pages copy into the flat view through an identity table; any
    table reads the same way.

    Arrays are integer bit views, so every bit is moved untouched.  A position
    whose slot lies outside ``[0, num_slots)`` is skipped, and every slot not
    written keeps its old contents (the pages leave the tail stale).  Returns
    copies of the flat caches ``[num_slots, Hkv, D]``.
    """
    k_out = np.array(k_flat, copy=True)
    v_out = np.array(v_flat, copy=True)
    num_slots = k_out.shape[0]
    for b in range(k_src.shape[0]):
        for j in range(n):
            s = paged_slot(block_table[b], j)
            if 0 <= s < num_slots:
                k_out[s] = k_src[b, :, j, :]
                v_out[s] = v_src[b, :, j, :]
    return k_out, v_out


def prefix_export(k_flat: np.ndarray, v_flat: np.ndarray, block_table: np.ndarray,
                  batch: int, n: int) -> tuple[np.ndarray, np.ndarray]:
    """``PagedDecodeCache.to_dynamic_cache``: the first ``n`` positions of each
    sequence read back out of the paged cache into a dense ``[B, Hkv, n, D]``
    cache (``out[b, :, j, :]`` is the slot row of position ``j``).  A position
    whose slot lies outside the cache reads as all-zero bits."""
    num_slots, H, D = k_flat.shape
    k_out = np.zeros((batch, H, n, D), dtype=k_flat.dtype)
    v_out = np.zeros((batch, H, n, D), dtype=v_flat.dtype)
    for b in range(batch):
        for j in range(n):
            s = paged_slot(block_table[b], j)
            if 0 <= s < num_slots:
                k_out[b, :, j, :] = k_flat[s]
                v_out[b, :, j, :] = v_flat[s]
    return k_out, v_out


# --------------------------------------------------------------------------
# Comparison.
# --------------------------------------------------------------------------


def compare(got: np.ndarray, ref: np.ndarray, skip=None) -> dict:
    """Element-wise comparison of an output with the oracle's.

    ``max_abs``: max |got - ref| over the elements where ``ref`` is finite;
    ``rms_rel``: RMS |got - ref| / RMS |ref| over the same elements;
    ``finite``: every ``got`` element is finite where ``ref`` is;
    ``nan_match``: ``got`` is NaN exactly where ``ref`` is NaN (a NaN that
    reaches a row through a key the row sees must show up, and only there).
    ``skip`` (bool, broadcastable to the leading axes of ``got``) leaves
    unspecified outputs out of every figure.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    keep = np.ones(got.shape, dtype=bool)
    if skip is not None:
        sk = np.asarray(skip, dtype=bool)
        sk = sk.reshape(sk.shape + (1,) * (got.ndim - sk.ndim))
        keep &= ~np.broadcast_to(sk, got.shape)
    fin = keep & np.isfinite(ref)
    d = np.abs(got - ref)[fin]
    r = ref[fin]
    rms_ref = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    rms_d = float(np.sqrt(np.mean(d * d))) if d.size else 0.0
    return {"max_abs": float(d.max()) if d.size else 0.0,
            "rms_rel": rms_d / rms_ref if rms_ref > 0 else rms_d,
            "finite": bool(np.isfinite(got[fin]).all()),
            "nan_match": bool(np.array_equal(np.isnan(got) & keep, np.isnan(ref) & keep))}
