"""Shared test helpers: host copies for the oracle, tolerances, comparisons."""
from __future__ import annotations

import numpy as np
import torch

import oracle

TOL = {"bf16": 2e-2, "f32": 1e-4}
RMS_TOL = {"bf16": 1e-2, "f32": 1e-5}


def dname(t: torch.Tensor) -> str:
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def raw(t: torch.Tensor) -> np.ndarray:
    """Exact host copy in the oracle's input form (uint16 bits for bf16)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bits(t: torch.Tensor) -> torch.Tensor:
    """Integer view for bitwise comparisons."""
    t = t.detach().contiguous()
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def check_close(got: torch.Tensor, ref: np.ndarray, dtype: str, what: str = "", skip=None) -> dict:
    """Every output element against the oracle: NaN exactly where the oracle
    has NaN, finite elsewhere, max |err| and RMS relative error within the
    dtype's bound.  ``skip`` [rows, heads] leaves unspecified outputs out."""
    err = oracle.compare(got.detach().float().cpu().numpy(), ref, skip=skip)
    assert err["finite"], f"{what}: non-finite output"
    assert err["nan_match"], f"{what}: NaN pattern differs from the oracle's"
    assert err["max_abs"] <= TOL[dtype], f"{what}: max |err| {err['max_abs']:.3e} > {TOL[dtype]}"
    assert err["rms_rel"] <= RMS_TOL[dtype], f"{what}: rms rel err {err['rms_rel']:.3e}"
    return err


def paged_slots(inp) -> torch.Tensor:
    """Append slots of a paged workload's new tokens (through the block table)."""
    s = oracle.paged_slots_for(inp.block_table.cpu().numpy(), inp.new_seq.cpu().numpy(),
                               inp.new_pos.cpu().numpy())
    return torch.from_numpy(s).to(inp.q.device)


def ring_slots(inp) -> torch.Tensor:
    s = oracle.ring_slots_for(inp.new_pos.cpu().numpy(), inp.new_col.cpu().numpy(), inp.rows,
                              inp.cols)
    return torch.from_numpy(s).to(inp.q.device)


def oracle_paged(inp, q=None, k=None, v=None, seqs=None, **kw) -> np.ndarray:
    q = inp.q if q is None else q
    k = inp.k_cache if k is None else k
    v = inp.v_cache if v is None else v
    args = dict(dtype=dname(q), scale=inp.scale, causal=inp.causal, window=inp.window,
                max_seqlen_q=inp.max_seqlen_q, max_seqlen_k=inp.max_seqlen_k)
    args.update(kw)
    return oracle.paged_attention(raw(q), raw(k), raw(v), inp.block_table.cpu().numpy(),
                                  inp.cu_seqlens_q.cpu().numpy(), inp.seqused_k.cpu().numpy(),
                                  seqs=seqs, **args)


def oracle_column(inp, q=None, k=None, v=None, segments=None, **kw) -> np.ndarray:
    q = inp.q if q is None else q
    k = inp.k_store if k is None else k
    v = inp.v_store if v is None else v
    args = dict(dtype=dname(q), scale=inp.scale, causal=inp.causal, window=inp.window,
                max_seqlen_q=inp.max_seqlen_q)
    args.update(kw)
    return oracle.column_attention(raw(q), raw(k), raw(v), inp.seq_info.cpu().numpy(),
                                   segments=segments, **args)
