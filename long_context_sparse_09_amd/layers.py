"""One attention layer of each type, composed from the five library calls.

The hot path of a layer ("Hybrid attention (§2.3)" of the DeepSeek-V4 model page):
  CSA     : csa_compress(kv) -> csa_compress(indexer keys) -> csa_index_topk -> swa_concat
            -> csa_attend
  HCA     : csa_compress(kv, m', disjoint) -> swa_concat -> hca_attend
  sliding : swa_concat -> hca_attend (no pool)
Buffers are torch device tensors allocated once per shape (LayerBuffers) and reused; every
computation runs in libdsv4attn.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import torch

from . import (attend_workspace_size, csa_attend, csa_compress, csa_index_topk,
               csa_index_topk_workspace_size, hca_attend, swa_concat)


@dataclasses.dataclass
class LayerShape:
    B: int
    S: int
    H: int
    D: int
    r: int
    m: int
    m_hca: int
    nI: int
    cI: int
    k: int
    W: int
    base: float
    dtype: torch.dtype


class LayerBuffers:
    """Intermediates and outputs of one prefill layer (positions 0 .. S-1)."""

    def __init__(self, sh: LayerShape, device="cuda", kinds=("csa", "hca", "sliding")):
        dev = torch.device(device)
        B, S = sh.B, sh.S
        self.sh = sh
        self.zeros_b = torch.zeros(B, dtype=torch.int32, device=dev)
        self.kv_win = torch.empty(B, S, sh.D, dtype=sh.dtype, device=dev)
        self.out = torch.empty(B, S, sh.H, sh.D, dtype=sh.dtype, device=dev)
        if "csa" in kinds:
            N = S // sh.m
            self.N = max(N, 1)
            self.n_pool = torch.full((B,), N, dtype=torch.int32, device=dev)
            self.pool = torch.zeros(B, self.N, sh.D, dtype=sh.dtype, device=dev)
            self.k_pool = torch.zeros(B, self.N, sh.cI, dtype=sh.dtype, device=dev)
            self.k_eff = min(sh.k, self.N)
            self.topk_idx = torch.empty(B, S, self.k_eff, dtype=torch.int32, device=dev)
            self.topk_score = torch.empty(B, S, self.k_eff, dtype=torch.float32, device=dev)
            ws = csa_index_topk_workspace_size(B, S, self.N, self.k_eff)
            self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)
        if "hca" in kinds:
            Nh = S // sh.m_hca
            self.Nh = Nh
            self.n_pool_h = torch.full((B,), Nh, dtype=torch.int32, device=dev)
            self.pool_h = torch.zeros(B, max(Nh, 1), sh.D, dtype=sh.dtype, device=dev)


def csa_layer(inp: Dict[str, torch.Tensor], buf: LayerBuffers, rope_pos_offset: int = 0,
              with_scores: bool = False, stream=None) -> torch.Tensor:
    sh = buf.sh
    csa_compress(inp["kv"], inp["gate"], inp["bias"], buf.pool, sh.m, True, rope_dim=sh.r,
                 rope_theta=sh.base, rope_pos_offset=rope_pos_offset, stream=stream)
    csa_compress(inp["k_idx"], inp["g_idx"], inp["bias_idx"], buf.k_pool, sh.m, True, rope_dim=0,
                 stream=stream)
    csa_index_topk(inp["q_idx"], inp["w_idx"], buf.k_pool, buf.zeros_b, buf.n_pool, buf.topk_idx,
                   buf.topk_score if with_scores else None, sh.m, buf.workspace, stream=stream)
    swa_concat(inp["kv"], buf.kv_win, buf.zeros_b, buf.zeros_b, sh.r, sh.base, rope_pos_offset,
               stream=stream)
    csa_attend(inp["q"], buf.kv_win, buf.zeros_b, buf.pool, buf.topk_idx, inp["sink"], buf.zeros_b,
               buf.out, sh.W, sh.r, sh.base, rope_pos_offset, stream=stream)
    return buf.out


def hca_layer(inp: Dict[str, torch.Tensor], buf: LayerBuffers, rope_pos_offset: int = 0,
              stream=None) -> torch.Tensor:
    sh = buf.sh
    if buf.Nh > 0:
        csa_compress(inp["kv"], inp["gate"], inp["bias_hca"], buf.pool_h, sh.m_hca, False,
                     rope_dim=sh.r, rope_theta=sh.base, rope_pos_offset=rope_pos_offset,
                     stream=stream)
    swa_concat(inp["kv"], buf.kv_win, buf.zeros_b, buf.zeros_b, sh.r, sh.base, rope_pos_offset,
               stream=stream)
    hca_attend(inp["q"], buf.kv_win, buf.zeros_b, buf.pool_h if buf.Nh > 0 else None,
               buf.n_pool_h, sh.m_hca, inp["sink"], buf.zeros_b, buf.out, sh.W, sh.r, sh.base,
               rope_pos_offset, stream=stream)
    return buf.out


def sliding_layer(inp: Dict[str, torch.Tensor], buf: LayerBuffers, rope_pos_offset: int = 0,
                  stream=None) -> torch.Tensor:
    sh = buf.sh
    swa_concat(inp["kv"], buf.kv_win, buf.zeros_b, buf.zeros_b, sh.r, sh.base, rope_pos_offset,
               stream=stream)
    hca_attend(inp["q"], buf.kv_win, buf.zeros_b, None, None, sh.m_hca, inp["sink"], buf.zeros_b,
               buf.out, sh.W, sh.r, sh.base, rope_pos_offset, stream=stream)
    return buf.out


def prefill_chunk(kind: str, inp: Dict[str, torch.Tensor], buf: LayerBuffers, c0: int, c1: int,
                  p0: torch.Tensor, rope_pos_offset: int = 0, stream=None) -> None:
    """Queries [c0, c1) of one layer's prefill (B = 1), with every earlier key visible.

    The chunk pools the entries its tokens close (entries [c0//m, c1//m); an overlapping CSA
    entry also reads the m tokens before its window, which earlier chunks hold), rotates its
    own window rows into kv_win (rows of earlier chunks are already there: the window halo),
    then scores and attends its queries.  p0 is a device int32 [1] holding c0.  Entries and
    window rows past the chunk are never visible to its queries, whatever they hold."""
    sh = buf.sh
    if sh.B != 1:
        raise ValueError("chunked prefill runs one sequence (B = 1)")
    q = inp["q"][:, c0:c1]
    out = buf.out[:, c0:c1]
    z = buf.zeros_b
    if kind == "csa":
        e0, e1 = c0 // sh.m, c1 // sh.m
        if e1 > e0:
            csa_compress(inp["kv"], inp["gate"], inp["bias"], buf.pool, sh.m, True, e0, e1,
                         rope_dim=sh.r, rope_theta=sh.base, rope_pos_offset=rope_pos_offset,
                         stream=stream)
            csa_compress(inp["k_idx"], inp["g_idx"], inp["bias_idx"], buf.k_pool, sh.m, True,
                         e0, e1, rope_dim=0, stream=stream)
        csa_index_topk(inp["q_idx"][:, c0:c1], inp["w_idx"][:, c0:c1], buf.k_pool, p0,
                       buf.n_pool, buf.topk_idx[:, c0:c1], None, sh.m, buf.workspace,
                       stream=stream)
    elif kind == "hca":
        e0, e1 = c0 // sh.m_hca, c1 // sh.m_hca
        if e1 > e0:
            csa_compress(inp["kv"], inp["gate"], inp["bias_hca"], buf.pool_h, sh.m_hca, False,
                         e0, e1, rope_dim=sh.r, rope_theta=sh.base,
                         rope_pos_offset=rope_pos_offset, stream=stream)
    elif kind != "sliding":
        raise ValueError(f"layer kind {kind!r}")
    swa_concat(inp["kv"][:, c0:c1], buf.kv_win, z, p0, sh.r, sh.base, rope_pos_offset,
               stream=stream)
    if kind == "csa":
        csa_attend(q, buf.kv_win, z, buf.pool, buf.topk_idx[:, c0:c1], inp["sink"], p0, out,
                   sh.W, sh.r, sh.base, rope_pos_offset, stream=stream)
    else:
        has_pool = kind == "hca" and buf.Nh > 0
        hca_attend(q, buf.kv_win, z, buf.pool_h if has_pool else None,
                   buf.n_pool_h if has_pool else None, sh.m_hca, inp["sink"], p0, out, sh.W,
                   sh.r, sh.base, rope_pos_offset, stream=stream)


def chunk_starts(S: int, chunk: int, device) -> torch.Tensor:
    """Device int32 start positions of the query chunks of one sequence of S tokens."""
    if chunk <= 0:
        raise ValueError("chunk must be positive")
    return torch.arange(0, S, chunk, dtype=torch.int32, device=device)


def prefill_chunked(kind: str, inp: Dict[str, torch.Tensor], buf: LayerBuffers, chunk: int,
                    rope_pos_offset: int = 0, stream=None) -> torch.Tensor:
    """One layer's prefill in query chunks of `chunk` tokens; same result as the one-shot layer."""
    S = buf.sh.S
    starts = chunk_starts(S, chunk, buf.kv_win.device)
    for i, c0 in enumerate(range(0, S, chunk)):
        prefill_chunk(kind, inp, buf, c0, min(S, c0 + chunk), starts[i:i + 1], rope_pos_offset,
                      stream)
    return buf.out


def stack_prefill_chunked(kinds, inps, bufs, chunk: int, stream=None):
    """A stack of layers prefilled chunk by chunk: every layer takes chunk c before any layer
    takes chunk c+1, the order a serving engine follows when each layer feeds the next.  The
    layers here have their own inputs (no projections between them), so the order changes
    no result."""
    if not (len(kinds) == len(inps) == len(bufs)):
        raise ValueError("one input set and one buffer set per layer")
    S = bufs[0].sh.S
    starts = chunk_starts(S, chunk, bufs[0].kv_win.device)
    for i, c0 in enumerate(range(0, S, chunk)):
        for kind, inp, buf in zip(kinds, inps, bufs):
            prefill_chunk(kind, inp, buf, c0, min(S, c0 + chunk), starts[i:i + 1], stream=stream)
    return [b.out for b in bufs]


def to_device(arrays: Dict, device="cuda") -> Dict[str, torch.Tensor]:
    """Storage-encoded numpy arrays (uint16 = bf16 bits, float32, int) -> device tensors."""
    import numpy as np

    out = {}
    for k, v in arrays.items():
        v = np.ascontiguousarray(v)
        if v.dtype == np.uint16:
            t = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(v)
        out[k] = t.to(device)
    return out


class DecodeState:
    """Caches of a batch of sequences for one CSA decode step (one new token per sequence).

    window [B, W, D]: K=V rows of positions L-W .. L-1 (rotated); the row of position L-1 is
    written by the step itself from kv_new.  pool [B, N_cap, D] (rotated) and k_pool
    [B, N_cap, cI] hold L//m valid rows each.
    """

    def __init__(self, t: Dict[str, torch.Tensor], sh: LayerShape, lengths, device="cuda"):
        dev = torch.device(device)
        self.sh = sh
        self.t = t
        L = torch.as_tensor(lengths, dtype=torch.int64)
        self.B = int(L.numel())
        self.q_pos0 = (L - 1).to(torch.int32).to(dev)
        self.kv_pos0 = (L - sh.W).to(torch.int32).to(dev)
        self.n_pool = (L // sh.m).to(torch.int32).to(dev)
        N_cap = t["pool"].shape[1]
        self.k_eff = min(sh.k, N_cap)
        self.topk_idx = torch.empty(self.B, 1, self.k_eff, dtype=torch.int32, device=dev)
        ws = csa_index_topk_workspace_size(self.B, 1, N_cap, self.k_eff)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)
        aw = attend_workspace_size(self.B, 1, sh.H, sh.D)  # key-range split of few queries
        self.attend_ws = torch.empty(aw, dtype=torch.uint8, device=dev) if aw > 0 else None
        self.out = torch.empty(self.B, 1, sh.H, sh.D, dtype=sh.dtype, device=dev)


def csa_decode_step(st: DecodeState, stream=None) -> torch.Tensor:
    sh, t = st.sh, st.t
    swa_concat(t["kv_new"], t["window"], st.kv_pos0, st.q_pos0, sh.r, sh.base, stream=stream)
    csa_index_topk(t["q_idx"], t["w_idx"], t["k_pool"], st.q_pos0, st.n_pool, st.topk_idx, None,
                   sh.m, st.workspace, stream=stream)
    csa_attend(t["q"], t["window"], st.kv_pos0, t["pool"], st.topk_idx, t["sink"], st.q_pos0,
               st.out, sh.W, sh.r, sh.base, workspace=st.attend_ws, stream=stream)
    return st.out
