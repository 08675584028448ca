"""Decode-time cache of one attention layer for a batch of sequences ("Cache layers" of the
DeepSeek-V4 model page: the HCA cache is a sliding K=V window plus the HCA compressor's
buffer / pool / count; the CSA cache adds the overlap state and the parallel indexer's
buffer / pool / count / overlap at index_head_dim).

State per sequence b, all in device buffers owned here:
  * window: rotated K=V rows in a linear buffer of W + G rows; row i holds sequence index
    kv_pos0[b] + i.  Each step appends one row; after G steps the last W rows are copied to
    the front of the other buffer of a pair (kv_pos0 += G), so no step moves W rows.
  * compressor rings: the last span raw tokens (kv and gate; for CSA also the indexer's key
    content and gate), token p in slot p mod span (span = 2m with overlap, m without).
  * pools: the closed entries (K=V pool, and for CSA the indexer keys), one emitted every m
    tokens by compressor_cache_update.
  * lengths L_b (tokens so far), host-side and as the device arrays the calls read.

Every computation runs in libdsv4attn; this module only sequences the calls and keeps the
integer bookkeeping (lengths, buffer offsets).
"""
from __future__ import annotations

from typing import Dict

import numpy as np
import torch

from . import (attend_workspace_size, compressor_cache_update, compressor_cache_update_pair, csa_attend, csa_compress,
               csa_index_topk, csa_index_topk_workspace_size, hca_attend, swa_concat)
from .layers import LayerShape


def _i32(vals, device):
    return torch.as_tensor(np.asarray(vals, dtype=np.int32), device=device)


class DecodeCache:
    """kind: "csa", "hca" or "sliding"; sh: the layer's shape (sh.B sequences, sh.S unused);
    n_cap: pool capacity in entries of rate m (CSA) or m_hca (HCA); G: window refill period."""

    def __init__(self, kind: str, sh: LayerShape, params: Dict[str, torch.Tensor], n_cap: int,
                 G: int = 256, device="cuda"):
        if kind not in ("csa", "hca", "sliding"):
            raise ValueError(f"layer kind {kind!r}")
        dev = torch.device(device)
        self.kind, self.sh, self.dev, self.G = kind, sh, dev, G
        self.params = params  # bias / bias_idx / bias_hca (fp32), sink
        B, D, W = sh.B, sh.D, sh.W
        self.win = [torch.zeros(B, W + G, D, dtype=sh.dtype, device=dev) for _ in range(2)]
        self.cur = 0          # which window buffer is live
        self.s = 0            # rows appended since the last refill
        self.L = np.zeros(B, dtype=np.int64)
        self.n_cap = n_cap
        if kind == "csa":
            span = 2 * sh.m
            self.ring = {n: torch.zeros(B, span, D, dtype=sh.dtype, device=dev) for n in ("kv", "gate")}
            self.ring.update({n: torch.zeros(B, span, sh.cI, dtype=sh.dtype, device=dev)
                              for n in ("k_idx", "g_idx")})
            self.pool = torch.zeros(B, n_cap, D, dtype=sh.dtype, device=dev)
            self.k_pool = torch.zeros(B, n_cap, sh.cI, dtype=sh.dtype, device=dev)
            self.k_eff = min(sh.k, n_cap)
            self.topk_idx = torch.empty(B, 1, self.k_eff, dtype=torch.int32, device=dev)
            ws = csa_index_topk_workspace_size(B, 1, n_cap, self.k_eff)
            self.idx_ws = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)
        elif kind == "hca":
            self.ring = {n: torch.zeros(B, sh.m_hca, D, dtype=sh.dtype, device=dev)
                         for n in ("kv", "gate")}
            self.pool = torch.zeros(B, max(n_cap, 1), D, dtype=sh.dtype, device=dev)
        # per-step int32 arrays: lengths, q_pos0, kv_pos0, n_pool; and the refill's two
        self.meta = torch.zeros(4, B, dtype=torch.int32, device=dev)
        self.refill_meta = torch.zeros(2, B, dtype=torch.int32, device=dev)
        aw = attend_workspace_size(B, 1, sh.H, D)
        self.att_ws = torch.empty(aw, dtype=torch.uint8, device=dev) if aw > 0 else None
        self.out = torch.empty(B, 1, sh.H, D, dtype=sh.dtype, device=dev)
        # pinned staging buffers for the per-step integers, and their last copies' events
        self._stage = [torch.empty(4, B, dtype=torch.int32, pin_memory=True) for _ in range(4)]
        self._stage_ev = [torch.cuda.Event() for _ in range(4)]
        self._stage_i = 0

    # ------------------------------------------------------------------ positions
    def _kv_pos0(self):
        return self.L - self.sh.W - self.s

    def _h2d(self, dst: torch.Tensor, host: np.ndarray) -> None:
        """dst (device int32) <- host, ordered on the current stream and asynchronous to the
        host: through one of four pinned staging buffers, each rewritten only after the copy
        that last read it has run.  (A copy from pageable memory makes the host wait for the
        device, and the device then idles while the host issues the step's launches.)"""
        i = self._stage_i
        self._stage_i = (i + 1) % len(self._stage)
        self._stage_ev[i].synchronize()
        buf = self._stage[i][: host.shape[0]]
        buf.copy_(torch.from_numpy(host))
        dst.copy_(buf, non_blocking=True)
        self._stage_ev[i].record()

    def _upload(self):
        """Copy this step's per-sequence integers to the device (current stream)."""
        sh = self.sh
        rate = {"csa": sh.m, "hca": sh.m_hca}.get(self.kind, 1)
        host = np.stack([self.L, self.L - 1, self._kv_pos0(),
                         np.minimum(self.L // rate, self.n_cap)]).astype(np.int32)
        self._h2d(self.meta, host)
        self.lengths_d, self.q_pos0_d, self.kv_pos0_d, self.n_pool_d = self.meta.unbind(0)

    # ------------------------------------------------------------------ prefill
    def prefill(self, b: int, seq: Dict[str, torch.Tensor]) -> None:
        """Fill sequence b's state from its first L0 tokens: seq holds [1, L0, ...] raw token
        tensors (kv, gate and, for CSA, k_idx, g_idx).  Pools are compressed in one call,
        the last W rows rotated into the window, the last span tokens copied into the rings.
        Call for every sequence, then start stepping."""
        sh, p = self.sh, self.params
        L0 = seq["kv"].shape[1]
        one = lambda t: t[b:b + 1]
        if self.kind == "csa":
            e1 = min(L0 // sh.m, self.n_cap)
            if e1 > 0:
                csa_compress(seq["kv"], seq["gate"], p["bias"], one(self.pool), sh.m, True, 0, e1,
                             rope_dim=sh.r, rope_theta=sh.base)
                csa_compress(seq["k_idx"], seq["g_idx"], p["bias_idx"], one(self.k_pool), sh.m,
                             True, 0, e1, rope_dim=0)
        elif self.kind == "hca":
            e1 = min(L0 // sh.m_hca, self.n_cap)
            if e1 > 0:
                csa_compress(seq["kv"], seq["gate"], p["bias_hca"], one(self.pool), sh.m_hca, False,
                             0, e1, rope_dim=sh.r, rope_theta=sh.base)
        # window: rows for sequence indices L0 - W .. L0 - 1 at rows 0 .. W - 1 (kv_pos0 = L0 - W)
        lo = max(0, L0 - sh.W)
        if self.s != 0:
            raise RuntimeError("prefill every sequence before the first step")
        swa_concat(seq["kv"][:, lo:L0].contiguous(), one(self.win[self.cur]),
                   _i32([L0 - sh.W], self.dev), _i32([lo], self.dev), sh.r, sh.base)
        # rings: token p in slot p mod span, copied without rotation in two contiguous pieces
        if self.kind != "sliding":
            span = self.ring["kv"].shape[1]
            p0 = max(0, L0 - span)
            cut = min(L0, (p0 // span + 1) * span)  # first position that wraps to slot 0
            for name, ring in self.ring.items():
                src = seq[name]
                for a, z in ((p0, cut), (cut, L0)):
                    if z > a:
                        base = (a // span) * span  # sequence index of slot 0 for this piece
                        swa_concat(src[:, a:z].contiguous(), one(ring), _i32([base], self.dev),
                                   _i32([a], self.dev), 0, 10000.0)
        self.L[b] = L0

    # ------------------------------------------------------------------ one decode step
    def step(self, tok: Dict[str, torch.Tensor]) -> torch.Tensor:
        """Append one token per sequence and attend its query, on the current stream.
        tok: q [B,1,H,D], kv, gate [B,1,D]; for CSA also k_idx, g_idx [B,1,cI],
        q_idx [B,1,nI,cI], w_idx [B,1,nI] (fp32).  Returns out [B,1,H,D] (reused)."""
        sh, p = self.sh, self.params
        if self.s == self.G:  # refill: the live W rows move to the front of the other buffer
            old = self._kv_pos0()
            self._h2d(self.refill_meta, np.stack([old + self.s, old]).astype(np.int32))
            swa_concat(self.win[self.cur], self.win[1 - self.cur], self.refill_meta[0],
                       self.refill_meta[1], 0, 10000.0)
            self.cur = 1 - self.cur
            self.s = 0
        self.L += 1
        self.s += 1
        self._upload()
        win = self.win[self.cur]
        flat = lambda t: t.reshape(t.shape[0], t.shape[-1])
        if self.kind == "csa":
            # the K=V compressor and the indexer's, one launch
            compressor_cache_update_pair(
                {"x_new": flat(tok["kv"]), "gate_new": flat(tok["gate"]), "x_ring": self.ring["kv"],
                 "gate_ring": self.ring["gate"], "bias": p["bias"], "pool": self.pool, "rope_dim": sh.r},
                {"x_new": flat(tok["k_idx"]), "gate_new": flat(tok["g_idx"]), "x_ring": self.ring["k_idx"],
                 "gate_ring": self.ring["g_idx"], "bias": p["bias_idx"], "pool": self.k_pool, "rope_dim": 0},
                self.lengths_d, sh.m, True, sh.base)
        elif self.kind == "hca":
            compressor_cache_update(flat(tok["kv"]), flat(tok["gate"]), self.ring["kv"],
                                    self.ring["gate"], p["bias_hca"], self.pool, self.lengths_d,
                                    sh.m_hca, False, sh.r, sh.base)
        swa_concat(tok["kv"], win, self.kv_pos0_d, self.q_pos0_d, sh.r, sh.base)
        if self.kind == "csa":
            csa_index_topk(tok["q_idx"], tok["w_idx"], self.k_pool, self.q_pos0_d, self.n_pool_d,
                           self.topk_idx, None, sh.m, self.idx_ws)
            csa_attend(tok["q"], win, self.kv_pos0_d, self.pool, self.topk_idx, p["sink"],
                       self.q_pos0_d, self.out, sh.W, sh.r, sh.base, workspace=self.att_ws)
        else:
            has_pool = self.kind == "hca"
            hca_attend(tok["q"], win, self.kv_pos0_d, self.pool if has_pool else None,
                       self.n_pool_d if has_pool else None, sh.m_hca, p["sink"], self.q_pos0_d,
                       self.out, sh.W, sh.r, sh.base, workspace=self.att_ws)
        return self.out
