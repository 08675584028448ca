"""MI355X (gfx950) DeepSeek-V4 hybrid attention core: CSA + HCA + sliding window.

Thin Python binding over libdsv4attn.so.  Each function marshals torch device tensors into
the pointers and sizes of the C entry point of the same name (include/dsv4attn.h) and
raises on a non-zero status; every step of the computation runs in the HIP kernels.
PyTorch supplies device memory and the current stream only.
"""
from __future__ import annotations

import ctypes
from typing import Optional

from . import _lib

__all__ = ["csa_compress", "compressor_cache_update", "compressor_cache_update_pair", "csa_index_topk",
           "csa_index_topk_workspace_size", "csa_index_topk_noalloc", "NOALLOC_SCRATCH_BYTES", "swa_concat", "csa_attend", "hca_attend", "hca_attend_pairs",
           "attend_workspace_size", "grouped_out_proj", "linear_bt", "linear_bt_multi", "input_projections", "attention_mask_dump",
           "abi_version", "DSV4Error", "lib"]

DSV4_FP32, DSV4_BF16 = 0, 1


class DSV4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib = _lib.load()
        self.status = status
        super().__init__(f"{fn}: {lib.dsv4_status_string(status).decode()} "
                         f"({lib.dsv4_last_error().decode()})")


def lib():
    return _lib.load()


def abi_version() -> int:
    return lib().dsv4_abi_version()


def _dtype(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return DSV4_BF16
    if t.dtype == torch.float32:
        return DSV4_FP32
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream) if isinstance(stream, int) else stream.cuda_stream
    import torch

    return torch.cuda.current_stream().cuda_stream


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise DSV4Error(fn, status)


def csa_compress(x, gate, bias, pool, m: int, overlap: bool, entry_begin: int = 0,
                 entry_end: Optional[int] = None, rope_dim: int = 0, rope_theta: float = 10000.0,
                 rope_pos_offset: int = 0, stream=None, x_prev=None, gate_prev=None) -> None:
    """x, gate [B,S,C]; bias [2m or m, C] fp32 or None; pool [B,N_cap,C] (rows written).
    x_prev, gate_prev [B,S,C]: the second projection of the earlier window halves (overlap
    only; calls csa_compress_split)."""
    B, S, C = x.shape
    N_cap = pool.shape[1]
    if bias is not None and tuple(bias.shape) != ((2 * m if overlap else m), C):
        raise ValueError(f"bias must be [{2 * m if overlap else m}, {C}], got {tuple(bias.shape)}")
    if entry_end is None:
        entry_end = min(S // m, N_cap)
    if x_prev is not None or gate_prev is not None:
        if not overlap:
            raise ValueError("a second projection needs overlapping windows")
        _check("csa_compress_split", lib().csa_compress_split(
            _ptr(x), _ptr(gate), _ptr(x_prev), _ptr(gate_prev), _ptr(bias), _ptr(pool), B, S, C, m,
            entry_begin, entry_end, N_cap, rope_dim, float(rope_theta), int(rope_pos_offset),
            _dtype(x), _stream(stream)))
        return
    _check("csa_compress", lib().csa_compress(
        _ptr(x), _ptr(gate), _ptr(bias), _ptr(pool), B, S, C, m, int(bool(overlap)), entry_begin,
        entry_end, N_cap, rope_dim, float(rope_theta), int(rope_pos_offset), _dtype(x),
        _stream(stream)))


def compressor_cache_update(x_new, gate_new, x_ring, gate_ring, bias, pool, lengths, m: int,
                            overlap: bool, rope_dim: int = 0, rope_theta: float = 10000.0,
                            rope_pos_offset: int = 0, emit: bool = True, stream=None,
                            x_prev_new=None, gate_prev_new=None, x_prev_ring=None,
                            gate_prev_ring=None) -> None:
    """x_new, gate_new [B,C]; x_ring, gate_ring [B,span,C]; bias [span,C] fp32 or None;
    pool [B,N_cap,C] (or None when emit is False); lengths [B] int32 (tokens incl. the new).
    The *_prev arguments (all four) select the second-projection compressor (overlap only)."""
    B, C = x_new.shape
    N_cap = 0 if pool is None else pool.shape[1]
    if x_prev_new is not None:
        if not overlap:
            raise ValueError("a second projection needs overlapping windows")
        _check("compressor_cache_update_split", lib().compressor_cache_update_split(
            _ptr(x_new), _ptr(gate_new), _ptr(x_prev_new), _ptr(gate_prev_new), _ptr(x_ring),
            _ptr(gate_ring), _ptr(x_prev_ring), _ptr(gate_prev_ring), _ptr(bias), _ptr(pool),
            _ptr(lengths), B, C, m, N_cap, rope_dim, float(rope_theta), int(rope_pos_offset),
            int(bool(emit)), _dtype(x_new), _stream(stream)))
        return
    _check("compressor_cache_update", lib().compressor_cache_update(
        _ptr(x_new), _ptr(gate_new), _ptr(x_ring), _ptr(gate_ring), _ptr(bias), _ptr(pool),
        _ptr(lengths), B, C, m, int(bool(overlap)), N_cap, rope_dim, float(rope_theta),
        int(rope_pos_offset), int(bool(emit)), _dtype(x_new), _stream(stream)))


def csa_index_topk_workspace_size(B: int, T: int, N_cap: int, k: int) -> int:
    return int(lib().csa_index_topk_workspace_size(B, T, N_cap, k))


def csa_index_topk(q_idx, w_idx, k_pool, q_pos0, n_pool, topk_idx, topk_score, m: int,
                   workspace, stream=None) -> None:
    """q_idx [B,T,nI,cI]; w_idx [B,T,nI] fp32; k_pool [B,N_cap,cI]; q_pos0/n_pool [B] int32;
    topk_idx [B,T,k] int32 out; topk_score [B,T,k] fp32 out or None; workspace uint8 tensor."""
    B, T, nI, cI = q_idx.shape
    N_cap = k_pool.shape[1]
    k = topk_idx.shape[2]
    nbytes = workspace.numel() * workspace.element_size()
    _check("csa_index_topk", lib().csa_index_topk(
        _ptr(q_idx), _ptr(w_idx), _ptr(k_pool), _ptr(q_pos0), _ptr(n_pool), _ptr(topk_idx),
        _ptr(topk_score), B, T, nI, cI, N_cap, m, k, _ptr(workspace), nbytes, _dtype(q_idx),
        _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 << 20


def csa_index_topk_noalloc(q_idx, w_idx, k_pool, q_pos0, n_pool, topk_idx, topk_score, m: int,
                           stream=None) -> None:
    """csa_index_topk with the library's static score scratch (no workspace argument); raises
    DSV4Error (status 2) when B*T*N_cap*4 bytes exceed NOALLOC_SCRATCH_BYTES."""
    B, T, nI, cI = q_idx.shape
    N_cap = k_pool.shape[1]
    k = topk_idx.shape[2]
    _check("csa_index_topk_noalloc", lib().csa_index_topk_noalloc(
        _ptr(q_idx), _ptr(w_idx), _ptr(k_pool), _ptr(q_pos0), _ptr(n_pool), _ptr(topk_idx),
        _ptr(topk_score), B, T, nI, cI, N_cap, m, k, _dtype(q_idx), _stream(stream)))


def swa_concat(kv_raw, kv_win, kv_pos0, new_pos0, rope_dim: int, rope_theta: float,
               rope_pos_offset: int = 0, stream=None) -> None:
    """kv_raw [B,S_new,D] -> rotated rows of kv_win [B,S_cap,D]; kv_pos0/new_pos0 [B] int32."""
    B, S_new, D = kv_raw.shape
    S_cap = kv_win.shape[1]
    _check("swa_concat", lib().swa_concat(
        _ptr(kv_raw), _ptr(kv_win), _ptr(kv_pos0), _ptr(new_pos0), B, S_new, S_cap, D, rope_dim,
        float(rope_theta), int(rope_pos_offset), _dtype(kv_raw), _stream(stream)))


def attend_workspace_size(B: int, T: int, H: int, D: int) -> int:
    return int(lib().attend_workspace_size(B, T, H, D))


def _ws(workspace):
    if workspace is None:
        return None, 0
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def csa_attend(q, kv_win, kv_pos0, pool, topk_idx, sink, q_pos0, out, window: int,
               rope_dim: int, rope_theta: float, rope_pos_offset: int = 0, scale: float = 0.0,
               workspace=None, stream=None) -> None:
    """q [B,T,H,D]; kv_win [B,S_kv,D]; pool [B,N_cap,D]; topk_idx [B,T,k]; sink [H] fp32;
    kv_pos0/q_pos0 [B] int32; out [B,T,H,D]; workspace: None or a uint8 device tensor of
    attend_workspace_size bytes."""
    B, T, H, D = q.shape
    wp, wb = _ws(workspace)
    _check("csa_attend", lib().csa_attend(
        _ptr(q), _ptr(kv_win), _ptr(kv_pos0), kv_win.shape[1], _ptr(pool), pool.shape[1],
        _ptr(topk_idx), topk_idx.shape[2], _ptr(sink), _ptr(q_pos0), _ptr(out), B, T, H, D,
        window, rope_dim, float(rope_theta), int(rope_pos_offset), float(scale), wp, wb,
        _dtype(q), _stream(stream)))


def hca_attend(q, kv_win, kv_pos0, pool, n_pool, m_hca: int, sink, q_pos0, out, window: int,
               rope_dim: int, rope_theta: float, rope_pos_offset: int = 0, scale: float = 0.0,
               workspace=None, stream=None) -> None:
    """As csa_attend, over every visible pool entry; pool None (and N_cap 0) = sliding only."""
    B, T, H, D = q.shape
    N_cap = 0 if pool is None else pool.shape[1]
    wp, wb = _ws(workspace)
    _check("hca_attend", lib().hca_attend(
        _ptr(q), _ptr(kv_win), _ptr(kv_pos0), kv_win.shape[1], _ptr(pool), N_cap, _ptr(n_pool),
        m_hca, _ptr(sink), _ptr(q_pos0), _ptr(out), B, T, H, D, window, rope_dim,
        float(rope_theta), int(rope_pos_offset), float(scale), wp, wb, _dtype(q),
        _stream(stream)))


def hca_attend_pairs(q, kv_win, kv_pos0, pool, n_pool, m_hca: int, sink, q_pos0, out, window: int,
                     rope_dim: int, rope_theta: float, rope_pos_offset: int = 0, scale: float = 0.0,
                     stream=None) -> None:
    """hca_attend computed by the query-pair kernel (bf16, 64 heads x 512 only)."""
    B, T, H, D = q.shape
    N_cap = 0 if pool is None else pool.shape[1]
    _check("hca_attend_pairs", lib().hca_attend_pairs(
        _ptr(q), _ptr(kv_win), _ptr(kv_pos0), kv_win.shape[1], _ptr(pool), N_cap, _ptr(n_pool),
        m_hca, _ptr(sink), _ptr(q_pos0), _ptr(out), B, T, H, D, window, rope_dim,
        float(rope_theta), int(rope_pos_offset), float(scale), _dtype(q), _stream(stream)))


def compressor_cache_update_pair(first, second, lengths, m: int, overlap: bool, rope_theta: float = 10000.0,
                                 rope_pos_offset: int = 0, emit: bool = True, stream=None) -> None:
    """Two compressor cache updates in one launch.  first / second: dicts with x_new, gate_new
    [B,C]; x_ring, gate_ring [B,span,C]; bias [span,C] fp32 or None; pool [B,N_cap,C]; rope_dim.
    Both share lengths [B] int32, m, overlap and N_cap (pool.shape[1])."""
    B, C = first["x_new"].shape
    C2 = second["x_new"].shape[1]
    N_cap = first["pool"].shape[1]
    if second["pool"].shape[1] != N_cap:
        raise ValueError("both pools must hold N_cap entries")
    _check("compressor_cache_update_pair", lib().compressor_cache_update_pair(
        _ptr(first["x_new"]), _ptr(first["gate_new"]), _ptr(first["x_ring"]), _ptr(first["gate_ring"]),
        _ptr(first.get("bias")), _ptr(first["pool"]), C, int(first.get("rope_dim", 0)),
        _ptr(second["x_new"]), _ptr(second["gate_new"]), _ptr(second["x_ring"]), _ptr(second["gate_ring"]),
        _ptr(second.get("bias")), _ptr(second["pool"]), C2, int(second.get("rope_dim", 0)),
        _ptr(lengths), B, m, int(bool(overlap)), N_cap, float(rope_theta), int(rope_pos_offset),
        int(bool(emit)), _dtype(first["x_new"]), _stream(stream)))


def grouped_out_proj(attn, w_a, w_b, mid, out, stream=None) -> None:
    """attn [T,H,D]; w_a [groups,rank,H/groups*D]; w_b [hidden,groups*rank]; mid [T,groups*rank]
    (written); out [T,hidden]."""
    T, H, D = attn.shape
    groups, rank, kg = w_a.shape
    hidden = w_b.shape[0]
    if kg * groups != H * D or tuple(w_b.shape) != (hidden, groups * rank):
        raise ValueError(f"w_a {tuple(w_a.shape)} / w_b {tuple(w_b.shape)} do not fit attn {tuple(attn.shape)}")
    if tuple(mid.shape) != (T, groups * rank) or tuple(out.shape) != (T, hidden):
        raise ValueError("mid must be [T, groups*rank] and out [T, hidden]")
    _check("grouped_out_proj", lib().grouped_out_proj(
        _ptr(attn), _ptr(w_a), _ptr(w_b), _ptr(mid), _ptr(out), T, H, D, groups, rank, hidden,
        _dtype(attn), _stream(stream)))


def linear_bt(x, w, y, stream=None) -> None:
    """y [M,N] = x [M,K] . w [N,K]^T."""
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K or tuple(y.shape) != (M, N):
        raise ValueError(f"shapes x {tuple(x.shape)}, w {tuple(w.shape)}, y {tuple(y.shape)}")
    _check("linear_bt", lib().linear_bt(_ptr(x), _ptr(w), _ptr(y), M, N, K, _dtype(x), _stream(stream)))


def linear_bt_multi(x, w, outs, stream=None) -> None:
    """outs[s] [M, width_s] = x [M,K] . (rows of w [sum width, K] for map s)^T; bf16 inputs may
    write fp32 outputs."""
    import torch

    M, K = x.shape
    if w.shape[1] != K or w.shape[0] != sum(o.shape[1] for o in outs):
        raise ValueError(f"w {tuple(w.shape)} does not stack the outputs' widths over K={K}")
    if any(o.dim() != 2 or o.shape[0] != M for o in outs):
        raise ValueError("every output must be [M, width]")
    n = len(outs)
    ptrs = (ctypes.c_void_p * n)(*[_ptr(o) for o in outs])
    widths = (ctypes.c_int * n)(*[o.shape[1] for o in outs])
    f32 = (ctypes.c_int * n)(*[int(o.dtype == torch.float32) for o in outs])
    _check("linear_bt_multi", lib().linear_bt_multi(_ptr(x), _ptr(w), M, K, n, ptrs, widths, f32,
                                                    _dtype(x), _stream(stream)))


def input_projections(kind: str, x, w_x, w_lat, c_q, q, kv, gate=None, q_idx=None, k_idx=None,
                      g_idx=None, w_idx=None, stream=None) -> None:
    """x [T,hidden]; w_x [q_rank + D (+ D) (+ 2 cI + nI), hidden]; w_lat [H*D (+ nI*cI), q_rank];
    c_q [T,q_rank]; q [T,H,D]; kv, gate [T,D]; q_idx [T,nI,cI]; k_idx, g_idx [T,cI]; w_idx [T,nI]
    fp32.  kind "sliding" / "hca" / "csa" (outputs the type lacks stay None)."""
    T, hidden = x.shape
    q_rank = c_q.shape[1]
    _, H, D = q.shape
    k = _MASK_KINDS[kind]
    nI, cI = (q_idx.shape[1], q_idx.shape[2]) if k == 1 else (0, 0)
    n_x = q_rank + D + (D if k else 0) + (2 * cI + nI if k == 1 else 0)
    n_lat = H * D + nI * cI
    if tuple(w_x.shape) != (n_x, hidden) or tuple(w_lat.shape) != (n_lat, q_rank):
        raise ValueError(f"w_x {tuple(w_x.shape)} / w_lat {tuple(w_lat.shape)}: expected "
                         f"{(n_x, hidden)} / {(n_lat, q_rank)}")
    want = {"c_q": (c_q, (T, q_rank)), "q": (q, (T, H, D)), "kv": (kv, (T, D))}
    if k:
        want["gate"] = (gate, (T, D))
    if k == 1:
        want.update(q_idx=(q_idx, (T, nI, cI)), k_idx=(k_idx, (T, cI)), g_idx=(g_idx, (T, cI)),
                    w_idx=(w_idx, (T, nI)))
    for name, (t, shape) in want.items():
        if t is None or tuple(t.shape) != shape:
            raise ValueError(f"{name} must be a tensor of shape {shape}")
    _check("input_projections", lib().input_projections(
        k, _ptr(x), _ptr(w_x), _ptr(w_lat), _ptr(c_q), _ptr(q), _ptr(kv), _ptr(gate), _ptr(q_idx),
        _ptr(k_idx), _ptr(g_idx), _ptr(w_idx), T, hidden, q_rank, H, D, nI, cI, _dtype(x),
        _stream(stream)))


_MASK_KINDS = {"sliding": 0, "csa": 1, "hca": 2}
_MASK_FORMATS = {"text": 0, "ansi": 1, "svg": 2, "lists": 3}


def attention_mask_dump(kind: str, S: int, window: int, m: int = 1, topk_idx=None,
                        n_entries: int = 0, q_pos0: int = 0, fmt: str = "text") -> str:
    """Visibility grid / SVG / index-list dump of one layer (host only).  topk_idx: [S, k]
    int32 lists (numpy array or tensor; copied to host memory) for kind "csa"."""
    import numpy as np

    ptr, k, keep = None, 0, None
    if topk_idx is not None:
        if hasattr(topk_idx, "detach"):
            topk_idx = topk_idx.detach().cpu().numpy()
        keep = np.ascontiguousarray(np.asarray(topk_idx, dtype=np.int32).reshape(S, -1))
        ptr, k = keep.ctypes.data, keep.shape[1]
    args = (_MASK_KINDS[kind], S, window, m, ptr, k, n_entries, q_pos0, _MASK_FORMATS[fmt])
    need = ctypes.c_size_t(0)
    st = lib().attention_mask_dump(*args, None, 0, ctypes.byref(need))
    if st != 4:  # anything but "buffer too small" is a real error
        _check("attention_mask_dump", st)
    buf = ctypes.create_string_buffer(need.value)
    _check("attention_mask_dump", lib().attention_mask_dump(*args, buf, need.value, ctypes.byref(need)))
    return buf.value.decode()
