"""Thin Python binding of the C-ABI attention library ``libfa.so``.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind ``fa_forward`` / ``fa_backward``. PyTorch supplies device memory
(outputs and workspace are allocated with torch on the inputs' device) and the
current stream. There is no fallback: if the library is missing or a call
fails, an exception is raised.
"""

import ctypes
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa.so")

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
MASK_BLOCK = 128
_DTYPES = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}

_lib = None


class FAError(RuntimeError):
    """A nonzero status returned by the library."""

    def __init__(self, status, where):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


def load():
    """Load libfa.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m exact_attention_110_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_forward.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, P, I, P]
    lib.fa_forward.restype = I
    lib.fa_backward_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.fa_backward_workspace_size.restype = S
    bw = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, I, P, I, P, S, P]
    lib.fa_backward.argtypes = bw
    lib.fa_backward.restype = I
    lib.fa_backward_noalloc.argtypes = bw[:18] + [P]
    lib.fa_backward_noalloc.restype = I
    lib.fa_backward_stage.argtypes = [I] + bw
    lib.fa_backward_stage.restype = I
    U64 = ctypes.c_ulonglong
    lib.fa_forward_dropout.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, P, I, F, U64, P]
    lib.fa_forward_dropout.restype = I
    bwd_drop = bw[:18] + [F, U64] + bw[18:]
    lib.fa_backward_dropout.argtypes = bwd_drop
    lib.fa_backward_dropout.restype = I
    lib.fa_backward_stage_dropout.argtypes = [I] + bwd_drop
    lib.fa_backward_stage_dropout.restype = I
    lib.fa_forward_qk.argtypes = [P, P, P, P, P, I, I, I, I, I, I, F, I, I, I, P, P, I, F, U64, P]
    lib.fa_forward_qk.restype = I
    lib.fa_backward_qk.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, I, I, P, P, I, F, U64, P,
                                   S, P]
    lib.fa_backward_qk.restype = I
    lib.fa_forward_varlen.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, I, I, P, I, F, U64, P]
    lib.fa_forward_varlen.restype = I
    lib.fa_backward_varlen.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, I, I, P, I,
                                       F, U64, P, S, P]
    lib.fa_backward_varlen.restype = I
    lib.fa_forward_select.argtypes = [I, P, P, P, P, P, I, I, I, I, I, I, F, I, I, I, P, P, I, F, U64, P]
    lib.fa_forward_select.restype = I
    lib.fa_forward_kernel_rows.argtypes = [I] * 12
    lib.fa_forward_kernel_rows.restype = I
    lib.fa_forward_bitmask.argtypes = [P, P, P, P, P, I, I, I, I, I, I, F, I, P, P, P, I, I, F, U64, P]
    lib.fa_forward_bitmask.restype = I
    lib.fa_backward_bitmask.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, P, P, P, I, I, F, U64,
                                        P, S, P]
    lib.fa_backward_bitmask.restype = I
    lib.fa_backward_launches.argtypes = [I, I, I, I, I, I, F, I, I, I]
    lib.fa_backward_launches.restype = I
    lib.fa_forward_fp8.argtypes = [P, P, P, P, P, I, I, I, I, I, F, F, F, F, I, I, P]
    lib.fa_forward_fp8.restype = I
    lib.fa_status_string.argtypes = [I]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = I
    _lib = lib
    return lib


def status_string(status):
    return load().fa_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_tensors(tensors, dtype):
    for name, t in tensors:
        if not t.is_cuda or not t.is_contiguous() or t.dtype != dtype:
            raise ValueError(f"{name} must be a contiguous device tensor of dtype {dtype}")
    if dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {dtype}")


def _shape4(q, k, v):
    """B, H, Hkv, Nq, Nk, d of q [B, H, Nq, d] and k, v [B, Hkv, Nk, d]."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, Nq, d] / [B, Hkv, Nk, d]")
    B, H, Nq, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    _check_tensors((("q", q), ("k", k), ("v", v)), q.dtype)
    return B, H, k.shape[1], Nq, k.shape[2], d


def _shape(q, k, v):
    B, H, Hkv, Nq, Nk, d = _shape4(q, k, v)
    if Nq != Nk:
        raise ValueError("q and k have different lengths")
    return B, H, Hkv, Nq, d


def _mask(block_mask, Nq, device, Nk=None):
    if block_mask is None:
        return None
    nbq = -(-Nq // MASK_BLOCK)
    nbk = nbq if Nk is None else -(-Nk // MASK_BLOCK)
    if not isinstance(block_mask, torch.Tensor):
        block_mask = torch.as_tensor(block_mask)
    if tuple(block_mask.shape) != (nbq, nbk) or block_mask.dtype != torch.uint8:
        raise ValueError(f"block_mask must be uint8 [{nbq}, {nbk}]")
    return block_mask.to(device).contiguous()


def _seed(seed):
    return int(seed) & (2**64 - 1)


def _slopes(alibi_slopes, H, device):
    """None, or the ALiBi slopes as a contiguous float32 [H] device tensor."""
    if alibi_slopes is None:
        return None
    t = torch.as_tensor(alibi_slopes, dtype=torch.float32).to(device).contiguous()
    if t.dim() != 1 or t.numel() != H:
        raise ValueError(f"alibi_slopes must hold one slope per query head ({H})")
    return t


def forward_kernel_rows(B, H, Hkv, Nq, Nk, d, causal=False, window=(-1, -1), alibi=False, block_mask=False,
                        dtype=torch.bfloat16):
    """Rows per wave of the forward kernel the library takes for these
    arguments (64 or 32; 0 for float32 inputs): fa_forward_kernel_rows."""
    r = load().fa_forward_kernel_rows(B, H, Hkv, Nq, Nk, d, int(bool(causal)), int(window[0]), int(window[1]),
                                      int(bool(alibi)), int(bool(block_mask)), _DTYPES[dtype])
    if r < 0:
        raise FAError(r, "fa_forward_kernel_rows")
    return r


def backward_stages(B, H, Hkv, Nq, Nk, d, dropout_rate=0.0, alibi=False, block_mask=False, dtype=torch.bfloat16):
    """The stages fa_backward runs for these arguments, in order: [0, 1, 2],
    or [0, 3] where dK/dV and dQ go out as one launch (fa_backward_launches)."""
    n = load().fa_backward_launches(B, H, Hkv, Nq, Nk, d, float(dropout_rate), int(bool(alibi)),
                                    int(bool(block_mask)), _DTYPES[dtype])
    if n < 0:
        raise FAError(n, "fa_backward_launches")
    return [0, 3] if n == 2 else [0, 1, 2]


def forward(q, k, v, scale=None, causal=False, block_mask=None, out=None, lse=None, dropout_rate=0.0,
            seed=0, window=(-1, -1), alibi_slopes=None, rows_per_wave=0):
    """O, LSE = attention(q, k, v); q [B,H,Nq,d], k, v [B,Hkv,Nk,d] on the GPU.

    Nq == Nk without a window or ALiBi slopes calls fa_forward
    (fa_forward_dropout with a positive dropout_rate); otherwise fa_forward_qk
    (causal masking aligned to the last query; window = (left, right), -1
    unbounded; alibi_slopes: one slope per query head). rows_per_wave 32 or
    64 forces that 16-bit forward kernel (fa_forward_select)."""
    B, H, Hkv, N, Nk, d = _shape4(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    m = _mask(block_mask, N, q.device, Nk)
    wl, wr = (int(x) for x in window)
    al = _slopes(alibi_slopes, H, q.device)
    if rows_per_wave:
        st = load().fa_forward_select(int(rows_per_wave), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H,
                                      Hkv, N, Nk, d, scale, int(bool(causal)), wl, wr, _ptr(al), _ptr(m),
                                      _DTYPES[q.dtype], float(dropout_rate), _seed(seed), _stream(q.device))
        if st != 0:
            raise FAError(st, "fa_forward_select")
        return o, lse_t
    if Nk != N or (wl, wr) != (-1, -1) or al is not None:
        st = load().fa_forward_qk(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, Hkv, N, Nk, d, scale,
                                  int(bool(causal)), wl, wr, _ptr(al), _ptr(m), _DTYPES[q.dtype],
                                  float(dropout_rate), _seed(seed), _stream(q.device))
        if st != 0:
            raise FAError(st, "fa_forward_qk")
        return o, lse_t
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, Hkv, N, d, scale, int(bool(causal)), _ptr(m),
            _DTYPES[q.dtype]]
    if dropout_rate:
        st = load().fa_forward_dropout(*args, float(dropout_rate), _seed(seed), _stream(q.device))
        where = "fa_forward_dropout"
    else:
        st = load().fa_forward(*args, _stream(q.device))
        where = "fa_forward"
    if st != 0:
        raise FAError(st, where)
    return o, lse_t


def workspace_size(B, H, Hkv, N, d, dtype):
    return int(load().fa_backward_workspace_size(B, H, Hkv, N, d, _DTYPES[dtype]))


def workspace(q, k):
    B, H, N, d = q.shape
    n = workspace_size(B, H, k.shape[1], N, d, q.dtype)
    if n == 0:
        raise ValueError("no backward for these arguments")
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def _bwd_args(q, k, v, o, lse, do, dq, dk, dv, scale, causal, m, ws, drop=None):
    B, H, Hkv, N, d = _shape(q, k, v)
    head = [_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv),
            B, H, Hkv, N, d, scale, int(bool(causal)), _ptr(m), _DTYPES[q.dtype]]
    mid = [] if drop is None else [float(drop[0]), _seed(drop[1])]
    return head + mid + [_ptr(ws), ws.numel(), _stream(q.device)]


def backward(q, k, v, o, lse, do, scale=None, causal=False, block_mask=None, ws=None, grads=None,
             dropout_rate=0.0, seed=0, window=(-1, -1), alibi_slopes=None):
    """dq, dk, dv of sum(O * do), recomputing P from q, k and lse (and, with a
    positive dropout_rate, the forward call's keep decisions from seed).
    Nq != Nk, a window or ALiBi slopes call fa_backward_qk."""
    B, H, Hkv, N, Nk, d = _shape4(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    for name, t in (("o", o), ("do", do)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError(f"{name} must match q")
    m = _mask(block_mask, N, q.device, Nk)
    ws = workspace(q, k) if ws is None else ws
    dq, dk, dv = grads if grads is not None else (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    wl, wr = (int(x) for x in window)
    al = _slopes(alibi_slopes, H, q.device)
    if Nk != N or (wl, wr) != (-1, -1) or al is not None:
        st = load().fa_backward_qk(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk),
                                   _ptr(dv), B, H, Hkv, N, Nk, d, scale, int(bool(causal)), wl, wr, _ptr(al),
                                   _ptr(m), _DTYPES[q.dtype], float(dropout_rate), _seed(seed), _ptr(ws),
                                   ws.numel(), _stream(q.device))
        if st != 0:
            raise FAError(st, "fa_backward_qk")
        return dq, dk, dv
    if dropout_rate:
        st = load().fa_backward_dropout(*_bwd_args(q, k, v, o, lse, do, dq, dk, dv, scale, causal, m, ws,
                                                   (dropout_rate, seed)))
        where = "fa_backward_dropout"
    else:
        st = load().fa_backward(*_bwd_args(q, k, v, o, lse, do, dq, dk, dv, scale, causal, m, ws))
        where = "fa_backward"
    if st != 0:
        raise FAError(st, where)
    return dq, dk, dv


def backward_noalloc(q, k, v, o, lse, do, scale=None, causal=False, block_mask=None, grads=None):
    """dq, dk, dv as ``backward``, through fa_backward_noalloc: no workspace,
    the library's per-GPU scratch array instead (calls overlapping on one GPU
    race)."""
    B, H, Hkv, N, d = _shape(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    for name, t in (("o", o), ("do", do)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError(f"{name} must match q")
    m = _mask(block_mask, N, q.device)
    dq, dk, dv = grads if grads is not None else (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    st = load().fa_backward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk),
                                    _ptr(dv), B, H, Hkv, N, d, scale, int(bool(causal)), _ptr(m), _DTYPES[q.dtype],
                                    _stream(q.device))
    if st != 0:
        raise FAError(st, "fa_backward_noalloc")
    return dq, dk, dv


def bit_block_mask(allow):
    """Block form of a boolean visibility matrix allow [Nq, Nk] (True = key j
    visible to query i), for fa_forward_bitmask / fa_backward_bitmask:
    (block_mask uint8 [nbq, nbk], block_tile int32 [nbq, nbk], tile_bits int32
    [n_tiles, 128, 4]) on allow's device. A block with no visible element is
    0 in block_mask; a block whose every element is visible has tile -1; the
    others get consecutive tiles whose bit j % 32 of word (j % 128) / 32 of
    row i % 128 is allow[i, j]. Rows and keys past Nq, Nk count as visible, so
    that a ragged last block whose real elements are all visible stays full."""
    allow = torch.as_tensor(allow, dtype=torch.bool)
    nq, nk = allow.shape
    nbq, nbk = -(-nq // MASK_BLOCK), -(-nk // MASK_BLOCK)
    pad = torch.ones((nbq * MASK_BLOCK, nbk * MASK_BLOCK), dtype=torch.bool, device=allow.device)
    pad[:nq, :nk] = allow
    blocks = pad.view(nbq, MASK_BLOCK, nbk, MASK_BLOCK).permute(0, 2, 1, 3)  # [nbq, nbk, 128, 128]
    real = torch.zeros_like(pad)
    real[:nq, :nk] = True
    any_real = (pad & real).view(nbq, MASK_BLOCK, nbk, MASK_BLOCK).permute(0, 2, 1, 3).flatten(2).any(dim=2)
    full = blocks.flatten(2).all(dim=2)
    block_mask = any_real.to(torch.uint8).contiguous()
    partial = any_real & ~full
    block_tile = torch.full((nbq, nbk), -1, dtype=torch.int32, device=allow.device)
    n_tiles = int(partial.sum())
    block_tile[partial] = torch.arange(n_tiles, dtype=torch.int32, device=allow.device)
    tiles = blocks[partial].reshape(n_tiles, MASK_BLOCK, 4, 32).to(torch.int64)
    weights = torch.tensor([1 << b for b in range(32)], dtype=torch.int64, device=allow.device)
    words = (tiles * weights).sum(dim=3)                                   # [n_tiles, 128, 4], < 2^32
    words = torch.where(words >= 1 << 31, words - (1 << 32), words).to(torch.int32)
    return block_mask, block_tile.contiguous(), words.contiguous()


def forward_bitmask(q, k, v, block_mask, block_tile, tile_bits, scale=None, causal=False, out=None, lse=None,
                    dropout_rate=0.0, seed=0):
    """O, LSE under a block mask with element masks of partial blocks
    (fa_forward_bitmask); the mask arrays as returned by ``bit_block_mask``."""
    B, H, Hkv, N, Nk, d = _shape4(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    m = _mask(block_mask, N, q.device, Nk)
    bt = block_tile.to(q.device, torch.int32).contiguous()
    tb = tile_bits.to(q.device, torch.int32).contiguous()
    st = load().fa_forward_bitmask(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, Hkv, N, Nk, d, scale,
                                   int(bool(causal)), _ptr(m), _ptr(bt), _ptr(tb) if tb.numel() else None,
                                   tb.shape[0], _DTYPES[q.dtype], float(dropout_rate), _seed(seed),
                                   _stream(q.device))
    if st != 0:
        raise FAError(st, "fa_forward_bitmask")
    return o, lse_t


def backward_bitmask(q, k, v, o, lse, do, block_mask, block_tile, tile_bits, scale=None, causal=False, ws=None,
                     grads=None, dropout_rate=0.0, seed=0):
    """dq, dk, dv under the mask of ``forward_bitmask`` (fa_backward_bitmask)."""
    B, H, Hkv, N, Nk, d = _shape4(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    for name, t in (("o", o), ("do", do)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError(f"{name} must match q")
    m = _mask(block_mask, N, q.device, Nk)
    bt = block_tile.to(q.device, torch.int32).contiguous()
    tb = tile_bits.to(q.device, torch.int32).contiguous()
    ws = workspace(q, k) if ws is None else ws
    dq, dk, dv = grads if grads is not None else (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    st = load().fa_backward_bitmask(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk),
                                    _ptr(dv), B, H, Hkv, N, Nk, d, scale, int(bool(causal)), _ptr(m), _ptr(bt),
                                    _ptr(tb) if tb.numel() else None, tb.shape[0], _DTYPES[q.dtype],
                                    float(dropout_rate), _seed(seed), _ptr(ws), ws.numel(), _stream(q.device))
    if st != 0:
        raise FAError(st, "fa_backward_bitmask")
    return dq, dk, dv


def backward_stage(stage, q, k, v, o, lse, do, dq, dk, dv, ws, scale=None, causal=False, block_mask=None,
                   dropout_rate=0.0, seed=0):
    """Run one stage of the backward pass (0, 1, 2, or 3 = stages 1 and 2 in one
    launch where fa_backward uses it); see fa_backward_stage."""
    d = q.shape[3]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    m = _mask(block_mask, q.shape[2], q.device)
    if dropout_rate:
        st = load().fa_backward_stage_dropout(int(stage), *_bwd_args(q, k, v, o, lse, do, dq, dk, dv, scale,
                                                                     causal, m, ws, (dropout_rate, seed)))
    else:
        st = load().fa_backward_stage(int(stage), *_bwd_args(q, k, v, o, lse, do, dq, dk, dv, scale, causal,
                                                             m, ws))
    if st != 0:
        raise FAError(st, f"fa_backward_stage({stage})")


def _varlen_shape(q, k, v, cu_seqlens_q, cu_seqlens_k):
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("packed q, k, v must be [H, total_q, d] / [Hkv, total_k, d]")
    H, tq, d = q.shape
    if k.shape != v.shape or k.shape[2] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    _check_tensors((("q", q), ("k", k), ("v", v)), q.dtype)
    for name, c in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if c.dtype != torch.int32 or c.dim() != 1 or not c.is_cuda or not c.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 device vector")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B + 1 offsets")
    return cu_seqlens_q.numel() - 1, H, k.shape[0], tq, k.shape[1], d


def forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale=None, causal=False,
                   out=None, lse=None, dropout_rate=0.0, seed=0, window=(-1, -1), alibi_slopes=None):
    """O [H, total_q, d], LSE [H, total_q] of packed sequences (fa_forward_varlen)."""
    B, H, Hkv, tq, tk, d = _varlen_shape(q, k, v, cu_seqlens_q, cu_seqlens_k)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((H, tq), dtype=torch.float32, device=q.device) if lse is None else lse
    al = _slopes(alibi_slopes, H, q.device)
    st = load().fa_forward_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), _ptr(cu_seqlens_q),
                                  _ptr(cu_seqlens_k), B, H, Hkv, tq, tk, int(max_seqlen_q), int(max_seqlen_k), d,
                                  scale, int(bool(causal)), int(window[0]), int(window[1]), _ptr(al),
                                  _DTYPES[q.dtype], float(dropout_rate), _seed(seed), _stream(q.device))
    if st != 0:
        raise FAError(st, "fa_forward_varlen")
    return o, lse_t


def backward_varlen(q, k, v, o, lse, do, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, scale=None,
                    causal=False, ws=None, grads=None, dropout_rate=0.0, seed=0, window=(-1, -1),
                    alibi_slopes=None):
    """dq, dk, dv of packed sequences (fa_backward_varlen)."""
    B, H, Hkv, tq, tk, d = _varlen_shape(q, k, v, cu_seqlens_q, cu_seqlens_k)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    for name, t in (("o", o), ("do", do)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError(f"{name} must match q")
    if ws is None:
        n = workspace_size(B, H, Hkv, int(max_seqlen_q), d, q.dtype)
        if n == 0:
            raise ValueError("no backward for these arguments")
        ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    dq, dk, dv = grads if grads is not None else (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    al = _slopes(alibi_slopes, H, q.device)
    st = load().fa_backward_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk),
                                   _ptr(dv), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, H, Hkv, tq, tk,
                                   int(max_seqlen_q), int(max_seqlen_k), d, scale, int(bool(causal)),
                                   int(window[0]), int(window[1]), _ptr(al), _DTYPES[q.dtype],
                                   float(dropout_rate), _seed(seed), _ptr(ws), ws.numel(), _stream(q.device))
    if st != 0:
        raise FAError(st, "fa_backward_varlen")
    return dq, dk, dv


def forward_fp8(q, k, v, q_descale, k_descale, v_descale, scale=None, causal=False, out_dtype=torch.bfloat16,
                out=None, lse=None):
    """O, LSE of attention over FP8 (E4M3) inputs (fa_forward_fp8).

    q [B,H,N,d], k, v [B,Hkv,N,d]: uint8 codes (or float8_e4m3fn tensors);
    the real inputs are codes times their descales. O has out_dtype."""
    q, k, v = (t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t for t in (q, k, v))
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[2:] != q.shape[2:]:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.uint8:
            raise ValueError(f"{name} must be a contiguous device tensor of E4M3 codes")
    if out_dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("out_dtype must be bfloat16 or float16")
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty(q.shape, dtype=out_dtype, device=q.device) if out is None else out
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    st = load().fa_forward_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, k.shape[1], N, d, scale,
                               float(q_descale), float(k_descale), float(v_descale), int(bool(causal)),
                               _DTYPES[out_dtype], _stream(q.device))
    if st != 0:
        raise FAError(st, "fa_forward_fp8")
    return o, lse_t
