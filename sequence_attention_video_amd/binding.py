"""ctypes binding of libspattn.so: same entry-point names as ``include/sp.h``.

Argument marshalling only: tensors become device pointers plus sizes and
strides, the stream is torch's current stream, and a status other than SP_OK
becomes an exception (``ValueError`` for SP_ERR_NOT_DIVISIBLE and
SP_ERR_INVALID_ARG, ``NotImplementedError`` for SP_ERR_UNSUPPORTED and
``RuntimeError`` for SP_ERR_HIP).  Every step of the path runs in the
library's HIP kernels; there is no fallback of any kind, and a missing library
raises at load time.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libspattn.so")

SP_OK, SP_ERR_NOT_DIVISIBLE, SP_ERR_INVALID_ARG, SP_ERR_UNSUPPORTED, SP_ERR_HIP, SP_ERR_SCRATCH = range(6)
SP_NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024
SP_F32, SP_BF16 = 0, 1
SP_TOKENS_TO_HEADS, SP_HEADS_TO_TOKENS = 0, 1
SP_GRID_TO_TILES, SP_TILES_TO_GRID = 0, 1

# names declared in include/sp.h (checked against the header by the tests)
EXPORTS = (
    "sp_status_string", "sp_version", "sp_partition", "sp_pad", "sp_relayout_heads",
    "sp_masked_attention_workspace_size", "sp_masked_attention", "sp_gather_unpad", "sp_optimal_split",
    "sp_tile_2d", "sp_tile_2d_relayout_heads", "sp_pad_relayout_heads", "sp_gather_heads_unpad",
    "sp_masked_attention_noalloc",
)


class ShardStrides(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int64), ("batch", ctypes.c_int64)]


class AttnStrides(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int64), ("batch", ctypes.c_int64),
                ("token", ctypes.c_int64), ("head", ctypes.c_int64)]


_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libspattn.so (once) and declare the signatures.  Raises if absent."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m sequence_attention_video_amd.build` "
                           "(there is no fallback path)")
    lib = ctypes.CDLL(p)
    i32, i64, vp, f32, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
    lib.sp_status_string.restype = ctypes.c_char_p
    lib.sp_status_string.argtypes = [ctypes.c_int]
    lib.sp_version.restype = i32
    lib.sp_version.argtypes = []
    lib.sp_partition.restype = ctypes.c_int
    lib.sp_partition.argtypes = [i64, i32, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.sp_pad.restype = ctypes.c_int
    lib.sp_pad.argtypes = [vp, i64, vp, i64, i64, i64, i64, ctypes.c_int, vp, vp, vp]
    lib.sp_relayout_heads.restype = ctypes.c_int
    lib.sp_relayout_heads.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), i32, i32, i64, i64, i32, i32,
                                      ctypes.c_int, ctypes.c_int, ShardStrides, ShardStrides, vp]
    lib.sp_masked_attention_workspace_size.restype = sz
    lib.sp_masked_attention_workspace_size.argtypes = [i32, i64, i64, i64, i32, i32, ctypes.c_int, i32, i64]
    lib.sp_masked_attention.restype = ctypes.c_int
    lib.sp_masked_attention.argtypes = [vp, AttnStrides, vp, AttnStrides, vp, AttnStrides, vp, AttnStrides,
                                        i32, i64, i64, i64, i32, i32, ctypes.c_int, i64, vp, i64, f32, vp, sz, vp]
    lib.sp_masked_attention_noalloc.restype = ctypes.c_int
    lib.sp_masked_attention_noalloc.argtypes = [vp, AttnStrides, vp, AttnStrides, vp, AttnStrides, vp, AttnStrides,
                                                i32, i64, i64, i64, i32, i32, ctypes.c_int, i64, vp, i64, f32, vp]
    lib.sp_gather_unpad.restype = ctypes.c_int
    lib.sp_gather_unpad.argtypes = [vp, ShardStrides, vp, i32, i64, i64, i64, ctypes.POINTER(i64), i64,
                                    ctypes.c_int, vp]
    lib.sp_optimal_split.restype = ctypes.c_int
    lib.sp_optimal_split.argtypes = [i32, i64, i64, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.sp_tile_2d.restype = ctypes.c_int
    lib.sp_tile_2d.argtypes = [vp, vp, i32, i32, i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                               ShardStrides, i64, vp]
    lib.sp_tile_2d_relayout_heads.restype = ctypes.c_int
    lib.sp_tile_2d_relayout_heads.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), i32, i32, i32, i64, i64, i64,
                                              i64, i32, i32, ctypes.c_int, ctypes.c_int, i64, ShardStrides, vp]
    lib.sp_pad_relayout_heads.restype = ctypes.c_int
    lib.sp_pad_relayout_heads.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), i32, i32, i64, i64, i64, i32, i32,
                                          ctypes.c_int, i64, ShardStrides, vp]
    lib.sp_gather_heads_unpad.restype = ctypes.c_int
    lib.sp_gather_heads_unpad.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), i32, i32, i64, i64, i32, i32,
                                          ctypes.c_int, ShardStrides, ctypes.POINTER(i64), i64, vp]
    if path is None:
        _lib = lib
    return lib


def check(status: int) -> None:
    if status == SP_OK:
        return
    msg = load().sp_status_string(status).decode()
    if status in (SP_ERR_NOT_DIVISIBLE, SP_ERR_INVALID_ARG, SP_ERR_SCRATCH):
        raise ValueError(msg)
    if status == SP_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise RuntimeError(msg)


# ---------------------------------------------------------------- helpers

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return SP_F32
    if t.dtype == torch.bfloat16:
        return SP_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on the GPU")


# ---------------------------------------------------------------- entry points

def sp_partition(total_tokens: int, world_size: int):
    """compute_sequence_partition: (offsets, lengths); ValueError if not divisible."""
    n = max(int(world_size), 0)
    offs = (ctypes.c_int64 * max(n, 1))()
    lens = (ctypes.c_int64 * max(n, 1))()
    check(load().sp_partition(int(total_tokens), int(world_size), offs, lens))
    return list(offs[:n]), list(lens[:n])


def sp_pad(x, y, T_pad: int, mask_in=None, mask_out=None, x_batch_stride: int | None = None,
           T: int | None = None, stream=None):
    """pad_modality_for_uniform_sharding on the GPU.

    x: (B, T, C) (or any tensor whose batch stride is ``x_batch_stride``); y:
    (B, T_pad, C) packed; optional user mask (B, T, T) uint8 -> (B, T_pad, T_pad).
    ``x``/``y`` may be None to extend only the mask.
    """
    _cuda(x, y, mask_in, mask_out)
    if x is not None:
        B, C = y.shape[0], y.shape[-1] if y.dim() == 3 else int(y[0, 0].numel())
        if T is None:
            T = x.shape[1]
        xbs = x.stride(0) if x_batch_stride is None else x_batch_stride
        dt = _dtype_code(x)
    else:
        B, C, dt, xbs = mask_in.shape[0], 0, SP_F32, 0
        T = mask_in.shape[1] if T is None else T
    if (mask_in is None) != (mask_out is None):
        raise ValueError("mask_in and mask_out go together")
    if mask_in is not None:
        # the library reads B*T*T mask bytes and writes B*T_pad*T_pad: both
        # buffers must hold exactly that (one shared mask: extend it alone)
        if tuple(mask_in.shape) != (B, T, T) or not mask_in.is_contiguous():
            raise ValueError(f"mask_in must be a packed ({B}, {T}, {T}) tensor, got {tuple(mask_in.shape)}")
        if tuple(mask_out.shape) != (B, T_pad, T_pad) or not mask_out.is_contiguous():
            raise ValueError(f"mask_out must be a packed ({B}, {T_pad}, {T_pad}) tensor, "
                             f"got {tuple(mask_out.shape)}")
    check(load().sp_pad(_ptr(x), int(xbs), _ptr(y), int(B), int(T), int(T_pad), int(C), dt,
                        _ptr(mask_in), _ptr(mask_out), _stream(stream)))


def sp_relayout_heads(src, dst, W: int, B: int, T_pad: int, H: int, D: int, direction: int,
                      tok_strides=None, head_strides=None, stream=None):
    """send_recv_heads (SP_TOKENS_TO_HEADS) or gather_heads (SP_HEADS_TO_TOKENS).

    ``src``/``dst``: lists of 1..3 tensors.  Default layouts: token side
    stacked (W, B, Ts, H, D), head side stacked (W, B, T_pad, Hl, D).
    """
    src, dst = list(src), list(dst)
    _cuda(*src, *dst)
    Ts, Hl = T_pad // max(W, 1), H // max(W, 1)
    tok = tok_strides or (B * Ts * H * D, Ts * H * D)
    head = head_strides or (B * T_pad * Hl * D, T_pad * Hl * D)
    n = len(src)
    sp = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in src])
    dp = (ctypes.c_void_p * max(len(dst), 1))(*[t.data_ptr() for t in dst])
    if len(dst) != n:
        raise ValueError("one destination per source")
    check(load().sp_relayout_heads(sp, dp, n, int(W), int(B), int(T_pad), int(H), int(D), _dtype_code(src[0]),
                                   int(direction), ShardStrides(*tok), ShardStrides(*head), _stream(stream)))


def sp_masked_attention_workspace_size(R, B, Tq, Tk, Hl, D, dtype_code, has_mask, mask_batch_stride) -> int:
    return int(load().sp_masked_attention_workspace_size(int(R), int(B), int(Tq), int(Tk), int(Hl), int(D),
                                                         int(dtype_code), int(has_mask), int(mask_batch_stride)))


def sp_masked_attention(q, k, v, o, R: int, B: int, Tq: int, Tk: int, Hl: int, D: int,
                        q_strides, k_strides, v_strides, o_strides, kv_valid_len: int | None = None,
                        mask=None, mask_batch_stride: int | None = None, scale: float | None = None,
                        workspace=None, stream=None):
    """Attention on the local heads of R rank shares; strides are (rank, batch, token, head)."""
    _cuda(q, k, v, o, mask, workspace)
    dt = _dtype_code(q)
    if kv_valid_len is None:
        kv_valid_len = Tk
    if scale is None:
        scale = 1.0 / (D ** 0.5)
    mbs = 0
    if mask is not None:
        mbs = (mask.stride(0) if mask.shape[0] > 1 else 0) if mask_batch_stride is None else mask_batch_stride
    need = sp_masked_attention_workspace_size(R, B, Tq, Tk, Hl, D, dt, mask is not None, mbs)
    if need and workspace is None:
        torch = _torch()
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(load().sp_masked_attention(_ptr(q), AttnStrides(*q_strides), _ptr(k), AttnStrides(*k_strides),
                                     _ptr(v), AttnStrides(*v_strides), _ptr(o), AttnStrides(*o_strides),
                                     int(R), int(B), int(Tq), int(Tk), int(Hl), int(D), dt, int(kv_valid_len),
                                     _ptr(mask), int(mbs), float(scale), _ptr(workspace), int(wbytes),
                                     _stream(stream)))


def sp_masked_attention_noalloc(q, k, v, o, R: int, B: int, Tq: int, Tk: int, Hl: int, D: int,
                                q_strides, k_strides, v_strides, o_strides, kv_valid_len: int | None = None,
                                mask=None, mask_batch_stride: int | None = None, scale: float | None = None,
                                stream=None):
    """sp_masked_attention on the library's fixed per-GPU scratch: no workspace
    argument and no allocation (calls on one GPU must not overlap)."""
    _cuda(q, k, v, o, mask)
    dt = _dtype_code(q)
    if kv_valid_len is None:
        kv_valid_len = Tk
    if scale is None:
        scale = 1.0 / (D ** 0.5)
    mbs = 0
    if mask is not None:
        mbs = (mask.stride(0) if mask.shape[0] > 1 else 0) if mask_batch_stride is None else mask_batch_stride
    check(load().sp_masked_attention_noalloc(_ptr(q), AttnStrides(*q_strides), _ptr(k), AttnStrides(*k_strides),
                                             _ptr(v), AttnStrides(*v_strides), _ptr(o), AttnStrides(*o_strides),
                                             int(R), int(B), int(Tq), int(Tk), int(Hl), int(D), dt,
                                             int(kv_valid_len), _ptr(mask), int(mbs), float(scale),
                                             _stream(stream)))


def sp_gather_unpad(inp, out, W: int, B: int, Ts: int, C: int, T: int, counts=None,
                    in_strides=None, stream=None):
    """gather_output_tokens: (W, B, Ts, C) rank pieces -> (B, T, C)."""
    _cuda(inp, out)
    st = in_strides or (B * Ts * C, Ts * C)
    carr = None
    if counts is not None:
        carr = (ctypes.c_int64 * len(counts))(*[int(c) for c in counts])
    check(load().sp_gather_unpad(_ptr(inp), ShardStrides(*st), _ptr(out), int(W), int(B), int(Ts), int(C),
                                 carr, int(T), _dtype_code(inp), _stream(stream)))


def sp_optimal_split(n_ranks: int, height: int, width: int):
    """(split_h, split_w): the near-square rank grid of the 2-D split."""
    a, b = ctypes.c_int32(0), ctypes.c_int32(0)
    check(load().sp_optimal_split(int(n_ranks), int(height), int(width), ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def sp_tile_2d(src, dst, split_h: int, split_w: int, B: int, F: int, height: int, width: int, C: int,
               direction: int, tile_strides=None, grid_batch_stride=None, stream=None):
    """split_cp_2d (SP_GRID_TO_TILES) or gather_cp_2d (SP_TILES_TO_GRID) on one device.
    Grid side (B, F*height*width, C); tile side (N, B, F*th*tw, C) stacked unless strides are given."""
    _cuda(src, dst)
    grid = src if direction == SP_GRID_TO_TILES else dst
    tt = F * (height // split_h) * (width // split_w)
    ts = tile_strides or (B * tt * C, tt * C)
    gbs = grid_batch_stride if grid_batch_stride is not None else F * height * width * C
    check(load().sp_tile_2d(_ptr(src), _ptr(dst), int(split_h), int(split_w), int(B), int(F), int(height),
                            int(width), int(C), _dtype_code(grid), int(direction), ShardStrides(*ts), int(gbs),
                            _stream(stream)))


def sp_tile_2d_relayout_heads(src, dst, split_h: int, split_w: int, B: int, F: int, height: int, width: int,
                              H: int, D: int, direction: int, grid_batch_stride=None, head_strides=None,
                              stream=None):
    """split_cp_2d + send_recv_heads (SP_TOKENS_TO_HEADS: grid -> head side) or
    gather_heads + gather_cp_2d (SP_HEADS_TO_TOKENS: head side -> grid) as one
    move.  ``src``/``dst``: lists of 1..3 tensors.  Default layouts: grid
    (B, F*height*width, H, D), head side stacked (W, B, T, Hl, D)."""
    src, dst = list(src), list(dst)
    _cuda(*src, *dst)
    if len(dst) != len(src):
        raise ValueError("one destination per source")
    W = int(split_h) * int(split_w)
    T = F * height * width
    Hl = H // max(W, 1)
    gbs = grid_batch_stride if grid_batch_stride is not None else T * H * D
    head = head_strides or (B * T * Hl * D, T * Hl * D)
    n = len(src)
    sp = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in src])
    dp = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in dst])
    check(load().sp_tile_2d_relayout_heads(sp, dp, n, int(split_h), int(split_w), int(B), int(F), int(height),
                                           int(width), int(H), int(D), _dtype_code(src[0]), int(direction), int(gbs),
                                           ShardStrides(*head), _stream(stream)))


def _ptr_array(ts):
    return (ctypes.c_void_p * max(len(ts), 1))(*[t.data_ptr() for t in ts])


def sp_pad_relayout_heads(src, dst, W: int, B: int, T: int, T_pad: int, H: int, D: int,
                          src_batch_stride=None, head_strides=None, stream=None):
    """pad_modality_for_uniform_sharding + send_recv_heads as one move.
    ``src``: 1..3 unpadded token tensors (B, T, H, D); ``dst``: as many head
    sides, stacked (W, B, T_pad, Hl, D) unless ``head_strides`` is given."""
    src, dst = list(src), list(dst)
    _cuda(*src, *dst)
    if len(dst) != len(src):
        raise ValueError("one destination per source")
    Hl = H // max(W, 1)
    sbs = src_batch_stride if src_batch_stride is not None else src[0].stride(0)
    head = head_strides or (B * T_pad * Hl * D, T_pad * Hl * D)
    check(load().sp_pad_relayout_heads(_ptr_array(src), _ptr_array(dst), len(src), int(W), int(B), int(T),
                                       int(T_pad), int(H), int(D), _dtype_code(src[0]), int(sbs),
                                       ShardStrides(*head), _stream(stream)))


def sp_gather_heads_unpad(src, dst, W: int, B: int, T_pad: int, H: int, D: int, T: int, counts=None,
                          head_strides=None, stream=None):
    """gather_heads + gather_output_tokens as one move: 1..3 head sides
    (W, B, T_pad, Hl, D) -> as many outputs (B, T, H, D)."""
    src, dst = list(src), list(dst)
    _cuda(*src, *dst)
    if len(dst) != len(src):
        raise ValueError("one destination per source")
    Hl = H // max(W, 1)
    head = head_strides or (B * T_pad * Hl * D, T_pad * Hl * D)
    carr = None
    if counts is not None:
        carr = (ctypes.c_int64 * len(counts))(*[int(c) for c in counts])
    check(load().sp_gather_heads_unpad(_ptr_array(src), _ptr_array(dst), len(src), int(W), int(B), int(T_pad),
                                       int(H), int(D), _dtype_code(src[0]), ShardStrides(*head), carr, int(T),
                                       _stream(stream)))
