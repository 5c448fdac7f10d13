"""Seeded sweep of small random shapes through every data-movement entry
point, bit-exact against the CPU oracle: sp_pad (tokens, in a separate and in
the same buffer, and the user-mask extension), sp_relayout_heads both ways
(one to three tensors), sp_gather_unpad with random per-rank counts, and
sp_tile_2d_relayout_heads both ways, and the fused moves (pad + send_recv_heads,
gather_heads + gather_output_tokens).  Shapes cover W = 1..8, B = 1..3, ragged
token counts, head groups of one to a few 16-byte vectors, fp32 and bf16.
Outputs are prefilled with 0xFF bytes, so anything left unwritten (or written
twice with other bytes) shows."""

import numpy as np
import pytest
import torch

import oracle as O
from sequence_attention_video_amd import binding as sp
from tests.gpu_util import raw, say, sentinel_like, to_dev

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "bf16": torch.bfloat16}
NP = {"f32": np.uint32, "bf16": np.uint16}
N_CASES = 40


def bits(rng, shape, dtype):
    """Random bit patterns of the element type (any bytes: copies never look at values)."""
    a = rng.integers(0, 1 << (32 if dtype == "f32" else 16), size=shape, dtype=np.uint64).astype(NP[dtype])
    return a.view(np.float32) if dtype == "f32" else a


def dev(a):
    return to_dev(a)


def case(i):
    rng = np.random.default_rng(5000 + i)
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    vec = 8 if dtype == "bf16" else 4                      # elements per 16-byte vector
    W = int(rng.integers(1, 9))
    B = int(rng.integers(1, 4))
    Ts = int(rng.integers(1, 40))
    Hl = int(rng.integers(1, 4))
    D = vec * int(rng.integers(1, 5))                        # Hl*D*eb is a multiple of 16
    T = int(rng.integers(max(1, W * Ts - W + 1), W * Ts + 1))  # ragged: up to W-1 pad rows
    return rng, dtype, W, B, Ts, Hl, D, T


@pytest.mark.parametrize("i", range(N_CASES))
def test_copies_random_shapes(i):
    rng, dtype, W, B, Ts, Hl, D, T = case(i)
    H, T_pad = W * Hl, W * Ts
    C = H * D
    say("copy shapes", i, dtype, W, B, Ts, Hl, D, T)
    # pad (separate buffers, then in place), and the user-mask extension
    x = bits(rng, (B, T, C), dtype)
    y = sentinel_like((B, T_pad, C), TD[dtype])
    sp.sp_pad(dev(x), y, T_pad)
    buf = sentinel_like((B, T_pad, C), TD[dtype])
    buf.view(torch.uint8)[:, :T] = dev(x).view(torch.uint8)   # bytes (any float bit patterns)
    sp.sp_pad(buf, buf, T_pad, x_batch_stride=T_pad * C, T=T)
    m = (rng.random((B, T, T)) < 0.5).astype(np.uint8)
    mo = torch.full((B, T_pad, T_pad), 0xAB, dtype=torch.uint8, device="cuda")
    sp.sp_pad(None, None, T_pad, mask_in=dev(m), mask_out=mo)
    torch.cuda.synchronize()
    padded = O.pad_tokens(x, T_pad)
    assert raw(y).tobytes() == padded.tobytes()
    assert raw(buf).tobytes() == padded.tobytes()
    assert np.array_equal(raw(mo), O.extend_user_mask(m, T_pad))
    # send_recv_heads of n tensors, then gather_heads back
    n = int(rng.integers(1, 4))
    xs = [bits(rng, (B, T_pad, H, D), dtype) for _ in range(n)]
    heads = [sentinel_like((W, B, T_pad, Hl, D), TD[dtype]) for _ in range(n)]
    tok_view = (Ts * H * D, T_pad * H * D)
    sp.sp_relayout_heads([dev(a) for a in xs], heads, W, B, T_pad, H, D, sp.SP_TOKENS_TO_HEADS, tok_strides=tok_view)
    toks = [sentinel_like((W, B, Ts, H, D), TD[dtype]) for _ in range(n)]
    sp.sp_relayout_heads(heads, toks, W, B, T_pad, H, D, sp.SP_HEADS_TO_TOKENS)
    torch.cuda.synchronize()
    for a, h, t in zip(xs, heads, toks):
        want = O.send_recv_heads(O.token_shards(a, W))
        assert raw(h).tobytes() == want.tobytes()
        assert raw(t).tobytes() == O.gather_heads(want).tobytes()
    # gather_output_tokens with random counts that still cover T
    pieces = bits(rng, (W, B, Ts, C), dtype)
    counts = [int(c) for c in rng.integers(0, Ts + 1, size=W)]
    short = T - sum(counts)
    r = 0
    while short > 0:                                     # top up ranks until T rows are kept
        add = min(Ts - counts[r], short)
        counts[r] += add
        short -= add
        r += 1
    out = sentinel_like((B, T, C), TD[dtype])
    sp.sp_gather_unpad(dev(pieces), out, W, B, Ts, C, T, counts=counts)
    torch.cuda.synchronize()
    assert raw(out).tobytes() == O.gather_output_tokens([pieces[k] for k in range(W)], counts, T).tobytes()


@pytest.mark.parametrize("i", range(N_CASES // 2))
def test_tile_2d_relayout_heads_random_shapes(i):
    rng = np.random.default_rng(7000 + i)
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    vec = 8 if dtype == "bf16" else 4
    sh, sw = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    W = sh * sw
    th, tw, F, B = (int(v) for v in rng.integers(1, 5, size=4))
    Hh, Ww = sh * th, sw * tw
    Hl, D = int(rng.integers(1, 3)), vec * int(rng.integers(1, 3))
    H, T = W * Hl, F * Hh * Ww
    n = int(rng.integers(1, 4))
    say("tile_2d_relayout_heads shapes", i, dtype, sh, sw, B, F, Hh, Ww, H, D, n)
    xs = [bits(rng, (B, T, H, D), dtype) for _ in range(n)]
    heads = [sentinel_like((W, B, T, Hl, D), TD[dtype]) for _ in range(n)]
    sp.sp_tile_2d_relayout_heads([dev(a) for a in xs], heads, sh, sw, B, F, Hh, Ww, H, D, sp.SP_TOKENS_TO_HEADS)
    backs = [sentinel_like((B, T, H, D), TD[dtype]) for _ in range(n)]
    sp.sp_tile_2d_relayout_heads(heads, backs, sh, sw, B, F, Hh, Ww, H, D, sp.SP_HEADS_TO_TOKENS)
    torch.cuda.synchronize()
    for a, h, back in zip(xs, heads, backs):
        assert raw(h).tobytes() == O.send_recv_heads(O.split_cp_2d(a, F, Hh, Ww, sh, sw)).tobytes()
        assert raw(back).tobytes() == a.tobytes()


@pytest.mark.parametrize("i", range(N_CASES))
def test_fused_moves_random_shapes(i):
    """pad + send_recv_heads and gather_heads + gather_output_tokens as single
    moves: bit-exact against the oracle's composition of the two steps, one
    to three tensors, a source batch stride above T*H*D, random trim counts."""
    rng, dtype, W, B, Ts, Hl, D, T = case(100 + i)
    H, T_pad = W * Hl, W * Ts
    n = int(rng.integers(1, 4))
    extra = int(rng.integers(0, 3)) * H * D               # rows of slack between batches of the source
    say("fused moves shapes", i, dtype, W, B, Ts, Hl, D, T, n, extra)
    xs = [bits(rng, (B, T * H * D + extra), dtype) for _ in range(n)]
    heads = [sentinel_like((W, B, T_pad, Hl, D), TD[dtype]) for _ in range(n)]
    srcs = [dev(a) for a in xs]
    sp.sp_pad_relayout_heads([s[:, :T * H * D].view(B, T, H, D) if extra == 0 else s for s in srcs], heads,
                             W, B, T, T_pad, H, D, src_batch_stride=T * H * D + extra)
    torch.cuda.synchronize()
    for a, h in zip(xs, heads):
        x = a[:, :T * H * D].reshape(B, T, H, D)
        want = O.send_recv_heads(O.token_shards(O.pad_tokens(x, T_pad), W))
        assert raw(h).tobytes() == want.tobytes()
    # the way back, with random per-rank counts that still cover T
    hs = [bits(rng, (W, B, T_pad, Hl, D), dtype) for _ in range(n)]
    counts = [int(c) for c in rng.integers(0, Ts + 1, size=W)]
    short = T - sum(counts)
    r = 0
    while short > 0:
        add = min(Ts - counts[r], short)
        counts[r] += add
        short -= add
        r += 1
    outs = [sentinel_like((B, T, H, D), TD[dtype]) for _ in range(n)]
    sp.sp_gather_heads_unpad([dev(a) for a in hs], outs, W, B, T_pad, H, D, T, counts=counts)
    torch.cuda.synchronize()
    for a, o in zip(hs, outs):
        tok = O.gather_heads(a)                                     # (W, B, Ts, H, D)
        want = O.gather_output_tokens([tok[k].reshape(B, Ts, H * D) for k in range(W)], counts, T)
        assert raw(o).reshape(B, T, H * D).tobytes() == want.tobytes()
