"""GPU parity of the data-movement entry points against the CPU oracle:
sp_relayout_heads, sp_pad (tokens and user mask) and sp_gather_unpad must be
bit-exact.  Outputs are prefilled with 0xFF bytes, so an element the kernel
failed to write shows up as a mismatch."""

import numpy as np
import pytest
import torch

import oracle as O
from sequence_attention_video_amd import binding as sp
from tests.gpu_util import raw, rand_bits, say, sentinel_like, to_dev

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "bf16": torch.bfloat16}

RELAYOUT_CASES = [
    # W, B, T_pad, H, D, dtype
    (4, 1, 52, 8, 16, "f32"),       # the tiny workload's shape
    (1, 1, 5, 4, 128, "bf16"),      # W = 1: identity
    (2, 2, 10, 4, 64, "bf16"),
    (3, 2, 9, 6, 64, "f32"),        # odd W, Hl = 2
    (8, 2, 40, 32, 128, "bf16"),
    (8, 1, 1024, 32, 64, "bf16"),   # the cross workload's K/V
    (8, 1, 6152, 32, 128, "bf16"),  # ragged shard length 769
    (4, 3, 4100, 12, 128, "bf16"),  # Hl = 3: 48 vectors per run
]


@pytest.mark.parametrize("W,B,T_pad,H,D,dtype", RELAYOUT_CASES)
def test_relayout_bit_exact(W, B, T_pad, H, D, dtype):
    say("relayout", W, B, T_pad, H, D, dtype)
    rng = np.random.default_rng(100 + W * 7 + T_pad)
    Ts, Hl = T_pad // W, H // W
    xs = [rand_bits(rng, (B, T_pad, H, D), dtype) for _ in range(3)]
    xd = [to_dev(x) for x in xs]
    heads = [sentinel_like((W, B, T_pad, Hl, D), TD[dtype]) for _ in range(3)]
    tok_view = (Ts * H * D, T_pad * H * D)     # rank shards as views of (B, T_pad, H, D)
    sp.sp_relayout_heads(xd, heads, W, B, T_pad, H, D, sp.SP_TOKENS_TO_HEADS, tok_strides=tok_view)
    torch.cuda.synchronize()
    for x, hd in zip(xs, heads):
        want = O.send_recv_heads(O.token_shards(x, W))
        assert raw(hd).tobytes() == want.tobytes()
    # swap back into the stacked per-rank layout (W, B, Ts, H, D)
    tok = sentinel_like((W, B, Ts, H, D), TD[dtype])
    sp.sp_relayout_heads([heads[0]], [tok], W, B, T_pad, H, D, sp.SP_HEADS_TO_TOKENS)
    # and into the (B, T_pad, H, D) layout: the byte-exact round trip
    back = sentinel_like((B, T_pad, H, D), TD[dtype])
    sp.sp_relayout_heads([heads[1]], [back], W, B, T_pad, H, D, sp.SP_HEADS_TO_TOKENS, tok_strides=tok_view)
    torch.cuda.synchronize()
    assert raw(tok).tobytes() == O.gather_heads(O.send_recv_heads(O.token_shards(xs[0], W))).tobytes()
    assert raw(tok).tobytes() == O.token_shards(xs[0], W).tobytes()
    assert raw(back).tobytes() == xs[1].tobytes()
    # all three tensors back in one launch
    toks = [sentinel_like((W, B, Ts, H, D), TD[dtype]) for _ in range(3)]
    sp.sp_relayout_heads(heads, toks, W, B, T_pad, H, D, sp.SP_HEADS_TO_TOKENS)
    torch.cuda.synchronize()
    for x, t in zip(xs, toks):
        assert raw(t).tobytes() == O.token_shards(x, W).tobytes()


@pytest.mark.parametrize("W,B,T_pad,H,D,dtype", [(4, 2, 64, 8, 64, "bf16"), (2, 3, 30, 4, 16, "f32")])
def test_gather_heads_strided_head_side(W, B, T_pad, H, D, dtype):
    """gather_heads from head-side shards that are views into longer buffers
    (rank and batch strides beyond the packed sizes)."""
    say("gather_heads strided", W, B, T_pad, H, D, dtype)
    rng = np.random.default_rng(7 + T_pad)
    Ts, Hl, extra = T_pad // W, H // W, 5
    big = rand_bits(rng, (W, B, T_pad + extra, Hl, D), dtype)
    tok = sentinel_like((W, B, Ts, H, D), TD[dtype])
    head_view = (B * (T_pad + extra) * Hl * D, (T_pad + extra) * Hl * D)
    sp.sp_relayout_heads([to_dev(big)], [tok], W, B, T_pad, H, D, sp.SP_HEADS_TO_TOKENS, head_strides=head_view)
    torch.cuda.synchronize()
    want = O.gather_heads(np.ascontiguousarray(big[:, :, :T_pad]))
    assert raw(tok).tobytes() == want.tobytes()


def test_relayout_rejects_bad_shapes():
    x = torch.zeros(1, 50, 8, 16, device="cuda")
    y = torch.zeros(4, 1, 52, 2, 16, device="cuda")
    with pytest.raises(ValueError):           # 50 tokens do not split over 4 ranks
        sp.sp_relayout_heads([x], [y], 4, 1, 50, 8, 16, sp.SP_TOKENS_TO_HEADS)
    with pytest.raises(ValueError):           # H = 6 does not split over 4 ranks
        sp.sp_relayout_heads([x], [y], 4, 1, 52, 6, 16, sp.SP_TOKENS_TO_HEADS)
    with pytest.raises(ValueError):           # in place is refused
        sp.sp_relayout_heads([y], [y], 4, 1, 52, 8, 16, sp.SP_TOKENS_TO_HEADS)


PAD_CASES = [
    # B, T, T_pad, C, dtype
    (1, 50, 52, 128, "f32"),
    (1, 6150, 6152, 4096, "bf16"),
    (1, 987, 1024, 2048, "bf16"),
    (2, 7, 16, 64, "bf16"),
    (3, 5, 5, 8, "f32"),        # nothing to pad: a plain copy
    (2, 0, 8, 64, "bf16"),      # empty input: all zeros
]


@pytest.mark.parametrize("B,T,T_pad,C,dtype", PAD_CASES)
def test_pad_tokens_bit_exact(B, T, T_pad, C, dtype):
    say("pad", B, T, T_pad, C, dtype)
    rng = np.random.default_rng(200 + T)
    x = rand_bits(rng, (B, T, C), dtype)
    xd = to_dev(x) if T > 0 else torch.empty(B, 0, C, dtype=TD[dtype], device="cuda")
    y = sentinel_like((B, T_pad, C), TD[dtype])
    sp.sp_pad(xd, y, T_pad, x_batch_stride=T * C, T=T)
    torch.cuda.synchronize()
    assert raw(y).tobytes() == O.pad_tokens(x, T_pad).tobytes()


def test_pad_in_place():
    say("pad in place")
    rng = np.random.default_rng(7)
    B, T, T_pad, C = 2, 13, 16, 64
    x = rand_bits(rng, (B, T, C), "bf16")
    buf = sentinel_like((B, T_pad, C), torch.bfloat16)
    buf[:, :T] = to_dev(x)
    sp.sp_pad(buf, buf, T_pad, x_batch_stride=T_pad * C, T=T)
    torch.cuda.synchronize()
    assert raw(buf).tobytes() == O.pad_tokens(x, T_pad).tobytes()


@pytest.mark.parametrize("B,T,T_pad", [(1, 3, 4), (1, 50, 52), (2, 13, 16), (1, 6150, 6152), (3, 1, 7), (1, 33, 33)])
def test_pad_mask_bit_exact(B, T, T_pad):
    say("pad mask", B, T, T_pad)
    rng = np.random.default_rng(300 + T)
    m = (rng.random((B, T, T)) < 0.5).astype(np.uint8)
    out = torch.full((B, T_pad, T_pad), 0xAB, dtype=torch.uint8, device="cuda")
    sp.sp_pad(None, None, T_pad, mask_in=to_dev(m), mask_out=out)
    torch.cuda.synchronize()
    assert np.array_equal(raw(out), O.extend_user_mask(m, T_pad))


GATHER_CASES = [
    # W, B, Ts, C, T, counts, dtype
    (4, 1, 13, 128, 50, None, "f32"),
    (8, 1, 769, 4096, 6150, None, "bf16"),
    (8, 2, 16, 256, 128, None, "bf16"),
    (3, 2, 5, 64, 11, [5, 3, 4], "bf16"),     # uneven counts (a rank trims rows)
    (2, 1, 4, 32, 4, [1, 4], "f32"),
    (8, 1, 768, 2048, 6144, None, "bf16"),    # the cross workload's output
]


@pytest.mark.parametrize("W,B,Ts,C,T,counts,dtype", GATHER_CASES)
def test_gather_unpad_bit_exact(W, B, Ts, C, T, counts, dtype):
    say("gather", W, B, Ts, C, T, counts, dtype)
    rng = np.random.default_rng(400 + Ts)
    x = rand_bits(rng, (W, B, Ts, C), dtype)
    out = sentinel_like((B, T, C), TD[dtype])
    sp.sp_gather_unpad(to_dev(x), out, W, B, Ts, C, T, counts=counts)
    torch.cuda.synchronize()
    cnt = counts if counts is not None else [Ts] * W
    want = O.gather_output_tokens([x[r] for r in range(W)], cnt, T)
    assert raw(out).tobytes() == want.tobytes()


def test_gather_unpad_from_strided_shards():
    """Rank pieces that are views of one (B, T_pad, C) tensor (rank stride Ts*C)."""
    say("gather strided")
    rng = np.random.default_rng(9)
    W, B, Ts, C, T = 4, 2, 6, 64, 22
    full = rand_bits(rng, (B, W * Ts, C), "bf16")
    out = sentinel_like((B, T, C), torch.bfloat16)
    sp.sp_gather_unpad(to_dev(full), out, W, B, Ts, C, T, in_strides=(Ts * C, W * Ts * C))
    torch.cuda.synchronize()
    pieces = [full[:, r * Ts:(r + 1) * Ts] for r in range(W)]
    assert raw(out).tobytes() == O.gather_output_tokens(pieces, [Ts] * W, T).tobytes()
