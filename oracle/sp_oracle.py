"""Plain CPU oracle for Ulysses-style sequence-parallel attention (TEST INFRASTRUCTURE).

This module is test infrastructure, not product code.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the HIP path (``sequence_attention_video_amd``)
and imports nothing from it: it takes NumPy arrays and returns NumPy arrays.

Everything is computed in float64 (bfloat16 inputs are widened exactly, see
``bf16_bits_to_f64``).  Each function is the plain definition of one step, in
the order the pages give the steps, with no blocking or fusion beyond the
query-row blocking of ``attention`` (which changes memory use, not results).

Pages cited (title, then the section on that page):

* [SP]  "LTX-2 序列并行拆解：token 切分、all2all 换头与 runner 接入全链路"
        (gtnt.cn news 105700).  Sections used:
        "token 切片、换头、gather 还原：数据在卡间怎么流转" and its four steps
        补齐 (pad), 切分 (partition), 换头 (head swap), 还原 (restore);
        "全局注意力没有变，只是分布方式变了" (the invariants).
* [MG]  "Multi-GPU Inference" (LTX-2 ``docs/multigpu/README.md``), table
        "Capabilities", row "Sequence parallelism (SP)".
* [LC]  "LongCat-Video上下文并行技术如何实现高效的多GPU推理", section
        "智能张量拆分策略" (the 2-D height x width split and its near-square
        choice of split ratio).

Readings of points the pages leave open are numbered R1..R13 and listed in the
repository's design notes; each function names the ones it relies on.

Pin status: every function below is pinned by ``tests/test_oracle_pins.py``
(worked examples under ``tests/golden/``, closed forms, a library routine on
the unsharded case, and pure-Python brute force on tiny inputs).  No function
is left parity unpinned.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "padded_length",
    "compute_sequence_partition",
    "pad_tokens",
    "key_padding_mask",
    "extend_user_mask",
    "tile_for_rank",
    "token_shards",
    "send_recv_heads",
    "gather_heads",
    "attention",
    "attention_heads",
    "gather_output_tokens",
    "ulysses_self_attention",
    "ulysses_cross_attention",
    "joint_av_block",
    "get_optimal_split",
    "split_cp_2d",
    "gather_cp_2d",
    "ulysses_self_attention_2d",
    "reference_attention",
]


# ---------------------------------------------------------------------------
# value decoding
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 values stored as uint16 bit patterns to float64, exactly.

    A bfloat16 is the upper 16 bits of an IEEE float32, so shifting the pattern
    left by 16 gives the float32 with the same value; float32 -> float64 is exact.
    """
    u = np.asarray(bits, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# [SP] step 补齐 (pad): pad_modality_for_uniform_sharding
# ---------------------------------------------------------------------------

def padded_length(total_tokens: int, world_size: int) -> int:
    """Smallest multiple of ``world_size`` that is >= ``total_tokens``.

    [SP] 补齐: the sequence dimension is padded up to a whole multiple of the
    world size.
    """
    if world_size < 1:
        raise ValueError("world_size must be >= 1")
    if total_tokens < 0:
        raise ValueError("total_tokens must be >= 0")
    return world_size * (-(-total_tokens // world_size))


def pad_tokens(x: np.ndarray, t_pad: int) -> np.ndarray:
    """Pad the token axis (axis 1) of ``x`` (B, T, ...) to ``t_pad`` rows.

    [SP] 补齐.  R2: the pad rows hold zero bytes.  R3: padding goes at the tail
    of the token axis.  Works on any dtype (bf16 bit patterns included), as a
    byte move.
    """
    x = np.asarray(x)
    b, t = x.shape[:2]
    if t_pad < t:
        raise ValueError(f"t_pad={t_pad} < T={t}")
    y = np.zeros((b, t_pad) + x.shape[2:], dtype=x.dtype)
    y[:, :t] = x
    return y


def key_padding_mask(t_valid: int, t_pad: int) -> np.ndarray:
    """Key-only padding mask of shape (1, 1, t_pad): True where the key is real.

    [SP] 补齐: with no user mask only an O(T) key mask is built, never a (B,T,T)
    matrix.  R4: True (1) means the key may be attended.
    """
    return (np.arange(t_pad) < t_valid).reshape(1, 1, t_pad)


def extend_user_mask(user_mask: np.ndarray, t_pad: int) -> np.ndarray:
    """Extend a user mask (B, T, T) to (B, t_pad, t_pad), as uint8 0/1.

    [SP] 补齐: the user mask gains pad rows and pad columns, and the pad query
    rows keep sight of the real keys so that no row is fully masked.
    R4: 1 = may attend.  R5: a pad query row sees every real key and no pad
    key.  R6: pad key columns are 0 for every query row.
    """
    m = np.asarray(user_mask)
    b, tq, tk = m.shape
    if tq != tk:
        raise ValueError("a self-attention user mask is square in its token axes")
    t = tq
    if t_pad < t:
        raise ValueError(f"t_pad={t_pad} < T={t}")
    out = np.zeros((b, t_pad, t_pad), dtype=np.uint8)
    out[:, :t, :t] = (m != 0)
    out[:, t:, :t] = 1
    return out


# ---------------------------------------------------------------------------
# [SP] step 切分 (partition): compute_sequence_partition, tile_modality_for_rank
# ---------------------------------------------------------------------------

def compute_sequence_partition(total_tokens: int, world_size: int):
    """Offsets and lengths of the ``world_size`` equal token shards.

    [SP] 切分: the total must divide evenly by the world size, otherwise a
    ValueError is raised; equal shards are what let the exchange derive its
    output shape from its input shape (times or divided by the world size).
    """
    if world_size < 1:
        raise ValueError("world_size must be >= 1")
    if total_tokens < 0:
        raise ValueError("total_tokens must be >= 0")
    if total_tokens % world_size != 0:
        raise ValueError(
            f"total_tokens={total_tokens} is not divisible by world_size={world_size}")
    ts = total_tokens // world_size
    offsets = [r * ts for r in range(world_size)]
    lengths = [ts] * world_size
    return offsets, lengths


def tile_for_rank(x: np.ndarray, rank: int, world_size: int) -> np.ndarray:
    """Rank ``rank``'s token slice of ``x`` (B, T_pad, ...): [SP] 切分."""
    offsets, lengths = compute_sequence_partition(x.shape[1], world_size)
    return x[:, offsets[rank]:offsets[rank] + lengths[rank]]


def token_shards(x: np.ndarray, world_size: int) -> np.ndarray:
    """Stack every rank's token slice: (B, T_pad, H, D) -> (W, B, Ts, H, D)."""
    return np.stack([tile_for_rank(x, r, world_size) for r in range(world_size)])


# ---------------------------------------------------------------------------
# [SP] step 换头 (head swap): send_recv_heads / gather_heads
# ---------------------------------------------------------------------------

def send_recv_heads(shards: np.ndarray) -> np.ndarray:
    """Token-sharded -> head-sharded exchange for W ranks.

    [SP] 换头: after the exchange every rank holds all tokens of H/W of the
    heads.  Input ``shards`` is (W, B, Ts, H, D): rank s's token shard.
    Output is (W, B, W*Ts, H/W, D): rank r's head shard, whose token rows
    s*Ts .. s*Ts+Ts-1 come from rank s and whose local head j is global head
    r*(H/W)+j.  H must divide by W (R9).
    """
    w, b, ts, h, d = shards.shape
    if h % w != 0:
        raise ValueError(f"H={h} is not divisible by world_size={w}")
    hl = h // w
    out = np.empty((w, b, w * ts, hl, d), dtype=shards.dtype)
    for r in range(w):          # receiving rank = head group
        for s in range(w):      # sending rank = token block
            out[r, :, s * ts:(s + 1) * ts] = shards[s, :, :, r * hl:(r + 1) * hl]
    return out


def gather_heads(heads: np.ndarray) -> np.ndarray:
    """Head-sharded -> token-sharded exchange, the inverse of ``send_recv_heads``.

    [SP] 换头: the attention output is swapped back.  Input (W, B, T_pad, Hl, D),
    output (W, B, T_pad/W, W*Hl, D).
    """
    w, b, t_pad, hl, d = heads.shape
    if t_pad % w != 0:
        raise ValueError(f"T_pad={t_pad} is not divisible by world_size={w}")
    ts = t_pad // w
    out = np.empty((w, b, ts, w * hl, d), dtype=heads.dtype)
    for s in range(w):          # receiving rank = token block
        for r in range(w):      # sending rank = head group
            out[s, :, :, r * hl:(r + 1) * hl] = heads[r, :, s * ts:(s + 1) * ts]
    return out


# ---------------------------------------------------------------------------
# [SP] step 换头, "就地算注意力": attention on the local heads
# ---------------------------------------------------------------------------

def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
              kv_valid_len: int | None = None, mask: np.ndarray | None = None,
              row_block: int = 1024) -> np.ndarray:
    """Softmax attention of one head, float64.

    q (Tq, D), k (Tk, D), v (Tk, Dv); ``mask`` (Tq, Tk) with nonzero = may attend.
    Query i attends key j iff j < kv_valid_len and (no mask or mask[i, j]).
    Score s_ij = scale * (q_i . k_j); over the visible keys,
    o_i = sum_j exp(s_ij - m_i) v_j / sum_j exp(s_ij - m_i) with m_i the largest
    visible score.  R7: a row with no visible key returns 0.
    R8: ``scale`` is explicit (callers pass 1/sqrt(D)).

    [SP] 补齐 (what the masks mean) and 换头 (attention runs over the full
    sequence on the local heads).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    tq, tk = q.shape[0], k.shape[0]
    if kv_valid_len is None:
        kv_valid_len = tk
    key_ok = np.arange(tk) < kv_valid_len
    out = np.zeros((tq, v.shape[1]), dtype=np.float64)
    for i0 in range(0, tq, row_block):
        i1 = min(tq, i0 + row_block)
        s = (q[i0:i1] @ k.T) * scale
        vis = np.broadcast_to(key_ok, s.shape)
        if mask is not None:
            vis = vis & (np.asarray(mask[i0:i1]) != 0)
        s = np.where(vis, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        has = np.isfinite(m[:, 0])
        m = np.where(np.isfinite(m), m, 0.0)
        p = np.where(vis, np.exp(s - m), 0.0)
        den = p.sum(axis=1, keepdims=True)
        num = p @ v
        out[i0:i1] = np.where(has[:, None], num / np.where(den > 0, den, 1.0), 0.0)
    return out


def attention_heads(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                    kv_valid_len: int | None = None, mask: np.ndarray | None = None,
                    rows: np.ndarray | None = None) -> np.ndarray:
    """``attention`` for every (batch, head) of (B, Tq, Hh, D) / (B, Tk, Hh, D).

    ``mask`` is (B, Tq, Tk) or (1, Tq, Tk) (broadcast over batch) or None.
    ``rows`` optionally restricts the query rows computed (the rest stay 0);
    attention is independent per query row, so a subset equals the same rows
    of the full result.
    """
    b, tq, hh, _ = q.shape
    out = np.zeros((b, tq, hh, v.shape[3]), dtype=np.float64)
    sel = np.arange(tq) if rows is None else np.asarray(rows)
    for bi in range(b):
        mb = None
        if mask is not None:
            mb = mask[bi if mask.shape[0] > 1 else 0][sel]
        for j in range(hh):
            out[bi, sel, j] = attention(q[bi, sel, j], k[bi, :, j], v[bi, :, j],
                                        scale, kv_valid_len, mb)
    return out


# ---------------------------------------------------------------------------
# [SP] step 还原 (restore): gather_output_tokens
# ---------------------------------------------------------------------------

def gather_output_tokens(local_outputs, counts, t_valid: int) -> np.ndarray:
    """Rebuild the caller's (B, T, C) output from each rank's (B, L_r, C) piece.

    [SP] 还原: every rank pads its local output to the longest length, the
    pieces are all-gathered, each is trimmed to that rank's real token count,
    the trimmed pieces are concatenated along tokens, and the result is
    unpadded to the caller's original length.  R10: the count kept per rank is
    given by ``counts`` (the shard length with uniform shards).
    """
    pieces = [np.asarray(p) for p in local_outputs]
    w = len(pieces)
    if len(counts) != w:
        raise ValueError("one count per rank")
    lmax = max(p.shape[1] for p in pieces)
    padded = [pad_tokens(p, lmax) for p in pieces]
    gathered = np.stack(padded)                     # what all_gather returns: (W, B, Lmax, C)
    kept = []
    for r in range(w):
        if not 0 <= counts[r] <= pieces[r].shape[1]:
            raise ValueError(f"count {counts[r]} out of range for rank {r}")
        kept.append(gathered[r, :, :counts[r]])
    joined = np.concatenate(kept, axis=1)
    if joined.shape[1] < t_valid:
        raise ValueError("fewer gathered tokens than the original length")
    return joined[:, :t_valid]


# ---------------------------------------------------------------------------
# the whole path, and the unsharded result it must equal
# ---------------------------------------------------------------------------

def ulysses_self_attention(q, k, v, world_size: int, scale: float,
                           user_mask=None, t_pad: int | None = None,
                           keep_intermediates: bool = False):
    """Self-attention through the whole sequence-parallel path, all W ranks.

    q, k, v: (B, T, H, D) float64 (already widened).  ``user_mask``: (B, T, T)
    or None.  Steps in the order of [SP] "token 切片、换头、gather 还原":
    pad -> partition -> tile -> send_recv_heads -> attention on the local
    heads -> gather_heads -> gather_output_tokens.  Returns (B, T, H, D).
    """
    b, t, h, d = q.shape
    if t_pad is None:
        t_pad = padded_length(t, world_size)
    qp, kp, vp = (pad_tokens(a, t_pad) for a in (q, k, v))
    if user_mask is None:
        kv_valid, mask = t, None
    else:
        kv_valid, mask = t_pad, extend_user_mask(user_mask, t_pad)
    offsets, lengths = compute_sequence_partition(t_pad, world_size)
    qh, kh, vh = (send_recv_heads(token_shards(a, world_size)) for a in (qp, kp, vp))
    oh = np.stack([attention_heads(qh[r], kh[r], vh[r], scale, kv_valid, mask)
                   for r in range(world_size)])
    ot = gather_heads(oh)                                   # (W, B, Ts, H, D)
    local = [ot[r].reshape(b, lengths[r], h * d) for r in range(world_size)]
    out = gather_output_tokens(local, lengths, t).reshape(b, t, h, d)
    if keep_intermediates:
        return out, dict(q_heads=qh, k_heads=kh, v_heads=vh, o_heads=oh, o_tokens=ot,
                         mask=mask, kv_valid=kv_valid, offsets=offsets)
    return out


def ulysses_cross_attention(q, k, v, world_size: int, scale: float,
                            kv_valid_len: int, t_kv_pad: int,
                            keep_intermediates: bool = False, t_q_pad: int | None = None):
    """Cross-attention variant: only K/V go through the exchange.

    [SP] 换头: for the video->audio cross-attention the query side is sliced on
    the rank itself and never exchanged; only K and V are swapped.  R11: rank r
    takes heads r*Hl..(r+1)*Hl of the whole query sequence q (B, Tq, H, D) in
    place; k, v (B, Tkv, H, D) hold ``kv_valid_len`` real keys, padded to
    ``t_kv_pad`` (R12) and exchanged; the output goes back through
    gather_heads and gather_output_tokens to (B, Tq, H, D).

    ``t_q_pad``: the query modality's own padded length ([SP] 补齐 pads each
    modality's sequence to a multiple of world_size; 还原 unpads the output to
    the caller's length).  Needed when Tq is not a multiple of world_size (an
    audio query sequence); pad query rows attend like any row and are dropped
    by the unpad.  Default: Tq itself.
    """
    b, tq, h, d = q.shape
    if h % world_size != 0:
        raise ValueError(f"H={h} is not divisible by world_size={world_size}")
    hl = h // world_size
    tq_pad = tq if t_q_pad is None else t_q_pad
    q = pad_tokens(q, tq_pad)
    kp, vp = pad_tokens(k[:, :kv_valid_len], t_kv_pad), pad_tokens(v[:, :kv_valid_len], t_kv_pad)
    compute_sequence_partition(t_kv_pad, world_size)
    kh, vh = (send_recv_heads(token_shards(a, world_size)) for a in (kp, vp))
    oh = np.stack([attention_heads(q[:, :, r * hl:(r + 1) * hl], kh[r], vh[r], scale,
                                   kv_valid_len, None)
                   for r in range(world_size)])             # (W, B, Tq_pad, Hl, D)
    ot = gather_heads(oh)                                   # (W, B, Tq_pad/W, H, D)
    offsets, lengths = compute_sequence_partition(tq_pad, world_size)
    local = [ot[r].reshape(b, lengths[r], h * d) for r in range(world_size)]
    out = gather_output_tokens(local, lengths, tq).reshape(b, tq, h, d)
    if keep_intermediates:
        return out, dict(k_heads=kh, v_heads=vh, o_heads=oh, o_tokens=ot)
    return out


def joint_av_block(parts: dict, world_size: int, video_tokens: int, audio_tokens: int):
    """The joint audio-video attention of one block on the sequence-parallel
    path, the pages' per-step chain around it ([SP] "token 切片、换头、gather
    还原": 补齐 per modality, 换头 for self-attention, and for the cross
    attentions only K/V exchanged while the rank slices the query side).

    Each modality is padded to its own multiple of world_size
    (pad_modality_for_uniform_sharding).  ``parts`` maps "video_self",
    "audio_self", "v2a" (video queries, audio keys) and "a2v" (audio queries,
    video keys) to dicts of float64 q, k, v (B, T, H, D) with the modality
    lengths of their roles; every part uses scale 1/sqrt(D).  Returns the four
    outputs, each (B, Tq, H, D) with the real query tokens.
    """
    tv_pad = padded_length(video_tokens, world_size)
    ta_pad = padded_length(audio_tokens, world_size)
    out = {}
    for name in ("video_self", "audio_self"):
        x = parts[name]
        d = x["q"].shape[-1]
        out[name] = ulysses_self_attention(x["q"], x["k"], x["v"], world_size, 1.0 / np.sqrt(d))
    for name, t_kv, t_kv_pad, t_q_pad in (("v2a", audio_tokens, ta_pad, tv_pad),
                                           ("a2v", video_tokens, tv_pad, ta_pad)):
        x = parts[name]
        d = x["q"].shape[-1]
        out[name] = ulysses_cross_attention(x["q"], x["k"], x["v"], world_size, 1.0 / np.sqrt(d),
                                            t_kv, t_kv_pad, t_q_pad=t_q_pad)
    return out


# ---------------------------------------------------------------------------
# the 2-D (height x width) split of the token grid
# ---------------------------------------------------------------------------

def get_optimal_split(n_ranks: int, height: int, width: int):
    """Rank grid (split_h, split_w) for ``n_ranks`` over a height x width
    token grid: [LC] "智能张量拆分策略" picks the split closest to a square.

    R17: among factor pairs split_h * split_w = n_ranks that divide the grid
    evenly (height % split_h == 0, width % split_w == 0), the pair closest to
    square (smallest |split_h - split_w|); between its two orientations the
    one whose tiles are closer to square (smallest |height/split_h -
    width/split_w|), then the smaller split_h.  No even split -> ValueError.
    """
    if n_ranks < 1:
        raise ValueError("n_ranks must be >= 1")
    best = None
    for a in range(1, n_ranks + 1):
        if n_ranks % a:
            continue
        b = n_ranks // a
        if height % a or width % b:
            continue
        key = (abs(a - b), abs(height // a - width // b), a)
        if best is None or key < best[0]:
            best = (key, (a, b))
    if best is None:
        raise ValueError(f"no even {n_ranks}-way split of a {height} x {width} grid")
    return best[1]


def split_cp_2d(x: np.ndarray, frames: int, height: int, width: int, split_h: int, split_w: int) -> np.ndarray:
    """Every rank's tile of the token grid ([LC] split_tensor_in_cp_2d).

    x: (B, T, ...) with T = frames*height*width tokens in raster order
    (token f*height*width + y*width + x_).  Rank r = i*split_w + j holds rows
    i*th..(i+1)*th-1 and columns j*tw..(j+1)*tw-1 of every frame (th =
    height/split_h, tw = width/split_w), its tokens in raster order within
    the tile.  Returns (split_h*split_w, B, frames*th*tw, ...).
    """
    b = x.shape[0]
    th, tw = height // split_h, width // split_w
    grid = x.reshape((b, frames, height, width) + x.shape[2:])
    out = []
    for i in range(split_h):
        for j in range(split_w):
            tile = grid[:, :, i * th:(i + 1) * th, j * tw:(j + 1) * tw]
            out.append(tile.reshape((b, frames * th * tw) + x.shape[2:]))
    return np.stack(out)


def gather_cp_2d(tiles: np.ndarray, frames: int, height: int, width: int, split_h: int, split_w: int) -> np.ndarray:
    """Inverse of ``split_cp_2d`` ([LC] gather_cp_2d): put every rank's tile
    back at its rows and columns; (N, B, frames*th*tw, ...) -> (B, T, ...)."""
    n, b = tiles.shape[:2]
    th, tw = height // split_h, width // split_w
    rest = tiles.shape[3:]
    grid = np.empty((b, frames, height, width) + rest, dtype=tiles.dtype)
    for i in range(split_h):
        for j in range(split_w):
            r = i * split_w + j
            grid[:, :, i * th:(i + 1) * th, j * tw:(j + 1) * tw] = tiles[r].reshape((b, frames, th, tw) + rest)
    return grid.reshape((b, frames * height * width) + rest)


def ulysses_self_attention_2d(q, k, v, frames: int, height: int, width: int, n_ranks: int, scale: float):
    """Self-attention with the 2-D split in place of the 1-D token split:
    split_cp_2d -> send_recv_heads (each rank gathers every token of its local
    heads, in rank-then-tile order) -> attention on the local heads ->
    gather_heads -> gather_cp_2d.  Attention needs no token order (no mask
    but the key-only one, and the grid needs no padding), so the result is
    unsharded attention; q, k, v: (B, T, H, D) float64."""
    split_h, split_w = get_optimal_split(n_ranks, height, width)
    qs, ks, vs = (split_cp_2d(a, frames, height, width, split_h, split_w) for a in (q, k, v))
    qh, kh, vh = (send_recv_heads(a) for a in (qs, ks, vs))
    oh = np.stack([attention_heads(qh[r], kh[r], vh[r], scale, None, None) for r in range(n_ranks)])
    return gather_cp_2d(gather_heads(oh), frames, height, width, split_h, split_w)


def reference_attention(q, k, v, scale: float, user_mask=None, kv_valid_len=None):
    """Unsharded attention on the unpadded problem, (B, T, H, D) in and out.

    [SP] "全局注意力没有变，只是分布方式变了" and [MG] Capabilities (SP row):
    the distributed path computes the same attention as one device would,
    differing only in the order of floating-point reductions.
    """
    return attention_heads(np.asarray(q, np.float64), np.asarray(k, np.float64),
                           np.asarray(v, np.float64), scale, kv_valid_len, user_mask)
