"""GPU parity of sp_masked_attention against the float64 CPU oracle.

Tolerance (max-abs vs the oracle on the same input bytes): 2e-2 for bf16 and
1e-4 for fp32.  Shapes span several query tiles (384 rows for bf16, 128 for
fp32) and 128-key tiles with ragged tails; masks exercise the empty / full / partial tile classes, the
key-only padding mask and rows with nothing visible."""

import math

import numpy as np
import pytest
import torch

import oracle as O
from sequence_attention_video_amd import binding as sp
from tests.gpu_util import f64, raw, rand_bits, say, sentinel_like, to_dev

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}
TD = {"f32": torch.float32, "bf16": torch.bfloat16}


def stacked(R, B, T, Hl, D):
    return (B * T * Hl * D, T * Hl * D, Hl * D, D)


def run_case(dtype, D, R, B, Tq, Tk, Hl, kv_valid, mask=None, seed=0, scale=None):
    rng = np.random.default_rng(seed)
    q = rand_bits(rng, (R, B, Tq, Hl, D), dtype)
    k = rand_bits(rng, (R, B, Tk, Hl, D), dtype)
    v = rand_bits(rng, (R, B, Tk, Hl, D), dtype)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    o = sentinel_like((R, B, Tq, Hl, D), TD[dtype])
    md = to_dev(mask) if mask is not None else None
    sp.sp_masked_attention(to_dev(q), to_dev(k), to_dev(v), o, R, B, Tq, Tk, Hl, D,
                           stacked(R, B, Tq, Hl, D), stacked(R, B, Tk, Hl, D), stacked(R, B, Tk, Hl, D),
                           stacked(R, B, Tq, Hl, D), kv_valid_len=kv_valid, mask=md, scale=scale)
    torch.cuda.synchronize()
    got = f64(raw(o))
    want = np.stack([O.attention_heads(f64(q[r]), f64(k[r]), f64(v[r]), scale, kv_valid, mask)
                     for r in range(R)])
    return got, want


CASES = [
    # dtype, D, R, B, Tq, Tk, Hl, kv_valid, mask kind
    ("bf16", 128, 2, 1, 300, 333, 2, 333, None),
    ("bf16", 128, 1, 1, 1000, 333, 2, 333, None),       # three query tiles, the last ragged
    ("bf16", 64, 1, 2, 800, 260, 2, 255, None),
    ("bf16", 128, 1, 2, 128, 64, 1, 64, None),          # exactly one tile each way
    ("bf16", 128, 2, 2, 257, 200, 3, 150, None),        # key-only padding inside a tile
    ("bf16", 64, 2, 1, 390, 1024, 4, 987, None),        # the cross workload's key padding
    ("bf16", 64, 1, 1, 77, 65, 2, 65, None),
    ("bf16", 64, 1, 1, 1000, 1024, 4, 987, None),       # few query tiles: 4-wave workgroups of 128 rows, ragged
    ("bf16", 64, 1, 1, 2048, 300, 32, 300, None),       # 256 query tiles of 256 rows: still 4-wave workgroups
    ("bf16", 64, 1, 1, 2049, 300, 29, 300, None),       # 261: 8-wave workgroups
    ("bf16", 128, 1, 1, 1, 1, 1, 1, None),              # one query, one key
    ("bf16", 64, 1, 1, 1, 300, 1, 299, None),           # one query against a padded key range
    ("bf16", 128, 1, 1, 300, 300, 2, 300, "random"),
    ("bf16", 128, 2, 2, 260, 260, 2, 258, "blocks"),    # empty/full/partial tiles + padding
    ("bf16", 64, 1, 3, 200, 190, 2, 190, "blocks_b"),   # per-batch masks
    ("bf16", 128, 1, 1, 1000, 700, 2, 690, "blocks"),   # class rows of three query tiles
    ("bf16", 64, 1, 2, 800, 400, 1, 400, "random"),
    ("bf16", 128, 1, 1, 777, 430, 2, 425, "random"),    # odd Tq, odd count of 64-key class tiles
    ("f32", 16, 4, 1, 52, 52, 2, 50, None),             # the tiny workload's rank share
    ("f32", 64, 1, 2, 200, 150, 2, 133, None),
    ("f32", 128, 1, 1, 140, 130, 2, 130, "random"),
    ("f32", 16, 2, 1, 52, 52, 2, 52, "blocks"),
]


def make_mask(kind, B, Tq, Tk, rng):
    if kind is None:
        return None
    if kind == "random":
        m = (rng.random((1, Tq, Tk)) < 0.5).astype(np.uint8)
        m[0, 5, :] = 0                                  # a row with nothing visible
        return m
    nb = B if kind == "blocks_b" else 1
    m = np.zeros((nb, Tq, Tk), np.uint8)
    for b in range(nb):
        for i in range(Tq):
            lim = (i // 64 + 1 + b) * 48                 # block-causal-like staircase
            m[b, i, :min(Tk, lim)] = 1
        m[b, :, Tk - 3:] = 1                             # a few keys visible to all
        m[b, 7, :] = 0                                   # a row with nothing visible
    return m


@pytest.mark.parametrize("dtype,D,R,B,Tq,Tk,Hl,kv,mask", CASES)
def test_attention_matches_oracle(dtype, D, R, B, Tq, Tk, Hl, kv, mask):
    say("attention", dtype, D, R, B, Tq, Tk, Hl, kv, mask)
    rng = np.random.default_rng(Tq * 31 + Tk)
    m = make_mask(mask, B, Tq, Tk, rng)
    got, want = run_case(dtype, D, R, B, Tq, Tk, Hl, kv, m, seed=Tq + D)
    assert np.isfinite(got).all()
    err = np.max(np.abs(got - want))
    assert err <= TOL[dtype], err


# Launches with too few query tiles to fill the GPU split every tile's key range
# over several workgroups and merge partial results; these shapes take that
# path on a 256-CU MI355X (the workspace size reports its partial records).
SPLIT_CASES = [
    # D, R, B, Tq, Tk, Hl, kv_valid, mask kind
    (128, 1, 1, 600, 2000, 2, 1990, None),       # 16 one-tile segments per query tile, key padding
    (128, 2, 1, 1280, 3000, 4, 2990, None),      # 4 tiles per workgroup, segments across query tiles
    (64, 1, 2, 700, 2500, 3, 2500, None),        # D = 64, two batches
    (128, 1, 1, 600, 2000, 2, 2000, "blocks"),   # staircase mask: empty, full and partial segments
    (128, 1, 2, 520, 1800, 2, 1800, "blocks_b"),  # per-batch masks
    (64, 1, 1, 300, 2100, 3, 2100, "random"),    # a row with no visible key stays 0
    (128, 1, 1, 599, 1990, 2, 1985, "blocks"),   # odd Tq and class-tile count
]


@pytest.mark.parametrize("D,R,B,Tq,Tk,Hl,kv,mask", SPLIT_CASES)
def test_attention_split_launch_matches_oracle(D, R, B, Tq, Tk, Hl, kv, mask):
    say("attention split", D, R, B, Tq, Tk, Hl, kv, mask)
    m = make_mask(mask, B, Tq, Tk, np.random.default_rng(Tq + Tk))
    mbs = 0 if m is None or m.shape[0] == 1 else Tq * Tk
    assert sp.sp_masked_attention_workspace_size(R, B, Tq, Tk, Hl, D, sp.SP_BF16, m is not None, mbs) > \
        (0 if m is None else sp.sp_masked_attention_workspace_size(8 * R, B, Tq, Tk, 32 * Hl, D, sp.SP_BF16, True,
                                                                   mbs))
    got, want = run_case("bf16", D, R, B, Tq, Tk, Hl, kv, m, seed=Tk + D)
    assert np.isfinite(got).all()
    err = np.max(np.abs(got - want))
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("D,Tq,Tk,Hl,mask", [
    (128, 1500, 3000, 4, None),       # four query tiles of 24 key tiles per head over 256 CUs
    (64, 700, 2500, 3, None),
    (128, 600, 2000, 2, "blocks"),
])
def test_attention_split_reused_workspace_and_replays(D, Tq, Tk, Hl, mask):
    """A split launch depends on nothing left in its workspace: with a
    workspace full of 0xFF bytes, two launches in a row and three replays of
    the launch recorded as a HIP graph (other writes to the workspace in
    between) all give the same bytes, within the oracle's tolerance.  The
    partial results are merged in a fixed order, so the bytes are the same on
    every run."""
    say("attention split reuse", D, Tq, Tk, Hl, mask)
    rng = np.random.default_rng(Tq + 7 * Tk)
    m = make_mask(mask, 1, Tq, Tk, rng)
    q, k, v = (rand_bits(rng, (1, 1, T, Hl, D), "bf16") for T in (Tq, Tk, Tk))
    need = sp.sp_masked_attention_workspace_size(1, 1, Tq, Tk, Hl, D, sp.SP_BF16, m is not None, 0)
    plain = 0 if m is None else sp.sp_masked_attention_workspace_size(8, 1, Tq, Tk, 32 * Hl, D, sp.SP_BF16, True, 0)
    assert need > plain                       # the launch splits
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    md = to_dev(m) if m is not None else None
    o = sentinel_like((1, 1, Tq, Hl, D), torch.bfloat16)
    st = lambda T: stacked(1, 1, T, Hl, D)
    call = lambda: sp.sp_masked_attention(qd, kd, vd, o, 1, 1, Tq, Tk, Hl, D, st(Tq), st(Tk), st(Tk), st(Tq),
                                          mask=md, workspace=ws)
    call()
    torch.cuda.synchronize()
    first = raw(o)
    want = O.attention_heads(f64(q[0]), f64(k[0]), f64(v[0]), 1 / math.sqrt(D), Tk, m)
    assert np.max(np.abs(f64(first) - want)) <= TOL["bf16"]
    o.view(torch.uint8).fill_(0xFF)
    call()
    torch.cuda.synchronize()
    assert np.array_equal(raw(o), first)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for i in range(3):
        o.view(torch.uint8).fill_(0xFF)
        ws[: need // 2].fill_(0xFF)           # eager work on the workspace between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(raw(o), first), i


@pytest.mark.parametrize("D,Tq,Tk,Hl,blank", [
    (128, 1000, 2000, 2, "tile"),     # query tile 1 (rows 384..767) sees no key: an item with no work
    (64, 700, 2500, 3, "tile"),
    (128, 1000, 2000, 2, "all"),      # nothing visible anywhere: no range has a unit
    (128, 600, 3000, 3, "ends"),      # only the first and the last key tiles visible
])
def test_attention_masked_split_uneven_work(D, Tq, Tk, Hl, blank):
    """Masked split launches over very uneven work: a query tile with no
    visible key, a mask with nothing visible, visible keys only at both ends.
    Every row is written once, rows that see nothing are 0."""
    say("attention masked split uneven", D, Tq, Tk, Hl, blank)
    rng = np.random.default_rng(Tq + Tk + Hl)
    m = (rng.random((1, Tq, Tk)) < 0.6).astype(np.uint8)
    BM = 384 if D == 128 else 256
    if blank == "tile":
        m[0, BM:2 * BM] = 0
    elif blank == "all":
        m[:] = 0
    else:
        m[0, :, 128:Tk - 128] = 0
    need = sp.sp_masked_attention_workspace_size(1, 1, Tq, Tk, Hl, D, sp.SP_BF16, True, 0)
    plain = sp.sp_masked_attention_workspace_size(8, 1, Tq, Tk, 32 * Hl, D, sp.SP_BF16, True, 0)
    assert need > plain                      # the launch splits
    got, want = run_case("bf16", D, 1, 1, Tq, Tk, Hl, Tk, m, seed=Tq + D)
    assert np.isfinite(got).all()
    assert np.max(np.abs(got - want)) <= TOL["bf16"]
    if blank == "all":
        assert not got.any()


@pytest.mark.parametrize("T,Hl,frame", [
    (3000, 6, 400),     # 48 items of 1..24 visible key tiles, about 3 units per range
    (1500, 16, 250),    # 64 items, ranges that start and end inside items' start units
    (6150, 4, 384),     # the uneven-mask share's shape: frames of 384 tokens, 6 prompt tokens
])
def test_attention_balanced_split_block_causal(T, Hl, frame):
    """Balanced split of a block-causal mask (frames see themselves and the
    earlier frames, the trailing prompt tokens see and are seen by all): the
    ranges count each item's non-empty key tiles plus the cost of a segment
    start, so they begin and end inside items, inside items' start units (a
    range that would end there stops at the item's first unit) and across
    several whole items.  Every row against the oracle."""
    say("attention balanced split block-causal", T, Hl, frame)
    n_prompt = 6 if T % frame else 0
    nv = T - n_prompt
    idx = np.arange(T)
    f = np.where(idx < nv, idx // frame, 1 << 20)
    m = ((f[None, :] <= f[:, None]) | (idx[None, :] >= nv) | (idx[:, None] >= nv)).astype(np.uint8)[None]
    need = sp.sp_masked_attention_workspace_size(1, 1, T, T, Hl, 128, sp.SP_BF16, True, 0)
    plain = sp.sp_masked_attention_workspace_size(8, 1, T, T, 32 * Hl, 128, sp.SP_BF16, True, 0)
    assert need > plain                      # the launch splits
    got, want = run_case("bf16", 128, 1, 1, T, T, Hl, T, m, seed=T + Hl)
    assert np.isfinite(got).all()
    assert np.max(np.abs(got - want)) <= TOL["bf16"]


@pytest.mark.parametrize("D,Tq,Tk,Hl,kv", [
    (128, 1000, 4000, 100, 3990),   # 300 query tiles of 32 key tiles: 256 run whole, 44 in ranges of 6 tiles
    (64, 600, 4000, 100, 4000),     # the same counts at D = 64 (two workgroups per CU)
])
def test_attention_split_ranges_spanning_items(D, Tq, Tk, Hl, kv):
    """More query tiles than CUs, unevenly: one whole round of items runs as
    in a plain launch, and the rest are cut into ranges that cover pieces of
    items (merged from records), some crossing from one item into the next.
    The oracle checks a sample of heads holding both kinds (head 85 holds
    query tile 255, the last whole one, and tiles 256, 257, the first in
    ranges); every other row is checked to be finite and written."""
    say("attention split spanning items", D, Tq, Tk, Hl, kv)
    ws = sp.sp_masked_attention_workspace_size(1, 1, Tq, Tk, Hl, D, sp.SP_BF16, False, 0)
    assert ws > 0
    rng = np.random.default_rng(Tq + Hl)
    q = rand_bits(rng, (1, 1, Tq, Hl, D), "bf16")
    k = rand_bits(rng, (1, 1, Tk, Hl, D), "bf16")
    v = rand_bits(rng, (1, 1, Tk, Hl, D), "bf16")
    o = sentinel_like((1, 1, Tq, Hl, D), torch.bfloat16)
    st = lambda T: stacked(1, 1, T, Hl, D)
    sp.sp_masked_attention(to_dev(q), to_dev(k), to_dev(v), o, 1, 1, Tq, Tk, Hl, D, st(Tq), st(Tk), st(Tk), st(Tq),
                           kv_valid_len=kv, workspace=torch.empty(ws, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    got = raw(o)
    assert np.isfinite(f64(got)).all()
    heads = [0, 1, 2, Hl // 2, 85, 86, Hl - 2, Hl - 1]
    want = O.attention_heads(f64(q[0][:, :, heads]), f64(k[0][:, :, heads]), f64(v[0][:, :, heads]),
                             1 / math.sqrt(D), kv)
    err = np.max(np.abs(f64(got[0][:, :, heads]) - want))
    assert err <= TOL["bf16"], err


def test_attention_single_visible_key_is_exact():
    """One visible key per row: p = 1 and the sum is 1, so o equals that V row
    bit for bit, also through bf16 MFMA."""
    say("attention one-key")
    rng = np.random.default_rng(3)
    R, B, T, Hl, D = 1, 1, 200, 2, 128
    pick = rng.integers(0, T, T)
    m = np.zeros((1, T, T), np.uint8)
    m[0, np.arange(T), pick] = 1
    q = rand_bits(rng, (R, B, T, Hl, D), "bf16")
    k = rand_bits(rng, (R, B, T, Hl, D), "bf16")
    v = rand_bits(rng, (R, B, T, Hl, D), "bf16")
    o = sentinel_like((R, B, T, Hl, D), torch.bfloat16)
    st = stacked(R, B, T, Hl, D)
    sp.sp_masked_attention(to_dev(q), to_dev(k), to_dev(v), o, R, B, T, T, Hl, D, st, st, st, st,
                           mask=to_dev(m))
    torch.cuda.synchronize()
    assert np.array_equal(raw(o)[0, 0], v[0, 0][pick])


def test_attention_degenerate_inputs():
    say("attention degenerate")
    R, B, T, Hl, D = 1, 1, 130, 2, 64
    rng = np.random.default_rng(4)
    q, k, v = (to_dev(rand_bits(rng, (R, B, T, Hl, D), "bf16")) for _ in range(3))
    st = stacked(R, B, T, Hl, D)
    # no visible key at all: every row is 0 (finite)
    o = sentinel_like((R, B, T, Hl, D), torch.bfloat16)
    sp.sp_masked_attention(q, k, v, o, R, B, T, T, Hl, D, st, st, st, st, kv_valid_len=0)
    torch.cuda.synchronize()
    assert not raw(o).any()
    # an all-zero user mask: every row is 0
    o = sentinel_like((R, B, T, Hl, D), torch.bfloat16)
    sp.sp_masked_attention(q, k, v, o, R, B, T, T, Hl, D, st, st, st, st,
                           mask=torch.zeros(1, T, T, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert not raw(o).any()
    # no keys at all (Tk = 0): every row is 0, in both kernels
    o = sentinel_like((R, B, T, Hl, D), torch.bfloat16)
    sp.sp_masked_attention(q, k, v, o, R, B, T, 0, Hl, D, st, st, st, st)
    of = sentinel_like((R, B, T, Hl, D), torch.float32)
    qf = q.float()
    sp.sp_masked_attention(qf, qf.clone(), qf.clone(), of, R, B, T, 0, Hl, D, st, st, st, st)
    torch.cuda.synchronize()
    assert not raw(o).any()
    assert not raw(of).any()
    # zero query rows / zero batches: nothing is written
    o = sentinel_like((R, B, T, Hl, D), torch.bfloat16)
    sp.sp_masked_attention(q, k, v, o, R, B, 0, T, Hl, D, st, st, st, st)
    sp.sp_masked_attention(q, k, v, o, R, 0, T, T, Hl, D, st, st, st, st)
    torch.cuda.synchronize()
    assert (raw(o) == 0xFFFF).all()


def test_attention_strided_query_heads():
    """Queries read through strides from an unexchanged (B, Tq, H, D) tensor,
    rank r using heads r*Hl..: the cross-attention layout."""
    say("attention strided q")
    rng = np.random.default_rng(5)
    W, B, Tq, Tk, H, D = 4, 1, 160, 96, 8, 64
    Hl = H // W
    q = rand_bits(rng, (B, Tq, H, D), "bf16")
    k = rand_bits(rng, (W, B, Tk, Hl, D), "bf16")
    v = rand_bits(rng, (W, B, Tk, Hl, D), "bf16")
    o = sentinel_like((W, B, Tq, Hl, D), torch.bfloat16)
    sp.sp_masked_attention(to_dev(q), to_dev(k), to_dev(v), o, W, B, Tq, Tk, Hl, D,
                           (Hl * D, Tq * H * D, H * D, D), stacked(W, B, Tk, Hl, D), stacked(W, B, Tk, Hl, D),
                           stacked(W, B, Tq, Hl, D), kv_valid_len=90)
    torch.cuda.synchronize()
    got = f64(raw(o))
    for r in range(W):
        want = O.attention_heads(f64(q[:, :, r * Hl:(r + 1) * Hl]), f64(k[r]), f64(v[r]), 1 / math.sqrt(D), 90)
        assert np.max(np.abs(got[r] - want)) <= 2e-2


def test_attention_large_scores_stay_finite():
    """Scores far apart (scale 4 on N(0,1) inputs): the running-max rescale path."""
    say("attention large scores")
    got, want = run_case("bf16", 128, 1, 1, 256, 512, 2, 512, None, seed=6, scale=0.35)
    assert np.isfinite(got).all()
    assert np.max(np.abs(got - want)) <= 2e-2


def test_attention_mask_at_widest_class_row():
    """A user mask over exactly 4096 64-key class tiles (the most the kernel's
    per-row class map holds) and a few query rows."""
    say("attention widest mask")
    R, B, Tq, Hl, D = 1, 1, 40, 1, 64
    Tk = 4096 * 64
    rng = np.random.default_rng(7)
    q = rand_bits(rng, (R, B, Tq, Hl, D), "bf16")
    k = rand_bits(rng, (R, B, Tk, Hl, D), "bf16")
    v = rand_bits(rng, (R, B, Tk, Hl, D), "bf16")
    m = np.zeros((1, Tq, Tk), np.uint8)
    m[0, :, -700:] = 1                                   # the last class tiles, partly
    m[0, :, :: 997] = 1                                  # sparse keys everywhere
    m[0, 3, :] = 0                                       # a row with nothing visible
    o = sentinel_like((R, B, Tq, Hl, D), torch.bfloat16)
    sp.sp_masked_attention(to_dev(q), to_dev(k), to_dev(v), o, R, B, Tq, Tk, Hl, D, stacked(R, B, Tq, Hl, D),
                           stacked(R, B, Tk, Hl, D), stacked(R, B, Tk, Hl, D), stacked(R, B, Tq, Hl, D),
                           mask=to_dev(m))
    torch.cuda.synchronize()
    got = f64(raw(o))
    want = O.attention_heads(f64(q[0]), f64(k[0]), f64(v[0]), 1 / math.sqrt(D), Tk, m)
    assert np.isfinite(got).all()
    assert np.max(np.abs(got[0] - want)) <= TOL["bf16"]


def test_attention_largest_key_token_stride():
    """K and V rows 8,000,000 elements apart (near the 32-bit byte offsets of
    one key tile), read through a ragged last tile."""
    say("attention largest stride")
    B, Tq, Tk, Hl, D = 1, 70, 3, 1, 128
    st_k = 8_000_000
    rng = np.random.default_rng(8)
    q = rand_bits(rng, (1, B, Tq, Hl, D), "bf16")
    kk = rand_bits(rng, (Tk, D), "bf16")
    vv = rand_bits(rng, (Tk, D), "bf16")
    kbuf = torch.zeros(Tk * st_k, dtype=torch.bfloat16, device="cuda")
    vbuf = torch.zeros(Tk * st_k, dtype=torch.bfloat16, device="cuda")
    kbuf.view(Tk, st_k)[:, :D] = to_dev(kk)
    vbuf.view(Tk, st_k)[:, :D] = to_dev(vv)
    o = sentinel_like((1, B, Tq, Hl, D), torch.bfloat16)
    sts = (Tk * st_k, Tk * st_k, st_k, D)
    sp.sp_masked_attention(to_dev(q), kbuf, vbuf, o, 1, B, Tq, Tk, Hl, D, stacked(1, B, Tq, Hl, D), sts, sts,
                           stacked(1, B, Tq, Hl, D))
    torch.cuda.synchronize()
    got = f64(raw(o))[0]
    want = O.attention_heads(f64(q[0]), f64(kk)[None, :, None, :], f64(vv)[None, :, None, :], 1 / math.sqrt(D), Tk)
    assert np.max(np.abs(got - want)) <= TOL["bf16"]


@pytest.mark.parametrize("D", [64, 128])
def test_attention_rising_scores_rescale_often(D):
    """Scores that rise along the keys (by up to 40 over 700 keys, in natural
    units, with noise) push the running max up part after part: the kernel's
    slow path (raise the max, rescale O and l, recompute the part) runs
    again and again, up to a key padding edge inside the last tile."""
    say("attention rising scores", D)
    rng = np.random.default_rng(11 + D)
    R, B, Tq, Tk, Hl = 1, 1, 200, 700, 2
    qf = np.zeros((R, B, Tq, Hl, D), np.float32)
    qf[..., 0] = 1.0
    qf[..., 1:] = 0.05 * rng.standard_normal((R, B, Tq, Hl, D - 1))
    kf = 0.05 * rng.standard_normal((R, B, Tk, Hl, D)).astype(np.float32)
    kf[..., 0] = (np.arange(Tk, dtype=np.float32) * (40.0 / Tk))[None, None, :, None]
    from sequence_attention_video_amd.workloads import f32_to_bf16_bits
    q, k = f32_to_bf16_bits(qf), f32_to_bf16_bits(kf)
    v = rand_bits(rng, (R, B, Tk, Hl, D), "bf16")
    st_q, st_k = stacked(R, B, Tq, Hl, D), stacked(R, B, Tk, Hl, D)
    o = sentinel_like((R, B, Tq, Hl, D), torch.bfloat16)
    sp.sp_masked_attention(to_dev(q), to_dev(k), to_dev(v), o, R, B, Tq, Tk, Hl, D, st_q, st_k, st_k, st_q,
                           kv_valid_len=690, scale=1.0)
    torch.cuda.synchronize()
    got = f64(raw(o))
    want = O.attention_heads(f64(q[0]), f64(k[0]), f64(v[0]), 1.0, 690)
    assert np.isfinite(got).all()
    assert np.max(np.abs(got[0] - want)) <= TOL["bf16"]
