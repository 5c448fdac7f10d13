"""Pin checks for the CPU oracle, written against an oracle-like namespace ``O``.

``tests/test_oracle_pins.py`` runs them on the real oracle; the mutation tests
run them on copies of the oracle with planted mistakes and expect a failure.
Nothing here calls the HIP path.
"""

import math

import numpy as np

from tests.conftest import load_golden


# ------------------------------------------------------------------ brute force

def brute_attention(q, k, v, scale, kv_valid_len, mask):
    """Pure-Python softmax attention of one head (lists of lists, math.exp)."""
    out = []
    for i, qi in enumerate(q):
        vis = [j for j in range(len(k))
               if j < kv_valid_len and (mask is None or mask[i][j])]
        if not vis:
            out.append([0.0] * len(v[0]))
            continue
        s = {j: scale * sum(a * b for a, b in zip(qi, k[j])) for j in vis}
        mx = max(s.values())
        w = {j: math.exp(s[j] - mx) for j in vis}
        den = sum(w.values())
        out.append([sum(w[j] * v[j][c] for j in vis) / den for c in range(len(v[0]))])
    return out


def brute_send_recv(x, w):
    """Element loop over the definition: out[r][b][s*Ts+t][j][d] = x[s][b][t][r*Hl+j][d]."""
    W, B, Ts, H, D = x.shape
    hl = H // w
    out = np.zeros((w, B, w * Ts, hl, D), dtype=x.dtype)
    writes = np.zeros(out.shape, dtype=np.int64)
    for r in range(w):
        for b in range(B):
            for tt in range(w * Ts):
                s, t = divmod(tt, Ts)
                for j in range(hl):
                    for d in range(D):
                        out[r, b, tt, j, d] = x[s, b, t, r * hl + j, d]
                        writes[r, b, tt, j, d] += 1
    assert (writes == 1).all()
    return out


# ------------------------------------------------------------------ partition / pad

def check_partition(O):
    g = load_golden("partition.txt")
    for case in g["cases"]:
        total, w = case[0], case[1]
        if case[2] == "ValueError":
            try:
                O.compute_sequence_partition(total, w)
            except ValueError:
                continue
            raise AssertionError(f"partition({total},{w}) must raise ValueError")
        offs, lens = O.compute_sequence_partition(total, w)
        assert list(offs) == case[2] and list(lens) == case[3], case
    for t, w, want in g["padded"]:
        assert O.padded_length(t, w) == want, (t, w)


def check_padded_length(O):
    for w in range(1, 9):
        for t in range(0, 40):
            p = O.padded_length(t, w)
            assert p % w == 0 and p >= t and p - t < w


def check_pad_tokens(O):
    g = load_golden("pad_mask_T3_P4.txt")
    x = np.array(g["tokens"])
    assert np.array_equal(O.pad_tokens(x, 4), np.array(g["tokens_padded"]))
    rng = np.random.default_rng(3)
    for dt in (np.uint16, np.float32):
        for (b, t, tp, c) in [(1, 5, 8, 3), (2, 7, 7, 4), (3, 1, 4, 2), (2, 0, 4, 2)]:
            raw = rng.integers(1, 2 ** 15, size=(b, t, c)).astype(dt)
            y = O.pad_tokens(raw, tp)
            assert y.shape == (b, tp, c) and y.dtype == raw.dtype
            assert y[:, :t].tobytes() == raw.tobytes()
            assert not y[:, t:].view(np.uint8).any()


def check_mask_extension(O):
    g = load_golden("pad_mask_T3_P4.txt")
    ext = O.extend_user_mask(np.array(g["user_mask"]), 4)
    assert ext.tolist() == g["extended"]
    assert O.key_padding_mask(3, 4).astype(int).tolist() == g["key_mask"]
    rng = np.random.default_rng(4)
    for (b, t, tp) in [(1, 6, 8), (2, 5, 5), (1, 1, 4)]:
        m = (rng.random((b, t, t)) < 0.5).astype(np.uint8)
        e = O.extend_user_mask(m, tp)
        assert e.shape == (b, tp, tp)
        assert np.array_equal(e[:, :t, :t], m)
        assert not e[:, :, t:].any()          # pad keys hidden from every row
        assert e[:, t:, :t].all()             # pad rows see every real key


# ------------------------------------------------------------------ head swap

def check_relayout_golden(O):
    g = load_golden("relayout_W2.txt")
    tok = np.array(g["token_side"], dtype=np.int64)
    head = np.array(g["head_side"], dtype=np.int64)
    assert np.array_equal(O.send_recv_heads(tok), head)
    assert np.array_equal(O.gather_heads(head), tok)


def check_relayout_brute_force(O):
    rng = np.random.default_rng(6)
    for (w, b, ts, h, d) in [(1, 1, 3, 2, 2), (2, 2, 3, 4, 2), (4, 1, 2, 8, 3), (3, 2, 2, 6, 1)]:
        x = rng.integers(0, 2 ** 16, size=(w, b, ts, h, d)).astype(np.uint16)
        want = brute_send_recv(x, w)
        got = O.send_recv_heads(x)
        assert np.array_equal(got, want)
        assert np.array_equal(O.gather_heads(want), x)


def check_relayout_round_trip(O):
    rng = np.random.default_rng(7)
    for (w, b, ts, h, d) in [(2, 1, 5, 4, 8), (4, 2, 3, 8, 16), (8, 1, 4, 32, 4), (1, 2, 6, 3, 5)]:
        for dt in (np.uint16, np.float32):
            x = rng.standard_normal((w, b, ts, h, d)).astype(np.float32)
            x = x.view(np.uint16).reshape(w, b, ts, h, 2 * d) if dt is np.uint16 else x
            y = O.gather_heads(O.send_recv_heads(x))
            assert y.dtype == x.dtype and y.tobytes() == x.tobytes()


def check_relayout_shapes(O):
    x = np.arange(2 * 1 * 3 * 4 * 5).reshape(2, 1, 3, 4, 5)
    y = O.send_recv_heads(x)
    assert y.shape == (2, 1, 6, 2, 5)          # tokens x W, heads // W
    assert O.gather_heads(y).shape == x.shape  # and back
    one = x[:1]
    assert np.array_equal(O.send_recv_heads(one)[0], one[0])   # W = 1 is the identity
    try:
        O.send_recv_heads(np.zeros((4, 1, 2, 6, 1)))           # H = 6 with W = 4
    except ValueError:
        return
    raise AssertionError("H not divisible by W must raise ValueError")


# ------------------------------------------------------------------ attention

def check_attention_golden(O):
    g = load_golden("attention_two_keys.txt")
    out = O.attention(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]), g["scale"],
                      g["kv_valid_len"], np.array(g["mask"]))
    assert np.max(np.abs(out - np.array(g["expected"]))) < g["tolerance"], out
    assert out[1].tolist() == g["expected"][1]          # one visible key: exact


def check_attention_brute_force(O):
    rng = np.random.default_rng(8)
    for (tq, tk, d, valid, use_mask) in [(5, 7, 3, 7, False), (6, 9, 4, 6, True),
                                         (4, 4, 2, 1, True), (7, 5, 3, 5, True)]:
        q = rng.standard_normal((tq, d))
        k = rng.standard_normal((tk, d))
        v = rng.standard_normal((tk, d + 1))
        m = (rng.random((tq, tk)) < 0.6).astype(np.uint8) if use_mask else None
        if m is not None:
            m[0] = 0                      # one row with nothing visible
        scale = 0.37
        got = O.attention(q, k, v, scale, valid, m)
        want = brute_attention(q.tolist(), k.tolist(), v.tolist(), scale, valid,
                               None if m is None else m.tolist())
        assert np.max(np.abs(got - np.array(want))) < 1e-12


def check_attention_sdpa(O):
    import torch
    import torch.nn.functional as F
    g = torch.Generator().manual_seed(9)
    for (b, h, tq, tk, d, use_mask) in [(1, 2, 9, 13, 8, False), (2, 3, 16, 11, 16, True)]:
        q = torch.randn(b, h, tq, d, generator=g, dtype=torch.float64)
        k = torch.randn(b, h, tk, d, generator=g, dtype=torch.float64)
        v = torch.randn(b, h, tk, d, generator=g, dtype=torch.float64)
        mask = None
        if use_mask:
            mask = torch.rand(b, 1, tq, tk, generator=g) < 0.7
            mask[..., 0] = True           # SDPA returns NaN on rows with nothing visible
        ref = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=1.0 / math.sqrt(d))
        qn, kn, vn = (t.permute(0, 2, 1, 3).numpy() for t in (q, k, v))
        mn = None if mask is None else mask[:, 0].numpy().astype(np.uint8)
        got = O.attention_heads(qn, kn, vn, 1.0 / math.sqrt(d), None, mn)
        assert np.max(np.abs(got - ref.permute(0, 2, 1, 3).numpy())) < 1e-12


def check_attention_closed_forms(O):
    rng = np.random.default_rng(10)
    tq, tk, d = 6, 9, 5
    q = rng.standard_normal((tq, d))
    v = rng.standard_normal((tk, d))
    m = (rng.random((tq, tk)) < 0.5).astype(np.uint8)
    m[:, 0] = 1
    # (i) all keys equal: uniform weights, o = mean of the visible V rows
    k_same = np.tile(rng.standard_normal((1, d)), (tk, 1))
    got = O.attention(q, k_same, v, 0.8, tk, m)
    want = np.stack([v[m[i] != 0].mean(axis=0) for i in range(tq)])
    assert np.max(np.abs(got - want)) < 1e-12
    # (ii) exactly one visible key per row: o = that V row, exactly
    k = rng.standard_normal((tk, d))
    one = np.zeros((tq, tk), np.uint8)
    pick = rng.integers(0, tk, tq)
    one[np.arange(tq), pick] = 1
    got = O.attention(q, k, v, 0.8, tk, one)
    assert np.array_equal(got, v[pick])
    # (iii) constant V: o = that constant wherever a key is visible
    got = O.attention(q, k, np.full((tk, d), 2.5), 0.8, tk, m)
    assert np.max(np.abs(got - 2.5)) < 1e-14
    # (iv) two visible keys: weight of key a is the logistic of the score gap
    two = np.zeros((tq, tk), np.uint8)
    two[:, 1] = two[:, 4] = 1
    got = O.attention(q, k, v, 0.8, tk, two)
    s1, s4 = 0.8 * (q @ k[1]), 0.8 * (q @ k[4])
    wa = 1.0 / (1.0 + np.exp(s4 - s1))
    want = wa[:, None] * v[1] + (1 - wa)[:, None] * v[4]
    assert np.max(np.abs(got - want)) < 1e-12


def check_garbage_pad_invariance(O):
    rng = np.random.default_rng(12)
    tq, tk, valid, d = 7, 12, 9, 4
    q, k, v = rng.standard_normal((tq, d)), rng.standard_normal((tk, d)), rng.standard_normal((tk, d))
    base = O.attention(q, k, v, 0.5, valid)
    k2, v2 = k.copy(), v.copy()
    k2[valid:] = 1e4 * np.sign(rng.standard_normal((tk - valid, d)))
    v2[valid:] = -1e4
    assert np.array_equal(O.attention(q, k2, v2, 0.5, valid), base)
    # and a key mask that hides nothing past ``valid`` equals the truncated problem
    trunc = O.attention(q, k[:valid], v[:valid], 0.5, valid)
    assert np.max(np.abs(trunc - base)) < 1e-15


# ------------------------------------------------------------------ restore

def check_gather_output(O):
    g = load_golden("gather_output_W2.txt")
    pieces = [np.array(p) for p in g["pieces"]]
    out = O.gather_output_tokens(pieces, g["counts"], g["t_valid"])
    assert out.tolist() == g["expected"]
    pieces = [np.array(p) for p in g["pieces_uniform"]]
    out = O.gather_output_tokens(pieces, g["counts_uniform"], g["t_valid_uniform"])
    assert out.tolist() == g["expected_uniform"]
    pieces = [np.array(p) for p in g["pieces_trim"]]
    out = O.gather_output_tokens(pieces, g["counts_trim"], g["t_valid_trim"])
    assert out.tolist() == g["expected_trim"]


# ------------------------------------------------------------------ whole path

def check_sharded_equals_unsharded_self(O):
    rng = np.random.default_rng(13)
    for (b, t, h, d, w) in [(1, 10, 4, 4, 4), (2, 13, 6, 3, 3), (1, 16, 8, 2, 8), (2, 7, 2, 5, 1)]:
        q, k, v = (rng.standard_normal((b, t, h, d)) for _ in range(3))
        sharded = O.ulysses_self_attention(q, k, v, w, 0.6)
        ref = O.reference_attention(q, k, v, 0.6)
        assert sharded.shape == ref.shape == (b, t, h, d)
        assert np.max(np.abs(sharded - ref)) < 1e-12


def check_sharded_equals_unsharded_mask(O):
    rng = np.random.default_rng(14)
    for (b, t, h, d, w) in [(1, 10, 4, 4, 4), (2, 11, 6, 3, 3)]:
        q, k, v = (rng.standard_normal((b, t, h, d)) for _ in range(3))
        m = (rng.random((b, t, t)) < 0.5).astype(np.uint8)
        sharded = O.ulysses_self_attention(q, k, v, w, 0.6, user_mask=m)
        ref = O.reference_attention(q, k, v, 0.6, user_mask=m)
        assert np.max(np.abs(sharded - ref)) < 1e-12


def check_sharded_equals_unsharded_cross(O):
    rng = np.random.default_rng(15)
    for (b, tq, tkv, tkv_pad, h, d, w) in [(1, 16, 9, 12, 8, 4, 4), (2, 6, 5, 6, 6, 3, 3)]:
        q = rng.standard_normal((b, tq, h, d))
        k, v = rng.standard_normal((b, tkv, h, d)), rng.standard_normal((b, tkv, h, d))
        sharded = O.ulysses_cross_attention(q, k, v, w, 0.45, tkv, tkv_pad)
        ref = O.reference_attention(q, k, v, 0.45)
        assert np.max(np.abs(sharded - ref)) < 1e-12


def check_cross_query_padding(O):
    """A query sequence that is not a multiple of W is padded to its own
    multiple ([SP] 补齐, per modality) and unpadded at the end (还原): the
    sharded result equals unsharded attention on the real queries; without
    the padding the partition raises (切分)."""
    rng = np.random.default_rng(16)
    for (b, tq, tkv, tkv_pad, h, d, w) in [(1, 13, 9, 12, 8, 4, 4), (2, 7, 6, 6, 6, 3, 3)]:
        q = rng.standard_normal((b, tq, h, d))
        k, v = rng.standard_normal((b, tkv, h, d)), rng.standard_normal((b, tkv, h, d))
        tq_pad = O.padded_length(tq, w)
        sharded = O.ulysses_cross_attention(q, k, v, w, 0.45, tkv, tkv_pad, t_q_pad=tq_pad)
        assert sharded.shape == q.shape
        assert np.max(np.abs(sharded - O.reference_attention(q, k, v, 0.45))) < 1e-12
        try:
            O.ulysses_cross_attention(q, k, v, w, 0.45, tkv, tkv_pad)
        except ValueError:
            pass
        else:
            raise AssertionError("an unpadded query length that W does not divide must raise")


def check_joint_av_block(O):
    """The joint audio-video block: each modality padded to its own multiple
    of W; all four attentions equal unsharded attention on the real tokens."""
    rng = np.random.default_rng(17)
    w, b, h, tv, ta = 4, 1, 8, 22, 7
    shapes = {"video_self": (tv, tv, 8), "audio_self": (ta, ta, 4), "v2a": (tv, ta, 4), "a2v": (ta, tv, 4)}
    parts = {}
    for name, (tq, tk, d) in shapes.items():
        parts[name] = dict(q=rng.standard_normal((b, tq, h, d)), k=rng.standard_normal((b, tk, h, d)),
                           v=rng.standard_normal((b, tk, h, d)))
    out = O.joint_av_block(parts, w, tv, ta)
    for name, x in parts.items():
        ref = O.reference_attention(x["q"], x["k"], x["v"], 1.0 / np.sqrt(x["q"].shape[-1]))
        assert out[name].shape == x["q"].shape, name
        assert np.max(np.abs(out[name] - ref)) < 1e-12, name


def check_split_2d_golden(O):
    """The hand-worked 2-D split ([LC] 智能张量拆分策略)."""
    from tests.conftest import load_golden
    g = load_golden("split_2d_F2_H2_W4_N4.txt")
    sh, sw = O.get_optimal_split(g["n_ranks"], g["height"], g["width"])
    assert [sh, sw] == g["split"]
    t = g["frames"] * g["height"] * g["width"]
    x = np.arange(t, dtype=np.int64).reshape(1, t)
    tiles = O.split_cp_2d(x, g["frames"], g["height"], g["width"], sh, sw)
    assert tiles.tolist() == g["tiles"]
    assert O.gather_cp_2d(tiles, g["frames"], g["height"], g["width"], sh, sw).tolist() == x.tolist()


def check_optimal_split(O):
    """Closed forms of the near-square choice (R17), and its error."""
    assert O.get_optimal_split(8, 16, 24) == (2, 4)      # 8 x 6 tiles beat 4 x 12
    assert O.get_optimal_split(8, 64, 64) == (2, 4)      # tie of orientations -> smaller split_h
    assert O.get_optimal_split(1, 5, 7) == (1, 1)
    assert O.get_optimal_split(7, 7, 5) == (7, 1)        # a prime: the only even split
    assert O.get_optimal_split(6, 6, 4) == (3, 2)        # 2 x 3 does not divide the width
    assert O.get_optimal_split(16, 32, 32) == (4, 4)
    for args in [(8, 3, 5), (0, 4, 4)]:
        try:
            O.get_optimal_split(*args)
        except ValueError:
            pass
        else:
            raise AssertionError(f"get_optimal_split{args} must raise")


def check_split_2d_brute_force(O):
    """Element loops in pure Python == split_cp_2d; every token lands exactly
    once; gather_cp_2d returns the input byte for byte."""
    rng = np.random.default_rng(18)
    for (b, f, hh, ww, n, c) in [(1, 2, 4, 6, 6, 3), (2, 3, 6, 4, 4, 2), (1, 1, 8, 8, 8, 1)]:
        sh, sw = O.get_optimal_split(n, hh, ww)
        th, tw = hh // sh, ww // sw
        x = rng.integers(0, 1 << 30, size=(b, f * hh * ww, c)).astype(np.int64)
        tiles = O.split_cp_2d(x, f, hh, ww, sh, sw)
        seen = np.zeros(f * hh * ww, dtype=np.int64)
        for r in range(n):
            i, j = divmod(r, sw)
            for bb in range(b):
                lt = 0
                for ff in range(f):
                    for y in range(th):
                        for xx in range(tw):
                            t = ff * hh * ww + (i * th + y) * ww + (j * tw + xx)
                            assert (tiles[r, bb, lt] == x[bb, t]).all()
                            if bb == 0:
                                seen[t] += 1
                            lt += 1
        assert (seen == 1).all()
        back = O.gather_cp_2d(tiles, f, hh, ww, sh, sw)
        assert back.tobytes() == x.tobytes()


def check_sharded_equals_unsharded_2d(O):
    """2-D split, exchange, attention, exchange back, gather: unsharded attention."""
    rng = np.random.default_rng(19)
    for (b, f, hh, ww, n, h, d) in [(1, 2, 4, 6, 8, 8, 4), (2, 1, 6, 6, 4, 4, 3)]:
        t = f * hh * ww
        q, k, v = (rng.standard_normal((b, t, h, d)) for _ in range(3))
        got = O.ulysses_self_attention_2d(q, k, v, f, hh, ww, n, 0.4)
        assert np.max(np.abs(got - O.reference_attention(q, k, v, 0.4))) < 1e-12
