"""Seeded sweep of random shapes through sp_masked_attention against the
float64 oracle (max-abs 2e-2 for bf16, 1e-4 for fp32): R = 1..3 rank shares,
B = 1..2, Hl = 1..3, D in the supported set (bf16 D = 16 in cases of its own), ragged Tq and Tk, key-only
padding anywhere in the last tiles, and random, staircase and per-batch user
masks (with rows that see nothing).  Launches with few query tiles split their
key range (the workspace size says which), so both kernel forms are covered.
Every output row must be written and finite."""

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
N_CASES = 30


def case(i):
    rng = np.random.default_rng(9000 + i)
    dtype = "bf16" if rng.random() < 0.75 else "f32"
    D = int(rng.choice([64, 128])) if dtype == "bf16" else int(rng.choice([16, 64, 128]))
    R, B, Hl = int(rng.integers(1, 4)), int(rng.integers(1, 3)), int(rng.integers(1, 4))
    Tq, Tk = int(rng.integers(1, 700)), int(rng.integers(1, 900))
    kv = int(rng.integers(max(0, Tk - 140), Tk + 1))
    kind = rng.choice(["none", "none", "random", "stairs", "stairs_b"])
    return rng, dtype, D, R, B, Hl, Tq, Tk, kv, str(kind)


def make_mask(kind, B, Tq, Tk, rng):
    if kind == "none":
        return None
    nb = B if kind == "stairs_b" else 1
    if kind == "random":
        m = (rng.random((nb, Tq, Tk)) < rng.uniform(0.05, 0.95)).astype(np.uint8)
    else:
        m = np.zeros((nb, Tq, Tk), np.uint8)
        step = int(rng.integers(16, 200))
        for b in range(nb):
            for q in range(Tq):
                m[b, q, :min(Tk, (q // step + 1 + b) * step)] = 1
    m[:, rng.integers(0, Tq, 2), :] = 0                       # rows with nothing visible
    return m


@pytest.mark.parametrize("i", range(N_CASES))
def test_attention_random_shapes(i):
    rng, dtype, D, R, B, Hl, Tq, Tk, kv, kind = case(i)
    m = make_mask(kind, B, Tq, Tk, rng)
    mbs = 0 if m is None or m.shape[0] == 1 else Tq * Tk
    ws = sp.sp_masked_attention_workspace_size(R, B, Tq, Tk, Hl, D, sp.SP_BF16 if dtype == "bf16" else sp.SP_F32,
                                               m is not None, mbs)
    say("attention shapes", i, dtype, D, R, B, Hl, Tq, Tk, kv, kind, "workspace", ws)
    q = rand_bits(rng, (R, B, Tq, Hl, D), dtype)
    k = rand_bits(rng, (R, B, Tk, Hl, D), dtype)
    v = rand_bits(rng, (R, B, Tk, Hl, D), dtype)
    o = sentinel_like((R, B, Tq, Hl, D), TD[dtype])
    st = lambda T: (B * T * Hl * D, T * Hl * D, Hl * D, D)
    scale = 1.0 / math.sqrt(D)
    sp.sp_masked_attention(to_dev(q), to_dev(k), to_dev(v), o, R, B, Tq, Tk, Hl, D, st(Tq), st(Tk), st(Tk), st(Tq),
                           kv_valid_len=kv, mask=to_dev(m) if m is not None else None, scale=scale)
    torch.cuda.synchronize()
    got = f64(raw(o))
    assert np.isfinite(got).all()
    want = np.stack([O.attention_heads(f64(q[r]), f64(k[r]), f64(v[r]), scale, kv, m) for r in range(R)])
    err = float(np.max(np.abs(got - want)))
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("i", range(10))
def test_attention_bf16_d16_random_shapes(i):
    """bf16 at D = 16 (values widened exactly to float32, float32 MFMA, output
    rounded to bf16): random shapes, masks and key padding against the oracle."""
    rng = np.random.default_rng(9500 + i)
    D, dtype = 16, "bf16"
    R, B, Hl = int(rng.integers(1, 4)), int(rng.integers(1, 3)), int(rng.integers(1, 4))
    Tq, Tk = int(rng.integers(1, 700)), int(rng.integers(1, 900))
    kv = int(rng.integers(max(0, Tk - 140), Tk + 1))
    kind = str(rng.choice(["none", "random", "stairs", "stairs_b"]))
    m = make_mask(kind, B, Tq, Tk, rng)
    say("attention bf16 D16", i, R, B, Hl, Tq, Tk, kv, kind)
    q = rand_bits(rng, (R, B, Tq, Hl, D), dtype)
    k = rand_bits(rng, (R, B, Tk, Hl, D), dtype)
    v = rand_bits(rng, (R, B, Tk, Hl, D), dtype)
    o = sentinel_like((R, B, Tq, Hl, D), TD[dtype])
    st = lambda T: (B * T * Hl * D, T * Hl * D, Hl * D, D)
    scale = 1.0 / math.sqrt(D)
    sp.sp_masked_attention(to_dev(q), to_dev(k), to_dev(v), o, R, B, Tq, Tk, Hl, D, st(Tq), st(Tk), st(Tk), st(Tq),
                           kv_valid_len=kv, mask=to_dev(m) if m is not None else None, scale=scale)
    torch.cuda.synchronize()
    got = f64(raw(o))
    assert np.isfinite(got).all()
    want = np.stack([O.attention_heads(f64(q[r]), f64(k[r]), f64(v[r]), scale, kv, m) for r in range(R)])
    err = float(np.max(np.abs(got - want)))
    assert err <= TOL[dtype], err
