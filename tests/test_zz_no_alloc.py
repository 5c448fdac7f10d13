"""sp_masked_attention_noalloc, the attention entry point that allocates
nothing (its workspace is the library's fixed per-GPU scratch), against
sp_masked_attention with a workspace from the size query: two calls in a row
through the C ABI, the second smaller, each compared byte for byte with the
existing entry point and within the tolerance of the float64 oracle.

First call: one rank's share of the 6144-token video workload (R = 1, bf16,
D = 128): a split launch whose partial records sit in the scratch.  Second
call: a smaller masked problem (R = 2, 1000 tokens, D = 64, random user mask
with an empty row): mask classes and visibility words in the scratch, over
what the first call left there.  Third: an fp32 call that needs no workspace.
A request beyond the scratch is refused before anything is launched.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
from sequence_attention_video_amd import binding as sp
from tests.gpu_util import f64, rand_bits, raw, say, sentinel_like, to_dev

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}
TD = {"f32": torch.float32, "bf16": torch.bfloat16}


def both_entry_points(R, B, Tq, Tk, Hl, D, dtype, kv, m, seed):
    rng = np.random.default_rng(seed)
    q = rand_bits(rng, (R, B, Tq, Hl, D), dtype)
    k = rand_bits(rng, (R, B, Tk, Hl, D), dtype)
    v = rand_bits(rng, (R, B, Tk, Hl, D), dtype)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    md = to_dev(m) if m is not None else None
    st = lambda T: (B * T * Hl * D, T * Hl * D, Hl * D, D)
    scale = 1.0 / math.sqrt(D)
    ref = sentinel_like((R, B, Tq, Hl, D), TD[dtype])
    got = sentinel_like((R, B, Tq, Hl, D), TD[dtype])
    mbs = 0 if m is None or m.shape[0] == 1 else Tq * Tk
    need = sp.sp_masked_attention_workspace_size(R, B, Tq, Tk, Hl, D, sp._dtype_code(qd), m is not None, mbs)
    say("no-alloc", R, B, Tq, Tk, Hl, D, dtype, "mask", m is not None, "workspace bytes", need)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
    sp.sp_masked_attention(qd, kd, vd, ref, R, B, Tq, Tk, Hl, D, st(Tq), st(Tk), st(Tk), st(Tq), kv_valid_len=kv,
                           mask=md, scale=scale, workspace=ws)
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    sp.sp_masked_attention_noalloc(qd, kd, vd, got, R, B, Tq, Tk, Hl, D, st(Tq), st(Tk), st(Tk), st(Tq),
                                   kv_valid_len=kv, mask=md, scale=scale)
    torch.cuda.synchronize()
    assert torch.cuda.memory_stats().get("allocation.all.allocated", 0) == before
    g, r_ = f64(raw(got)), f64(raw(ref))
    assert np.isfinite(g).all()
    assert float(np.max(np.abs(g - r_))) <= TOL[dtype]
    assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8))
    want = np.stack([O.attention_heads(f64(q[i]), f64(k[i]), f64(v[i]), scale, kv, m) for i in range(R)])
    err = float(np.max(np.abs(g - want)))
    assert err <= TOL[dtype], err
    return need


def test_noalloc_matches_workspace_entry_point_twice():
    # 1: one share of the video workload, split over the GPU (records in the scratch)
    need1 = both_entry_points(1, 1, 6144, 6144, 4, 128, "bf16", 6144, None, 11)
    # 2: smaller, with a user mask (classes and words in the scratch, after call 1)
    rng = np.random.default_rng(12)
    m = (rng.random((1, 1000, 1000)) < 0.4).astype(np.uint8)
    m[0, 3] = 0
    need2 = both_entry_points(2, 1, 1000, 1000, 2, 64, "bf16", 1000, m, 13)
    assert 0 < need2 < need1
    # 3: no workspace needed at all
    assert both_entry_points(1, 1, 50, 52, 2, 16, "f32", 50, None, 14) == 0


def test_noalloc_refuses_requests_beyond_the_scratch():
    """A user mask over 40000 x 40000 tokens needs 40000 x 625 visibility words
    (200 MB) > the 128 MiB scratch: refused before any launch (the mask
    buffer here is 16 bytes and is never read)."""
    import ctypes
    T, Hl, D = 40000, 1, 128
    need = sp.sp_masked_attention_workspace_size(1, 1, T, T, Hl, D, sp.SP_BF16, True, 0)
    assert need > sp.SP_NOALLOC_SCRATCH_BYTES
    x = torch.empty(4, T, Hl, D, dtype=torch.bfloat16, device="cuda")
    mk = torch.empty(16, dtype=torch.uint8, device="cuda")
    st = sp.AttnStrides(0, 0, Hl * D, D)
    q_, k_, v_, o_ = (ctypes.c_void_p(x[i].data_ptr()) for i in range(4))
    status = sp.load().sp_masked_attention_noalloc(q_, st, k_, st, v_, st, o_, st, 1, 1, T, T, Hl, D, sp.SP_BF16, T,
                                                   ctypes.c_void_p(mk.data_ptr()), 0, 1.0 / math.sqrt(D), None)
    assert status == sp.SP_ERR_SCRATCH
    with pytest.raises(ValueError):
        sp.check(status)
