"""The five workloads at full size, in the launch configuration bench.py times
(sequence_attention_video_amd.pipeline.UlyssesStep, all W virtual ranks per
launch), checked stage by stage against the CPU oracle:

* pad, mask extension, both relayouts and gather/unpad: bit-exact, in full;
* attention: the tiny workload in full; the large ones on sampled query rows
  of every (rank, head) -- first and last rows, shard boundaries, the last
  real row and pad rows -- within 2e-2 of the float64 oracle;
* the final output: sampled (token, head) rows against unsharded attention on
  the unpadded problem (the sharded == unsharded invariant).
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
from sequence_attention_video_amd.pipeline import UlyssesStep
from sequence_attention_video_amd.workloads import ORDER, WORKLOADS, make_inputs
from tests.gpu_util import f64, raw, say, to_dev

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}


def sample_rows(n_rows, shard, valid, rng, extra=8):
    rows = {0, 1, n_rows - 1, valid - 1, min(valid, n_rows - 1)}
    for s in range(1, n_rows // shard):
        if s % 3 == 0:
            rows.update({s * shard - 1, s * shard})
    rows.update(int(x) for x in rng.integers(0, n_rows, extra))
    return np.array(sorted(r for r in rows if 0 <= r < n_rows))


@pytest.mark.parametrize("name", ORDER)
def test_workload_stages(name):
    wl = WORKLOADS[name]
    say("workload", name)
    x = make_inputs(wl)
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    mask = to_dev(x["mask"]) if x["mask"] is not None else None
    step = UlyssesStep(wl, q, k, v, mask)
    say("workload run", name)
    out = step.run()
    torch.cuda.synchronize()
    say("workload check", name)
    W, B, H, D, Hl = wl.W, wl.B, wl.H, wl.D, wl.Hl
    T, Tp = wl.T, wl.T_pad
    scale = 1.0 / math.sqrt(D)
    rng = np.random.default_rng(wl.index)

    # -- pad (bit-exact)
    names = ["k", "v"] if wl.cross else ["q", "k", "v"]
    padded = {n: O.pad_tokens(x[n], Tp) for n in names}
    if step.need_pad:
        for n in names:
            assert raw(getattr(step, n + "p")).tobytes() == padded[n].tobytes(), n
    mask_ext = None
    if x["mask"] is not None:
        mask_ext = O.extend_user_mask(x["mask"], Tp)
        assert np.array_equal(raw(step.mask_ext), mask_ext)
    # -- partition (host)
    offs, lens = step.partition()
    assert (offs, lens) == tuple(map(list, O.compute_sequence_partition(Tp, W)))
    # -- send_recv_heads (bit-exact)
    heads = {n: O.send_recv_heads(O.token_shards(padded[n], W)) for n in names}
    for n in names:
        assert raw(getattr(step, n + "h")).tobytes() == heads[n].tobytes(), n
    # -- attention, per rank share
    oh = raw(step.oh)
    ohf = f64(oh)
    assert np.isfinite(ohf).all()
    Tq = wl.Tq if wl.cross else Tp
    kv_valid = T if mask_ext is None else Tp
    worst = 0.0
    for r in range(W):
        kr, vr = f64(heads["k"][r]), f64(heads["v"][r])
        if wl.cross:
            qr = f64(x["q"][:, :, r * Hl:(r + 1) * Hl])
        else:
            qr = f64(heads["q"][r])
        if name == "tiny":
            rows = None
            want = O.attention_heads(qr, kr, vr, scale, kv_valid, mask_ext)
            got = ohf[r]
        else:
            rows = sample_rows(Tq, Tq // W, T if not wl.cross else Tq, rng)
            want = O.attention_heads(qr, kr, vr, scale, kv_valid, mask_ext, rows=rows)[:, rows]
            got = ohf[r][:, rows]
        worst = max(worst, float(np.max(np.abs(got - want))))
    assert worst <= TOL[wl.dtype], worst
    # -- gather_heads on the GPU's own attention output (bit-exact)
    ot = raw(step.ot)
    assert ot.tobytes() == O.gather_heads(oh).tobytes()
    # -- gather_output_tokens (bit-exact)
    Tsq = Tq // W
    pieces = [ot[r].reshape(B, Tsq, H * D) for r in range(W)]
    Tout = wl.Tq if wl.cross else T
    want_out = O.gather_output_tokens(pieces, [Tsq] * W, Tout)
    got_out = raw(out)
    assert got_out.reshape(B, Tout, H * D).tobytes() == want_out.tobytes()
    # -- end to end: sharded == unsharded on sampled (token, head) rows
    rows = sample_rows(Tout, max(1, Tout // W), Tout, rng, extra=6)
    outf = f64(got_out).reshape(B, Tout, H, D)
    qf = f64(x["q"])
    kf, vf = f64(x["k"]), f64(x["v"])
    heads_to_check = range(H) if H <= 8 else list(range(0, H, 5)) + [H - 1]
    for hh in heads_to_check:
        ref = O.attention_heads(qf[:, :, hh:hh + 1], kf[:, :, hh:hh + 1], vf[:, :, hh:hh + 1], scale,
                                None if x["mask"] is None else T, x["mask"], rows=rows)
        err = np.max(np.abs(outf[:, rows, hh] - ref[:, rows, 0]))
        assert err <= TOL[wl.dtype], (hh, err)


@pytest.mark.parametrize("name", ORDER)
def test_workload_zero_copy_matches_exchange_path(name):
    """Both exchanges folded into attention's addressing (strided views of the
    padded token-side tensors, output written in token layout): the same
    arithmetic in the same order as the exchange path, so the same bytes."""
    wl = WORKLOADS[name]
    say("zero-copy", name)
    x = make_inputs(wl)
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    mask = to_dev(x["mask"]) if x["mask"] is not None else None
    step = UlyssesStep(wl, q, k, v, mask)
    out = step.run().clone()
    outz = step.run_zero_copy()
    torch.cuda.synchronize()
    assert torch.equal(outz.view(torch.uint8), out.view(torch.uint8))
    # the token-layout attention output is the exchange path's gather_heads result
    Tq = wl.Tq if wl.cross else wl.T_pad
    ot = step.ot.view(wl.W, wl.B, Tq // wl.W, wl.H, wl.D).permute(1, 0, 2, 3, 4).reshape(wl.B, Tq, wl.H, wl.D)
    assert torch.equal(step.oz.view(torch.uint8), ot.contiguous().view(torch.uint8))


@pytest.mark.parametrize("name", [n for n in ORDER if n != "tiny"])
def test_workload_rank_share(name):
    """One rank's share alone (R = 1), the launch each GPU runs when the ranks
    are devices and the one bench.py times as the share: split over the GPU
    where the share has too few query tiles.  Ranks 0 and W-1 on sampled rows
    against the oracle."""
    wl = WORKLOADS[name]
    say("rank share", name)
    x = make_inputs(wl)
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    mask = to_dev(x["mask"]) if x["mask"] is not None else None
    step = UlyssesStep(wl, q, k, v, mask)
    step.run()
    W, Hl, D, T, Tp = wl.W, wl.Hl, wl.D, wl.T, wl.T_pad
    scale = 1.0 / math.sqrt(D)
    rng = np.random.default_rng(100 + wl.index)
    names = ["k", "v"] if wl.cross else ["q", "k", "v"]
    padded = {n: O.pad_tokens(x[n], Tp) for n in names}
    heads = {n: O.send_recv_heads(O.token_shards(padded[n], W)) for n in names}
    mask_ext = O.extend_user_mask(x["mask"], Tp) if x["mask"] is not None else None
    Tq = wl.Tq if wl.cross else Tp
    kv_valid = T if mask_ext is None else Tp
    for r in (0, W - 1):
        out = torch.empty_like(step.oh[r])
        out.view(torch.uint8).fill_(0xFF)
        step.attention_rank(r, out)
        torch.cuda.synchronize()
        got = f64(raw(out))
        assert np.isfinite(got).all()
        qr = f64(x["q"][:, :, r * Hl:(r + 1) * Hl]) if wl.cross else f64(heads["q"][r])
        rows = sample_rows(Tq, Tq // W, T if not wl.cross else Tq, rng)
        want = O.attention_heads(qr, f64(heads["k"][r]), f64(heads["v"][r]), scale, kv_valid, mask_ext,
                                 rows=rows)[:, rows]
        err = float(np.max(np.abs(got[:, rows] - want)))
        assert err <= TOL[wl.dtype], (r, err)


@pytest.mark.parametrize("name", ["video_self", "uneven_mask", "cross_v2a", "tiny"])
def test_workload_step_graph_replays(name):
    """The step recorded as a HIP graph: every replay, with eager work and
    synchronisation between replays, writes the same output bytes as the eager
    step."""
    wl = WORKLOADS[name]
    say("graph", name)
    x = make_inputs(wl)
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    mask = to_dev(x["mask"]) if x["mask"] is not None else None
    step = UlyssesStep(wl, q, k, v, mask)
    want = step.run().clone()
    torch.cuda.synchronize()
    g = step.capture()
    for i in range(4):
        step.out.view(torch.uint8).fill_(0xFF)       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out.view(torch.uint8), want.view(torch.uint8)), i


def _allocations():
    return torch.cuda.memory_stats().get("allocation.all.allocated", 0)


@pytest.mark.parametrize("name", ORDER)
def test_workload_step_allocates_nothing(name):
    """Buffers and workspaces are made when the step is built: run() and
    run_zero_copy() make no device allocation (so a captured graph or a
    serving loop reuses the same memory every step)."""
    wl = WORKLOADS[name]
    say("step allocations", name)
    x = make_inputs(wl)
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    mask = to_dev(x["mask"]) if x["mask"] is not None else None
    step = UlyssesStep(wl, q, k, v, mask)
    step.run()
    step.run_zero_copy()                   # its buffers are made on first use
    torch.cuda.synchronize()
    before = _allocations()
    for _ in range(2):
        step.run()
        step.run_zero_copy()
    torch.cuda.synchronize()
    assert _allocations() == before


def test_joint_and_2d_steps_allocate_nothing():
    from sequence_attention_video_amd.pipeline import JointAVStep, Ulysses2DStep
    from sequence_attention_video_amd.workloads import GRIDS, JOINT_AV, make_joint_inputs
    say("step allocations joint_av and 2-D")
    joint = JointAVStep(JOINT_AV, make_joint_inputs(JOINT_AV))
    joint.run()
    joint.run_concurrent()
    wl = WORKLOADS["video_self"]
    x = make_inputs(wl)
    step2 = Ulysses2DStep(wl, GRIDS["video_self"], to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]))
    step2.run()
    torch.cuda.synchronize()
    before = _allocations()
    joint.run()
    joint.run_concurrent()
    step2.run()
    torch.cuda.synchronize()
    assert _allocations() == before
