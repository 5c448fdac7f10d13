"""The five workloads at full size, in the launch configuration bench.py times
(sequence_attention_video_amd.pipeline.UlyssesStep, all W virtual ranks per
launch), checked against the CPU oracle:

* the five separate calls (run_separate): pad, mask extension, both
  relayouts and gather/unpad bit-exact in full; attention within the
  tolerance on every output row of every (rank, head) for the tiny,
  video_self, uneven_mask and cross_v2a workloads, and for long_hires on the
  whole of rank 0's share plus 512 seeded rows per head of every other rank
  (first, last and shard-boundary rows among them);
* the fused step (run, each pair of moves as one call): the same head sides
  and output bytes as run_separate;
* the zero-copy step (both exchanges folded into attention's strides) and the
  fused step: their outputs against the oracle's whole path directly, on the
  same rows;
* sharded == unsharded: sampled output rows against unsharded attention on the
  unpadded problem ([SP] "全局注意力没有变，只是分布方式变了"; [MG]
  "Capabilities", sequence-parallel row).

The video workloads draw activations N(0, 1/D), so their softmax rows are
nearly uniform and outputs are about 1e-3: below the bf16 tolerance, a result
that dropped the scores or the mask would pass.  Each of them therefore also
runs as a unit-spread variant (Q, K, V drawn N(0, 1)), where the test asserts
negative controls on the checked rows: the all-zero output, the mean of the
visible V rows (the scores ignored) and, with a user mask, attention over
every real key (the mask ignored) each miss the tolerance.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
from sequence_attention_video_amd.pipeline import UlyssesStep
from sequence_attention_video_amd.workloads import (ORDER, UNIT_SEED_OFFSET, UNIT_SPREAD, WORKLOADS, make_inputs,
                                                    unit_spread)
from tests.gpu_util import f64, oracle_heads, raw, say, to_dev

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}
FULL_ROWS_LIMIT = 8192          # above this many query rows per head: rank 0 in full, others sampled
OTHER_RANK_ROWS = 512

CASES = [(n, "config") for n in ORDER] + [(n, "unit") for n in UNIT_SPREAD]


def workload_and_inputs(name, variant):
    wl = WORKLOADS[name]
    if variant == "unit":
        wl = unit_spread(wl)
        return wl, make_inputs(wl, UNIT_SEED_OFFSET)
    return wl, make_inputs(wl)


def discriminating(wl) -> bool:
    """Inputs whose outputs are large enough that the negative controls miss
    the tolerance: N(0, 1) activations."""
    return wl.std == "1"


def sampled_rows(n_rows, shard, rng, count):
    rows = {0, 1, n_rows - 1}
    for s in range(1, n_rows // shard):
        rows.update({s * shard - 1, s * shard})
    while len(rows) < count:
        rows.add(int(rng.integers(0, n_rows)))
    return np.array(sorted(rows))


def checked_rows(wl, Tq):
    """Rows checked per (rank, head): every row, or for long sequences every
    row of rank 0 and OTHER_RANK_ROWS seeded rows of each other rank."""
    if Tq <= FULL_ROWS_LIMIT:
        return [np.arange(Tq)] * wl.W
    rng = np.random.default_rng(7000 + wl.index)
    return [np.arange(Tq)] + [sampled_rows(Tq, Tq // wl.W, rng, OTHER_RANK_ROWS) for _ in range(wl.W - 1)]


def mean_of_visible(v, kv_valid, mask, rows, block=1024):
    """The scores-ignored output: for each query row the mean of the V rows it
    may see (uniform weights).  v (B, Tk, Hh, D) float64; mask (Bm, Tq, Tk)."""
    B, Tk = v.shape[:2]
    out = np.zeros((B, len(rows)) + v.shape[2:])
    for b in range(B):
        vb = v[b].reshape(Tk, -1)
        if mask is None:
            out[b] = vb[:kv_valid].mean(axis=0).reshape(v.shape[2:]) if kv_valid > 0 else 0.0
            continue
        mb = mask[b if mask.shape[0] > 1 else 0]
        for i0 in range(0, len(rows), block):
            sel = rows[i0:i0 + block]
            w = (mb[sel] != 0).astype(np.float64)
            w[:, kv_valid:] = 0.0
            cnt = w.sum(axis=1, keepdims=True)
            out[b, i0:i0 + len(sel)] = (np.where(cnt > 0, (w @ vb) / np.maximum(cnt, 1.0), 0.0)
                                        .reshape((len(sel),) + v.shape[2:]))
    return out


def run_case(name, variant):
    wl, x = workload_and_inputs(name, variant)
    say("workload", wl.name)
    W, B, H, D, Hl = wl.W, wl.B, wl.H, wl.D, wl.Hl
    T, Tp = wl.T, wl.T_pad
    # the padded lengths come from the oracle (the workloads carry the same
    # numbers; the cross workload's 1024-key buffer is the page's reading R12)
    if wl.cross:
        assert Tp == 1024 and wl.q_tokens_pad == O.padded_length(wl.Tq, W)
    else:
        assert Tp == O.padded_length(T, W)
    scale = 1.0 / math.sqrt(D)
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    mask = to_dev(x["mask"]) if x["mask"] is not None else None
    step = UlyssesStep(wl, q, k, v, mask)

    # ---- the five separate calls
    say("workload run_separate", wl.name)
    out_sep = step.run_separate().clone()
    torch.cuda.synchronize()
    names = ["k", "v"] if wl.cross else ["q", "k", "v"]
    padded = {n: O.pad_tokens(x[n], Tp) for n in names}
    if step.need_pad:
        for n in names:
            assert raw(getattr(step, n + "p")).tobytes() == padded[n].tobytes(), n
    mask_ext = None
    if x["mask"] is not None:
        mask_ext = O.extend_user_mask(x["mask"], Tp)
        assert np.array_equal(raw(step.mask_ext), mask_ext)
    offs, lens = step.partition()
    assert (offs, lens) == tuple(map(list, O.compute_sequence_partition(Tp, W)))
    heads = {n: O.send_recv_heads(O.token_shards(padded[n], W)) for n in names}
    for n in names:
        assert raw(getattr(step, n + "h")).tobytes() == heads[n].tobytes(), n
    oh = raw(step.oh)
    ot = raw(step.ot)
    assert ot.tobytes() == O.gather_heads(oh).tobytes()
    Tq = wl.q_tokens_pad
    Tsq = Tq // W
    Tout = wl.Tq if wl.cross else T
    pieces = [ot[r].reshape(B, Tsq, H * D) for r in range(W)]
    assert raw(out_sep).reshape(B, Tout, H * D).tobytes() == O.gather_output_tokens(pieces, [Tsq] * W, Tout).tobytes()

    # ---- the fused step: same head sides, same output bytes
    for n in names:
        getattr(step, n + "h").view(torch.uint8).fill_(0xFF)
    step.out.view(torch.uint8).fill_(0xFF)
    say("workload run (fused moves)", wl.name)
    out = step.run().clone()
    torch.cuda.synchronize()
    for n in names:
        assert raw(getattr(step, n + "h")).tobytes() == heads[n].tobytes(), n
    assert torch.equal(out.view(torch.uint8), out_sep.view(torch.uint8))
    say("workload run_zero_copy", wl.name)
    outz = step.run_zero_copy().clone()
    torch.cuda.synchronize()
    assert torch.equal(outz.view(torch.uint8), out.view(torch.uint8))

    # ---- attention against the oracle, rank by rank, on the checked rows
    ohf = f64(oh)
    assert np.isfinite(ohf).all()
    kv_valid = T if mask_ext is None else Tp
    rows_of = checked_rows(wl, Tq)
    want_oh = {}
    worst = 0.0
    zero_err = uniform_err = nomask_err = 0.0
    for r in range(W):
        rows = rows_of[r]
        say("workload oracle", wl.name, "rank", r, "rows", len(rows))
        qr = f64(x["q"][:, :, r * Hl:(r + 1) * Hl]) if wl.cross else f64(heads["q"][r])
        kr, vr = f64(heads["k"][r]), f64(heads["v"][r])
        if wl.cross and Tq != wl.Tq:
            qr = O.pad_tokens(qr, Tq)
        want = oracle_heads(qr, kr, vr, scale, kv_valid, mask_ext, rows)
        want_oh[r] = want
        worst = max(worst, float(np.max(np.abs(ohf[r][:, rows] - want))))
        if discriminating(wl):
            zero_err = max(zero_err, float(np.max(np.abs(want))))
            uniform_err = max(uniform_err, float(np.max(np.abs(mean_of_visible(vr, kv_valid, mask_ext, rows) - want))))
            if mask_ext is not None:
                ignore = oracle_heads(qr, kr, vr, scale, T, None, rows)
                nomask_err = max(nomask_err, float(np.max(np.abs(ignore - want))))
    say("workload attention", wl.name, "max err", worst, "zero", zero_err, "uniform", uniform_err,
        "mask ignored", nomask_err)
    assert worst <= TOL[wl.dtype], worst
    if discriminating(wl):
        assert zero_err > TOL[wl.dtype], zero_err
        assert uniform_err > TOL[wl.dtype], uniform_err
        if mask_ext is not None:
            assert nomask_err > TOL[wl.dtype], nomask_err

    # ---- the fused and zero-copy outputs against the oracle's whole path on
    #      the same rows: head-side row t of rank r, head j is output token t
    #      (t < Tout), head r*Hl + j
    outf, outzf = f64(raw(out)), f64(raw(outz))
    worst_out = 0.0
    for r in range(W):
        rows = rows_of[r]
        keep = rows < Tout
        got = outf[:, rows[keep], r * Hl:(r + 1) * Hl]
        gotz = outzf[:, rows[keep], r * Hl:(r + 1) * Hl]
        want = want_oh[r][:, keep]
        worst_out = max(worst_out, float(np.max(np.abs(got - want))), float(np.max(np.abs(gotz - want))))
    assert worst_out <= TOL[wl.dtype], worst_out

    # ---- sharded == unsharded on sampled (token, head) rows
    rng = np.random.default_rng(wl.index)
    rows = sampled_rows(Tout, max(1, Tout // W), rng, 24)
    qf, kf, vf = f64(x["q"]), f64(x["k"]), f64(x["v"])
    for hh in [0, 1, H // 2, H - 1]:
        ref = O.attention_heads(qf[:, rows, hh:hh + 1], kf[:, :, hh:hh + 1], vf[:, :, hh:hh + 1], scale,
                                None if x["mask"] is None else T,
                                None if x["mask"] is None else x["mask"][:, rows])
        err = np.max(np.abs(outf[:, rows, hh] - ref[:, :, 0]))
        assert err <= TOL[wl.dtype], (hh, err)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,variant", CASES, ids=[f"{n}-{v}" for n, v in CASES])
def test_workload_full(name, variant):
    run_case(name, variant)


SHARE_CASES = [(n, "config") for n in ORDER if n != "tiny"] + [(n, "unit") for n in UNIT_SPREAD]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,variant", SHARE_CASES, ids=[f"{n}-{v}" for n, v in SHARE_CASES])
def test_workload_rank_share(name, variant):
    """One rank's share alone (R = 1), the launch each GPU runs when the ranks
    are devices and the one bench.py times as the share: split over the GPU
    where the share has too few query tiles.  Ranks 0 and W-1 against the
    oracle: every row (512 seeded rows per head for long sequences)."""
    wl, x = workload_and_inputs(name, variant)
    say("rank share", wl.name)
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
    Tq = wl.q_tokens_pad
    kv_valid = T if mask_ext is None else Tp
    for r in (0, W - 1):
        out = torch.empty_like(step.oh[r])
        out.view(torch.uint8).fill_(0xFF)
        step.attention_rank(r, out)
        torch.cuda.synchronize()
        got = f64(raw(out))
        assert np.isfinite(got).all()
        qr = f64(x["q"][:, :, r * Hl:(r + 1) * Hl]) if wl.cross else f64(heads["q"][r])
        rows = np.arange(Tq) if Tq <= FULL_ROWS_LIMIT else sampled_rows(Tq, Tq // W, rng, OTHER_RANK_ROWS)
        want = oracle_heads(qr, f64(heads["k"][r]), f64(heads["v"][r]), scale, kv_valid, mask_ext, rows)
        err = float(np.max(np.abs(got[:, rows] - want)))
        say("rank share", wl.name, "rank", r, "max err", err)
        assert err <= TOL[wl.dtype], (r, err)
        if discriminating(wl):
            assert float(np.max(np.abs(want))) > TOL[wl.dtype]


def test_shared_mask_over_batches():
    """One (1, T, T) user mask shared by both batches of a B = 2 step: the mask
    is extended on its own (1, T_pad, T_pad) and read by every batch (batch
    stride 0).  Mask extension bit-exact; attention and the output against the
    oracle on every row."""
    from sequence_attention_video_amd.workloads import Workload, seeded_normal
    wl = Workload(9, "shared_mask", B=2, T=1001, W=8, H=16, D=64, dtype="bf16", std="1", mask="block_causal")
    rng = np.random.default_rng(99)
    Tp = wl.T_pad
    m = np.tril(np.ones((wl.T, wl.T), np.uint8))[None]            # causal
    m[0, rng.integers(0, wl.T, 200), :] |= (rng.random((200, wl.T)) < 0.3).astype(np.uint8)
    m[0, 17, :] = 0                                                # a real row that sees nothing
    x = {n: seeded_normal(9000 + i, (wl.B, wl.T, wl.H, wl.D), 1.0, "bf16") for i, n in enumerate("qkv")}
    say("shared mask", wl.B, wl.T, Tp)
    step = UlyssesStep(wl, to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(m))
    assert tuple(step.mask_ext.shape) == (1, Tp, Tp)
    out_sep = step.run_separate().clone()
    out = step.run().clone()
    torch.cuda.synchronize()
    assert np.array_equal(raw(step.mask_ext), O.extend_user_mask(m, Tp))
    assert torch.equal(out.view(torch.uint8), out_sep.view(torch.uint8))
    want = O.ulysses_self_attention(f64(x["q"]), f64(x["k"]), f64(x["v"]), wl.W, 1.0 / math.sqrt(wl.D), m)
    got = f64(raw(out))
    assert np.isfinite(got).all()
    assert np.all(got[:, 17] == 0.0)
    err = float(np.max(np.abs(got - want)))
    assert err <= TOL["bf16"], err


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
    """Buffers and workspaces are made when the step is built: run(),
    run_separate() and run_zero_copy() make no device allocation (so a
    captured graph or a serving loop reuses the same memory every step)."""
    wl = WORKLOADS[name]
    say("step allocations", name)
    x = make_inputs(wl)
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    mask = to_dev(x["mask"]) if x["mask"] is not None else None
    step = UlyssesStep(wl, q, k, v, mask)
    step.run()
    step.run_separate()
    step.run_zero_copy()                   # its buffers are made on first use
    torch.cuda.synchronize()
    before = _allocations()
    for _ in range(2):
        step.run()
        step.run_separate()
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
