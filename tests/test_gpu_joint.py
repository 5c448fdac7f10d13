"""The joint audio-video block (video self-attention, audio self-attention,
video->audio and audio->video cross-attention, each modality padded to its own
multiple of W) at full size on the GPU, against the CPU oracle:

* the audio query modality's padding (987 -> 992 rows) bit-exact;
* every part's final output on every query row within 2e-2 of unsharded
  float64 attention on the real tokens (the sharded == unsharded invariant);
* the zero-copy form of every part byte-identical to its exchange path, and
  against the same oracle rows directly;
* the four parts run concurrently on their own streams give the same bytes
  as run one after another, on several steps in a row.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
from sequence_attention_video_amd.pipeline import JointAVStep
from sequence_attention_video_amd.workloads import JOINT_AV, make_joint_inputs
from tests.gpu_util import f64, oracle_heads, raw, say

pytestmark = pytest.mark.gpu

TOL = 2e-2


def test_joint_av_block():
    say("joint_av")
    jw = JOINT_AV
    x = make_joint_inputs(jw)
    step = JointAVStep(jw, x)
    outs = step.run()
    torch.cuda.synchronize()
    parts = jw.parts()
    # the audio queries of the audio->video cross-attention, padded on their own
    a2v = step.steps["a2v"]
    assert a2v.need_q_pad
    assert raw(a2v.qc).tobytes() == O.pad_tokens(x["a2v"]["q"], parts["a2v"].q_tokens_pad).tobytes()
    for name, wl in parts.items():
        say("joint_av check", name)
        got = f64(raw(outs[name]))
        tq = wl.q_tokens
        assert got.shape == (wl.B, tq, wl.H, wl.D)
        assert np.isfinite(got).all()
        want = oracle_heads(f64(x[name]["q"]), f64(x[name]["k"]), f64(x[name]["v"]), 1.0 / math.sqrt(wl.D), wl.T,
                            None)
        err = np.max(np.abs(got - want))
        assert err <= TOL, (name, err)


def test_joint_av_zero_copy_matches_exchange_path_and_oracle():
    """The zero-copy form of each part (both exchanges folded into
    attention's strides): byte-identical to the exchange path, and on every
    query row within the tolerance of unsharded float64 attention."""
    say("joint_av zero-copy")
    jw = JOINT_AV
    x = make_joint_inputs(jw)
    step = JointAVStep(jw, x)
    parts = jw.parts()
    for name in JointAVStep.PARTS:
        s = step.steps[name]
        out = s.run().clone()
        outz = s.run_zero_copy().clone()
        torch.cuda.synchronize()
        assert torch.equal(outz.view(torch.uint8), out.view(torch.uint8)), name
        wl = parts[name]
        want = oracle_heads(f64(x[name]["q"]), f64(x[name]["k"]), f64(x[name]["v"]), 1.0 / math.sqrt(wl.D), wl.T,
                            None)
        got = f64(raw(outz))
        assert np.isfinite(got).all()
        err = np.max(np.abs(got - want))
        assert err <= TOL, (name, err)


def test_joint_av_concurrent_streams_match_sequential():
    say("joint_av concurrent")
    jw = JOINT_AV
    step = JointAVStep(jw, make_joint_inputs(jw))
    ref = {n: o.clone() for n, o in step.run().items()}
    torch.cuda.synchronize()
    for i in range(3):
        for o in step.run().values():
            o.view(torch.uint8).fill_(0xFF)       # stale bytes would show
        outs = step.run_concurrent()
        torch.cuda.synchronize()
        for name in JointAVStep.PARTS:
            assert torch.equal(outs[name].view(torch.uint8), ref[name].view(torch.uint8)), (i, name)
