"""The C ABI used from native code alone: tests/native_step.cpp (built by
build() into tests/bin/native_step) runs pad, partition, send_recv_heads,
masked attention over every rank, gather_heads and gather_output_tokens with
hipMalloc'd buffers on a stream of its own, in a child process; its output is
checked against the float64 oracle (fp32: 1e-4)."""

import math
import os
import subprocess

import numpy as np
import pytest

import oracle as O
from sequence_attention_video_amd import build
from sequence_attention_video_amd.workloads import WORKLOADS, make_inputs
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", ["tiny", (2, 301, 4, 8, 64)])
def test_native_consumer_runs_the_path(tmp_path, shape):
    if not os.path.exists(build.NATIVE_BIN):
        pytest.fail("tests/bin/native_step is not built (run __graft_entry__.build())")
    if shape == "tiny":
        wl = WORKLOADS["tiny"]
        x = make_inputs(wl)
        B, T, W, H, D = wl.B, wl.T, wl.W, wl.H, wl.D
        q, k, v = x["q"], x["k"], x["v"]
    else:
        B, T, W, H, D = shape
        rng = np.random.default_rng(T)
        q, k, v = (rng.standard_normal((B, T, H, D)).astype(np.float32) for _ in range(3))
    say("native step", B, T, W, H, D)
    for name, a in zip("qkv", (q, k, v)):
        np.ascontiguousarray(a, dtype=np.float32).tofile(tmp_path / f"{name}.bin")
    run = subprocess.run([build.NATIVE_BIN, str(tmp_path), str(B), str(T), str(W), str(H), str(D)],
                         capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stderr
    got = np.fromfile(tmp_path / "out.bin", dtype=np.float32).reshape(B, T, H, D).astype(np.float64)
    want = O.ulysses_self_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), W,
                                    1.0 / math.sqrt(D))
    assert np.isfinite(got).all()
    assert np.max(np.abs(got - want)) <= 1e-4
