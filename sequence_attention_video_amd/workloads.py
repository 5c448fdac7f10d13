"""Seeded synthetic workloads for the sequence-parallel attention path.

This module only makes inputs: shapes, seeded normal draws, their bfloat16
encoding and the user mask of the masked workload.  It holds none of the
path's arithmetic, so both the HIP path's tests and the CPU oracle can be fed
the very same bytes from it.

The five workloads stand in for the video DiT activations of the pages
(121-frame LTX-2 video generation, 10-second LongCat videos), which need model
weights, prompts and latents that are not available here.  Recipe:

* generator ``numpy.random.default_rng(1000 * index + {q: 0, k: 1, v: 2})``;
* standard normals drawn in float64, in chunks of 2**24 values, multiplied by
  the workload's ``std`` (1 or 1/sqrt(D)), cast to float32, then for bf16
  workloads rounded to bfloat16 (round to nearest, ties to even) and kept as
  uint16 bit patterns;
* the masked workload's user mask is block-causal over 16 frames of 384 tokens
  with 6 trailing prompt tokens (see ``block_causal_mask``).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np

CHUNK = 1 << 24


@dataclass(frozen=True)
class Workload:
    index: int            # 1-based, fixes the seeds
    name: str
    B: int
    T: int                # valid tokens on the exchanged (self-attention) side
    W: int                # virtual ranks
    H: int
    D: int
    dtype: str            # "f32" or "bf16"
    std: str              # "1" or "1/sqrt(D)"
    mask: str             # "key" (key-only padding mask) or "block_causal"
    cross: bool = False   # queries are not exchanged, only K/V
    Tq: int = 0           # cross only: query tokens
    T_pad_override: int = 0  # cross only: K/V buffer length (>= T, divisible by W)

    @property
    def T_pad(self) -> int:
        if self.T_pad_override:
            return self.T_pad_override
        return self.W * (-(-self.T // self.W))

    @property
    def Hl(self) -> int:
        return self.H // self.W

    @property
    def eb(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def scale_std(self) -> float:
        return 1.0 if self.std == "1" else 1.0 / math.sqrt(self.D)

    @property
    def q_tokens(self) -> int:
        """Query tokens of the whole problem (equals T for self-attention)."""
        return self.Tq if self.cross else self.T

    @property
    def q_tokens_pad(self) -> int:
        """Query rows the path computes: the query modality padded to a
        multiple of W (cross-attention queries are padded on their own)."""
        return self.W * (-(-self.Tq // self.W)) if self.cross else self.T_pad


WORKLOADS = {
    "tiny": Workload(1, "tiny", B=1, T=50, W=4, H=8, D=16, dtype="f32", std="1", mask="key"),
    "video_self": Workload(2, "video_self", B=1, T=6144, W=8, H=32, D=128, dtype="bf16",
                           std="1/sqrt(D)", mask="key"),
    "uneven_mask": Workload(3, "uneven_mask", B=1, T=6150, W=8, H=32, D=128, dtype="bf16",
                            std="1/sqrt(D)", mask="block_causal"),
    "cross_v2a": Workload(4, "cross_v2a", B=1, T=987, W=8, H=32, D=64, dtype="bf16", std="1",
                          mask="key", cross=True, Tq=6144, T_pad_override=1024),
    "long_hires": Workload(5, "long_hires", B=2, T=32768, W=8, H=32, D=128, dtype="bf16",
                           std="1/sqrt(D)", mask="key"),
}

ORDER = ["tiny", "video_self", "uneven_mask", "cross_v2a", "long_hires"]


@dataclass(frozen=True)
class JointWorkload:
    """One joint audio-video attention block: video self-attention, audio
    self-attention, video->audio and audio->video cross-attention, each
    modality padded to its own multiple of W.  Video: 16 latent frames of
    16 x 24 tokens (as video_self); audio: 987 tokens (as cross_v2a's keys),
    padded to 992.  Video self-attention uses D = 128, the audio and cross
    attentions D = 64 (the audio stream's width); activations N(0, 1/D)."""
    index: int = 6
    name: str = "joint_av"
    B: int = 1
    W: int = 8
    H: int = 32
    Tv: int = 6144
    Ta: int = 987
    Dv: int = 128
    Da: int = 64
    dtype: str = "bf16"

    def parts(self) -> dict:
        common = dict(B=self.B, W=self.W, H=self.H, dtype=self.dtype, std="1/sqrt(D)", mask="key")
        return {
            "video_self": Workload(self.index, "joint_video_self", T=self.Tv, D=self.Dv, **common),
            "audio_self": Workload(self.index, "joint_audio_self", T=self.Ta, D=self.Da, **common),
            "v2a": Workload(self.index, "joint_v2a", T=self.Ta, D=self.Da, cross=True, Tq=self.Tv, **common),
            "a2v": Workload(self.index, "joint_a2v", T=self.Tv, D=self.Da, cross=True, Tq=self.Ta, **common),
        }


# latent grids (frames, height, width) of the workloads whose tokens are one
# video: 16 frames of 16 x 24 (video_self), 8 frames of 64 x 64 (long_hires)
GRIDS = {"video_self": (16, 16, 24), "long_hires": (8, 64, 64)}

JOINT_AV = JointWorkload()
JOINT_SEED_OFFSET = {"video_self": 0, "audio_self": 10, "v2a": 20, "a2v": 30}


def make_joint_inputs(jw: JointWorkload) -> dict:
    """Per part (see JointWorkload.parts) the make_inputs dict, seeds
    1000 * index + part offset + {q: 0, k: 1, v: 2}."""
    return {name: make_inputs(wl, JOINT_SEED_OFFSET[name]) for name, wl in jw.parts().items()}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 patterns.

    Only finite inputs are produced here (normal draws), so NaN handling is
    not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def seeded_normal(seed: int, shape, std: float, dtype: str) -> np.ndarray:
    """Seeded N(0, std^2) values in the workload's storage type.

    float32 array for "f32"; uint16 bfloat16 patterns for "bf16".
    """
    n = int(np.prod(shape))
    rng = np.random.default_rng(seed)
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
    for i0 in range(0, n, CHUNK):
        i1 = min(n, i0 + CHUNK)
        z = (rng.standard_normal(i1 - i0) * std).astype(np.float32)
        out[i0:i1] = z if dtype == "f32" else f32_to_bf16_bits(z)
    return out.reshape(shape)


def block_causal_mask(t_valid: int, frames: int, frame_len: int, n_prompt: int) -> np.ndarray:
    """User mask (1, T, T), uint8, 1 = may attend.

    Token layout: ``frames`` video frames of ``frame_len`` tokens, then
    ``n_prompt`` prompt tokens (T = frames * frame_len + n_prompt).  A video
    token of frame f sees the video tokens of frames 0..f and every prompt
    token; a prompt token sees every token.
    """
    n_video = frames * frame_len
    if n_video + n_prompt != t_valid:
        raise ValueError("frames * frame_len + n_prompt must equal T")
    idx = np.arange(t_valid)
    frame_of = np.where(idx < n_video, idx // frame_len, frames)   # prompt = "frame" F
    q_frame = frame_of[:, None]
    k_frame = frame_of[None, :]
    q_prompt = (idx >= n_video)[:, None]
    k_prompt = (idx >= n_video)[None, :]
    vis = (k_frame <= q_frame) | k_prompt | q_prompt
    return vis.astype(np.uint8)[None]


# Unit-spread variants of the video workloads: the same shapes and masks with
# Q, K, V drawn N(0, 1) (seeds 1000 * index + 500 + {q: 0, k: 1, v: 2}).  With
# N(0, 1/D) activations the scores q.k/sqrt(D) spread by about 1/D, every
# softmax row is nearly uniform and outputs are about 1e-3, below the bf16
# tolerance: a result that ignored the scores or the mask would pass.  With
# unit-spread scores the softmax is far from uniform and such results miss the
# tolerance by a wide margin.
UNIT_SEED_OFFSET = 500
UNIT_SPREAD = ("video_self", "uneven_mask", "long_hires")


def unit_spread(wl: Workload) -> Workload:
    """The workload with Q, K, V drawn N(0, 1) (see UNIT_SPREAD)."""
    return replace(wl, std="1", name=wl.name + "_unit")


def make_inputs(wl: Workload, seed_offset: int = 0) -> dict:
    """Q, K, V (and the user mask) of a workload, on the host.

    Self-attention: q, k, v are (B, T, H, D) with the T valid tokens.
    Cross-attention: q is (B, Tq, H, D); k, v are (B, T, H, D) with the T real
    keys.  Arrays are float32 ("f32") or uint16 bfloat16 patterns ("bf16").
    """
    base = 1000 * wl.index + seed_offset
    std = wl.scale_std
    tq = wl.q_tokens
    out = {
        "q": seeded_normal(base + 0, (wl.B, tq, wl.H, wl.D), std, wl.dtype),
        "k": seeded_normal(base + 1, (wl.B, wl.T, wl.H, wl.D), std, wl.dtype),
        "v": seeded_normal(base + 2, (wl.B, wl.T, wl.H, wl.D), std, wl.dtype),
        "mask": None,
    }
    if wl.mask == "block_causal":
        out["mask"] = block_causal_mask(wl.T, 16, 384, wl.T - 16 * 384)
    return out

