"""One step of the sequence-parallel attention path on one GPU, W virtual ranks.

Calls the library's entry points in the order of page "LTX-2 序列并行拆解：token
切分、all2all 换头与 runner 接入全链路", section "token 切片、换头、gather 还原":
补齐 (sp_pad) -> 切分 (sp_partition) -> 换头 (sp_relayout_heads, then
sp_masked_attention on every rank's local heads, then sp_relayout_heads back)
-> 还原 (sp_gather_unpad).  This module only allocates buffers and passes
pointers, sizes and strides; every byte of the path is produced by HIP kernels.

Memory layout in HBM (elements, row-major):
  inputs   q, k, v            (B, T, H, D)       self-attention
           q                  (B, Tq, H, D)      cross-attention (never exchanged)
  padded   q, k, v            (B, T_pad, H, D)   rank s's token shard = rows s*Ts..s*Ts+Ts-1
  head side q, k, v, o        (W, B, T_pad, Hl, D)   rank r's local heads r*Hl..r*Hl+Hl-1
  token side o                (W, B, Ts, H, D)   rank s's local output
  output                      (B, T, H, D)
  mask                        (B, T, T) uint8 -> extended (B, T_pad, T_pad)
"""

from __future__ import annotations

import math

import torch

from . import binding as sp
from .workloads import Workload

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def to_device(arr, dtype: str, device) -> torch.Tensor:
    """Host array (float32, or uint16 bf16 patterns) -> device tensor of the same bytes."""
    t = torch.from_numpy(arr)
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to(device)


class UlyssesStep:
    """Buffers and launch sequence for one workload (all W ranks in each launch)."""

    def __init__(self, wl: Workload, q, k, v, mask=None, device="cuda"):
        self.wl = wl
        B, H, D, W = wl.B, wl.H, wl.D, wl.W
        T, Tp, Hl = wl.T, wl.T_pad, wl.Hl
        self.Ts = Tp // W
        dt = TORCH_DTYPE[wl.dtype]
        e = lambda *s, d=dt: torch.empty(*s, dtype=d, device=device)
        self.q, self.k, self.v, self.mask = q, k, v, mask
        self.need_pad = Tp != T
        self.need_q_pad = False
        if wl.cross:
            self.kp, self.vp = (e(B, Tp, H, D), e(B, Tp, H, D)) if self.need_pad else (k, v)
            self.kh, self.vh = e(W, B, Tp, Hl, D), e(W, B, Tp, Hl, D)
            # the query modality is padded on its own to a multiple of W (it is
            # sliced on the rank, never exchanged); output unpadded to Tq
            Tq, Tqp = wl.Tq, wl.q_tokens_pad
            self.need_q_pad = Tqp != Tq
            self.qc = e(B, Tqp, H, D) if self.need_q_pad else q
            self.Tsq = Tqp // W
            self.oh = e(W, B, Tqp, Hl, D)
            self.ot = e(W, B, self.Tsq, H, D)
            self.out = e(B, Tq, H, D)
        else:
            if self.need_pad:
                self.qp, self.kp, self.vp = e(B, Tp, H, D), e(B, Tp, H, D), e(B, Tp, H, D)
            else:
                self.qp, self.kp, self.vp = q, k, v
            self.qh, self.kh, self.vh = (e(W, B, Tp, Hl, D) for _ in range(3))
            self.oh = e(W, B, Tp, Hl, D)
            self.ot = e(W, B, self.Ts, H, D)
            self.out = e(B, T, H, D)
        self.mask_ext = None
        self.workspace = None
        if mask is not None:
            if self.need_pad:
                self.mask_ext = torch.empty(mask.shape[0], Tp, Tp, dtype=torch.uint8, device=device)
            else:
                self.mask_ext = mask          # already (B, T_pad, T_pad): extension is the identity
        # the all-ranks attention launch's workspace (mask classes, or the
        # partial records of a split launch), allocated once: run() allocates
        # nothing
        tq_attn = wl.q_tokens_pad if wl.cross else Tp
        need = sp.sp_masked_attention_workspace_size(W, B, tq_attn, Tp, Hl, D, sp._dtype_code(self.kh),
                                                     mask is not None,
                                                     Tp * Tp if mask is not None and mask.shape[0] > 1 else 0)
        if need:
            self.workspace = torch.empty(need, dtype=torch.uint8, device=device)
        self.scale = 1.0 / math.sqrt(D)

    # -- the step's stages, each one library call (or one host call) ----------
    def pad(self):
        wl = self.wl
        C = wl.H * wl.D
        if self.need_q_pad:
            sp.sp_pad(self.q.view(wl.B, wl.Tq, C), self.qc.view(wl.B, wl.q_tokens_pad, C), wl.q_tokens_pad)
        if not self.need_pad:
            return
        if wl.cross:
            pairs = [(self.k, self.kp), (self.v, self.vp)]
        else:
            pairs = [(self.q, self.qp), (self.k, self.kp), (self.v, self.vp)]
        for x, y in pairs:
            sp.sp_pad(x.view(wl.B, wl.T, C), y.view(wl.B, wl.T_pad, C), wl.T_pad)
        self.pad_mask()

    def pad_mask(self):
        """The user mask's extension (补齐), in a call of its own: the mask may
        be one (1, T, T) mask shared by every batch."""
        if self.mask is not None and self.need_pad:
            sp.sp_pad(None, None, self.wl.T_pad, mask_in=self.mask, mask_out=self.mask_ext)

    def partition(self):
        return sp.sp_partition(self.wl.T_pad, self.wl.W)

    def send_recv_heads(self):
        wl = self.wl
        tok = (self.Ts * wl.H * wl.D, wl.T_pad * wl.H * wl.D)   # rank shards are views of (B, T_pad, H, D)
        if wl.cross:
            src, dst = [self.kp, self.vp], [self.kh, self.vh]
        else:
            src, dst = [self.qp, self.kp, self.vp], [self.qh, self.kh, self.vh]
        sp.sp_relayout_heads(src, dst, wl.W, wl.B, wl.T_pad, wl.H, wl.D, sp.SP_TOKENS_TO_HEADS, tok_strides=tok)

    def attention(self):
        wl = self.wl
        B, Tp, Hl, D, H = wl.B, wl.T_pad, wl.Hl, wl.D, wl.H
        head_side = (B * Tp * Hl * D, Tp * Hl * D, Hl * D, D)
        if wl.cross:
            Tq = wl.q_tokens_pad
            qs = (Hl * D, Tq * H * D, H * D, D)            # rank r's heads of the unexchanged Q
            os_ = (B * Tq * Hl * D, Tq * Hl * D, Hl * D, D)
            sp.sp_masked_attention(self.qc, self.kh, self.vh, self.oh, wl.W, B, Tq, Tp, Hl, D,
                                   qs, head_side, head_side, os_, kv_valid_len=wl.T, scale=self.scale,
                                   workspace=self.workspace)
            return
        if self.mask is not None:
            sp.sp_masked_attention(self.qh, self.kh, self.vh, self.oh, wl.W, B, Tp, Tp, Hl, D,
                                   head_side, head_side, head_side, head_side, kv_valid_len=Tp,
                                   mask=self.mask_ext, scale=self.scale, workspace=self.workspace)
        else:
            sp.sp_masked_attention(self.qh, self.kh, self.vh, self.oh, wl.W, B, Tp, Tp, Hl, D,
                                   head_side, head_side, head_side, head_side, kv_valid_len=wl.T,
                                   scale=self.scale, workspace=self.workspace)

    def attention_rank(self, r: int, out, workspace=None):
        """Rank r's share alone (R = 1): the attention launch one GPU runs when
        the ranks are real devices.  out: (B, Tq, Hl, D) head-side buffer.  A
        share has few query tiles, so the library usually splits their key
        ranges over the GPU (by non-empty tiles under a user mask; workspace
        from the size query, allocated here when not given)."""
        wl = self.wl
        B, Tp, Hl, D, H = wl.B, wl.T_pad, wl.Hl, wl.D, wl.H
        head_side = (B * Tp * Hl * D, Tp * Hl * D, Hl * D, D)
        if wl.cross:
            Tq = wl.q_tokens_pad
            qs = (Hl * D, Tq * H * D, H * D, D)
            os_ = (B * Tq * Hl * D, Tq * Hl * D, Hl * D, D)
            q = self.qc[:, :, r * Hl:(r + 1) * Hl]
            sp.sp_masked_attention(q, self.kh[r], self.vh[r], out, 1, B, Tq, Tp, Hl, D, qs, head_side, head_side,
                                   os_, kv_valid_len=wl.T, scale=self.scale, workspace=workspace)
        elif self.mask is not None:
            sp.sp_masked_attention(self.qh[r], self.kh[r], self.vh[r], out, 1, B, Tp, Tp, Hl, D, head_side,
                                   head_side, head_side, head_side, kv_valid_len=Tp, mask=self.mask_ext,
                                   scale=self.scale, workspace=workspace)
        else:
            sp.sp_masked_attention(self.qh[r], self.kh[r], self.vh[r], out, 1, B, Tp, Tp, Hl, D, head_side,
                                   head_side, head_side, head_side, kv_valid_len=wl.T, scale=self.scale,
                                   workspace=workspace)

    def gather_heads(self):
        wl = self.wl
        Tq_pad = wl.q_tokens_pad if wl.cross else wl.T_pad
        sp.sp_relayout_heads([self.oh], [self.ot], wl.W, wl.B, Tq_pad, wl.H, wl.D, sp.SP_HEADS_TO_TOKENS)

    def gather_output_tokens(self, lengths):
        wl = self.wl
        C = wl.H * wl.D
        if wl.cross:
            sp.sp_gather_unpad(self.ot, self.out, wl.W, wl.B, self.Tsq, C, wl.Tq, counts=[self.Tsq] * wl.W)
        else:
            sp.sp_gather_unpad(self.ot, self.out, wl.W, wl.B, self.Ts, C, wl.T, counts=lengths)

    # -- the step with each pair of moves fused (the default) ------------------
    # On one device pad followed by send_recv_heads is one permutation of the
    # token rows (pad rows become zero runs on the head side), and so is
    # gather_heads followed by gather_output_tokens: each pair is one library
    # call that moves every byte once, with the same bytes as the two calls.
    def pad_send(self):
        wl = self.wl
        C = wl.H * wl.D
        if self.need_q_pad:
            sp.sp_pad(self.q.view(wl.B, wl.Tq, C), self.qc.view(wl.B, wl.q_tokens_pad, C), wl.q_tokens_pad)
        self.pad_mask()
        if wl.cross:
            src, dst = [self.k, self.v], [self.kh, self.vh]
        else:
            src, dst = [self.q, self.k, self.v], [self.qh, self.kh, self.vh]
        sp.sp_pad_relayout_heads(src, dst, wl.W, wl.B, wl.T, wl.T_pad, wl.H, wl.D)

    def gather_unpad(self, lengths):
        wl = self.wl
        if wl.cross:
            sp.sp_gather_heads_unpad([self.oh], [self.out], wl.W, wl.B, wl.q_tokens_pad, wl.H, wl.D, wl.Tq,
                                     counts=[self.Tsq] * wl.W)
        else:
            sp.sp_gather_heads_unpad([self.oh], [self.out], wl.W, wl.B, wl.T_pad, wl.H, wl.D, wl.T, counts=lengths)

    def run(self):
        self.pad_send()
        _, lengths = self.partition()
        self.attention()
        self.gather_unpad(lengths)
        return self.out

    def run_separate(self):
        """The step as the five separate calls (pad, partition, send_recv_heads,
        attention, gather_heads, gather_output_tokens): the same output bytes
        as run(), with the padded token tensors and the token-side output
        written along the way."""
        self.pad()
        _, lengths = self.partition()
        self.send_recv_heads()
        self.attention()
        self.gather_heads()
        self.gather_output_tokens(lengths)
        return self.out

    def capture(self):
        """Record run() into a HIP graph (torch.cuda.CUDAGraph) and return it:
        replay() re-issues the step's kernels on the same buffers with the same
        arguments, without the per-launch host work.  The library allocates
        nothing and records no memset, so every node is one of its kernels."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.run()                      # first launches outside the capture
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run()
        return g

    # -- the same step with every move folded into attention's addressing -----
    # On one device rank r's head-side view is a strided view of the token
    # layout: heads r*Hl.. of every token (rank stride Hl*D, token stride
    # H*D).  Attention reads Q/K/V and writes O through those strides, so
    # send_recv_heads and gather_heads move no bytes.  Padding exists only so
    # that the exchange splits the sequence evenly, so with no exchange the
    # launch runs on the caller's unpadded tensors and mask (Tq = Tk = T, the
    # user mask as given) and writes the final (B, T, H, D) output: pad, the
    # mask extension and gather_output_tokens move no bytes either.  The real
    # query rows see the same key tiles, visibility bits and summation order
    # as in run() (the padded keys had zero weight; the padded rows are
    # dropped by the unpad), hence the same bytes.
    def attention_zero_copy(self):
        wl = self.wl
        B, T, Hl, D, H, W = wl.B, wl.T, wl.Hl, wl.D, wl.H, wl.W
        Tq = wl.Tq if wl.cross else T
        if not hasattr(self, "outz"):
            self.outz = torch.empty(B, Tq, H, D, dtype=self.k.dtype, device=self.k.device)
            mbs = 0 if self.mask is None or self.mask.shape[0] == 1 else T * T
            need = sp.sp_masked_attention_workspace_size(W, B, Tq, T, Hl, D, sp._dtype_code(self.k),
                                                         self.mask is not None, mbs)
            self.workspace_z = torch.empty(need, dtype=torch.uint8, device=self.k.device) if need else None
        qs = (Hl * D, Tq * H * D, H * D, D)                  # rank, batch, token, head
        ks = (Hl * D, T * H * D, H * D, D)
        sp.sp_masked_attention(self.q, self.k, self.v, self.outz, W, B, Tq, T, Hl, D, qs, ks, ks, qs,
                               kv_valid_len=T, mask=self.mask, scale=self.scale, workspace=self.workspace_z)

    def run_zero_copy(self):
        self.partition()
        self.attention_zero_copy()
        return self.outz


class JointAVStep:
    """The joint audio-video attention of one block: video self-attention,
    audio self-attention, video->audio and audio->video cross-attention, each
    on the sequence-parallel path over the same W virtual ranks (page "LTX-2
    序列并行拆解", section "token 切片、换头、gather 还原": 补齐 per modality;
    for cross-attention the rank slices the query side and only K/V go
    through the exchange).  Each part is one UlyssesStep; the modalities are
    padded independently (video 6144 -> 6144, audio 987 -> 992 at W = 8)."""

    PARTS = ("video_self", "audio_self", "v2a", "a2v")

    def __init__(self, jw, inputs: dict, device="cuda"):
        self.jw = jw
        self.steps = {}
        for name, wl in jw.parts().items():
            x = inputs[name]
            q, k, v = (to_device(x[n], wl.dtype, device) for n in "qkv")
            self.steps[name] = UlyssesStep(wl, q, k, v, None, device=device)
        self._streams = {name: torch.cuda.Stream(device=device) for name in self.PARTS}   # run_concurrent()

    def run(self) -> dict:
        return {name: self.steps[name].run() for name in self.PARTS}

    # The four parts share no buffer, so they may run at once: each on a
    # stream of its own (default priority), forked from and joined back into
    # the caller's current stream.  The audio-sized launches leave most of
    # the GPU idle (the audio->video part has 128 query tiles for 256 CUs);
    # side by side they fill it.  Same kernels on the same inputs, hence the
    # same bytes as run().  The video self-attention is issued first: of the
    # groupings measured (one stream per part in either order, the audio-sized
    # parts on one or two shared streams) this one was fastest.
    CONCURRENT_ORDER = ("video_self", "a2v", "v2a", "audio_self")

    def run_concurrent(self) -> dict:
        cur = torch.cuda.current_stream()
        outs = {}
        for name in self.CONCURRENT_ORDER:
            s = self._streams[name]
            s.wait_stream(cur)
            with torch.cuda.stream(s):
                outs[name] = self.steps[name].run()
        for name in self.CONCURRENT_ORDER:
            cur.wait_stream(self._streams[name])
        return {name: outs[name] for name in self.PARTS}


class Ulysses2DStep:
    """Self-attention with the 2-D (height x width) split of page
    "LongCat-Video上下文并行技术如何实现高效的多GPU推理" (section 智能张量拆分策略)
    in place of the 1-D token split: the W ranks form a near-square
    split_h x split_w grid over the latent's height x width (sp_optimal_split);
    split_cp_2d gives each rank its tile of every frame (sp_tile_2d), the head
    exchange, attention and the way back run as in UlyssesStep on those
    shards, and gather_cp_2d (sp_tile_2d) restores raster order.  Attention
    does not depend on token order (key-only mask, no padding: the grid must
    split evenly), so the output is the same attention up to summation order.
    run() does each split and exchange pair as one move; run_separate() keeps
    them apart (same bytes).
    Memory: tiles (W, B, Tt, H, D) with Tt = F*th*tw; head side
    (W, B, T, Hl, D) in rank-then-tile token order."""

    def __init__(self, wl: Workload, grid, q, k, v, device="cuda"):
        self.wl = wl
        F, Hh, Ww = grid
        if F * Hh * Ww != wl.T or wl.T_pad != wl.T:
            raise ValueError("the grid must hold exactly the workload's tokens")
        self.grid = grid
        B, H, D, W, T, Hl = wl.B, wl.H, wl.D, wl.W, wl.T, wl.Hl
        self.split = sp.sp_optimal_split(W, Hh, Ww)
        self.Tt = T // W
        dt = TORCH_DTYPE[wl.dtype]
        e = lambda *s: torch.empty(*s, dtype=dt, device=device)
        self.q, self.k, self.v = q, k, v
        self.qt, self.kt, self.vt = (e(W, B, self.Tt, H, D) for _ in range(3))
        self.qh, self.kh, self.vh = (e(W, B, T, Hl, D) for _ in range(3))
        self.oh = e(W, B, T, Hl, D)
        self.ot = e(W, B, self.Tt, H, D)
        self.out = e(B, T, H, D)
        need = sp.sp_masked_attention_workspace_size(W, B, T, T, Hl, D, sp._dtype_code(self.qh), False, 0)
        self.workspace = torch.empty(need, dtype=torch.uint8, device=device) if need else None
        self.scale = 1.0 / math.sqrt(D)

    def split_cp_2d(self):
        wl = self.wl
        F, Hh, Ww = self.grid
        for x, y in ((self.q, self.qt), (self.k, self.kt), (self.v, self.vt)):
            sp.sp_tile_2d(x, y, *self.split, wl.B, F, Hh, Ww, wl.H * wl.D, sp.SP_GRID_TO_TILES)

    def send_recv_heads(self):
        wl = self.wl
        sp.sp_relayout_heads([self.qt, self.kt, self.vt], [self.qh, self.kh, self.vh], wl.W, wl.B, wl.T, wl.H,
                             wl.D, sp.SP_TOKENS_TO_HEADS)

    def attention(self):
        wl = self.wl
        B, T, Hl, D = wl.B, wl.T, wl.Hl, wl.D
        hs = (B * T * Hl * D, T * Hl * D, Hl * D, D)
        sp.sp_masked_attention(self.qh, self.kh, self.vh, self.oh, wl.W, B, T, T, Hl, D, hs, hs, hs, hs,
                               kv_valid_len=T, scale=self.scale, workspace=self.workspace)

    def gather_heads(self):
        wl = self.wl
        sp.sp_relayout_heads([self.oh], [self.ot], wl.W, wl.B, wl.T, wl.H, wl.D, sp.SP_HEADS_TO_TOKENS)

    def gather_cp_2d(self):
        wl = self.wl
        F, Hh, Ww = self.grid
        sp.sp_tile_2d(self.ot, self.out, *self.split, wl.B, F, Hh, Ww, wl.H * wl.D, sp.SP_TILES_TO_GRID)

    # On one device the split and the exchange are one permutation each way
    # (sp_tile_2d_relayout_heads): the grid goes straight to the head side
    # and back, with the same bytes as the two separate moves.
    def split_send_heads(self):
        wl = self.wl
        F, Hh, Ww = self.grid
        sp.sp_tile_2d_relayout_heads([self.q, self.k, self.v], [self.qh, self.kh, self.vh], *self.split, wl.B, F,
                                     Hh, Ww, wl.H, wl.D, sp.SP_TOKENS_TO_HEADS)

    def gather_heads_cp_2d(self):
        wl = self.wl
        F, Hh, Ww = self.grid
        sp.sp_tile_2d_relayout_heads([self.oh], [self.out], *self.split, wl.B, F, Hh, Ww, wl.H, wl.D,
                                     sp.SP_HEADS_TO_TOKENS)

    def run(self):
        self.split_send_heads()
        self.attention()
        self.gather_heads_cp_2d()
        return self.out

    def run_separate(self):
        """The same step with the split and the exchange as separate moves
        (split_cp_2d, send_recv_heads; gather_heads, gather_cp_2d)."""
        self.split_cp_2d()
        self.send_recv_heads()
        self.attention()
        self.gather_heads()
        self.gather_cp_2d()
        return self.out
