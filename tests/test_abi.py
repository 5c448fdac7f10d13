"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/sp.h declares, and its host-only logic (partition, status names,
argument validation that returns before anything is launched) behaves as the
header says."""

import ctypes
import os
import re
import shutil
import subprocess

import pytest

from tests.conftest import ROOT, load_golden

HEADER = os.path.join(ROOT, "include", "sp.h")
LIB = os.path.join(ROOT, "sequence_attention_video_amd", "libspattn.so")


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sp_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libspattn.so is not built (run __graft_entry__.build())")
    from sequence_attention_video_amd import binding
    return binding.load()


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("sp_pad", "sp_partition", "sp_relayout_heads", "sp_masked_attention", "sp_gather_unpad"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (sp_[a-z_0-9]+)$", out, flags=re.M))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    from sequence_attention_video_amd import binding
    assert sorted(binding.EXPORTS) == declared_functions()


def test_partition_through_the_abi(lib):
    from sequence_attention_video_amd import binding
    g = load_golden("partition.txt")
    for case in g["cases"]:
        if case[2] == "ValueError":
            with pytest.raises(ValueError):
                binding.sp_partition(case[0], case[1])
        else:
            assert binding.sp_partition(case[0], case[1]) == (case[2], case[3])
    with pytest.raises(ValueError):
        binding.sp_partition(8, 0)
    assert lib.sp_partition(52, 4, None, None) == binding.SP_OK
    assert lib.sp_partition(50, 4, None, None) == binding.SP_ERR_NOT_DIVISIBLE


def test_status_strings(lib):
    for s in range(5):
        assert lib.sp_status_string(s).startswith(b"SP_")
    assert lib.sp_status_string(99) == b"SP_ERR_UNKNOWN"
    assert lib.sp_version() >= 100


def test_validation_returns_before_launch(lib):
    """Invalid requests are refused on the host; nothing is launched (null
    pointers would fault if anything were)."""
    from sequence_attention_video_amd import binding as b
    S, A = b.ShardStrides, b.AttnStrides
    nul = (ctypes.c_void_p * 3)(None, None, None)
    # relayout: T_pad not divisible by W -> NOT_DIVISIBLE (checked before pointers)
    assert lib.sp_relayout_heads(nul, nul, 3, 8, 1, 6150, 32, 128, b.SP_BF16, b.SP_TOKENS_TO_HEADS,
                                 S(0, 0), S(0, 0), None) == b.SP_ERR_NOT_DIVISIBLE
    # H not divisible by W
    assert lib.sp_relayout_heads(nul, nul, 3, 8, 1, 6152, 30, 128, b.SP_BF16, b.SP_TOKENS_TO_HEADS,
                                 S(0, 0), S(0, 0), None) == b.SP_ERR_INVALID_ARG
    # null tensors
    assert lib.sp_relayout_heads(nul, nul, 3, 8, 1, 6152, 32, 128, b.SP_BF16, b.SP_TOKENS_TO_HEADS,
                                 S(0, 0), S(0, 0), None) == b.SP_ERR_INVALID_ARG
    # n_tensors out of range
    assert lib.sp_relayout_heads(nul, nul, 4, 8, 1, 6152, 32, 128, b.SP_BF16, b.SP_TOKENS_TO_HEADS,
                                 S(0, 0), S(0, 0), None) == b.SP_ERR_INVALID_ARG
    # pad: T_pad < T, unpaired pointers
    assert lib.sp_pad(None, 0, None, 1, 10, 8, 64, b.SP_BF16, None, None, None) == b.SP_ERR_INVALID_ARG
    assert lib.sp_pad(ctypes.c_void_p(16), 640, None, 1, 10, 12, 64, b.SP_BF16, None, None, None) == b.SP_ERR_INVALID_ARG
    # attention: unsupported head dim, negative kv_valid_len, missing workspace for a mask
    z = A(0, 0, 0, 0)
    assert lib.sp_masked_attention(None, z, None, z, None, z, None, z, 1, 1, 64, 64, 1, 96, b.SP_BF16, 64,
                                   None, 0, 0.1, None, 0, None) == b.SP_ERR_UNSUPPORTED
    # bf16 at D = 16 is supported (float32 MFMA on widened values): refused here
    # only for its null tensors
    assert lib.sp_masked_attention(None, z, None, z, None, z, None, z, 1, 1, 64, 64, 1, 16, b.SP_BF16, 64,
                                   None, 0, 0.1, None, 0, None) == b.SP_ERR_INVALID_ARG
    assert lib.sp_masked_attention(None, z, None, z, None, z, None, z, 1, 1, 64, 64, 1, 128, b.SP_BF16, -1,
                                   None, 0, 0.1, None, 0, None) == b.SP_ERR_INVALID_ARG
    assert lib.sp_masked_attention(None, z, None, z, None, z, None, z, 1, 1, 64, 64, 1, 128, b.SP_BF16, 64,
                                   None, 0, 0.1, None, 0, None) == b.SP_ERR_INVALID_ARG
    # bf16 K/V token strides beyond the kernel's 32-bit tile offsets; a user
    # mask over more key tiles than the kernel keeps in LDS (4096 x 64 keys).
    # Fake, far-apart 16-byte aligned addresses: validation fails before any launch.
    qa, ka, va, oa = (ctypes.c_void_p(x << 40) for x in (1, 2, 3, 4))
    st = A(0, 0, 512, 128)
    big = A(0, 0, 9_000_000, 128)
    assert lib.sp_masked_attention(qa, st, ka, big, va, st, oa, st, 1, 1, 64, 64, 4, 128, b.SP_BF16, 64,
                                   None, 0, 0.1, None, 0, None) == b.SP_ERR_UNSUPPORTED
    tk = 4096 * 64 + 1
    assert lib.sp_masked_attention(qa, st, ka, st, va, st, oa, st, 1, 1, 64, tk, 4, 128, b.SP_BF16, tk,
                                   ctypes.c_void_p(5 << 40), 0, 0.1, None, 0, None) == b.SP_ERR_UNSUPPORTED
    # a user mask beyond the classifier's grid: more than 65535 batches with
    # per-batch masks, or more than 65535 class-tile rows of queries
    wsp = ctypes.c_void_p(6 << 40)
    nb = 65536
    bst = A(0, 64 * 4 * 128, 512, 128)
    need = lib.sp_masked_attention_workspace_size(1, nb, 64, 64, 4, 128, b.SP_BF16, 1, 64 * 64)
    assert lib.sp_masked_attention(qa, bst, ka, bst, va, bst, oa, bst, 1, nb, 64, 64, 4, 128, b.SP_BF16, 64,
                                   ctypes.c_void_p(5 << 40), 64 * 64, 0.1, wsp, need, None) == b.SP_ERR_UNSUPPORTED
    tq = 65536 * 384
    need = lib.sp_masked_attention_workspace_size(1, 1, tq, 64, 4, 128, b.SP_BF16, 1, 0)
    assert lib.sp_masked_attention(qa, st, ka, st, va, st, oa, st, 1, 1, tq, 64, 4, 128, b.SP_BF16, 64,
                                   ctypes.c_void_p(5 << 40), 0, 0.1, wsp, need, None) == b.SP_ERR_UNSUPPORTED
    # empty problems are a no-op success
    assert lib.sp_masked_attention(None, z, None, z, None, z, None, z, 1, 1, 0, 64, 1, 128, b.SP_BF16, 64,
                                   None, 0, 0.1, None, 0, None) == b.SP_OK
    # gather: counts inconsistent with T, count above Ts
    c = (ctypes.c_int64 * 2)(3, 2)
    assert lib.sp_gather_unpad(None, S(0, 0), None, 2, 1, 3, 64, c, 6, b.SP_BF16, None) == b.SP_ERR_INVALID_ARG
    c = (ctypes.c_int64 * 2)(4, 2)
    assert lib.sp_gather_unpad(None, S(0, 0), None, 2, 1, 3, 64, c, 5, b.SP_BF16, None) == b.SP_ERR_INVALID_ARG


def test_attention_scale_must_be_positive_and_normal(lib):
    """The kernels hide a key with a -inf raw score and take the row maximum of
    raw scores before scaling, so only a positive, finite, normal scale (and
    scale * log2 e) is accepted; the rest are refused before any launch
    (these fake pointers would fault if anything ran)."""
    from sequence_attention_video_amd import binding as b
    A = b.AttnStrides
    qa, ka, va, oa = (ctypes.c_void_p(x << 40) for x in (1, 2, 3, 4))
    st = A(0, 0, 512, 128)
    for scale in (0.0, -0.0, -0.088, float("nan"), float("inf"), -float("inf"), 1e-40, 1e-45):
        for dt, d in ((b.SP_BF16, 128), (b.SP_BF16, 64), (b.SP_F32, 16), (b.SP_BF16, 16)):
            got = lib.sp_masked_attention(qa, st, ka, st, va, st, oa, st, 1, 1, 64, 64, 4, d, dt, 64,
                                          None, 0, scale, None, 0, None)
            assert got == b.SP_ERR_INVALID_ARG, (scale, dt, d, got)
    with pytest.raises(ValueError):
        b.check(lib.sp_masked_attention(qa, st, ka, st, va, st, oa, st, 1, 1, 64, 64, 4, 128, b.SP_BF16, 64,
                                        None, 0, 0.0, None, 0, None))


def test_pad_mask_alignment_and_shapes(lib):
    """sp_pad reads the input mask as 4-byte words from its first byte on, so
    a mask_in that is not 4-byte aligned is refused, as is a mask_out that is
    not 16-byte aligned (host checks, no launch)."""
    from sequence_attention_video_amd import binding as b
    base_in, base_out = 1 << 40, 1 << 41
    for off in (1, 2, 3):
        assert lib.sp_pad(None, 0, None, 1, 6, 8, 0, b.SP_BF16, ctypes.c_void_p(base_in + off),
                          ctypes.c_void_p(base_out), None) == b.SP_ERR_INVALID_ARG
    assert lib.sp_pad(None, 0, None, 1, 6, 8, 0, b.SP_BF16, ctypes.c_void_p(base_in),
                      ctypes.c_void_p(base_out + 4), None) == b.SP_ERR_INVALID_ARG
    # the binding checks the mask shapes against B, T and T_pad before the call:
    # a (1, T, T) mask shared by every batch is extended on its own, never
    # with B > 1 token tensors
    class FakeCuda:
        def __init__(self, shape):
            self.shape = shape
            self.is_cuda = True

        def is_contiguous(self):
            return True

    with pytest.raises(ValueError):
        b.sp_pad(None, None, 8, mask_in=FakeCuda((1, 6, 6)), mask_out=FakeCuda((1, 8, 7)))
    with pytest.raises(ValueError):
        b.sp_pad(None, None, 8, mask_in=FakeCuda((1, 6, 6)), mask_out=None)


def test_fused_moves_validation(lib):
    """Argument checks of pad + send_recv_heads and gather_heads +
    gather_output_tokens as single moves (all rejected, or nothing to move,
    before any launch)."""
    from sequence_attention_video_amd import binding as b
    S = b.ShardStrides
    vp = ctypes.c_void_p
    src = (vp * 3)(vp(1 << 40), vp((1 << 40) + (1 << 32)), vp((1 << 40) + (2 << 32)))
    dst = (vp * 3)(vp(1 << 41), vp((1 << 41) + (1 << 32)), vp((1 << 41) + (2 << 32)))
    H, D, T, Tp, W = 32, 128, 6150, 6152, 8
    hs = S(Tp * 4 * D, Tp * 4 * D)
    pr = lib.sp_pad_relayout_heads
    # T_pad not a multiple of W; T_pad < T; H not divisible by W
    assert pr(src, dst, 3, W, 1, T, 6150, H, D, b.SP_BF16, T * H * D, hs, None) == b.SP_ERR_NOT_DIVISIBLE
    assert pr(src, dst, 3, W, 1, T, 6144, H, D, b.SP_BF16, T * H * D, hs, None) == b.SP_ERR_INVALID_ARG
    assert pr(src, dst, 3, W, 1, T, Tp, 12, D, b.SP_BF16, T * 12 * D, hs, None) == b.SP_ERR_INVALID_ARG
    # tensor count, null array, source batch stride below T*H*D, misaligned source
    assert pr(src, dst, 4, W, 1, T, Tp, H, D, b.SP_BF16, T * H * D, hs, None) == b.SP_ERR_INVALID_ARG
    assert pr(None, dst, 3, W, 1, T, Tp, H, D, b.SP_BF16, T * H * D, hs, None) == b.SP_ERR_INVALID_ARG
    assert pr(src, dst, 3, W, 2, T, Tp, H, D, b.SP_BF16, T * H * D - 8, hs, None) == b.SP_ERR_INVALID_ARG
    src_bad = (vp * 3)(vp((1 << 40) + 8), src[1], src[2])
    assert pr(src_bad, dst, 3, W, 1, T, Tp, H, D, b.SP_BF16, T * H * D, hs, None) == b.SP_ERR_INVALID_ARG
    # a destination overlapping a source; head blocks overlapping each other
    dst_bad = (vp * 3)(vp((1 << 40) + 4096), dst[1], dst[2])
    assert pr(src, dst_bad, 3, W, 1, T, Tp, H, D, b.SP_BF16, T * H * D, hs, None) == b.SP_ERR_INVALID_ARG
    assert pr(src, dst, 3, W, 2, T, Tp, H, D, b.SP_BF16, T * H * D, S(Tp * 4 * D, 100), None) == \
        b.SP_ERR_INVALID_ARG
    # a head group that is not whole 16-byte vectors; nothing to move
    assert pr(src, dst, 1, W, 1, 50, 56, 8, 1, b.SP_F32, 50 * 8, S(56, 56), None) == b.SP_ERR_UNSUPPORTED
    assert pr(src, dst, 3, W, 0, T, Tp, H, D, b.SP_BF16, T * H * D, hs, None) == b.SP_OK

    gu = lib.sp_gather_heads_unpad
    c = lambda *v: (ctypes.c_int64 * len(v))(*v)
    assert gu(src, dst, 1, W, 1, 6150, H, D, b.SP_BF16, hs, None, T, None) == b.SP_ERR_NOT_DIVISIBLE
    # a count above Ts; counts summing to less than T; W above 128 ranks
    assert gu(src, dst, 1, W, 1, Tp, H, D, b.SP_BF16, hs, c(770, 769, 769, 769, 769, 769, 769, 769), T, None) == \
        b.SP_ERR_INVALID_ARG
    assert gu(src, dst, 1, W, 1, Tp, H, D, b.SP_BF16, hs, c(769, 769, 769, 769, 769, 769, 769, 766), T, None) == \
        b.SP_ERR_INVALID_ARG
    assert gu(src, dst, 1, 256, 1, 256 * 4, 256, 16, b.SP_BF16, S(1024 * 16, 1024 * 16), None, 1000, None) == \
        b.SP_ERR_UNSUPPORTED
    assert gu(None, dst, 1, W, 1, Tp, H, D, b.SP_BF16, hs, None, T, None) == b.SP_ERR_INVALID_ARG
    dst_bad = (vp * 3)(vp((1 << 40) + 4096), dst[1], dst[2])
    assert gu(src, dst_bad, 1, W, 1, Tp, H, D, b.SP_BF16, hs, None, T, None) == b.SP_ERR_INVALID_ARG
    assert gu(src, dst, 1, W, 1, Tp, H, D, b.SP_BF16, hs, None, 0, None) == b.SP_OK


def test_noalloc_host_checks(lib):
    """sp_masked_attention_noalloc checks its arguments like
    sp_masked_attention, and refuses a request whose workspace exceeds its
    fixed scratch with SP_ERR_SCRATCH, all before any HIP call (fake
    pointers: anything launched would fault)."""
    from sequence_attention_video_amd import binding as b
    A = b.AttnStrides
    qa, ka, va, oa, ma = (ctypes.c_void_p(x << 40) for x in (1, 2, 3, 4, 5))
    st = A(0, 0, 512, 128)
    na = lib.sp_masked_attention_noalloc
    assert na(None, st, None, st, None, st, None, st, 1, 1, 64, 64, 4, 128, b.SP_BF16, 64, None, 0, 0.1,
              None) == b.SP_ERR_INVALID_ARG
    assert na(qa, st, ka, st, va, st, oa, st, 1, 1, 64, 64, 4, 96, b.SP_BF16, 64, None, 0, 0.1,
              None) == b.SP_ERR_UNSUPPORTED
    assert na(qa, st, ka, st, va, st, oa, st, 1, 1, 64, 64, 4, 128, b.SP_BF16, 64, None, 0, 0.0,
              None) == b.SP_ERR_INVALID_ARG
    assert na(qa, st, ka, st, va, st, oa, st, 1, 1, 0, 64, 4, 128, b.SP_BF16, 64, None, 0, 0.1, None) == b.SP_OK
    T = 40000
    s1 = A(0, 0, 128, 128)
    assert lib.sp_masked_attention_workspace_size(1, 1, T, T, 1, 128, b.SP_BF16, 1, 0) > b.SP_NOALLOC_SCRATCH_BYTES
    assert na(qa, s1, ka, s1, va, s1, oa, s1, 1, 1, T, T, 1, 128, b.SP_BF16, T, ma, 0, 0.088,
              None) == b.SP_ERR_SCRATCH
    assert lib.sp_status_string(b.SP_ERR_SCRATCH).startswith(b"SP_ERR_SCRATCH")
    with pytest.raises(ValueError):
        b.check(b.SP_ERR_SCRATCH)


def test_workspace_size(lib):
    from sequence_attention_video_amd import binding as b
    # one class byte per (384-row, 64-key) tile of the mask (17 x 97 of them),
    # padded to 256 bytes, then one 64-bit word per mask row and 64-key tile
    assert b.sp_masked_attention_workspace_size(8, 1, 6152, 6152, 4, 128, b.SP_BF16, True, 0) == \
        1792 + 6152 * 97 * 8
    assert b.sp_masked_attention_workspace_size(1, 2, 300, 128, 4, 64, b.SP_BF16, True, 300 * 128) == \
        256 + 2 * 300 * 2 * 8
    # Without a mask the workspace holds the partial records of split launches:
    # one rank's share of the 6144-token video workload (64 query tiles of 48
    # key tiles) splits over the 256 CUs (assumed when no GPU can be queried):
    # two records per workgroup, each 384 rows of O/l in bf16 (128 values)
    # and m, l in float32.
    rec128 = 384 * (128 * 2 + 8)
    assert b.sp_masked_attention_workspace_size(1, 1, 6144, 6144, 4, 128, b.SP_BF16, False, 0) == \
        2 * 256 * rec128
    # all eight shares fill the GPU evenly (512 query tiles, two per CU); the
    # cross share's 8 key tiles are too few to pay for the merge; the fp32
    # kernel never splits
    assert b.sp_masked_attention_workspace_size(8, 1, 6144, 6144, 4, 128, b.SP_BF16, False, 0) == 0
    assert b.sp_masked_attention_workspace_size(1, 1, 6144, 1024, 4, 64, b.SP_BF16, False, 0) == 0
    assert b.sp_masked_attention_workspace_size(1, 1, 6144, 6144, 4, 64, b.SP_F32, False, 0) == 0
    # Past whole rounds of the GPU only the rest of the query tiles can split.
    # 544 query tiles of 49 key tiles: two whole rounds, then 32 tiles that
    # take one more round of 49 tile-times unsplit against ranges of 7 (+ 4
    # for the records and the merge) split, so eight shares of the
    # 6152-token workload split when no user mask makes the tiles' costs uneven
    assert b.sp_masked_attention_workspace_size(8, 1, 6152, 6152, 4, 128, b.SP_BF16, False, 0) == \
        2 * 256 * rec128
    # the long_hires share, 688 query tiles of 256 key tiles: two whole
    # rounds, then 176 tiles: 256 tile-times unsplit against 176 + 4 split
    assert b.sp_masked_attention_workspace_size(1, 2, 32768, 32768, 4, 128, b.SP_BF16, False, 0) == \
        2 * 256 * rec128
    # all eight shares of it, 5504 query tiles: 21 whole rounds, then 128
    # tiles: 256 tile-times unsplit against 128 + 4 split
    assert b.sp_masked_attention_workspace_size(8, 2, 32768, 32768, 4, 128, b.SP_BF16, False, 0) == \
        2 * 256 * rec128
    # a whole number of rounds never splits: 1024 query tiles
    assert b.sp_masked_attention_workspace_size(16, 1, 6144, 6144, 4, 128, b.SP_BF16, False, 0) == 0


def test_fast_division_host_twin(tmp_path):
    """The multiply-high division used by the relayout kernel, exhaustively on
    small values and on sampled large ones, against plain integer division."""
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    src = tmp_path / "fd.cpp"
    src.write_text(r"""
#include "sp_fastdiv.h"
#include <cstdio>
#include <cstdint>
#include <initializer_list>
int main() {
  uint64_t bad = 0, x = 88172645463325252ull;
  for (uint32_t d = 1; d < 2000; ++d) {
    sp::FastDiv f = sp::make_fastdiv(d);
    for (uint32_t n = 0; n < 5000; ++n) bad += sp::fdiv_host(n, f) != n / d;
    for (int i = 0; i < 2000; ++i) {
      x ^= x << 13; x ^= x >> 7; x ^= x << 17;
      uint32_t n = uint32_t(x);
      bad += sp::fdiv_host(n, f) != n / d;
    }
    bad += sp::fdiv_host(0xffffffffu, f) != 0xffffffffu / d;
  }
  const uint32_t big[] = {65536u, 65537u, 1u << 31, (1u << 31) + 1, 0xfffffffeu, 0xffffffffu, 3000000019u};
  for (uint32_t d : big) {
    sp::FastDiv f = sp::make_fastdiv(d);
    for (uint32_t n : {0u, 1u, d - 1, d, d + 1, 0xffffffffu, 0x80000000u}) bad += sp::fdiv_host(n, f) != n / d;
  }
  printf("%llu\n", (unsigned long long)bad);
  return bad != 0;
}
""")
    exe = tmp_path / "fd"
    subprocess.run([gxx, "-O2", "-std=c++17", "-I", os.path.join(ROOT, "sequence_attention_video_amd", "csrc"),
                    str(src), "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0 and res.stdout.strip() == "0", res.stdout


def test_mask_bit_packing_host_twin(tmp_path):
    """The byte-to-bit packing of the mask classifier against a byte-by-byte
    loop.  Bytes cannot carry into each other (each adds at most 0x7f to its
    low 7 bits), so every value of each byte against a set of values of the
    other three covers the 32-bit packing; sampled 64-bit inputs check the
    two halves' placement."""
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    src = tmp_path / "bits.cpp"
    src.write_text(r"""
#include "sp_bits.h"
#include <cstdio>
#include <cstdint>
static uint64_t slow(uint64_t x, int n) {
  uint64_t r = 0;
  for (int j = 0; j < n; ++j) r |= uint64_t(((x >> (8 * j)) & 0xff) != 0) << j;
  return r;
}
int main() {
  uint64_t bad = 0, x = 88172645463325252ull;
  const uint32_t others[] = {0, 1, 2, 0x40, 0x7f, 0x80, 0x81, 0xfe, 0xff};
  for (int pos = 0; pos < 4; ++pos)
    for (uint32_t v = 0; v < 256; ++v)
      for (uint32_t a : others) for (uint32_t b : others) for (uint32_t c : others) {
        const uint32_t o[3] = {a, b, c};
        uint32_t w = 0;
        for (int q = 0, k = 0; q < 4; ++q) w |= (q == pos ? v : o[k++]) << (8 * q);
        bad += sp::nonzero_bytes_to_bits4(w) != slow(w, 4);
      }
  for (int i = 0; i < 1000000; ++i) {
    x ^= x << 13; x ^= x >> 7; x ^= x << 17;
    uint64_t y = x & (x >> 3) & (x >> 5);   // sparse bytes: many zero bytes
    bad += sp::nonzero_bytes_to_bits8(x) != slow(x, 8);
    bad += sp::nonzero_bytes_to_bits8(y) != slow(y, 8);
  }
  printf("%llu\n", (unsigned long long)bad);
  return bad != 0;
}
""")
    exe = tmp_path / "bits"
    subprocess.run([gxx, "-O2", "-std=c++17", "-I", os.path.join(ROOT, "sequence_attention_video_amd", "csrc"),
                    str(src), "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0 and res.stdout.strip() == "0", res.stdout


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus N > 1 exits with a message (no GPU touched)."""
    import sys
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_optimal_split_matches_oracle(lib):
    """The library's near-square split (host code) against the oracle's, over
    every rank count up to 16 and small grids, errors included."""
    import oracle as O
    from sequence_attention_video_amd import binding as b
    for n in range(1, 17):
        for h in range(1, 13):
            for w in range(1, 13):
                try:
                    want = O.get_optimal_split(n, h, w)
                except ValueError:
                    want = None
                if want is None:
                    with pytest.raises(ValueError):
                        b.sp_optimal_split(n, h, w)
                else:
                    assert b.sp_optimal_split(n, h, w) == want, (n, h, w)
    assert b.sp_optimal_split(8, 16, 24) == (2, 4)
    assert b.sp_optimal_split(8, 64, 64) == (2, 4)
    assert lib.sp_optimal_split(0, 4, 4, None, None) == b.SP_ERR_INVALID_ARG


def test_tile_2d_validation(lib):
    from sequence_attention_video_amd import binding as b
    S = b.ShardStrides
    C = 4096
    src, dst = ctypes.c_void_p(1 << 40), ctypes.c_void_p(2 << 40)
    st = S(6144 * C, 768 * C)
    # height not divisible by split_h
    assert lib.sp_tile_2d(src, dst, 3, 4, 1, 16, 16, 24, C, b.SP_BF16, b.SP_GRID_TO_TILES, st, 6144 * C,
                          None) == b.SP_ERR_NOT_DIVISIBLE
    # row not a multiple of 16 bytes; bad direction; overlapping sides; null pointer
    assert lib.sp_tile_2d(src, dst, 2, 4, 1, 16, 16, 24, 3, b.SP_BF16, b.SP_GRID_TO_TILES, S(768 * 3, 768 * 3),
                          6144 * 3, None) == b.SP_ERR_UNSUPPORTED
    assert lib.sp_tile_2d(src, dst, 2, 4, 1, 16, 16, 24, C, b.SP_BF16, 7, st, 6144 * C, None) == b.SP_ERR_INVALID_ARG
    assert lib.sp_tile_2d(src, ctypes.c_void_p((1 << 40) + 4096), 2, 4, 1, 16, 16, 24, C, b.SP_BF16,
                          b.SP_GRID_TO_TILES, st, 6144 * C, None) == b.SP_ERR_INVALID_ARG
    assert lib.sp_tile_2d(None, dst, 2, 4, 1, 16, 16, 24, C, b.SP_BF16, b.SP_GRID_TO_TILES, st, 6144 * C,
                          None) == b.SP_ERR_INVALID_ARG
    # tile blocks that overlap each other; grid batch stride too small
    assert lib.sp_tile_2d(src, dst, 2, 4, 2, 16, 16, 24, C, b.SP_BF16, b.SP_GRID_TO_TILES, S(768 * C, 100),
                          6144 * C, None) == b.SP_ERR_INVALID_ARG
    assert lib.sp_tile_2d(src, dst, 2, 4, 2, 16, 16, 24, C, b.SP_BF16, b.SP_GRID_TO_TILES, S(2 * 768 * C, 768 * C),
                          6000 * C, None) == b.SP_ERR_INVALID_ARG
    # nothing to copy is a no-op
    assert lib.sp_tile_2d(None, None, 2, 4, 0, 16, 16, 24, C, b.SP_BF16, b.SP_GRID_TO_TILES, st, 6144 * C,
                          None) == b.SP_OK


def test_tile_2d_relayout_heads_validation(lib):
    """Argument checks of the fused 2-D split + head exchange (host only: every
    call here is rejected, or has nothing to move, before any launch)."""
    from sequence_attention_video_amd import binding as b
    S = b.ShardStrides
    vp = ctypes.c_void_p
    src = (vp * 3)(vp(1 << 40), vp((1 << 40) + (1 << 32)), vp((1 << 40) + (2 << 32)))
    dst = (vp * 3)(vp(1 << 41), vp((1 << 41) + (1 << 32)), vp((1 << 41) + (2 << 32)))
    H, D, T = 32, 128, 6144
    hs = S(T * 4 * D, T * 4 * D)
    call = lambda *a: lib.sp_tile_2d_relayout_heads(*a)
    # 16 x 24 does not split into 3 x 4 rank rows; H not divisible by the 8 ranks
    assert call(src, dst, 3, 3, 4, 1, 16, 16, 24, H, D, b.SP_BF16, b.SP_TOKENS_TO_HEADS, T * H * D, hs,
                None) == b.SP_ERR_NOT_DIVISIBLE
    assert call(src, dst, 3, 2, 4, 1, 16, 16, 24, 12, D, b.SP_BF16, b.SP_TOKENS_TO_HEADS, T * 12 * D, hs,
                None) == b.SP_ERR_INVALID_ARG
    # bad tensor count, bad direction, null array, grid batch stride too small
    assert call(src, dst, 4, 2, 4, 1, 16, 16, 24, H, D, b.SP_BF16, b.SP_TOKENS_TO_HEADS, T * H * D, hs,
                None) == b.SP_ERR_INVALID_ARG
    assert call(src, dst, 3, 2, 4, 1, 16, 16, 24, H, D, b.SP_BF16, 5, T * H * D, hs, None) == b.SP_ERR_INVALID_ARG
    assert call(None, dst, 3, 2, 4, 1, 16, 16, 24, H, D, b.SP_BF16, b.SP_TOKENS_TO_HEADS, T * H * D, hs,
                None) == b.SP_ERR_INVALID_ARG
    assert call(src, dst, 3, 2, 4, 1, 16, 16, 24, H, D, b.SP_BF16, b.SP_TOKENS_TO_HEADS, T * H * D - 8, hs,
                None) == b.SP_ERR_INVALID_ARG
    # a destination overlapping a source; head blocks that overlap each other
    dst_bad = (vp * 3)(vp((1 << 40) + 4096), dst[1], dst[2])
    assert call(src, dst_bad, 3, 2, 4, 1, 16, 16, 24, H, D, b.SP_BF16, b.SP_TOKENS_TO_HEADS, T * H * D, hs,
                None) == b.SP_ERR_INVALID_ARG
    assert call(src, dst, 3, 2, 4, 2, 16, 16, 24, H, D, b.SP_BF16, b.SP_TOKENS_TO_HEADS, T * H * D,
                S(T * 4 * D, 100), None) == b.SP_ERR_INVALID_ARG
    # a head group of 2 x 1 fp32 values is not a whole 16-byte vector
    assert call(src, dst, 1, 2, 4, 1, 16, 16, 24, 16, 1, b.SP_F32, b.SP_TOKENS_TO_HEADS, T * 16, S(T * 2, T * 2),
                None) == b.SP_ERR_UNSUPPORTED
    # nothing to move is a no-op
    assert call(src, dst, 3, 2, 4, 0, 16, 16, 24, H, D, b.SP_BF16, b.SP_HEADS_TO_TOKENS, T * H * D, hs,
                None) == b.SP_OK


def test_header_is_plain_c_and_links(tmp_path):
    """include/sp.h compiles as C99 with every warning an error, and a C
    program linked against libspattn.so runs the host-only entry points
    (partition, optimal split, status strings, host-side argument checks)."""
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.exists(LIB):
        pytest.skip("gcc or the built library is missing")
    exe = tmp_path / "c_consumer"
    src = os.path.join(ROOT, "tests", "c_consumer.c")
    libdir = os.path.dirname(LIB)
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"), src,
           "-L", libdir, "-lspattn", "-Wl,-rpath," + libdir, "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stderr
    assert "c consumer ok" in run.stdout
