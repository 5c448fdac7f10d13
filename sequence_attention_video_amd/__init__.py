"""Ulysses-style sequence-parallel attention hot path, native on MI355X (gfx950).

The compute lives in ``libspattn.so`` (hand-written HIP kernels behind the C ABI
declared in ``include/sp.h``); ``sequence_attention_video_amd.binding`` is a thin
ctypes layer over it with the same entry-point names.  ``workloads`` makes the
seeded synthetic inputs.
"""
