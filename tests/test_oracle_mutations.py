"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
at least one pin catches each.  The real oracle is never modified: each mutant
is the oracle's source with one textual change, executed as a fresh module."""

import os
import types

import pytest

from tests import pin_checks as P
from tests.conftest import ROOT

SRC = open(os.path.join(ROOT, "oracle", "sp_oracle.py"), encoding="utf-8").read()

CHECKS = [
    P.check_partition, P.check_padded_length, P.check_pad_tokens, P.check_mask_extension,
    P.check_relayout_golden, P.check_relayout_brute_force, P.check_relayout_round_trip,
    P.check_relayout_shapes, P.check_attention_golden, P.check_attention_brute_force,
    P.check_attention_closed_forms, P.check_garbage_pad_invariance, P.check_gather_output,
    P.check_sharded_equals_unsharded_self, P.check_sharded_equals_unsharded_mask,
    P.check_sharded_equals_unsharded_cross, P.check_attention_sdpa, P.check_cross_query_padding,
    P.check_joint_av_block, P.check_split_2d_golden, P.check_optimal_split, P.check_split_2d_brute_force,
    P.check_sharded_equals_unsharded_2d,
]

MUTANTS = {
    "scale dropped": ("s = (q[i0:i1] @ k.T) * scale", "s = (q[i0:i1] @ k.T)"),
    "wrong operand in PV": ("num = p @ v", "num = p @ k[:, :v.shape[1]]"),
    "key mask off by one": ("key_ok = np.arange(tk) < kv_valid_len",
                            "key_ok = np.arange(tk) <= kv_valid_len"),
    "masked row not zero": ("num / np.where(den > 0, den, 1.0), 0.0)",
                            "num / np.where(den > 0, den, 1.0), 1.0)"),
    "send: rank indices swapped": ("out[r, :, s * ts:(s + 1) * ts] = shards[s, :, :, r * hl:(r + 1) * hl]",
                                   "out[r, :, s * ts:(s + 1) * ts] = shards[r, :, :, s * hl:(s + 1) * hl]"),
    "gather: rank indices swapped": ("out[s, :, :, r * hl:(r + 1) * hl] = heads[r, :, s * ts:(s + 1) * ts]",
                                     "out[s, :, :, r * hl:(r + 1) * hl] = heads[s, :, r * ts:(r + 1) * ts]"),
    "pad rows see pad keys": ("out[:, t:, :t] = 1", "out[:, t:, :] = 1"),
    "pad rows see nothing": ("out[:, t:, :t] = 1", "pass"),
    "pad value not zero": ("y = np.zeros((b, t_pad) + x.shape[2:], dtype=x.dtype)",
                           "y = np.ones((b, t_pad) + x.shape[2:], dtype=x.dtype)"),
    "no trim by count": ("kept.append(gathered[r, :, :counts[r]])", "kept.append(gathered[r])"),
    "divisibility unchecked": ("if total_tokens % world_size != 0:", "if False:"),
    "padded length floors": ("return world_size * (-(-total_tokens // world_size))",
                             "return world_size * (total_tokens // world_size)"),
    "cross: all ranks use the first heads": ("attention_heads(q[:, :, r * hl:(r + 1) * hl], kh[r]",
                                             "attention_heads(q[:, :, 0:hl], kh[r]"),
    "user mask rows/cols transposed": ("out[:, :t, :t] = (m != 0)", "out[:, :t, :t] = (m != 0).transpose(0, 2, 1)"),
    "cross: query padding ignored": ("q = pad_tokens(q, tq_pad)", "q = q"),
    "2-D: ranks numbered column-major": ("r = i * split_w + j\n            grid[", "r = j * split_h + i\n            grid["),
    "2-D: split ratio farthest from square": ("key = (abs(a - b), abs(height // a - width // b), a)",
                                             "key = (-abs(a - b), abs(height // a - width // b), a)"),
    "2-D: tile ignores the frames": ("tile = grid[:, :, i * th:(i + 1) * th, j * tw:(j + 1) * tw]",
                                     "tile = grid[:, :1, i * th:(i + 1) * th, j * tw:(j + 1) * tw]"),
    "joint: cross keys from the wrong modality": ('(("v2a", audio_tokens, ta_pad, tv_pad),',
                                                 '(("v2a", video_tokens, tv_pad, tv_pad),'),
    "row max over every key, hidden ones too": ("m = s.max(axis=1, keepdims=True)",
                                                "m = ((q[i0:i1] @ k.T) * scale).max(axis=1, keepdims=True)"),
    "key padding dropped under a user mask": ("vis = vis & (np.asarray(mask[i0:i1]) != 0)",
                                              "vis = np.asarray(mask[i0:i1]) != 0"),
    "batch 0's mask for every batch": ("mb = mask[bi if mask.shape[0] > 1 else 0][sel]", "mb = mask[0][sel]"),
}


def _mutant(old, new):
    assert SRC.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(*MUTANTS[name])
    caught = []
    for check in CHECKS:
        try:
            check(mod)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((check.__name__, type(e).__name__))
            break
    assert caught, f"mutant '{name}' passed every pin"
