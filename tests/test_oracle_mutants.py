"""The oracle's pins must catch plausible mistakes.

Each mutant is a one-line change to the oracle's source (a dropped term, a wrong
index or sign, a transposed operand).  The mutated module replaces the oracle for
the duration of one check, and at least one pin of test_oracle.py must fail.
Mistakes are planted in the oracle on the CPU only.
"""
import importlib.util
import os
import re
import sys
import types

import pytest

import oracle
import oracle.kv_oracle as real
from tests import test_oracle as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = open(os.path.join(ROOT, "oracle", "kv_oracle.py")).read()
HEADER = open(os.path.join(ROOT, "include", "kvshare.h")).read()


def test_oracle_layout_is_the_header_formula():
    """The pool map in the oracle is the one the library header documents."""
    k_expr = re.search(r"K\(t, d\) = tile \+ (.+)", HEADER).group(1).strip()
    v_expr = re.search(r"V\(t, d\) = tile \+ 16\*D \+ (.+)", HEADER).group(1).strip()
    tile_expr = re.search(r"tile\(layer, page, head\) = (.+)", HEADER).group(1).strip()
    c_to_py = lambda e: e.replace("/", "//")       # non-negative C integer division
    for D in (64, 128):
        for t in range(16):
            for d in range(D):
                env = {"t": t, "d": d, "D": D}
                assert eval(c_to_py(k_expr), env) == oracle.k_offset(t, d)
                assert eval(c_to_py(v_expr), env) == oracle.v_offset(t, d)
    env = {"layer": 1, "page": 5, "head": 3, "num_pages": 7, "num_kv_heads": 4, "D": 64}
    assert eval(c_to_py(tile_expr), env) == oracle.tile_start(1, 5, 3, 7, 4, 64)


MUTANTS = {
    "gqa_modulo": ("g = h // G", "g = h % G"),
    "causal_without_diagonal": ("attend(q[r, h], K[: p + 1, g], V[: p + 1, g], scale)",
                                "attend(q[r, h], K[:p, g], V[:p, g], scale)"),
    "no_normalisation": ("return (w @ V) / w.sum()", "return (w @ V) / w.size"),
    "keys_as_values": ("return (w @ V) / w.sum()", "return (w @ K) / w.sum()"),
    "scale_dropped": ("s = scale * (K @ q)", "s = K @ q"),
    "gather_wrong_slot": ("        slot = p % PAGE\n        for h in range(H):",
                          "        slot = (p + 1) % PAGE\n        for h in range(H):"),
    "append_wrong_position": ("p = int(seq_lens[b]) + j", "p = int(seq_lens[b]) + j + 1"),
    "bf16_wrong_shift": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "layout_lane_order": ("lane = sub * 16 + t", "lane = t * 4 + sub"),
    "v_layout_run": ("run = (t // 8) * 16 + d % 16", "run = (t // 8) * 16 + d % 8"),
    "v_layout_slab": ("slab = d // 16 ", "slab = d // 32 "),
    "decode_prefix_off_by_one": ("K, V = gather(pool, shape, layer, block_table[b], L)",
                                 "K, V = gather(pool, shape, layer, block_table[b], max(L - 1, 0))"),
    "fetch_v_from_k": ("                V[row, h] = pool[base + vt[slot]]", "                V[row, h] = pool[base + kt[slot]]"),
    "pack_layer_offset": ("base = tile_start(layer_begin + li, int(pid), h, shape.num_pages, H, D)\n                buf[li, i, h]",
                          "base = tile_start(li, int(pid), h, shape.num_pages, H, D)\n                buf[li, i, h]"),
    "unpack_head_order": ("out[base:base + te] = buf[li, i, h]", "out[base:base + te] = buf[li, i, H - 1 - h]"),
    "private_row_order": ("priv_table[b * N + n], int(priv_lens[b * N + n])",
                          "priv_table[n * B + b], int(priv_lens[n * B + b])"),
    "private_suffix_dropped": ("K = np.concatenate([Ks, Kp])\n            V = np.concatenate([Vs, Vp])",
                               "K = Ks\n            V = Vs"),
    "private_prefix_dropped": ("K = np.concatenate([Ks, Kp])\n            V = np.concatenate([Vs, Vp])",
                               "K = Kp\n            V = Vp"),
}

PIN_CHECKS = [
    pins.test_bf16_decoding_known_patterns,
    lambda: pins.test_layout_is_a_bijection_per_tile(64),
    lambda: pins.test_layout_lane_operand_runs(128),
    test_oracle_layout_is_the_header_formula,
    pins.test_append_then_gather_roundtrip,
    pins.test_append_split_equals_one_shot_and_touches_only_its_slots,
    pins.test_tiny_decode_matches_brute_force_over_logical_sequence,
    lambda: pins.test_decode_matches_torch_sdpa([1, 17, 33], 3, 2, 5, 128),
    pins.test_closed_form_single_token_returns_v,
    pins.test_closed_form_zero_query_gives_mean_of_v,
    lambda: pins.test_extend_equals_causal_sdpa_over_whole_sequence([40, 0, 16], [9, 20, 1]),
    pins.test_private_decode_matches_brute_force_over_prefix_then_suffix,
    pins.test_private_suffix_reaches_only_its_decoder,
    pins.test_fetch_returns_the_logical_rows_that_were_appended,
    pins.test_handoff_to_another_pool_preserves_every_session,
    pins.test_pack_of_a_layer_range_is_a_slice_of_the_full_pack,
]


def _mutant_module(old, new):
    assert SRC.count(old) >= 1, f"mutation site not found: {old!r}"
    mod = types.ModuleType("kv_oracle_mutant")
    mod.__file__ = "<mutant>"
    exec(compile(SRC.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    mod = _mutant_module(*MUTANTS[name])
    for attr in ("bf16_to_f64", "k_offset", "v_offset", "tile_start", "append", "gather", "attend",
                 "decode", "decode_private", "extend", "decode_from_logical", "extend_from_logical", "PoolShape",
                 "fetch", "pack", "unpack",
                 "tile_elems", "pool_elems"):
        monkeypatch.setattr(oracle, attr, getattr(mod, attr))
    failed = []
    for check in PIN_CHECKS:
        try:
            check()
        except AssertionError:
            failed.append(check)
        except (IndexError, ValueError):
            failed.append(check)
    assert failed, f"mutant {name} survived every pin"
