"""The byte figures the pages print, reproduced by the oracle's accounting.

Fixture: tests/golden/page_numbers.json (each entry cites its page and section).
CPU only.
"""
import json
import os

import numpy as np

import oracle as O

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


def test_bytes_per_token_formula_values():
    for e in GOLDEN["kv_bytes_per_token"]:
        assert O.kv_bytes_fp16_per_token(e["n_layers"], e["n_kv_heads"], e["head_dim"], e["bytes_per_elem"]) == e["bytes"]


def test_total_bytes_values():
    a, b = GOLDEN["kv_bytes_total"]
    tot = O.kv_bytes_fp16_per_token(a["n_layers"], a["n_kv_heads"], a["head_dim"], a["bytes_per_elem"]) * a["n_tokens"]
    assert tot == a["bytes"] and round(tot / 2 ** 30, 1) == a["gib"]
    tot = O.kv_bytes_fp16_per_token(b["n_layers"], b["n_kv_heads"], b["head_dim"], b["bytes_per_elem"]) * b["n_tokens"]
    assert round(tot / 2 ** 30, 3) == b["gib_rounded_3"]


def _packed_bytes_per_token(n_layers, n_kv_heads, bits, n_tokens=4):
    """Decode bytes of a packed cache with every unit at `bits`, per token, summed over segments."""
    lay = O.Layout(1, 1, 1, 1, 128, n_tokens, 16 * n_tokens, 2048, 1)
    r = np.random.default_rng(0)
    K = r.standard_normal((1, 1, 1, n_tokens, 128)).astype(np.float16)
    V = r.standard_normal((1, 1, 1, n_tokens, 128)).astype(np.float16)
    bt = np.full((1, 1, 1, n_tokens), bits, np.uint8)
    bc = np.full((1, 1, 1, 128), bits, np.uint8)
    blob = O.pack_cache(lay, K, V, bt, bc)      # one segment; every (layer, head) is alike
    per_seg_dec = O.segment_decode_bytes(blob, lay, 0, 0)
    per_seg_pay = O.segment_payload_bytes(blob, lay, 0)
    n_seg = n_layers * n_kv_heads
    return per_seg_dec * n_seg / n_tokens, per_seg_pay * n_seg / n_tokens


def test_packed_fp16_cache_moves_exactly_the_printed_bytes_per_token():
    for e in GOLDEN["kv_bytes_per_token"]:
        dec, pay = _packed_bytes_per_token(e["n_layers"], e["n_kv_heads"], 16)
        assert dec == e["bytes"] and pay == e["bytes"]


def test_packed_int4_payload_matches_printed_gib():
    b = GOLDEN["kv_bytes_total"][1]
    _, pay = _packed_bytes_per_token(b["n_layers"], b["n_kv_heads"], 4)
    assert round(pay * b["n_tokens"] / 2 ** 30, 3) == b["gib_rounded_3"]
