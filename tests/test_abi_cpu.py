"""The C ABI on a machine without a GPU: library loading, exported symbols,
host-side layout arithmetic against the oracle's independent implementation,
and argument validation (every error is returned before anything is enqueued,
so none of these calls reaches the HIP runtime)."""
import ctypes
import os
import re

import pytest

import oracle as O
from decode_attention_rdkv_amd import rdkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rdkv.h")

OK, NULL, SHAPE, UNSUP, BUDGET, ALIGN, WORKSPACE, CAPACITY, HIP, OVERFLOW = range(10)


@pytest.fixture(scope="module")
def lib():
    return rdkv.load()


def test_every_declared_entry_point_is_exported(lib):
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:[a-z_0-9]+\s*\*?\s+)+(rdkv_[a-z_0-9]+)\s*\(", text, re.M))
    assert declared == set(rdkv.SIGNATURES), declared ^ set(rdkv.SIGNATURES)
    for name in declared:
        assert getattr(lib, name) is not None


def test_status_strings(lib):
    for s in range(10):
        assert lib.rdkv_status_string(s) != b"unknown status"
    assert lib.rdkv_status_string(10) == b"unknown status"
    assert lib.rdkv_version() >> 16 == O.VERSION


SHAPES = [
    # (S, L, Hq, Hkv, N, budget_v, budget_k, cap)
    (1, 1, 4, 1, 1024, 4096, 512, 128),
    (1, 1, 32, 8, 32768, 65536, 256, 128),
    (1, 32, 32, 8, 131072, 83886, 81, 128),
    (16, 1, 32, 8, 32768, 98304, 384, 256),
    (1, 80, 64, 8, 262144, 524288, 256, 128),
    (2, 3, 8, 8, 1, 0, 0, 0),
    (1, 1, 2, 1, 77, 10 ** 9, 10 ** 6, 5),
    (3, 2, 16, 2, 1000, 7, 3, 1),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_layout_matches_oracle(shape):
    S, L, Hq, Hkv, N, bv, bk, cap = shape
    lay = rdkv.layout(rdkv.make_dims(S, L, Hq, Hkv, N), bv, bk, cap)
    ol = O.Layout(S, L, Hq, Hkv, 128, N, bv, bk, cap)
    assert lay.n_seg == ol.n_seg
    assert lay.nk_max == ol.nk_max
    assert lay.rec_max == ol.rec_max
    assert lay.slot_bytes == ol.slot_bytes
    assert lay.slots_offset == ol.slots_offset
    assert lay.cache_bytes == ol.cache_bytes
    assert (lay.slot_off_v, lay.slot_off_krec, lay.slot_off_pos) == (ol.off_v, ol.off_krec, ol.off_pos)


def _dims(**kw):
    base = dict(n_seq=1, n_layers=1, n_q_heads=4, n_kv_heads=1, n_tokens=64)
    base.update(kw)
    return rdkv.make_dims(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), UNSUP),
    (dict(n_q_heads=3, n_kv_heads=1), UNSUP),
    (dict(n_q_heads=32, n_kv_heads=1), UNSUP),
    (dict(n_q_heads=6, n_kv_heads=4), SHAPE),
    (dict(n_tokens=0), SHAPE),
    (dict(n_tokens=(1 << 19) + 1), SHAPE),
    (dict(n_seq=0), SHAPE),
])
def test_layout_rejects_bad_dims(lib, kw, status):
    out = rdkv.Layout()
    assert lib.rdkv_layout_init(ctypes.byref(_dims(**kw)), 128, 128, 4, ctypes.byref(out)) == status


def test_layout_rejects_bad_budgets_and_null(lib):
    out = rdkv.Layout()
    d = _dims()
    assert lib.rdkv_layout_init(ctypes.byref(d), -1, 128, 4, ctypes.byref(out)) == BUDGET
    assert lib.rdkv_layout_init(ctypes.byref(d), 128, -1, 4, ctypes.byref(out)) == BUDGET
    assert lib.rdkv_layout_init(ctypes.byref(d), 128, 128, -1, ctypes.byref(out)) == SHAPE
    assert lib.rdkv_layout_init(None, 128, 128, 4, ctypes.byref(out)) == NULL
    assert lib.rdkv_layout_init(ctypes.byref(d), 128, 128, 4, None) == NULL


A = 0x7f0000000000  # a 256-aligned stand-in address; never dereferenced (validation fails first)


def test_score_validation(lib):
    d = _dims()
    ws = lib.rdkv_score_workspace_bytes(ctypes.byref(d))
    assert ws > 0
    assert lib.rdkv_score(ctypes.byref(d), None, A, A, A, A, A, A, ws, None) == NULL
    assert lib.rdkv_score(ctypes.byref(d), A + 8, A, A, A, A, A, A, ws, None) == ALIGN
    assert lib.rdkv_score(ctypes.byref(d), A, A, A, A, A, A, A, ws - 1, None) == WORKSPACE
    assert lib.rdkv_score(ctypes.byref(_dims(head_dim=96)), A, A, A, A, A, A, A, ws, None) == UNSUP


def test_score_halves_validation(lib):
    d = _dims()
    ws = lib.rdkv_score_workspace_bytes(ctypes.byref(d))
    assert lib.rdkv_score_lse(ctypes.byref(d), A, A, None, None) == NULL
    assert lib.rdkv_score_lse(ctypes.byref(d), A, A + 4, A, None) == ALIGN
    assert lib.rdkv_score_lse(ctypes.byref(_dims(head_dim=96)), A, A, A, None) == UNSUP
    assert lib.rdkv_score_from_lse(ctypes.byref(d), A, A, A, None, A, A, A, A, ws, None) == NULL
    assert lib.rdkv_score_from_lse(ctypes.byref(d), A, A, A, A + 8, A, A, A, A, ws, None) == ALIGN
    assert lib.rdkv_score_from_lse(ctypes.byref(d), A, A, A, A, A, A, A, A, ws - 1, None) == WORKSPACE
    assert lib.rdkv_score_from_lse(ctypes.byref(_dims(head_dim=96)), A, A, A, A, A, A, A, A, ws, None) == UNSUP


def test_allocate_validation(lib):
    d = _dims()
    args = [A] * 4
    assert lib.rdkv_allocate(ctypes.byref(d), *args, -5, 8, A, A, A, A, A, 0, None) == BUDGET
    assert lib.rdkv_allocate(ctypes.byref(d), *args, 8, -5, A, A, A, A, A, 0, None) == BUDGET
    assert lib.rdkv_allocate(ctypes.byref(d), *args, 8, 8, A, None, A, A, A, 0, None) == NULL
    assert lib.rdkv_allocate(ctypes.byref(d), *args, 8, 8, A, A, A + 4, A, A, 0, None) == ALIGN
    assert lib.rdkv_allocate(ctypes.byref(d), *args, 8, 8, A, A, A, A, A + 8, 0, None) == ALIGN
    # a problem spread over several workgroups per segment needs the workspace
    big = _dims(n_tokens=100000)
    ws = lib.rdkv_allocate_workspace_bytes(ctypes.byref(big), 1)
    assert ws > 0
    assert lib.rdkv_allocate(ctypes.byref(big), *args, 8, 8, A, A, A, A, None, ws, None) == NULL
    assert lib.rdkv_allocate(ctypes.byref(big), *args, 8, 8, A, A, A, A, A, ws - 1, None) == WORKSPACE


def test_allocate_workspace_size(lib):
    """The size query is 0 for problems of one workgroup each, grows with the
    segments and tokens it covers, and is 0 for a group that does not divide
    the segments."""
    small, mid, big = _dims(n_tokens=1000), _dims(n_tokens=100000), _dims(n_tokens=100000, n_layers=4)
    assert lib.rdkv_allocate_workspace_bytes(ctypes.byref(small), 1) == 0
    assert 0 < lib.rdkv_allocate_workspace_bytes(ctypes.byref(mid), 1) < \
        lib.rdkv_allocate_workspace_bytes(ctypes.byref(big), 1)
    assert lib.rdkv_allocate_workspace_bytes(ctypes.byref(big), 4) > 0
    for g in (0, -1, 3):
        assert lib.rdkv_allocate_workspace_bytes(ctypes.byref(big), g) == 0, g


def test_allocate_shared_validation(lib):
    d = _dims(n_layers=3, n_kv_heads=2)   # 6 segments
    args = lambda g: (ctypes.byref(d), A, A, A, A, 10, 10, g, A, A, A, A, A, 0, None)
    for g in (0, -1, 4, 5, 7):
        assert lib.rdkv_allocate_shared(*args(g)) == SHAPE, g
    assert lib.rdkv_allocate_shared(ctypes.byref(d), None, A, A, A, 10, 10, 1, A, A, A, A, A, 0, None) == NULL
    assert lib.rdkv_allocate_shared(ctypes.byref(d), A, A, A, A, -1, 10, 1, A, A, A, A, A, 0, None) == BUDGET
    big = _dims(n_layers=3, n_kv_heads=2, n_tokens=100000)
    ws3 = lib.rdkv_allocate_workspace_bytes(ctypes.byref(big), 3)
    assert ws3 > 0
    assert lib.rdkv_allocate_shared(ctypes.byref(big), A, A, A, A, 10, 10, 3, A, A, A, A, A, ws3 - 1, None) == WORKSPACE


def test_cache_pack_decode_validation(lib):
    lay = rdkv.layout(_dims(n_layers=2), 64, 32, 4)
    nb = lay.cache_bytes
    ws = lay.decode_workspace_bytes
    assert lib.rdkv_cache_init(ctypes.byref(lay), A, nb - 1, None) == WORKSPACE
    assert lib.rdkv_cache_init(ctypes.byref(lay), A + 2, nb, None) == ALIGN
    assert lib.rdkv_cache_init(ctypes.byref(lay), None, nb, None) == NULL
    bad = rdkv.Layout.from_buffer_copy(lay)
    bad.cache_bytes -= 256                       # not a layout rdkv_layout_init produced
    assert lib.rdkv_cache_init(ctypes.byref(bad), A, nb, None) == SHAPE
    # pack: layer range
    assert lib.rdkv_pack(ctypes.byref(lay), 1, 2, A, A, A, A, A, nb, None) == SHAPE
    assert lib.rdkv_pack(ctypes.byref(lay), -1, 1, A, A, A, A, A, nb, None) == SHAPE
    assert lib.rdkv_pack(ctypes.byref(lay), 0, 0, A, A, A, A, A, nb, None) == SHAPE
    assert lib.rdkv_pack(ctypes.byref(lay), 0, 1, A, A, None, A, A, nb, None) == NULL
    # pack status
    assert lib.rdkv_pack_status(ctypes.byref(lay), A, nb, None, None) == NULL
    assert lib.rdkv_pack_status(ctypes.byref(lay), A + 4, nb, A, None) == ALIGN
    assert lib.rdkv_pack_status(ctypes.byref(lay), A, nb - 1, A, None) == WORKSPACE
    assert lib.rdkv_pack_status(ctypes.byref(bad), A, nb, A, None) == SHAPE
    # decode: zone-C capacity, append pair, workspace
    assert lib.rdkv_decode(ctypes.byref(lay), A, nb, 4, A, A, A, A, A, ws, None) == CAPACITY
    assert lib.rdkv_decode(ctypes.byref(lay), A, nb, 5, A, None, None, A, A, ws, None) == CAPACITY
    assert lib.rdkv_decode(ctypes.byref(lay), A, nb, -1, A, None, None, A, A, ws, None) == CAPACITY
    assert lib.rdkv_decode(ctypes.byref(lay), A, nb, 0, A, A, None, A, A, ws, None) == NULL
    assert lib.rdkv_decode(ctypes.byref(lay), A, nb, 0, A, None, None, A, A, ws - 1, None) == WORKSPACE
    assert lib.rdkv_decode(ctypes.byref(lay), A, nb, 0, A + 8, None, None, A, A, ws, None) == ALIGN
    assert lib.rdkv_unpack(ctypes.byref(lay), A, nb, lay.n_seg, A, A, None) == SHAPE


def test_two_phase_decode_validation(lib):
    lay = rdkv.layout(_dims(n_layers=2), 64, 32, 4)
    nb, ws = lay.cache_bytes, lay.decode_workspace_bytes
    assert lib.rdkv_decode_partials(ctypes.byref(lay), A, nb, 4, A, A, A, A, ws, None) == CAPACITY
    assert lib.rdkv_decode_partials(ctypes.byref(lay), A, nb, 0, None, None, None, A, ws, None) == NULL
    assert lib.rdkv_decode_partials(ctypes.byref(lay), A, nb, 0, A, None, None, A, ws - 16, None) == WORKSPACE
    assert lib.rdkv_decode_merge(ctypes.byref(lay), A, nb, 5, A, A, ws, None) == CAPACITY
    assert lib.rdkv_decode_merge(ctypes.byref(lay), A, nb, -1, A, A, ws, None) == CAPACITY
    assert lib.rdkv_decode_merge(ctypes.byref(lay), A, nb, 0, None, A, ws, None) == NULL
    assert lib.rdkv_decode_merge(ctypes.byref(lay), A, nb, 0, A + 4, A, ws, None) == ALIGN


@pytest.mark.parametrize("shape", [(1, 1, 4, 1, 1024, 4096, 512, 128, 3, 512, 512),
                                   (2, 3, 8, 2, 777, 1500, 300, 64, 5, 128, 256),
                                   (16, 1, 32, 8, 32768, 98304, 384, 256, 2, 768, 384),
                                   (1, 2, 16, 2, 300, 0, 0, 300, 1, 0, 0)])
def test_rollover_layout_matches_oracle(shape):
    S, L, Hq, Hkv, N, bv, bk, cap, n_gen, gbv, gbk = shape
    lay = rdkv.layout_rollover(rdkv.make_dims(S, L, Hq, Hkv, N), bv, bk, cap, n_gen, gbv, gbk)
    ol = O.Layout(S, L, Hq, Hkv, 128, N, bv, bk, cap, n_generations=n_gen, gen_budget_v=gbv, gen_budget_k=gbk)
    plain = rdkv.layout(rdkv.make_dims(S, L, Hq, Hkv, N), bv, bk, cap)
    assert (lay.cache_bytes, lay.gen_offset, lay.gen_bytes) == (ol.cache_bytes, ol.gen_offset, ol.gen_bytes)
    assert lay.slot_bytes == plain.slot_bytes and lay.gen_offset == plain.cache_bytes
    gen = rdkv.layout(rdkv.make_dims(S, L, Hq, Hkv, cap), gbv, gbk, 0)
    assert lay.max_chunks == plain.token_slots + n_gen * gen.max_chunks + -(-cap // 256)
    assert lay.token_slots == plain.token_slots
    assert lay.zc_stats_bytes == S * L * Hkv * (Hq // Hkv) * (cap + 128) * 4
    assert lay.decode_workspace_bytes == S * L * Hkv * lay.max_chunks * (Hq // Hkv) * 132 * 4
    assert lay.rollover_workspace_bytes >= S * L * Hkv * cap * 2 * 256


def test_rollover_validation(lib):
    d = _dims(n_layers=2)
    out = rdkv.Layout()
    assert lib.rdkv_layout_init_rollover(ctypes.byref(d), 64, 32, 4, 0, 8, 8, ctypes.byref(out)) == SHAPE
    assert lib.rdkv_layout_init_rollover(ctypes.byref(d), 64, 32, 0, 2, 8, 8, ctypes.byref(out)) == SHAPE
    assert lib.rdkv_layout_init_rollover(ctypes.byref(d), 64, 32, 4, 2, -1, 8, ctypes.byref(out)) == BUDGET
    assert lib.rdkv_layout_init_rollover(ctypes.byref(d), 64, 32, 4, 5000, 8, 8, ctypes.byref(out)) == SHAPE
    plain = rdkv.layout(d, 64, 32, 4)
    assert plain.n_generations == 0 and plain.zc_stats_bytes == 0 and plain.gen_offset == 0
    lay = rdkv.layout_rollover(d, 64, 32, 4, 2, 8, 8)
    nb, ws, rws = lay.cache_bytes, lay.decode_workspace_bytes, lay.rollover_workspace_bytes
    # decode with accumulation
    assert lib.rdkv_decode_accumulate(ctypes.byref(plain), A, plain.cache_bytes, 0, A, None, None, A, A, A,
                                      plain.decode_workspace_bytes, None) == SHAPE
    assert lib.rdkv_decode_accumulate(ctypes.byref(lay), A, nb, 0, A, None, None, A, None, A, ws, None) == NULL
    assert lib.rdkv_decode_accumulate(ctypes.byref(lay), A, nb, 0, A, None, None, A, A + 4, A, ws, None) == ALIGN
    assert lib.rdkv_decode_accumulate(ctypes.byref(lay), A, nb, 4, A, A, A, A, A, A, ws, None) == CAPACITY
    # scoring and rolling over
    assert lib.rdkv_rollover_score(ctypes.byref(plain), A, plain.cache_bytes, A, A, A, A, None) == SHAPE
    assert lib.rdkv_rollover_score(ctypes.byref(lay), A, nb, A, None, A, A, None) == NULL
    assert lib.rdkv_rollover_score(ctypes.byref(lay), A, nb - 1, A, A, A, A, None) == WORKSPACE
    assert lib.rdkv_rollover(ctypes.byref(lay), A, nb, 2, A, A, rws, None) == CAPACITY
    assert lib.rdkv_rollover(ctypes.byref(lay), A, nb, -1, A, A, rws, None) == CAPACITY
    assert lib.rdkv_rollover(ctypes.byref(lay), A, nb, 0, A, A, rws - 1, None) == WORKSPACE
    assert lib.rdkv_rollover(ctypes.byref(lay), A, nb, 0, None, A, rws, None) == NULL
    assert lib.rdkv_rollover(ctypes.byref(plain), A, plain.cache_bytes, 0, A, A, rws, None) == SHAPE
    bad = rdkv.Layout.from_buffer_copy(lay)
    bad.gen_bytes += 256
    assert lib.rdkv_rollover(ctypes.byref(bad), A, nb, 0, A, A, rws, None) == SHAPE


def test_static_decode_validation(lib):
    """rdkv_decode_static validates like rdkv_decode (minus the workspace) and
    refuses layouts whose split-K partials exceed its static scratch, all
    before touching the device."""
    lay = rdkv.layout(_dims(n_layers=2), 64, 32, 4)
    nb = lay.cache_bytes
    assert lay.decode_workspace_bytes <= rdkv.STATIC_SCRATCH_BYTES
    assert lib.rdkv_decode_static(ctypes.byref(lay), A, nb, 4, A, A, A, A, None) == CAPACITY
    assert lib.rdkv_decode_static(ctypes.byref(lay), A, nb, -1, A, None, None, A, None) == CAPACITY
    assert lib.rdkv_decode_static(ctypes.byref(lay), A, nb, 0, A, A, None, A, None) == NULL
    assert lib.rdkv_decode_static(ctypes.byref(lay), A, nb, 0, A, None, None, None, None) == NULL
    assert lib.rdkv_decode_static(ctypes.byref(lay), None, nb, 0, A, None, None, A, None) == NULL
    assert lib.rdkv_decode_static(ctypes.byref(lay), A, nb, 0, A + 8, None, None, A, None) == ALIGN
    assert lib.rdkv_decode_static(ctypes.byref(lay), A, nb, 0, A, None, None, A + 4, None) == ALIGN
    assert lib.rdkv_decode_static(ctypes.byref(lay), A, nb - 1, 0, A, None, None, A, None) == WORKSPACE
    big = rdkv.layout(rdkv.make_dims(8, 80, 64, 8, 262144), 524288, 256, 128)
    assert big.decode_workspace_bytes > rdkv.STATIC_SCRATCH_BYTES
    assert lib.rdkv_decode_static(ctypes.byref(big), A, big.cache_bytes, 0, A, None, None, A, None) == WORKSPACE
    # the largest workload's partials fit
    c5 = rdkv.layout(rdkv.make_dims(1, 80, 64, 8, 262144), 524288, 256, 128)
    assert c5.decode_workspace_bytes <= rdkv.STATIC_SCRATCH_BYTES


def test_decode_byte_accounting_against_the_oracle_blob():
    """The benchmark's algorithmic bytes per decode step (read from the
    descriptors) equal the oracle's count of payload bits plus one
    (scale, zero) word per quantized V row and per present K part; adding the
    record padding gives exactly the bytes the packed segments hold."""
    import numpy as np
    import torch
    from decode_attention_rdkv_amd import synth
    S, L, Hq, Hkv, N, cap = 1, 2, 4, 2, 300, 3
    bt, bc = synth.random_bits(L * Hkv, N, 5)
    bc[1] = 0
    bc[1, :7] = 2                        # a segment with a single, partly filled 2-bit K part
    bv, bk = int(bt.sum(axis=1).max()), int(bc.sum(axis=1).max())
    ol = O.Layout(S, L, Hq, Hkv, 128, N, bv, bk, cap)
    K, V = synth.random_kv(L * Hkv, N, 6)
    shp = (S, L, Hkv)
    blob = O.pack_cache(ol, K.reshape(shp + (N, 128)), V.reshape(shp + (N, 128)), bt.reshape(shp + (N,)),
                        bc.reshape(shp + (128,)))
    lay = rdkv.layout(rdkv.make_dims(S, L, Hq, Hkv, N), bv, bk, cap)
    desc = rdkv.descriptors(lay, torch.from_numpy(blob))
    n_c = 2
    b = rdkv.decode_bytes(lay, desc, n_c)
    n_seg = L * Hkv
    payload = sum(O.segment_payload_bytes(blob, ol, s) for s in range(n_seg))
    stored = sum(O.segment_decode_bytes(blob, ol, s, n_c) for s in range(n_seg))
    assert abs((b["v"] + b["k"]) - payload) < 1
    n_zone_a = int((bt > 0).sum() - (bt == 16).sum())
    assert b["v_meta"] == 4 * n_zone_a
    kept = (bt > 0).sum(axis=1)
    parts = [sum(int((bc[s] == w).any()) for w in (8, 4, 2)) for s in range(n_seg)]
    assert b["k_meta"] == 4 * int(sum(k * p for k, p in zip(kept, parts)))
    assert b["v"] + b["v_meta"] + b["k"] + b["k_meta"] + b["k_padding"] + b["zone_c"] == stored
    assert b["k_padding"] >= 0
    assert b["total"] == b["v"] + b["v_meta"] + b["k"] + b["k_meta"] + b["zone_c"] + b["q_out"]


@pytest.mark.parametrize("shape", [(16, 1, 32, 8, 32768, 98304, 384, 256, 4096), (4, 2, 8, 2, 333, 900, 512, 40, 300),
                                   (1, 1, 4, 1, 64, 1, 0, 1, 1), (2, 3, 16, 2, 5000, 80000, 2048, 130, 77)])
def test_paged_layout_matches_oracle(shape):
    S, L, Hq, Hkv, N, bv, bk, cap, n_pages = shape
    pl = rdkv.paged_layout(rdkv.make_dims(S, L, Hq, Hkv, N), bv, bk, cap, n_pages)
    op = O.PagedLayout(S, L, Hq, Hkv, N, bv, bk, cap, n_pages)
    assert (pl.max_pages, pl.table_offset, pl.pool_offset, pl.cache_bytes) == \
        (op.max_pages, op.table_offset, op.pool_offset, op.cache_bytes)
    flat = rdkv.layout(rdkv.make_dims(S, L, Hq, Hkv, N), bv, bk, cap)
    assert (pl.rec_max, pl.nk_max) == (flat.rec_max, flat.nk_max)
    # chunk size: the contiguous rule, capped by what the pool can hold (2-bit V rows of 32 bytes)
    t2 = 512
    while t2 < flat.chunk_tok2 and (n_pages * 32768 // 32) // (2 * t2) >= 512:
        t2 *= 2
    assert pl.chunk_tok2 == t2 <= flat.chunk_tok2
    assert pl.token_slots == min(bv // 2, 8 * N) // t2 + 4
    assert pl.max_chunks == pl.token_slots + -(-cap // 256)
    assert pl.decode_workspace_bytes == S * L * Hkv * pl.max_chunks * (Hq // Hkv) * 132 * 4
    if t2 == flat.chunk_tok2:                 # a pool that does not bind chunks like the contiguous layout
        assert (pl.max_chunks, pl.token_slots) == (flat.max_chunks, flat.token_slots)


def test_paged_shape_validation(lib):
    """The decode-shape entry points reject missing arguments, a workspace
    too small for the shape, and a shape outside the layout's bounds, before
    anything is enqueued."""
    d = rdkv.make_dims(3, 2, 8, 2, 300)
    pl = rdkv.paged_layout(d, 600, 256, 32, 50)
    nb, ws = pl.cache_bytes, pl.decode_workspace_bytes
    out = rdkv.LaunchShape()
    assert lib.rdkv_paged_decode_shape(ctypes.byref(pl), None, nb, A, 8, None, ctypes.byref(out)) == NULL
    assert lib.rdkv_paged_decode_shape(ctypes.byref(pl), A, nb, A, 8, None, None) == NULL
    assert lib.rdkv_paged_decode_shape(ctypes.byref(pl), A, nb, A, 4, None, ctypes.byref(out)) == WORKSPACE
    assert lib.rdkv_paged_decode_shape(ctypes.byref(pl), A, nb - 1, A, 8, None, ctypes.byref(out)) == WORKSPACE
    assert lib.rdkv_paged_decode_shape(ctypes.byref(pl), A + 4, nb, A, 8, None, ctypes.byref(out)) == ALIGN
    c_len = (ctypes.c_int32 * 3)(0, 0, 0)

    def shaped(sh, ws_bytes=ws):
        return lib.rdkv_paged_decode_shaped(ctypes.byref(pl), sh, A, nb, c_len, A, None, None, A, A, ws_bytes, None)

    assert shaped(None) == NULL
    G, zc = 4, pl.max_chunks - pl.token_slots
    for ts, rec, res, status in ((pl.token_slots + 1, 0, 0, SHAPE), (-1, 0, 0, SHAPE), (1, pl.rec_max + 4, 0, SHAPE),
                                 (1, 6, 0, SHAPE), (1, 4, 1, SHAPE)):
        sh = rdkv.LaunchShape(ts, rec, ts + zc, res, 0)
        assert shaped(ctypes.byref(sh)) == status, (ts, rec, res)
    # a smaller shape needs a smaller workspace: its own size passes validation
    # (and then fails only at the launch, on a machine without a GPU)
    sh = rdkv.LaunchShape(1, 4, 1 + zc, 0, 0)
    need = pl.n_seg * (1 + zc) * G * 132 * 4
    assert shaped(ctypes.byref(sh), need - 1) == WORKSPACE
    assert shaped(ctypes.byref(sh), need) == HIP


def test_contiguous_shape_validation(lib):
    """rdkv_decode_shape / rdkv_decode_shaped reject missing arguments, a
    short workspace and a shape outside the layout's bounds before anything
    is enqueued; a shape's own workspace size passes validation."""
    lay = rdkv.layout(rdkv.make_dims(1, 2, 8, 2, 3000), 6000, 160, 16)
    nb, ws = lay.cache_bytes, lay.decode_workspace_bytes
    out = rdkv.LaunchShape()
    assert lib.rdkv_decode_shape(ctypes.byref(lay), None, nb, A, 8, None, ctypes.byref(out)) == NULL
    assert lib.rdkv_decode_shape(ctypes.byref(lay), A, nb, A, 7, None, ctypes.byref(out)) == WORKSPACE
    assert lib.rdkv_decode_shape(ctypes.byref(lay), A, nb, A + 8, 8, None, ctypes.byref(out)) == ALIGN

    def shaped(sh, ws_bytes=ws):
        return lib.rdkv_decode_shaped(ctypes.byref(lay), sh, A, nb, 0, A, None, None, A, A, ws_bytes, None)

    assert shaped(None) == NULL
    other = lay.max_chunks - lay.token_slots
    for ts, rec, res in ((lay.token_slots + 1, 0, 0), (1, lay.rec_max + 4, 0), (1, 2, 0), (1, 4, 3)):
        assert shaped(ctypes.byref(rdkv.LaunchShape(ts, rec, ts + other, res, 0))) == SHAPE, (ts, rec, res)
    sh = rdkv.LaunchShape(2, 8, 2 + other, 0, 0)
    need = lay.n_seg * (2 + other) * 4 * 132 * 4
    assert shaped(ctypes.byref(sh), need - 1) == WORKSPACE
    assert shaped(ctypes.byref(sh), need) == HIP


def test_paged_validation(lib):
    d = rdkv.make_dims(3, 2, 8, 2, 300)
    pl = rdkv.paged_layout(d, 600, 256, 32, 50)
    out = rdkv.PagedLayout()
    assert lib.rdkv_paged_layout_init(ctypes.byref(rdkv.make_dims(257, 1, 4, 1, 10)), 10, 10, 4, 5,
                                      ctypes.byref(out)) == SHAPE
    assert lib.rdkv_paged_layout_init(ctypes.byref(d), 600, 256, 32, 0, ctypes.byref(out)) == SHAPE
    nb, ws = pl.cache_bytes, pl.decode_workspace_bytes
    assert lib.rdkv_paged_cache_init(ctypes.byref(pl), A, nb - 1, None) == WORKSPACE
    bad = rdkv.PagedLayout.from_buffer_copy(pl)
    bad.max_pages += 1
    assert lib.rdkv_paged_cache_init(ctypes.byref(bad), A, nb, None) == SHAPE
    # staging: length and budgets within the bounds
    assert lib.rdkv_paged_staging_bytes(ctypes.byref(pl), 301, 100, 100) == 0
    assert lib.rdkv_paged_staging_bytes(ctypes.byref(pl), 300, 601, 100) == 0
    sb = lib.rdkv_paged_staging_bytes(ctypes.byref(pl), 200, 300, 100)
    assert sb == rdkv.layout(rdkv.make_dims(1, 2, 8, 2, 200), 300, 100, 0).cache_bytes
    assert lib.rdkv_paged_stage(ctypes.byref(pl), 200, 300, 100, A, A, A, A, A, sb - 1, A, None) == WORKSPACE
    assert lib.rdkv_paged_stage(ctypes.byref(pl), 200, 300, 257, A, A, A, A, A, sb, A, None) == BUDGET
    assert lib.rdkv_paged_stage(ctypes.byref(pl), 0, 300, 100, A, A, A, A, A, sb, A, None) == SHAPE
    assert lib.rdkv_paged_stage(ctypes.byref(pl), 200, 300, 100, A, A, A, A, A, sb, None, None) == NULL
    assert lib.rdkv_paged_commit(ctypes.byref(pl), 3, 200, 300, 100, A, sb, A, A, nb, None) == SHAPE
    assert lib.rdkv_paged_commit(ctypes.byref(pl), -1, 200, 300, 100, A, sb, A, A, nb, None) == SHAPE
    assert lib.rdkv_paged_commit(ctypes.byref(pl), 0, 200, 300, 100, A, sb, None, A, nb, None) == NULL
    assert lib.rdkv_paged_release(ctypes.byref(pl), 3, A, nb, None) == SHAPE
    c_ok = (ctypes.c_int32 * 3)(0, 5, 31)
    c_full = (ctypes.c_int32 * 3)(0, 32, 1)
    assert lib.rdkv_paged_decode(ctypes.byref(pl), A, nb, c_full, A, A, A, A, A, ws, None) == CAPACITY
    assert lib.rdkv_paged_decode(ctypes.byref(pl), A, nb, c_ok, A, A, None, A, A, ws, None) == NULL
    assert lib.rdkv_paged_decode(ctypes.byref(pl), A, nb, c_ok, A, None, None, A, A, ws - 1, None) == WORKSPACE
    assert lib.rdkv_paged_decode(ctypes.byref(pl), A, nb, None, A, None, None, A, A, ws, None) == NULL
