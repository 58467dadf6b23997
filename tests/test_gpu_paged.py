"""Paged zones (a shared pool of fixed-size pages found through a block table
per segment, the aistudio.id article's "Solusi 1") on the GPU against the
oracle, through the C ABI.

Sequences of different prefill lengths and budgets are staged, given pages
by a host allocator that hands them out shuffled (so no segment's pages are
contiguous), committed, decoded with per-sequence zone-C lengths, released
and replaced.  Bars: the whole paged cache byte-equal to the oracle's after
every commit, release and decode step (descriptors, block table, every page);
the page counts the library asks for equal the oracle's; decode outputs within
2e-3; and, for equal-length sequences, the paged decode bit-identical to the
contiguous one.
"""
import numpy as np
import pytest
import torch

import oracle as O
from decode_attention_rdkv_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 2e-3


@pytest.fixture(scope="module")
def rdkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_attention_rdkv_amd import rdkv as lib
    lib.load()
    return lib


def host(t):
    return t.detach().cpu().numpy()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float((np.abs(got - ref).max(axis=-1) / np.maximum(np.abs(ref).max(axis=-1), 1e-30)).max())


class Pool:
    """Host page allocator: a free list handed out in shuffled order."""

    def __init__(self, n, seed):
        self.free = [int(x) for x in np.random.default_rng(seed).permutation(n)]

    def take(self, k):
        assert k <= len(self.free), "pool exhausted"
        out, self.free = self.free[:k], self.free[k:]
        return out

    def give(self, pages):
        self.free = list(pages) + self.free


def _sequence(L, Hkv, N, bv, bk, seed):
    n = L * Hkv
    bt, bc = synth.random_bits(n, N, seed)
    K, V = synth.random_kv(n, N, seed + 1)
    K[..., 5] *= np.float16(6)
    for i in range(n):
        while int(bt[i].astype(np.int64).sum()) > bv:
            bt[i, np.nonzero(bt[i])[0][: max(1, len(np.nonzero(bt[i])[0]) // 50)]] = 0
        while int(bc[i].astype(np.int64).sum()) > bk:
            bc[i, np.nonzero(bc[i])[0][0]] = 0
    shp = (L, Hkv)
    return K.reshape(shp + (N, 128)), V.reshape(shp + (N, 128)), bt.reshape(shp + (N,)), bc.reshape(shp + (128,))


def _add(rdkv, pl, cache, oblob, op, pool, s, shape, seq):
    """Stage, allocate and commit one sequence on both sides; returns its pages."""
    N, bv, bk = shape
    K, V, bt, bc = seq
    staging, need = rdkv.paged_stage(pl, N, bv, bk, dev(K), dev(V), dev(bt), dev(bc))
    need = host(need)
    ref_need = [O.paged_pages_needed(op, O.segment_content(K[l, h], V[l, h], bt[l, h], bc[l, h]))
                for l in range(pl.dims.n_layers) for h in range(pl.dims.n_kv_heads)]
    assert list(need) == ref_need
    pages = [pool.take(int(k)) for k in need]
    table = np.full((len(pages), pl.max_pages), -1, np.int32)
    for i, p in enumerate(pages):
        table[i, :len(p)] = p
    rdkv.paged_commit(pl, cache, s, N, bv, bk, staging, dev(table))
    O.paged_pack_sequence(oblob, op, s, K, V, bt, bc, pages)
    return [x for p in pages for x in p]


def _same_bytes(cache, oblob, what):
    got = host(cache)
    if not np.array_equal(got, oblob):
        diff = np.nonzero(got != oblob)[0]
        pytest.fail(f"{what}: {diff.size} bytes differ, first at {diff[:6]}")


@pytest.mark.parametrize("G", [4, 8, 1])
def test_variable_length_batch_on_shuffled_pages(rdkv, G):
    L, Hkv, cap = 2, 2, 80
    Hq = G * Hkv
    shapes = [(700, 1400, 256), (2100, 6000, 512), (300, 300, 100), (1500, 3000, 384)]   # (N, bv, bk)
    N_max, bv_max, bk_max = 2100, 6000, 512
    n_pages = 900
    pl = rdkv.paged_layout(rdkv.make_dims(len(shapes), L, Hq, Hkv, N_max), bv_max, bk_max, cap, n_pages)
    op = O.PagedLayout(len(shapes), L, Hq, Hkv, N_max, bv_max, bk_max, cap, n_pages)
    cache = rdkv.paged_cache_init(pl)
    oblob = O.paged_empty(op)
    _same_bytes(cache, oblob, "empty cache")
    pool = Pool(n_pages, 7 + G)
    seqs = [_sequence(L, Hkv, *sh, seed=10 * i + G) for i, sh in enumerate(shapes)]
    held = {}
    for s, (sh, seq) in enumerate(zip(shapes, seqs)):
        held[s] = _add(rdkv, pl, cache, oblob, op, pool, s, sh, seq)
    _same_bytes(cache, oblob, "after commits")
    r = np.random.default_rng(G)
    ws = rdkv.paged_decode_workspace(pl)
    c_len = [0, 3, 17, 64]                                   # each sequence at its own zone-C length
    for s in range(len(shapes)):                             # bring zone C there (oracle and GPU alike)
        for i in range(c_len[s]):
            k = r.standard_normal((L, Hkv, 128)).astype(np.float16)
            v = r.standard_normal((L, Hkv, 128)).astype(np.float16)
            for l in range(L):
                for h in range(Hkv):
                    O.paged_write_zone_c(oblob, op, op.seg_index(s, l, h), i, k[l, h], v[l, h])
    cache.copy_(dev(oblob))
    worst = 0.0
    for step in range(12):
        q = r.standard_normal((len(shapes), L, Hq, 128)).astype(np.float16)
        kn = r.standard_normal((len(shapes), L, Hkv, 128)).astype(np.float16)
        vn = r.standard_normal((len(shapes), L, Hkv, 128)).astype(np.float16)
        append = step % 4 != 3
        out = rdkv.paged_decode(pl, cache, c_len, dev(q), dev(kn) if append else None, dev(vn) if append else None,
                                workspace=ws)
        ref = O.paged_decode_step(oblob, op, q, c_len, kn if append else None, vn if append else None)
        e = rel_err(host(out), ref)
        worst = max(worst, e)
        assert e <= TOL, f"step {step}: rel err {e:.3g}"
        if append:
            c_len = [c + 1 for c in c_len]
    _same_bytes(cache, oblob, "after decode steps")
    # a sequence leaves; a longer one takes its pages (and more)
    freed = O.paged_release_sequence(oblob, op, 2)
    rdkv.paged_release(pl, cache, 2)
    assert sorted(freed) == sorted(held[2])
    pool.give(freed)
    _same_bytes(cache, oblob, "after release")
    new_shape = (1900, 5000, 448)
    held[2] = _add(rdkv, pl, cache, oblob, op, pool, 2, new_shape, _sequence(L, Hkv, *new_shape, seed=99 + G))
    _same_bytes(cache, oblob, "after the new sequence")
    c_len[2] = 0
    q = r.standard_normal((len(shapes), L, Hq, 128)).astype(np.float16)
    out = rdkv.paged_decode(pl, cache, c_len, dev(q), workspace=ws)
    e = rel_err(host(out), O.paged_decode_step(oblob, op, q, c_len))
    assert e <= TOL
    print(f"G={G}: worst rel err {max(worst, e):.3g}; pages in use {sum(len(v) for v in held.values())} of {n_pages}")


def test_paged_decode_equals_contiguous_decode(rdkv):
    """Equal-length sequences: the paged cache on shuffled pages decodes to the
    same bits as the contiguous blob (same chunks, same arithmetic, same merge
    order), with appends."""
    S, L, Hq, Hkv, N, bv, bk, cap = 3, 2, 8, 2, 1500, 3200, 300, 70
    seqs = [_sequence(L, Hkv, N, bv, bk, seed=200 + s) for s in range(S)]
    lay = rdkv.layout(rdkv.make_dims(S, L, Hq, Hkv, N), bv, bk, cap)
    flat = rdkv.cache_init(lay)
    rdkv.pack(lay, flat, *(dev(np.stack([q[i] for q in seqs])) for i in range(4)))
    pl = rdkv.paged_layout(rdkv.make_dims(S, L, Hq, Hkv, N), bv, bk, cap, 400)
    op = O.PagedLayout(S, L, Hq, Hkv, N, bv, bk, cap, 400)
    paged = rdkv.paged_cache_init(pl)
    oblob = O.paged_empty(op)
    pool = Pool(400, 5)
    for s in range(S):
        _add(rdkv, pl, paged, oblob, op, pool, s, (N, bv, bk), seqs[s])
    r = np.random.default_rng(1)
    for step in range(cap):
        q = dev(r.standard_normal((S, L, Hq, 128)).astype(np.float16))
        kn = dev(r.standard_normal((S, L, Hkv, 128)).astype(np.float16))
        vn = dev(r.standard_normal((S, L, Hkv, 128)).astype(np.float16))
        a = rdkv.decode(lay, flat, step, q, kn, vn)
        b = rdkv.paged_decode(pl, paged, [step] * S, q, kn, vn)
        assert torch.equal(a, b), f"step {step}"


def test_paged_decode_mixed_record_lengths(rdkv):
    """A paged layout whose record bound passes 20 words: a sequence with
    5-word K records and one with 27-word records on shuffled pages of one
    pool, decoded through the 32-word ring, against the oracle."""
    S, L, Hkv, G, N, cap, n_pages = 2, 1, 2, 4, 1800, 40, 300
    Hq = G * Hkv
    bv, bk = 8000, 800
    pl = rdkv.paged_layout(rdkv.make_dims(S, L, Hq, Hkv, N), bv, bk, cap, n_pages)
    assert pl.rec_max // 4 > 20
    op = O.PagedLayout(S, L, Hq, Hkv, N, bv, bk, cap, n_pages)
    cache = rdkv.paged_cache_init(pl)
    oblob = O.paged_empty(op)
    pool = Pool(n_pages, 3)
    r = np.random.default_rng(11)
    for s, (n8, n4) in enumerate([(0, 24), (100, 0)]):
        K, V = synth.random_kv(L * Hkv, N, 40 + s)
        bt = r.choice(np.array([0, 2, 4, 8, 16], np.uint8), size=(L * Hkv, N), p=[0.5, 0.2, 0.15, 0.1, 0.05])
        while int(bt.astype(np.int64).sum(axis=1).max()) > bv:
            bt[:, r.integers(N)] = 0
        bc = np.zeros((L * Hkv, 128), np.uint8)
        for h in range(L * Hkv):
            ch = r.permutation(128)
            bc[h, ch[:n8]] = 8
            bc[h, ch[n8:n8 + n4]] = 4
        seq = (K.reshape(L, Hkv, N, 128), V.reshape(L, Hkv, N, 128), bt.reshape(L, Hkv, N), bc.reshape(L, Hkv, 128))
        _add(rdkv, pl, cache, oblob, op, pool, s, (N, bv, bk), seq)
    _same_bytes(cache, oblob, "after commits")
    ws = rdkv.paged_decode_workspace(pl)
    c_len = [0, 0]
    for step in range(4):
        q = r.standard_normal((S, L, Hq, 128)).astype(np.float16)
        kn = r.standard_normal((S, L, Hkv, 128)).astype(np.float16)
        vn = r.standard_normal((S, L, Hkv, 128)).astype(np.float16)
        out = rdkv.paged_decode(pl, cache, c_len, dev(q), dev(kn), dev(vn), workspace=ws)
        ref = O.paged_decode_step(oblob, op, q, c_len, kn, vn)
        e = rel_err(host(out), ref)
        assert e <= TOL, f"step {step}: rel err {e:.3g}"
        c_len = [c + 1 for c in c_len]
    _same_bytes(cache, oblob, "after decode steps")


def _seg_shapes(pl, cache):
    """Per segment in use (zone-C capacity of the layout; None for a free
    slot), from its descriptor on the host: prefill-token chunks
    (chunk_tok2 >> g tokens of group g) and K record bytes."""
    ints = host(cache)[256:256 + 256 * pl.n_seg].reshape(pl.n_seg, 256).view(np.int32)
    out = []
    for seg in range(pl.n_seg):
        if ints[seg, 10] != pl.zone_c_capacity:
            out.append(None)
            continue
        n_tok = ints[seg, 0:4]
        out.append((sum(-(-int(n) // (pl.chunk_tok2 >> g)) for g, n in enumerate(n_tok)), int(ints[seg, 9])))
    return out


def _host_shape(pl, cache):
    """The most chunks and the longest record over the segments in use."""
    used = [x for x in _seg_shapes(pl, cache) if x is not None]
    return max(c for c, _ in used), max(r for _, r in used)


@pytest.mark.parametrize("G", [4, 8])
def test_shaped_decode_follows_the_sequences_in_use(rdkv, G):
    """A pool laid out for loose bounds (a segment may hold 16,000 V bits and
    1,024 K bits) holding sequences that use far less: the measured shape
    matches the descriptors, launches fewer chunk slots and a smaller record
    ring, and decodes bit for bit like the layout's shape (appends included),
    within 2e-3 of the oracle.  A later, larger sequence that the old shape
    does not cover gets NaN outputs from it; a new shape covers it again.
    The two launches merge the same chunk partials in the same order; only
    the zone-C chunk sits at another slot, so the wave sum of the softmax
    denominators may round differently: outputs agree within 1e-6, the caches
    byte for byte."""
    S, L, Hkv, N, cap, n_pages = 3, 2, 2, 3000, 24, 2000
    Hq = G * Hkv
    bv, bk = 16000, 1024
    pl = rdkv.paged_layout(rdkv.make_dims(S, L, Hq, Hkv, N), bv, bk, cap, n_pages)
    op = O.PagedLayout(S, L, Hq, Hkv, N, bv, bk, cap, n_pages)
    cache = rdkv.paged_cache_init(pl)
    oblob = O.paged_empty(op)
    pool = Pool(n_pages, 5)
    for s, seed in ((0, 201), (1, 202)):
        _add(rdkv, pl, cache, oblob, op, pool, s, (N, 2500, 120), _sequence(L, Hkv, N, 2500, 120, seed))
    _same_bytes(cache, oblob, "after commits")
    shape = rdkv.paged_decode_shape(pl, cache)
    chunks, rec = _host_shape(pl, cache)
    assert (shape.token_slots, shape.rec_max) == (chunks, -(-rec // 4) * 4)
    assert shape.max_chunks == chunks + pl.max_chunks - pl.token_slots
    assert shape.token_slots < pl.token_slots and shape.rec_max < pl.rec_max
    assert shape.decode_workspace_bytes < pl.decode_workspace_bytes
    other = cache.clone()
    ws = rdkv.paged_decode_workspace(pl)
    ws_shape = torch.empty(int(shape.decode_workspace_bytes), dtype=torch.uint8, device=DEV)
    r = np.random.default_rng(17)
    c_len = [0, 0, 0]
    for step in range(3):
        q = r.standard_normal((S, L, Hq, 128)).astype(np.float16)
        kn = r.standard_normal((S, L, Hkv, 128)).astype(np.float16)
        vn = r.standard_normal((S, L, Hkv, 128)).astype(np.float16)
        got = host(rdkv.paged_decode(pl, cache, c_len, dev(q), dev(kn), dev(vn), workspace=ws_shape, shape=shape))
        want = host(rdkv.paged_decode(pl, other, c_len, dev(q), dev(kn), dev(vn), workspace=ws))
        assert rel_err(got, want) <= 1e-6, f"step {step}: shaped and unshaped decode differ"
        ref = O.paged_decode_step(oblob, op, q, c_len, kn, vn)
        assert rel_err(got[:2], ref[:2]) <= TOL
        c_len = [c + 1 if s < 2 else 0 for s, c in enumerate(c_len)]
    assert torch.equal(cache, other)
    # a larger sequence in slot 2, outside the old shape
    big = _sequence(L, Hkv, N, 12000, 700, 203)
    for c in (cache, other):
        staging, need = rdkv.paged_stage(pl, N, 12000, 700, dev(big[0]), dev(big[1]), dev(big[2]), dev(big[3]))
        pages = [pool.take(int(k)) for k in host(need)]
        table = np.full((len(pages), pl.max_pages), -1, np.int32)
        for i, pg in enumerate(pages):
            table[i, :len(pg)] = pg
        rdkv.paged_commit(pl, c, 2, N, 12000, 700, staging, dev(table))
    chunks2, rec2 = _host_shape(pl, cache)
    assert chunks2 > shape.token_slots or rec2 > shape.rec_max
    q = r.standard_normal((S, L, Hq, 128)).astype(np.float16)
    want = host(rdkv.paged_decode(pl, other, c_len, dev(q), workspace=ws))
    stale = host(rdkv.paged_decode(pl, cache, c_len, dev(q), workspace=ws_shape, shape=shape))
    assert rel_err(stale[:2], want[:2]) <= 1e-6
    for i, sh in enumerate(_seg_shapes(pl, cache)[2 * L * Hkv:]):
        l, h = divmod(i, Hkv)
        rows = stale[2, l, h * G:(h + 1) * G]
        if sh[0] > shape.token_slots or sh[1] > shape.rec_max:
            assert np.isnan(rows).all(), f"segment {i} of slot 2 outside the shape"
        else:
            assert rel_err(rows, want[2, l, h * G:(h + 1) * G]) <= 1e-6
    shape2 = rdkv.paged_decode_shape(pl, cache)
    assert (shape2.token_slots, shape2.rec_max) == (chunks2, -(-rec2 // 4) * 4)
    ws2 = torch.empty(int(shape2.decode_workspace_bytes), dtype=torch.uint8, device=DEV)
    assert rel_err(host(rdkv.paged_decode(pl, cache, c_len, dev(q), workspace=ws2, shape=shape2)), want) <= 1e-6
