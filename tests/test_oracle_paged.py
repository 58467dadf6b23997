"""Pins of the oracle's paged cache (fixed-size pages of a shared pool found
through a block table per segment, as in the aistudio.id article's
"Solusi 1") against the contiguous cache format, which the other oracle pins
tie to exact attention: the same sequences must decode to the same outputs
whichever pages hold them, sequences of different lengths and budgets must
each decode as if alone, and pages must be reusable after a sequence
leaves.  CPU only."""
import numpy as np
import pytest

import oracle as O


def _rng(seed):
    return np.random.default_rng(seed)


def _sequence(r, L, Hkv, N, bv, bk):
    """Seeded fp16 K, V and an allocation within (bv, bk) for one sequence."""
    K = r.standard_normal((L, Hkv, N, 128)).astype(np.float16)
    V = r.standard_normal((L, Hkv, N, 128)).astype(np.float16)
    bt = r.choice(np.array([0, 2, 4, 8, 16], np.uint8), size=(L, Hkv, N), p=[0.4, 0.25, 0.15, 0.12, 0.08])
    bc = r.choice(np.array([0, 2, 4, 8, 16], np.uint8), size=(L, Hkv, 128), p=[0.3, 0.3, 0.2, 0.15, 0.05])
    for idx in np.ndindex(L, Hkv):
        while int(bt[idx].astype(int).sum()) > bv:
            bt[idx][np.nonzero(bt[idx])[0][0]] = 0
        while int(bc[idx].astype(int).sum()) > bk:
            bc[idx][np.nonzero(bc[idx])[0][0]] = 0
    return K, V, bt, bc


class _Pool:
    """A host page allocator handing out pages in a shuffled order, so that
    a segment's pages are never contiguous."""

    def __init__(self, n, seed):
        self.free = list(_rng(seed).permutation(n))

    def take(self, k):
        out, self.free = self.free[:k], self.free[k:]
        assert len(out) == k, "pool exhausted"
        return out

    def give(self, pages):
        self.free = list(pages) + self.free


def _pack(blob, play, s, seq, pool):
    K, V, bt, bc = seq
    pages = []
    for l in range(play.L):
        for h in range(play.Hkv):
            sc = O.segment_content(K[l, h], V[l, h], bt[l, h], bc[l, h])
            pages.append(pool.take(O.paged_pages_needed(play, sc)))
    O.paged_pack_sequence(blob, play, s, K, V, bt, bc, pages)


def test_paged_cache_decodes_like_the_contiguous_cache():
    r = _rng(1)
    S, L, Hq, Hkv, N, bv, bk, cap = 3, 2, 8, 2, 200, 500, 300, 70
    seqs = [_sequence(r, L, Hkv, N, bv, bk) for _ in range(S)]
    lay = O.Layout(S, L, Hq, Hkv, 128, N, bv, bk, cap)
    K = np.stack([q[0] for q in seqs]); V = np.stack([q[1] for q in seqs])
    bt = np.stack([q[2] for q in seqs]); bc = np.stack([q[3] for q in seqs])
    blob = O.pack_cache(lay, K, V, bt, bc)
    play = O.PagedLayout(S, L, Hq, Hkv, N, bv, bk, cap, 400)
    pblob = O.paged_empty(play)
    pool = _Pool(400, 2)
    for s in range(S):
        _pack(pblob, play, s, seqs[s], pool)
    for step in range(cap - 1):
        q = r.standard_normal((S, L, Hq, 128)).astype(np.float16)
        kn = r.standard_normal((S, L, Hkv, 128)).astype(np.float16)
        vn = r.standard_normal((S, L, Hkv, 128)).astype(np.float16)
        ref = O.decode_step(blob, lay, q, step, kn, vn)
        got = O.paged_decode_step(pblob, play, q, [step] * S, kn, vn)
        if step in (0, 1, 63, 64, 65, cap - 2):          # zone-C tile and page boundaries
            assert np.allclose(got, ref, rtol=1e-12, atol=1e-14), f"step {step}"
    for s in range(S):                                   # positions survive the paging
        for l in range(L):
            for h in range(Hkv):
                _, _, pos, _ = O.unpack_segment(blob, lay, lay.seg_index(s, l, h))
                assert np.array_equal(O.paged_positions(pblob, play, play.seg_index(s, l, h)), pos)


def test_sequences_of_different_lengths_and_budgets_decode_as_if_alone():
    """A variable-length batch: each sequence has its own prefill length,
    budget and zone-C length, and decodes exactly as a one-sequence
    contiguous cache of its own shape."""
    r = _rng(3)
    L, Hq, Hkv, cap = 1, 4, 2, 40
    shapes = [(120, 240, 100), (333, 900, 256), (50, 60, 40), (256, 512, 512)]   # (N, bv, bk)
    N_max, bv_max, bk_max = 333, 900, 512
    play = O.PagedLayout(len(shapes), L, Hq, Hkv, N_max, bv_max, bk_max, cap, 300)
    pblob = O.paged_empty(play)
    pool = _Pool(300, 4)
    seqs = [_sequence(r, L, Hkv, *sh) for sh in shapes]
    for s, seq in enumerate(seqs):
        _pack(pblob, play, s, seq, pool)
    alone = []
    for (N, bv, bk), seq in zip(shapes, seqs):
        lay = O.Layout(1, L, Hq, Hkv, 128, N, bv, bk, cap)
        alone.append((lay, O.pack_cache(lay, *(x[None] for x in seq))))
    c_len = [0, 5, 17, 39]
    for s, (lay, blob) in enumerate(alone):             # bring each zone C to its own length
        for i in range(c_len[s]):
            kn = r.standard_normal((1, L, Hkv, 128)).astype(np.float16)
            vn = r.standard_normal((1, L, Hkv, 128)).astype(np.float16)
            O.append_zone_c(blob, lay, i, kn, vn)
            for l in range(L):
                for h in range(Hkv):
                    O.paged_write_zone_c(pblob, play, play.seg_index(s, l, h), i, kn[0, l, h], vn[0, l, h])
    q = r.standard_normal((len(shapes), L, Hq, 128)).astype(np.float16)
    kn = r.standard_normal((len(shapes), L, Hkv, 128)).astype(np.float16)
    vn = r.standard_normal((len(shapes), L, Hkv, 128)).astype(np.float16)
    got = O.paged_decode_step(pblob, play, q, c_len, kn, vn)
    for s, (lay, blob) in enumerate(alone):
        ref = O.decode_step(blob, lay, q[s:s + 1], c_len[s], kn[s:s + 1], vn[s:s + 1])
        assert np.allclose(got[s:s + 1], ref, rtol=1e-12, atol=1e-14), f"sequence {s}"
    with pytest.raises(ValueError):                    # a full zone C cannot take another token
        O.paged_decode_step(pblob.copy(), play, q, [0, 0, 0, cap], kn, vn)


def test_released_pages_are_reused_without_disturbing_the_rest():
    r = _rng(5)
    S, L, Hq, Hkv, N, bv, bk, cap = 3, 1, 4, 1, 150, 400, 256, 16
    play = O.PagedLayout(S, L, Hq, Hkv, N, bv, bk, cap, 60)
    pblob = O.paged_empty(play)
    pool = _Pool(60, 6)
    seqs = [_sequence(r, L, Hkv, N, bv, bk) for _ in range(S)]
    for s in range(S):
        _pack(pblob, play, s, seqs[s], pool)
    q = r.standard_normal((S, L, Hq, 128)).astype(np.float16)
    before = O.paged_decode_step(pblob, play, q, [0] * S)
    freed = O.paged_release_sequence(pblob, play, 1)
    assert len(freed) > 0 and len(set(freed)) == len(freed)
    after_release = O.paged_decode_step(pblob, play, q, [0] * S)
    assert not after_release[1].any()                   # a free slot gives zeros
    assert np.array_equal(after_release[[0, 2]], before[[0, 2]])
    pool.give(freed)
    new = _sequence(r, L, Hkv, N, bv, bk)
    _pack(pblob, play, 1, new, pool)
    after = O.paged_decode_step(pblob, play, q, [0] * S)
    assert np.array_equal(after[[0, 2]], before[[0, 2]])
    lay = O.Layout(1, L, Hq, Hkv, 128, N, bv, bk, cap)
    ref = O.decode_step(O.pack_cache(lay, *(x[None] for x in new)), lay, q[1:2], 0)
    assert np.allclose(after[1:2], ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("N,bv,bk,cap", [(1000, 2000, 256, 128), (300, 16 * 300, 16 * 128, 256),
                                         (4096, 2621, 81, 128), (64, 1, 0, 1), (200, 3200, 0, 5)])
def test_page_bound_and_tile_layout(N, bv, bk, cap):
    """At the budget extremes a segment's pages stay within the layout's bound,
    and every region's tiles fit their pages whole."""
    play = O.PagedLayout(1, 1, 4, 1, N, bv, bk, cap, 1)
    r = _rng(N + bv)
    for trial in range(6):
        # all budget on one group, or spread; all budget on one K bitwidth
        g = trial % 4
        bt = np.zeros(N, np.uint8)
        bt[:min(N, bv // (2 << g))] = 2 << g
        bc = np.zeros(128, np.uint8)
        bc[:min(128, bk // (2 << (trial % 4)))] = 2 << (trial % 4)
        sc = O.segment_content(r.standard_normal((N, 128)).astype(np.float16),
                               r.standard_normal((N, 128)).astype(np.float16), bt, bc)
        need = O.paged_pages_needed(play, sc)
        assert need <= play.max_pages
        rows = sc["n_tok"] + sc["n_tok"] + [cap, cap, sc["n_kept"]]
        for reg in range(O.N_REGIONS):
            tb = O.region_tile_bytes(reg, sc["rec"])
            assert tb <= O.PAGE_BYTES and (tb > 0 or reg == O.R_REC + 3)
            assert O.region_pages(rows[reg], tb) == (0 if rows[reg] == 0 or tb == 0 else
                                                     -(-(-(-rows[reg] // O.TILE)) // (O.PAGE_BYTES // tb)))


def test_sixteen_bit_tokens_with_every_k_channel_dropped():
    """A segment whose K channels all have 0 bits still keeps 16-bit V rows;
    their K records are empty (0 bytes, no pages), their logits 0."""
    r = _rng(7)
    N, cap = 90, 3
    play = O.PagedLayout(1, 1, 2, 1, N, 16 * N, 0, cap, 10)
    lay = O.Layout(1, 1, 2, 1, 128, N, 16 * N, 0, cap)
    K = r.standard_normal((1, 1, N, 128)).astype(np.float16)
    V = r.standard_normal((1, 1, N, 128)).astype(np.float16)
    bt = np.zeros((1, 1, N), np.uint8)
    bt[0, 0, ::2] = 16
    bc = np.zeros((1, 1, 128), np.uint8)
    pblob = O.paged_empty(play)
    _pack(pblob, play, 0, (K, V, bt, bc), _Pool(10, 8))
    q = r.standard_normal((1, 1, 2, 128)).astype(np.float16)
    ref = O.decode_step(O.pack_cache(lay, K[None], V[None], bt[None], bc[None]), lay, q, 0)
    assert np.allclose(O.paged_decode_step(pblob, play, q, [0]), ref, rtol=1e-12, atol=1e-14)
    # the output is then the plain mean of the kept V rows
    assert np.allclose(ref[0, 0], V[0, 0, ::2].astype(np.float64).mean(axis=0)[None], rtol=1e-10, atol=1e-12)
