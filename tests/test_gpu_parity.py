"""Parity of the HIP library against the CPU oracle, stage by stage, on the
same seeded inputs, through the C ABI.

Bars: bit-exact for the allocation (bits, exact channel variances, lambda),
the packed bytes and the dequantized values; max relative error <= 2e-3 for
the weights and the decode outputs (fp32 accumulation of fp16 inputs against
fp64).  Decode error metric per (step, query head): max_i |o_i - r_i| /
max_i |r_i|.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle as O
from decode_attention_rdkv_amd import synth

pytestmark = pytest.mark.gpu

TOL = 2e-3
DEV = "cuda"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    return t.detach().cpu().numpy()


def rel_err_rows(got, ref):
    """max |got - ref| / max |ref| along the last axis, reduced with max."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(got - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return float((num / den).max())


# ------------------------------------------------------------------ packing cases

def _bits_case(name, n_seg, N, seed):
    bt, bc = synth.random_bits(n_seg, N, seed)
    if name == "all16":
        bt[:] = 16
        bc[:] = 16
    elif name == "evict_only":
        bt = np.where(bt > 0, 16, 0).astype(np.uint8)
    elif name == "two_bit":
        bt = np.where(bt > 0, 2, 0).astype(np.uint8)
        bc[:] = 2
    elif name == "k_dropped":
        bc[:] = 0
    elif name == "odd16":
        bc[:] = 0
        bc[:, :5] = 16
        bc[:, 5:8] = 8
        bc[:, 8:9] = 2
    elif name == "mid_k":                    # 12-word record bound: the SW = 12 decode path
        bc[:] = 0
        bc[:, 10:30] = 8
        bc[:, 40:45] = 2
    elif name == "k20":                      # 19-word record bound: the SW = 20 decode path
        bc[:] = 0
        bc[:, 0:40] = 4
        bc[:, 40:100] = 2
        bc[:, 100:105] = 8
    elif name == "empty_and_single":
        bt[0] = 0
        if n_seg > 1:
            bt[1] = 0
            bt[1, N // 2] = 4
    return bt, bc


PACK_CASES = [
    # (name, S, L, Hq, Hkv, N, cap)
    ("mixed", 1, 1, 4, 1, 1024, 16),
    ("mixed", 2, 2, 4, 2, 777, 5),
    ("all16", 1, 1, 8, 1, 300, 4),
    ("evict_only", 1, 2, 2, 1, 513, 3),
    ("two_bit", 1, 1, 8, 8, 129, 2),
    ("k_dropped", 2, 1, 4, 2, 64, 1),
    ("odd16", 1, 1, 4, 1, 1500, 3),
    ("empty_and_single", 1, 1, 2, 2, 200, 2),
    ("mid_k", 1, 1, 8, 2, 700, 4),
    ("k20", 1, 2, 8, 2, 600, 4),
]


def _pack_case(case):
    from decode_attention_rdkv_amd import rdkv
    name, S, L, Hq, Hkv, N, cap = case
    n_seg = S * L * Hkv
    seed = zlib.crc32(repr(case).encode()) % 1000
    bt, bc = _bits_case(name, n_seg, N, seed)
    K, V = synth.random_kv(n_seg, N, seed, scale=1.0)
    K[..., 3] *= np.float16(8)                        # an outlier channel
    bv = int(bt.astype(np.int64).sum(axis=1).max())
    bk = int(bc.astype(np.int64).sum(axis=1).max())
    lay = rdkv.layout(rdkv.make_dims(S, L, Hq, Hkv, N), bv, bk, cap)
    ol = O.Layout(S, L, Hq, Hkv, 128, N, bv, bk, cap)
    shp = (S, L, Hkv)
    Kr, Vr = K.reshape(shp + (N, 128)), V.reshape(shp + (N, 128))
    btr, bcr = bt.reshape(shp + (N,)), bc.reshape(shp + (128,))
    oblob = O.pack_cache(ol, Kr, Vr, btr, bcr)
    return lay, ol, oblob, (Kr, Vr, btr, bcr)


def test_cache_init_matches_oracle(gpu_lib):
    rdkv = gpu_lib
    lay = rdkv.layout(rdkv.make_dims(2, 3, 8, 2, 100), 130, 77, 3)
    ol = O.Layout(2, 3, 8, 2, 128, 100, 130, 77, 3)
    blob = host(rdkv.cache_init(lay))
    assert np.array_equal(blob, O.empty_blob(ol))


@pytest.mark.parametrize("case", PACK_CASES, ids=lambda c: f"{c[0]}-S{c[1]}L{c[2]}H{c[3]}/{c[4]}N{c[5]}")
def test_pack_bytes_and_dequant_bit_exact(gpu_lib, case):
    rdkv = gpu_lib
    lay, ol, oblob, (K, V, bt, bc) = _pack_case(case)
    cache = rdkv.cache_init(lay)
    rdkv.pack(lay, cache, dev(K), dev(V), dev(bt), dev(bc))
    gblob = host(cache)
    if not np.array_equal(gblob, oblob):
        diff = np.nonzero(gblob != oblob)[0]
        pytest.fail(f"{diff.size} bytes differ, first at {diff[:8]} of {gblob.size}")
    for seg in range(lay.n_seg):
        kh, vh = rdkv.unpack(lay, cache, seg)
        okh, ovh, _, _ = O.unpack_segment(oblob, ol, seg)
        n = okh.shape[0]
        assert np.array_equal(host(kh)[:n].view(np.uint32), okh.view(np.uint32))
        assert np.array_equal(host(vh)[:n].view(np.uint32), ovh.view(np.uint32))


def test_pack_layer_by_layer_equals_whole(gpu_lib):
    rdkv = gpu_lib
    lay, ol, oblob, (K, V, bt, bc) = _pack_case(("mixed", 2, 3, 4, 2, 300, 4))
    cache = rdkv.cache_init(lay)
    for l in (2, 0, 1):
        rdkv.pack(lay, cache, dev(K[:, l:l + 1]), dev(V[:, l:l + 1]), dev(bt[:, l:l + 1]), dev(bc[:, l:l + 1]),
                  layer_begin=l)
    assert np.array_equal(host(cache), oblob)


def test_pack_over_budget_segment_is_flagged_empty(gpu_lib):
    rdkv = gpu_lib
    N = 100
    lay = rdkv.layout(rdkv.make_dims(1, 1, 4, 2, N), 40, 16, 2)
    K, V = synth.random_kv(2, N, 5)
    bt = np.zeros((2, N), np.uint8)
    bt[0, :10] = 4                                    # 40 bits: fits
    bt[1, :30] = 2                                    # 30 tokens > nk_max = 20: does not fit
    bc = np.zeros((2, 128), np.uint8)
    bc[:, :2] = 8
    cache = rdkv.cache_init(lay)
    args = (dev(K.reshape(1, 1, 2, N, 128)), dev(V.reshape(1, 1, 2, N, 128)), dev(bt.reshape(1, 1, 2, N)),
            dev(bc.reshape(1, 1, 2, 128)))
    with pytest.raises(rdkv.RdkvError) as err:
        rdkv.pack(lay, cache, *args)
    assert err.value.name == "RDKV_ERR_OVERFLOW"
    d = rdkv.descriptors(lay, cache)
    assert list(d["n_kept"]) == [10, 0] and list(d["flags"]) == [0, 1]
    assert rdkv.pack_status(lay, cache).item() == 1
    # three 16-bit tokens (48 bits > 40) fit the slot's V bytes and kept-token
    # bound, but not its V units (sum of b_t / 2 <= 20), from which decode's
    # chunk slots are sized: flagged as well
    bt[1] = 0
    bt[1, :3] = 16
    cache = rdkv.cache_init(lay)
    rdkv.pack(lay, cache, *args[:2], dev(bt.reshape(1, 1, 2, N)), args[3], check=False)
    d = rdkv.descriptors(lay, cache)
    assert list(d["n_kept"]) == [10, 0] and list(d["flags"]) == [0, 1]
    # a fitting allocation packs without complaint
    bt[1, 2] = 0
    cache = rdkv.cache_init(lay)
    rdkv.pack(lay, cache, *args[:2], dev(bt.reshape(1, 1, 2, N)), args[3])
    assert rdkv.pack_status(lay, cache).item() == 0


# ------------------------------------------------------------------ decode

def _decode_run(rdkv, lay, ol, cache, oblob, steps, seed, check_every=1):
    """Runs `steps` decode steps on both sides (appending on most steps) and
    checks the outputs; returns the worst relative error seen."""
    d = lay.dims
    S, L, Hq, Hkv = d.n_seq, d.n_layers, d.n_q_heads, d.n_kv_heads
    r = np.random.default_rng(seed)
    ws = rdkv.decode_workspace(lay)
    worst, c_len = 0.0, 0
    for step in range(steps):
        q = r.standard_normal((S, L, Hq, 128)).astype(np.float16)
        append = (step % 3 != 2) and c_len < lay.zone_c_capacity
        kn = r.standard_normal((S, L, Hkv, 128)).astype(np.float16) if append else None
        vn = r.standard_normal((S, L, Hkv, 128)).astype(np.float16) if append else None
        out = rdkv.decode(lay, cache, c_len, dev(q), None if kn is None else dev(kn),
                          None if vn is None else dev(vn), workspace=ws)
        if step % check_every == 0 or step == steps - 1:
            ref = O.decode_step(oblob, ol, q, c_len, kn, vn)
            e = rel_err_rows(host(out), ref)
            worst = max(worst, e)
            assert e <= TOL, f"step {step}: rel err {e:.3g}"
        elif append:
            O.append_zone_c(oblob, ol, c_len, kn, vn)
        c_len += int(append)
    return worst


@pytest.mark.parametrize("case", PACK_CASES, ids=lambda c: f"{c[0]}-S{c[1]}L{c[2]}H{c[3]}/{c[4]}N{c[5]}")
def test_decode_matches_oracle(gpu_lib, case):
    rdkv = gpu_lib
    lay, ol, oblob, (K, V, bt, bc) = _pack_case(case)
    cache = rdkv.cache_init(lay)
    rdkv.pack(lay, cache, dev(K), dev(V), dev(bt), dev(bc))
    _decode_run(rdkv, lay, ol, cache, oblob, 4, 7)
    # zone C and the rest of the blob stay byte-identical to the oracle's
    assert np.array_equal(host(cache), oblob)


def test_decode_empty_cache_gives_zero(gpu_lib):
    rdkv = gpu_lib
    lay = rdkv.layout(rdkv.make_dims(1, 2, 8, 2, 50), 100, 64, 2)
    cache = rdkv.cache_init(lay)
    q = torch.randn((1, 2, 8, 128), device=DEV).half()
    out = rdkv.decode(lay, cache, 0, q)
    assert torch.all(out == 0)


def test_decode_split_k_chunks_and_long_rows(gpu_lib):
    """Several chunks per group (ragged tails) for every bitwidth, G = 8."""
    rdkv = gpu_lib
    N = 9000
    r = np.random.default_rng(3)
    bt = r.choice(np.array([0, 2, 4, 8, 16], np.uint8), size=(1, N), p=[0.2, 0.3, 0.2, 0.2, 0.1])
    bc = r.choice(np.array([0, 2, 4, 8, 16], np.uint8), size=(1, 128))
    K, V = synth.random_kv(1, N, 11)
    bv, bk = int(bt.sum()), int(bc.sum())
    lay = rdkv.layout(rdkv.make_dims(1, 1, 8, 1, N), bv, bk, 300)
    ol = O.Layout(1, 1, 8, 1, 128, N, bv, bk, 300)
    shp = (1, 1, 1)
    oblob = O.pack_cache(ol, K.reshape(shp + (N, 128)), V.reshape(shp + (N, 128)), bt.reshape(shp + (N,)),
                         bc.reshape(shp + (128,)))
    cache = rdkv.cache_init(lay)
    rdkv.pack(lay, cache, dev(K.reshape(shp + (N, 128))), dev(V.reshape(shp + (N, 128))),
              dev(bt.reshape(shp + (N,))), dev(bc.reshape(shp + (128,))))
    assert np.array_equal(host(cache), oblob)
    d = rdkv.descriptors(lay, cache)
    assert all(d["n_tok"][0] > np.array([1024, 512, 256, 128]))   # more than one chunk per group
    _decode_run(rdkv, lay, ol, cache, oblob, 3, 5)


@pytest.mark.parametrize("n16,slots", [(1500, (1, 32)), (6000, (33, 128)), (12000, (129, 256))])
def test_decode_merge_over_many_chunk_slots(gpu_lib, n16, slots):
    """One segment whose fp16 group alone fills dozens to hundreds of 64-row
    chunks: the merge's narrow form (up to 32 chunk slots), its wide form in
    one round (33..128) and over two rounds (more than 128), each against the
    oracle."""
    rdkv = gpu_lib
    N = n16 + 1000
    r = np.random.default_rng(n16)
    bt = np.zeros((1, N), np.uint8)
    bt[0, r.permutation(N)[:n16]] = 16
    bt[0, bt[0] == 0] = 2
    bc = np.zeros((1, 128), np.uint8)
    bc[0, :24], bc[0, 24:40] = 4, 8
    K, V = synth.random_kv(1, N, n16 + 1)
    bv, bk = int(bt.sum()), int(bc.sum())
    lay = rdkv.layout(rdkv.make_dims(1, 1, 4, 1, N), bv, bk, 70)
    assert slots[0] <= lay.max_chunks <= slots[1]
    ol = O.Layout(1, 1, 4, 1, 128, N, bv, bk, 70)
    shp = (1, 1, 1)
    Ks, Vs, bts, bcs = K.reshape(shp + (N, 128)), V.reshape(shp + (N, 128)), bt.reshape(shp + (N,)), bc.reshape(shp + (128,))
    oblob = O.pack_cache(ol, Ks, Vs, bts, bcs)
    cache = rdkv.cache_init(lay)
    rdkv.pack(lay, cache, dev(Ks), dev(Vs), dev(bts), dev(bcs))
    assert np.array_equal(host(cache), oblob)
    _decode_run(rdkv, lay, ol, cache, oblob, 3, n16)


@pytest.mark.parametrize("G,bk", [(4, 800), (4, 1100), (8, 800), (1, 1100)])
def test_decode_mixed_record_lengths(gpu_lib, G, bk):
    """Segments with K records of 5, 20, 21 and 27 words in one layout whose
    record bound passes 20 words: decoded through the ring of the bound (32
    words at bk = 800) or with no ring (bk = 1100) while zone C grows, every
    segment against the oracle."""
    rdkv = gpu_lib
    Hkv, N, cap = 4, 3000, 8
    r = np.random.default_rng(bk + G)
    bt = r.choice(np.array([0, 2, 4, 8, 16], np.uint8), size=(Hkv, N), p=[0.5, 0.2, 0.15, 0.1, 0.05])
    bc = np.zeros((Hkv, 128), np.uint8)
    for h, (n8, n4) in enumerate([(0, 24), (72, 0), (76, 0), (100, 0)]):   # 5, 20, 21, 27 words
        ch = r.permutation(128)
        bc[h, ch[:n8]] = 8
        bc[h, ch[n8:n8 + n4]] = 4
    K, V = synth.random_kv(Hkv, N, bk + G + 1)
    bv = int(bt.astype(np.int64).sum(axis=1).max())
    lay = rdkv.layout(rdkv.make_dims(1, 1, G * Hkv, Hkv, N), bv, bk, cap)
    assert lay.rec_max // 4 > 20
    ol = O.Layout(1, 1, G * Hkv, Hkv, 128, N, bv, bk, cap)
    shp = (1, 1, Hkv)
    Ks, Vs, bts, bcs = K.reshape(shp + (N, 128)), V.reshape(shp + (N, 128)), bt.reshape(shp + (N,)), bc.reshape(shp + (128,))
    oblob = O.pack_cache(ol, Ks, Vs, bts, bcs)
    cache = rdkv.cache_init(lay)
    rdkv.pack(lay, cache, dev(Ks), dev(Vs), dev(bts), dev(bcs))
    assert np.array_equal(host(cache), oblob)
    assert sorted(rdkv.descriptors(lay, cache)["rec"] // 4) == [5, 20, 21, 27]
    _decode_run(rdkv, lay, ol, cache, oblob, 4, bk)
    assert np.array_equal(host(cache), oblob)


@pytest.mark.parametrize("G", [1, 4, 8])
def test_zone_c_grows_to_300_rows(gpu_lib, G):
    """Zone C (fp16 rows of new tokens, RDKV summary section 2.3) appended row
    by row up to 300 rows next to a packed zone A/B: one zone-C tile (n_c <=
    64), several tiles of one chunk (65..256; at G = 8 the two head halves walk
    each tile), and a second zone-C chunk (n_c > 256).  Checked against the
    oracle at every tile and chunk boundary."""
    rdkv = gpu_lib
    S, L, Hkv, N, cap = 1, 1, 2, 200, 300
    Hq = G * Hkv
    bt, bc = synth.random_bits(Hkv, N, 17 + G)
    K, V = synth.random_kv(Hkv, N, 18 + G)
    bv, bk = int(bt.astype(np.int64).sum(axis=1).max()), int(bc.astype(np.int64).sum(axis=1).max())
    lay = rdkv.layout(rdkv.make_dims(S, L, Hq, Hkv, N), bv, bk, cap)
    ol = O.Layout(S, L, Hq, Hkv, 128, N, bv, bk, cap)
    shp = (S, L, Hkv)
    args = (K.reshape(shp + (N, 128)), V.reshape(shp + (N, 128)), bt.reshape(shp + (N,)), bc.reshape(shp + (128,)))
    oblob = O.pack_cache(ol, *args)
    cache = rdkv.cache_init(lay)
    rdkv.pack(lay, cache, *(dev(a) for a in args))
    assert np.array_equal(host(cache), oblob)
    ws = rdkv.decode_workspace(lay)
    r = np.random.default_rng(100 + G)
    checks = {1, 63, 64, 65, 128, 129, 256, 257, 300}
    for c_len in range(cap):
        q = r.standard_normal((S, L, Hq, 128)).astype(np.float16)
        kn = (r.standard_normal((S, L, Hkv, 128)) * 2).astype(np.float16)
        vn = r.standard_normal((S, L, Hkv, 128)).astype(np.float16)
        out = rdkv.decode(lay, cache, c_len, dev(q), dev(kn), dev(vn), workspace=ws)
        if c_len + 1 in checks:
            ref = O.decode_step(oblob, ol, q, c_len, kn, vn)
            e = rel_err_rows(host(out), ref)
            assert e <= TOL, f"G={G}, {c_len + 1} zone-C rows: rel err {e:.3g}"
        else:
            O.append_zone_c(oblob, ol, c_len, kn, vn)
    assert np.array_equal(host(cache), oblob)
    # a step that attends the full zone without appending
    q = r.standard_normal((S, L, Hq, 128)).astype(np.float16)
    e = rel_err_rows(host(rdkv.decode(lay, cache, cap, dev(q), workspace=ws)), O.decode_step(oblob, ol, q, cap))
    assert e <= TOL
    with pytest.raises(rdkv.RdkvError):
        rdkv.decode(lay, cache, cap, dev(q), dev(kn), dev(vn), workspace=ws)


# ------------------------------------------------------------------ allocation

@pytest.mark.parametrize("N,budget_avg", [(5000, "2"), (1024, "4"), (777, "0.5"), (300, "0"), (64, "17"),
                                          (4096, "0.64")])
def test_allocate_bit_exact(gpu_lib, N, budget_avg):
    from fractions import Fraction
    rdkv = gpu_lib
    S, L, Hkv = 1, 2, 2
    n_seg = S * L * Hkv
    w_tok, var_tok, w_chan = synth.random_unit_inputs(n_seg, N, seed=N)
    K, _ = synth.random_kv(n_seg, N, seed=N + 1)
    K[:, :, :4] *= np.float16(8)
    bv = int(Fraction(budget_avg) * N)
    bk = int(Fraction(budget_avg) * 128)
    shp = (S, L, Hkv)
    bits_tok, bits_chan, var_chan, lam = rdkv.allocate(
        rdkv.make_dims(S, L, 4, Hkv, N), dev(w_tok.reshape(shp + (N,))), dev(var_tok.reshape(shp + (N,))),
        dev(w_chan.reshape(shp + (128,))), dev(K.reshape(shp + (N, 128))), bv, bk)
    bits_tok, bits_chan = host(bits_tok).reshape(n_seg, N), host(bits_chan).reshape(n_seg, 128)
    var_chan, lam = host(var_chan).reshape(n_seg, 128), host(lam).reshape(n_seg, 2)
    for s in range(n_seg):
        ref = O.allocate_segment(w_tok[s], var_tok[s], w_chan[s], K[s], bv, bk)
        assert np.array_equal(bits_tok[s], ref["bits_tok"]), f"seg {s}: V bits differ"
        assert lam[s, 0] == ref["lambda_v"]
        assert np.array_equal(var_chan[s].view(np.uint32), ref["var_chan"].view(np.uint32)), f"seg {s}: var_chan"
        assert np.array_equal(bits_chan[s], ref["bits_chan"]), f"seg {s}: K bits differ"
        assert lam[s, 1] == ref["lambda_k"]
        assert int(bits_tok[s].astype(np.int64).sum()) <= bv and int(bits_chan[s].astype(np.int64).sum()) <= bk


@pytest.mark.parametrize("group,budget_avg,ties", [(1, "0.64", False), (1, "2", True), (1, "0", False),
                                                   (1, "17", False), (2, "0.5", True), (2, "3", False)])
def test_allocate_many_workgroups_bit_exact(gpu_lib, group, budget_avg, ties):
    """Segments long enough that the V selection runs over several
    workgroups per group (histograms added in the workspace, one pick per
    pass) and the K sums over several token blocks: bits, lambdas and
    variances bit for bit against the oracle, with zero and saturating
    budgets and with many equal costs (ties at the crossing)."""
    from fractions import Fraction
    rdkv = gpu_lib
    S, L, Hkv, N = 1, 1, 4, 40000
    n_seg = S * L * Hkv
    w_tok, var_tok, w_chan = synth.random_unit_inputs(n_seg, N, seed=77)
    if ties:   # a few distinct values: many units share each product
        w_tok = np.float32(2.0) ** np.round(np.log2(w_tok)).clip(-20, 20).astype(np.float32)
        var_tok = np.float32(2.0) ** np.round(np.log2(var_tok)).clip(-20, 20).astype(np.float32)
    K, _ = synth.random_kv(n_seg, N, seed=78)
    bv, bk = int(Fraction(budget_avg) * N) * group, int(Fraction(budget_avg) * 128) * group
    dims = rdkv.make_dims(S, L, 4 * Hkv, Hkv, N)
    assert rdkv.allocate_workspace_bytes(dims, group) > 0   # the many-workgroup path
    shp = (S, L, Hkv)
    bt, bc, vc, lam = (host(x) for x in rdkv.allocate_shared(
        dims, dev(w_tok.reshape(shp + (N,))), dev(var_tok.reshape(shp + (N,))), dev(w_chan.reshape(shp + (128,))),
        dev(K.reshape(shp + (N, 128))), bv, bk, group))
    bt, bc, vc, lam = bt.reshape(n_seg, N), bc.reshape(n_seg, 128), vc.reshape(n_seg, 128), lam.reshape(n_seg, 2)
    for g0 in range(0, n_seg, group):
        sl = slice(g0, g0 + group)
        ref = O.allocate_group(w_tok[sl], var_tok[sl], w_chan[sl], K[sl], bv, bk)
        assert np.array_equal(bt[sl], ref["bits_tok"]), f"group at {g0}: V bits differ"
        assert np.all(lam[sl, 0] == ref["lambda_v"])
        assert np.array_equal(vc[sl].view(np.uint32), ref["var_chan"].view(np.uint32)), f"group at {g0}: var_chan"
        assert np.array_equal(bc[sl], ref["bits_chan"]) and np.all(lam[sl, 1] == ref["lambda_k"])
    if budget_avg == "0":
        assert not bt.any()
    if budget_avg == "17":
        assert np.all(bt == 16) and np.all(lam[:, 0] == 0.0)


def test_allocate_reuses_a_dirty_workspace(gpu_lib):
    """One caller workspace, filled with 0xFF first, serves three allocations
    in a row (per segment, one budget per group of 2, then a smaller
    problem): each is bit-exact against the oracle, so nothing depends on the
    workspace's contents before a call (the histograms and selection states
    are cleared by a kernel of the call itself)."""
    rdkv = gpu_lib
    S, L, Hkv = 1, 1, 2
    ws = None
    for N, group, seed in ((30000, 1, 81), (30000, 2, 82), (9000, 1, 83)):
        n_seg = S * L * Hkv
        w_tok, var_tok, w_chan = synth.random_unit_inputs(n_seg, N, seed=seed)
        K, _ = synth.random_kv(n_seg, N, seed=seed + 100)
        bv, bk = int(0.8 * N) * group, 100 * group
        dims = rdkv.make_dims(S, L, 4 * Hkv, Hkv, N)
        if ws is None:
            size = max(rdkv.allocate_workspace_bytes(dims, 1), rdkv.allocate_workspace_bytes(dims, 2))
            ws = torch.full((size,), 0xFF, dtype=torch.uint8, device=DEV)
        assert ws.numel() >= rdkv.allocate_workspace_bytes(dims, group) > 0
        shp = (S, L, Hkv)
        bt, bc, vc, lam = (host(x) for x in rdkv.allocate_shared(
            dims, dev(w_tok.reshape(shp + (N,))), dev(var_tok.reshape(shp + (N,))),
            dev(w_chan.reshape(shp + (128,))), dev(K.reshape(shp + (N, 128))), bv, bk, group, workspace=ws))
        bt, bc, vc, lam = bt.reshape(n_seg, N), bc.reshape(n_seg, 128), vc.reshape(n_seg, 128), lam.reshape(n_seg, 2)
        for g0 in range(0, n_seg, group):
            sl = slice(g0, g0 + group)
            ref = O.allocate_group(w_tok[sl], var_tok[sl], w_chan[sl], K[sl], bv, bk)
            assert np.array_equal(bt[sl], ref["bits_tok"]), f"N={N} group={group}: V bits differ"
            assert np.all(lam[sl, 0] == ref["lambda_v"]) and np.all(lam[sl, 1] == ref["lambda_k"])
            assert np.array_equal(vc[sl].view(np.uint32), ref["var_chan"].view(np.uint32))
            assert np.array_equal(bc[sl], ref["bits_chan"])


@pytest.mark.parametrize("group,budget_scale", [(1, 1.0), (2, 1.0), (4, 1.0), (8, 1.0), (4, 0.0), (8, 40.0)])
def test_allocate_shared_bit_exact(gpu_lib, group, budget_scale):
    """One budget per group of consecutive segments (2 layers x 4 KV heads:
    group 4 = per layer, 8 = the whole sequence) against the oracle's pooled
    allocation on the same fp32 inputs; group 1 is rdkv_allocate."""
    rdkv = gpu_lib
    S, L, Hkv, N = 1, 2, 4, 600
    n_seg = S * L * Hkv
    w_tok, var_tok, w_chan = synth.random_unit_inputs(n_seg, N, seed=41)
    w_tok *= np.arange(1, n_seg + 1, dtype=np.float32)[:, None]   # heads of unequal importance
    K, _ = synth.random_kv(n_seg, N, seed=42)
    K[:, :, :4] *= np.float16(8)
    # budget_scale 0: everything evicted; 40: more than 16 bits for every unit
    bv, bk = int(1.5 * N * budget_scale) * group, int(96 * budget_scale) * group
    dims = rdkv.make_dims(S, L, 4 * Hkv, Hkv, N)
    shp = (S, L, Hkv)
    args = (dims, dev(w_tok.reshape(shp + (N,))), dev(var_tok.reshape(shp + (N,))), dev(w_chan.reshape(shp + (128,))),
            dev(K.reshape(shp + (N, 128))), bv, bk)
    bt, bc, vc, lam = (host(x) for x in rdkv.allocate_shared(*args, group))
    bt, bc, vc, lam = bt.reshape(n_seg, N), bc.reshape(n_seg, 128), vc.reshape(n_seg, 128), lam.reshape(n_seg, 2)
    for g0 in range(0, n_seg, group):
        sl = slice(g0, g0 + group)
        ref = O.allocate_group(w_tok[sl], var_tok[sl], w_chan[sl], K[sl], bv, bk)
        assert np.array_equal(bt[sl], ref["bits_tok"]), f"group at {g0}: V bits differ"
        assert np.array_equal(vc[sl].view(np.uint32), ref["var_chan"].view(np.uint32))
        assert np.array_equal(bc[sl], ref["bits_chan"]), f"group at {g0}: K bits differ"
        assert np.all(lam[sl, 0] == ref["lambda_v"]) and np.all(lam[sl, 1] == ref["lambda_k"])
        assert int(bt[sl].astype(np.int64).sum()) <= bv and int(bc[sl].astype(np.int64).sum()) <= bk
    if budget_scale == 0.0:
        assert not bt.any() and not bc.any()
    if budget_scale == 40.0:
        assert np.all(bt == 16) and np.all(lam[:, 0] == 0.0)
    if group == 1:
        one = [host(x) for x in rdkv.allocate(*args)]
        assert all(np.array_equal(a.reshape(-1), b.reshape(-1)) for a, b in zip(one, (bt, bc, vc, lam)))


def test_shared_budget_cache_packs_and_decodes(gpu_lib):
    """A per-layer budget (group = the KV heads of a layer) moves bits between
    heads; the blob, laid out with the group budget as each segment's bound,
    packs byte for byte as the oracle's and decodes within 2e-3."""
    rdkv = gpu_lib
    S, L, Hq, Hkv, N, cap = 1, 2, 8, 2, 900, 8
    n_seg = S * L * Hkv
    w_tok, var_tok, w_chan = synth.random_unit_inputs(n_seg, N, seed=43)
    w_tok[1::2] *= np.float32(20.0)                                # the second head of each layer matters more
    K, V = synth.random_kv(n_seg, N, seed=44)
    bv, bk = int(1.2 * N) * Hkv, 80 * Hkv
    dims = rdkv.make_dims(S, L, Hq, Hkv, N)
    shp = (S, L, Hkv)
    bt, bc, _, _ = rdkv.allocate_shared(dims, dev(w_tok.reshape(shp + (N,))), dev(var_tok.reshape(shp + (N,))),
                                        dev(w_chan.reshape(shp + (128,))), dev(K.reshape(shp + (N, 128))), bv, bk,
                                        Hkv)
    per_seg = host(bt).reshape(n_seg, N).astype(np.int64).sum(axis=1)
    assert per_seg[1] > bv // Hkv and per_seg[0] < bv // Hkv      # not an even split
    lay = rdkv.layout(dims, bv, bk, cap)
    ol = O.Layout(S, L, Hq, Hkv, 128, N, bv, bk, cap)
    cache = rdkv.cache_init(lay)
    rdkv.pack(lay, cache, dev(K.reshape(shp + (N, 128))), dev(V.reshape(shp + (N, 128))), bt, bc)
    oblob = O.pack_cache(ol, K.reshape(shp + (N, 128)), V.reshape(shp + (N, 128)), host(bt), host(bc))
    assert np.array_equal(host(cache), oblob)
    _decode_run(rdkv, lay, ol, cache, oblob, 4, 45)


def _seg_shapes_contiguous(lay, cache):
    """(prefill-token chunks, K record bytes) of each segment of the prefill
    blob, from its descriptor on the host."""
    ints = host(cache)[256:256 + 256 * lay.n_seg].reshape(lay.n_seg, 256).view(np.int32)
    return [(sum(-(-int(n) // (lay.chunk_tok2 >> g)) for g, n in enumerate(ints[s, 0:4])), int(ints[s, 9]))
            for s in range(lay.n_seg)]


@pytest.mark.parametrize("G", [4, 1, 8])
def test_shared_budget_cache_decodes_with_measured_shape(gpu_lib, G):
    """A contiguous blob laid out for a per-layer budget (each segment's
    bound is the layer's budget): the measured launch shape matches the
    descriptors and stays within the bounds, the shaped decode agrees with the
    bounds-shaped one within 1e-6 over steps with appends (caches byte-equal),
    and after layer 1 is repacked with one head holding nearly the whole
    budget, the old shape gives that segment NaN outputs and the others the
    same values; a new shape covers it."""
    rdkv = gpu_lib
    S, L, Hkv, N, cap = 1, 2, 2, 3000, 16
    Hq, n_seg = G * Hkv, S * L * Hkv
    w_tok, var_tok, w_chan = synth.random_unit_inputs(n_seg, N, seed=61)
    K, V = synth.random_kv(n_seg, N, seed=62)
    bv, bk = int(1.0 * N) * Hkv, 80 * Hkv
    dims = rdkv.make_dims(S, L, Hq, Hkv, N)
    shp = (S, L, Hkv)
    Kd, Vd = dev(K.reshape(shp + (N, 128))), dev(V.reshape(shp + (N, 128)))

    def allocation(wt, budget_v):
        bt, bc, _, _ = rdkv.allocate_shared(dims, dev(wt.reshape(shp + (N,))), dev(var_tok.reshape(shp + (N,))),
                                            dev(w_chan.reshape(shp + (128,))), Kd, budget_v, bk, Hkv)
        return bt, bc

    lay = rdkv.layout(dims, bv, bk, cap)
    cache = rdkv.cache_init(lay)
    rdkv.pack(lay, cache, Kd, Vd, *allocation(w_tok, bv // 4))   # a quarter of what the layout allows
    shape = rdkv.decode_shape(lay, cache)
    segs = _seg_shapes_contiguous(lay, cache)
    assert (shape.token_slots, shape.rec_max) == (max(c for c, _ in segs), -(-max(r for _, r in segs) // 4) * 4)
    assert shape.token_slots < lay.token_slots and shape.rec_max <= lay.rec_max
    assert shape.max_chunks == shape.token_slots + lay.max_chunks - lay.token_slots
    other = cache.clone()
    ws = rdkv.decode_workspace(lay)
    ws_shape = torch.empty(int(shape.decode_workspace_bytes), dtype=torch.uint8, device=DEV)
    r = np.random.default_rng(63)
    for c_len in range(3):
        q = dev(r.standard_normal((S, L, Hq, 128)).astype(np.float16))
        kn = dev(r.standard_normal((S, L, Hkv, 128)).astype(np.float16))
        vn = dev(r.standard_normal((S, L, Hkv, 128)).astype(np.float16))
        got = host(rdkv.decode(lay, cache, c_len, q, kn, vn, workspace=ws_shape, shape=shape))
        want = host(rdkv.decode(lay, other, c_len, q, kn, vn, workspace=ws))
        assert rel_err_rows(got, want) <= 1e-6, f"step {c_len}"
    assert torch.equal(cache, other)
    # layer 1 repacked with head 0 holding nearly the whole layer budget
    w2 = w_tok.copy()
    w2[2] *= np.float32(1e4)
    bt2, bc2 = allocation(w2, bv)
    for c in (cache, other):
        rdkv.pack(lay, c, Kd[:, 1:2].contiguous(), Vd[:, 1:2].contiguous(), bt2[:, 1:2].contiguous(),
                  bc2[:, 1:2].contiguous(), layer_begin=1)
    segs2 = _seg_shapes_contiguous(lay, cache)
    assert segs2[2][0] > shape.token_slots
    q = dev(r.standard_normal((S, L, Hq, 128)).astype(np.float16))
    want = host(rdkv.decode(lay, other, 0, q, workspace=ws))
    stale = host(rdkv.decode(lay, cache, 0, q, workspace=ws_shape, shape=shape))
    for seg, (c, rec) in enumerate(segs2):
        l, h = divmod(seg, Hkv)
        rows, ref = stale[0, l, h * G:(h + 1) * G], want[0, l, h * G:(h + 1) * G]
        if c > shape.token_slots or rec > shape.rec_max:
            assert np.isnan(rows).all(), f"segment {seg} outside the shape"
        else:
            assert rel_err_rows(rows, ref) <= 1e-6, f"segment {seg}"
    shape2 = rdkv.decode_shape(lay, cache)
    ws2 = torch.empty(int(shape2.decode_workspace_bytes), dtype=torch.uint8, device=DEV)
    assert rel_err_rows(host(rdkv.decode(lay, cache, 0, q, workspace=ws2, shape=shape2)), want) <= 1e-6


# ------------------------------------------------------------------ scoring

def _score_case(w, seq=0, layer=0):
    Q, K, V = synth.prefill_layer(w, seq, layer)
    return Q, K, V


@pytest.mark.parametrize("G,Hkv,N", [(4, 1, 1024), (2, 2, 777), (8, 1, 200), (1, 1, 65)])
def test_score_matches_oracle(gpu_lib, G, Hkv, N):
    rdkv = gpu_lib
    w = synth.WORKLOADS["tiny-gqa4-n1k"].with_(n_q_heads=G * Hkv, n_kv_heads=Hkv, n_tokens=N)
    Q, K, V = _score_case(w)
    dims = rdkv.make_dims(1, 1, G * Hkv, Hkv, N)
    wt, vt, wc = rdkv.score(dims, dev(Q[None, None]), dev(K[None, None]), dev(V[None, None]))
    wt, vt, wc = host(wt)[0, 0], host(vt)[0, 0], host(wc)[0, 0]
    for h in range(Hkv):
        ref_w, ref_v, ref_c = O.score_segment(Q[h * G:(h + 1) * G], K[h], V[h])
        assert np.max(np.abs(wt[h] - ref_w) / ref_w) <= TOL
        assert np.max(np.abs(vt[h] - ref_v) / ref_v) <= TOL
        assert np.max(np.abs(wc[h] - ref_c) / ref_c) <= TOL
        assert abs(wt[h].astype(np.float64).sum() - G * N) <= TOL * G * N


@pytest.mark.parametrize("G,Hkv,N", [(4, 2, 900), (1, 1, 65), (8, 1, 200)])
def test_score_halves_match_oracle_and_compose_to_score(gpu_lib, G, Hkv, N):
    """rdkv_score_lse against the oracle's row LSE (an LSE error of 2e-3 is a
    2e-3 relative error in every attention weight of the row); rdkv_score_from_lse
    fed the oracle's LSE, as a model's prefill forward would feed it, against
    the oracle's weights; and the two halves in a row against rdkv_score."""
    rdkv = gpu_lib
    w = synth.WORKLOADS["tiny-gqa4-n1k"].with_(n_q_heads=G * Hkv, n_kv_heads=Hkv, n_tokens=N)
    Q, K, V = _score_case(w)
    dims = rdkv.make_dims(1, 1, G * Hkv, Hkv, N)
    Qd, Kd, Vd = dev(Q[None, None]), dev(K[None, None]), dev(V[None, None])
    lse = host(rdkv.score_lse(dims, Qd, Kd))[0, 0]
    ref_lse = np.stack([O.row_lse(Q[hq], K[hq // G]) for hq in range(G * Hkv)])
    assert np.max(np.abs(lse - ref_lse)) <= TOL
    wt, vt, wc = rdkv.score_from_lse(dims, Qd, Kd, Vd, dev(ref_lse.astype(np.float32)[None, None]))
    wt, vt, wc = host(wt)[0, 0], host(vt)[0, 0], host(wc)[0, 0]
    for h in range(Hkv):
        ref_w = O.token_weights_from_lse(Q[h * G:(h + 1) * G], K[h], ref_lse[h * G:(h + 1) * G])
        _, ref_v, ref_c = O.score_segment(Q[h * G:(h + 1) * G], K[h], V[h])
        assert np.max(np.abs(wt[h] - ref_w) / ref_w) <= TOL
        assert np.max(np.abs(vt[h] - ref_v) / ref_v) <= TOL
        assert np.max(np.abs(wc[h] - ref_c) / ref_c) <= TOL
    full = host(rdkv.score(dims, Qd, Kd, Vd)[0])
    comp = host(rdkv.score_from_lse(dims, Qd, Kd, Vd, rdkv.score_lse(dims, Qd, Kd))[0])
    assert np.max(np.abs(comp - full) / full) <= 1e-5


def test_score_with_a_late_dominant_key(gpu_lib):
    """A key planted at position 1500 whose logit is 60 nats (86.6 base-2
    units) while every other score is N(0, 1): pass 1's running reference, set
    by the earlier tiles, must be raised for every row that sees it (the tile
    is redone), and the rows after it put almost all their attention there,
    leaving the later tokens weights near e^-60.  Row LSE and token weights
    (RDKV summary section 2.1, w_t = sum over rows of a_{tau,t}) element by
    element against the oracle."""
    rdkv = gpu_lib
    G, N, t_hot = 4, 4096, 1500
    w = synth.WORKLOADS["tiny-gqa4-n1k"].with_(n_q_heads=G, n_kv_heads=1, n_tokens=N, outlier_channels=0)
    Q, K, V = synth.prefill_layer(w, 0, 0)
    Q[..., 0] = np.float16(4.0)
    K[..., 0] = np.float16(0.0)
    K[0, t_hot, :] = np.float16(0.0)
    K[0, t_hot, 0] = np.float16(60.0 * np.sqrt(128.0) / 4.0)
    dims = rdkv.make_dims(1, 1, G, 1, N)
    Qd, Kd, Vd = dev(Q[None, None]), dev(K[None, None]), dev(V[None, None])
    lse = host(rdkv.score_lse(dims, Qd, Kd))[0, 0]
    ref_lse = np.stack([O.row_lse(Q[g], K[0]) for g in range(G)])
    assert np.all(ref_lse[:, t_hot:] > 59.9)                      # the planted key dominates
    assert np.max(np.abs(lse - ref_lse)) <= TOL
    wt = host(rdkv.score(dims, Qd, Kd, Vd)[0])[0, 0, 0]
    ref = O.token_weights(Q, K[0])
    assert ref[t_hot] > 0.99 * G * (N - t_hot)
    assert np.max(np.abs(wt - ref) / ref) <= TOL
    assert abs(wt.astype(np.float64).sum() - G * N) <= TOL * G * N


# ------------------------------------------------------------------ end to end, tiny workload

def test_end_to_end_tiny_workload(gpu_lib):
    """score -> allocate -> pack -> 8 decode steps, all on the GPU, on the
    tiny single-layer workload, each stage held to its bar against the oracle:
    weights within 2e-3 of the fp64 oracle; the allocation bit-exact with the
    oracle's allocate_segment on the GPU's own fp32 weights and variances; the
    GPU-packed blob byte-equal to the oracle's packing of those bits; every
    decode step within 2e-3.  How closely the oracle's fully independent
    pipeline (fp64 weights) agrees on the bits is printed, not gated: a unit
    can fall on the other side of lambda only when its cost is within ~1e-6
    of it."""
    rdkv = gpu_lib
    w = synth.WORKLOADS["tiny-gqa4-n1k"]
    Q, K, V = synth.prefill_layer(w, 0, 0)
    dims = rdkv.make_dims(1, 1, w.n_q_heads, w.n_kv_heads, w.n_tokens)
    Qd, Kd, Vd = dev(Q[None, None]), dev(K[None, None]), dev(V[None, None])
    wt, vt, wc = rdkv.score(dims, Qd, Kd, Vd)
    ow, ov, oc = O.score_segment(Q, K[0], V[0])
    g_wt, g_vt, g_wc = host(wt)[0, 0, 0], host(vt)[0, 0, 0], host(wc)[0, 0, 0]
    assert np.max(np.abs(g_wt - ow) / ow) <= TOL
    assert np.max(np.abs(g_vt - ov) / ov) <= TOL
    assert np.max(np.abs(g_wc - oc) / oc) <= TOL
    bt, bc, vc, lam = rdkv.allocate(dims, wt, vt, wc, Kd, w.budget_v, w.budget_k)
    g_bt, g_bc = host(bt)[0, 0, 0], host(bc)[0, 0, 0]
    same = O.allocate_segment(g_wt, g_vt, g_wc, K[0], w.budget_v, w.budget_k)
    assert np.array_equal(g_bt, same["bits_tok"])
    assert np.array_equal(g_bc, same["bits_chan"])
    assert np.array_equal(host(vc)[0, 0, 0].view(np.uint32), same["var_chan"].view(np.uint32))
    assert tuple(host(lam)[0, 0, 0]) == (same["lambda_v"], same["lambda_k"])
    indep = O.allocate_segment(ow.astype(np.float32), ov.astype(np.float32), oc.astype(np.float32), K[0],
                               w.budget_v, w.budget_k)
    print(f"bit agreement with the oracle's fp64-weight allocation (informational): tokens "
          f"{np.mean(g_bt == indep['bits_tok']):.5f}, channels {np.mean(g_bc == indep['bits_chan']):.5f}")
    lay = rdkv.layout(dims, w.budget_v, w.budget_k, w.zone_c_capacity)
    ol = O.Layout(**w.dims(), budget_v=w.budget_v, budget_k=w.budget_k, zone_c_capacity=w.zone_c_capacity)
    cache = rdkv.cache_init(lay)
    rdkv.pack(lay, cache, Kd, Vd, bt, bc)
    oblob = O.pack_cache(ol, K[None, None], V[None, None], g_bt[None, None, None], g_bc[None, None, None])
    assert np.array_equal(host(cache), oblob)
    worst, c_len = 0.0, 0
    for step in range(w.decode_steps):
        q, kn, vn = synth.decode_inputs(w, step)
        out = rdkv.decode(lay, cache, c_len, dev(q), dev(kn), dev(vn))
        e = rel_err_rows(host(out), O.decode_step(oblob, ol, q, c_len, kn, vn))
        assert e <= TOL, f"step {step}: rel err {e:.3g}"
        worst = max(worst, e)
        c_len += 1
    assert np.array_equal(host(cache), oblob)
    print(f"end-to-end decode rel err vs the oracle: {worst:.3g}")


def test_decode_equals_its_two_phases(gpu_lib):
    rdkv = gpu_lib
    lay, ol, oblob, (K, V, bt, bc) = _pack_case(("mixed", 2, 2, 4, 2, 777, 5))
    c1 = rdkv.cache_init(lay)
    rdkv.pack(lay, c1, dev(K), dev(V), dev(bt), dev(bc))
    c2 = c1.clone()
    r = np.random.default_rng(2)
    q = dev(r.standard_normal((2, 2, 4, 128)).astype(np.float16))
    kn = dev(r.standard_normal((2, 2, 2, 128)).astype(np.float16))
    vn = dev(r.standard_normal((2, 2, 2, 128)).astype(np.float16))
    a = rdkv.decode(lay, c1, 3, q, kn, vn)
    ws = rdkv.decode_partials(lay, c2, 3, q, kn, vn)
    b = rdkv.decode_merge(lay, c2, 4, ws)
    assert torch.equal(a, b) and torch.equal(c1, c2)
    # decode is deterministic run to run
    assert torch.equal(rdkv.decode(lay, c1, 4, q), rdkv.decode(lay, c1, 4, q))


def test_decode_captured_in_a_graph_replays_like_eager(gpu_lib):
    """rdkv_decode enqueues only kernels (no memset, no allocation), so a
    caller can capture a per-layer decode loop in a HIP graph.  Every replay,
    with eager work and synchronisation between replays, must equal the eager
    call bit for bit, and the oracle within the tolerance."""
    rdkv = gpu_lib
    lay, ol, oblob, (K, V, bt, bc) = _pack_case(("mixed", 1, 2, 4, 2, 777, 5))
    cache = rdkv.cache_init(lay)
    rdkv.pack(lay, cache, dev(K), dev(V), dev(bt), dev(bc))
    r = np.random.default_rng(9)
    q = r.standard_normal((1, 2, 4, 128)).astype(np.float16)
    kn = r.standard_normal((1, 2, 2, 128)).astype(np.float16)
    vn = r.standard_normal((1, 2, 2, 128)).astype(np.float16)
    qd, knd, vnd = dev(q), dev(kn), dev(vn)
    ws = rdkv.decode_workspace(lay)
    out = torch.empty((1, 2, 4, 128), dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        rdkv.decode(lay, cache, 0, qd, knd, vnd, workspace=ws, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = out.clone()
    ref = O.decode_step(oblob, ol, q, 0, kn, vn)
    assert rel_err_rows(host(eager), ref) <= TOL
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rdkv.decode(lay, cache, 0, qd, knd, vnd, workspace=ws, out=out)
    junk = torch.empty_like(out)
    for i in range(4):
        out.fill_(float("nan"))
        junk.normal_()                           # eager work between replays
        ws.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from the eager call"
    # the appended zone-C row is the same bytes the oracle wrote
    assert np.array_equal(host(cache), oblob)


def test_decode_merge_ignores_stale_workspace(gpu_lib):
    """The partials phase writes every chunk slot of the workspace (slots past
    a segment's last chunk as empty), so whatever the workspace held before
    (here NaN everywhere) cannot leak into the merged output."""
    rdkv = gpu_lib
    lay, ol, oblob, (K, V, bt, bc) = _pack_case(("empty_and_single", 1, 2, 8, 2, 300, 4))
    cache = rdkv.cache_init(lay)
    rdkv.pack(lay, cache, dev(K), dev(V), dev(bt), dev(bc))
    r = np.random.default_rng(4)
    q = r.standard_normal((1, 2, 8, 128)).astype(np.float16)
    ws = rdkv.decode_workspace(lay)
    clean = rdkv.decode(lay, cache.clone(), 1, dev(q), workspace=ws.zero_())
    ws.view(torch.float32).fill_(float("nan"))
    dirty = rdkv.decode(lay, cache, 1, dev(q), workspace=ws)
    assert torch.equal(clean, dirty)
    assert not torch.isnan(dirty).any()
    ref = O.decode_step(oblob, ol, q, 1)
    assert rel_err_rows(host(dirty), ref) <= TOL
