"""Guard bands around every buffer the library writes.

Each output, workspace, cache and staging buffer is placed inside a larger
allocation with 4 KiB of a known byte pattern on both sides, sized exactly as
the library's size queries say (so a write one byte past the end lands in a
guard), and the whole path runs through the C ABI: scoring (both halves too),
allocation (per segment and shared), cache init and pack, decode (one call
and two phases), decode with zone-C statistics and rollover, and the paged
stage / commit / decode / release.  Shapes have ragged tails (N not a multiple
of 64, partial chunks) and G = 4 and 8.  After every call the guards must be
intact.
"""
import ctypes

import numpy as np
import pytest
import torch

from decode_attention_rdkv_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
GUARD = 4096
PATTERN = 0xA5


@pytest.fixture(scope="module")
def rdkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_attention_rdkv_amd import rdkv as lib
    lib.load()
    return lib


class Guarded:
    """A tensor view with GUARD bytes of PATTERN on both sides."""

    def __init__(self, shape, dtype, fill=None):
        shape = tuple(shape) if isinstance(shape, (tuple, list)) else (shape,)
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        self.n = n
        self.raw = torch.full((n + 2 * GUARD,), PATTERN, dtype=torch.uint8, device=DEV)
        body = self.raw[GUARD:GUARD + n]
        if fill is not None:
            body.fill_(fill)
        self.t = body.view(dtype).view(shape)

    def check(self, what):
        torch.cuda.synchronize()
        g = torch.cat([self.raw[:GUARD], self.raw[GUARD + self.n:]]).cpu().numpy()
        bad = np.nonzero(g != PATTERN)[0]
        assert bad.size == 0, f"{what}: {bad.size} guard bytes overwritten (first at {bad[:4]})"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _inputs(S, L, Hq, Hkv, N, seed):
    r = np.random.default_rng(seed)
    Q = (r.standard_normal((S, L, Hq, N, 128)) * 0.5).astype(np.float16)
    K = r.standard_normal((S, L, Hkv, N, 128)).astype(np.float16)
    V = r.standard_normal((S, L, Hkv, N, 128)).astype(np.float16)
    return dev(Q), dev(K), dev(V)


@pytest.mark.parametrize("G", [4, 8])
def test_score_allocate_pack_decode_write_only_their_buffers(rdkv, G):
    lib = rdkv.load()
    S, L, Hkv, N, cap = 2, 2, 2, 1000, 70
    Hq = G * Hkv
    bv, bk = 2 * N, 2 * 128
    dims = rdkv.make_dims(S, L, Hq, Hkv, N)
    Q, K, V = _inputs(S, L, Hq, Hkv, N, G)
    shp = (S, L, Hkv)
    # scoring, one call and its two halves
    ws = Guarded(lib.rdkv_score_workspace_bytes(ctypes.byref(dims)), torch.uint8)
    wt, vt, wc = Guarded(shp + (N,), torch.float32), Guarded(shp + (N,), torch.float32), Guarded(shp + (128,), torch.float32)
    assert lib.rdkv_score(ctypes.byref(dims), Q.data_ptr(), K.data_ptr(), V.data_ptr(), wt.t.data_ptr(),
                          vt.t.data_ptr(), wc.t.data_ptr(), ws.t.data_ptr(), ws.n, stream()) == 0
    for b, what in ((ws, "score workspace"), (wt, "w_tok"), (vt, "var_tok"), (wc, "w_chan")):
        b.check(what)
    lse = Guarded((S, L, Hq, N), torch.float32)
    assert lib.rdkv_score_lse(ctypes.byref(dims), Q.data_ptr(), K.data_ptr(), lse.t.data_ptr(), stream()) == 0
    lse.check("row LSE")
    wt2, vt2, wc2 = Guarded(shp + (N,), torch.float32), Guarded(shp + (N,), torch.float32), Guarded(shp + (128,), torch.float32)
    assert lib.rdkv_score_from_lse(ctypes.byref(dims), Q.data_ptr(), K.data_ptr(), V.data_ptr(), lse.t.data_ptr(),
                                   wt2.t.data_ptr(), vt2.t.data_ptr(), wc2.t.data_ptr(), ws.t.data_ptr(), ws.n,
                                   stream()) == 0
    for b, what in ((ws, "score workspace"), (wt2, "w_tok from LSE"), (vt2, "var_tok from LSE"), (wc2, "w_chan from LSE")):
        b.check(what)
    # allocation, per segment and with one budget per layer
    outs = [Guarded(shp + (N,), torch.uint8), Guarded(shp + (128,), torch.uint8), Guarded(shp + (128,), torch.float32),
            Guarded(shp + (2,), torch.float64)]
    aws = Guarded(lib.rdkv_allocate_workspace_bytes(ctypes.byref(dims), 1), torch.uint8)
    assert lib.rdkv_allocate(ctypes.byref(dims), wt.t.data_ptr(), vt.t.data_ptr(), wc.t.data_ptr(), K.data_ptr(), bv, bk,
                             *(o.t.data_ptr() for o in outs), aws.t.data_ptr(), aws.n, stream()) == 0
    for o, what in zip(outs + [aws], ("bits_tok", "bits_chan", "var_chan", "lambda", "allocation workspace")):
        o.check(what)
    shared = [Guarded(shp + (N,), torch.uint8), Guarded(shp + (128,), torch.uint8), Guarded(shp + (128,), torch.float32),
              Guarded(shp + (2,), torch.float64)]
    aws = Guarded(lib.rdkv_allocate_workspace_bytes(ctypes.byref(dims), Hkv), torch.uint8)
    assert lib.rdkv_allocate_shared(ctypes.byref(dims), wt.t.data_ptr(), vt.t.data_ptr(), wc.t.data_ptr(), K.data_ptr(),
                                    bv * Hkv, bk * Hkv, Hkv, *(o.t.data_ptr() for o in shared), aws.t.data_ptr(),
                                    aws.n, stream()) == 0
    for o, what in zip(shared + [aws], ("shared bits_tok", "shared bits_chan", "shared var_chan", "shared lambda",
                                        "shared allocation workspace")):
        o.check(what)
    bt, bc = outs[0].t, outs[1].t
    # cache init, pack, decode (one call, two phases), with appends
    lay = rdkv.layout(dims, bv, bk, cap)
    cache = Guarded(lay.cache_bytes, torch.uint8)
    rdkv.cache_init(lay, cache.t)
    cache.check("cache after init")
    rdkv.pack(lay, cache.t, K, V, bt, bc)
    cache.check("cache after pack")
    wsd = Guarded(lay.decode_workspace_bytes, torch.uint8)
    out = Guarded((S, L, Hq, 128), torch.float32)
    r = np.random.default_rng(7)
    for step in range(cap):
        q = dev(r.standard_normal((S, L, Hq, 128)).astype(np.float16))
        kn = dev(r.standard_normal((S, L, Hkv, 128)).astype(np.float16))
        vn = dev(r.standard_normal((S, L, Hkv, 128)).astype(np.float16))
        if step % 2:
            rdkv.decode(lay, cache.t, step, q, kn, vn, workspace=wsd.t, out=out.t)
        else:
            rdkv.decode_partials(lay, cache.t, step, q, kn, vn, workspace=wsd.t)
            rdkv.decode_merge(lay, cache.t, step + 1, wsd.t, out.t)
        if step in (0, 1, 63, 64, cap - 1):
            for b, what in ((cache, "cache"), (wsd, "decode workspace"), (out, "decode output")):
                b.check(f"{what} at step {step}")
    assert torch.isfinite(out.t).all()


def test_rollover_writes_only_its_buffers(rdkv):
    S, L, Hq, Hkv, N, cap, n_gen = 1, 2, 8, 2, 500, 64, 2
    n_seg = S * L * Hkv
    bt, bc = synth.random_bits(n_seg, N, 3)
    K, V = synth.random_kv(n_seg, N, 4)
    bv, bk = int(bt.astype(np.int64).sum(axis=1).max()), int(bc.astype(np.int64).sum(axis=1).max())
    dims = rdkv.make_dims(S, L, Hq, Hkv, N)
    lay = rdkv.layout_rollover(dims, bv, bk, cap, n_gen, 2 * cap, 2 * 128)
    cache = Guarded(lay.cache_bytes, torch.uint8)
    rdkv.cache_init(lay, cache.t)
    shp = (S, L, Hkv)
    rdkv.pack(lay, cache.t, *(dev(a.reshape(shp + a.shape[1:])) for a in (K, V, bt, bc)))
    stats = Guarded((S, L, Hkv, Hq // Hkv, cap + 128), torch.float32, fill=0)
    wsd = Guarded(lay.decode_workspace_bytes, torch.uint8)
    rws = Guarded(lay.rollover_workspace_bytes, torch.uint8)
    out = Guarded((S, L, Hq, 128), torch.float32)
    r = np.random.default_rng(5)
    for gen in range(n_gen):
        for t in range(cap):
            q = dev(r.standard_normal((S, L, Hq, 128)).astype(np.float16))
            kn = dev(r.standard_normal((S, L, Hkv, 128)).astype(np.float16))
            vn = dev(r.standard_normal((S, L, Hkv, 128)).astype(np.float16))
            rdkv.decode_accumulate(lay, cache.t, t, q, kn, vn, stats.t, workspace=wsd.t, out=out.t)
        for b, what in ((cache, "cache"), (stats, "zone-C statistics"), (wsd, "decode workspace"), (out, "output")):
            b.check(f"{what} before rollover {gen}")
        rdkv.rollover(lay, cache.t, gen, stats.t, workspace=rws.t)
        for b, what in ((cache, "cache"), (stats, "zone-C statistics"), (rws, "rollover workspace")):
            b.check(f"{what} after rollover {gen}")
    q = dev(r.standard_normal((S, L, Hq, 128)).astype(np.float16))
    rdkv.decode(lay, cache.t, 0, q, workspace=wsd.t, out=out.t)
    out.check("output over every generation")
    assert torch.isfinite(out.t).all()
    # the same step with the prefill blob's measured launch shape (the
    # generations keep their own slots): only its buffers written, and the
    # same outputs up to the merge's rounding
    scan = Guarded(8, torch.uint8)
    shape = rdkv.decode_shape(lay, cache.t, scan.t)
    wss = Guarded(int(shape.decode_workspace_bytes), torch.uint8)
    out2 = Guarded((S, L, Hq, 128), torch.float32)
    rdkv.decode(lay, cache.t, 0, q, workspace=wss.t, out=out2.t, shape=shape)
    for b, what in ((scan, "shape scan buffer"), (cache, "cache"), (wss, "shaped decode workspace"),
                    (out2, "shaped output")):
        b.check(f"{what} with the measured shape")
    a, b = out2.t.double(), out.t.double()
    assert float(((a - b).abs().amax(-1) / b.abs().amax(-1).clamp_min(1e-30)).max()) <= 1e-6


def test_paged_path_writes_only_its_buffers(rdkv):
    S, L, Hq, Hkv, cap, n_pages = 3, 2, 8, 2, 70, 300
    shapes = [(700, 1400, 256), (1100, 3000, 384), (200, 200, 100)]
    pl = rdkv.paged_layout(rdkv.make_dims(S, L, Hq, Hkv, 1100), 3000, 384, cap, n_pages)
    cache = Guarded(pl.cache_bytes, torch.uint8)
    rdkv.paged_cache_init(pl, cache.t)
    cache.check("paged cache after init")
    free = list(np.random.default_rng(1).permutation(n_pages))
    for s, (N, bv, bk) in enumerate(shapes):
        n = L * Hkv
        bt, bc = synth.random_bits(n, N, 10 + s)
        for i in range(n):
            while int(bt[i].astype(np.int64).sum()) > bv:
                bt[i, np.nonzero(bt[i])[0][:10]] = 0
            while int(bc[i].astype(np.int64).sum()) > bk:
                bc[i, np.nonzero(bc[i])[0][0]] = 0
        K, V = synth.random_kv(n, N, 20 + s)
        staging = Guarded(rdkv.paged_staging_bytes(pl, N, bv, bk), torch.uint8)
        shp = (L, Hkv)
        _, need = rdkv.paged_stage(pl, N, bv, bk, *(dev(a.reshape(shp + a.shape[1:])) for a in (K, V, bt, bc)),
                                   staging=staging.t)
        staging.check(f"staging of sequence {s}")
        need = need.cpu().numpy()
        table = np.full((n, pl.max_pages), -1, np.int32)
        for i, k in enumerate(need):
            table[i, :k] = free[:k]
            free = free[k:]
        rdkv.paged_commit(pl, cache.t, s, N, bv, bk, staging.t, dev(table))
        cache.check(f"paged cache after committing sequence {s}")
    wsd = Guarded(pl.decode_workspace_bytes, torch.uint8)
    out = Guarded((S, L, Hq, 128), torch.float32)
    r = np.random.default_rng(2)
    c_len = [0, 5, 63]
    for step in range(4):
        q = dev(r.standard_normal((S, L, Hq, 128)).astype(np.float16))
        kn = dev(r.standard_normal((S, L, Hkv, 128)).astype(np.float16))
        vn = dev(r.standard_normal((S, L, Hkv, 128)).astype(np.float16))
        rdkv.paged_decode(pl, cache.t, c_len, q, kn, vn, workspace=wsd.t, out=out.t)
        for b, what in ((cache, "paged cache"), (wsd, "paged decode workspace"), (out, "paged output")):
            b.check(f"{what} at step {step}")
        c_len = [c + 1 for c in c_len]
    # the measured launch shape: its 8-byte scan buffer, then a shaped step in
    # a workspace of exactly the shape's size
    scan = Guarded(8, torch.uint8)
    shape = rdkv.paged_decode_shape(pl, cache.t, scan.t)
    scan.check("shape scan buffer")
    cache.check("paged cache after the shape scan")
    wss = Guarded(int(shape.decode_workspace_bytes), torch.uint8)
    q = dev(r.standard_normal((S, L, Hq, 128)).astype(np.float16))
    kn = dev(r.standard_normal((S, L, Hkv, 128)).astype(np.float16))
    vn = dev(r.standard_normal((S, L, Hkv, 128)).astype(np.float16))
    rdkv.paged_decode(pl, cache.t, c_len, q, kn, vn, workspace=wss.t, out=out.t, shape=shape)
    for b, what in ((cache, "paged cache"), (wss, "shaped decode workspace"), (out, "paged output")):
        b.check(f"{what} after a shaped step")
    rdkv.paged_release(pl, cache.t, 1)
    cache.check("paged cache after release")
    assert torch.isfinite(out.t).all()
