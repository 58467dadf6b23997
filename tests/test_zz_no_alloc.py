"""rdkv_decode_static, the decode entry point that allocates nothing (its
split-K partials live in a library-owned device array), against rdkv_decode
through the C ABI: the same outputs and the same zone-C appends, bit for bit,
on two calls in a row, the second on a smaller cache; and the outputs within
2e-3 of the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
from decode_attention_rdkv_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 2e-3


def _case(rdkv, S, L, Hq, Hkv, N, cap, seed):
    bt, bc = synth.random_bits(S * L * Hkv, N, seed)
    K, V = synth.random_kv(S * L * Hkv, N, seed + 1)
    bv, bk = int(bt.astype(np.int64).sum(axis=1).max()), int(bc.astype(np.int64).sum(axis=1).max())
    lay = rdkv.layout(rdkv.make_dims(S, L, Hq, Hkv, N), bv, bk, cap)
    ol = O.Layout(S, L, Hq, Hkv, 128, N, bv, bk, cap)
    shp = (S, L, Hkv)
    args = (K.reshape(shp + (N, 128)), V.reshape(shp + (N, 128)), bt.reshape(shp + (N,)), bc.reshape(shp + (128,)))
    cache = rdkv.cache_init(lay)
    rdkv.pack(lay, cache, *(torch.from_numpy(a).to(DEV) for a in args))
    return lay, ol, cache, O.pack_cache(ol, *args)


def test_static_decode_equals_workspace_decode():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_attention_rdkv_amd import rdkv
    rdkv.load()
    # the second call has fewer segments, tokens and chunk slots than the first,
    # so it leaves the first call's partials in the scratch beyond its own
    shapes = [(2, 3, 8, 2, 3000, 6, 11), (1, 1, 4, 1, 500, 3, 12)]
    for S, L, Hq, Hkv, N, cap, seed in shapes:
        lay, ol, cache, oblob = _case(rdkv, S, L, Hq, Hkv, N, cap, seed)
        print(f"S={S} L={L} Hq={Hq} Hkv={Hkv} N={N}: {lay.n_seg} segments x {lay.max_chunks} chunk slots, "
              f"partials {lay.decode_workspace_bytes} B", flush=True)
        r = np.random.default_rng(seed)
        q = torch.from_numpy(r.standard_normal((S, L, Hq, 128)).astype(np.float16)).to(DEV)
        kn = torch.from_numpy(r.standard_normal((S, L, Hkv, 128)).astype(np.float16)).to(DEV)
        vn = torch.from_numpy(r.standard_normal((S, L, Hkv, 128)).astype(np.float16)).to(DEV)
        ref_cache = cache.clone()
        ref = rdkv.decode(lay, ref_cache, 1, q, kn, vn)
        out = torch.full((S, L, Hq, 128), float("nan"), dtype=torch.float32, device=DEV)
        rdkv.decode_static(lay, cache, 1, q, kn, vn, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "static-scratch decode differs from the workspace decode"
        assert torch.equal(cache, ref_cache), "zone-C append differs"
        O.append_zone_c(oblob, ol, 1, kn.cpu().numpy(), vn.cpu().numpy())
        oref = O.decode_step(oblob, ol, q.cpu().numpy(), 2)
        got = out.cpu().numpy().astype(np.float64)
        err = float((np.abs(got - oref).max(-1) / np.maximum(np.abs(oref).max(-1), 1e-30)).max())
        assert err <= TOL, f"rel err {err:.3g}"
        # and without an append
        ref2 = rdkv.decode(lay, ref_cache, 2, q)
        out2 = rdkv.decode_static(lay, cache, 2, q, out=torch.empty_like(out))
        assert torch.equal(out2, ref2)
