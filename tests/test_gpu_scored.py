"""The whole path on the workloads' own inputs at full size: scored,
allocated and packed on the GPU, then decoded, each stage against the oracle.

Scoring is compared element by element with the fp64 oracle where the oracle
finishes in seconds (one KV head of the 32K layer); the allocation with the
oracle's allocation of the GPU's own fp32 weights (bit-exact); the packed
bytes with the oracle's packing of the GPU's bits (bit-exact); decode within
2e-3 (per query head, max |out - ref| over the channels / max |ref|), in the
launch configuration the benchmark times: one launch over every segment of
the cache.  Where the oracle cannot afford every segment it takes a sample,
named in each test; segments are independent in the format and the kernels.
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


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float((np.abs(got - ref).max(axis=-1) / np.maximum(np.abs(ref).max(axis=-1), 1e-30)).max())


def _score_alloc_layer(rdkv, w, seq, layer, dims1):
    """Score and allocate one (sequence, layer) on the GPU; returns device K,
    V, bits and the fp32 weights (host) the allocation was computed from."""
    Q, K, V = synth.prefill_layer(w, seq, layer, device=DEV)
    K5, V5 = K[None, None].contiguous(), V[None, None].contiguous()
    wt, vt, wc = rdkv.score(dims1, Q[None, None].contiguous(), K5, V5)
    del Q
    bt, bc, vc, lam = rdkv.allocate(dims1, wt, vt, wc, K5, w.budget_v, w.budget_k)
    return K5, V5, bt, bc, dict(wt=wt, vt=vt, wc=wc, vc=vc, lam=lam)


def _check_allocation(rdkv, w, K5, bt, bc, st, heads):
    """Bits, variances and lambdas of the given heads against the oracle's
    allocation of the GPU's own fp32 weights."""
    wt, vt, wc = host(st["wt"])[0, 0], host(st["vt"])[0, 0], host(st["wc"])[0, 0]
    bth, bch, vch, lam = host(bt)[0, 0], host(bc)[0, 0], host(st["vc"])[0, 0], host(st["lam"])[0, 0]
    Kh = host(K5)[0, 0]
    for h in heads:
        ref = O.allocate_segment(wt[h], vt[h], wc[h], Kh[h], w.budget_v, w.budget_k)
        assert np.array_equal(bth[h], ref["bits_tok"]), f"head {h}: V bits"
        assert np.array_equal(bch[h], ref["bits_chan"]), f"head {h}: K bits"
        assert np.array_equal(vch[h].view(np.uint32), ref["var_chan"].view(np.uint32)), f"head {h}: var_chan"
        assert tuple(lam[h]) == (ref["lambda_v"], ref["lambda_k"]), f"head {h}: lambda"


def _oracle_blob_skeleton(ol):
    """Header and empty descriptors of every segment, as rdkv_cache_init
    writes them; slots of segments the oracle does not pack stay zero."""
    blob = np.zeros(ol.cache_bytes, np.uint8)
    blob[:O.HEADER_BYTES] = np.frombuffer(ol.header_bytes(), np.uint8)
    z16 = np.zeros((0, 128), np.float16)
    for seg in range(ol.n_seg):
        O.pack_segment(ol, blob, seg, z16, z16, np.zeros(0, np.uint8), np.zeros(128, np.uint8))
    return blob


def _segment_bytes_equal(cache, oblob, ol, seg):
    d0 = ol.desc_offset + seg * O.DESC_BYTES
    b0 = ol.slot_base(seg)
    assert np.array_equal(host(cache[d0:d0 + O.DESC_BYTES]), oblob[d0:d0 + O.DESC_BYTES]), f"descriptor {seg}"
    assert np.array_equal(host(cache[b0:b0 + ol.slot_bytes]), oblob[b0:b0 + ol.slot_bytes]), f"slot {seg}"


class _SegmentRef:
    """The oracle's decode of one segment over several steps: its kept rows are
    dequantized once (O.unpack_segment), zone C is re-read from the oracle's
    blob at every step, and the output is O.attention over both, which is
    what O.decode_segment computes."""

    def __init__(self, oblob, ol, seg):
        self.oblob, self.ol, self.seg = oblob, ol, seg
        self.Kh, self.Vh, _, _ = O.unpack_segment(oblob, ol, seg)

    def out(self, qg, n_c):
        kc, vc = O.zone_c_rows(self.oblob, self.ol, self.seg, n_c)
        return O.attention(np.asarray(qg, np.float16).astype(np.float64), np.concatenate([self.Kh, kc]),
                           np.concatenate([self.Vh, vc]))


# ------------------------------------------------------------------ 32K layer: scoring at full length

@pytest.fixture(scope="module")
def layer32k(rdkv):
    w = synth.WORKLOADS["llama8b-layer-n32k"]
    Q, K, V = synth.prefill_layer(w, 0, 0)
    dims = rdkv.make_dims(1, 1, w.n_q_heads, w.n_kv_heads, w.n_tokens)
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    Qd, Kd, Vd = to(Q[None, None]), to(K[None, None]), to(V[None, None])
    wt, vt, wc = rdkv.score(dims, Qd, Kd, Vd)
    lse = rdkv.score_lse(dims, Qd, Kd)
    return dict(w=w, Q=Q, K=K, V=V, wt=host(wt)[0, 0], vt=host(vt)[0, 0], wc=host(wc)[0, 0],
                lse=host(lse)[0, 0], dims=dims, Kd=Kd, Vd=Vd, wt_d=wt, vt_d=vt, wc_d=wc)


def test_token_weights_of_a_32k_head_elementwise(layer32k):
    """w_t of KV head 0 of the 32K layer (its 4 query heads, 10% of tokens at
    +3 logits) against the fp64 oracle at every one of the 32,768 tokens
    (RDKV summary section 2.1: w_t = sum over query rows of a_{tau,t}); the
    token variances and channel weights of all 8 heads likewise."""
    c = layer32k
    G = c["w"].group
    ref = O.token_weights(c["Q"][:G], c["K"][0])
    err = float(np.max(np.abs(c["wt"][0] - ref) / ref))
    print(f"32K head 0: max rel err of w_t {err:.3g}")
    assert err <= TOL
    for h in range(c["w"].n_kv_heads):
        ref_v = O.token_variance(c["V"][h])
        ref_c = O.channel_weights(c["Q"][h * G:(h + 1) * G], c["K"][h])
        assert np.max(np.abs(c["vt"][h] - ref_v) / ref_v) <= TOL
        assert np.max(np.abs(c["wc"][h] - ref_c) / ref_c) <= TOL


def test_row_lse_of_a_32k_head_elementwise(layer32k):
    """The row LSE of the 4 query heads of KV head 0 of the 32K layer against
    the oracle's, at every row (an error of 2e-3 in it is a 2e-3 relative
    error in every attention weight of the row)."""
    c = layer32k
    G = c["w"].group
    ref = np.stack([O.row_lse(c["Q"][g], c["K"][0]) for g in range(G)])
    err = float(np.max(np.abs(c["lse"][:G] - ref)))
    print(f"32K head 0: max abs err of the row LSE {err:.3g}")
    assert err <= TOL


def test_scored_32k_layer_packs_and_decodes_64_steps(rdkv, layer32k):
    """The 32K layer's GPU allocation (all 8 segments) bit-exact with the
    oracle's on the same fp32 weights, the whole packed blob byte-equal, then
    64 decode steps appending one token each, checked on all 8 segments at
    every 8th step and the last."""
    c = layer32k
    w, dims = c["w"], c["dims"]
    bt, bc, vc, lam = rdkv.allocate(dims, c["wt_d"], c["vt_d"], c["wc_d"], c["Kd"], w.budget_v, w.budget_k)
    st = dict(wt=c["wt_d"], vt=c["vt_d"], wc=c["wc_d"], vc=vc, lam=lam)
    _check_allocation(rdkv, w, c["Kd"], bt, bc, st, range(w.n_kv_heads))
    lay = rdkv.layout(dims, w.budget_v, w.budget_k, w.zone_c_capacity)
    ol = O.Layout(**w.dims(), budget_v=w.budget_v, budget_k=w.budget_k, zone_c_capacity=w.zone_c_capacity)
    cache = rdkv.cache_init(lay)
    rdkv.pack(lay, cache, c["Kd"], c["Vd"], bt, bc)
    oblob = O.pack_cache(ol, c["K"][None, None], c["V"][None, None], host(bt), host(bc))
    assert np.array_equal(host(cache), oblob)
    refs = [_SegmentRef(oblob, ol, seg) for seg in range(lay.n_seg)]
    ws = rdkv.decode_workspace(lay)
    G = w.group
    worst = 0.0
    for step in range(w.decode_steps):
        q, kn, vn = synth.decode_inputs(w, step)
        out = rdkv.decode(lay, cache, step, torch.from_numpy(q).to(DEV), torch.from_numpy(kn).to(DEV),
                          torch.from_numpy(vn).to(DEV), workspace=ws)
        O.append_zone_c(oblob, ol, step, kn, vn)
        if step % 8 == 0 or step == w.decode_steps - 1:
            out = host(out)
            for h, ref in enumerate(refs):
                e = rel_err(out[0, 0, h * G:(h + 1) * G], ref.out(q[0, 0, h * G:(h + 1) * G], step + 1))
                worst = max(worst, e)
                assert e <= TOL, f"step {step} head {h}: rel err {e:.3g}"
    print(f"32K layer, 64 steps: worst rel err {worst:.3g}")
    assert np.array_equal(host(cache), oblob)


# ------------------------------------------------------------------ 128K x 32 layers, one launch

def test_scored_128k_cache_single_launch(rdkv):
    """The headline cache as the benchmark builds it: all 32 layers scored,
    allocated and packed on the GPU, decoded in one launch over all 256
    segments.  Sampled segments (layers 0, 13, 31; heads 0, 5, 7): allocation
    bit-exact, packed bytes equal, two decode steps (append, then none)
    within 2e-3."""
    w = synth.WORKLOADS["llama8b-32layer-n128k"]
    S, L, Hq, Hkv, N, G = w.n_seq, w.n_layers, w.n_q_heads, w.n_kv_heads, w.n_tokens, w.group
    dims1 = rdkv.make_dims(S, 1, Hq, Hkv, N)
    lay = rdkv.layout(rdkv.make_dims(S, L, Hq, Hkv, N), w.budget_v, w.budget_k, w.zone_c_capacity)
    ol = O.Layout(**w.dims(), budget_v=w.budget_v, budget_k=w.budget_k, zone_c_capacity=w.zone_c_capacity)
    sampled = {0: (0,), 13: (5,), 31: (7,)}
    cache = rdkv.cache_init(lay)
    oblob = _oracle_blob_skeleton(ol)
    for l in range(L):
        K5, V5, bt, bc, st = _score_alloc_layer(rdkv, w, 0, l, dims1)
        rdkv.pack(lay, cache, K5, V5, bt, bc, layer_begin=l, check=False)
        if l in sampled:
            _check_allocation(rdkv, w, K5, bt, bc, st, sampled[l])
            Kh, Vh, bth, bch = host(K5)[0, 0], host(V5)[0, 0], host(bt)[0, 0], host(bc)[0, 0]
            for h in sampled[l]:
                O.pack_segment(ol, oblob, ol.seg_index(0, l, h), Kh[h], Vh[h], bth[h], bch[h])
            print(f"layer {l}: token bits 0/2/4/8/16 {np.bincount(bth.ravel(), minlength=17)[[0, 2, 4, 8, 16]]}",
                  flush=True)
        del K5, V5, bt, bc, st
    assert rdkv.pack_status(lay, cache).item() == 0
    segs = [ol.seg_index(0, l, h) for l, hs in sampled.items() for h in hs]
    for seg in segs:
        _segment_bytes_equal(cache, oblob, ol, seg)
    refs = {seg: _SegmentRef(oblob, ol, seg) for seg in segs}
    ws = rdkv.decode_workspace(lay)
    for step, append in enumerate((True, False)):
        q, kn, vn = synth.decode_inputs(w, step)
        c_len = 0 if append else 1
        out = host(rdkv.decode(lay, cache, c_len, torch.from_numpy(q).to(DEV),
                               torch.from_numpy(kn).to(DEV) if append else None,
                               torch.from_numpy(vn).to(DEV) if append else None, workspace=ws))
        if append:
            O.append_zone_c(oblob, ol, 0, kn, vn)
        for l, hs in sampled.items():
            for h in hs:
                seg = ol.seg_index(0, l, h)
                e = rel_err(out[0, l, h * G:(h + 1) * G], refs[seg].out(q[0, l, h * G:(h + 1) * G], 1))
                print(f"  step {step} layer {l} head {h}: rel err {e:.3g}", flush=True)
                assert e <= TOL


# ------------------------------------------------------------------ 16 x 32K batch, 256 appends

def test_scored_batch_256_appends(rdkv):
    """The 16-sequence batch: every sequence scored and allocated on its own
    (zone sizes differ per sequence), packed into one blob, then 256 decode
    steps each appending one token per segment (zone C fills to its 256 rows),
    decoded in one launch per step.  One segment per sequence (KV head
    s mod 8) is checked: allocation bit-exact, bytes equal, and outputs at
    steps 0, 127 and 255."""
    w = synth.WORKLOADS["llama8b-batch16-n32k"]
    S, Hq, Hkv, N, G = w.n_seq, w.n_q_heads, w.n_kv_heads, w.n_tokens, w.group
    dims1 = rdkv.make_dims(1, 1, Hq, Hkv, N)
    lay = rdkv.layout(rdkv.make_dims(S, 1, Hq, Hkv, N), w.budget_v, w.budget_k, w.zone_c_capacity)
    ol = O.Layout(**w.dims(), budget_v=w.budget_v, budget_k=w.budget_k, zone_c_capacity=w.zone_c_capacity)
    cache = rdkv.cache_init(lay)
    oblob = _oracle_blob_skeleton(ol)
    Ks, Vs, bts, bcs = [], [], [], []
    kept = []
    for s in range(S):
        K5, V5, bt, bc, st = _score_alloc_layer(rdkv, w, s, 0, dims1)
        h = s % Hkv
        _check_allocation(rdkv, w, K5, bt, bc, st, (h,))
        O.pack_segment(ol, oblob, ol.seg_index(s, 0, h), host(K5)[0, 0, h], host(V5)[0, 0, h], host(bt)[0, 0, h],
                       host(bc)[0, 0, h])
        kept.append(int((host(bt)[0, 0, h] > 0).sum()))
        Ks.append(K5), Vs.append(V5), bts.append(bt), bcs.append(bc)
        del st
    rdkv.pack(lay, cache, torch.cat(Ks), torch.cat(Vs), torch.cat(bts), torch.cat(bcs))
    del Ks, Vs, bts, bcs
    print(f"kept tokens of the checked segments: {kept}", flush=True)
    assert len(set(kept)) > 1                      # zone sizes differ between sequences
    segs = [ol.seg_index(s, 0, s % Hkv) for s in range(S)]
    for seg in segs:
        _segment_bytes_equal(cache, oblob, ol, seg)
    refs = {seg: _SegmentRef(oblob, ol, seg) for seg in segs}
    ws = rdkv.decode_workspace(lay)
    worst = 0.0
    for step in range(w.decode_steps):
        q, kn, vn = synth.decode_inputs(w, step)
        out = rdkv.decode(lay, cache, step, torch.from_numpy(q).to(DEV), torch.from_numpy(kn).to(DEV),
                          torch.from_numpy(vn).to(DEV), workspace=ws)
        O.append_zone_c(oblob, ol, step, kn, vn)
        if step in (0, 127, 255):
            out = host(out)
            for s in range(S):
                h = s % Hkv
                e = rel_err(out[s, 0, h * G:(h + 1) * G], refs[segs[s]].out(q[s, 0, h * G:(h + 1) * G], step + 1))
                worst = max(worst, e)
                assert e <= TOL, f"step {step} sequence {s}: rel err {e:.3g}"
            print(f"  step {step}: worst rel err so far {worst:.3g}", flush=True)
    for seg in segs:
        _segment_bytes_equal(cache, oblob, ol, seg)


# ------------------------------------------------------------------ 72B-shaped layer at 256K (G = 8)

def test_scored_256k_layer_g8(rdkv):
    """One layer of the 72B-shaped stack (64 query heads over 8 KV heads,
    log-normal K channel scales, 262,144 tokens) scored, allocated and packed
    on the GPU; heads 0, 4 and 7 checked: allocation bit-exact, bytes equal,
    two decode steps within 2e-3 (8 query heads per KV head: the kernel's
    paired waves)."""
    w = synth.WORKLOADS["qwen72b-80layer-n256k"]
    Hq, Hkv, N, G = w.n_q_heads, w.n_kv_heads, w.n_tokens, w.group
    dims1 = rdkv.make_dims(1, 1, Hq, Hkv, N)
    lay = rdkv.layout(dims1, w.budget_v, w.budget_k, w.zone_c_capacity)
    ol = O.Layout(**w.dims(n_layers=1), budget_v=w.budget_v, budget_k=w.budget_k, zone_c_capacity=w.zone_c_capacity)
    heads = (0, 4, 7)
    K5, V5, bt, bc, st = _score_alloc_layer(rdkv, w, 0, 40, dims1)
    _check_allocation(rdkv, w, K5, bt, bc, st, heads)
    cache = rdkv.cache_init(lay)
    rdkv.pack(lay, cache, K5, V5, bt, bc)
    oblob = _oracle_blob_skeleton(ol)
    Kh, Vh, bth, bch = host(K5)[0, 0], host(V5)[0, 0], host(bt)[0, 0], host(bc)[0, 0]
    del K5, V5, st
    for h in heads:
        O.pack_segment(ol, oblob, h, Kh[h], Vh[h], bth[h], bch[h])
        _segment_bytes_equal(cache, oblob, ol, h)
    refs = {h: _SegmentRef(oblob, ol, h) for h in heads}
    ws = rdkv.decode_workspace(lay)
    for step, append in enumerate((True, False)):
        q, kn, vn = synth.decode_inputs(w.with_(n_layers=1), step)
        c_len = 0 if append else 1
        out = host(rdkv.decode(lay, cache, c_len, torch.from_numpy(q).to(DEV),
                               torch.from_numpy(kn).to(DEV) if append else None,
                               torch.from_numpy(vn).to(DEV) if append else None, workspace=ws))
        if append:
            O.append_zone_c(oblob, ol, 0, kn, vn)
        for h in heads:
            e = rel_err(out[0, 0, h * G:(h + 1) * G], refs[h].out(q[0, 0, h * G:(h + 1) * G], 1))
            print(f"  step {step} head {h}: rel err {e:.3g}", flush=True)
            assert e <= TOL
