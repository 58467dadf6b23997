"""Pack and decode at the workloads' full sizes, checked on sampled segments.

Each workload's full layout (every layer, every KV head, full context) is
packed on the GPU layer by layer and decoded in the launch configuration the
benchmark uses (one launch over all segments).  The oracle cannot score a
128K or 256K context in reasonable time, so the allocation here is drawn at
random with a bit mix like the workload's (fitted to the per-segment budgets)
instead of being scored; the K/V values are the workload's own synthetic
prefill tensors.  For a few sampled segments the oracle packs the same inputs
(bytes compared exactly) and decodes them (outputs within 2e-3); segments
are independent in both the format and the kernel.
"""
import numpy as np
import pytest
import torch

import oracle as O
from decode_attention_rdkv_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 2e-3


def host(t):
    return t.detach().cpu().numpy()

# workload -> (token bit mix over 0/2/4/8/16, channel bit mix)
MIXES = {
    "llama8b-32layer-n128k": ((0.83, 0.16, 0.062, 0.008, 0.00005), (0.71, 0.28, 0.0, 0.008, 0.0)),
    "llama8b-layer-n32k": ((0.6, 0.2, 0.1, 0.05, 0.05), (0.5, 0.25, 0.15, 0.08, 0.02)),
    "llama8b-batch16-n32k": ((0.5, 0.2, 0.15, 0.1, 0.05), (0.3, 0.3, 0.2, 0.15, 0.05)),
    "qwen72b-80layer-n256k": ((0.6, 0.2, 0.1, 0.05, 0.05), (0.5, 0.25, 0.15, 0.08, 0.02)),
}


@pytest.fixture(scope="module")
def gpu_lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decode_attention_rdkv_amd import rdkv
    rdkv.load()
    return rdkv


def _fit(bits: np.ndarray, budget: int) -> np.ndarray:
    """Zero the units past the point where the running bit count exceeds the
    budget, row by row (keeps a valid allocation: sum <= budget)."""
    over = np.cumsum(bits.astype(np.int64), axis=-1) > budget
    return np.where(over, 0, bits).astype(np.uint8)


def _layer_bits(w, seq, layer):
    tok_p, chan_p = MIXES[w.name]
    bt, bc = synth.random_bits(w.n_kv_heads, w.n_tokens, 1000 * w.wid + 37 * seq + layer, tok_p=tok_p,
                               chan_p=chan_p)
    return _fit(bt, w.budget_v), _fit(bc, w.budget_k)


@pytest.mark.parametrize("name", list(MIXES))
def test_full_size_pack_and_decode_sampled(gpu_lib, name):
    rdkv = gpu_lib
    w = synth.WORKLOADS[name]
    S, L, Hq, Hkv, N, G = w.n_seq, w.n_layers, w.n_q_heads, w.n_kv_heads, w.n_tokens, w.group
    lay = rdkv.layout(rdkv.make_dims(S, L, Hq, Hkv, N), w.budget_v, w.budget_k, w.zone_c_capacity)
    ol = O.Layout(S, L, Hq, Hkv, 128, N, w.budget_v, w.budget_k, w.zone_c_capacity)
    n_seg = lay.n_seg
    sampled = sorted({0, n_seg // 2 + 1, n_seg - 1})
    print(f"{name}: {n_seg} segments, blob {lay.cache_bytes / 2**30:.2f} GiB, sampled {sampled}", flush=True)

    cache = rdkv.cache_init(lay)
    oblob = np.zeros(ol.cache_bytes, np.uint8)    # pages of unsampled segments stay untouched
    oblob[:O.HEADER_BYTES] = np.frombuffer(ol.header_bytes(), np.uint8)
    for seg in range(n_seg):                      # empty descriptors, as rdkv_cache_init writes them
        O.pack_segment(ol, oblob, seg, np.zeros((0, 128), np.float16), np.zeros((0, 128), np.float16),
                       np.zeros(0, np.uint8), np.zeros(128, np.uint8))
    for l in range(L):                            # one pack call per layer, all sequences
        Ks, Vs, bts, bcs = [], [], [], []
        for s in range(S):
            _, K, V = synth.prefill_layer(w, s, l, device=DEV, kv_only=True)
            bt, bc = _layer_bits(w, s, l)
            Ks.append(K), Vs.append(V), bts.append(bt), bcs.append(bc)
            for h in range(Hkv):
                seg = ol.seg_index(s, l, h)
                if seg in sampled:
                    O.pack_segment(ol, oblob, seg, K[h].cpu().numpy(), V[h].cpu().numpy(), bt[h], bc[h])
        rdkv.pack(lay, cache, torch.stack(Ks)[:, None], torch.stack(Vs)[:, None],
                  torch.from_numpy(np.stack(bts)[:, None]).to(DEV), torch.from_numpy(np.stack(bcs)[:, None]).to(DEV),
                  layer_begin=l)
        del Ks, Vs
    torch.cuda.synchronize()

    def seg_bytes(blob_slice, seg):
        d0 = ol.desc_offset + seg * O.DESC_BYTES
        b0 = ol.slot_base(seg)
        return blob_slice(d0, d0 + O.DESC_BYTES), blob_slice(b0, b0 + ol.slot_bytes)

    gpu_slice = lambda a, b: cache[a:b].cpu().numpy()
    ora_slice = lambda a, b: oblob[a:b]
    for seg in sampled:
        gd, gs = seg_bytes(gpu_slice, seg)
        od, os_ = seg_bytes(ora_slice, seg)
        assert np.array_equal(gd, od), f"descriptor of segment {seg}"
        assert np.array_equal(gs, os_), f"slot of segment {seg}"

    ws = rdkv.decode_workspace(lay)
    for step, append in enumerate((True, False)):
        q, kn, vn = synth.decode_inputs(w, step)
        c_len = 0 if append else 1
        out = rdkv.decode(lay, cache, c_len, torch.from_numpy(q).to(DEV),
                          torch.from_numpy(kn).to(DEV) if append else None,
                          torch.from_numpy(vn).to(DEV) if append else None, workspace=ws)
        out = out.cpu().numpy()
        if append:
            O.append_zone_c(oblob, ol, c_len, kn, vn)
        n_c = c_len + 1 if append else c_len
        for seg in sampled:
            s, rem = divmod(seg, L * Hkv)
            l, h = divmod(rem, Hkv)
            ref = O.decode_segment(oblob, ol, seg, q[s, l, h * G:(h + 1) * G], n_c)
            got = out[s, l, h * G:(h + 1) * G].astype(np.float64)
            err = float((np.abs(got - ref).max(axis=-1) / np.maximum(np.abs(ref).max(axis=-1), 1e-30)).max())
            print(f"  step {step} segment {seg}: rel err {err:.3g}", flush=True)
            assert err <= TOL, f"step {step} segment {seg}: rel err {err:.3g}"

    # Every segment (not only the sampled ones): repeated decodes of the same
    # cache and query agree bit for bit.  The chunk kernel's LDS record ring is
    # filled by asynchronous copies; a copy landing late (for instance in the
    # region a wave's partial output reuses) shows up here as a difference.
    q = torch.from_numpy(synth.decode_inputs(w, 1)[0]).to(DEV)
    outs = [rdkv.decode(lay, cache, 1, q, None, None, workspace=ws) for _ in range(3)]
    for o in outs[1:]:
        assert torch.equal(o, outs[0]), "repeated decodes differ"
    assert bool(torch.isfinite(outs[0]).all()), "non-finite decode output"


# ------------------------------------------------------------------ scoring at full context length

def test_score_uniform_attention_closed_form_at_256k(gpu_lib):
    """With Q = 0 every causal row attends uniformly, so the token weight has
    the closed form w_t = G * (H_N - H_t), H_n the n-th harmonic number
    (t 0-indexed; the weight of a token is the summed attention it receives,
    RDKV summary section 2.1).  At N = 262,144, the 72B-shaped stack's context
    (G = 8), this pins both scoring passes over their longest accumulations
    without an oracle run."""
    rdkv = gpu_lib
    G, N = 8, 262144
    dims = rdkv.make_dims(1, 1, G, 1, N)
    Q = torch.zeros((1, 1, G, N, 128), dtype=torch.float16, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(11)
    K = torch.randn((1, 1, 1, N, 128), generator=gen, device=DEV).half()
    V = torch.randn((1, 1, 1, N, 128), generator=gen, device=DEV).half()
    wt, _, _ = rdkv.score(dims, Q, K, V)
    got = wt[0, 0, 0].double().cpu().numpy()
    inv = 1.0 / np.arange(1, N + 1, dtype=np.float64)
    suffix = np.cumsum(inv[::-1])[::-1]          # sum_{tau >= t} 1 / (tau + 1) = H_N - H_t
    ref = G * suffix
    err = float(np.max(np.abs(got - ref) / ref))
    print(f"closed-form w_t at N={N}: max rel err {err:.3g}")
    assert err <= TOL
    assert abs(got.sum() - G * N) <= TOL * G * N


def test_score_weights_sum_to_query_rows_on_a_128k_layer(gpu_lib):
    """On one layer of the 128K, 8B-shaped workload (32 query heads over 8 KV
    heads, biased synthetic activations) every KV head's token weights sum to
    G * N, the number of query rows that each distribute one unit of
    attention, and all are positive."""
    rdkv = gpu_lib
    w = synth.WORKLOADS["llama8b-32layer-n128k"]
    Q, K, V = synth.prefill_layer(w, 0, 5, device=DEV)
    dims = rdkv.make_dims(1, 1, w.n_q_heads, w.n_kv_heads, w.n_tokens)
    wt, vt, wc = rdkv.score(dims, Q[None, None].contiguous(), K[None, None].contiguous(), V[None, None].contiguous())
    sums = wt[0, 0].double().sum(dim=-1).cpu().numpy()
    G = w.n_q_heads // w.n_kv_heads
    print(f"sum of w_t per KV head / (G N): {sums / (G * w.n_tokens)}")
    assert np.all(np.abs(sums - G * w.n_tokens) <= TOL * G * w.n_tokens)
    assert bool((wt > 0).all()) and bool((vt > 0).all()) and bool((wc > 0).all())


def test_score_halves_compose_to_score_on_a_128k_layer(gpu_lib):
    """On the same 128K layer, rdkv_score_lse followed by rdkv_score_from_lse
    (the launch configuration of both halves at full size) gives rdkv_score's
    weights up to the rounding of the natural-log round trip of the LSE."""
    rdkv = gpu_lib
    w = synth.WORKLOADS["llama8b-32layer-n128k"]
    Q, K, V = synth.prefill_layer(w, 0, 5, device=DEV)
    dims = rdkv.make_dims(1, 1, w.n_q_heads, w.n_kv_heads, w.n_tokens)
    Qd, Kd, Vd = Q[None, None].contiguous(), K[None, None].contiguous(), V[None, None].contiguous()
    wt = rdkv.score(dims, Qd, Kd, Vd)[0]
    lse = rdkv.score_lse(dims, Qd, Kd)
    wt2, vt2, wc2 = rdkv.score_from_lse(dims, Qd, Kd, Vd, lse)
    rel = float(((wt2.double() - wt.double()).abs() / wt.double()).max())
    print(f"max rel diff of w_t, halves vs rdkv_score: {rel:.2e}")
    assert rel <= 1e-4
    assert bool(torch.isfinite(lse).all())


# ------------------------------------------------------------------ allocation at full context length

@pytest.mark.parametrize("name,seq,layer,heads", [
    ("llama8b-layer-n32k", 0, 0, range(8)),
    ("llama8b-batch16-n32k", 5, 0, range(8)),
    ("llama8b-32layer-n128k", 0, 7, (0, 3, 7)),
    ("qwen72b-80layer-n256k", 0, 40, (0, 5)),
])
def test_full_size_allocation_bit_exact_on_scored_weights(gpu_lib, name, seq, layer, heads):
    """One layer of each workload at its full context: scored on the GPU, then
    allocated on the GPU and by the oracle from the same fp32 weights and
    variances (the allocation is a deterministic function of them).  Bits,
    lambdas and the kept-token channel variances agree bit for bit."""
    rdkv = gpu_lib
    w = synth.WORKLOADS[name]
    Hq, Hkv, N = w.n_q_heads, w.n_kv_heads, w.n_tokens
    Q, K, V = synth.prefill_layer(w, seq, layer, device=DEV)
    dims = rdkv.make_dims(1, 1, Hq, Hkv, N)
    K5 = K[None, None].contiguous()
    wt, vt, wc = rdkv.score(dims, Q[None, None].contiguous(), K5, V[None, None].contiguous())
    del Q, V
    bt, bc, vc, lam = rdkv.allocate(dims, wt, vt, wc, K5, w.budget_v, w.budget_k)
    wt, vt, wc = host(wt)[0, 0], host(vt)[0, 0], host(wc)[0, 0]
    bt, bc, vc, lam = host(bt)[0, 0], host(bc)[0, 0], host(vc)[0, 0], host(lam)[0, 0]
    for h in heads:
        ref = O.allocate_segment(wt[h], vt[h], wc[h], host(K[h]), w.budget_v, w.budget_k)
        hist = np.bincount(bt[h], minlength=17)[[0, 2, 4, 8, 16]]
        print(f"{name} layer {layer} head {h}: token bits 0/2/4/8/16 {hist.tolist()}, "
              f"channels {np.bincount(bc[h], minlength=17)[[0, 2, 4, 8, 16]].tolist()}", flush=True)
        assert np.array_equal(bt[h], ref["bits_tok"]), f"head {h}: V bits differ"
        assert lam[h, 0] == ref["lambda_v"]
        assert np.array_equal(vc[h].view(np.uint32), ref["var_chan"].view(np.uint32)), f"head {h}: var_chan"
        assert np.array_equal(bc[h], ref["bits_chan"]), f"head {h}: K bits differ"
        assert lam[h, 1] == ref["lambda_k"]


def test_full_size_shared_budget_allocation_bit_exact(gpu_lib):
    """One 128K layer of the 8B-shaped workload scored on the GPU, then
    allocated with one budget shared by its 8 KV heads (8x the per-head budget)
    on the GPU and by the oracle's pooled allocation from the same fp32
    inputs: bits, lambdas and variances agree bit for bit, and the heads'
    shares differ (the pooled budget moves bits between heads)."""
    rdkv = gpu_lib
    w = synth.WORKLOADS["llama8b-32layer-n128k"]
    Hq, Hkv, N = w.n_q_heads, w.n_kv_heads, w.n_tokens
    Q, K, V = synth.prefill_layer(w, 0, 11, device=DEV)
    dims = rdkv.make_dims(1, 1, Hq, Hkv, N)
    K5 = K[None, None].contiguous()
    wt, vt, wc = rdkv.score(dims, Q[None, None].contiguous(), K5, V[None, None].contiguous())
    del Q, V
    bv, bk = w.budget_v * Hkv, w.budget_k * Hkv
    bt, bc, vc, lam = rdkv.allocate_shared(dims, wt, vt, wc, K5, bv, bk, Hkv)
    wt, vt, wc = host(wt)[0, 0], host(vt)[0, 0], host(wc)[0, 0]
    bt, bc, vc, lam = host(bt)[0, 0], host(bc)[0, 0], host(vc)[0, 0], host(lam)[0, 0]
    ref = O.allocate_group(wt, vt, wc, host(K), bv, bk)
    per_head = bt.astype(np.int64).sum(axis=1)
    print(f"V bits per head with one layer budget of {bv}: {per_head.tolist()}", flush=True)
    assert np.array_equal(bt, ref["bits_tok"])
    assert np.array_equal(vc.view(np.uint32), ref["var_chan"].view(np.uint32))
    assert np.array_equal(bc, ref["bits_chan"])
    assert np.all(lam[:, 0] == ref["lambda_v"]) and np.all(lam[:, 1] == ref["lambda_k"])
    assert int(per_head.sum()) <= bv and per_head.max() > per_head.min()
