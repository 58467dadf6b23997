"""Pins of the oracle's zone-C rollover (decode-time scoring of the new
tokens, then allocation and packing into a generation) against things other
than itself: the prefill token weights and channel weights of the decode
queries, torch's scaled_dot_product_attention with an explicit mask, the
harmonic closed form of uniform attention, and the special cases where a
rollover must lose nothing (every new token kept at 16 bits) or everything
(a zero budget).  CPU only."""
import math

import numpy as np
import pytest
import torch

import oracle as O


def _rng(seed):
    return np.random.default_rng(seed)


def _empty_cache(N=16, G=2, Hkv=1, cap=12, n_gen=2, gbv=0, gbk=0, S=1, L=1):
    lay = O.Layout(S, L, G * Hkv, Hkv, 128, N, 0, 0, cap, n_generations=n_gen, gen_budget_v=gbv,
                   gen_budget_k=gbk)
    return lay, O.empty_blob(lay)


def _steps(lay, blob, T, seed, qscale=1.0):
    """T decode steps, each appending one token; returns (stats, q [T][S][L][Hq][d],
    k [T][...], v [T][...]) with fp16 inputs."""
    r = _rng(seed)
    stats = O.new_zone_c_stats(lay)
    qs, ks, vs = [], [], []
    for t in range(T):
        q = (r.standard_normal((lay.S, lay.L, lay.Hq, 128)) * qscale).astype(np.float16)
        k = r.standard_normal((lay.S, lay.L, lay.Hkv, 128)).astype(np.float16)
        v = r.standard_normal((lay.S, lay.L, lay.Hkv, 128)).astype(np.float16)
        O.decode_step_accumulate(blob, lay, q, t, k, v, stats)
        qs.append(q), ks.append(k), vs.append(v)
    return stats, np.stack(qs), np.stack(ks), np.stack(vs)


def test_layout_reserves_generation_blobs():
    lay = O.Layout(2, 3, 8, 2, 128, 1000, 900, 100, 64, n_generations=3, gen_budget_v=80, gen_budget_k=64)
    base = O.Layout(2, 3, 8, 2, 128, 1000, 900, 100, 64)
    gen = O.Layout(2, 3, 8, 2, 128, 64, 80, 64, 0)
    assert lay.gen_offset == base.cache_bytes
    assert lay.gen_bytes == -(-gen.cache_bytes // 256) * 256 and lay.gen_bytes % 256 == 0
    assert lay.cache_bytes == base.cache_bytes + 3 * lay.gen_bytes
    blob = O.empty_blob(lay)
    assert np.array_equal(blob[:base.cache_bytes][256:], O.empty_blob(base)[256:])   # main part unchanged
    h = blob[:256]
    assert list(h[88:96].view(np.int32)) == [3, 0]
    assert list(h[96:128].view(np.int64)) == [lay.gen_offset, lay.gen_bytes, 80, 64]
    for g in range(3):
        assert np.array_equal(O.gen_view(blob, lay, g)[:gen.cache_bytes], O.empty_blob(gen))
    with pytest.raises(ValueError):
        O.Layout(1, 1, 2, 1, 128, 10, 10, 10, 0, n_generations=1)


def test_decode_time_mass_is_the_token_weight_of_the_decode_queries():
    """With nothing kept, step t's query sees zone-C rows 0..t: the decode
    queries over zone C are a causal prefill, and the accumulated mass must be
    the prefill token weight w_t of [RDKV] 2.1 (token_weights, itself pinned
    to SDPA column sums) of those queries over those keys; the channel weight
    the same way (channel_weights)."""
    G, T = 4, 12
    lay, blob = _empty_cache(G=G, cap=T)
    stats, q, k, v = _steps(lay, blob, T, 1)
    Qg = np.transpose(q[:, 0, 0], (1, 0, 2))            # [G][T][d]
    Kc = k[:, 0, 0, 0]                                   # [T][d]
    assert np.allclose(stats[0, :, :T].sum(axis=0), O.token_weights(Qg, Kc), rtol=1e-12, atol=0)
    w_tok, var_tok, w_chan = O.rollover_weights(blob, lay, stats)
    assert np.allclose(w_tok[0], O.token_weights(Qg, Kc), rtol=1e-12, atol=0)
    assert np.allclose(w_chan[0], O.channel_weights(Qg, Kc), rtol=1e-12, atol=0)
    assert np.allclose(var_tok[0], O.token_variance(v[:, 0, 0, 0]), rtol=1e-12, atol=0)
    assert abs(w_tok[0].sum() - G * T) < 1e-9            # every step distributes one unit per head


def test_decode_time_mass_next_to_kept_tokens_matches_sdpa():
    """With kept tokens in the cache (all at 16 bits, so they are exact), each
    step's softmax runs over the kept tokens and zone-C rows 0..t.  The mass of
    the zone-C rows is checked against torch SDPA (fp64, V = identity gives
    the probabilities) with an explicit mask."""
    r = _rng(2)
    G, N, T = 2, 20, 9
    lay = O.Layout(1, 1, G, 1, 128, N, 16 * N, 16 * 128, T, n_generations=1, gen_budget_v=8, gen_budget_k=8)
    Kp = r.standard_normal((N, 128)).astype(np.float16)
    Vp = r.standard_normal((N, 128)).astype(np.float16)
    bt = np.full(N, 16, np.uint8)
    bt[::3] = 0                                          # some evicted: absent from the softmax
    blob = O.pack_cache(lay, Kp[None, None, None], Vp[None, None, None], bt[None, None, None],
                        np.full((1, 1, 1, 128), 16, np.uint8), blob=O.empty_blob(lay))
    stats, q, k, v = _steps(lay, blob, T, 3)
    kept = Kp[bt > 0].astype(np.float64)
    n_k = kept.shape[0]
    keys = np.concatenate([kept, k[:, 0, 0, 0].astype(np.float64)])          # [n_k + T][d]
    qq = torch.from_numpy(np.transpose(q[:, 0, 0], (1, 0, 2)).astype(np.float64))[None]   # [1][G][T][d]
    kk = torch.from_numpy(np.broadcast_to(keys, (G,) + keys.shape).copy())[None]
    eye = torch.eye(n_k + T, dtype=torch.float64).expand(1, G, n_k + T, n_k + T).contiguous()
    mask = torch.ones(T, n_k + T, dtype=torch.bool)
    for t in range(T):
        mask[t, n_k + t + 1:] = False                    # zone-C rows appended after step t
    P = torch.nn.functional.scaled_dot_product_attention(qq, kk, eye, attn_mask=mask)[0].numpy()
    ref = P[:, :, n_k:].sum(axis=1)                      # [G][T]: mass per head of each zone-C row
    assert np.allclose(stats[0, :, :T], ref, rtol=1e-10, atol=1e-15)
    assert np.allclose(stats[0, :, T:], (q[:, 0, 0].astype(np.float64) ** 2).sum(axis=0), rtol=1e-14)


def test_uniform_decode_attention_has_the_harmonic_mass():
    """Q = 0 and nothing kept: step tau spreads 1/(tau + 1) over rows 0..tau,
    so row j accumulates G * (H_T - H_j) (0-indexed j)."""
    G, T = 3, 10
    lay, blob = _empty_cache(G=G, cap=T)
    stats, _, _, _ = _steps(lay, blob, T, 4, qscale=0.0)
    H = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, T + 1))])
    ref = G * (H[T] - H[:T])
    assert np.allclose(stats[0, :, :T].sum(axis=0), ref, rtol=1e-13)


def _mixed_cache(n_gen, gbv, gbk, cap=10, seed=5):
    r = _rng(seed)
    S, L, G, Hkv, N = 1, 2, 2, 2, 40
    lay = O.Layout(S, L, G * Hkv, Hkv, 128, N, 60, 200, cap, n_generations=n_gen, gen_budget_v=gbv,
                   gen_budget_k=gbk)
    K = r.standard_normal((S, L, Hkv, N, 128)).astype(np.float16)
    V = r.standard_normal((S, L, Hkv, N, 128)).astype(np.float16)
    bt = r.choice(np.array([0, 2, 4, 8, 16], np.uint8), size=(S, L, Hkv, N), p=[0.5, 0.2, 0.15, 0.1, 0.05])
    bt[..., 20:] = 0
    bc = r.choice(np.array([0, 2, 4, 8, 16], np.uint8), size=(S, L, Hkv, 128), p=[0.3, 0.3, 0.2, 0.15, 0.05])
    for idx in np.ndindex(S, L, Hkv):
        while bt[idx].astype(int).sum() > 60:
            bt[idx][np.nonzero(bt[idx])[0][0]] = 0
        while bc[idx].astype(int).sum() > 200:
            bc[idx][np.nonzero(bc[idx])[0][0]] = 0
    blob = O.pack_cache(lay, K, V, bt, bc, blob=O.empty_blob(lay))
    return lay, blob


def test_full_budget_rollover_loses_nothing():
    """Generation budgets of 16 bits for every new token and channel keep the
    whole of zone C exactly (fp16 rows): decoding after the rollover (zone C
    empty) equals decoding before it (zone C full) -- the same rows, moved."""
    cap = 10
    lay, blob = _mixed_cache(2, 16 * cap, 16 * 128, cap)
    stats, _, _, _ = _steps(lay, blob, cap, 6)
    q = _rng(7).standard_normal((lay.S, lay.L, lay.Hq, 128)).astype(np.float16)
    before = O.decode_step(blob, lay, q, cap)
    w = O.rollover_weights(blob, lay, stats)
    allocs = O.rollover_pack(blob, lay, 0, *w)
    assert all(np.all(a["bits_tok"] == 16) and np.all(a["bits_chan"] == 16) for a in allocs)
    assert O.gens_in_use(blob) == 1
    after = O.decode_step(blob, lay, q, 0)
    assert np.allclose(after, before, rtol=1e-12, atol=1e-14)
    # zone C was cleared
    for seg in range(lay.n_seg):
        kc, vc = O.zone_c_rows(blob, lay, seg, cap)
        assert not kc.any() and not vc.any()


def test_zero_budget_rollover_evicts_zone_c():
    """A zero generation budget evicts every new token: after the rollover a
    step attends the prefill generation's kept tokens only."""
    cap = 8
    lay, blob = _mixed_cache(1, 0, 0, cap)
    ref_blob = blob.copy()
    stats, _, _, _ = _steps(lay, blob, cap, 8)
    O.rollover_pack(blob, lay, 0, *O.rollover_weights(blob, lay, stats))
    q = _rng(9).standard_normal((lay.S, lay.L, lay.Hq, 128)).astype(np.float16)
    assert np.allclose(O.decode_step(blob, lay, q, 0), O.decode_step(ref_blob, lay, q, 0), rtol=1e-13, atol=0)


def test_rollover_keeps_the_heaviest_new_tokens_and_fills_generations_in_order():
    """A small budget keeps the new tokens that drew the most attention (the
    cost c_t = w_t sigma_t ranks them); generations are used in order and a
    full set of generations refuses another rollover."""
    cap = 12
    lay, blob = _mixed_cache(2, 2 * 2 * 3, 64, cap)
    r = _rng(10)
    stats = O.new_zone_c_stats(lay)
    hot = 5
    for t in range(cap):
        q = r.standard_normal((lay.S, lay.L, lay.Hq, 128)).astype(np.float16)
        k = r.standard_normal((lay.S, lay.L, lay.Hkv, 128)).astype(np.float16)
        v = r.standard_normal((lay.S, lay.L, lay.Hkv, 128)).astype(np.float16)
        if t == hot:                                   # a key aligned with every later query's channel 0
            k[..., :] = 0
            k[..., 0] = 40
        q[..., 0] = np.abs(q[..., 0]) + 1
        O.decode_step_accumulate(blob, lay, q, t, k, v, stats)
    w = O.rollover_weights(blob, lay, stats)
    assert np.all(np.argmax(w[0], axis=1) == hot)
    with pytest.raises(ValueError):
        O.rollover_pack(blob.copy(), lay, 1, *w)       # out of order
    allocs = O.rollover_pack(blob, lay, 0, *w)
    for a in allocs:
        assert a["bits_tok"][hot] > 0
        assert int(a["bits_tok"].astype(int).sum()) <= lay.gen_budget_v
    # the generation's descriptors hold what was kept
    for seg, a in enumerate(allocs):
        ds = O.read_descriptor(O.gen_view(blob, lay, 0), lay.gen, seg)
        assert ds["n_kept"] == int((a["bits_tok"] > 0).sum())
    stats, _, _, _ = _steps(lay, blob, cap, 11)
    O.rollover_pack(blob, lay, 1, *O.rollover_weights(blob, lay, stats))
    assert O.gens_in_use(blob) == 2
    with pytest.raises(ValueError):
        O.rollover_pack(blob, lay, 2, *O.rollover_weights(blob, lay, stats))
