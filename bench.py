#!/usr/bin/env python3
"""Decode-attention benchmark of the RDKV hot path on one MI355X.

Workload (default): the Llama-3.1-8B-shaped 32-layer cache at 131,072 tokens,
batch 1, 8 KV heads x 32 query heads, head dim 128, compressed to ~2.5%
retention (0.64 bits per unit on average).  Setup, untimed: for every layer,
seeded synthetic Q/K/V are drawn on the GPU, scored (rdkv_score), allocated
(rdkv_allocate) and packed (rdkv_pack) into one blob.  Timed: exactly
--steps decode steps (rdkv_decode: append one token to zone C and attend over
every layer's kept tokens), each bracketed by HIP events on the stream the
kernel runs on, with the 256 MB last-level cache cleared between steps (by
reading a 1 GiB buffer, which leaves no dirty lines behind) so
every step streams the cache from HBM.

Prints one JSON line: the metric of the decode step (us per token), the
roofline of the decode kernel (algorithmic bytes from the packed descriptors /
measured kernel time, against 8 TB/s), an fp16 full-cache decode on the same
GPU for comparison, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
# VALU issue peak: 256 CUs x 4 SIMDs, one wave64 instruction per 4 cycles each, at 2.4 GHz
VALU_PEAK_GINSTR = 256 * 4 / 4 * 2.4
MFMA_FP16_PEAK_TFS = 2500.0


ROOT = os.path.dirname(os.path.abspath(__file__))


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def counter_traffic(kernel, workload):
    """HBM bytes and VALU instructions per launch of `kernel` from the
    committed rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, each scaled
    by a plain copy of known size; SQ_INSTS_VALU), as (traffic, valu, source);
    None for each when there is no summary or the kernel's source has changed
    since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None, None, None
    text = open(path).read()
    fields = dict(re.findall(r"^(kernel_source|kernel_source_sha256|traffic_bytes_per_launch|"
                             r"valu_instructions_per_launch): (\S+)$", text, re.M))
    if not {"kernel_source", "kernel_source_sha256", "traffic_bytes_per_launch"} <= set(fields):
        return None, None, None
    src = os.path.join(ROOT, fields["kernel_source"])
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != fields["kernel_source_sha256"]:
        return None, None, os.path.relpath(path, ROOT) + " (stale: kernel source changed)"
    valu = int(fields["valu_instructions_per_launch"]) if "valu_instructions_per_launch" in fields else None
    return int(fields["traffic_bytes_per_launch"]), valu, os.path.relpath(path, ROOT)


def gpu_busy(torch, ms=3.0):
    """Keeps the GPU busy for a few milliseconds, so that launches issued
    next are queued before it reaches them."""
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(int(ms * 2e6))   # cycles, at about 2 GHz
    else:
        a = torch.ones((4096, 4096), dtype=torch.float16, device="cuda")
        for _ in range(int(ms * 10)):
            a = a @ a * 0.0001


def build_cache(rdkv, synth, torch, w, lay, dims1, fp16_only=False, lay1=None, keep=False):
    """Score, allocate and pack every layer into a fresh cache; returns stats.
    With `lay1` (a one-layer layout), each layer is also packed into a blob of
    its own (stats["layer_caches"]), for the per-layer decode loop.  With
    `keep`, stats["kept"] holds every layer's K, V and allocation
    ([S][L][Hkv]...) and the allocation with one budget per layer shared by
    its KV heads, for the paged and rollover measurements."""
    cache = rdkv.cache_init(lay)
    layer_caches = []
    kept = None
    if keep:
        shp = (w.n_seq, w.n_layers, w.n_kv_heads)
        kept = dict(K=torch.empty(shp + (w.n_tokens, 128), dtype=torch.float16, device="cuda"),
                    V=torch.empty(shp + (w.n_tokens, 128), dtype=torch.float16, device="cuda"),
                    bt=torch.empty(shp + (w.n_tokens,), dtype=torch.uint8, device="cuda"),
                    bc=torch.empty(shp + (128,), dtype=torch.uint8, device="cuda"),
                    bt_shared=torch.empty(shp + (w.n_tokens,), dtype=torch.uint8, device="cuda"),
                    bc_shared=torch.empty(shp + (128,), dtype=torch.uint8, device="cuda"))
    S = w.n_seq
    ws = None
    hist_tok = np.zeros(5, np.int64)
    hist_chan = np.zeros(5, np.int64)
    score_ms = 0.0
    halves = None   # layer 0: the two halves of scoring on their own (prefill-LSE reuse)
    t0 = time.time()
    for l in range(w.n_layers):
        parts = [synth.prefill_layer(w, s, l, device="cuda") for s in range(S)]
        K = torch.stack([p[1] for p in parts])[:, None].contiguous()
        V = torch.stack([p[2] for p in parts])[:, None].contiguous()
        if fp16_only:
            del parts
            bt = torch.full((S, 1, w.n_kv_heads, w.n_tokens), 16, dtype=torch.uint8, device="cuda")
            bc = torch.full((S, 1, w.n_kv_heads, 128), 16, dtype=torch.uint8, device="cuda")
        else:
            Q = torch.stack([p[0] for p in parts])[:, None].contiguous()
            del parts
            if ws is None:
                ws = torch.empty(rdkv.score_workspace_bytes(dims1), dtype=torch.uint8, device="cuda")
            if l == 0:
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                ev[0].record()
                lse = rdkv.score_lse(dims1, Q, K)
                ev[1].record()
                rdkv.score_from_lse(dims1, Q, K, V, lse, workspace=ws)
                ev[2].record()
                ev[2].synchronize()
                halves = (ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2]))
                del lse
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            wt, vt, wc = rdkv.score(dims1, Q, K, V, workspace=ws)
            e1.record()
            del Q
            e2 = torch.cuda.Event(enable_timing=True)
            bt, bc, _, _ = rdkv.allocate(dims1, wt, vt, wc, K, w.budget_v, w.budget_k)
            e2.record()
            e2.synchronize()
            score_ms += e0.elapsed_time(e1)
            if l == 0 or keep:
                # the same layer with one budget shared by its KV heads
                e3, e4 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e3.record()
                bts, bcs, _, _ = rdkv.allocate_shared(dims1, wt, vt, wc, K, w.budget_v * w.n_kv_heads,
                                                      w.budget_k * w.n_kv_heads, w.n_kv_heads)
                e4.record()
                e4.synchronize()
                if l == 0:
                    halves = halves + (e0.elapsed_time(e1), e1.elapsed_time(e2), e3.elapsed_time(e4))
                    # the same two calls queued behind other GPU work, so that the
                    # events time their kernels rather than the host's launches
                    for g in (1, w.n_kv_heads):
                        gpu_busy(torch)
                        e5, e6 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        e5.record()
                        rdkv.allocate_shared(dims1, wt, vt, wc, K, w.budget_v * g, w.budget_k * g, g)
                        e6.record()
                        e6.synchronize()
                        halves = halves + (e5.elapsed_time(e6),)
                if keep:
                    kept["bt_shared"][:, l] = bts[:, 0]
                    kept["bc_shared"][:, l] = bcs[:, 0]
                del bts, bcs
            del wt, vt, wc
        rdkv.pack(lay, cache, K, V, bt, bc, layer_begin=l)
        if lay1 is not None:
            layer_caches.append(rdkv.cache_init(lay1))
            rdkv.pack(lay1, layer_caches[-1], K, V, bt, bc, layer_begin=0)
        for i, b in enumerate((0, 2, 4, 8, 16)):
            hist_tok[i] += int((bt == b).sum())
            hist_chan[i] += int((bc == b).sum())
        if keep:
            kept["K"][:, l] = K[:, 0]
            kept["V"][:, l] = V[:, 0]
            kept["bt"][:, l] = bt[:, 0]
            kept["bc"][:, l] = bc[:, 0]
        del K, V, bt, bc
        if l % 8 == 7 or l == w.n_layers - 1:
            torch.cuda.synchronize()
            log(f"{'fp16 ' if fp16_only else ''}layer {l + 1}/{w.n_layers} packed, {time.time() - t0:.1f}s")
    torch.cuda.synchronize()
    return cache, dict(hist_tok=hist_tok, hist_chan=hist_chan, score_ms=score_ms, setup_s=time.time() - t0,
                       layer_caches=layer_caches, score_halves=halves, kept=kept)


def time_decode(rdkv, torch, lay, cache, q, kn, vn, steps, warmup, flush, grow=False):
    """Per-step event times (ms) of the two decode phases over `steps` steps.

    Each step is rdkv_decode_partials (the chunk kernel: append + split-K
    partials) then rdkv_decode_merge, i.e. exactly rdkv_decode, with an event
    before, between and after on the stream both kernels run on.  By default
    every step appends at zone-C row 0 and attends over one zone-C row; with
    `grow`, step i appends at row i (mod capacity) and attends over i + 1 rows,
    as a generation loop does.
    """
    ws = rdkv.decode_workspace(lay)
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    # The caches are cleared between steps by READING a 1 GiB buffer: it
    # evicts the blob from the L2s and the 256 MB last-level cache without
    # leaving dirty lines whose write-back would land inside the next step
    # (a 1 GiB fill costs the following decode step ~20-50 us of such
    # write-back traffic that is not the decode's own).
    fbuf = torch.ones(1 << 27, dtype=torch.int64, device="cuda") if flush else None

    def clear_caches():
        if fbuf is not None:
            fbuf.sum()

    cap = max(lay.zone_c_capacity, 1)
    row = (lambda i: i % cap) if grow else (lambda i: 0)

    def step(i):
        rdkv.decode_partials(lay, cache, row(i), q, kn, vn, workspace=ws)

    def merge(i):
        rdkv.decode_merge(lay, cache, row(i) + 1, ws, out)

    # events exist before the warmup, so the timed loop follows the
    # synchronization with no host work in between (the part clocks down
    # within a millisecond of idling)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(warmup):
        step(i)
        merge(i)
        clear_caches()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record()
        step(i)
        ev[i][1].record()
        merge(i)
        ev[i][2].record()
        clear_caches()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    chunk = np.array([a.elapsed_time(b) for a, b, _ in ev])
    merge_ms = np.array([b.elapsed_time(c) for _, b, c in ev])
    total = np.array([a.elapsed_time(c) for a, _, c in ev])
    del fbuf
    mean_rows = float(np.mean([row(i) + 1 for i in range(steps)]))
    return dict(step=float(total.mean()), step_median=float(np.median(total)), chunk=float(chunk.mean()),
                chunk_median=float(np.median(chunk)), merge=float(merge_ms.mean()), wall=wall, out=out,
                mean_zone_c_rows=mean_rows, total_ms=float(total.sum()))


def settle_decode(rdkv, torch, lay, cache, q, kn, vn, seconds, flush, grow=False):
    """Untimed decode steps (the timed loop's steps, cache clearing included)
    for about `seconds` of wall time; returns how many ran."""
    if seconds <= 0:
        return 0
    ws = rdkv.decode_workspace(lay)
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    fbuf = torch.ones(1 << 27, dtype=torch.int64, device="cuda") if flush else None
    cap = max(lay.zone_c_capacity, 1)
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            row = n % cap if grow else 0
            rdkv.decode(lay, cache, row, q, kn, vn, workspace=ws, out=out)
            if fbuf is not None:
                fbuf.sum()
            n += 1
        torch.cuda.synchronize()
    del fbuf
    return n


def time_layer_graph(rdkv, torch, lay1, caches, q, kn, vn, steps, warmup, flush, ref):
    """The same decode step issued the way a model's layer loop issues it: one
    rdkv_decode (chunk + merge kernel) per layer on that layer's own blob, the
    whole loop captured once in a HIP graph and replayed per step.  Returns
    the mean/median replay time (ms) and the largest relative difference of
    any replay's output from `ref` (the single-launch output)."""
    L = len(caches)
    ws = rdkv.decode_workspace(lay1)
    ql = [q[:, l:l + 1].contiguous() for l in range(L)]
    kl = [kn[:, l:l + 1].contiguous() for l in range(L)]
    vl = [vn[:, l:l + 1].contiguous() for l in range(L)]
    outs = [torch.empty(x.shape, dtype=torch.float32, device="cuda") for x in ql]

    def loop():
        for l in range(L):
            rdkv.decode(lay1, caches[l], 0, ql[l], kl[l], vl[l], workspace=ws, out=outs[l])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        loop()                      # eager pass on the capture stream before capturing
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = torch.cat(outs, dim=1).clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        loop()
    fbuf = torch.ones(1 << 27, dtype=torch.int64, device="cuda") if flush else None
    worst = 0.0
    for i in range(warmup):
        g.replay()
        if fbuf is not None:
            fbuf.sum()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        g.replay()
        ev[i][1].record()
        if fbuf is not None:
            fbuf.sum()
        # every replay must reproduce the eager per-layer loop exactly
        if i < 3:
            torch.cuda.synchronize()
            got = torch.cat(outs, dim=1)
            if not torch.equal(got, eager):
                raise RuntimeError(f"graph replay {i} differs from the eager per-layer loop")
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    got = torch.cat(outs, dim=1)
    rel = ((got - ref).abs().amax(-1) / ref.abs().amax(-1).clamp_min(1e-30)).max().item()
    del g, fbuf
    return dict(step=float(t.mean()), step_median=float(np.median(t)), rel_diff=rel)


def inputs_digest(torch, q, kn, vn, cache, lay):
    """SHA-256 of the decode inputs and of the packed blob's header and
    descriptors (what a rerun on the same seeds must reproduce)."""
    import hashlib
    out = {}
    for name, t in (("q", q), ("k_new", kn), ("v_new", vn)):
        out[name] = hashlib.sha256(t.contiguous().cpu().numpy().tobytes()).hexdigest()[:16]
    out["blob_descriptors"] = hashlib.sha256(cache[:lay.slots_offset].cpu().numpy().tobytes()).hexdigest()[:16]
    return out


def time_calls(torch, call, steps, warmup, flush):
    """Event time (ms) of call(i), i = 0..steps-1, after call(0..warmup-1),
    with the caches cleared between calls (see time_decode): mean, median."""
    fbuf = torch.ones(1 << 27, dtype=torch.int64, device="cuda") if flush else None
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(warmup):
        call(i)
        if fbuf is not None:
            fbuf.sum()
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record()
        call(i)
        ev[i][1].record()
        if fbuf is not None:
            fbuf.sum()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    del fbuf
    return float(t.mean()), float(np.median(t))


def chunk_stats(chunk_tok2, token_slots, desc):
    """Decode chunks per segment (the token groups' chunks of chunk_tok2 >> g
    tokens) against the chunk slots the layout reserves."""
    n = np.zeros(len(desc["n_tok"]), np.int64)
    for g in range(4):
        t = chunk_tok2 >> g
        n += (desc["n_tok"][:, g] + t - 1) // t
    return {"chunk_tok2": int(chunk_tok2), "slots_per_segment": int(token_slots), "total": int(n.sum()),
            "per_segment_max": int(n.max()), "per_segment_mean": round(float(n.mean()), 2)}


def record_stats(rec_max, desc):
    """K-record words per segment (zone-A records): the layout's bound against
    what the segments hold; decode takes records of up to 20 words through its
    three-workgroups-per-CU ring and a longer bound's ring in a second launch."""
    words = desc["rec"][desc["n_kept"] > 0] // 4
    if words.size == 0:
        return {"bound": int(rec_max // 4)}
    return {"bound": int(rec_max // 4), "max": int(words.max()), "median": float(np.median(words)),
            "segments_over_20": int((words > 20).sum()), "segments": int(words.size)}


def build_paged(rdkv, torch, w, K, V, bt, bc, budget_v, budget_k, seed=0):
    """Every sequence of K, V, bt, bc ([S][L][Hkv]...) staged, given pages
    from a host free list in shuffled order (no segment's pages contiguous)
    and committed into a paged cache whose pool holds exactly the pages
    needed.  Returns (paged layout, cache, pages in use)."""
    S, L, Hkv, N = K.shape[0], K.shape[1], K.shape[2], K.shape[3]
    dims = rdkv.make_dims(S, L, w.n_q_heads, Hkv, N)
    staged, total = [], 0
    pl0 = rdkv.paged_layout(dims, budget_v, budget_k, w.zone_c_capacity, 1)
    for s in range(S):
        stg, need = rdkv.paged_stage(pl0, N, budget_v, budget_k, K[s], V[s], bt[s], bc[s])
        need = need.cpu().numpy()
        staged.append((stg, need))
        total += int(need.sum())
    pl = rdkv.paged_layout(dims, budget_v, budget_k, w.zone_c_capacity, total)
    cache = rdkv.paged_cache_init(pl)
    free = np.random.default_rng(seed).permutation(total).astype(np.int32)
    at = 0
    for s, (stg, need) in enumerate(staged):
        table = np.full((L * Hkv, pl.max_pages), -1, np.int32)
        for i, k in enumerate(need):
            table[i, :k] = free[at:at + k]
            at += int(k)
        rdkv.paged_commit(pl, cache, s, N, budget_v, budget_k, stg, torch.from_numpy(table).cuda())
    torch.cuda.synchronize()
    del staged
    flags = cache[256:256 + 256 * pl.n_seg].view(-1, 256)[:, 44:48].cpu().numpy().view(np.int32)
    if flags.any():
        raise RuntimeError(f"{int((flags != 0).sum())} segments did not fit their pages")
    return pl, cache, total


def extras(rdkv, torch, w, lay, cache, kept, q, kn, vn, ref_out, steps, warmup, flush, grow, n_c):
    """Paged zones (per-segment budgets, and one budget per layer shared by
    its KV heads) and zone-C rollover on the same data as the headline
    decode."""
    res = {}
    S, cap = w.n_seq, w.zone_c_capacity
    row = (lambda i: i % cap) if grow else (lambda i: 0)
    K, V = kept["K"], kept["V"]
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")

    def algo_bytes(cache):
        # the paged descriptors carry the counts at the contiguous offsets
        b = rdkv.decode_bytes(lay, rdkv.descriptors(lay, cache), n_c)
        return b["total"] + lay.n_seg * (256 + 2 * 128 * 2)

    # per-segment budgets on pages: the same allocation as the contiguous blob
    pl, pc, used = build_paged(rdkv, torch, w, K, V, kept["bt"], kept["bc"], w.budget_v, w.budget_k, seed=1)
    ws = rdkv.paged_decode_workspace(pl)
    wsc = rdkv.decode_workspace(lay)
    outc = torch.empty_like(out)
    tc, _ = time_calls(torch, lambda i: rdkv.decode(lay, cache, row(i), q, kn, vn, workspace=wsc, out=outc),
                       steps, warmup, flush)
    t, tm = time_calls(torch, lambda i: rdkv.paged_decode(pl, pc, [row(i)] * S, q, kn, vn, workspace=ws, out=out),
                       steps, warmup, flush)
    del wsc, outc
    res["paged"] = {
        "us_per_step": round(t * 1e3, 2), "us_per_step_median": round(tm * 1e3, 2),
        "contiguous_us_per_step_just_before": round(tc * 1e3, 2),
        "bit_identical_to_contiguous": bool(torch.equal(out, ref_out)),
        "achieved_GBs": round(algo_bytes(pc) / (t * 1e-3) / 1e9, 1),
        "chunks": chunk_stats(pl.chunk_tok2, pl.token_slots, rdkv.descriptors(lay, pc)),
        "pages_in_use": used, "page_bytes": rdkv.PAGE_BYTES, "resident_bytes": int(pl.pool_offset + used * rdkv.PAGE_BYTES),
        "contiguous_blob_bytes": int(lay.cache_bytes),
        "note": "the same packed segments on 32 KiB pages of a shared pool, given out shuffled; one rdkv_paged_decode "
                "(chunk + merge kernels) per step; resident bytes = header, descriptors, block table and the pages in use"}
    log(f"paged: {t * 1e3:.1f} us per step, {used} pages, bit-identical {res['paged']['bit_identical_to_contiguous']}")
    del pc, ws
    torch.cuda.empty_cache()

    # one budget per layer, shared by its KV heads, on pages
    Hkv = w.n_kv_heads
    bvs, bks = w.budget_v * Hkv, w.budget_k * Hkv
    pl, pc, used = build_paged(rdkv, torch, w, K, V, kept["bt_shared"], kept["bc_shared"], bvs, bks, seed=2)
    ws = rdkv.paged_decode_workspace(pl)
    shape = rdkv.paged_decode_shape(pl, pc, ws)
    pc_shaped = pc.clone()
    out_shaped = torch.empty_like(out)
    t_sh, tm_sh = time_calls(torch, lambda i: rdkv.paged_decode(pl, pc_shaped, [row(i)] * S, q, kn, vn, workspace=ws,
                                                                out=out_shaped, shape=shape), steps, warmup, flush)
    t, tm = time_calls(torch, lambda i: rdkv.paged_decode(pl, pc, [row(i)] * S, q, kn, vn, workspace=ws, out=out),
                       steps, warmup, flush)
    shaped_diff = float(((out_shaped.double() - out.double()).abs().amax(-1) /
                         out.double().abs().amax(-1).clamp_min(1e-30)).max())
    shaped_cache_same = bool(torch.equal(pc, pc_shaped))
    del pc_shaped, out_shaped
    lay_shared = rdkv.layout(rdkv.make_dims(S, w.n_layers, w.n_q_heads, Hkv, w.n_tokens), bvs, bks, cap)
    res["shared_budget_paged"] = {
        "us_per_step": round(t * 1e3, 2), "us_per_step_median": round(tm * 1e3, 2),
        "budget_v_per_layer": bvs, "budget_k_per_layer": bks,
        "algorithmic_bytes_per_step": int(algo_bytes(pc)), "achieved_GBs": round(algo_bytes(pc) / (t * 1e-3) / 1e9, 1),
        "pages_in_use": used, "resident_bytes": int(pl.pool_offset + used * rdkv.PAGE_BYTES),
        "contiguous_blob_bytes_same_budgets": int(lay_shared.cache_bytes),
        "contiguous_blob_bytes_per_segment_budgets": int(lay.cache_bytes),
        "resident_vs_per_segment_blob": round((pl.pool_offset + used * rdkv.PAGE_BYTES) / lay.cache_bytes, 4),
        "chunks": chunk_stats(pl.chunk_tok2, pl.token_slots, rdkv.descriptors(lay, pc)),
        "record_words": record_stats(pl.rec_max, rdkv.descriptors(lay, pc)),
        "shaped": {"us_per_step": round(t_sh * 1e3, 2), "us_per_step_median": round(tm_sh * 1e3, 2),
                   "achieved_GBs": round(algo_bytes(pc) / (t_sh * 1e-3) / 1e9, 1),
                   "token_slots": int(shape.token_slots), "record_words": int(shape.rec_max) // 4,
                   "max_rel_diff_vs_unshaped": shaped_diff, "cache_identical_to_unshaped": shaped_cache_same,
                   "note": "rdkv_paged_decode_shaped with the shape rdkv_paged_decode_shape measured on the "
                           "sequences in use: chunk slots and record ring from the segments, not the bounds"},
        "note": "rdkv_allocate_shared with one budget per layer (its KV heads' budgets pooled), packed on pages: "
                "memory follows what each segment keeps instead of a slot sized for the whole layer's budget"}
    log(f"shared budget on pages: {t * 1e3:.1f} us per step ({t_sh * 1e3:.1f} with the measured shape), "
        f"{used} pages")
    del pc, ws
    torch.cuda.empty_cache()

    # zone-C rollover, n_gen times: cap steps with the decode-time statistics,
    # then a rollover; then decode over the prefill blob and the generations
    n_gen = 4
    gbv, gbk = max(1, w.budget_v * cap // w.n_tokens), w.budget_k
    dims = rdkv.make_dims(S, w.n_layers, w.n_q_heads, Hkv, w.n_tokens)
    lr = rdkv.layout_rollover(dims, w.budget_v, w.budget_k, cap, n_gen, gbv, gbk)
    cr = rdkv.cache_init(lr)
    rdkv.pack(lr, cr, K, V, kept["bt"], kept["bc"])
    ws = rdkv.decode_workspace(lr)
    stats = rdkv.zone_c_stats(lr)
    rws = torch.empty(max(int(lr.rollover_workspace_bytes), 16), dtype=torch.uint8, device="cuda")
    t_plain, _ = time_calls(torch, lambda i: rdkv.decode(lr, cr, i, q, kn, vn, workspace=ws, out=out), cap, 0, flush)
    t_acc, t_roll = [], []
    for g in range(n_gen):
        t_acc.append(time_calls(torch, lambda i: rdkv.decode_accumulate(lr, cr, i, q, kn, vn, stats, workspace=ws,
                                                                        out=out), cap, 0, flush)[0])
        t_roll.append(time_calls(torch, lambda i: rdkv.rollover(lr, cr, g, stats, workspace=rws), 1, 0, flush)[0])
    t_gen, t_gen_med = time_calls(torch, lambda i: rdkv.decode(lr, cr, row(i), q, kn, vn, workspace=ws, out=out),
                                  steps, warmup, flush)
    res["rollover"] = {
        "zone_c_capacity": cap, "generations": n_gen, "gen_budget_v": gbv, "gen_budget_k": gbk,
        "decode_us_per_step": round(t_plain * 1e3, 2),
        "decode_accumulate_us_per_step": round(float(np.mean(t_acc)) * 1e3, 2),
        "rollover_us": [round(x * 1e3, 1) for x in t_roll],
        "decode_us_per_step_all_generations": round(t_gen * 1e3, 2),
        "generation_blob_bytes": int(lr.gen_bytes),
        "note": "decode and decode_accumulate averaged over zone-C lengths 1..cap (accumulate over every generation's "
                "fill); rollover = score, allocate and pack the full zone C of every segment into the next generation "
                "blob and clear it, once per generation; then decode over the prefill blob and every generation"}
    log(f"rollover: decode {t_plain * 1e3:.1f} us, accumulate {np.mean(t_acc) * 1e3:.1f} us, rollover "
        f"{[round(x * 1e3, 1) for x in t_roll]} us, decode with {n_gen} generations {t_gen * 1e3:.1f} us")
    del cr, ws, stats, rws
    torch.cuda.empty_cache()
    return res


def cpu_scoring_baseline(w, n_sample: int = 8192):
    """The oracle's stage-1 token weights of one (layer, KV head), timed on the
    first n_sample prefill rows and keys of a seeded layer (its G query heads)
    and scaled by (N / n_sample)^2, the causal score count; single-threaded."""
    import oracle as O
    from decode_attention_rdkv_amd import synth
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        threadpool_limits = None
    n = min(n_sample, w.n_tokens)
    Q, K, _ = synth.prefill_layer(w.with_(n_tokens=n), 0, 0)
    G = w.group
    ctx = threadpool_limits(1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        t0 = time.perf_counter()
        O.token_weights(Q[:G], K[0])
        dt = time.perf_counter() - t0
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    scale = (w.n_tokens / n) ** 2
    return dict(value=round(dt * scale, 2), unit="s per (layer, KV head)", cores=1, kind="oracle",
                sample=f"token weights of one KV head ({G} query heads) over the first {n} of {w.n_tokens} "
                       f"prefill positions, {dt:.2f} s, scaled by (N/{n})^2")


def cpu_baseline_all_stages(name: str = "tiny-gqa4-n1k"):
    """Every stage of the oracle, single-threaded, on the tiny one-layer
    workload: token and channel weights and variances, the allocation, the
    packed blob, then the workload's decode steps with appends."""
    import oracle as O
    from decode_attention_rdkv_amd import synth
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        threadpool_limits = None
    w = synth.WORKLOADS[name]
    Q, K, V = synth.prefill_layer(w, 0, 0)
    G, N = w.group, w.n_tokens
    lay = O.Layout(1, 1, w.n_q_heads, w.n_kv_heads, 128, N, w.budget_v, w.budget_k, w.zone_c_capacity)
    t = {}
    ctx = threadpool_limits(1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        t0 = time.perf_counter()
        bts, bcs = [], []
        for h in range(w.n_kv_heads):
            w_tok = O.token_weights(Q[h * G:(h + 1) * G], K[h]).astype(np.float32)
            w_chan = O.channel_weights(Q[h * G:(h + 1) * G], K[h]).astype(np.float32)
            var_tok = O.token_variance(V[h]).astype(np.float32)
            t1 = time.perf_counter()
            a = O.allocate_segment(w_tok, var_tok, w_chan, K[h], w.budget_v, w.budget_k)
            t2 = time.perf_counter()
            t["score"] = t.get("score", 0.0) + t1 - t0
            t["allocate"] = t.get("allocate", 0.0) + t2 - t1
            bts.append(a["bits_tok"])
            bcs.append(a["bits_chan"])
            t0 = time.perf_counter()
        blob = O.pack_cache(lay, K[None, None], V[None, None], np.stack(bts)[None, None], np.stack(bcs)[None, None])
        t["pack"] = time.perf_counter() - t0
        t0 = time.perf_counter()
        for step in range(w.decode_steps):
            q, kn, vn = synth.decode_inputs(w, step)
            O.decode_step(blob, lay, q, step, kn, vn)
        t["decode"] = time.perf_counter() - t0
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    total = sum(t.values())
    return dict(value=round(total, 3), unit="s", cores=1, kind="oracle",
                stages_s={k: round(v, 3) for k, v in t.items()},
                sample=f"the whole {name} workload ({w.n_kv_heads} KV head, {w.n_q_heads} query heads, {N} tokens, "
                       f"{w.decode_steps} decode steps): scoring, allocation, packing and decode, single-threaded")


def cpu_baseline_c2_all_stages(decode_steps_sample: int = 4):
    """Every stage of the oracle on the single 32K layer (8 KV heads, 32 query
    heads, 32,768 tokens, 64 decode steps), single-threaded, within a bounded
    time: the token weights of one KV head timed on the first 8,192 rows and
    scaled by the causal score count and the 8 heads; channel weights and
    token variances in full; the allocation of every head in full, on seeded
    weights of the workload's shape (the scored weights would take the full
    scoring first); the packed blob in full; decode_steps_sample decode steps
    with appends, scaled to the workload's 64."""
    import oracle as O
    from decode_attention_rdkv_amd import synth
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        threadpool_limits = None
    w = synth.WORKLOADS["llama8b-layer-n32k"]
    G, N, H = w.group, w.n_tokens, w.n_kv_heads
    t = {}
    score_one = cpu_scoring_baseline(w)["value"]
    Q, K, V = synth.prefill_layer(w, 0, 0)
    w_tok, var_tok, w_chan = synth.random_unit_inputs(H, N, seed=2)
    lay = O.Layout(1, 1, w.n_q_heads, H, 128, N, w.budget_v, w.budget_k, w.zone_c_capacity)
    ctx = threadpool_limits(1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        t0 = time.perf_counter()
        for h in range(H):
            O.channel_weights(Q[h * G:(h + 1) * G], K[h])
            O.token_variance(V[h])
        t["score"] = score_one * H + time.perf_counter() - t0
        t0 = time.perf_counter()
        bts, bcs = [], []
        for h in range(H):
            a = O.allocate_segment(w_tok[h], var_tok[h], w_chan[h], K[h], w.budget_v, w.budget_k)
            bts.append(a["bits_tok"])
            bcs.append(a["bits_chan"])
        t["allocate"] = time.perf_counter() - t0
        t0 = time.perf_counter()
        blob = O.pack_cache(lay, K[None, None], V[None, None], np.stack(bts)[None, None], np.stack(bcs)[None, None])
        t["pack"] = time.perf_counter() - t0
        t0 = time.perf_counter()
        for step in range(decode_steps_sample):
            q, kn, vn = synth.decode_inputs(w, step)
            O.decode_step(blob, lay, q, step, kn, vn)
        t["decode"] = (time.perf_counter() - t0) * w.decode_steps / decode_steps_sample
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    return dict(value=round(sum(t.values()), 1), unit="s", cores=1, kind="oracle",
                stages_s={k: round(v, 2) for k, v in t.items()},
                sample=f"llama8b-layer-n32k ({H} KV heads, {w.n_q_heads} query heads, {N} tokens, {w.decode_steps} "
                       f"decode steps): token weights of one KV head on the first 8,192 rows scaled by (N/8192)^2 "
                       f"and {H} heads; allocation (on seeded weights of the same shape) and packing in full; "
                       f"{decode_steps_sample} decode steps scaled to {w.decode_steps}; single-threaded")


def host_info():
    """What the host offers the oracle: cores, the cores this process may use,
    and numpy's BLAS threads (the timed oracle runs are limited to one)."""
    info = {"cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0))}
    try:
        from threadpoolctl import threadpool_info
        info["blas_threads"] = [p.get("num_threads") for p in threadpool_info() if p.get("user_api") == "blas"]
    except ImportError:
        info["blas_threads"] = None
    return info


def cpu_baseline(w, hist_tok, hist_chan, n_seg, n_c, sample_segments):
    """The oracle's decode of one step, timed on `sample_segments` segments of
    the same shape (kept-token mix and K-channel mix of the measured
    allocation; seeded K/V), scaled to the whole step."""
    import oracle as O
    from decode_attention_rdkv_amd import synth
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        threadpool_limits = None
    N = w.n_tokens
    p_tok = hist_tok / hist_tok.sum()
    p_chan = hist_chan / hist_chan.sum()
    lay = O.Layout(1, 1, w.group, 1, 128, N, w.budget_v, w.budget_k, w.zone_c_capacity)
    total = 0.0
    ctx = threadpool_limits(1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        for s in range(sample_segments):
            bt, bc = synth.random_bits(1, N, 1000 + s, tok_p=p_tok, chan_p=p_chan)
            # keep the allocation inside the budget the layout was sized for
            while int(bt.astype(np.int64).sum()) > w.budget_v:
                nz = np.nonzero(bt[0])[0]
                bt[0, nz[: len(nz) // 100 + 1]] = 0
            while int(bc.astype(np.int64).sum()) > w.budget_k:
                bc[0, np.nonzero(bc[0])[0][0]] = 0
            K, V = synth.random_kv(1, N, 2000 + s)
            blob = O.pack_cache(lay, K[None, None], V[None, None], bt[None, None], bc[None, None])
            r = np.random.default_rng(s)
            q = r.standard_normal((1, 1, w.group, 128)).astype(np.float16)
            kn = r.standard_normal((1, 1, 1, 128)).astype(np.float16)
            vn = r.standard_normal((1, 1, 1, 128)).astype(np.float16)
            t0 = time.perf_counter()
            O.decode_step(blob, lay, q, n_c - 1, kn, vn)
            total += time.perf_counter() - t0
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    per_step_s = total / sample_segments * n_seg
    if w.n_seq > 1:      # batched workload: throughput over the batch, like the GPU figure
        value, unit = w.n_seq / per_step_s, "tokens/s"
    else:
        value, unit = per_step_s * 1e6 / w.n_seq, "us/token"
    return dict(value=value, unit=unit, cores=1, kind="oracle", host=host_info(),
                sample=f"{sample_segments} sampled segments (one KV head of one layer each, {N} tokens, "
                       f"measured bit mix, seeded K/V), oracle decode step timed single-threaded; the mean per "
                       f"segment times the step's {n_seg} segments; host has {os.cpu_count()} cpus")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama8b-32layer-n128k")
    ap.add_argument("--no-flush", action="store_true", help="do not flush the last-level cache between steps")
    ap.add_argument("--grow", action="store_true",
                    help="append each step's token at the next zone-C row and attend over all rows so far "
                         "(always on for batched workloads, whose metric is decode throughput)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp16-baseline", action="store_true")
    ap.add_argument("--cpu-sample-segments", type=int, default=32)
    ap.add_argument("--no-layer-loop", action="store_true",
                    help="skip the per-layer decode loop (one launch pair per layer, captured in a HIP graph)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the paged-zone, shared-budget and rollover measurements (on by default when the "
                         "workload's fp16 K/V fits in 40 GB)")
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="untimed decode steps for this many seconds right before the headline's warmup "
                         "(the part's clocks settle under sustained decode work)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, run one plain 384 MiB device-to-device copy (for counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the RDKV hot path has no "
                                   "cross-GPU exchange (segments are independent); run with --gpus 1"}))
        sys.exit(2)

    import torch
    from decode_attention_rdkv_amd import rdkv, synth
    rdkv.load()
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    w = synth.WORKLOADS[args.workload]
    log(f"workload {w.name}: S={w.n_seq} L={w.n_layers} Hq={w.n_q_heads} Hkv={w.n_kv_heads} N={w.n_tokens} "
        f"avg bits {w.avg_bits} (B_V={w.budget_v}, B_K={w.budget_k})")
    dims = rdkv.make_dims(w.n_seq, w.n_layers, w.n_q_heads, w.n_kv_heads, w.n_tokens)
    dims1 = rdkv.make_dims(w.n_seq, 1, w.n_q_heads, w.n_kv_heads, w.n_tokens)
    lay = rdkv.layout(dims, w.budget_v, w.budget_k, w.zone_c_capacity)
    per_layer = w.n_layers > 1 and not args.no_layer_loop
    lay1 = rdkv.layout(dims1, w.budget_v, w.budget_k, w.zone_c_capacity) if per_layer else None
    kv_bytes = 2 * w.n_seq * w.n_layers * w.n_kv_heads * w.n_tokens * 128 * 2
    do_extras = not args.no_extras and kv_bytes <= 40e9
    cache, st = build_cache(rdkv, synth, torch, w, lay, dims1, lay1=lay1, keep=do_extras)
    q, kn, vn = synth.decode_inputs(w, 0, device="cuda")
    batched = w.n_seq > 1
    grow = args.grow or batched
    # The same decode step is timed twice: first right after the setup, then,
    # for the headline, after the other measurements below.  The part's clocks
    # settle only after a few hundred milliseconds of sustained decode work
    # (and drop again after idling): right after the setup, and after any
    # pause, the same K steps run 10-15% slower than in the steady state a
    # generation loop runs in.
    tm0 = time_decode(rdkv, torch, lay, cache, q, kn, vn, args.steps, args.warmup, not args.no_flush, grow=grow)
    n_c = int(round(tm0["mean_zone_c_rows"]))
    log(f"decode right after the setup: step mean {tm0['step'] * 1e3:.1f} us (chunk kernel "
        f"{tm0['chunk'] * 1e3:.1f} us)")

    layer_loop = None
    if per_layer:
        tg = time_layer_graph(rdkv, torch, lay1, st["layer_caches"], q, kn, vn, args.steps, args.warmup,
                              not args.no_flush, tm0["out"])
        layer_loop = {"us_per_token": round(tg["step"] * 1e3 / w.n_seq, 2),
                      "us_per_token_median": round(tg["step_median"] * 1e3 / w.n_seq, 2),
                      "launches_per_step": 2 * w.n_layers, "max_rel_diff_vs_single_launch": tg["rel_diff"],
                      "note": "one rdkv_decode per layer on its own one-layer blob, the loop captured in a "
                              "HIP graph and replayed per step (every replay checked against the eager loop)"}
        log(f"per-layer graph loop: {tg['step'] * 1e3:.1f} us per step")
    st.pop("layer_caches", None)
    extra = None
    if do_extras:
        extra = extras(rdkv, torch, w, lay, cache, st["kept"], q, kn, vn, tm0["out"], args.steps, args.warmup,
                       not args.no_flush, grow, n_c)
    st.pop("kept", None)
    torch.cuda.empty_cache()

    # The headline: W warmup steps, then exactly K timed steps, after the
    # other measurements and an untimed settling run of the same steps (the
    # frees and host work just above can leave the part idle long enough for
    # its clocks to drop, and they take a few hundred milliseconds of
    # sustained decode work to come back).
    settle = settle_decode(rdkv, torch, lay, cache, q, kn, vn, args.settle_s, not args.no_flush, grow=grow)
    tm = time_decode(rdkv, torch, lay, cache, q, kn, vn, args.steps, args.warmup, not args.no_flush, grow=grow)
    warm = None
    if not args.no_flush and lay.cache_bytes < (200 << 20):
        # a cache this small fits the 256 MB last-level cache: the same steps without clearing it
        tw = time_decode(rdkv, torch, lay, cache, q, kn, vn, args.steps, args.warmup, False, grow=grow)
        warm = {"ms_per_step": round(tw["step"], 5), "kernel_ms": round(tw["chunk"], 5),
                "note": "the same steps with the last-level cache not cleared between them (the blob stays "
                        "resident in it); not an HBM figure"}
    if not torch.equal(tm["out"], tm0["out"]):
        raise RuntimeError("the same decode steps gave different outputs")
    ms_mean, ms_med, wall = tm["step"], tm["step_median"], tm["wall"]
    if args.calibrate_copy:
        src = torch.empty(384 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log(f"decode: step mean {ms_mean * 1e3:.1f} us (chunk kernel {tm['chunk'] * 1e3:.1f} us, "
        f"merge {tm['merge'] * 1e3:.1f} us)")

    desc = rdkv.descriptors(lay, cache)
    b = rdkv.decode_bytes(lay, desc, n_c)
    algo = b["total"] + lay.n_seg * (256 + 2 * 128 * 2)        # descriptors read, new row written
    achieved = algo / (tm["chunk"] * 1e-3) / 1e9
    traffic, valu, traffic_src = counter_traffic("decode_chunk_kernel", w.name)
    N, d = w.n_tokens, 128
    payload_bits = float((st["hist_tok"] * np.array([0, 2, 4, 8, 16])).sum() * d)
    kept = int(desc["n_kept"].sum())
    payload_bits += float(sum(int(desc["n_kept"][i]) * int((desc["n_chan"][i] * np.array([16, 8, 4, 2])).sum())
                              for i in range(lay.n_seg)))
    retention = payload_bits / (32.0 * N * d * lay.n_seg)
    score_flops = 2 * w.n_layers * w.n_seq * w.n_q_heads * (N * (N + 1) / 2) * 2 * d   # two passes
    if batched:
        metric, unit, hib = "decode throughput, generated tokens/s over all sequences", "tokens/s", True
        value = round(w.n_seq * args.steps / (tm["total_ms"] * 1e-3), 1)
    else:
        metric, unit, hib = "decode-attention us/token & effective HBM GB/s (% of peak), one decode step over all layers", "us/token", False
        if w.name == "llama8b-32layer-n128k":
            metric = "decode-attention \u00b5s/token & effective HBM GB/s (% of peak) at 128K, 8B-shape"
        value = round(ms_mean * 1e3 / w.n_seq, 3)
    result = {
        "metric": metric,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_mean, 5),
        "higher_is_better": hib,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1) fp16 activations with heavy-hitter and sink logit bias, "
                "scored, allocated and packed on the GPU)",
        "config": {"workload": w.name, "n_seq": w.n_seq, "n_layers": w.n_layers, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": d, "n_tokens": N, "avg_bits": w.avg_bits,
                   "budget_v": w.budget_v, "budget_k": w.budget_k, "zone_c_rows_mean": tm["mean_zone_c_rows"],
                   "zone_c_grows": grow,
                   "retention": round(retention, 5), "kept_tokens": kept,
                   "bits_tok_hist_0_2_4_8_16": st["hist_tok"].tolist(),
                   "bits_chan_hist_0_2_4_8_16": st["hist_chan"].tolist(),
                   "llc_flushed_between_steps": not args.no_flush, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "traffic_unit": "bytes per launch", "traffic_source": traffic_src,
                     "kernel": "decode_chunk_kernel", "algorithmic_bytes_per_launch": int(algo),
                     "bytes_breakdown": {k: int(v) for k, v in b.items()},
                     "metadata_share": round((b["v_meta"] + b["k_meta"]) / algo, 4),
                     "record_padding_share_of_reads": round(b["k_padding"] / (algo + b["k_padding"]), 4),
                     "kernel_ms": round(tm["chunk"], 5), "kernel_ms_median": round(tm["chunk_median"], 5),
                     "merge_kernel_ms": round(tm["merge"], 5),
                     "step_GBs": round(algo / (ms_mean * 1e-3) / 1e9, 1),
                     "valu": None if valu is None else {
                         "instructions_per_launch": valu, "source": traffic_src,
                         "achieved_Ginstr_per_s": round(valu / (tm["chunk"] * 1e-3) / 1e9, 1),
                         "peak_Ginstr_per_s": VALU_PEAK_GINSTR,
                         "frac": round(valu / (tm["chunk"] * 1e-3) / 1e9 / VALU_PEAK_GINSTR, 4),
                         "lane_instructions_per_algorithmic_byte": round(valu * 64 / algo, 2),
                         "note": "wave64 VALU instructions (SQ_INSTS_VALU) over the same kernel time; the "
                                 "co-limit of this kernel at low bitwidths"}},
        "memory": {"blob_bytes": int(lay.cache_bytes),
                   "fp16_kv_bytes": int(2 * w.n_seq * w.n_layers * w.n_kv_heads * N * d * 2),
                   "kv_bytes_read_per_step": int(algo - b["q_out"]),
                   "blob_vs_fp16": round(lay.cache_bytes / (2 * w.n_seq * w.n_layers * w.n_kv_heads * N * d * 2), 4),
                   "hbm_capacity_share": round(lay.cache_bytes / 288e9, 4),
                   "note": "the blob is allocated for the budget bounds (slot capacity); kv_bytes_read_per_step is "
                           "what the packed cache actually holds and decode reads"},
        "stages": {"setup_s": round(st["setup_s"], 2), "score_ms_total": round(st["score_ms"], 2),
                   "score_tflops_executed": round(score_flops / (st["score_ms"] * 1e-3) / 1e12, 2)
                   if st["score_ms"] > 0 else None,
                   "score_mfma_frac": round(score_flops / (st["score_ms"] * 1e-3) / 1e12 / MFMA_FP16_PEAK_TFS, 4)
                   if st["score_ms"] > 0 else None,
                   "score_mfma_frac_algorithmic": round(score_flops / 2 / (st["score_ms"] * 1e-3) / 1e12 /
                                                        MFMA_FP16_PEAK_TFS, 4) if st["score_ms"] > 0 else None,
                   "score_layer0_ms": None if st.get("score_halves") is None else {
                       "rdkv_score": round(st["score_halves"][2], 2),
                       "rdkv_score_lse": round(st["score_halves"][0], 2),
                       "rdkv_score_from_lse": round(st["score_halves"][1], 2),
                       "note": "layer 0 alone; rdkv_score_from_lse is what scoring costs when the prefill "
                               "forward supplies the row LSE"},
                   "allocate_layer0_ms": None if st.get("score_halves") is None else {
                       "rdkv_allocate": round(st["score_halves"][5], 3),
                       "rdkv_allocate_shared_per_layer": round(st["score_halves"][6], 3),
                       "from_idle_gpu": {"rdkv_allocate": round(st["score_halves"][3], 3),
                                         "rdkv_allocate_shared_per_layer": round(st["score_halves"][4], 3)},
                       "note": "per-segment budgets, and one budget shared by the layer's KV heads; event time "
                               "with the call's launches queued behind other GPU work (its kernels), and from an "
                               "idle GPU (then the host's launches set the pace)"}},
        "wall_s_timed_loop": round(wall, 4),
        "inputs_sha256": inputs_digest(torch, q, kn, vn, cache, lay),
        "settle_steps_before_headline": settle,
        "right_after_setup": {"ms_per_step": round(tm0["step"], 5), "kernel_ms": round(tm0["chunk"], 5),
                              "note": "the same K steps timed right after the cache is built, before the other "
                                      "measurements; the headline is timed after them, in the clocks' steady "
                                      "state"},
    }
    if layer_loop is not None:
        result["per_layer_graph_loop"] = layer_loop
    if warm is not None:
        result["llc_resident"] = warm
    if extra is not None:
        result.update(extra)
    del cache
    torch.cuda.empty_cache()
    if not args.no_fp16_baseline:
        lay16 = rdkv.layout(dims, 16 * w.n_tokens, 16 * 128, w.zone_c_capacity)
        cache16, _ = build_cache(rdkv, synth, torch, w, lay16, dims1, fp16_only=True)
        t16 = time_decode(rdkv, torch, lay16, cache16, q, kn, vn, max(3, args.steps // 4), 2, not args.no_flush)
        ms16 = t16["step"]
        b16 = rdkv.decode_bytes(lay16, rdkv.descriptors(lay16, cache16), n_c)
        result["fp16_full_cache"] = {
            "us_per_token": round(ms16 * 1e3 / w.n_seq, 2),
            "achieved_GBs": round(b16["total"] / (ms16 * 1e-3) / 1e9, 1),
            "bytes_per_step": int(b16["total"]),
            "speedup_of_rdkv": round(ms16 / ms_mean, 2),
            "note": "same kernel on an all-16-bit, nothing-evicted cache (the exact fp16 K/V bytes)"}
        del cache16
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        t0 = time.time()
        result["cpu_baseline"] = cpu_baseline(w, st["hist_tok"], st["hist_chan"], lay.n_seg, n_c,
                                              args.cpu_sample_segments)
        log(f"cpu baseline {time.time() - t0:.1f}s")
        t0 = time.time()
        result["cpu_baseline_scoring"] = cpu_scoring_baseline(w)
        log(f"cpu scoring baseline {time.time() - t0:.1f}s")
        t0 = time.time()
        result["cpu_baseline_tiny_all_stages"] = cpu_baseline_all_stages()
        log(f"cpu all-stage baseline (tiny workload) {time.time() - t0:.1f}s")
        t0 = time.time()
        result["cpu_baseline_32k_layer_all_stages"] = cpu_baseline_c2_all_stages()
        log(f"cpu all-stage baseline (32K layer, sampled) {time.time() - t0:.1f}s")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
