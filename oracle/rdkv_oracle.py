"""Plain, slow, obviously-correct CPU oracle of the RDKV hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module;
it exists so tests, the smoke check and the CPU-baseline leg of the benchmark
can check the HIP library against an independent implementation.  It shares no
code, tables or constants with the HIP sources: the blob format below is
re-implemented here from its written specification.

Everything is numpy.  Floating point is fp64 except where the method fixes a
narrower type (fp16 storage, the fp32 unit cost, the fp32/fp16 quantizer steps),
which are then evaluated with numpy's IEEE fp32/fp16 arithmetic (round to
nearest even).

Sources (cited by page title and section):

* [RDKV] "RDKV - distortion-bit allocation for joint KV cache eviction and
  quantization" (gist.science technical summary of paper 2605.08317):
  section 2.1 (token and channel distortion weights, the rate-distortion
  objective), 2.2 (bitwidth set {0,2,4,8,16}, reverse water-filling /
  Lagrangian relaxation, stage 1 weighting after prefill, stage 2 V-token
  allocation with 0 = eviction, stage 3 K-channel allocation over kept
  tokens), 2.3 (TriZone: zone A packed 2/4/8-bit rows grouped by bitwidth,
  zone B fp16 V rows of 16-bit tokens, zone C fp16 rows of new tokens; fused
  dequantization inside attention).
* [KVMATH] "Matematika KV Cache Compression" (aistudio.id), section
  "Solusi 3: Kuantisasi KV Cache Tingkat Rendah": asymmetric uniform
  quantization with a scale and zero-point per vector; section "Anatomi
  Krisis": bytes of a KV cache = 2 * L * H_kv * D * P * N.

Readings where the pages leave a step open are marked READING and are the
same as in the design notes; they are listed again next to each function.

Parity status: every function below is pinned by tests/test_oracle_*.py
against closed forms, brute force, library routines or printed values.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

D = 128                       # head dimension supported by the format
BITWIDTHS = (0, 2, 4, 8, 16)  # [RDKV] 2.2

# Increments of the Lagrangian water-filling.  Raising a unit from bitwidth
# b_j to b_{j+1} lowers its distortion c * 2^-b by c * (2^-b_j - 2^-b_{j+1})
# at a cost of (b_{j+1} - b_j) bits; the per-bit gain (slope) is
#   0->2: 3/8,  2->4: 3/32,  4->8: 15/1024,  8->16: 255/524288   (times c).
# Every product c * slope is exact in fp64 for an fp32 c.
_STEP_FROM = (0, 2, 4, 8)
_STEP_TO = (2, 4, 8, 16)
STEP_BITS = np.array([b1 - b0 for b0, b1 in zip(_STEP_FROM, _STEP_TO)], dtype=np.int64)
STEP_SLOPE = np.array([(2.0 ** -b0 - 2.0 ** -b1) / (b1 - b0) for b0, b1 in zip(_STEP_FROM, _STEP_TO)])

MAGIC = 0x564B4452            # "RDKV" little-endian
VERSION = 2
HEADER_BYTES = 256
DESC_BYTES = 256
ALIGN = 256


# --------------------------------------------------------------------------
# Stage 1: distortion weights  ([RDKV] 2.1, 2.2 stage 1)
# --------------------------------------------------------------------------

def token_weights(Qg: np.ndarray, Kh: np.ndarray, block: int = 512) -> np.ndarray:
    """w_t = sum over query heads g of the group and query rows tau of a_{g,tau,t}.

    [RDKV] 2.1: the distortion weight of a V token is the attention mass it
    receives, summed over all query positions.  READING: prefill attention is
    causal (token t is visible to rows tau >= t), every prefill position is a
    query, and with GQA the weights of the G query heads that share the KV
    head are summed.

    Qg: [G][N][d] fp16, Kh: [N][d] fp16.  Returns [N] float64.
    """
    G, N, d = Qg.shape
    K64 = Kh.astype(np.float64)
    inv = 1.0 / math.sqrt(d)
    w = np.zeros(N)
    for g in range(G):
        Q64 = Qg[g].astype(np.float64)
        for r0 in range(0, N, block):
            r1 = min(N, r0 + block)
            S = (Q64[r0:r1] @ K64[:r1].T) * inv
            S[np.arange(r1)[None, :] > np.arange(r0, r1)[:, None]] = -np.inf
            S -= S.max(axis=1, keepdims=True)
            P = np.exp(S)
            P /= P.sum(axis=1, keepdims=True)
            w[:r1] += P.sum(axis=0)
    return w


def row_lse(Qh: np.ndarray, Kh: np.ndarray, block: int = 512) -> np.ndarray:
    """LSE_tau = ln sum_{t <= tau} exp(Q[tau].K[t] / sqrt(d)) for one query head.

    The normaliser of the causal prefill softmax whose entries a_{tau,t}
    [RDKV] 2.1 sums into w_t (a_{tau,t} = exp(s_{tau,t} - LSE_tau)); stage 1
    runs after prefill ([RDKV] 2.2), whose attention forward yields it.
    READING as in token_weights (causal, every prefill position a query).
    Qh: [N][d] fp16, Kh: [N][d] fp16.  Returns [N] float64 (natural log).
    """
    N, d = Qh.shape
    Q64, K64 = Qh.astype(np.float64), Kh.astype(np.float64)
    inv = 1.0 / math.sqrt(d)
    out = np.empty(N)
    for r0 in range(0, N, block):
        r1 = min(N, r0 + block)
        S = (Q64[r0:r1] @ K64[:r1].T) * inv
        S[np.arange(r1)[None, :] > np.arange(r0, r1)[:, None]] = -np.inf
        m = S.max(axis=1)
        out[r0:r1] = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
    return out


def token_weights_from_lse(Qg: np.ndarray, Kh: np.ndarray, lse: np.ndarray, block: int = 512) -> np.ndarray:
    """w_t of token_weights, with each row's normaliser taken as given.

    w_t = sum_g sum_{tau >= t} exp(Q_g[tau].K[t] / sqrt(d) - lse[g][tau])
    ([RDKV] 2.1, a_{tau,t} written with its log-normaliser).  Qg: [G][N][d]
    fp16, Kh: [N][d] fp16, lse: [G][N].  Returns [N] float64.
    """
    G, N, d = Qg.shape
    K64 = Kh.astype(np.float64)
    inv = 1.0 / math.sqrt(d)
    w = np.zeros(N)
    for g in range(G):
        Q64 = Qg[g].astype(np.float64)
        for r0 in range(0, N, block):
            r1 = min(N, r0 + block)
            S = (Q64[r0:r1] @ K64[:r1].T) * inv - np.asarray(lse[g][r0:r1], dtype=np.float64)[:, None]
            S[np.arange(r1)[None, :] > np.arange(r0, r1)[:, None]] = -np.inf
            w[:r1] += np.exp(S).sum(axis=0)
    return w


def channel_weights(Qg: np.ndarray, Kh: np.ndarray) -> np.ndarray:
    """w_c = ||Q_{:,c}||_2 * ||K_{:,c}||_2 / sqrt(d)   ([RDKV] 2.1).

    READING: Q_{:,c} stacks the G*N query rows of the heads in the group, and
    K_{:,c} runs over all N prefill tokens (stage 1 uses the full cache).
    Qg: [G][N][d], Kh: [N][d].  Returns [d] float64.
    """
    G, N, d = Qg.shape
    q = np.sqrt(np.sum(Qg.astype(np.float64).reshape(G * N, d) ** 2, axis=0))
    k = np.sqrt(np.sum(Kh.astype(np.float64) ** 2, axis=0))
    return q * k / math.sqrt(d)


def token_variance(Vh: np.ndarray) -> np.ndarray:
    """sigma_t = population variance of the d values of V row t.

    The objective of [RDKV] 2.1 multiplies each unit's weight by sigma_u, the
    spread of the values quantized as that unit.  READING: the variance
    (ddof 0) of the unit's values; for a V token the unit is its row.
    Vh: [N][d].  Returns [N] float64.
    """
    return np.var(Vh.astype(np.float64), axis=1)


# --------------------------------------------------------------------------
# Exact fp32 rounding helpers
# --------------------------------------------------------------------------

def round_rational_to_f32(num: int, den: int) -> np.float32:
    """Correctly rounded (nearest, ties to even) fp32 value of num/den >= 0.

    Exact integer arithmetic; restricted to the normal fp32 range, which is all
    the variance below can produce.
    """
    if num < 0 or den <= 0:
        raise ValueError("num >= 0, den > 0 required")
    if num == 0:
        return np.float32(0.0)
    # choose e with 2^23 <= num / den / 2^e < 2^24
    e = num.bit_length() - den.bit_length() - 24
    while True:
        a, b = (num, den << e) if e >= 0 else (num << -e, den)
        if a >= (b << 24):
            e += 1
        elif a < (b << 23):
            e -= 1
        else:
            break
    m, r = divmod(a, b)
    if 2 * r > b or (2 * r == b and (m & 1)):
        m += 1
    if m == 1 << 24:
        m >>= 1
        e += 1
    if not (-149 <= e and e + 24 <= 128):
        raise OverflowError("value outside the fp32 range handled here")
    if e + 23 < -126:
        raise OverflowError("subnormal fp32 results are not produced by this method")
    return np.float32(math.ldexp(m, e))


def exact_population_variance(x16: np.ndarray) -> Fraction:
    """Exact population variance of fp16 values, as a rational number.

    Every fp16 value is an integer multiple of 2^-24, so with X = x * 2^24,
    var = (n * sum X^2 - (sum X)^2) / (n^2 * 2^48) exactly.  The sums are
    done with Python integers.  An empty input has variance 0.
    """
    n = int(np.size(x16))
    if n == 0:
        return Fraction(0)
    X = [int(v) for v in (np.asarray(x16, np.float16).astype(np.float64) * float(1 << 24)).astype(np.int64).ravel()]
    s1 = sum(X)
    s2 = sum(v * v for v in X)
    return Fraction(n * s2 - s1 * s1, n * n << 48)


def exact_population_variance_f32(x16: np.ndarray) -> np.float32:
    """The exact population variance rounded once (nearest-even) to fp32."""
    v = exact_population_variance(x16)
    return round_rational_to_f32(v.numerator, v.denominator)


def masked_channel_variance(Kh: np.ndarray, bits_tok: np.ndarray) -> np.ndarray:
    """sigma_c over the tokens kept by the V allocation, one value per channel.

    [RDKV] 2.2 stage 3 solves the K-channel problem only over the tokens kept
    in stage 2.  READING: sigma_c is the population variance of K[:, c] over
    the kept tokens (b_t > 0), taken exactly and rounded once to fp32 so that
    the fp32 unit costs are well defined.  No kept tokens gives 0.
    Kh: [N][d] fp16, bits_tok: [N] uint8.  Returns [d] float32.
    """
    kept = Kh[bits_tok > 0]
    return np.array([exact_population_variance_f32(kept[:, c]) for c in range(Kh.shape[1])],
                    dtype=np.float32)


# --------------------------------------------------------------------------
# Stages 2-3: Lagrangian bit allocation  ([RDKV] 2.1 objective, 2.2)
# --------------------------------------------------------------------------

def unit_costs(w: np.ndarray, sigma: np.ndarray) -> np.ndarray:
    """c_u = w_u * sigma_u rounded once to fp32 (both factors are fp32)."""
    return np.asarray(w, np.float32) * np.asarray(sigma, np.float32)


def lagrangian_allocate(c: np.ndarray, budget: int):
    """Bitwidths in {0,2,4,8,16} from reverse water-filling on the unit costs.

    The problem of [RDKV] 2.1 is  min sum_u c_u 2^-b_u  s.t.  sum_u b_u <= B,
    solved by Lagrangian relaxation ([RDKV] 2.2).  For a multiplier lambda each
    unit independently minimises c_u 2^-b + lambda*b over the bitwidth set.
    Because the per-bit gains 3/8 > 3/32 > 15/1024 > 255/524288 decrease, all
    five bitwidths lie on every unit's lower convex hull and the minimiser is
    "take step j iff c_u * slope_j > lambda" (ties stay at the lower
    bitwidth, READING).  The multiplier is the smallest lambda in
    {0} U {c_u * slope_j} whose allocation meets the budget (READING: no greedy
    use of leftover bits).  Units with c_u <= 0 (or NaN) get 0 bits.

    Returns (bits uint8 [n], lambda float64).
    """
    c = np.asarray(c, np.float32)
    if budget < 0:
        raise ValueError("budget must be >= 0")
    v = c.astype(np.float64)[:, None] * STEP_SLOPE[None, :]          # exact
    wts = np.broadcast_to(STEP_BITS[None, :], v.shape)
    pos = v > 0
    if int(wts[pos].sum()) <= budget:
        lam = 0.0
    else:
        vals = v[pos]
        vw = wts[pos]
        order = np.argsort(vals, kind="stable")
        sv, sw = vals[order], vw[order]
        # cost(lambda) = total bits of increments strictly above lambda
        suffix = np.concatenate([np.cumsum(sw[::-1])[::-1], [0]])
        cand = np.unique(sv)
        above = suffix[np.searchsorted(sv, cand, side="right")]
        lam = float(cand[np.argmax(above <= budget)])               # first feasible
    bits = ((v > lam) * wts).sum(axis=1)
    return bits.astype(np.uint8), lam


def allocate_segment(w_tok, var_tok, w_chan, Kh, budget_v: int, budget_k: int):
    """Stage 2 (V tokens) then stage 3 (K channels over kept tokens).

    Inputs are fp32 weights/variances of one segment and its fp16 K [N][d].
    Returns dict(bits_tok, bits_chan, var_chan, lambda_v, lambda_k).
    """
    bt, lv = lagrangian_allocate(unit_costs(w_tok, var_tok), budget_v)
    vc = masked_channel_variance(Kh, bt)
    bc, lk = lagrangian_allocate(unit_costs(w_chan, vc), budget_k)
    return dict(bits_tok=bt, bits_chan=bc, var_chan=vc, lambda_v=lv, lambda_k=lk)


def allocate_group(w_toks, var_toks, w_chans, Ks, budget_v: int, budget_k: int):
    """Stages 2 and 3 with one budget for a group of segments.

    [RDKV] 2.1 states B as the total bit budget; here the units of several
    segments (e.g. the KV heads of a layer) are pooled into one problem per
    stage, each with one multiplier: the V tokens of all segments, then the K
    channels of all segments, whose variances stay per segment over that
    segment's kept tokens.  Inputs are lists (or stacked arrays) over the
    group's segments.  Returns dict(bits_tok [n][N], bits_chan [n][d],
    var_chan [n][d], lambda_v, lambda_k).
    """
    n = len(w_toks)
    N = len(w_toks[0])
    c_v = np.concatenate([unit_costs(w_toks[i], var_toks[i]) for i in range(n)])
    bt, lv = lagrangian_allocate(c_v, budget_v)
    bt = bt.reshape(n, N)
    vc = np.stack([masked_channel_variance(Ks[i], bt[i]) for i in range(n)])
    c_k = np.concatenate([unit_costs(w_chans[i], vc[i]) for i in range(n)])
    bc, lk = lagrangian_allocate(c_k, budget_k)
    return dict(bits_tok=bt, bits_chan=bc.reshape(n, -1), var_chan=vc, lambda_v=lv, lambda_k=lk)


# --------------------------------------------------------------------------
# Quantizer  ([KVMATH] Solusi 3; fp16 scale/zero per (token, bit-segment))
# --------------------------------------------------------------------------

def quantize(x16: np.ndarray, b: int):
    """Asymmetric uniform b-bit quantization of fp16 vectors (last axis).

    scale = (max - min) / (2^b - 1), zero = min, q = round((x - zero) / scale)
    ([KVMATH] Solusi 3), one (scale, zero) per vector.  Fixed precisions: the
    range and the quotient are IEEE fp32 operations, the scale is stored
    rounded to fp16, the zero is the fp16 minimum itself, codes use
    round-half-to-even on the fp32 quotient and are clamped to [0, 2^b - 1];
    a zero scale gives all-zero codes.

    Returns (codes uint32 [..., n], scale fp16 [...], zero fp16 [...]).
    """
    x = np.asarray(x16, np.float16).astype(np.float32)
    mn = x.min(axis=-1)
    mx = x.max(axis=-1)
    rng = (mx - mn).astype(np.float32)
    scale = (rng / np.float32((1 << b) - 1)).astype(np.float32).astype(np.float16)
    zero = mn.astype(np.float16)
    s = scale.astype(np.float32)[..., None]
    diff = (x - zero.astype(np.float32)[..., None]).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = (diff / s).astype(np.float32)
    q = np.clip(np.rint(quot), 0, (1 << b) - 1)
    q = np.where(s == 0, 0, q)
    return q.astype(np.uint32), scale, zero


def dequantize(codes, scale, zero) -> np.ndarray:
    """x_hat = code * scale + zero with a single rounding to fp32 (fused multiply-add).

    code * scale + zero is a multiple of 2^-24 below 2^24, so the fp64
    evaluation is exact and the one rounding to fp32 is that of the fused
    multiply-add.
    """
    s64 = np.asarray(scale, np.float16).astype(np.float64)
    z64 = np.asarray(zero, np.float16).astype(np.float64)
    return (np.asarray(codes, np.float64) * s64 + z64).astype(np.float32)


# --------------------------------------------------------------------------
# Blob format (TriZone, [RDKV] 2.3) -- written from the format specification
# --------------------------------------------------------------------------

def _align(x: int, a: int = ALIGN) -> int:
    return (x + a - 1) // a * a


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


class Layout:
    """Sizes and fixed offsets of a packed cache.

    The blob is: a 256-byte header, one 256-byte descriptor per segment
    (segment = (sequence, layer, KV head), index (s*L + l)*Hkv + h), then one
    fixed-size slot per segment.  A slot holds, at fixed offsets, zone C
    (K then V, [cap][128] fp16 each), the V rows of kept tokens (groups of
    2/4/8-bit code rows then fp16 rows, each group 256-byte aligned), the
    per-token K records and the int32 original positions of kept tokens.
    Region sizes are bounds that follow from the budgets alone.

    With n_generations > 0 the blob also reserves that many generation blobs,
    each a complete blob of this same format (own header, descriptors, slots;
    offsets relative to its own start) for cap tokens per segment, the
    generation budgets, and no zone C: zone C rolls over into the next one
    when it fills (see rollover_pack).  They follow the main blob at
    gen_offset, gen_bytes apart.
    """

    def __init__(self, n_seq, n_layers, n_q_heads, n_kv_heads, head_dim, n_tokens,
                 budget_v, budget_k, zone_c_capacity, n_generations=0, gen_budget_v=0, gen_budget_k=0):
        if head_dim != D:
            raise ValueError("head_dim must be 128")
        self.S, self.L, self.Hq, self.Hkv = n_seq, n_layers, n_q_heads, n_kv_heads
        self.d, self.N = head_dim, n_tokens
        self.budget_v, self.budget_k, self.cap = budget_v, budget_k, zone_c_capacity
        self.n_seg = n_seq * n_layers * n_kv_heads
        self.nk_max = min(n_tokens, budget_v // 2)
        bk = min(budget_k, 16 * D)
        self.rec_max = 4 * ((bk + 98) // 32 + 4)
        self.off_kc = 0
        self.off_vc = zone_c_capacity * D * 2
        self.off_v = _align(2 * zone_c_capacity * D * 2)
        self.v_reserve = _align(min(16 * budget_v, 2 * D * n_tokens) + 768)
        self.off_krec = self.off_v + self.v_reserve
        self.off_pos = self.off_krec + _align(self.nk_max * self.rec_max)
        self.slot_bytes = self.off_pos + _align(4 * self.nk_max)
        self.desc_offset = HEADER_BYTES
        self.slots_offset = _align(HEADER_BYTES + DESC_BYTES * self.n_seg)
        self.cache_bytes = self.slots_offset + self.n_seg * self.slot_bytes
        self.n_gen = n_generations
        self.gen_budget_v, self.gen_budget_k = gen_budget_v, gen_budget_k
        self.gen = None
        self.gen_offset = self.gen_bytes = 0
        if n_generations > 0:
            if zone_c_capacity < 1:
                raise ValueError("generations need a zone C to roll over")
            self.gen = Layout(n_seq, n_layers, n_q_heads, n_kv_heads, head_dim, zone_c_capacity,
                              gen_budget_v, gen_budget_k, 0)
            self.gen_offset = self.cache_bytes
            self.gen_bytes = _align(self.gen.cache_bytes)
            self.cache_bytes = self.gen_offset + n_generations * self.gen_bytes

    def gen_base(self, g):
        return self.gen_offset + g * self.gen_bytes

    def seg_index(self, s, l, h):
        return (s * self.L + l) * self.Hkv + h

    def slot_base(self, seg):
        return self.slots_offset + seg * self.slot_bytes

    def header_bytes(self) -> bytes:
        h = np.zeros(HEADER_BYTES, np.uint8)
        i32 = [MAGIC, VERSION, self.S, self.L, self.Hq, self.Hkv, self.d, self.cap]
        h[0:32] = np.array(i32, np.uint32).view(np.uint8)
        i64 = [self.N, self.budget_v, self.budget_k, self.n_seg, self.desc_offset,
               self.slots_offset, self.slot_bytes]
        h[32:88] = np.array(i64, np.int64).view(np.uint8)
        # generations: count reserved, count in use (0 until a rollover), where
        h[88:96] = np.array([self.n_gen, 0], np.int32).view(np.uint8)
        h[96:128] = np.array([self.gen_offset, self.gen_bytes, self.gen_budget_v, self.gen_budget_k],
                             np.int64).view(np.uint8)
        return h.tobytes()


def channel_permutation(bits_chan: np.ndarray) -> np.ndarray:
    """Channels ordered by bitwidth 16, 8, 4, 2, 0; ties by ascending index."""
    rank = {16: 0, 8: 1, 4: 2, 2: 3, 0: 4}
    return np.array(sorted(range(D), key=lambda c: (rank[int(bits_chan[c])], c)), np.uint8)


def pack_codes(codes, b) -> np.ndarray:
    """LSB-first packing of b-bit codes (last axis) into little-endian uint32 words.

    Element i lands in word i // (32/b) at bit offset (i % (32/b)) * b; a
    partial last word is zero-filled.
    """
    codes = np.asarray(codes, np.uint64)
    per = 32 // b
    n = codes.shape[-1]
    nw = _cdiv(n, per)
    padded = np.zeros(codes.shape[:-1] + (nw * per,), np.uint64)
    padded[..., :n] = codes
    shifts = (np.arange(per, dtype=np.uint64) * np.uint64(b))
    words = (padded.reshape(codes.shape[:-1] + (nw, per)) << shifts).sum(axis=-1)
    return words.astype(np.uint32)


def unpack_codes(words, b, n) -> np.ndarray:
    """Inverse of pack_codes: the first n b-bit codes of the words (last axis)."""
    words = np.asarray(words, np.uint32).astype(np.uint64)
    per = 32 // b
    shifts = (np.arange(per, dtype=np.uint64) * np.uint64(b))
    codes = (words[..., :, None] >> shifts) & np.uint64((1 << b) - 1)
    return codes.reshape(words.shape[:-1] + (words.shape[-1] * per,))[..., :n].astype(np.uint32)


def half2_words(scale, zero) -> np.ndarray:
    """uint32 words holding fp16 scale in the low half and fp16 zero in the high half."""
    sb = np.asarray(scale, np.float16).view(np.uint16).astype(np.uint32)
    zb = np.asarray(zero, np.float16).view(np.uint16).astype(np.uint32)
    return sb | (zb << np.uint32(16))


def record_words(n_chan):
    """Word counts of a K record: (w16, w8, w4, w2, n_meta), n_chan = (n16, n8, n4, n2)."""
    n16, n8, n4, n2 = n_chan
    n_meta = sum(1 for n in (n8, n4, n2) if n > 0)
    return _cdiv(n16, 2), _cdiv(n8, 4), _cdiv(n4, 8), _cdiv(n2, 16), n_meta


def segment_content(Kh, Vh, bits_tok, bits_chan) -> dict:
    """What one segment's packed form holds, independent of where it is placed.

    Kept tokens (b_t > 0) are grouped by bitwidth 2, 4, 8 (zone A) and 16
    (zone B), ascending position inside a group ([RDKV] 2.3, rows grouped by
    bitwidth; the group order is a format choice).  V rows: 2/4/8-bit rows hold
    the 128 codes of the token, LSB-first in uint32 words; 16-bit rows are the
    fp16 values.  One K record per kept token, in the same order: fp16 values
    of the 16-bit channels, then the codes of the 8-, 4- and 2-bit channels
    (channels in permutation order, each part padded to a whole word), then one
    (scale, zero) fp16 pair per present integer part (order 8, 4, 2), then,
    for a 2/4/8-bit token only, the (scale, zero) of its V row; the records of
    16-bit tokens are one word shorter.  0-bit channels are not stored.

    Returns dict(n_tok [4], n_kept, n_chan [4] (16, 8, 4, 2 bits), rec (bytes of
    a zone-A record), perm uint8 [128], v_rows (4 uint8 arrays, one per group),
    records (4 uint32 arrays [n_g][words], one per group), positions int32).
    """
    bits_tok = np.asarray(bits_tok)
    bits_chan = np.asarray(bits_chan)
    Kh = np.asarray(Kh, np.float16)
    Vh = np.asarray(Vh, np.float16)
    groups = [np.nonzero(bits_tok == b)[0] for b in (2, 4, 8, 16)]
    kept = np.concatenate(groups).astype(np.int64)
    nk = len(kept)
    perm = channel_permutation(bits_chan)
    n_chan = [int(np.sum(bits_chan == b)) for b in (16, 8, 4, 2)]
    w16, w8, w4, w2, n_meta = record_words(n_chan)
    rec_words = w16 + w8 + w4 + w2 + n_meta + 1

    # V rows group by group, and the (scale, zero) word of each kept V row
    v_rows = []
    vmeta = []
    for b, toks in zip((2, 4, 8, 16), groups):
        if b == 16:
            v_rows.append(Vh[toks].reshape(len(toks), D).view(np.uint8).reshape(-1))
            vmeta.append(np.zeros(len(toks), np.uint32))
        else:
            q, sc, z = quantize(Vh[toks].reshape(len(toks), D), b)
            v_rows.append(pack_codes(q, b).view(np.uint8).reshape(-1))
            vmeta.append(half2_words(sc, z))

    # K records
    kp = Kh[kept][:, perm.astype(np.int64)].reshape(nk, D)
    c = np.cumsum([0] + n_chan)
    parts = []
    part16 = np.zeros((nk, 2 * w16), np.float16)
    part16[:, :n_chan[0]] = kp[:, c[0]:c[1]]
    parts.append(part16.view(np.uint32).reshape(nk, w16))
    metas = []
    for j, b in zip((1, 2, 3), (8, 4, 2)):
        if n_chan[j] == 0:
            continue
        q, sc, z = quantize(kp[:, c[j]:c[j + 1]], b)
        parts.append(pack_codes(q, b))
        metas.append(half2_words(sc, z).reshape(nk, 1))
    parts += metas
    parts.append(np.concatenate(vmeta).reshape(nk, 1))
    words = np.concatenate(parts, axis=1).astype(np.uint32)
    assert words.shape == (nk, rec_words)
    # zone-A tokens take the full record; 16-bit tokens drop the trailing V
    # word, which they do not have
    starts = np.cumsum([0] + [len(g) for g in groups])
    records = [np.ascontiguousarray(words[starts[g]:starts[g + 1], :rec_words - (g == 3)]) for g in range(4)]
    return dict(n_tok=[len(g) for g in groups], n_kept=nk, n_chan=n_chan, rec=4 * rec_words, perm=perm,
                v_rows=v_rows, records=records, positions=kept.astype(np.int32))


def pack_segment(lay: Layout, blob: np.ndarray, seg: int, Kh, Vh, bits_tok, bits_chan):
    """Write one segment's descriptor and slot into `blob` (uint8 array), the
    content of segment_content placed in the segment's fixed-size slot: V rows
    group after group (each group 256-byte aligned), the K records of all kept
    tokens back to back in kept order, the positions."""
    base = lay.slot_base(seg)
    sc = segment_content(Kh, Vh, bits_tok, bits_chan)
    off_v = []
    cur = base + lay.off_v
    for g in range(4):
        off_v.append(cur)
        blob[cur:cur + sc["v_rows"][g].size] = sc["v_rows"][g]
        cur = _align(cur + sc["v_rows"][g].size)
    off_rec = cur = base + lay.off_krec
    for g in range(4):
        r = sc["records"][g].reshape(-1).view(np.uint8)
        blob[cur:cur + r.size] = r
        cur += r.size
    pos0 = base + lay.off_pos
    blob[pos0: pos0 + 4 * sc["n_kept"]] = sc["positions"].view(np.uint8)
    dsc = np.zeros(DESC_BYTES, np.uint8)
    i32 = sc["n_tok"] + [sc["n_kept"]] + sc["n_chan"] + [sc["rec"], lay.cap, 0]
    dsc[0:48] = np.array(i32, np.int32).view(np.uint8)
    u64 = off_v + [off_rec, pos0, base + lay.off_kc, base + lay.off_vc]
    dsc[48:112] = np.array(u64, np.uint64).view(np.uint8)
    dsc[128:256] = sc["perm"]
    d0 = lay.desc_offset + seg * DESC_BYTES
    blob[d0:d0 + DESC_BYTES] = dsc


def empty_blob(lay: Layout) -> np.ndarray:
    """A cache with every segment empty: header, descriptors with zero counts
    (and the same for every reserved generation blob)."""
    blob = np.zeros(lay.cache_bytes, np.uint8)
    blob[:HEADER_BYTES] = np.frombuffer(lay.header_bytes(), np.uint8)
    for seg in range(lay.n_seg):
        pack_segment(lay, blob, seg, np.zeros((0, D), np.float16), np.zeros((0, D), np.float16),
                     np.zeros(0, np.uint8), np.zeros(D, np.uint8))
    if lay.n_gen:
        empty_gen = empty_blob(lay.gen)
        for g in range(lay.n_gen):
            gen_view(blob, lay, g)[:lay.gen.cache_bytes] = empty_gen
    return blob


def gen_view(blob, lay: Layout, g: int) -> np.ndarray:
    """The bytes of generation blob g (a view: writes go to `blob`)."""
    return blob[lay.gen_base(g):lay.gen_base(g) + lay.gen_bytes]


def gens_in_use(blob) -> int:
    """Generation blobs filled by rollovers so far (header field)."""
    return int(blob[92:96].view(np.int32)[0])


def pack_cache(lay: Layout, K, V, bits_tok, bits_chan, layer_begin: int = 0, blob=None):
    """Pack segments of layers [layer_begin, layer_begin + L_in) into a blob.

    K, V: [S][L_in][Hkv][N][d] fp16; bits_tok [S][L_in][Hkv][N]; bits_chan
    [S][L_in][Hkv][d].  Segments not covered keep their previous content
    (a fresh blob starts empty).
    """
    if blob is None:
        blob = empty_blob(lay)
    S, Lin = K.shape[0], K.shape[1]
    for s in range(S):
        for l in range(Lin):
            for h in range(lay.Hkv):
                seg = lay.seg_index(s, layer_begin + l, h)
                pack_segment(lay, blob, seg, K[s, l, h], V[s, l, h], bits_tok[s, l, h], bits_chan[s, l, h])
    return blob


# --------------------------------------------------------------------------
# Blob parsing and decode  ([RDKV] 2.3, fused dequant attention over A+B+C)
# --------------------------------------------------------------------------

def _u32(blob, off, n):
    return blob[off:off + 4 * n].view(np.uint32)


def _half_pairs(words):
    """(scale, zero) fp16 arrays from uint32 words (scale in the low half)."""
    h = np.asarray(words, np.uint32).reshape(-1, 1).view(np.float16)
    return h[:, 0], h[:, 1]


def read_descriptor(blob, lay: Layout, seg: int) -> dict:
    d0 = lay.desc_offset + seg * DESC_BYTES
    i32 = blob[d0:d0 + 48].view(np.int32)
    u64 = blob[d0 + 48:d0 + 112].view(np.uint64)
    return dict(n_tok=[int(x) for x in i32[0:4]], n_kept=int(i32[4]),
                n_chan=[int(x) for x in i32[5:9]], rec=int(i32[9]), cap=int(i32[10]),
                off_v=[int(x) for x in u64[0:4]], off_krec=int(u64[4]), off_pos=int(u64[5]),
                off_kc=int(u64[6]), off_vc=int(u64[7]),
                perm=blob[d0 + 128:d0 + 256].copy())


def dequantize_content(n_tok, n_chan, rec, perm, v_rows, words):
    """Dequantized kept rows from a segment's content (any placement).

    v_rows: the 4 groups' V row bytes; words: uint32 [n_kept][rec/4] records
    in kept order (a 16-bit token's missing V word as 0).  Returns (K_hat,
    V_hat) float32 [n_kept][128], K_hat in original channel order with 0 on
    0-bit channels."""
    nk = sum(n_tok)
    n16, n8, n4, n2 = n_chan
    w16, w8, w4, w2, n_meta = record_words(n_chan)
    vs, vz = _half_pairs(words[:, -1])
    Vh = np.zeros((nk, D), np.float32)
    i = 0
    for gi, b in enumerate((2, 4, 8, 16)):
        n = n_tok[gi]
        row = D * b // 8
        raw = np.asarray(v_rows[gi][:n * row], np.uint8)
        if b == 16:
            Vh[i:i + n] = raw.view(np.float16).reshape(n, D).astype(np.float32)
        else:
            codes = unpack_codes(raw.view(np.uint32).reshape(n, row // 4), b, D)
            Vh[i:i + n] = dequantize(codes, vs[i:i + n, None], vz[i:i + n, None])
        i += n
    kp = np.zeros((nk, D), np.float32)
    kp[:, :n16] = words[:, :w16].copy().view(np.float16)[:, :n16].astype(np.float32)
    wo, mo, c0 = w16, w16 + w8 + w4 + w2, n16
    for n, b, nw in ((n8, 8, w8), (n4, 4, w4), (n2, 2, w2)):
        if n == 0:
            continue
        s, z = _half_pairs(words[:, mo])
        kp[:, c0:c0 + n] = dequantize(unpack_codes(words[:, wo:wo + nw], b, n), s[:, None], z[:, None])
        mo, wo, c0 = mo + 1, wo + nw, c0 + n
    Kh = np.zeros((nk, D), np.float32)
    Kh[:, np.asarray(perm).astype(np.int64)] = kp
    return Kh, Vh


def unpack_segment(blob, lay: Layout, seg: int):
    """Dequantized kept rows of one segment, in kept order.

    Returns (K_hat [n_kept][128] float32 with 0 on 0-bit channels,
    V_hat [n_kept][128] float32, positions [n_kept] int32, bits [n_kept]).
    """
    ds = read_descriptor(blob, lay, seg)
    nk, rec = ds["n_kept"], ds["rec"]
    n_a = nk - ds["n_tok"][3]
    ra = _u32(blob, ds["off_krec"], n_a * rec // 4).reshape(n_a, rec // 4)
    rb = _u32(blob, ds["off_krec"] + n_a * rec, (nk - n_a) * (rec // 4 - 1)).reshape(nk - n_a, rec // 4 - 1)
    words = np.concatenate([ra, np.concatenate([rb, np.zeros((nk - n_a, 1), np.uint32)], axis=1)])
    tb = np.concatenate([np.full(n, b, np.int32) for n, b in zip(ds["n_tok"], (2, 4, 8, 16))])
    v_rows = [blob[ds["off_v"][g]:ds["off_v"][g] + ds["n_tok"][g] * D * (2 << g) // 8] for g in range(4)]
    Kh, Vh = dequantize_content(ds["n_tok"], ds["n_chan"], rec, ds["perm"], v_rows, words)
    pos = blob[ds["off_pos"]:ds["off_pos"] + 4 * nk].view(np.int32).copy()
    return Kh, Vh, pos, tb


def zone_c_rows(blob, lay: Layout, seg: int, n_rows: int):
    ds = read_descriptor(blob, lay, seg)
    kc = blob[ds["off_kc"]:ds["off_kc"] + n_rows * D * 2].view(np.float16).reshape(n_rows, D)
    vc = blob[ds["off_vc"]:ds["off_vc"] + n_rows * D * 2].view(np.float16).reshape(n_rows, D)
    return kc.astype(np.float32), vc.astype(np.float32)


def append_zone_c(blob, lay: Layout, c_len: int, k_new, v_new):
    """Write the new token's fp16 k, v at row c_len of every segment's zone C."""
    if not (0 <= c_len < lay.cap):
        raise ValueError("zone C is full")
    for s in range(lay.S):
        for l in range(lay.L):
            for h in range(lay.Hkv):
                ds = read_descriptor(blob, lay, lay.seg_index(s, l, h))
                o = ds["off_kc"] + c_len * D * 2
                blob[o:o + D * 2] = np.asarray(k_new[s, l, h], np.float16).view(np.uint8)
                o = ds["off_vc"] + c_len * D * 2
                blob[o:o + D * 2] = np.asarray(v_new[s, l, h], np.float16).view(np.uint8)


def attention(q64: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """softmax(q K^T / sqrt(d)) V in fp64 for q [G][d], K, V [n][d]; empty n -> 0."""
    if K.shape[0] == 0:
        return np.zeros((q64.shape[0], V.shape[1]))
    s = (q64 @ K.astype(np.float64).T) / math.sqrt(q64.shape[1])
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ V.astype(np.float64)


def decode_step(blob, lay: Layout, q, c_len: int, k_new=None, v_new=None):
    """One decode step over every segment; returns out [S][L][Hq][d] float64.

    If k_new/v_new are given they are first appended at zone-C row c_len and
    the step attends over c_len + 1 zone-C rows, else over c_len rows.
    Attention runs over the kept tokens (zones A and B, dequantized, 0-bit K
    channels contributing 0) and the zone-C rows; evicted tokens take no part
    in the softmax (READING of bitwidth 0 = eviction, [RDKV] 2.2).
    The logit scale stays 1/sqrt(128).
    """
    n_c = c_len
    if k_new is not None:
        append_zone_c(blob, lay, c_len, k_new, v_new)
        n_c = c_len + 1
    G = lay.Hq // lay.Hkv
    out = np.zeros((lay.S, lay.L, lay.Hq, D))
    for s in range(lay.S):
        for l in range(lay.L):
            for h in range(lay.Hkv):
                seg = lay.seg_index(s, l, h)
                out[s, l, h * G:(h + 1) * G] = decode_segment(blob, lay, seg, q[s, l, h * G:(h + 1) * G], n_c)
    return out


def kept_rows(blob, lay: Layout, seg: int):
    """Dequantized K and V rows of every kept token of a segment: the prefill
    generation, then each rolled-over generation in use, in that order."""
    Ks, Vs = [], []
    Kh, Vh, _, _ = unpack_segment(blob, lay, seg)
    Ks.append(Kh), Vs.append(Vh)
    for g in range(gens_in_use(blob) if lay.n_gen else 0):
        Kg, Vg, _, _ = unpack_segment(gen_view(blob, lay, g), lay.gen, seg)
        Ks.append(Kg), Vs.append(Vg)
    return np.concatenate(Ks), np.concatenate(Vs)


def decode_segment(blob, lay: Layout, seg: int, qg, n_c: int):
    """Attention output [G][d] (float64) of one segment's G query heads over its
    kept tokens (every generation) and its first n_c zone-C rows (the
    per-segment part of decode_step; segments are independent)."""
    Kh, Vh = kept_rows(blob, lay, seg)
    kc, vc = zone_c_rows(blob, lay, seg, n_c)
    Ka = np.concatenate([Kh, kc])
    Va = np.concatenate([Vh, vc])
    return attention(np.asarray(qg, np.float16).astype(np.float64), Ka, Va)


# --------------------------------------------------------------------------
# Zone-C rollover: decode-time scoring of the new tokens, then allocation and
# packing into a new generation ([RDKV] 2.3 zone C holds the new tokens;
# [KVMATH] "Solusi 2": attention accumulated over decode steps, summed over
# heads, as the importance of a token; [RDKV] 2.1-2.2 for the weights and the
# allocation)
# --------------------------------------------------------------------------

def new_zone_c_stats(lay: Layout) -> np.ndarray:
    """Decode-time statistics of zone C, float64 [n_seg][G][cap + d]: per query
    head, the attention mass each zone-C row has received so far, then the sum
    of squares of each query channel over the steps so far."""
    return np.zeros((lay.n_seg, lay.Hq // lay.Hkv, lay.cap + D))


def decode_step_accumulate(blob, lay: Layout, q, c_len: int, k_new, v_new, stats):
    """decode_step that also accumulates the step into `stats`.

    READING ([RDKV] 2.1 applied to the decode queries, [KVMATH] Solusi 2): the
    weight of a new token is the attention it receives from every query that
    sees it -- each decode step's query heads, the token's own step included --
    taken from the step's softmax over the whole cache (every generation and
    zone C).  Per head g and zone-C row j < n_c, stats[seg][g][j] gains that
    softmax probability; stats[seg][g][cap + c] gains q_g[c]^2, the square of
    the fp16 query value (the query side of the channel weight).
    Returns out [S][L][Hq][d] like decode_step.
    """
    n_c = c_len
    if k_new is not None:
        append_zone_c(blob, lay, c_len, k_new, v_new)
        n_c = c_len + 1
    G = lay.Hq // lay.Hkv
    out = np.zeros((lay.S, lay.L, lay.Hq, D))
    for s in range(lay.S):
        for l in range(lay.L):
            for h in range(lay.Hkv):
                seg = lay.seg_index(s, l, h)
                qg = np.asarray(q[s, l, h * G:(h + 1) * G], np.float16).astype(np.float64)
                Kh, Vh = kept_rows(blob, lay, seg)
                kc, vc = zone_c_rows(blob, lay, seg, n_c)
                Ka, Va = np.concatenate([Kh, kc]), np.concatenate([Vh, vc])
                if Ka.shape[0]:
                    sc = (qg @ Ka.astype(np.float64).T) / math.sqrt(D)
                    p = np.exp(sc - sc.max(axis=1, keepdims=True))
                    p /= p.sum(axis=1, keepdims=True)
                    out[s, l, h * G:(h + 1) * G] = p @ Va.astype(np.float64)
                    stats[seg, :, :n_c] += p[:, Kh.shape[0]:]
                stats[seg, :, lay.cap:] += qg * qg
    return out


def rollover_weights(blob, lay: Layout, stats):
    """Stage-1 weights of the cap zone-C tokens of every segment, from the
    decode-time statistics ([RDKV] 2.1 with the decode queries in place of the
    prefill rows):
      w_tok[seg][j]  = sum over heads of the accumulated attention mass of row j
      var_tok[seg][j]= population variance of V_C row j (as token_variance)
      w_chan[seg][c] = ||Q_{:,c}|| ||K_C[:, c]|| / sqrt(d), with ||Q_{:,c}||^2
                       the accumulated sum of squares over heads and steps
    Returns float64 arrays [n_seg][cap], [n_seg][cap], [n_seg][d]."""
    n = lay.n_seg
    w_tok = stats[:, :, :lay.cap].sum(axis=1)
    var_tok = np.zeros((n, lay.cap))
    w_chan = np.zeros((n, D))
    for seg in range(n):
        kc, vc = zone_c_rows(blob, lay, seg, lay.cap)
        var_tok[seg] = token_variance(vc)
        qn = np.sqrt(stats[seg, :, lay.cap:].sum(axis=0))
        kn = np.sqrt(np.sum(kc.astype(np.float64) ** 2, axis=0))
        w_chan[seg] = qn * kn / math.sqrt(D)
    return w_tok, var_tok, w_chan


def rollover_pack(blob, lay: Layout, gen: int, w_tok, var_tok, w_chan):
    """Roll the full zone C of every segment into generation blob `gen`.

    The cap zone-C tokens of a segment are one more unit set of the problem of
    [RDKV] 2.1, allocated by the same stages ([RDKV] 2.2: V tokens with the
    generation's V budget, then K channels over the kept ones with its K
    budget) from the given fp32 weights (rounded to fp32 here), quantized and
    packed like the prefill generation ([RDKV] 2.3) into the generation blob,
    whose descriptors then hold them.  Afterwards zone C is cleared and the
    header counts gen + 1 generations in use.  Generations are filled in
    order (gen == generations in use so far).  Returns the per-segment
    allocations (dicts of allocate_segment).
    """
    if not (0 <= gen < lay.n_gen) or gen != gens_in_use(blob):
        raise ValueError("generation index out of order or beyond the reserved ones")
    view = gen_view(blob, lay, gen)
    allocs = []
    for s in range(lay.S):
        for l in range(lay.L):
            for h in range(lay.Hkv):
                seg = lay.seg_index(s, l, h)
                kc, vc = zone_c_rows(blob, lay, seg, lay.cap)
                k16, v16 = kc.astype(np.float16), vc.astype(np.float16)
                a = allocate_segment(np.asarray(w_tok[seg], np.float32), np.asarray(var_tok[seg], np.float32),
                                     np.asarray(w_chan[seg], np.float32), k16, lay.gen_budget_v, lay.gen_budget_k)
                pack_segment(lay.gen, view, seg, k16, v16, a["bits_tok"], a["bits_chan"])
                allocs.append(a)
    for seg in range(lay.n_seg):
        ds = read_descriptor(blob, lay, seg)
        blob[ds["off_kc"]:ds["off_kc"] + lay.cap * D * 2] = 0
        blob[ds["off_vc"]:ds["off_vc"] + lay.cap * D * 2] = 0
    blob[92:96] = np.array([gen + 1], np.int32).view(np.uint8)
    return allocs


# --------------------------------------------------------------------------
# Paged cache for batched serving ([KVMATH] "Solusi 1": the KV cache cut into
# fixed-size blocks of a shared pool, non-contiguous, found through a block
# table per sequence; here the blocks hold the packed zones of [RDKV] 2.3)
# --------------------------------------------------------------------------

PAGED_MAGIC = 0x504B4452      # "RDKP" little-endian
PAGE_BYTES = 32768
TILE = 64
# Regions of a segment, each an array of 64-row tiles laid page by page
# (a tile never straddles a page; a page holds PAGE_BYTES // tile bytes
# tiles): V rows of the 2/4/8/16-bit groups, K records of the same groups,
# zone-C keys, zone-C values, kept positions.
N_REGIONS = 11
R_V, R_REC, R_KC, R_VC, R_POS = 0, 4, 8, 9, 10


def region_tile_bytes(region: int, rec: int) -> int:
    """Bytes of a 64-row tile of a region; rec = bytes of a zone-A K record."""
    if region < R_REC:
        return TILE * D * (2 << region) // 8
    if region < R_KC:
        return TILE * (rec - 4 * (region - R_REC == 3))
    if region < R_POS:
        return TILE * D * 2
    return TILE * 4


def region_pages(rows: int, tile_bytes: int) -> int:
    if rows <= 0 or tile_bytes <= 0:
        return 0
    return _cdiv(_cdiv(rows, TILE), PAGE_BYTES // tile_bytes)


def segment_region_pages(n_tok, n_kept, rec, cap):
    """Pages of each of the 11 regions of a segment."""
    rows = list(n_tok) + list(n_tok) + [cap, cap, n_kept]
    return [region_pages(rows[r], region_tile_bytes(r, rec)) for r in range(N_REGIONS)]


class PagedLayout:
    """A paged cache: 256-byte header, one 256-byte descriptor per segment
    slot (sequence slot s, layer, KV head), the block table int32
    [n_seg][max_pages] (physical page of each virtual page of a segment, -1
    where unused), then the pool of n_pages pages of PAGE_BYTES.  Sequences
    come and go: each is packed with its own prefill length and budgets (up
    to the layout's bounds) into pages its caller gives it.
    """

    def __init__(self, n_seq, n_layers, n_q_heads, n_kv_heads, n_tokens_max, budget_v_max, budget_k_max,
                 zone_c_capacity, n_pages):
        self.S, self.L, self.Hq, self.Hkv = n_seq, n_layers, n_q_heads, n_kv_heads
        self.N, self.bv, self.bk, self.cap, self.n_pages = n_tokens_max, budget_v_max, budget_k_max, \
            zone_c_capacity, n_pages
        self.n_seg = n_seq * n_layers * n_kv_heads
        nk_max = min(n_tokens_max, budget_v_max // 2)
        rec_max = 4 * ((min(budget_k_max, 16 * D) + 98) // 32 + 4)
        rows = [min(n_tokens_max, budget_v_max // (2 << g)) for g in range(4)]
        # (at least one entry per segment, so every table row exists)
        self.max_pages = max(1, sum(region_pages(rows[g], region_tile_bytes(R_V + g, rec_max)) for g in range(4))
                             + sum(region_pages(rows[g], TILE * rec_max) for g in range(4))
                             + 2 * region_pages(zone_c_capacity, TILE * D * 2) + region_pages(nk_max, TILE * 4))
        self.desc_offset = HEADER_BYTES
        self.table_offset = _align(HEADER_BYTES + DESC_BYTES * self.n_seg)
        self.pool_offset = _align(self.table_offset + 4 * self.n_seg * self.max_pages, 4096)
        self.cache_bytes = self.pool_offset + n_pages * PAGE_BYTES

    def seg_index(self, s, l, h):
        return (s * self.L + l) * self.Hkv + h

    def header_bytes(self) -> bytes:
        h = np.zeros(HEADER_BYTES, np.uint8)
        i32 = [PAGED_MAGIC, VERSION, self.S, self.L, self.Hq, self.Hkv, D, self.cap]
        h[0:32] = np.array(i32, np.uint32).view(np.uint8)
        i64 = [self.N, self.bv, self.bk, self.n_seg, self.desc_offset, self.table_offset, self.pool_offset,
               self.max_pages, self.n_pages, PAGE_BYTES]
        h[32:112] = np.array(i64, np.int64).view(np.uint8)
        return h.tobytes()


def paged_empty(play: PagedLayout) -> np.ndarray:
    """A paged cache with every sequence slot free: header, zero descriptors
    (zone-C capacity 0 marks a free slot), block table all -1, pool zero."""
    blob = np.zeros(play.cache_bytes, np.uint8)
    blob[:HEADER_BYTES] = np.frombuffer(play.header_bytes(), np.uint8)
    blob[play.table_offset:play.table_offset + 4 * play.n_seg * play.max_pages] = 0xFF
    return blob


def _paged_table(blob, play: PagedLayout, seg: int) -> np.ndarray:
    o = play.table_offset + 4 * seg * play.max_pages
    return blob[o:o + 4 * play.max_pages].view(np.int32)


def paged_pages_needed(play: PagedLayout, content: dict) -> int:
    """Pages one segment of this content takes (its zone C included)."""
    return sum(segment_region_pages(content["n_tok"], content["n_kept"], content["rec"], play.cap))


def _tile_offset(blob, play: PagedLayout, seg: int, vpage: int, tile: int, tile_bytes: int) -> int:
    """Blob offset of tile `tile` of the region starting at virtual page vpage."""
    tpp = PAGE_BYTES // tile_bytes
    phys = int(_paged_table(blob, play, seg)[vpage + tile // tpp])
    if not (0 <= phys < play.n_pages):
        raise ValueError("block table entry outside the pool")
    return play.pool_offset + phys * PAGE_BYTES + (tile % tpp) * tile_bytes


def _region_rw(blob, play, seg, vpage, tile_bytes, row_bytes, nrows, data=None):
    """Write (data given) or read the nrows rows of a region, tile by tile.
    Rows of 0 bytes (the K record of a 16-bit token when every K channel has
    0 bits) take no pages."""
    if row_bytes == 0:
        return None if data is not None else np.zeros(0, np.uint8)
    out = []
    for t in range(_cdiv(nrows, TILE)):
        r = min(TILE, nrows - t * TILE)
        o = _tile_offset(blob, play, seg, vpage, t, tile_bytes)
        if data is None:
            out.append(blob[o:o + r * row_bytes].copy())
        else:
            blob[o:o + r * row_bytes] = data[t * TILE * row_bytes:(t * TILE + r) * row_bytes]
    return None if data is not None else (np.concatenate(out) if out else np.zeros(0, np.uint8))


def paged_pack_sequence(blob, play: PagedLayout, s: int, K, V, bits_tok, bits_chan, pages):
    """Pack one sequence into slot s of the paged cache.

    K, V: fp16 [L][Hkv][N_s][d] (the sequence's own prefill length N_s <= the
    layout's bound); bits_tok [L][Hkv][N_s], bits_chan [L][Hkv][d] within the
    layout's budget bounds; pages: for each of its L*Hkv segments (layer-major,
    then KV head) the list of physical pages it takes, paged_pages_needed of
    them.  Regions are laid out in order, each from a fresh virtual page;
    zone C starts empty.
    """
    for l in range(play.L):
        for h in range(play.Hkv):
            seg = play.seg_index(s, l, h)
            sc = segment_content(K[l][h], V[l][h], bits_tok[l][h], bits_chan[l][h])
            rp = segment_region_pages(sc["n_tok"], sc["n_kept"], sc["rec"], play.cap)
            pg = list(pages[l * play.Hkv + h])
            if len(pg) != sum(rp) or sum(rp) > play.max_pages or sc["n_kept"] > min(play.N, play.bv // 2) \
                    or sc["rec"] > 4 * ((min(play.bk, 16 * D) + 98) // 32 + 4):
                raise ValueError("allocation beyond the layout's bounds or wrong page count")
            table = _paged_table(blob, play, seg)
            table[:] = -1
            table[:len(pg)] = pg
            vpage = np.concatenate([[0], np.cumsum(rp)[:-1]]).astype(np.int64)
            for g in range(4):
                rb = D * (2 << g) // 8
                _region_rw(blob, play, seg, int(vpage[R_V + g]), region_tile_bytes(R_V + g, sc["rec"]), rb,
                           sc["n_tok"][g], sc["v_rows"][g])
                recb = sc["rec"] - 4 * (g == 3)
                _region_rw(blob, play, seg, int(vpage[R_REC + g]), region_tile_bytes(R_REC + g, sc["rec"]), recb,
                           sc["n_tok"][g], sc["records"][g].reshape(-1).view(np.uint8))
            # zone C starts empty: its tiles are cleared whole
            rows_c = _cdiv(play.cap, TILE) * TILE
            zero = np.zeros(rows_c * D * 2, np.uint8)
            for r in (R_KC, R_VC):
                _region_rw(blob, play, seg, int(vpage[r]), region_tile_bytes(r, sc["rec"]), D * 2, rows_c, zero)
            _region_rw(blob, play, seg, int(vpage[R_POS]), TILE * 4, 4, sc["n_kept"], sc["positions"].view(np.uint8))
            dsc = np.zeros(DESC_BYTES, np.uint8)
            i32 = sc["n_tok"] + [sc["n_kept"]] + sc["n_chan"] + [sc["rec"], play.cap, 0]
            dsc[0:48] = np.array(i32, np.int32).view(np.uint8)
            dsc[48:96] = np.array(list(vpage) + [sum(rp)], np.int32).view(np.uint8)
            dsc[128:256] = sc["perm"]
            d0 = play.desc_offset + seg * DESC_BYTES
            blob[d0:d0 + DESC_BYTES] = dsc


def paged_release_sequence(blob, play: PagedLayout, s: int):
    """Free slot s: its descriptors become empty (capacity 0) and its block
    table rows -1.  Returns the physical pages it held, for the caller to reuse."""
    freed = []
    for l in range(play.L):
        for h in range(play.Hkv):
            seg = play.seg_index(s, l, h)
            t = _paged_table(blob, play, seg)
            freed += [int(x) for x in t if x >= 0]
            t[:] = -1
            d0 = play.desc_offset + seg * DESC_BYTES
            blob[d0:d0 + DESC_BYTES] = 0
    return freed


def paged_read_descriptor(blob, play: PagedLayout, seg: int) -> dict:
    d0 = play.desc_offset + seg * DESC_BYTES
    i32 = blob[d0:d0 + 96].view(np.int32)
    return dict(n_tok=[int(x) for x in i32[0:4]], n_kept=int(i32[4]), n_chan=[int(x) for x in i32[5:9]],
                rec=int(i32[9]), cap=int(i32[10]), flags=int(i32[11]), vpage=[int(x) for x in i32[12:23]],
                n_pages=int(i32[23]), perm=blob[d0 + 128:d0 + 256].copy())


def paged_segment_rows(blob, play: PagedLayout, seg: int, n_c: int):
    """Dequantized kept rows and the first n_c zone-C rows of a segment, read
    through its block table: (K_hat, V_hat, K_C, V_C) float32."""
    ds = paged_read_descriptor(blob, play, seg)
    if ds["cap"] == 0:
        z = np.zeros((0, D), np.float32)
        return z, z, z, z
    rec, vp = ds["rec"], ds["vpage"]
    v_rows = [_region_rw(blob, play, seg, vp[R_V + g], region_tile_bytes(R_V + g, rec), D * (2 << g) // 8,
                         ds["n_tok"][g]) for g in range(4)]
    words = []
    for g in range(4):
        recb = rec - 4 * (g == 3)
        w = _region_rw(blob, play, seg, vp[R_REC + g], region_tile_bytes(R_REC + g, rec), recb,
                       ds["n_tok"][g]).view(np.uint32).reshape(ds["n_tok"][g], recb // 4)
        if g == 3:
            w = np.concatenate([w, np.zeros((w.shape[0], 1), np.uint32)], axis=1)
        words.append(w)
    Kh, Vh = dequantize_content(ds["n_tok"], ds["n_chan"], rec, ds["perm"], v_rows, np.concatenate(words))
    kc = _region_rw(blob, play, seg, vp[R_KC], TILE * D * 2, D * 2, n_c).view(np.float16).reshape(n_c, D)
    vc = _region_rw(blob, play, seg, vp[R_VC], TILE * D * 2, D * 2, n_c).view(np.float16).reshape(n_c, D)
    return Kh, Vh, kc.astype(np.float32), vc.astype(np.float32)


def paged_positions(blob, play: PagedLayout, seg: int) -> np.ndarray:
    ds = paged_read_descriptor(blob, play, seg)
    return _region_rw(blob, play, seg, ds["vpage"][R_POS], TILE * 4, 4, ds["n_kept"]).view(np.int32)


def paged_write_zone_c(blob, play: PagedLayout, seg: int, row: int, k, v):
    """Write fp16 k, v [d] at zone-C row `row` of a segment, through its pages."""
    ds = paged_read_descriptor(blob, play, seg)
    for r, src in ((R_KC, k), (R_VC, v)):
        o = _tile_offset(blob, play, seg, ds["vpage"][r], row // TILE, TILE * D * 2) + (row % TILE) * D * 2
        blob[o:o + D * 2] = np.asarray(src, np.float16).view(np.uint8)


def paged_decode_step(blob, play: PagedLayout, q, c_len, k_new=None, v_new=None):
    """One decode step over every sequence slot in use; out [S][L][Hq][d].

    c_len[s]: zone-C rows of sequence s before the step.  With k_new/v_new
    (fp16 [S][L][Hkv][d]) each sequence in use appends its token at its own row
    c_len[s] and attends c_len[s] + 1 rows.  Attention as decode_step: kept
    tokens (dequantized) and zone C, evicted tokens absent; free slots give 0.
    """
    G = play.Hq // play.Hkv
    out = np.zeros((play.S, play.L, play.Hq, D))
    for s in range(play.S):
        for l in range(play.L):
            for h in range(play.Hkv):
                seg = play.seg_index(s, l, h)
                ds = paged_read_descriptor(blob, play, seg)
                if ds["cap"] == 0:
                    continue
                n_c = int(c_len[s])
                if k_new is not None:
                    if not (0 <= n_c < play.cap):
                        raise ValueError("zone C is full")
                    paged_write_zone_c(blob, play, seg, n_c, k_new[s, l, h], v_new[s, l, h])
                    n_c += 1
                Kh, Vh, kc, vc = paged_segment_rows(blob, play, seg, n_c)
                out[s, l, h * G:(h + 1) * G] = attention(np.asarray(q[s, l, h * G:(h + 1) * G], np.float16)
                                                         .astype(np.float64), np.concatenate([Kh, kc]),
                                                         np.concatenate([Vh, vc]))
    return out


# --------------------------------------------------------------------------
# Byte accounting  ([KVMATH] Anatomi Krisis; [RDKV] 1: decode rereads the cache)
# --------------------------------------------------------------------------

def kv_bytes_fp16_per_token(n_layers: int, n_kv_heads: int, head_dim: int, bytes_per_elem: float = 2.0):
    """Bytes of an uncompressed KV cache per token: 2 (K and V) * L * H_kv * D * P."""
    return 2 * n_layers * n_kv_heads * head_dim * bytes_per_elem


def segment_decode_bytes(blob, lay: Layout, seg: int, n_c: int) -> int:
    """Bytes one decode step must read for a segment: V rows, K records, zone C.

    Counted from the packed descriptor: code/fp16 payload of every kept row,
    the (scale, zero) words, and n_c fp16 K and V rows of zone C.  Word padding
    inside records is included (it is read); alignment gaps are not.
    """
    ds = read_descriptor(blob, lay, seg)
    v = sum(n * D * b // 8 for n, b in zip(ds["n_tok"], (2, 4, 8, 16)))
    k = ds["n_kept"] * ds["rec"] - 4 * ds["n_tok"][3]
    return v + k + 2 * n_c * D * 2


def segment_payload_bytes(blob, lay: Layout, seg: int) -> float:
    """Bytes of quantized/fp16 values alone (no scale/zero words, no padding).

    sum over kept tokens of (d * b_t + sum_c b_c) / 8: the rate of the
    allocation in bytes.
    """
    ds = read_descriptor(blob, lay, seg)
    vbits = sum(n * D * b for n, b in zip(ds["n_tok"], (2, 4, 8, 16)))
    kbits = ds["n_kept"] * sum(n * b for n, b in zip(ds["n_chan"], (16, 8, 4, 2)))
    return (vbits + kbits) / 8


# --------------------------------------------------------------------------
# Whole pipeline on one segment (convenience for tests and the CPU baseline)
# --------------------------------------------------------------------------

def score_segment(Qg, Kh, Vh):
    """Stage 1 on one segment: (w_tok, var_tok, w_chan) in float64."""
    return token_weights(Qg, Kh), token_variance(Vh), channel_weights(Qg, Kh)
