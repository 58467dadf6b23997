"""Seeded synthetic workloads for the RDKV hot path.

This module only *draws inputs*: prefill Q/K/V, decode-step q/k_new/v_new and
the per-workload bit budgets.  It contains none of the method's arithmetic
(no attention, no weights, no allocation, no quantization), so both the HIP
path and the CPU oracle can be fed from it in tests.

Workload structure follows what the RDKV technical summary (gist.science
2605.08317, section 4 "Experimental results") evaluates on: LLaMA-3.1-8B and
Qwen2.5-72B shaped layers at 32K..256K context.  The models, weights and
benchmark suites are not available, so activations are N(0,1) fp16 with the
structure each workload names:

* outlier K channels (a few channels scaled by a constant, or log-normal
  per-channel scales);
* heavy-hitter tokens: a seeded subset of tokens whose attention logit is
  raised by a constant.  The bias is realised inside Q and K themselves:
  channel 0 is reserved, every query row holds ``alpha`` there and a biased
  token holds ``beta * sqrt(d) / alpha``, so q.k/sqrt(d) gains exactly
  ``beta`` (up to fp16 rounding of the stored K value);
* attention sinks: the first few tokens get a larger bias, mirroring the
  sink/recent attention-mass picture in the aistudio.id article ("Solusi 2").

Random streams: numpy PCG64 seeded by SeedSequence([base_seed, workload id,
sequence, layer, tensor id]) on the host; for device-resident workloads too
large for the host, torch's generator on the GPU seeded from the same tuple.
The two backends give different N(0,1) bulk values for the same tuple; the
structured parts (bias sets, outlier channels, scales) are always drawn on
the host, so they are identical either way.
"""
from __future__ import annotations

import dataclasses
import hashlib
from fractions import Fraction
from typing import Optional, Tuple

import numpy as np

BASE_SEED = 1234
HEAD_DIM = 128

# tensor ids inside a seed tuple
T_Q, T_K, T_V, T_BIAS, T_SCALES, T_QDEC, T_KNEW, T_VNEW = range(8)

BIAS_ALPHA = 4.0


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, value structure and bit budget."""

    name: str
    wid: int                      # workload id used in seed tuples
    n_seq: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    n_tokens: int
    avg_bits: str                 # average bits per unit, as a decimal string
    zone_c_capacity: int
    decode_steps: int
    head_dim: int = HEAD_DIM
    outlier_channels: int = 0     # number of K channels scaled by outlier_scale
    outlier_scale: float = 8.0
    bias_fraction: str = "0"      # fraction of tokens with logit bias +bias_beta
    bias_beta: float = 3.0
    n_sinks: int = 0              # first n_sinks tokens get logit bias +sink_beta
    sink_beta: float = 9.0
    lognormal_kscale: bool = False  # per (layer, head, channel) K scale ~ LogNormal(0,1)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_seg(self) -> int:
        return self.n_seq * self.n_layers * self.n_kv_heads

    @property
    def budget_v(self) -> int:
        """Bit budget of the V-token problem of one segment: floor(avg * N)."""
        return int(Fraction(self.avg_bits) * self.n_tokens)

    @property
    def budget_k(self) -> int:
        """Bit budget of the K-channel problem of one segment: floor(avg * d)."""
        return int(Fraction(self.avg_bits) * self.head_dim)

    @property
    def biased(self) -> bool:
        return Fraction(self.bias_fraction) > 0 or self.n_sinks > 0

    def dims(self, n_layers: Optional[int] = None) -> dict:
        return dict(n_seq=self.n_seq,
                    n_layers=self.n_layers if n_layers is None else n_layers,
                    n_q_heads=self.n_q_heads, n_kv_heads=self.n_kv_heads,
                    head_dim=self.head_dim, n_tokens=self.n_tokens)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    w.name: w for w in [
        # single layer, 1 KV head with 4 query heads, 1024 tokens, 4 outlier K
        # channels x8, 4 bits per unit on average, 128-row append zone.
        Workload("tiny-gqa4-n1k", 1, n_seq=1, n_layers=1, n_q_heads=4, n_kv_heads=1,
                 n_tokens=1024, avg_bits="4", zone_c_capacity=128, decode_steps=8,
                 outlier_channels=4),
        # one Llama-3.1-8B-shaped layer (32 q heads, 8 KV heads) at 32K tokens,
        # 10% heavy-hitter tokens at +3 logits, 2 bits per unit.
        Workload("llama8b-layer-n32k", 2, n_seq=1, n_layers=1, n_q_heads=32, n_kv_heads=8,
                 n_tokens=32768, avg_bits="2", zone_c_capacity=128, decode_steps=64,
                 bias_fraction="0.1"),
        # the full 32-layer 8B-shaped cache at 128K tokens, ~2.5% retention:
        # 0.64 bits per unit, heavy hitters plus 4 sink tokens.
        Workload("llama8b-32layer-n128k", 3, n_seq=1, n_layers=32, n_q_heads=32, n_kv_heads=8,
                 n_tokens=131072, avg_bits="0.64", zone_c_capacity=128, decode_steps=1,
                 bias_fraction="0.1", n_sinks=4),
        # 16 sequences of 32K tokens on one 8B-shaped layer, 3 bits per unit,
        # 256 decode steps appending to a 256-row zone.
        Workload("llama8b-batch16-n32k", 4, n_seq=16, n_layers=1, n_q_heads=32, n_kv_heads=8,
                 n_tokens=32768, avg_bits="3", zone_c_capacity=256, decode_steps=256,
                 bias_fraction="0.1"),
        # Qwen2.5-72B-shaped stack: 80 layers, 64 q heads / 8 KV heads, 256K
        # tokens, log-normal per-channel K scales, 2 bits per unit.
        Workload("qwen72b-80layer-n256k", 5, n_seq=1, n_layers=80, n_q_heads=64, n_kv_heads=8,
                 n_tokens=262144, avg_bits="2", zone_c_capacity=128, decode_steps=1,
                 lognormal_kscale=True),
    ]
}


def seed_tuple(w: Workload, seq: int, layer: int, tensor: int, step: int = 0) -> Tuple[int, ...]:
    return (BASE_SEED, w.wid, seq, layer, tensor, step)


def _rng(w: Workload, seq: int, layer: int, tensor: int, step: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        list(seed_tuple(w, seq, layer, tensor, step)))))


def _torch_seed(t: Tuple[int, ...]) -> int:
    return int.from_bytes(hashlib.sha256(repr(t).encode()).digest()[:8], "little") & ((1 << 63) - 1)


def _normal_f16(w: Workload, shape, seq, layer, tensor, step=0, device=None):
    """N(0,1) fp32 draws cast to fp16 (RNE). Host numpy, or torch on `device`."""
    if device is None:
        return _rng(w, seq, layer, tensor, step).standard_normal(shape, dtype=np.float32).astype(np.float16)
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(seed_tuple(w, seq, layer, tensor, step)))
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.float16)


def bias_per_token(w: Workload, seq: int, layer: int) -> np.ndarray:
    """Logit bias beta_t per prefill token (0 for unbiased tokens), float64."""
    beta = np.zeros(w.n_tokens)
    nb = int(Fraction(w.bias_fraction) * w.n_tokens)
    if nb:
        idx = _rng(w, seq, layer, T_BIAS).choice(w.n_tokens, size=nb, replace=False)
        beta[idx] = w.bias_beta
    beta[: w.n_sinks] = w.sink_beta
    return beta


def outlier_channels(w: Workload, seq: int, layer: int) -> np.ndarray:
    if not w.outlier_channels:
        return np.zeros(0, dtype=np.int64)
    lo = 1 if w.biased else 0
    return np.sort(_rng(w, seq, layer, T_SCALES).choice(
        np.arange(lo, w.head_dim), size=w.outlier_channels, replace=False))


def k_channel_scales(w: Workload, seq: int, layer: int) -> np.ndarray:
    """Per (KV head, channel) multiplicative K scale, float32 [Hkv][d]."""
    s = np.ones((w.n_kv_heads, w.head_dim), dtype=np.float32)
    if w.lognormal_kscale:
        s = _rng(w, seq, layer, T_SCALES).lognormal(0.0, 1.0, size=s.shape).astype(np.float32)
    oc = outlier_channels(w, seq, layer)
    if oc.size:
        s[:, oc] *= np.float32(w.outlier_scale)
    return s


def _apply_k_structure(w, K, seq, layer, scales, beta, device):
    """K [Hkv][N][d]: per-channel scales, then the reserved bias channel."""
    if device is None:
        if not np.all(scales == 1):
            K = (K.astype(np.float32) * scales[:, None, :]).astype(np.float16)
        if w.biased:
            K[..., 0] = np.float16(0)
            kb = (beta * np.sqrt(w.head_dim) / BIAS_ALPHA).astype(np.float16)
            K[..., 0] = kb[None, :]
        return K
    import torch
    if not np.all(scales == 1):
        K = (K.float() * torch.from_numpy(scales).to(device)[:, None, :]).half()
    if w.biased:
        kb = torch.from_numpy((beta * np.sqrt(w.head_dim) / BIAS_ALPHA).astype(np.float16)).to(device)
        K[..., 0] = kb[None, :]
    return K


def prefill_layer(w: Workload, seq: int, layer: int, device=None, kv_only: bool = False):
    """Q [Hq][N][d], K [Hkv][N][d], V [Hkv][N][d] fp16 for one (sequence, layer).
    With kv_only, Q is not drawn (returned as None); K and V are unchanged."""
    H, Hk, N, d = w.n_q_heads, w.n_kv_heads, w.n_tokens, w.head_dim
    Q = None if kv_only else _normal_f16(w, (H, N, d), seq, layer, T_Q, device=device)
    K = _normal_f16(w, (Hk, N, d), seq, layer, T_K, device=device)
    V = _normal_f16(w, (Hk, N, d), seq, layer, T_V, device=device)
    if w.biased and Q is not None:
        Q[..., 0] = BIAS_ALPHA
    K = _apply_k_structure(w, K, seq, layer, k_channel_scales(w, seq, layer),
                           bias_per_token(w, seq, layer), device)
    return Q, K, V


def decode_inputs(w: Workload, step: int, device=None):
    """q [S][L][Hq][d], k_new and v_new [S][L][Hkv][d] fp16 for one decode step.

    New tokens carry no logit bias (K channel 0 is 0 when the workload is
    biased) but do carry the per-channel K scales of their layer.
    """
    S, L, H, Hk, d = w.n_seq, w.n_layers, w.n_q_heads, w.n_kv_heads, w.head_dim
    q = _normal_f16(w, (S, L, H, d), 0, 0, T_QDEC, step, device=device)
    kn = _normal_f16(w, (S, L, Hk, d), 0, 0, T_KNEW, step, device=device)
    vn = _normal_f16(w, (S, L, Hk, d), 0, 0, T_VNEW, step, device=device)
    if w.biased:
        q[..., 0] = BIAS_ALPHA
        kn[..., 0] = 0
    for s in range(S):
        for l in range(L):
            sc = k_channel_scales(w, s, l)
            if np.all(sc == 1):
                continue
            if device is None:
                kn[s, l] = (kn[s, l].astype(np.float32) * sc).astype(np.float16)
            else:
                import torch
                kn[s, l] = (kn[s, l].float() * torch.from_numpy(sc).to(device)).half()
    return q, kn, vn


def random_unit_inputs(n_seg: int, n_tokens: int, seed: int, head_dim: int = HEAD_DIM):
    """Seeded fp32 token weights, token variances and channel weights.

    Shapes [n_seg][N], [n_seg][N], [n_seg][d].  Token weights are log-normal
    with a heavy tail (a few tokens far above the rest), variances are
    chi-square-like around 1, channel weights log-normal.  Used to drive the
    allocator on identical inputs from both sides.
    """
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, 99, seed])))
    w_tok = np.exp(r.standard_normal((n_seg, n_tokens)) * 1.5).astype(np.float32)
    hh = r.random((n_seg, n_tokens)) < 0.02
    w_tok[hh] *= np.float32(50.0)
    var_tok = (r.chisquare(head_dim, (n_seg, n_tokens)) / head_dim).astype(np.float32)
    w_chan = np.exp(r.standard_normal((n_seg, head_dim))).astype(np.float32)
    return w_tok, var_tok, w_chan


def random_bits(n_seg: int, n_tokens: int, seed: int, head_dim: int = HEAD_DIM,
                tok_p=(0.5, 0.2, 0.15, 0.1, 0.05), chan_p=(0.3, 0.2, 0.2, 0.2, 0.1)):
    """Seeded per-token and per-channel bitwidths in {0,2,4,8,16} (uint8)."""
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, 98, seed])))
    choices = np.array([0, 2, 4, 8, 16], dtype=np.uint8)
    bt = choices[r.choice(5, size=(n_seg, n_tokens), p=np.asarray(tok_p) / np.sum(tok_p))]
    bc = choices[r.choice(5, size=(n_seg, head_dim), p=np.asarray(chan_p) / np.sum(chan_p))]
    return bt, bc


def random_kv(n_seg: int, n_tokens: int, seed: int, head_dim: int = HEAD_DIM, scale=1.0):
    """Seeded fp16 K and V of shape [n_seg][N][d] (N(0,1) * scale)."""
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, 97, seed])))
    K = (r.standard_normal((n_seg, n_tokens, head_dim), dtype=np.float32) * scale).astype(np.float16)
    V = (r.standard_normal((n_seg, n_tokens, head_dim), dtype=np.float32) * scale).astype(np.float16)
    return K, V
