// Fused split-K decode attention over the packed cache (RDKV summary, section
// 2.3: dequantization fused into the logit and output products over zones A,
// B and C; section 1: decode is bandwidth-bound, it rereads the cache every
// step).
//
// decode_chunk_kernel: one 256-thread workgroup per (segment, chunk).  A chunk
// is up to 1024 tokens of the 2-bit V group (512 of the 4-bit, 256 of the
// 8-bit, 128 of the fp16 group) or up to 256 zone-C rows.  Each wave walks
// 64-token tiles of the chunk.  Per tile, every load the tile needs is issued
// first (the token's K record words into registers, the lane's parts of the
// V rows), then:
//   * logits, lane = token: q.k_hat for the G query heads of the KV head with
//     each bit-segment's scale and zero factored out,
//     q.(s*code + z) = s*(q.code) + z*sum(q); 0-bit channels are absent;
//   * online softmax over the wave (DPP max), p*scale per token to LDS;
//   * values, lane = (16-channel block, token pair): accumulates
//     (p*s)*code per head for two tokens at a time; the p*z part is summed
//     once per token.
// The 4 waves' partials are merged in LDS into one (m, l, o[128]) per query
// head and chunk.  decode_merge_kernel then combines each segment's chunks in
// chunk order, so the result does not depend on scheduling.  Merging in a
// second launch keeps the chunk kernel free of device-wide fences, which on a
// multi-XCD part write back and invalidate the L2 and cost more than the
// merge itself.
// No MFMA: 1..8 query rows per KV head make this a matrix-vector stream,
// bounded by HBM bandwidth and VALU issue.
#include "rdkv_internal.h"

namespace rdkv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr float kLog2eOverSqrtD = 1.4426950408889634f / 11.313708498984761f;

// ---------------------------------------------------------------- wave reductions (DPP)

template <bool kMax>
__device__ inline float wave_reduce(float v) {
  const int id = __float_as_int(kMax ? -INFINITY : 0.0f);
  int x = __float_as_int(v);
  auto op = [](int a, int b) {
    const float fa = __int_as_float(a), fb = __int_as_float(b);
    return __float_as_int(kMax ? fmaxf(fa, fb) : fa + fb);
  };
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x111, 0xf, 0xf, false));   // row_shr:1
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x112, 0xf, 0xf, false));   // row_shr:2
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x114, 0xf, 0xf, false));   // row_shr:4
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x118, 0xf, 0xf, false));   // row_shr:8
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x142, 0xa, 0xf, false));   // row_bcast:15
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x143, 0xc, 0xf, false));   // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(x, 63));
}

// ---------------------------------------------------------------- segment and chunk

struct SegInfo {
  int n_tok[4];
  int n_chan[4];
  int rec_a;        // words of a zone-A record
  uint64_t off_v[4], off_krec, off_kc, off_vc;
  bool zc_ok;
};

// Reads a descriptor and treats anything inconsistent with the layout as an
// empty segment, so a damaged blob can never drive reads out of bounds.
__device__ inline SegInfo load_segment(const DecodeParams& p, int64_t seg) {
  const uint8_t* d = p.cache + kHeaderBytes + uint64_t(seg) * kDescBytes;
  SegInfo s;
  int n_kept_sum = 0, n_chan_sum = 0;
  bool ok = true;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s.n_tok[i] = *reinterpret_cast<const int32_t*>(d + kDescNTok + 4 * i);
    s.n_chan[i] = *reinterpret_cast<const int32_t*>(d + kDescNChan + 4 * i);
    s.off_v[i] = *reinterpret_cast<const uint64_t*>(d + kDescOffV + 8 * i);
    ok = ok && s.n_tok[i] >= 0 && s.n_chan[i] >= 0;
    n_kept_sum += s.n_tok[i];
    n_chan_sum += s.n_chan[i];
  }
  const int n_kept = *reinterpret_cast<const int32_t*>(d + kDescNKept);
  const int rec = *reinterpret_cast<const int32_t*>(d + kDescRec);
  s.off_krec = *reinterpret_cast<const uint64_t*>(d + kDescOffKrec);
  s.off_kc = *reinterpret_cast<const uint64_t*>(d + kDescOffKc);
  s.off_vc = *reinterpret_cast<const uint64_t*>(d + kDescOffVc);
  const RecordShape rs = record_shape(s.n_chan[0], s.n_chan[1], s.n_chan[2], s.n_chan[3]);
  ok = ok && n_kept == n_kept_sum && n_kept <= p.nk_max && n_chan_sum <= kHeadDim && rec == 4 * rs.words_a() &&
       rec <= p.rec_max;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    ok = ok && s.off_v[i] + uint64_t(s.n_tok[i]) * (kHeadDim * group_bits(i) / 8) <= p.cache_bytes;
  ok = ok && s.off_krec + uint64_t(n_kept) * rec <= p.cache_bytes;
  if (!ok) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s.n_tok[i] = s.n_chan[i] = 0;
  }
  s.rec_a = ok ? rec / 4 : 1;
  s.zc_ok = s.off_vc + uint64_t(p.n_c) * kHeadDim * 2 <= p.cache_bytes &&
            s.off_kc + uint64_t(p.n_c) * kHeadDim * 2 <= p.cache_bytes;
  return s;
}

struct Plan {
  int kind;          // 0..3 token group, 4 zone C, -1 none
  int start, end;    // rows of the group (or zone C) in this chunk
  uint64_t vbase;    // blob offset of the group's first V row (or of V_C)
  int64_t rec0;      // word offset of the group's first K record from off_krec
  int rec_words;     // words per record in this group
};

__device__ inline Plan plan_chunk(const SegInfo& si, int n_c, int k) {
  Plan pl{-1, 0, 0, 0, 0, 0};
  int kept = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int T = chunk_tokens(g);
    const int nch = (si.n_tok[g] + T - 1) / T;
    if (pl.kind < 0) {
      if (k < nch) {
        pl.kind = g;
        pl.start = k * T;
        pl.end = min(si.n_tok[g], (k + 1) * T);
        pl.vbase = si.off_v[g];
        // zone-A records come first; the fp16 group's shorter records follow them
        pl.rec0 = int64_t(kept) * si.rec_a;
        pl.rec_words = g < 3 ? si.rec_a : si.rec_a - 1;
      } else {
        k -= nch;
      }
    }
    kept += si.n_tok[g];
  }
  if (pl.kind < 0) {
    const int nch = (n_c + kChunkRowsC - 1) / kChunkRowsC;
    if (k < nch) {
      pl.kind = 4;
      pl.start = k * kChunkRowsC;
      pl.end = min(n_c, (k + 1) * kChunkRowsC);
      pl.vbase = si.off_vc;
    }
  }
  return pl;
}

__device__ inline int n_chunks_of(const SegInfo& si, int n_c) { return chunk_count(si.n_tok, n_c); }

// ---------------------------------------------------------------- shared memory

template <int G>
struct Smem {
  float q[kHeadDim + 32][G];   // query in record channel order, zero padded
  float qsum[3][G];            // sum of q over the 8-, 4-, 2-bit channel parts
  float coef[kWaves][64][G];   // p * scale per token of the current tile
  float part_o[kWaves][G][kHeadDim];
  float part_ml[kWaves][G][2];
};

// ---------------------------------------------------------------- value rows

// A lane's part of one V row: 16 channels (cb*16 .. +16) at b bits.
template <int B> struct VPart;
template <> struct VPart<2> { uint32_t w; };
template <> struct VPart<4> { uint2 w; };
template <> struct VPart<8> { uint4 w; };
template <> struct VPart<16> { uint4 a, b; };

template <int B>
__device__ inline VPart<B> load_vpart(const uint8_t* row, int cb) {
  VPart<B> v;
  if constexpr (B == 2) v.w = reinterpret_cast<const uint32_t*>(row)[cb];
  if constexpr (B == 4) v.w = reinterpret_cast<const uint2*>(row)[cb];
  if constexpr (B == 8) v.w = reinterpret_cast<const uint4*>(row)[cb];
  if constexpr (B == 16) {
    v.a = reinterpret_cast<const uint4*>(row)[2 * cb];
    v.b = reinterpret_cast<const uint4*>(row)[2 * cb + 1];
  }
  return v;
}

// The 16 values of a part: codes as floats, or fp16 values.
template <int B>
__device__ inline void unpack_vpart(const VPart<B>& v, float (&x)[16]) {
  if constexpr (B == 2) {
#pragma unroll
    for (int e = 0; e < 16; ++e) x[e] = float((v.w >> (2 * e)) & 3u);
  } else if constexpr (B == 4) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = float((v.w.x >> (4 * e)) & 15u);
      x[8 + e] = float((v.w.y >> (4 * e)) & 15u);
    }
  } else if constexpr (B == 8) {
    const uint32_t ws[4] = {v.w.x, v.w.y, v.w.z, v.w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * j + e] = float((ws[j] >> (8 * e)) & 255u);
  } else {
    const uint32_t ws[8] = {v.a.x, v.a.y, v.a.z, v.a.w, v.b.x, v.b.y, v.b.z, v.b.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x[2 * j] = half_lo(ws[j]);
      x[2 * j + 1] = half_hi(ws[j]);
    }
  }
}

// ---------------------------------------------------------------- logits from a K record

// s[g] = q_g . k_hat for one token whose record words are in kw[0..nw).
template <int G, int KW>
__device__ inline void record_logits(const uint32_t (&kw)[KW], int nw, const RecordShape& rs, int c8, int c4, int c2,
                                     bool has_vmeta, const Smem<G>& sm, float (&s)[G], float& vs, float& vz) {
  const int e16 = rs.w16, e8 = e16 + rs.w8, e4 = e8 + rs.w4, e2 = e4 + rs.w2;
  int mi = e2;
  const int m8 = c4 > c8 ? mi++ : -1;
  const int m4 = c2 > c4 ? mi++ : -1;
  const int m2 = rs.w2 > 0 ? mi++ : -1;
  const int vm = has_vmeta ? mi : -1;
  float d8[G], d4[G], d2[G];
  uint32_t w8m = 0, w4m = 0, w2m = 0, wvm = 0;
#pragma unroll
  for (int g = 0; g < G; ++g) s[g] = d8[g] = d4[g] = d2[g] = 0.f;
#pragma unroll
  for (int w = 0; w < KW; ++w) {
    if (w >= nw) break;
    const uint32_t x = kw[w];
    if (w < e16) {
      const float k0 = half_lo(x), k1 = half_hi(x);
#pragma unroll
      for (int g = 0; g < G; ++g) s[g] = fmaf(sm.q[2 * w + 1][g], k1, fmaf(sm.q[2 * w][g], k0, s[g]));
    } else if (w < e8) {
      const int c = c8 + 4 * (w - e16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float code = float((x >> (8 * e)) & 255u);
#pragma unroll
        for (int g = 0; g < G; ++g) d8[g] = fmaf(sm.q[c + e][g], code, d8[g]);
      }
    } else if (w < e4) {
      const int c = c4 + 8 * (w - e8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float code = float((x >> (4 * e)) & 15u);
#pragma unroll
        for (int g = 0; g < G; ++g) d4[g] = fmaf(sm.q[c + e][g], code, d4[g]);
      }
    } else if (w < e2) {
      const int c = c2 + 16 * (w - e4);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float code = float((x >> (2 * e)) & 3u);
#pragma unroll
        for (int g = 0; g < G; ++g) d2[g] = fmaf(sm.q[c + e][g], code, d2[g]);
      }
    } else {
      if (w == m8) w8m = x;
      if (w == m4) w4m = x;
      if (w == m2) w2m = x;
      if (w == vm) wvm = x;
    }
  }
  if (m8 >= 0) {
    const float sc = half_lo(w8m), z = half_hi(w8m);
#pragma unroll
    for (int g = 0; g < G; ++g) s[g] = fmaf(sc, d8[g], fmaf(z, sm.qsum[0][g], s[g]));
  }
  if (m4 >= 0) {
    const float sc = half_lo(w4m), z = half_hi(w4m);
#pragma unroll
    for (int g = 0; g < G; ++g) s[g] = fmaf(sc, d4[g], fmaf(z, sm.qsum[1][g], s[g]));
  }
  if (m2 >= 0) {
    const float sc = half_lo(w2m), z = half_hi(w2m);
#pragma unroll
    for (int g = 0; g < G; ++g) s[g] = fmaf(sc, d2[g], fmaf(z, sm.qsum[2][g], s[g]));
  }
  vs = 1.f;
  vz = 0.f;
  if (has_vmeta) {
    vs = half_lo(wvm);
    vz = half_hi(wvm);
  }
}

// ---------------------------------------------------------------- per-wave state

template <int G>
struct WaveState {
  float m[G], l[G], z[G], acc[G][16];
};

template <int G>
__device__ inline void state_init(WaveState<G>& st) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    st.m[g] = -INFINITY;
    st.l[g] = 0.f;
    st.z[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) st.acc[g][e] = 0.f;
  }
}

// Online softmax update for one tile; writes p*vs per token to LDS.
template <int G>
__device__ inline void softmax_tile(WaveState<G>& st, const float (&s)[G], bool valid, float vs, float vz,
                                    Smem<G>& sm, int wave, int lane) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float t = valid ? s[g] * kLog2eOverSqrtD : -INFINITY;
    const float mnew = fmaxf(st.m[g], wave_reduce<true>(t));
    const float alpha = exp2f(st.m[g] - mnew);
    const float pr = exp2f(t - mnew);
    st.m[g] = mnew;
    st.l[g] = fmaf(st.l[g], alpha, pr);
    st.z[g] = fmaf(st.z[g], alpha, pr * vz);
#pragma unroll
    for (int e = 0; e < 16; ++e) st.acc[g][e] *= alpha;
    sm.coef[wave][lane][g] = pr * vs;
  }
}

__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// acc[g][e] += c0[g] * x0[e] + c1[g] * x1[e]
template <int G, int B>
__device__ inline void accumulate_pair(WaveState<G>& st, const Smem<G>& sm, int wave, int j0, const VPart<B>& v0,
                                       const VPart<B>& v1) {
  float c0[G], c1[G], x0[16], x1[16];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    c0[g] = sm.coef[wave][j0][g];
    c1[g] = sm.coef[wave][j0 + 1][g];
  }
  unpack_vpart<B>(v0, x0);
  unpack_vpart<B>(v1, x1);
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 16; ++e) st.acc[g][e] = fmaf(c1[g], x1[e], fmaf(c0[g], x0[e], st.acc[g][e]));
}

// Wave partial (m, l, o) into LDS.
template <int G>
__device__ inline void wave_finish(WaveState<G>& st, Smem<G>& sm, int wave, int lane) {
  const int cb = lane & 7, ts = lane >> 3;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    st.l[g] = wave_reduce<false>(st.l[g]);
    st.z[g] = wave_reduce<false>(st.z[g]);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float v = st.acc[g][e];
      v += __shfl_xor(v, 8, 64);
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      st.acc[g][e] = v;
    }
  }
  if (ts == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 16; ++e) sm.part_o[wave][g][cb * 16 + e] = st.acc[g][e] + st.z[g];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      sm.part_ml[wave][g][0] = st.m[g];
      sm.part_ml[wave][g][1] = st.l[g];
    }
  }
}

// ---------------------------------------------------------------- token groups (zones A and B)

template <int G, int B, int KW>
__device__ void run_group(const DecodeParams& p, const SegInfo& si, const Plan& pl, Smem<G>& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cb = lane & 7, ts = lane >> 3;
  const RecordShape rs = record_shape(si.n_chan[0], si.n_chan[1], si.n_chan[2], si.n_chan[3]);
  const int c8 = si.n_chan[0], c4 = c8 + si.n_chan[1], c2 = c4 + si.n_chan[2];
  const int nw = pl.rec_words;
  const uint32_t* rbase = reinterpret_cast<const uint32_t*>(p.cache + si.off_krec) + pl.rec0;
  const uint8_t* vbase = p.cache + pl.vbase;
  constexpr int kRowBytes = kHeadDim * B / 8;
  constexpr int kPrefetch = B == 16 ? 2 : 4;   // token pairs whose V parts are loaded ahead
  const int last = pl.end - 1;

  WaveState<G> st;
  state_init(st);
  for (int base = pl.start + 64 * wave; base < pl.end; base += kThreads) {
    // ---- loads for the whole tile
    const int r = min(base + lane, last);
    const uint32_t* rp = rbase + int64_t(r) * nw;
    uint32_t kw[KW];
#pragma unroll
    for (int w = 0; w < KW; ++w) kw[w] = w < nw ? rp[w] : 0u;
    VPart<B> vp[kPrefetch][2];
#pragma unroll
    for (int rr = 0; rr < kPrefetch; ++rr)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        vp[rr][h] = load_vpart<B>(vbase + int64_t(min(base + 16 * rr + 2 * ts + h, last)) * kRowBytes, cb);

    // ---- logits and softmax, lane = token
    float s[G], vs, vz;
    record_logits<G, KW>(kw, nw, rs, c8, c4, c2, B < 16, sm, s, vs, vz);
    softmax_tile<G>(st, s, base + lane < pl.end, vs, vz, sm, wave, lane);
    wave_lds_sync();

    // ---- values, lane = (channel block, token pair)
#pragma unroll
    for (int rr = 0; rr < kPrefetch; ++rr) accumulate_pair<G, B>(st, sm, wave, 16 * rr + 2 * ts, vp[rr][0], vp[rr][1]);
    if constexpr (kPrefetch < 4) {
#pragma unroll
      for (int rr = kPrefetch; rr < 4; ++rr) {
        VPart<B> a = load_vpart<B>(vbase + int64_t(min(base + 16 * rr + 2 * ts, last)) * kRowBytes, cb);
        VPart<B> b = load_vpart<B>(vbase + int64_t(min(base + 16 * rr + 2 * ts + 1, last)) * kRowBytes, cb);
        accumulate_pair<G, B>(st, sm, wave, 16 * rr + 2 * ts, a, b);
      }
    }
    wave_lds_sync();
  }
  wave_finish<G>(st, sm, wave, lane);
}

// ---------------------------------------------------------------- zone C (fp16 rows, natural order)

template <int G>
__device__ void run_zone_c(const DecodeParams& p, const SegInfo& si, int64_t seg, const Plan& pl, Smem<G>& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cb = lane & 7, ts = lane >> 3;
  const int last = pl.end - 1;
  const uint8_t* kc = p.cache + si.off_kc;
  const uint8_t* vc = p.cache + si.off_vc;
  const uint8_t* knew = reinterpret_cast<const uint8_t*>(p.k_new + seg * kHeadDim);
  const uint8_t* vnew = reinterpret_cast<const uint8_t*>(p.v_new + seg * kHeadDim);
  auto krow = [&](int r) { return (p.append && r == p.c_len) ? knew : kc + int64_t(r) * kHeadDim * 2; };
  auto vrow = [&](int r) { return (p.append && r == p.c_len) ? vnew : vc + int64_t(r) * kHeadDim * 2; };

  WaveState<G> st;
  state_init(st);
  for (int base = pl.start + 64 * wave; base < pl.end; base += kThreads) {
    const int r = min(base + lane, last);
    const uint4* k4 = reinterpret_cast<const uint4*>(krow(r));
    float s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) s[g] = 0.f;
#pragma unroll 2
    for (int c = 0; c < 16; ++c) {
      const uint4 x = k4[c];
      const uint32_t ws[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ch = 8 * c + 2 * j;
        const float k0 = half_lo(ws[j]), k1 = half_hi(ws[j]);
#pragma unroll
        for (int g = 0; g < G; ++g) s[g] = fmaf(sm.q[ch + 1][g], k1, fmaf(sm.q[ch][g], k0, s[g]));
      }
    }
    softmax_tile<G>(st, s, base + lane < pl.end, 1.f, 0.f, sm, wave, lane);
    wave_lds_sync();
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int j0 = 16 * rr + 2 * ts;
      VPart<16> a = load_vpart<16>(vrow(min(base + j0, last)), cb);
      VPart<16> b = load_vpart<16>(vrow(min(base + j0 + 1, last)), cb);
      accumulate_pair<G, 16>(st, sm, wave, j0, a, b);
    }
    wave_lds_sync();
  }
  wave_finish<G>(st, sm, wave, lane);
}

// ---------------------------------------------------------------- kernel

// out[seg][g][c] = sum_k e^{m_k - M} o_k[c] / sum_k e^{m_k - M} l_k over the
// segment's chunks, in chunk order; a segment with nothing to attend to gives 0.
template <int G>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(DecodeParams p) {
  const int64_t seg = blockIdx.x;
  const SegInfo si = load_segment(p, seg);
  const int n = min(n_chunks_of(si, si.zc_ok ? p.n_c : 0), p.max_chunks);
  const float* part = p.partials + int64_t(seg) * p.max_chunks * G * kPartialFloats;
  for (int i = threadIdx.x; i < G * kHeadDim; i += kThreads) {
    const int g = i / kHeadDim, c = i % kHeadDim;
    float M = -INFINITY;
    for (int k = 0; k < n; ++k) M = fmaxf(M, part[(k * G + g) * kPartialFloats]);
    float L = 0.f, O = 0.f;
#pragma unroll 4
    for (int k = 0; k < n; ++k) {
      const float* pk = part + (k * G + g) * kPartialFloats;
      const float f = exp2f(pk[0] - M);
      L = fmaf(pk[1], f, L);
      O = fmaf(pk[4 + c], f, O);
    }
    p.out[(seg * G + g) * kHeadDim + c] = L > 0.f ? O / L : 0.f;
  }
}

template <int G, int KW>
__global__ __launch_bounds__(kThreads) void decode_chunk_kernel(DecodeParams p) {
  __shared__ Smem<G> sm;
  const int64_t seg = blockIdx.x / p.max_chunks;
  const int k = int(blockIdx.x % p.max_chunks);
  const SegInfo si = load_segment(p, seg);
  const int n_c = si.zc_ok ? p.n_c : 0;
  const Plan pl = plan_chunk(si, n_c, k);
  const int tid = threadIdx.x;
  if (pl.kind < 0) return;

  // query of the G heads, in the channel order the rows use
  const uint8_t* perm = p.cache + kHeaderBytes + uint64_t(seg) * kDescBytes + kDescPerm;
  const int c_stored = si.n_chan[0] + si.n_chan[1] + si.n_chan[2] + si.n_chan[3];
  for (int i = tid; i < (kHeadDim + 32) * G; i += kThreads) {
    const int pos = i / G, g = i % G;
    float v = 0.f;
    if (pl.kind == 4) {
      if (pos < kHeadDim) v = __half2float(p.q[(seg * G + g) * kHeadDim + pos]);
    } else if (pos < c_stored) {
      v = __half2float(p.q[(seg * G + g) * kHeadDim + perm[pos]]);
    }
    sm.q[pos][g] = v;
  }
  __syncthreads();
  if (tid < 3 * G) {
    const int j = tid / G, g = tid % G;
    const int lo = si.n_chan[0] + (j > 0 ? si.n_chan[1] : 0) + (j > 1 ? si.n_chan[2] : 0);
    const int hi = lo + (j == 0 ? si.n_chan[1] : j == 1 ? si.n_chan[2] : si.n_chan[3]);
    float acc = 0.f;
    for (int c = lo; c < hi; ++c) acc += sm.q[c][g];
    sm.qsum[j][g] = acc;
  }
  // append the new token to zone C (only the chunk holding row c_len does it)
  if (pl.kind == 4 && p.append && p.c_len >= pl.start && p.c_len < pl.end) {
    uint32_t* kc = reinterpret_cast<uint32_t*>(p.cache + si.off_kc) + int64_t(p.c_len) * (kHeadDim / 2);
    uint32_t* vc = reinterpret_cast<uint32_t*>(p.cache + si.off_vc) + int64_t(p.c_len) * (kHeadDim / 2);
    if (tid < 64) kc[tid] = reinterpret_cast<const uint32_t*>(p.k_new + seg * kHeadDim)[tid];
    else if (tid < 128) vc[tid - 64] = reinterpret_cast<const uint32_t*>(p.v_new + seg * kHeadDim)[tid - 64];
  }
  __syncthreads();

  switch (pl.kind) {
    case 0: run_group<G, 2, KW>(p, si, pl, sm); break;
    case 1: run_group<G, 4, KW>(p, si, pl, sm); break;
    case 2: run_group<G, 8, KW>(p, si, pl, sm); break;
    case 3: run_group<G, 16, KW>(p, si, pl, sm); break;
    default: run_zone_c<G>(p, si, seg, pl, sm); break;
  }
  __syncthreads();

  // merge the waves' partials into the chunk's partial
  float* out = p.partials + (int64_t(seg) * p.max_chunks + k) * G * kPartialFloats;
  for (int i = tid; i < G * kHeadDim; i += kThreads) {
    const int g = i / kHeadDim, c = i % kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.part_ml[w][g][0]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = exp2f(sm.part_ml[w][g][0] - M);
      L = fmaf(sm.part_ml[w][g][1], f, L);
      O = fmaf(sm.part_o[w][g][c], f, O);
    }
    out[g * kPartialFloats + 4 + c] = O;
    if (c == 0) {
      out[g * kPartialFloats + 0] = M;
      out[g * kPartialFloats + 1] = L;
    }
  }
}

template <int G, int KW>
hipError_t launch_chunks_gk(const DecodeParams& p, hipStream_t stream) {
  const uint64_t grid = uint64_t(p.n_seg) * p.max_chunks;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((decode_chunk_kernel<G, KW>), dim3(unsigned(grid)), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int G>
hipError_t launch_chunks_g(const DecodeParams& p, hipStream_t stream) {
  // record words held in registers: the layout's bound on a record
  const int words = (p.rec_max + 3) / 4;
  if (words <= 8) return launch_chunks_gk<G, 8>(p, stream);
  if (words <= 16) return launch_chunks_gk<G, 16>(p, stream);
  if (words <= 32) return launch_chunks_gk<G, 32>(p, stream);
  return launch_chunks_gk<G, 72>(p, stream);
}

template <int G>
hipError_t launch_merge_g(const DecodeParams& p, hipStream_t stream) {
  if (p.n_seg == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_merge_kernel<G>, dim3(unsigned(p.n_seg)), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_chunks(const DecodeParams& p, hipStream_t stream) {
  switch (p.group) {
    case 1: return launch_chunks_g<1>(p, stream);
    case 2: return launch_chunks_g<2>(p, stream);
    case 4: return launch_chunks_g<4>(p, stream);
    case 8: return launch_chunks_g<8>(p, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_merge(const DecodeParams& p, hipStream_t stream) {
  switch (p.group) {
    case 1: return launch_merge_g<1>(p, stream);
    case 2: return launch_merge_g<2>(p, stream);
    case 4: return launch_merge_g<4>(p, stream);
    case 8: return launch_merge_g<8>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace rdkv
