// Fused split-K decode attention over the packed cache (RDKV summary, section
// 2.3: dequantization fused into the logit and output products over zones A,
// B and C; section 1: decode is bandwidth-bound, it rereads the cache every
// step).
//
// decode_chunk_kernel: one 256-thread workgroup per (segment, chunk).  A chunk
// is up to 1024 tokens of the 2-bit V group (512 of the 4-bit, 256 of the
// 8-bit, 128 of the fp16 group) or up to 256 zone-C rows.  Each wave walks
// 64-token steps of the chunk:
//   * logits, lane = token: the lane reads its token's K record (fp16 values,
//     then 8/4/2-bit codes of the permuted channels, then the scale/zero words)
//     and forms q.k_hat for the G query heads of the KV head, with the scale
//     and zero factored out of each bit-segment:  q.(s*code + z) =
//     s*(q.code) + z*sum(q);  0-bit channels are simply absent;
//   * online softmax across the wave (max and sum by lane shuffles);
//   * values, lane = (16-channel block, token slot): the lane reads 2b bytes
//     of a V row and accumulates p*(s*code + z) = (p*s)*code + p*z per head,
//     the p*z part summed once per token.
// The 4 waves' partials are merged in LDS and one (m, l, o[128]) per query
// head is written for the chunk; the last workgroup of a segment to finish
// (a counter in the segment's descriptor) combines the segment's chunks, so a
// decode step is a single launch.  No MFMA: a product with 1..8 query rows per KV head is a
// matrix-vector stream, bounded by HBM bandwidth and VALU issue.
#include "rdkv_internal.h"

namespace rdkv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr float kLog2eOverSqrtD = 1.4426950408889634f / 11.313708498984761f;

struct SegInfo {
  int n_tok[4];
  int n_chan[4];
  int rec_a;        // words of a zone-A record
  int gbase[4];     // kept index of each group's first token
  uint64_t off_v[4], off_krec, off_kc, off_vc;
};

// Reads a descriptor and treats anything inconsistent with the layout as an
// empty segment, so a damaged blob can never drive reads out of bounds.
__device__ inline SegInfo load_segment(const DecodeParams& p, int64_t seg) {
  const uint8_t* d = p.cache + kHeaderBytes + uint64_t(seg) * kDescBytes;
  SegInfo s;
  int n_kept_sum = 0, n_chan_sum = 0;
  bool ok = true;
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
  for (int i = 0; i < 4 && ok; ++i)
    ok = s.off_v[i] + uint64_t(s.n_tok[i]) * (kHeadDim * group_bits(i) / 8) <= p.cache_bytes;
  ok = ok && s.off_krec + uint64_t(n_kept) * rec <= p.cache_bytes;
  if (!ok)
    for (int i = 0; i < 4; ++i) s.n_tok[i] = s.n_chan[i] = 0;
  s.rec_a = ok ? rec / 4 : 1;
  s.gbase[0] = 0;
  for (int i = 1; i < 4; ++i) s.gbase[i] = s.gbase[i - 1] + s.n_tok[i - 1];
  // zone C must lie inside the blob too
  if (s.off_vc + uint64_t(p.n_c) * kHeadDim * 2 > p.cache_bytes || s.off_kc + uint64_t(p.n_c) * kHeadDim * 2 > p.cache_bytes)
    s.off_kc = s.off_vc = ~uint64_t(0);
  return s;
}

__device__ inline int zone_c_rows(const DecodeParams& p, const SegInfo& s) {
  return s.off_kc == ~uint64_t(0) ? 0 : p.n_c;
}

// Accumulates coef[g] * x[e] into acc[g][e] for the lane's 16 values.
template <int G>
__device__ inline void accumulate16(float (&acc)[G][16], const float (&coef)[G], const float (&x)[16]) {
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[g][e] = fmaf(coef[g], x[e], acc[g][e]);
}

// The lane's 16 values of a row: codes as floats (b < 16) or fp16 values.
template <int B>
__device__ inline void load_row16(const uint8_t* row, int cb, float (&x)[16]) {
  if constexpr (B == 2) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(row)[cb];
#pragma unroll
    for (int e = 0; e < 16; ++e) x[e] = float((w >> (2 * e)) & 3u);
  } else if constexpr (B == 4) {
    const uint2 w = reinterpret_cast<const uint2*>(row)[cb];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = float((w.x >> (4 * e)) & 15u);
      x[8 + e] = float((w.y >> (4 * e)) & 15u);
    }
  } else if constexpr (B == 8) {
    const uint4 w = reinterpret_cast<const uint4*>(row)[cb];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * j + e] = float((ws[j] >> (8 * e)) & 255u);
  } else {
    const uint4* r4 = reinterpret_cast<const uint4*>(row) + 2 * cb;
    const uint4 a = r4[0], b = r4[1];
    const uint32_t ws[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x[2 * j] = half_lo(ws[j]);
      x[2 * j + 1] = half_hi(ws[j]);
    }
  }
}

template <int G>
struct Smem {
  float q[kHeadDim + 16][G];   // query in record channel order, zero padded
  float qsum[3][G];            // sum of q over the 8-, 4-, 2-bit channel parts
  float coef[kWaves][64][G];   // p * scale per token of the current step
  float part_o[kWaves][G][kHeadDim];
  float part_ml[kWaves][G][2];
};

template <int G, int B>
__device__ void run_rows(const DecodeParams& p, const SegInfo& si, int64_t seg, const Chunk& ch, Smem<G>& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cb = lane & 7, ts = lane >> 3;
  const bool zone_c = ch.kind == 4;
  const RecordShape rs = record_shape(si.n_chan[0], si.n_chan[1], si.n_chan[2], si.n_chan[3]);
  const int c8 = si.n_chan[0], c4 = c8 + si.n_chan[1], c2 = c4 + si.n_chan[2];
  const int n_a = si.gbase[3];
  const uint32_t* krec = reinterpret_cast<const uint32_t*>(p.cache + si.off_krec);
  const uint8_t* vbase = zone_c ? p.cache + si.off_vc : p.cache + si.off_v[ch.kind];
  constexpr int kRowBytes = kHeadDim * B / 8;

  float m_run[G], l_run[G], zacc[G], acc[G][16];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
    zacc[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[g][e] = 0.f;
  }

  for (int base = ch.start + wave * 64; base < ch.end; base += kThreads) {
    const int r_raw = base + lane;
    const bool valid = r_raw < ch.end;
    const int r = valid ? r_raw : ch.end - 1;
    float s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) s[g] = 0.f;
    float vs = 1.f, vz = 0.f;
    if (!zone_c) {
      const int i = si.gbase[ch.kind] + r;
      const uint32_t* rp = krec + (ch.kind < 3 ? int64_t(i) * si.rec_a
                                               : int64_t(n_a) * si.rec_a + int64_t(i - n_a) * (si.rec_a - 1));
      for (int w = 0; w < rs.w16; ++w) {
        const uint32_t x = rp[w];
        const float k0 = half_lo(x), k1 = half_hi(x);
#pragma unroll
        for (int g = 0; g < G; ++g) s[g] = fmaf(sm.q[2 * w + 1][g], k1, fmaf(sm.q[2 * w][g], k0, s[g]));
      }
      int wo = rs.w16, mo = rs.w16 + rs.w8 + rs.w4 + rs.w2;
      // integer parts: 8-bit (4 codes a word), 4-bit (8), 2-bit (16)
      if (c4 > c8) {
        float dsum[G];
#pragma unroll
        for (int g = 0; g < G; ++g) dsum[g] = 0.f;
        for (int w = 0; w < rs.w8; ++w) {
          const uint32_t x = rp[wo + w];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float c = float((x >> (8 * e)) & 255u);
#pragma unroll
            for (int g = 0; g < G; ++g) dsum[g] = fmaf(sm.q[c8 + 4 * w + e][g], c, dsum[g]);
          }
        }
        const uint32_t m = rp[mo++];
        const float sc = half_lo(m), z = half_hi(m);
#pragma unroll
        for (int g = 0; g < G; ++g) s[g] = fmaf(sc, dsum[g], fmaf(z, sm.qsum[0][g], s[g]));
        wo += rs.w8;
      }
      if (c2 > c4) {
        float dsum[G];
#pragma unroll
        for (int g = 0; g < G; ++g) dsum[g] = 0.f;
        for (int w = 0; w < rs.w4; ++w) {
          const uint32_t x = rp[wo + w];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float c = float((x >> (4 * e)) & 15u);
#pragma unroll
            for (int g = 0; g < G; ++g) dsum[g] = fmaf(sm.q[c4 + 8 * w + e][g], c, dsum[g]);
          }
        }
        const uint32_t m = rp[mo++];
        const float sc = half_lo(m), z = half_hi(m);
#pragma unroll
        for (int g = 0; g < G; ++g) s[g] = fmaf(sc, dsum[g], fmaf(z, sm.qsum[1][g], s[g]));
        wo += rs.w4;
      }
      if (rs.w2 > 0) {
        float dsum[G];
#pragma unroll
        for (int g = 0; g < G; ++g) dsum[g] = 0.f;
        for (int w = 0; w < rs.w2; ++w) {
          const uint32_t x = rp[wo + w];
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float c = float((x >> (2 * e)) & 3u);
#pragma unroll
            for (int g = 0; g < G; ++g) dsum[g] = fmaf(sm.q[c2 + 16 * w + e][g], c, dsum[g]);
          }
        }
        const uint32_t m = rp[mo++];
        const float sc = half_lo(m), z = half_hi(m);
#pragma unroll
        for (int g = 0; g < G; ++g) s[g] = fmaf(sc, dsum[g], fmaf(z, sm.qsum[2][g], s[g]));
      }
      if (ch.kind < 3) {
        const uint32_t m = rp[si.rec_a - 1];
        vs = half_lo(m);
        vz = half_hi(m);
      }
    } else {
      const bool fresh = p.append && r == p.c_len;
      const uint32_t* kr = fresh ? reinterpret_cast<const uint32_t*>(p.k_new + seg * kHeadDim)
                                 : reinterpret_cast<const uint32_t*>(p.cache + si.off_kc) + int64_t(r) * (kHeadDim / 2);
      for (int w = 0; w < kHeadDim / 2; ++w) {
        const uint32_t x = kr[w];
        const float k0 = half_lo(x), k1 = half_hi(x);
#pragma unroll
        for (int g = 0; g < G; ++g) s[g] = fmaf(sm.q[2 * w + 1][g], k1, fmaf(sm.q[2 * w][g], k0, s[g]));
      }
    }

    // online softmax over this step
    float coef[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float t = valid ? s[g] * kLog2eOverSqrtD : -INFINITY;
      const float mnew = fmaxf(m_run[g], wave_max(t));
      const float alpha = exp2f(m_run[g] - mnew);
      const float pr = exp2f(t - mnew);
      m_run[g] = mnew;
      l_run[g] = fmaf(l_run[g], alpha, pr);
      zacc[g] = fmaf(zacc[g], alpha, pr * vz);
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[g][e] *= alpha;
      coef[g] = pr * vs;
      sm.coef[wave][lane][g] = coef[g];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // values: lane = (channel block cb, token slot ts)
#pragma unroll 2
    for (int rr = 0; rr < 8; ++rr) {
      const int j = rr * 8 + ts;
      const int row = base + j;
      if (row < ch.end) {
        float cf[G];
#pragma unroll
        for (int g = 0; g < G; ++g) cf[g] = sm.coef[wave][j][g];
        const uint8_t* vrow = (zone_c && p.append && row == p.c_len)
                                  ? reinterpret_cast<const uint8_t*>(p.v_new + seg * kHeadDim)
                                  : vbase + int64_t(row) * kRowBytes;
        float x[16];
        load_row16<B>(vrow, cb, x);
        accumulate16<G>(acc, cf, x);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // wave partial: sums over lanes
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l_run[g] = wave_sum(l_run[g]);
    zacc[g] = wave_sum(zacc[g]);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float v = acc[g][e];
      v += __shfl_xor(v, 8, 64);
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      acc[g][e] = v;
    }
  }
  if (ts == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 16; ++e) sm.part_o[wave][g][cb * 16 + e] = acc[g][e] + zacc[g];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      sm.part_ml[wave][g][0] = m_run[g];
      sm.part_ml[wave][g][1] = l_run[g];
    }
  }
}

// out[seg][g][c] = sum_k e^{m_k - M} o_k[c] / sum_k e^{m_k - M} l_k over the
// segment's chunks, in chunk order (so the result does not depend on which
// workgroup merges).
template <int G>
__device__ void merge_segment(const DecodeParams& p, int64_t seg, int n) {
  const float* part = p.partials + int64_t(seg) * p.max_chunks * G * kPartialFloats;
  for (int i = threadIdx.x; i < G * kHeadDim; i += kThreads) {
    const int g = i / kHeadDim, c = i % kHeadDim;
    float M = -INFINITY;
    for (int k = 0; k < n; ++k) M = fmaxf(M, part[(k * G + g) * kPartialFloats]);
    float L = 0.f, O = 0.f;
    for (int k = 0; k < n; ++k) {
      const float* pk = part + (k * G + g) * kPartialFloats;
      const float f = exp2f(pk[0] - M);
      L = fmaf(pk[1], f, L);
      O = fmaf(pk[4 + c], f, O);
    }
    p.out[(seg * G + g) * kHeadDim + c] = L > 0.f ? O / L : 0.f;
  }
}

template <int G>
__global__ __launch_bounds__(kThreads) void decode_chunk_kernel(DecodeParams p) {
  __shared__ Smem<G> sm;
  const int64_t seg = blockIdx.x / p.max_chunks;
  const int k = int(blockIdx.x % p.max_chunks);
  const SegInfo si = load_segment(p, seg);
  const int n_chunks = min(chunk_count(si.n_tok, zone_c_rows(p, si)), p.max_chunks);
  const Chunk ch = chunk_of(si.n_tok, zone_c_rows(p, si), k);
  const int tid = threadIdx.x;
  if (ch.kind < 0) {
    // a segment with nothing to attend to has a zero output
    if (k == 0 && n_chunks == 0)
      for (int i = tid; i < G * kHeadDim; i += kThreads) p.out[seg * G * kHeadDim + i] = 0.f;
    return;
  }

  // query of the G heads, in the channel order the rows use
  const uint8_t* perm = p.cache + kHeaderBytes + uint64_t(seg) * kDescBytes + kDescPerm;
  const int c_stored = si.n_chan[0] + si.n_chan[1] + si.n_chan[2] + si.n_chan[3];
  for (int i = tid; i < (kHeadDim + 16) * G; i += kThreads) {
    const int pos = i / G, g = i % G;
    float v = 0.f;
    if (ch.kind == 4) {
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
    const int hi = lo + si.n_chan[1 + j];
    float acc = 0.f;
    for (int c = lo; c < hi; ++c) acc += sm.q[c][g];
    sm.qsum[j][g] = acc;
  }
  // append the new token to zone C (only the chunk holding row c_len does it)
  if (ch.kind == 4 && p.append && p.c_len >= ch.start && p.c_len < ch.end) {
    uint32_t* kc = reinterpret_cast<uint32_t*>(p.cache + si.off_kc) + int64_t(p.c_len) * (kHeadDim / 2);
    uint32_t* vc = reinterpret_cast<uint32_t*>(p.cache + si.off_vc) + int64_t(p.c_len) * (kHeadDim / 2);
    if (tid < 64) kc[tid] = reinterpret_cast<const uint32_t*>(p.k_new + seg * kHeadDim)[tid];
    else if (tid < 128) vc[tid - 64] = reinterpret_cast<const uint32_t*>(p.v_new + seg * kHeadDim)[tid - 64];
  }
  __syncthreads();

  switch (ch.kind) {
    case 0: run_rows<G, 2>(p, si, seg, ch, sm); break;
    case 1: run_rows<G, 4>(p, si, seg, ch, sm); break;
    case 2: run_rows<G, 8>(p, si, seg, ch, sm); break;
    default: run_rows<G, 16>(p, si, seg, ch, sm); break;
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

  // The last workgroup of the segment to finish merges all its chunks.  The
  // counter lives in the descriptor, is 0 between calls and is reset here.
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    int* counter = reinterpret_cast<int*>(p.cache + kHeaderBytes + uint64_t(seg) * kDescBytes + kDescCounter);
    const int prev = atomicAdd(counter, 1);
    s_last = prev == n_chunks - 1;
    if (s_last) atomicExch(counter, 0);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  merge_segment<G>(p, seg, n_chunks);
}

template <int G>
hipError_t launch_g(const DecodeParams& p, hipStream_t stream) {
  const uint64_t grid = uint64_t(p.n_seg) * p.max_chunks;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_chunk_kernel<G>, dim3(unsigned(grid)), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  switch (p.group) {
    case 1: return launch_g<1>(p, stream);
    case 2: return launch_g<2>(p, stream);
    case 4: return launch_g<4>(p, stream);
    case 8: return launch_g<8>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace rdkv
