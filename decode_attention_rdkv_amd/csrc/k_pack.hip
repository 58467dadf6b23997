// TriZone packing (RDKV summary, section 2.3) with the asymmetric uniform
// quantizer of "Matematika KV Cache Compression", section "Solusi 3".
//
// rdkv_pack runs two kernels per call:
//   pack_index_kernel  one workgroup per segment: token-group counts, channel
//                      permutation, kept positions (group-major, ascending),
//                      descriptor; checks that the allocation fits the slot.
//   pack_rows_kernel   one wave per kept token: quantizes the V row and the
//                      permuted K row bit-segment by bit-segment, packs codes
//                      LSB-first, writes the V row and the K record.
// Quantizer, bit-exact with the format specification: zero = fp16 min,
// scale = fp16_rne(fl32(fl32(max - min) / (2^b - 1))),
// q = clamp(rint_even(fl32(fl32(x - zero) / scale)), 0, 2^b - 1), scale 0 -> q 0.
#include <algorithm>

#include "rdkv_internal.h"

namespace rdkv {
namespace {

constexpr int kIndexThreads = 1024;
constexpr int kRowsThreads = 256;
constexpr int kRowsWgPerSeg = 64;

struct SegGeom {
  uint64_t slots_offset, slot_bytes, off_v, off_krec, off_pos;
  int64_t n_tok_total;   // N
  int64_t nk_max;
  int64_t v_reserve;
  int64_t v_units;       // bound on sum_g n_g 2^g: min(B_V / 2, 8 N) (decode's chunk count follows from it)
  int32_t cap, rec_max;
};

__device__ inline void st_u32(uint8_t* base, uint64_t off, uint32_t v) {
  *reinterpret_cast<uint32_t*>(base + off) = v;
}
__device__ inline void st_i32(uint8_t* base, uint64_t off, int32_t v) {
  *reinterpret_cast<int32_t*>(base + off) = v;
}
__device__ inline void st_u64(uint8_t* base, uint64_t off, uint64_t v) {
  *reinterpret_cast<uint64_t*>(base + off) = v;
}

// Writes a segment descriptor.  n_tok/n_chan may be zero (empty segment).
__device__ void write_descriptor(uint8_t* cache, int64_t seg, const SegGeom& g, const int n_tok[4],
                                 const int n_chan[4], int flags, const uint8_t* perm, int tid, int nthreads) {
  uint8_t* d = cache + kHeaderBytes + uint64_t(seg) * kDescBytes;
  const uint64_t slot = g.slots_offset + uint64_t(seg) * g.slot_bytes;
  if (tid == 0) {
    int n_kept = 0;
    for (int i = 0; i < 4; ++i) {
      st_i32(d, kDescNTok + 4 * i, n_tok[i]);
      n_kept += n_tok[i];
    }
    st_i32(d, kDescNKept, n_kept);
    for (int i = 0; i < 4; ++i) st_i32(d, kDescNChan + 4 * i, n_chan[i]);
    const RecordShape rs = record_shape(n_chan[0], n_chan[1], n_chan[2], n_chan[3]);
    st_i32(d, kDescRec, 4 * rs.words_a());
    st_i32(d, kDescCap, g.cap);
    st_i32(d, kDescFlags, flags);
    uint64_t cur = slot + g.off_v;
    for (int i = 0; i < 4; ++i) {
      st_u64(d, kDescOffV + 8 * i, cur);
      cur = align_up(cur + uint64_t(n_tok[i]) * (kHeadDim * group_bits(i) / 8), kAlign);
    }
    st_u64(d, kDescOffKrec, slot + g.off_krec);
    st_u64(d, kDescOffPos, slot + g.off_pos);
    st_u64(d, kDescOffKc, slot);
    st_u64(d, kDescOffVc, slot + uint64_t(g.cap) * kHeadDim * 2);
    for (int i = 112; i < 128; i += 4) st_u32(d, i, 0u);
  }
  for (int c = tid; c < kHeadDim; c += nthreads) d[kDescPerm + c] = perm ? perm[c] : uint8_t(c);
}

// ------------------------------------------------------------------ init

__global__ void cache_zero_kernel(uint4* p, uint64_t n16) {
  const uint64_t stride = uint64_t(gridDim.x) * blockDim.x;
  for (uint64_t i = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
}

__global__ void cache_header_kernel(uint8_t* cache, rdkv_layout lay, SegGeom g) {
  const int64_t seg = int64_t(blockIdx.x) * (blockDim.x / 64) + threadIdx.x / 64;
  const int lane = threadIdx.x & 63;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    const int32_t h32[8] = {int32_t(kMagic), kFormatVersion, lay.dims.n_seq, lay.dims.n_layers,
                            lay.dims.n_q_heads, lay.dims.n_kv_heads, lay.dims.head_dim, lay.zone_c_capacity};
    for (int i = 0; i < 8; ++i) st_i32(cache, 4 * i, h32[i]);
    const int64_t h64[7] = {lay.dims.n_tokens, lay.budget_v, lay.budget_k, lay.n_seg,
                            int64_t(kHeaderBytes), int64_t(lay.slots_offset), int64_t(lay.slot_bytes)};
    for (int i = 0; i < 7; ++i) st_u64(cache, 32 + 8 * i, uint64_t(h64[i]));
    // generations (all zero without rollover): reserved, in use, where, budgets
    st_i32(cache, kHdrNGen, lay.n_generations);
    st_i32(cache, kHdrNGenUsed, 0);
    st_u64(cache, kHdrGenOffset, lay.gen_offset);
    st_u64(cache, kHdrGenBytes, lay.gen_bytes);
    st_u64(cache, kHdrGenBudgetV, uint64_t(lay.gen_budget_v));
    st_u64(cache, kHdrGenBudgetK, uint64_t(lay.gen_budget_k));
  }
  if (seg >= lay.n_seg) return;
  const int z[4] = {0, 0, 0, 0};
  write_descriptor(cache, seg, g, z, z, 0, nullptr, lane, 64);
}

SegGeom geom_of(const rdkv_layout& lay) {
  SegGeom g;
  g.slots_offset = lay.slots_offset;
  g.slot_bytes = lay.slot_bytes;
  g.off_v = lay.slot_off_v;
  g.off_krec = lay.slot_off_krec;
  g.off_pos = lay.slot_off_pos;
  g.n_tok_total = lay.dims.n_tokens;
  g.nk_max = lay.nk_max;
  g.v_reserve = int64_t(lay.slot_off_krec - lay.slot_off_v);
  g.v_units = std::min<int64_t>(lay.budget_v / 2, 8 * lay.dims.n_tokens);
  g.cap = lay.zone_c_capacity;
  g.rec_max = lay.rec_max;
  return g;
}

// ------------------------------------------------------------------ index

struct IndexArgs {
  uint8_t* cache;
  SegGeom g;
  int32_t L, Hkv, layer_begin, n_layers_in;
  const uint8_t* bits_tok;
  const uint8_t* bits_chan;
};

__global__ __launch_bounds__(kIndexThreads) void pack_index_kernel(IndexArgs a) {
  const int64_t seg_in = blockIdx.x;                // [S][n_layers_in][Hkv]
  const int h = int(seg_in % a.Hkv);
  const int l_in = int((seg_in / a.Hkv) % a.n_layers_in);
  const int s = int(seg_in / (int64_t(a.Hkv) * a.n_layers_in));
  const int64_t seg = (int64_t(s) * a.L + a.layer_begin + l_in) * a.Hkv + h;
  const int64_t N = a.g.n_tok_total;
  const uint8_t* bt = a.bits_tok + seg_in * N;
  const uint8_t* bc = a.bits_chan + seg_in * kHeadDim;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int kWaves = kIndexThreads / 64;

  __shared__ int s_cnt[kWaves][4];
  __shared__ int s_tot[4];
  __shared__ uint8_t s_perm[kHeadDim];
  __shared__ int s_nchan[4];

  // counts of kept tokens per group
  int cnt[4] = {0, 0, 0, 0};
  for (int64_t t = tid; t < N; t += kIndexThreads) {
    const int gi = bits_group(bt[t]);
    if (gi >= 0) cnt[gi]++;
  }
  for (int i = 0; i < 4; ++i) {
    const int v = wave_sum_i(cnt[i]);
    if (lane == 0) s_cnt[wave][i] = v;
  }
  // channel permutation: bitwidth 16, 8, 4, 2 then 0, ascending channel index
  if (tid < kHeadDim) {
    auto rank = [](int b) { return b == 16 ? 0 : b == 8 ? 1 : b == 4 ? 2 : b == 2 ? 3 : 4; };
    const int rc = rank(bc[tid]);
    int pos = 0;
    for (int c = 0; c < kHeadDim; ++c) {
      const int r = rank(bc[c]);
      pos += (r < rc) || (r == rc && c < tid);
    }
    s_perm[pos] = uint8_t(tid);
  }
  if (tid < 4) {
    int n = 0;
    const int want = 16 >> tid;   // 16, 8, 4, 2
    for (int c = 0; c < kHeadDim; ++c) n += (bc[c] == want);
    s_nchan[tid] = n;
  }
  __syncthreads();
  if (tid < 4) {
    int n = 0;
    for (int w = 0; w < kWaves; ++w) n += s_cnt[w][tid];
    s_tot[tid] = n;
  }
  __syncthreads();
  int n_tok[4], n_chan[4];
  for (int i = 0; i < 4; ++i) {
    n_tok[i] = s_tot[i];
    n_chan[i] = s_nchan[i];
  }
  // does the allocation fit the slot?
  const int64_t n_kept = int64_t(n_tok[0]) + n_tok[1] + n_tok[2] + n_tok[3];
  // end of the last V group; group starts are 256-aligned, its end is not
  uint64_t vbytes = 0;
  for (int i = 0; i < 4; ++i) {
    if (i) vbytes = align_up(vbytes, kAlign);
    vbytes += uint64_t(n_tok[i]) * (kHeadDim * group_bits(i) / 8);
  }
  const RecordShape rs = record_shape(n_chan[0], n_chan[1], n_chan[2], n_chan[3]);
  // a g-group token costs 2^(g+1) bits, so sum_b b_t <= B_V gives sum_g n_g 2^g <= B_V / 2
  const int64_t v_units = int64_t(n_tok[0]) + 2 * int64_t(n_tok[1]) + 4 * int64_t(n_tok[2]) + 8 * int64_t(n_tok[3]);
  const bool fits = n_kept <= a.g.nk_max && int64_t(vbytes) <= a.g.v_reserve && v_units <= a.g.v_units &&
                    4 * rs.words_a() <= a.g.rec_max;
  if (!fits) {
    const int z[4] = {0, 0, 0, 0};
    write_descriptor(a.cache, seg, a.g, z, z, 1, nullptr, tid, kIndexThreads);
  } else {
    write_descriptor(a.cache, seg, a.g, n_tok, n_chan, 0, s_perm, tid, kIndexThreads);
  }
  // clear zone C (K_C and V_C are contiguous at the slot start)
  {
    const uint64_t slot = a.g.slots_offset + uint64_t(seg) * a.g.slot_bytes;
    uint4* zc = reinterpret_cast<uint4*>(a.cache + slot);
    const int64_t n16 = int64_t(a.g.cap) * kHeadDim * 2 * 2 / 16;
    for (int64_t i = tid; i < n16; i += kIndexThreads) zc[i] = make_uint4(0, 0, 0, 0);
  }
  if (!fits) return;

  // kept positions, group-major, ascending inside a group
  int32_t* pos = reinterpret_cast<int32_t*>(a.cache + a.g.slots_offset + uint64_t(seg) * a.g.slot_bytes + a.g.off_pos);
  int gbase[4];
  gbase[0] = 0;
  for (int i = 1; i < 4; ++i) gbase[i] = gbase[i - 1] + n_tok[i - 1];
  int run[4] = {0, 0, 0, 0};
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t t0 = 0; t0 < N; t0 += kIndexThreads) {
    const int64_t t = t0 + tid;
    const int gi = t < N ? bits_group(bt[t]) : -1;
    int my_rank = 0;
    __syncthreads();   // s_cnt reuse
    for (int i = 0; i < 4; ++i) {
      const uint64_t m = __ballot(gi == i);
      if (gi == i) my_rank = __popcll(m & lt_mask);
      if (lane == 0) s_cnt[wave][i] = __popcll(m);
    }
    __syncthreads();
    if (gi >= 0) {
      int before = 0;
      for (int w = 0; w < wave; ++w) before += s_cnt[w][gi];
      pos[gbase[gi] + run[gi] + before + my_rank] = int32_t(t);
    }
    for (int i = 0; i < 4; ++i) {
      int tot = 0;
      for (int w = 0; w < kWaves; ++w) tot += s_cnt[w][i];
      run[i] += tot;
    }
  }
}

// ------------------------------------------------------------------ rows

struct RowsArgs {
  uint8_t* cache;
  SegGeom g;
  int32_t L, Hkv, layer_begin, n_layers_in;
  const __half* K;
  const __half* V;
};

// Quantize one value with the segment's (zero, scale): bit-exact IEEE steps.
__device__ inline uint32_t quant_code(float x, float zero, float scale, int b) {
  if (scale == 0.0f) return 0u;
  float q = rintf(__fdiv_rn(__fsub_rn(x, zero), scale));
  q = fminf(fmaxf(q, 0.0f), float((1 << b) - 1));
  return uint32_t(q);
}

struct QParams {
  float zero, scale;
  uint32_t word;   // half2: scale low, zero high
};
__device__ inline QParams quant_params(float mn, float mx, int b) {
  const float rng = __fsub_rn(mx, mn);
  const __half s16 = __float2half_rn(__fdiv_rn(rng, float((1 << b) - 1)));
  const __half z16 = __float2half_rn(mn);   // exact: mn is an fp16 value
  QParams p;
  p.scale = __half2float(s16);
  p.zero = __half2float(z16);
  p.word = uint32_t(__half_as_ushort(s16)) | (uint32_t(__half_as_ushort(z16)) << 16);
  return p;
}

__global__ __launch_bounds__(kRowsThreads) void pack_rows_kernel(RowsArgs a) {
  const int64_t seg_in = blockIdx.y;
  const int h = int(seg_in % a.Hkv);
  const int l_in = int((seg_in / a.Hkv) % a.n_layers_in);
  const int s = int(seg_in / (int64_t(a.Hkv) * a.n_layers_in));
  const int64_t seg = (int64_t(s) * a.L + a.layer_begin + l_in) * a.Hkv + h;
  const int64_t N = a.g.n_tok_total;
  const uint8_t* d = a.cache + kHeaderBytes + uint64_t(seg) * kDescBytes;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kWaves = kRowsThreads / 64;

  __shared__ uint16_t s_code[kWaves][kHeadDim];
  __shared__ uint8_t s_perm[kHeadDim];

  int n_tok[4], n_chan[4];
  for (int i = 0; i < 4; ++i) {
    n_tok[i] = *reinterpret_cast<const int32_t*>(d + kDescNTok + 4 * i);
    n_chan[i] = *reinterpret_cast<const int32_t*>(d + kDescNChan + 4 * i);
  }
  const int n_kept = *reinterpret_cast<const int32_t*>(d + kDescNKept);
  const int rec_a = *reinterpret_cast<const int32_t*>(d + kDescRec) / 4;   // words
  uint64_t off_v[4];
  for (int i = 0; i < 4; ++i) off_v[i] = *reinterpret_cast<const uint64_t*>(d + kDescOffV + 8 * i);
  const uint64_t off_krec = *reinterpret_cast<const uint64_t*>(d + kDescOffKrec);
  const uint64_t off_pos = *reinterpret_cast<const uint64_t*>(d + kDescOffPos);
  for (int c = threadIdx.x; c < kHeadDim; c += kRowsThreads) s_perm[c] = d[kDescPerm + c];
  __syncthreads();
  if (n_kept == 0) return;

  const RecordShape rs = record_shape(n_chan[0], n_chan[1], n_chan[2], n_chan[3]);
  const int n_a = n_tok[0] + n_tok[1] + n_tok[2];
  const int c8 = n_chan[0], c4 = c8 + n_chan[1], c2 = c4 + n_chan[2], c0 = c2 + n_chan[3];
  const int32_t* pos = reinterpret_cast<const int32_t*>(a.cache + off_pos);
  const __half* Kseg = a.K + seg_in * N * kHeadDim;
  const __half* Vseg = a.V + seg_in * N * kHeadDim;
  uint16_t* code = s_code[wave];

  const int waves_total = gridDim.x * kWaves;
  for (int i = blockIdx.x * kWaves + wave; i < n_kept; i += waves_total) {
    const int t = pos[i];
    int gi = 0, r = i;
    while (gi < 3 && r >= n_tok[gi]) r -= n_tok[gi++];
    const int b = group_bits(gi);

    // ---- V row: lane holds channels 2*lane, 2*lane+1
    const uint32_t vw = reinterpret_cast<const uint32_t*>(Vseg + int64_t(t) * kHeadDim)[lane];
    uint32_t vmeta = 0;
    uint8_t* vrow = a.cache + off_v[gi] + uint64_t(r) * (kHeadDim * b / 8);
    if (b == 16) {
      reinterpret_cast<uint32_t*>(vrow)[lane] = vw;
    } else {
      const float v0 = half_lo(vw), v1 = half_hi(vw);
      const float mn = wave_min(fminf(v0, v1)), mx = wave_max(fmaxf(v0, v1));
      const QParams qp = quant_params(mn, mx, b);
      vmeta = qp.word;
      const uint32_t q0 = quant_code(v0, qp.zero, qp.scale, b);
      const uint32_t q1 = quant_code(v1, qp.zero, qp.scale, b);
      const int bit = (2 * lane * b) & 31;
      uint32_t part = (q0 << bit) | (q1 << (bit + b));
      const int lanes_per_word = 16 / b;
      for (int m = 1; m < lanes_per_word; m <<= 1) part |= __shfl_xor(part, m, 64);
      if ((lane & (lanes_per_word - 1)) == 0) reinterpret_cast<uint32_t*>(vrow)[(2 * lane * b) >> 5] = part;
    }

    // ---- K row in permuted channel order: lane holds positions 2*lane, 2*lane+1
    const __half* krow = Kseg + int64_t(t) * kHeadDim;
    const int p0 = 2 * lane, p1 = 2 * lane + 1;
    const __half h0 = krow[s_perm[p0]], h1 = krow[s_perm[p1]];
    const float k0 = __half2float(h0), k1 = __half2float(h1);
    QParams kq[3];
    const int lo[3] = {c8, c4, c2}, hi[3] = {c4, c2, c0};
    for (int j = 0; j < 3; ++j) {
      const int bj = 8 >> j;
      const bool in0 = p0 >= lo[j] && p0 < hi[j], in1 = p1 >= lo[j] && p1 < hi[j];
      const float mn = wave_min(fminf(in0 ? k0 : INFINITY, in1 ? k1 : INFINITY));
      const float mx = wave_max(fmaxf(in0 ? k0 : -INFINITY, in1 ? k1 : -INFINITY));
      kq[j] = (hi[j] > lo[j]) ? quant_params(mn, mx, bj) : QParams{0.f, 0.f, 0u};
    }
    auto kcode = [&](int p, float kv, __half hv) -> uint16_t {
      if (p < c8) return __half_as_ushort(hv);
      if (p < c4) return uint16_t(quant_code(kv, kq[0].zero, kq[0].scale, 8));
      if (p < c2) return uint16_t(quant_code(kv, kq[1].zero, kq[1].scale, 4));
      if (p < c0) return uint16_t(quant_code(kv, kq[2].zero, kq[2].scale, 2));
      return 0;
    };
    code[p0] = kcode(p0, k0, h0);
    code[p1] = kcode(p1, k1, h1);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    const bool is_a = gi < 3;
    const int nwords = is_a ? rec_a : rec_a - 1;
    uint32_t* rec = reinterpret_cast<uint32_t*>(a.cache + off_krec) +
                    (is_a ? int64_t(i) * rec_a : int64_t(n_a) * rec_a + int64_t(i - n_a) * (rec_a - 1));
    for (int w = lane; w < nwords; w += 64) {
      uint32_t word = 0;
      int x = w;
      if (x < rs.w16) {
        const int p = 2 * x;
        word = uint32_t(code[p]) | ((p + 1 < c8) ? uint32_t(code[p + 1]) << 16 : 0u);
      } else if ((x -= rs.w16) < rs.w8) {
        for (int e = 0; e < 4; ++e) {
          const int p = c8 + 4 * x + e;
          if (p < c4) word |= uint32_t(code[p]) << (8 * e);
        }
      } else if ((x -= rs.w8) < rs.w4) {
        for (int e = 0; e < 8; ++e) {
          const int p = c4 + 8 * x + e;
          if (p < c2) word |= uint32_t(code[p]) << (4 * e);
        }
      } else if ((x -= rs.w4) < rs.w2) {
        for (int e = 0; e < 16; ++e) {
          const int p = c2 + 16 * x + e;
          if (p < c0) word |= uint32_t(code[p]) << (2 * e);
        }
      } else if ((x -= rs.w2) < rs.n_meta) {
        // the x-th present integer part, in order 8, 4, 2
        int seen = 0;
        for (int j = 0; j < 3; ++j) {
          if (hi[j] > lo[j]) {
            if (seen == x) word = kq[j].word;
            ++seen;
          }
        }
      } else {
        word = vmeta;   // only reached for zone-A tokens
      }
      rec[w] = word;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");   // s_code is rewritten by the next token
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// ------------------------------------------------------------------ unpack (test support)

struct UnpackArgs {
  const uint8_t* cache;
  int64_t seg;
  float* k_hat;
  float* v_hat;
};

__global__ __launch_bounds__(256) void unpack_kernel(UnpackArgs a) {
  const uint8_t* d = a.cache + kHeaderBytes + uint64_t(a.seg) * kDescBytes;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int n_tok[4], n_chan[4];
  for (int i = 0; i < 4; ++i) {
    n_tok[i] = *reinterpret_cast<const int32_t*>(d + kDescNTok + 4 * i);
    n_chan[i] = *reinterpret_cast<const int32_t*>(d + kDescNChan + 4 * i);
  }
  const int n_kept = *reinterpret_cast<const int32_t*>(d + kDescNKept);
  const int rec_a = *reinterpret_cast<const int32_t*>(d + kDescRec) / 4;
  uint64_t off_v[4];
  for (int i = 0; i < 4; ++i) off_v[i] = *reinterpret_cast<const uint64_t*>(d + kDescOffV + 8 * i);
  const uint64_t off_krec = *reinterpret_cast<const uint64_t*>(d + kDescOffKrec);
  const uint8_t* perm = d + kDescPerm;
  const RecordShape rs = record_shape(n_chan[0], n_chan[1], n_chan[2], n_chan[3]);
  const int n_a = n_tok[0] + n_tok[1] + n_tok[2];
  const int c8 = n_chan[0], c4 = c8 + n_chan[1], c2 = c4 + n_chan[2], c0 = c2 + n_chan[3];

  for (int i = blockIdx.x * 4 + wave; i < n_kept; i += gridDim.x * 4) {
    int gi = 0, r = i;
    while (gi < 3 && r >= n_tok[gi]) r -= n_tok[gi++];
    const int b = group_bits(gi);
    const bool is_a = gi < 3;
    const uint32_t* rec = reinterpret_cast<const uint32_t*>(a.cache + off_krec) +
                          (is_a ? int64_t(i) * rec_a : int64_t(n_a) * rec_a + int64_t(i - n_a) * (rec_a - 1));
    const uint8_t* vrow = a.cache + off_v[gi] + uint64_t(r) * (kHeadDim * b / 8);
    for (int c = lane; c < kHeadDim; c += 64) {
      float v;
      if (b == 16) {
        v = __half2float(reinterpret_cast<const __half*>(vrow)[c]);
      } else {
        const uint32_t w = reinterpret_cast<const uint32_t*>(vrow)[(c * b) >> 5];
        const uint32_t q = (w >> ((c * b) & 31)) & ((1u << b) - 1);
        const uint32_t m = rec[rec_a - 1];
        v = fmaf(float(q), half_lo(m), half_hi(m));
      }
      a.v_hat[int64_t(i) * kHeadDim + c] = v;
    }
    for (int p = lane; p < kHeadDim; p += 64) {
      float k = 0.0f;
      if (p < c8) {
        k = (p & 1) ? half_hi(rec[p >> 1]) : half_lo(rec[p >> 1]);
      } else if (p < c0) {
        int j, lo, bj, wbase;
        if (p < c4) { j = 0; lo = c8; bj = 8; wbase = rs.w16; }
        else if (p < c2) { j = 1; lo = c4; bj = 4; wbase = rs.w16 + rs.w8; }
        else { j = 2; lo = c2; bj = 2; wbase = rs.w16 + rs.w8 + rs.w4; }
        int mi = rs.w16 + rs.w8 + rs.w4 + rs.w2;
        for (int jj = 0; jj < j; ++jj) mi += (n_chan[1 + jj] > 0);
        const int e = p - lo;
        const uint32_t w = rec[wbase + ((e * bj) >> 5)];
        const uint32_t q = (w >> ((e * bj) & 31)) & ((1u << bj) - 1);
        k = fmaf(float(q), half_lo(rec[mi]), half_hi(rec[mi]));
      }
      a.k_hat[int64_t(i) * kHeadDim + perm[p]] = k;
    }
  }
}

// ------------------------------------------------------------------ status

// out[0] = number of segments whose descriptor carries the "did not fit"
// flag (bit 0): their allocation exceeded the layout's bounds and they were
// packed empty.  One workgroup; a fixed-order reduction.
__global__ __launch_bounds__(256) void pack_status_kernel(const uint8_t* cache, int64_t n_seg, int32_t* out) {
  __shared__ int s_part[4];
  int n = 0;
  for (int64_t seg = threadIdx.x; seg < n_seg; seg += 256)
    n += *reinterpret_cast<const int32_t*>(cache + kHeaderBytes + uint64_t(seg) * kDescBytes + kDescFlags) & 1;
  n = wave_sum_i(n);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = n;
  __syncthreads();
  if (threadIdx.x == 0) out[0] = s_part[0] + s_part[1] + s_part[2] + s_part[3];
}

// ------------------------------------------------------------------ paged cache

__global__ void paged_header_kernel(uint8_t* cache, rdkv_paged_layout pl) {
  const uint64_t n = uint64_t(pl.n_seg) * pl.max_pages;
  int32_t* table = reinterpret_cast<int32_t*>(cache + pl.table_offset);
  const uint64_t stride = uint64_t(gridDim.x) * blockDim.x;
  for (uint64_t i = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) table[i] = -1;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    const int32_t h32[8] = {int32_t(kPagedMagic), kFormatVersion, pl.dims.n_seq, pl.dims.n_layers,
                            pl.dims.n_q_heads, pl.dims.n_kv_heads, pl.dims.head_dim, pl.zone_c_capacity};
    for (int i = 0; i < 8; ++i) st_i32(cache, 4 * i, h32[i]);
    const int64_t h64[10] = {pl.dims.n_tokens, pl.budget_v_max, pl.budget_k_max, pl.n_seg, int64_t(kHeaderBytes),
                             int64_t(pl.table_offset), int64_t(pl.pool_offset), pl.max_pages, pl.n_pages,
                             int64_t(kPageBytes)};
    for (int i = 0; i < 10; ++i) st_u64(cache, 32 + 8 * i, uint64_t(h64[i]));
  }
}

// What the staged (contiguous-format) descriptor of one segment says, and
// where its regions would go in pages.
struct StagedSeg {
  int n_tok[4], n_kept, n_chan[4], rec;
  uint64_t src[kRegions];      // staging offset of each region's first row (zone-C regions: none)
  int rows[kRegions];
  int row_bytes[kRegions];
  int pages[kRegions];
  int vpage[kRegions];
  int total;
  bool ok;
};

__device__ StagedSeg read_staged(const uint8_t* staging, uint64_t staging_bytes, int si, int cap, int64_t nk_max,
                                 int rec_max) {
  const uint8_t* d = staging + kHeaderBytes + uint64_t(si) * kDescBytes;
  StagedSeg g;
  int sum = 0;
  g.ok = true;
  for (int i = 0; i < 4; ++i) {
    g.n_tok[i] = *reinterpret_cast<const int32_t*>(d + kDescNTok + 4 * i);
    g.n_chan[i] = *reinterpret_cast<const int32_t*>(d + kDescNChan + 4 * i);
    g.ok = g.ok && g.n_tok[i] >= 0 && g.n_chan[i] >= 0;
    sum += g.n_tok[i];
  }
  g.n_kept = *reinterpret_cast<const int32_t*>(d + kDescNKept);
  g.rec = *reinterpret_cast<const int32_t*>(d + kDescRec);
  const RecordShape rs = record_shape(g.n_chan[0], g.n_chan[1], g.n_chan[2], g.n_chan[3]);
  g.ok = g.ok && sum == g.n_kept && g.n_kept <= nk_max && g.rec == 4 * rs.words_a() && g.rec <= rec_max;
  if (!g.ok) {
    for (int i = 0; i < 4; ++i) g.n_tok[i] = 0;
    g.n_kept = 0;
    g.rec = 4;
  }
  const uint64_t off_krec = *reinterpret_cast<const uint64_t*>(d + kDescOffKrec);
  uint64_t rec_at = off_krec;
  for (int i = 0; i < 4; ++i) {
    g.rows[kRegV + i] = g.n_tok[i];
    g.row_bytes[kRegV + i] = kHeadDim * group_bits(i) / 8;
    g.src[kRegV + i] = *reinterpret_cast<const uint64_t*>(d + kDescOffV + 8 * i);
    g.rows[kRegRec + i] = g.n_tok[i];
    g.row_bytes[kRegRec + i] = g.rec - 4 * (i == 3);
    g.src[kRegRec + i] = rec_at;
    rec_at += uint64_t(g.n_tok[i]) * g.row_bytes[kRegRec + i];
  }
  g.rows[kRegKC] = g.rows[kRegVC] = cap;
  g.row_bytes[kRegKC] = g.row_bytes[kRegVC] = kHeadDim * 2;
  g.src[kRegKC] = g.src[kRegVC] = 0;
  g.rows[kRegPos] = g.n_kept;
  g.row_bytes[kRegPos] = 4;
  g.src[kRegPos] = *reinterpret_cast<const uint64_t*>(d + kDescOffPos);
  g.total = 0;
  for (int r = 0; r < kRegions; ++r) {
    g.pages[r] = paged_region_pages(g.rows[r], paged_tile_bytes(r, g.rec));
    g.vpage[r] = g.total;
    g.total += g.pages[r];
    if (r != kRegKC && r != kRegVC && g.rows[r] > 0)
      g.ok = g.ok && g.src[r] + uint64_t(g.rows[r]) * g.row_bytes[r] <= staging_bytes;
  }
  return g;
}

struct PagedKArgs {
  uint8_t* cache;
  rdkv_paged_layout pl;
  const uint8_t* staging;
  uint64_t staging_bytes;
  int32_t seq;
  const int32_t* pages;
  int32_t* pages_needed;
};

// pages_needed[si] for the staged segments; one thread per segment
__global__ void paged_plan_kernel(PagedKArgs a) {
  const int seg_per_seq = a.pl.dims.n_layers * a.pl.dims.n_kv_heads;
  const int si = blockIdx.x * blockDim.x + threadIdx.x;
  if (si >= seg_per_seq) return;
  const StagedSeg g = read_staged(a.staging, a.staging_bytes, si, a.pl.zone_c_capacity, a.pl.nk_max, a.pl.rec_max);
  a.pages_needed[si] = g.total;
}

// One workgroup per segment of the sequence: block-table row, descriptor,
// and the regions' rows copied tile by tile into the given pages (zone C
// zeroed).  Invalid page lists leave the slot's segment empty and flagged.
__global__ __launch_bounds__(256) void paged_commit_kernel(PagedKArgs a) {
  const int seg_per_seq = a.pl.dims.n_layers * a.pl.dims.n_kv_heads;
  const int si = blockIdx.x;
  const int64_t seg = int64_t(a.seq) * seg_per_seq + si;
  const int tid = threadIdx.x;
  const int cap = a.pl.zone_c_capacity;
  const StagedSeg g = read_staged(a.staging, a.staging_bytes, si, cap, a.pl.nk_max, a.pl.rec_max);
  const int32_t* pg = a.pages + int64_t(si) * a.pl.max_pages;
  __shared__ int s_bad;
  if (tid == 0) s_bad = !g.ok || g.total > a.pl.max_pages;
  __syncthreads();
  for (int i = tid; i < g.total && i < a.pl.max_pages; i += 256)
    if (pg[i] < 0 || pg[i] >= a.pl.n_pages) s_bad = 1;
  __syncthreads();
  const bool ok = !s_bad;
  int32_t* row = reinterpret_cast<int32_t*>(a.cache + a.pl.table_offset) + seg * a.pl.max_pages;
  for (int i = tid; i < a.pl.max_pages; i += 256) row[i] = (ok && i < g.total) ? pg[i] : -1;
  uint8_t* d = a.cache + kHeaderBytes + uint64_t(seg) * kDescBytes;
  const uint8_t* sd = a.staging + kHeaderBytes + uint64_t(si) * kDescBytes;
  if (tid < kDescBytes / 4) {
    uint32_t w = 0;
    const int b = 4 * tid;
    if (ok) {
      if (b < kDescNTok + 16) w = uint32_t(g.n_tok[b / 4]);
      else if (b == kDescNKept) w = uint32_t(g.n_kept);
      else if (b < kDescNChan + 16) w = uint32_t(g.n_chan[(b - kDescNChan) / 4]);
      else if (b == kDescRec) w = uint32_t(g.rec);
      else if (b == kDescCap) w = uint32_t(cap);
      else if (b >= kPDescVpage && b < kPDescVpage + 4 * kRegions) w = uint32_t(g.vpage[(b - kPDescVpage) / 4]);
      else if (b == kPDescNPages) w = uint32_t(g.total);
      else if (b >= kDescPerm) w = *reinterpret_cast<const uint32_t*>(sd + b);
    } else if (b == kDescFlags) {
      w = 1u;
    }
    st_u32(d, b, w);
  }
  if (!ok) return;
  uint8_t* pool = a.cache + a.pl.pool_offset;
  for (int r = 0; r < kRegions; ++r) {
    const int rb = g.row_bytes[r];
    if (g.rows[r] == 0 || rb == 0) continue;
    const uint32_t tb = paged_tile_bytes(r, g.rec);
    const int tpp = int(kPageBytes / tb);
    const bool zero = r == kRegKC || r == kRegVC;
    // whole tiles of zone C are cleared; the other regions copy their rows
    const int64_t words = zero ? int64_t((g.rows[r] + kPagedTile - 1) / kPagedTile) * (tb / 4)
                               : int64_t(g.rows[r]) * (rb / 4);
    for (int64_t j = tid; j < words; j += 256) {
      const int64_t byte = j * 4;
      const int64_t tile = zero ? byte / tb : (byte / rb) / kPagedTile;
      const int64_t in_tile = zero ? byte % tb : byte - tile * kPagedTile * rb;
      const int page = pg[g.vpage[r] + int(tile / tpp)];
      uint32_t* dst = reinterpret_cast<uint32_t*>(pool + uint64_t(page) * kPageBytes + (tile % tpp) * tb + in_tile);
      *dst = zero ? 0u : *reinterpret_cast<const uint32_t*>(a.staging + g.src[r] + byte);
    }
  }
}

__global__ __launch_bounds__(256) void paged_release_kernel(uint8_t* cache, rdkv_paged_layout pl, int32_t seq) {
  const int seg_per_seq = pl.dims.n_layers * pl.dims.n_kv_heads;
  const int64_t seg = int64_t(seq) * seg_per_seq + blockIdx.x;
  int32_t* row = reinterpret_cast<int32_t*>(cache + pl.table_offset) + seg * pl.max_pages;
  for (int i = threadIdx.x; i < pl.max_pages; i += 256) row[i] = -1;
  if (threadIdx.x < kDescBytes / 4) st_u32(cache + kHeaderBytes + uint64_t(seg) * kDescBytes, 4 * threadIdx.x, 0u);
}

// ---------------------------------------------------------------- decode launch shape

// A segment in use (zone-C capacity of the layout: a committed paged slot, or
// any segment of a contiguous blob) and its prefill-token chunk count and K
// record bytes, as decode counts them; -1 chunks for a free slot or one the
// layout's own bounds already reject (decode reads it as empty either way).
struct SegShape {
  int chunks, rec;
};
__device__ inline SegShape seg_shape(const uint8_t* cache, const ShapeGeom& g, int64_t seg) {
  const uint8_t* d = cache + kHeaderBytes + uint64_t(seg) * kDescBytes;
  SegShape r{-1, 0};
  if (*reinterpret_cast<const int32_t*>(d + kDescCap) != g.zone_c_capacity) return r;
  int chunks = 0;
  for (int i = 0; i < 4; ++i) {
    const int n = *reinterpret_cast<const int32_t*>(d + kDescNTok + 4 * i);
    if (n < 0) return r;
    chunks += (n + chunk_tokens(g.chunk_tok2, i) - 1) >> chunk_shift(g.chunk_tok2, i);
  }
  const int rec = *reinterpret_cast<const int32_t*>(d + kDescRec);
  if (rec < 0 || rec > g.rec_max || chunks > g.token_slots) return r;
  r.chunks = chunks;
  r.rec = rec;
  return r;
}

// The most chunks and record bytes over the segments in use (out[0], out[1],
// zero on entry).
__global__ __launch_bounds__(256) void shape_scan_kernel(const uint8_t* cache, ShapeGeom g, int32_t* out) {
  int c = 0, r = 0;
  for (int64_t seg = int64_t(blockIdx.x) * 256 + threadIdx.x; seg < g.n_seg; seg += int64_t(gridDim.x) * 256) {
    const SegShape sh = seg_shape(cache, g, seg);
    if (sh.chunks < 0) continue;
    c = max(c, sh.chunks);
    r = max(r, sh.rec);
  }
  for (int x = 32; x >= 1; x >>= 1) {
    c = max(c, __shfl_xor(c, x, 64));
    r = max(r, __shfl_xor(r, x, 64));
  }
  if ((threadIdx.x & 63) == 0) {
    atomicMax(&out[0], c);
    atomicMax(&out[1], r);
  }
}

__global__ __launch_bounds__(64) void zero_words_kernel(int32_t* p, int n) {
  if (int(threadIdx.x) < n) p[threadIdx.x] = 0;
}

// After a decode with a shape: the outputs of every segment in use that the
// shape does not cover (more chunks or longer records than it allows, so the
// decode read it as empty) are set to NaN.
__global__ __launch_bounds__(256) void shape_check_kernel(const uint8_t* cache, ShapeGeom g, int32_t token_slots,
                                                          int32_t rec_max, float* out) {
  for (int64_t seg = blockIdx.x; seg < g.n_seg; seg += gridDim.x) {
    const SegShape sh = seg_shape(cache, g, seg);
    if (sh.chunks < 0 || (sh.chunks <= token_slots && sh.rec <= rec_max)) continue;   // (uniform)
    for (int i = threadIdx.x; i < g.group * kHeadDim; i += 256)
      out[seg * g.group * kHeadDim + i] = __builtin_nanf("");
  }
}

}  // namespace

hipError_t launch_paged_init(uint8_t* cache, const rdkv_paged_layout& pl, hipStream_t stream) {
  LaunchErrors le;
  const uint64_t n16 = pl.cache_bytes / 16;
  const unsigned grid = unsigned(std::min<uint64_t>(cdiv(n16, 256), 8192));
  hipLaunchKernelGGL(cache_zero_kernel, dim3(grid), dim3(256), 0, stream, reinterpret_cast<uint4*>(cache), n16);
  le.check();
  const unsigned tgrid = unsigned(std::min<uint64_t>(cdiv(uint64_t(pl.n_seg) * pl.max_pages, 256) + 1, 4096));
  hipLaunchKernelGGL(paged_header_kernel, dim3(tgrid), dim3(256), 0, stream, cache, pl);
  le.check();
  return le.status();
}

hipError_t launch_paged_plan(const PagedPackParams& p, hipStream_t stream) {
  const int seg_per_seq = p.play->dims.n_layers * p.play->dims.n_kv_heads;
  PagedKArgs a{p.cache, *p.play, p.staging, p.staging_bytes, p.seq, p.pages, p.pages_needed};
  hipLaunchKernelGGL(paged_plan_kernel, dim3(unsigned(cdiv(seg_per_seq, 64))), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_paged_commit(const PagedPackParams& p, hipStream_t stream) {
  const int seg_per_seq = p.play->dims.n_layers * p.play->dims.n_kv_heads;
  PagedKArgs a{p.cache, *p.play, p.staging, p.staging_bytes, p.seq, p.pages, p.pages_needed};
  hipLaunchKernelGGL(paged_commit_kernel, dim3(unsigned(seg_per_seq)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_paged_release(uint8_t* cache, const rdkv_paged_layout& pl, int32_t seq, hipStream_t stream) {
  const int seg_per_seq = pl.dims.n_layers * pl.dims.n_kv_heads;
  hipLaunchKernelGGL(paged_release_kernel, dim3(unsigned(seg_per_seq)), dim3(256), 0, stream, cache, pl, seq);
  return hipGetLastError();
}

hipError_t launch_pack_status(const uint8_t* cache, int64_t n_seg, int32_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(pack_status_kernel, dim3(1), dim3(256), 0, stream, cache, n_seg, out);
  return hipGetLastError();
}

hipError_t launch_cache_init(uint8_t* cache, const rdkv_layout& lay, const rdkv_layout* gen, hipStream_t stream) {
  LaunchErrors le;
  const uint64_t n16 = lay.cache_bytes / 16;
  const unsigned grid = unsigned(std::min<uint64_t>(cdiv(n16, 256), 8192));
  hipLaunchKernelGGL(cache_zero_kernel, dim3(grid), dim3(256), 0, stream, reinterpret_cast<uint4*>(cache), n16);
  le.check();
  const unsigned ggrid = unsigned(cdiv(lay.n_seg, 4));
  hipLaunchKernelGGL(cache_header_kernel, dim3(ggrid), dim3(256), 0, stream, cache, lay, geom_of(lay));
  le.check();
  // every generation blob starts as an empty blob of its own layout
  for (int g = 0; gen && g < lay.n_generations; ++g) {
    hipLaunchKernelGGL(cache_header_kernel, dim3(ggrid), dim3(256), 0, stream, cache + lay.gen_offset + g * lay.gen_bytes,
                       *gen, geom_of(*gen));
    le.check();
  }
  return le.status();
}

hipError_t launch_pack(const PackParams& p, hipStream_t stream) {
  LaunchErrors le;
  const rdkv_layout& lay = *p.lay;
  const int64_t n_seg_in = int64_t(lay.dims.n_seq) * p.n_layers_in * lay.dims.n_kv_heads;
  IndexArgs ia{p.cache, geom_of(lay), lay.dims.n_layers, lay.dims.n_kv_heads, p.layer_begin, p.n_layers_in,
               p.bits_tok, p.bits_chan};
  hipLaunchKernelGGL(pack_index_kernel, dim3(unsigned(n_seg_in)), dim3(kIndexThreads), 0, stream, ia);
  le.check();
  RowsArgs ra{p.cache, geom_of(lay), lay.dims.n_layers, lay.dims.n_kv_heads, p.layer_begin, p.n_layers_in, p.K, p.V};
  hipLaunchKernelGGL(pack_rows_kernel, dim3(kRowsWgPerSeg, unsigned(n_seg_in)), dim3(kRowsThreads), 0, stream, ra);
  le.check();
  return le.status();
}

hipError_t launch_unpack(const uint8_t* cache, uint64_t, const rdkv_layout& lay, int64_t seg, float* k_hat,
                         float* v_hat, hipStream_t stream) {
  (void)lay;
  UnpackArgs ua{cache, seg, k_hat, v_hat};
  hipLaunchKernelGGL(unpack_kernel, dim3(64), dim3(256), 0, stream, ua);
  return hipGetLastError();
}

hipError_t launch_shape_scan(const uint8_t* cache, const ShapeGeom& g, int32_t* out, hipStream_t stream) {
  LaunchErrors le;
  hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(64), 0, stream, out, 2);
  le.check();
  const unsigned grid = unsigned(std::min<int64_t>(cdiv(g.n_seg, 256), 1024));
  hipLaunchKernelGGL(shape_scan_kernel, dim3(grid), dim3(256), 0, stream, cache, g, out);
  le.check();
  return le.status();
}

hipError_t launch_shape_check(const uint8_t* cache, const ShapeGeom& g, int32_t token_slots, int32_t rec_max,
                              float* out, hipStream_t stream) {
  const unsigned grid = unsigned(std::min<int64_t>(g.n_seg, 4096));
  hipLaunchKernelGGL(shape_check_kernel, dim3(grid), dim3(256), 0, stream, cache, g, token_slots, rec_max, out);
  return hipGetLastError();
}

}  // namespace rdkv
