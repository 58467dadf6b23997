// Fused split-K decode attention over the packed cache (RDKV summary, section
// 2.3: dequantization fused into the logit and output products over zones A,
// B and C; section 1: decode rereads the whole cache every step).
//
// decode_chunk_kernel: one 256-thread workgroup per (segment, chunk).  A chunk
// is chunk_tok2 >> g tokens of V group g (equal V bytes per chunk) or up to
// 256 zone-C rows.  Each wave walks 64-token tiles of the chunk:
//   * K records: each tile's records are one contiguous block, copied by
//     global_load_lds (no registers) into a per-wave ring of LDS stages two
//     tiles ahead; the wave waits on the memory counter for the stage it
//     reads;
//   * logits, lane = token: per bit-part of the record, code pairs (two
//     channels of one word, fp16 subnormals code * 2^-24) meet the matching
//     fp16 query pairs in v_dot2_f32_f16; each part's scale and zero are
//     factored out: q.(s*code + z) = s*(q.code) + z*sum(q); 0-bit channels are
//     absent;
//   * online softmax: the running max moves (with a DPP wave reduction) only
//     when some lane's logit exceeds it; fp16 p*scale per token goes to LDS;
//   * values, lane = (8-channel block, token slot): a register holds the
//     lane's channels of two tokens (j, j + 32) in its two halves, masked in
//     place into fp16 subnormals and met with the fp16 (p*scale) pair in
//     v_dot2; the p*zero part is summed once per token.  2- and 4-bit rows
//     are loaded one tile ahead.
// With 8 query heads per KV head, pairs of waves walk the same tiles for the
// two halves of the heads.  The waves' partials are merged in LDS into one
// (m, l, o[128]) per query head and chunk; decode_merge_kernel combines each
// segment's chunks in chunk order, so the result does not depend on
// scheduling.  Merging in a second
// launch keeps the chunk kernel free of device-wide fences, which on a
// multi-XCD part write back and invalidate the L2.  No MFMA: 1..8 query rows
// per KV head make this a matrix-vector stream, bounded by HBM bandwidth and
// VALU issue.
#include <type_traits>

#include "lds_dma.h"
#include "rdkv_internal.h"

namespace rdkv {
namespace {

using dma::buffer_rsrc;
using dma::buffer_rsrc4;
using dma::lds_addr;
using dma::rsrc4;
using dma::wait_vmem;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// Query heads a wave carries.  With 8 heads per KV head the waves split them:
// waves w and w + 2 walk the same tiles for heads 0-3 and 4-7, so a wave keeps
// the 4-head register footprint (accumulators, coefficients) of the smaller
// groups instead of spilling.
template <int G> constexpr int kHeadsPerWave = G > 4 ? 4 : G;
// Tile streams of a workgroup: waves with the same stream index walk the same tiles.
template <int G> constexpr int kStreams = kWaves / (G / kHeadsPerWave<G>);
constexpr int kTile = 64;
// Paged decode: the most tiles one wave walks in a chunk, and whether its tile
// offsets go through LDS (more than 64: one list per tile stream, [stream][V,
// records][tile], which the two waves of a stream write alike) instead of a
// register per lane.
template <int G> constexpr int kWaveTilesMax = kChunkTok2Max / kTile / kStreams<G>;
template <int G, bool kPaged> constexpr bool kPgLds = kPaged && (kWaveTilesMax<G> > 64);
template <int G, bool kPaged>
constexpr int kPgLdsWords = kPgLds<G, kPaged> ? kStreams<G> * 2 * kWaveTilesMax<G> : 1;
constexpr float kLog2eOverSqrtD = 1.4426950408889634f / 11.313708498984761f;
constexpr float kTwo24 = 16777216.0f;   // codes enter dot2 as fp16 subnormals code * 2^-24
constexpr int kPairSlots = 80;          // >= w16 + 2*w8 + 4*w4 + 8*w2 for any split of 128 channels
constexpr int kMaxStagedWords = 32;     // longer K records are read from global directly

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

// The wave's index in the workgroup, as a wave-uniform (scalar) value.
__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6); }

__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, a), __builtin_bit_cast(half2v, b), c, false);
}
// (byte k of lo) in bits 0-7 and (byte k of hi) in bits 16-23, zeros elsewhere
__device__ inline uint32_t pair_bytes(uint32_t lo, uint32_t hi, int k) {
  return __builtin_amdgcn_perm(hi, lo, uint32_t(k) | 0x0c00u | (uint32_t(4 + k) << 16) | 0x0c000000u);
}
// (half h of lo) in bits 0-15 and (half h of hi) in bits 16-31
__device__ inline uint32_t pair_halves(uint32_t lo, uint32_t hi, int h) {
  return h == 0 ? __builtin_amdgcn_perm(hi, lo, 0x05040100u) : __builtin_amdgcn_perm(hi, lo, 0x07060302u);
}

// ---------------------------------------------------------------- segment and chunk

struct SegInfo {
  int n_tok[4];
  int n_chan[4];
  int rec_a;        // words of a zone-A record
  uint64_t off_v[4], off_krec, off_kc, off_vc;   // from the cache base
  uint64_t desc;                                 // offset of the segment's descriptor
  bool zc_ok;
  // paged cache: the segment's block-table row and each region's first virtual page
  const int32_t* table;
  int vpage[kRegions];
};

// One blob inside the cache: the prefill generation (base 0) or a rolled-over
// generation blob.  Its descriptors' offsets are relative to its own base.
struct BlobRef {
  uint64_t base, bytes;
  int64_t nk_max;
  int rec_max, chunk_tok2, token_slots;
};

__device__ inline BlobRef main_blob(const DecodeParams& p) {
  return BlobRef{0, p.main_bytes, p.nk_max, p.rec_max, p.chunk_tok2, p.token_slots};
}
__device__ inline BlobRef gen_blob(const DecodeParams& p, int g) {
  return BlobRef{p.gen_offset + uint64_t(g) * p.gen_bytes, p.gen_cache_bytes, p.gen_nk_max, p.gen_rec_max,
                 p.gen_chunk_tok2, p.gen_slots};
}

// Reads a descriptor and treats anything inconsistent with the layout as an
// empty segment, so a damaged blob can never drive reads out of bounds.
// n_c: zone-C rows to check room for (prefill generation only).
__device__ inline SegInfo load_segment(const DecodeParams& p, const BlobRef& b, int64_t seg, int n_c) {
  const uint8_t* d = p.cache + b.base + kHeaderBytes + uint64_t(seg) * kDescBytes;
  SegInfo s;
  s.desc = b.base + kHeaderBytes + uint64_t(seg) * kDescBytes;
  s.table = nullptr;
#pragma unroll
  for (int r = 0; r < kRegions; ++r) s.vpage[r] = 0;
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
  ok = ok && n_kept == n_kept_sum && n_kept <= b.nk_max && n_chan_sum <= kHeadDim && rec == 4 * rs.words_a() &&
       rec <= b.rec_max;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    ok = ok && s.off_v[i] + uint64_t(s.n_tok[i]) * (kHeadDim * group_bits(i) / 8) <= b.bytes;
  ok = ok && s.off_krec + uint64_t(n_kept) * rec <= b.bytes;
  // the layout sized the chunk slots for sum_g n_g 2^g <= min(B_V / 2, 8 N); a
  // descriptor with more chunks than its slots would leave chunks unlaunched
  int n_chunks = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int T = chunk_tokens(b.chunk_tok2, i);
    n_chunks += (max(s.n_tok[i], 0) + T - 1) >> chunk_shift(b.chunk_tok2, i);
  }
  ok = ok && n_chunks <= b.token_slots;
  if (!ok) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s.n_tok[i] = s.n_chan[i] = 0;
  }
  s.rec_a = ok ? rec / 4 : 1;
  s.zc_ok = s.off_vc + uint64_t(n_c) * kHeadDim * 2 <= b.bytes && s.off_kc + uint64_t(n_c) * kHeadDim * 2 <= b.bytes;
#pragma unroll
  for (int i = 0; i < 4; ++i) s.off_v[i] += b.base;
  s.off_krec += b.base;
  s.off_kc += b.base;
  s.off_vc += b.base;
  return s;
}

// Blob offset of tile `tile` of a paged segment's region that starts at
// virtual page vp0 (tpp tiles of tile_bytes per page).  An entry outside the
// block table or the pool gives page 0 and ok = false: callers then read
// nothing through it.
__device__ inline uint64_t paged_tile(const DecodeParams& p, const int32_t* table, int vp0, int tile, uint32_t tpp,
                                      uint32_t tile_bytes, bool& ok) {
  const int vp = vp0 + int(uint32_t(tile) / tpp);
  const int phys = (vp >= 0 && vp < p.max_pages) ? table[vp] : -1;
  ok = phys >= 0 && phys < p.pool_pages;
  return p.pool_offset + uint64_t(ok ? phys : 0) * kPageBytes + uint64_t(uint32_t(tile) % tpp) * tile_bytes;
}

// The same offset in 256-byte units (every tile of a paged cache starts on a
// 256-byte boundary and the cache is below 2^40 bytes, so it fits 32 bits);
// kNoPage for an entry outside the block table or the pool.
constexpr uint32_t kNoPage = 0xffffffffu;
__device__ inline uint32_t paged_tile_units(const DecodeParams& p, const int32_t* table, int vp0, uint32_t tile,
                                            uint32_t tpp, uint32_t tile_bytes) {
  const int vp = vp0 + int(tile / tpp);
  const int phys = (vp >= 0 && vp < p.max_pages) ? table[vp] : -1;
  if (phys < 0 || phys >= p.pool_pages) return kNoPage;
  return uint32_t((p.pool_offset + uint64_t(phys) * kPageBytes + uint64_t(tile % tpp) * tile_bytes) >> 8);
}

// A paged segment's descriptor (the contiguous fields' meaning for counts,
// then the regions' first virtual pages).  Anything inconsistent with the
// layout, or a free slot, reads as an empty segment.  n_c: zone-C rows this
// step attends; their pages must be in the pool.
__device__ inline SegInfo load_segment_paged(const DecodeParams& p, int64_t seg, int n_c) {
  const uint8_t* d = p.cache + kHeaderBytes + uint64_t(seg) * kDescBytes;
  SegInfo s;
  s.desc = kHeaderBytes + uint64_t(seg) * kDescBytes;
  s.table = reinterpret_cast<const int32_t*>(p.cache + p.table_offset) + seg * p.max_pages;
  int n_kept_sum = 0, n_chan_sum = 0;
  bool ok = true;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s.n_tok[i] = *reinterpret_cast<const int32_t*>(d + kDescNTok + 4 * i);
    s.n_chan[i] = *reinterpret_cast<const int32_t*>(d + kDescNChan + 4 * i);
    ok = ok && s.n_tok[i] >= 0 && s.n_chan[i] >= 0;
    n_kept_sum += s.n_tok[i];
    n_chan_sum += s.n_chan[i];
  }
  const int n_kept = *reinterpret_cast<const int32_t*>(d + kDescNKept);
  const int rec = *reinterpret_cast<const int32_t*>(d + kDescRec);
  const int cap = *reinterpret_cast<const int32_t*>(d + kDescCap);
  const int n_pages = *reinterpret_cast<const int32_t*>(d + kPDescNPages);
  const RecordShape rs = record_shape(s.n_chan[0], s.n_chan[1], s.n_chan[2], s.n_chan[3]);
  ok = ok && cap == p.zc_cap && n_kept == n_kept_sum && n_kept <= p.nk_max && n_chan_sum <= kHeadDim &&
       rec == 4 * rs.words_a() && rec <= p.rec_max && n_pages >= 0 && n_pages <= p.max_pages;
  const int rows[kRegions] = {s.n_tok[0], s.n_tok[1], s.n_tok[2], s.n_tok[3], s.n_tok[0], s.n_tok[1], s.n_tok[2],
                              s.n_tok[3], cap, cap, n_kept};
#pragma unroll
  for (int r = 0; r < kRegions; ++r) {
    s.vpage[r] = *reinterpret_cast<const int32_t*>(d + kPDescVpage + 4 * r);
    ok = ok && s.vpage[r] >= 0 && s.vpage[r] + paged_region_pages(rows[r], paged_tile_bytes(r, rec)) <= n_pages;
  }
  int n_chunks = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int T = chunk_tokens(p.chunk_tok2, i);
    n_chunks += (max(s.n_tok[i], 0) + T - 1) >> chunk_shift(p.chunk_tok2, i);
  }
  ok = ok && n_chunks <= p.token_slots;
  if (!ok) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s.n_tok[i] = s.n_chan[i] = 0;
  }
  s.rec_a = ok ? rec / 4 : 1;
  // the zone-C pages this step touches (at most a few)
  bool zc = ok && n_c <= cap;
  const int zc_pages = paged_region_pages(n_c, paged_tile_bytes(kRegKC, 0));
  for (int t = 0; zc && t < zc_pages; ++t) {
    const int a = s.table[s.vpage[kRegKC] + t], b = s.table[s.vpage[kRegVC] + t];
    zc = a >= 0 && a < p.pool_pages && b >= 0 && b < p.pool_pages;
  }
  s.zc_ok = zc;
#pragma unroll
  for (int i = 0; i < 4; ++i) s.off_v[i] = 0;
  s.off_krec = s.off_kc = s.off_vc = 0;
  return s;
}

struct Plan {
  int kind;          // 0..3 token group, 4 zone C, -1 none
  int start, end;    // rows of the group (or zone C) in this chunk
  uint64_t vbase;    // blob offset of the group's first V row (or of V_C)
  int64_t rec0;      // word offset of the group's first K record from off_krec
  int rec_words;     // words per record in this group
  int vp_a, vp_b;    // paged: first virtual page of the group's V rows and K records (or of K_C and V_C)
};

// Chunk k of a segment's kept tokens: groups 2, 4, 8, 16 bits in turn, each
// cut into chunks of chunk_tok2 >> g tokens; kind -1 past the last one.
__device__ inline Plan plan_tokens(const SegInfo& si, int chunk_tok2, int k) {
  Plan pl{-1, 0, 0, 0, 0, 0, 0, 0};
  int kept = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int T = chunk_tokens(chunk_tok2, g);
    const int nch = (si.n_tok[g] + T - 1) >> chunk_shift(chunk_tok2, g);
    if (pl.kind < 0) {
      if (k < nch) {
        pl.kind = g;
        pl.start = k * T;
        pl.end = min(si.n_tok[g], (k + 1) * T);
        pl.vbase = si.off_v[g];
        // zone-A records come first; the fp16 group's shorter records follow them
        pl.rec0 = int64_t(kept) * si.rec_a;
        pl.rec_words = g < 3 ? si.rec_a : si.rec_a - 1;
        pl.vp_a = si.vpage[kRegV + g];
        pl.vp_b = si.vpage[kRegRec + g];
      } else {
        k -= nch;
      }
    }
    kept += si.n_tok[g];
  }
  return pl;
}

// Zone-C chunk k: rows [256 k, min(n_c, 256 (k + 1))); kind -1 past the last.
__device__ inline Plan plan_zone_c(const SegInfo& si, int n_c, int k) {
  Plan pl{-1, 0, 0, 0, 0, 0, si.vpage[kRegKC], si.vpage[kRegVC]};
  const int nch = (n_c + kChunkRowsC - 1) / kChunkRowsC;
  if (k < nch) {
    pl.kind = 4;
    pl.start = k * kChunkRowsC;
    pl.end = min(n_c, (k + 1) * kChunkRowsC);
    pl.vbase = si.off_vc;
  }
  return pl;
}

// ---------------------------------------------------------------- shared memory

// LDS ring of K-record stages per wave.  A stage holds a tile's record block
// copied in 16-byte chunks from the 16-byte-aligned address at or below its
// start (up to 3 words before it): stage_copies 1-KiB copies of 64 lanes.
// Three stages (two tiles in flight) while that stays within 9 KiB per wave,
// else two (one in flight).
template <int SW>
__host__ __device__ constexpr int stage_copies() { return (kTile * SW + 3 + 255) / 256; }
template <int SW>
__host__ __device__ constexpr int stage_words() { return stage_copies<SW>() * 256; }
template <int SW>
__host__ __device__ constexpr int ring_stages() { return SW == 0 ? 0 : 3 * stage_words<SW>() <= 2304 ? 3 : 2; }

// Per wave, the record ring and, once the wave's last tile is done, its
// partial output share one region.
template <int GW, int SW>
union __align__(16) WaveLds {
  uint32_t ring[SW > 0 ? ring_stages<SW>() * stage_words<SW>() : 1];
  float o[GW][kHeadDim];
};

template <int G, int SW>
struct __align__(16) Smem {
  uint32_t qpair[kPairSlots][G];         // fp16 query pairs matching the records' code pairs
  float qsum[4][G];                      // sum of q over the 8-, 4-, 2-bit channel parts
  uint8_t perm[kHeadDim];                // record order -> channel
  // the query copy lives only while the tables are built; the tiles' fp16
  // (p*scale) coefficients of tokens (j, j + 32) take its place after it
  union {
    uint16_t qnat[G][kHeadDim];          // query as given
    uint32_t coefh[kWaves][kTile / 2][kHeadsPerWave<G>];
  };
  WaveLds<kHeadsPerWave<G>, SW> wv[kWaves];
  float part_ml[kWaves][kHeadsPerWave<G>][2];
};

// The query pairs of heads hb .. hb + GW - 1 for one pair slot.
template <int GW, int G, int SW>
__device__ inline void load_qp(const Smem<G, SW>& sm, int slot, int hb, uint32_t (&q)[GW]) {
  if constexpr (GW == 4) {
    const uint4 t = *reinterpret_cast<const uint4*>(&sm.qpair[slot][hb]);
    q[0] = t.x, q[1] = t.y, q[2] = t.z, q[3] = t.w;
  } else if constexpr (GW == 2) {
    const uint2 t = *reinterpret_cast<const uint2*>(&sm.qpair[slot][hb]);
    q[0] = t.x, q[1] = t.y;
  } else {
    q[0] = sm.qpair[slot][hb];
  }
}

// The segment's G query rows and its channel permutation (at byte offset
// `desc` + kDescPerm of the cache), copied to LDS as the workgroup starts:
// these reads need nothing from the descriptor, so they overlap its reads
// instead of following them.  Word loads (device pointers are 16-byte
// aligned); build_query_tables reads the copies after a barrier.
template <int G, int SW>
__device__ inline void stage_query(const DecodeParams& p, int64_t seg, uint64_t desc, Smem<G, SW>& sm) {
  constexpr int kWords = G * kHeadDim / 2;
  const uint32_t* q32 = reinterpret_cast<const uint32_t*>(p.q) + seg * kWords;
  uint32_t* qn = reinterpret_cast<uint32_t*>(&sm.qnat[0][0]);
  for (int i = threadIdx.x; i < kWords; i += kThreads) qn[i] = q32[i];
  if (threadIdx.x < kHeadDim / 4)
    reinterpret_cast<uint32_t*>(sm.perm)[threadIdx.x] =
        reinterpret_cast<const uint32_t*>(p.cache + desc + kDescPerm)[threadIdx.x];
}

// fp16 query pairs in the order the rows' code pairs come in, and the sum of
// q over each integer part (for the zero terms), from the copies stage_query
// made.  Zone C uses natural order.  The part sums are wave reductions.
template <int G, int SW>
__device__ void build_query_tables(const SegInfo& si, const Plan& pl, Smem<G, SW>& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const RecordShape rs = record_shape(si.n_chan[0], si.n_chan[1], si.n_chan[2], si.n_chan[3]);
  const int c8 = si.n_chan[0], c4 = c8 + si.n_chan[1], c2 = c4 + si.n_chan[2], c0 = c2 + si.n_chan[3];
  const bool natural = pl.kind == 4;
  // q_g at record position pos (a permutation entry past the head dimension,
  // possible only in a damaged descriptor, is wrapped into it)
  auto qat = [&](int g, int pos) -> uint16_t { return sm.qnat[g][natural ? pos : sm.perm[pos] & (kHeadDim - 1)]; };
  __syncthreads();
  for (int i = tid; i < kPairSlots * G; i += kThreads) {
    const int sl = i / G, g = i % G;
    int pa, pb, hi_end;   // permuted channel positions of the pair
    int shift = 0;        // log2 of the in-place position scale of the slot's codes
    if (natural) {
      pa = 2 * sl, pb = 2 * sl + 1, hi_end = kHeadDim;
    } else if (sl < rs.w16) {
      pa = 2 * sl, pb = 2 * sl + 1, hi_end = c8;
    } else if (sl < rs.w16 + 2 * rs.w8) {
      const int t = sl - rs.w16;
      pa = c8 + 4 * (t >> 1) + (t & 1), pb = pa + 2, hi_end = c4;
    } else if (sl < rs.w16 + 2 * rs.w8 + 4 * rs.w4) {
      const int t = sl - rs.w16 - 2 * rs.w8;
      pa = c4 + 8 * (t >> 2) + (t & 3), pb = pa + 4, hi_end = c2;
      shift = 4 * (t & 1);
    } else {
      const int t = sl - rs.w16 - 2 * rs.w8 - 4 * rs.w4;
      pa = c2 + 16 * (t >> 3) + (t & 7), pb = pa + 8, hi_end = c0;
      shift = 2 * (t & 3);
    }
    // the slot's codes reach dot2 as code * 2^shift (masked in place), so the
    // query is stored divided by 2^shift (exact unless it becomes subnormal)
    auto qbits = [&](int pos) -> uint32_t {
      if (pos >= hi_end || pos >= kHeadDim) return 0u;
      const uint16_t h = qat(g, pos);
      if (shift == 0) return h;
      return __half_as_ushort(__float2half_rn(ldexpf(__half2float(__ushort_as_half(h)), -shift)));
    };
    sm.qpair[sl][g] = qbits(pa) | (qbits(pb) << 16);
  }
  if (!natural) {
    for (int i = wave; i < 3 * G; i += kWaves) {
      const int j = i / G, g = i % G;
      const int lo = j == 0 ? c8 : j == 1 ? c4 : c2;
      const int hi = j == 0 ? c4 : j == 1 ? c2 : c0;
      float v = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = lane + 64 * h;
        if (c >= lo && c < hi) v += __half2float(__ushort_as_half(qat(g, c)));
      }
      v = wave_reduce<false>(v);
      if (lane == 0) sm.qsum[j][g] = v;
    }
  }
}

// Word counts of a segment's K record as the logit loop walks it.
struct QkShape {
  int w16;        // fp16 words
  int words[3];   // words of the 8-, 4-, 2-bit parts
  int tail[3];    // pair slots the part's last word fills (a word of a b-bit part holds 32/b
                  // channels as 16/b pairs (e, e + 16/b))
  int meta;       // index of the first scale/zero word
};

__device__ inline QkShape qk_shape(const SegInfo& si) {
  const RecordShape rs = record_shape(si.n_chan[0], si.n_chan[1], si.n_chan[2], si.n_chan[3]);
  QkShape k;
  k.w16 = rs.w16;
  k.words[0] = rs.w8, k.words[1] = rs.w4, k.words[2] = rs.w2;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int pairs = 2 << i;   // pair slots per word
    k.tail[i] = k.words[i] > 0 ? min(pairs, si.n_chan[i + 1] - (k.words[i] - 1) * 2 * pairs) : 0;
  }
  k.meta = rs.w16 + rs.w8 + rs.w4 + rs.w2;
  return k;
}

// d[g] += q_g . codes over one integer part (P pair slots per word).  Slots
// past the part's last channel are skipped; their table entries stay unread.
// A word's pair e = (channel e, channel e + P) sits at bits kBits*e of both
// halves; the first P/2 pairs are masked in place, the rest after one shift
// by 8, so a code arrives as code * 2^(kBits * (e mod P/2)) * 2^-24, which the
// query table has divided out.
template <int GW, int G, int SW, int P>
__device__ inline void int_part(const uint32_t* rec, int& w, int& sl, int words, int tail, const Smem<G, SW>& sm,
                                int hb, float (&d)[GW]) {
  constexpr int kBits = 16 / P;
  constexpr uint32_t kMask = ((1u << kBits) - 1u) * 0x00010001u;
  uint32_t q[GW];
  auto slot = [&](uint32_t x, int e) {
    load_qp<GW>(sm, sl + e, hb, q);
    const int half = e >= P / 2;
    const uint32_t pr = (half ? x >> 8 : x) & (kMask << (kBits * (e - half * (P / 2))));
#pragma unroll
    for (int g = 0; g < GW; ++g) d[g] = dot2(pr, q[g], d[g]);
  };
  // full words without per-slot tests, then the last word's `tail` slots
  for (int j = 0; j + 1 < words; ++j, ++w, sl += P) {
    const uint32_t x = rec[w];
#pragma unroll
    for (int e = 0; e < P; ++e) slot(x, e);
  }
  const uint32_t x = rec[w++];
#pragma unroll
  for (int e = 0; e < P; ++e)
    if (e < tail) slot(x, e);
  sl += P;
}

// s[g] = q_g . k_hat for one token whose record words are rec[0..).  The
// record may live in LDS (staged) or in global memory.
template <int GW, int G, int SW>
__device__ inline void record_logits(const uint32_t* rec, const QkShape& ks, int nw, bool has_vmeta,
                                     const Smem<G, SW>& sm, int hb, float (&s)[GW], float& vs, float& vz) {
  uint32_t q[GW];
#pragma unroll
  for (int g = 0; g < GW; ++g) s[g] = 0.f;
  int w = 0, sl = 0, mo = ks.meta;
  for (; w < ks.w16; ++w, ++sl) {
    const uint32_t x = rec[w];
    load_qp<GW>(sm, sl, hb, q);
#pragma unroll
    for (int g = 0; g < GW; ++g) s[g] = dot2(x, q[g], s[g]);
  }
  auto part = [&](auto pairs, int i) {
    if (ks.words[i] == 0) return;
    float d[GW];
#pragma unroll
    for (int g = 0; g < GW; ++g) d[g] = 0.f;
    int_part<GW, G, SW, decltype(pairs)::value>(rec, w, sl, ks.words[i], ks.tail[i], sm, hb, d);
    const uint32_t m = rec[mo++];
    const float sc = half_lo(m) * kTwo24, z = half_hi(m);
#pragma unroll
    for (int g = 0; g < GW; ++g) s[g] = fmaf(sc, d[g], fmaf(z, sm.qsum[i][hb + g], s[g]));
  };
  part(std::integral_constant<int, 2>{}, 0);
  part(std::integral_constant<int, 4>{}, 1);
  part(std::integral_constant<int, 8>{}, 2);
  vs = 1.f;
  vz = 0.f;
  if (has_vmeta) {
    const uint32_t m = rec[nw - 1];
    vs = half_lo(m);
    vz = half_hi(m);
  }
}

// ---------------------------------------------------------------- value rows

// PV lane layout: lane = 16 * ts + cb holds channels 8cb .. 8cb+7 and token
// slot ts; a tile's 32 token pairs (j, j + 32) go to slots j mod 4.
constexpr int kPairsPerLane = kTile / 2 / 4;

// The lane's channels of tokens (j, j + 32) of one V group, as loaded.
template <int B> struct VPair;
template <> struct VPair<2> { uint32_t a, b; };      // the dword holding the lane's 16 bits of each
                                                     // token (the half is picked at use)
template <> struct VPair<4> { uint32_t a, b; };      // 32 bits per token
template <> struct VPair<8> { uint2 a, b; };         // 64 bits per token
template <> struct VPair<16> { uint4 a, b; };        // 8 fp16 per token

// Byte offset, within a V row of B-bit codes, of what lane block cb loads.
template <int B>
__device__ constexpr int lane_row_offset(int cb) {
  return B == 2 ? (cb >> 1) * 4 : cb * (kHeadDim * B / 8 / 16);
}

// Tokens (j, j + 32) from a buffer whose range starts at the tile's first row:
// the lane's parts of the rows at byte offsets off0 and off1.
template <int B>
__device__ inline VPair<B> load_vpair_buf(__amdgpu_buffer_rsrc_t r, uint32_t off0, uint32_t off1) {
  VPair<B> v;
  if constexpr (B <= 4) {
    v.a = __builtin_amdgcn_raw_buffer_load_b32(r, off0, 0, 0);
    v.b = __builtin_amdgcn_raw_buffer_load_b32(r, off1, 0, 0);
  } else if constexpr (B == 8) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b64(r, off0, 0, 0);
    const auto y = __builtin_amdgcn_raw_buffer_load_b64(r, off1, 0, 0);
    v.a = make_uint2(x[0], x[1]);
    v.b = make_uint2(y[0], y[1]);
  } else {
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, off0, 0, 0);
    const auto y = __builtin_amdgcn_raw_buffer_load_b128(r, off1, 0, 0);
    v.a = make_uint4(x[0], x[1], x[2], x[3]);
    v.b = make_uint4(y[0], y[1], y[2], y[3]);
  }
  return v;
}

// Zone C: fp16 rows through plain pointers.
__device__ inline VPair<16> load_vpair16(const uint8_t* row0, const uint8_t* row1, int cb) {
  VPair<16> v;
  v.a = reinterpret_cast<const uint4*>(row0)[cb];
  v.b = reinterpret_cast<const uint4*>(row1)[cb];
  return v;
}

// Scale that turns channel e's accumulator into p*code units: codes enter
// dot2 as subnormals code * 2^-24, shifted left by their in-place position.
// A 2-bit code must stay below bit 10 (the fp16 exponent field): channels
// 5..7 of the 16-bit lane part are shifted down by 10 first.
template <int B>
__device__ constexpr float channel_scale(int e) {
  if constexpr (B == 2) return kTwo24 / float(1 << (2 * (e < 5 ? e : e - 5)));
  if constexpr (B == 4) return (e & 1) ? kTwo24 / 16.0f : kTwo24;
  if constexpr (B == 8) return kTwo24;
  return 1.0f;
}

// acc[g][e] += dot2((x_t0[e], x_t1[e]), (c_t0[g], c_t1[g])) for the lane's 8
// channels (see channel_scale for the in-place code positions).  sel2 picks
// the lane's halves of the two 2-bit dwords.
template <int G, int B>
__device__ inline void pv_pair(float (&acc)[G][8], const VPair<B>& v, const uint32_t (&cf)[G], uint32_t sel2) {
  auto fma_e = [&](int e, uint32_t pr) {
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g][e] = dot2(pr, cf[g], acc[g][e]);
  };
  if constexpr (B == 2) {
    const uint32_t w = __builtin_amdgcn_perm(v.b, v.a, sel2);   // t0 in the low half, t1 in the high half
    const uint32_t hi = w >> 10;
#pragma unroll
    for (int e = 0; e < 5; ++e) fma_e(e, w & (0x00030003u << (2 * e)));
#pragma unroll
    for (int e = 5; e < 8; ++e) fma_e(e, hi & (0x00030003u << (2 * (e - 5))));
  } else if constexpr (B == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t t = pair_bytes(v.a, v.b, k);
      fma_e(2 * k, t & 0x000F000Fu);
      fma_e(2 * k + 1, t & 0x00F000F0u);
    }
  } else if constexpr (B == 8) {
    const uint32_t a[2] = {v.a.x, v.a.y}, b[2] = {v.b.x, v.b.y};
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int k = 0; k < 4; ++k) fma_e(4 * d + k, pair_bytes(a[d], b[d], k));
  } else {
    const uint32_t a[4] = {v.a.x, v.a.y, v.a.z, v.a.w}, b[4] = {v.b.x, v.b.y, v.b.z, v.b.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      fma_e(2 * d, pair_halves(a[d], b[d], 0));
      fma_e(2 * d + 1, pair_halves(a[d], b[d], 1));
    }
  }
}

// ---------------------------------------------------------------- per-wave state

template <int G>
struct WaveState {
  float m[G], l[G], z[G], acc[G][8];
};

template <int G>
__device__ inline void state_init(WaveState<G>& st) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    st.m[g] = -INFINITY;
    st.l[g] = 0.f;
    st.z[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.acc[g][e] = 0.f;
  }
}

// Online softmax update for one tile (lane = token).  The running max m (log2
// units, wave-uniform) is a reference, not necessarily the maximum: the
// partial (m, l, o) is exact for any m, so it is raised, with the sums
// rescaled, only when some lane's p = 2^(t - m) would pass kLazy or its fp16
// coefficient p*vs would overflow (and on the first tile, where m = -inf).
// A tile in which a logit merely exceeds m (more than one in four tiles of a
// long chunk) then costs no wave reduction.  Writes fp16 p*vs per token to LDS.
template <int GW, int G, int SW, bool kMasked>
__device__ inline void softmax_tile(WaveState<GW>& st, const float (&s)[GW], bool valid, float vs, float vz,
                                    Smem<G, SW>& sm, int wave, int lane) {
  constexpr float kLazy = 16.f;
  float t[GW], pr[GW], c[GW];
#pragma unroll
  for (int g = 0; g < GW; ++g) {
    t[g] = (!kMasked || valid) ? s[g] * kLog2eOverSqrtD : -INFINITY;
    pr[g] = __builtin_amdgcn_exp2f(t[g] - st.m[g]);
    c[g] = pr[g] * vs;
  }
  // one wave-uniform branch per tile, rescaling every head (a head whose
  // logits stay below its m keeps it: alpha = 1); masked lanes of the first
  // tile give p = NaN here, which passes no test, and 0 once m is finite
  bool up = false;
#pragma unroll
  for (int g = 0; g < GW; ++g) up = up || pr[g] > kLazy || c[g] > 65504.f;
  if (__builtin_amdgcn_ballot_w64(up) != 0) {
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      const float mnew = fmaxf(st.m[g], wave_reduce<true>(t[g]));
      const float alpha = __builtin_amdgcn_exp2f(st.m[g] - mnew);
      st.m[g] = mnew;
      st.l[g] *= alpha;
      st.z[g] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) st.acc[g][e] *= alpha;
      pr[g] = __builtin_amdgcn_exp2f(t[g] - mnew);
      c[g] = pr[g] * vs;
    }
  }
#pragma unroll
  for (int g = 0; g < GW; ++g) {
    st.l[g] += pr[g];
    st.z[g] = fmaf(pr[g], vz, st.z[g]);
    reinterpret_cast<uint16_t*>(&sm.coefh[wave][lane & 31][g])[lane >> 5] = __half_as_ushort(__float2half_rn(c[g]));
  }
}

template <int GW, int G, int SW>
__device__ inline void load_coefs(const Smem<G, SW>& sm, int wave, int j, uint32_t (&cf)[GW]) {
  if constexpr (GW == 4) {
    const uint4 t = *reinterpret_cast<const uint4*>(&sm.coefh[wave][j][0]);
    cf[0] = t.x, cf[1] = t.y, cf[2] = t.z, cf[3] = t.w;
  } else {
#pragma unroll
    for (int g = 0; g < GW; ++g) cf[g] = sm.coefh[wave][j][g];
  }
}

// Wave partial (m, l, o) into LDS.  acc is summed over the 4 token slots
// (lanes cb, cb + 16, cb + 32, cb + 48) by two rounds of lane-half swaps:
// v_permlane32_swap pairs values (2j, 2j + 1) into one register holding
// their lane-32 sums in its two halves, v_permlane16_swap pairs those again,
// so quarter q of register k ends up with value 4k + {0, 2, 1, 3}[q] of the
// flat index 8g + e.
template <int GW, int B, int G, int SW>
__device__ inline void wave_finish(WaveState<GW>& st, Smem<G, SW>& sm, int wave, int lane) {
  const int cb = lane & 15, qr = lane >> 4;
#pragma unroll
  for (int g = 0; g < GW; ++g) {
    st.l[g] = wave_reduce<false>(st.l[g]);
    st.z[g] = wave_reduce<false>(st.z[g]);
  }
  constexpr int kN = 8 * GW;
  float u[kN / 2];
#pragma unroll
  for (int j = 0; j < kN / 2; ++j) {
    const float v0 = st.acc[(2 * j) / 8][(2 * j) % 8], v1 = st.acc[(2 * j + 1) / 8][(2 * j + 1) % 8];
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v0), __float_as_uint(v1), false, false);
    u[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const int sel = ((qr & 1) << 1) | (qr >> 1);
#pragma unroll
  for (int k = 0; k < kN / 4; ++k) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(u[2 * k]), __float_as_uint(u[2 * k + 1]), false,
                                                    false);
    const float t = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    const int g = k / 2, e = 4 * (k & 1) + sel;
    float sc;
    if constexpr (B == 2) sc = ldexpf(1.0f, 24 - 2 * (e < 5 ? e : e - 5));
    else if constexpr (B == 4) sc = (e & 1) ? kTwo24 / 16.0f : kTwo24;
    else sc = channel_scale<B>(0);
    sm.wv[wave].o[g][cb * 8 + e] = fmaf(t, sc, st.z[g]);
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      sm.part_ml[wave][g][0] = st.m[g];
      sm.part_ml[wave][g][1] = st.l[g];
    }
  }
}

// ---------------------------------------------------------------- K-record ring

// N (1..4) buffer_load_dwordx4 ... lds: copy j moves the 16 bytes at range
// offset voff + 1024 j (voff = 16 * lane) to LDS byte lds + 1024 j + 16 * lane;
// the instruction offset moves both addresses.  Dwords past the range arrive
// as zeros.  Inline assembly, so the compiler's memory-counter bookkeeping
// does not see the copies (it would otherwise wait for every outstanding copy
// before any LDS read); the tile loop waits explicitly.  M0 (the LDS base) is
// saved and restored around them.
#define RDKV_LDS_COPY(off) "buffer_load_dwordx4 %1, %2, 0 offen offset:" #off " lds\n\t"
template <int N>
__device__ inline void lds_copy_block(rsrc4 r, uint32_t voff, uint32_t lds) {
  static_assert(N >= 1 && N <= 4, "copies per block");
  uint32_t saved;
  if constexpr (N == 1) {
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t" RDKV_LDS_COPY(0) "s_mov_b32 m0, %0"
                 : "=&s"(saved) : "v"(voff), "s"(r), "s"(lds) : "memory");
  } else if constexpr (N == 2) {
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t" RDKV_LDS_COPY(0) RDKV_LDS_COPY(1024)
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved) : "v"(voff), "s"(r), "s"(lds) : "memory");
  } else if constexpr (N == 3) {
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t" RDKV_LDS_COPY(0) RDKV_LDS_COPY(1024)
                 RDKV_LDS_COPY(2048) "s_mov_b32 m0, %0"
                 : "=&s"(saved) : "v"(voff), "s"(r), "s"(lds) : "memory");
  } else {
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t" RDKV_LDS_COPY(0) RDKV_LDS_COPY(1024)
                 RDKV_LDS_COPY(2048) RDKV_LDS_COPY(3072) "s_mov_b32 m0, %0"
                 : "=&s"(saved) : "v"(voff), "s"(r), "s"(lds) : "memory");
  }
}
#undef RDKV_LDS_COPY

// Copies a tile's K-record block (`bytes` bytes from the 16-byte-aligned
// src) into an LDS stage with exactly stage_copies<SW> copies, in blocks of
// four (one M0 and one resource per block).  Past `bytes` the stage gets
// zeros; no memory beyond the block is read.
template <int SW, int C0 = 0>
__device__ inline void dma_records(const uint8_t* src, uint32_t bytes, uint32_t* stage, uint32_t voff) {
  constexpr int n = stage_copies<SW>();
  if constexpr (C0 < n) {
    constexpr uint32_t off = uint32_t(C0) * 1024;
    const rsrc4 r = buffer_rsrc4(src + off, bytes > off ? bytes - off : 0u);
    lds_copy_block<(n - C0 < 4 ? n - C0 : 4)>(r, voff, lds_addr(stage) + off);
    dma_records<SW, C0 + 4>(src, bytes, stage, voff);
  }
}

// ---------------------------------------------------------------- token groups (zones A and B)

// SW > 0: records (at most SW words) go through the wave's LDS ring; SW == 0:
// each lane reads its record from global memory.  PIPE: the lane's V pairs
// are loaded one tile ahead (two register sets used in turn); otherwise at
// the start of the tile, before the logits.
//
// Every tile's V rows and record block are read through buffer resources that
// end at the chunk's last row, so the rows of a partial tile past the chunk
// (and the whole of a tile past the wave's last) read as zeros without
// touching memory: no per-lane clamping, and tile addresses stay scalar.
//
// kPaged: the group's V rows and K records are 64-row tiles on pages found
// through the segment's block table (a chunk starts on a tile boundary, so
// tile i is the group's tile tile_row(i) / 64, whole on one page); each
// tile's resource or copy covers just that tile.  The wave looks its tiles up
// once, at the start of the chunk (lane j: the wave's tiles j, j + 64, ...),
// and a tile step takes its two offsets with a readlane each, so no table
// read sits between a tile's turn and its loads.
template <int G, int B, int SW, bool PIPE, bool kPaged>
__device__ void run_group(const DecodeParams& p, const SegInfo& si, const Plan& pl, int64_t seg, Smem<G, SW>& sm,
                          uint32_t* pg_lds) {
  constexpr int GW = kHeadsPerWave<G>, kNS = kStreams<G>, kStride = kTile * kNS;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int cb = lane & 15, ts = lane >> 4;
  const int hb = kNS == kWaves ? 0 : (wave / kNS) * GW;           // the wave's first query head
  const QkShape ks = qk_shape(si);
  const int nw = pl.rec_words;
  const uint8_t* rbytes = p.cache + si.off_krec;                   // 256-byte aligned
  const uint8_t* vbase = p.cache + pl.vbase;
  constexpr int kRowBytes = kHeadDim * B / 8;
  const int first = pl.start + kTile * (wave % kNS);               // the wave's tiles: first + kStride i
  const int n_tiles = first < pl.end ? (pl.end - first + kStride - 1) / kStride : 0;
  auto tile_row = [&](int i) { return first + kStride * min(i, n_tiles - 1); };
  // rows of tile i inside the chunk; none for the tiles past the wave's last
  auto tile_rows = [&](int i) { return i < n_tiles ? min(kTile, pl.end - (first + kStride * i)) : 0; };

  // Ring: tile i's records live in stage i mod S.  The first S - 1 tiles are
  // copied up front; the end of step i copies tile i + S - 1 into the stage
  // of tile i - 1.  Each step begins with its V loads (for the next tile, or
  // this tile without PIPE), so the compiler's own wait for V data never
  // covers a record copy issued in the same step.
  constexpr int kStages = ring_stages<SW>();
  constexpr int kS = kStages > 0 ? kStages : 1;
  constexpr int kAhead = kS - 1;
  constexpr int kNV = kPairsPerLane * 2;                           // V load instructions per step
  // V loads per step issued before the wait (PIPE: tile i + 1's; 8-bit: this
  // tile's) and after it (fp16 rows: each pair just before its products).
  constexpr bool kLateV = !PIPE && B == 16;
  constexpr int kPre = kLateV ? 0 : kNV, kPost = kLateV ? kNV : 0;
  constexpr int kCopies = SW > 0 ? stage_copies<SW>() : 0;          // record copies per step
  // Issued after tile i's record copies by the time step i waits for them,
  // at the least: with three stages, step 0 (after the prologue) or a steady
  // step (two step starts, one step body, one refill); with two, one start.
  // Every step issues the same instructions (tiles past the last read zeros).
  constexpr int kWaitRec =
      kS == 3 ? kCopies + (((PIPE ? kNV : 0) + kPre) < (2 * kPre + kPost) ? (PIPE ? kNV : 0) + kPre : 2 * kPre + kPost)
              : kPre;
  const bool use_ring = SW > 0 && nw > 0 && n_tiles > 0;           // uniform
  auto stage = [&](int i) { return sm.wv[wave].ring + (i % kS) * (SW > 0 ? stage_words<SW>() : 0); };
  // word offset (from off_krec) of tile i's first record
  auto rec_word = [&](int i) { return pl.rec0 + int64_t(tile_row(i)) * nw; };
  const uint32_t voff16 = uint32_t(lane) * 16u;
  // paged: per lane, the V and record tile offsets (256-byte units) of the
  // wave's tiles lane + 64 k; record tiles are 64 * nw words, kPageBytes /
  // that per page
  // (at most 64 tiles per wave: one register per lane and region; more
  // (G = 8) go through the stream's LDS list, pg_lds)
  constexpr int kWaveTiles = kWaveTilesMax<G>;
  constexpr bool kLds = kPgLds<G, kPaged>;
  uint32_t* const pgl = pg_lds + (wave % kNS) * 2 * kWaveTiles;
  uint32_t pg_v = kNoPage, pg_r = kNoPage;
  if constexpr (kPaged) {
    constexpr uint32_t kVTileBytes = uint32_t(kTile) * kRowBytes;
    const uint32_t rec_tile_bytes = uint32_t(kTile) * 4u * uint32_t(nw);
    const uint32_t rec_tpp = nw > 0 ? uint32_t(kPageBytes) / rec_tile_bytes : 1u;
#pragma unroll
    for (int k = 0; k < (kWaveTiles + 63) / 64; ++k) {
      const int j = lane + 64 * k;
      uint32_t v = kNoPage, r = kNoPage;
      if (j < n_tiles) {
        const uint32_t t = uint32_t(first + kStride * j) / kTile;
        v = paged_tile_units(p, si.table, pl.vp_a, t, kPageBytes / kVTileBytes, kVTileBytes);
        if (nw > 0) r = paged_tile_units(p, si.table, pl.vp_b, t, rec_tpp, rec_tile_bytes);
      }
      if constexpr (kLds) {
        pgl[j] = v;                  // (the stream's other wave writes the same values)
        pgl[kWaveTiles + j] = r;
      } else {
        pg_v = v;
        pg_r = r;
      }
    }
    if constexpr (kLds) wave_lds_sync();
  }
  // tile i's entry, region 0 (V) or 1 (records); tiles past the wave's last
  // take its last tile's, as tile_row does
  auto lane_tile = [&](int region, int i) -> uint32_t {
    const int j = max(min(i, n_tiles - 1), 0);
    if constexpr (kLds) return __builtin_amdgcn_readfirstlane(pgl[region * kWaveTiles + j]);
    else return __builtin_amdgcn_readlane(region ? pg_r : pg_v, j);
  };
  // An entry outside the table or the pool reads as the pool's first page
  // with ok = false (callers then read nothing through it).
  auto tile_ptr = [&](uint32_t u, bool& ok) {
    ok = u != kNoPage;
    return p.cache + (ok ? uint64_t(u) << 8 : p.pool_offset);
  };
  auto fetch_records = [&](int i) {
    if constexpr (SW > 0) {
      const int rows = tile_rows(i);
      if constexpr (kPaged) {
        bool ok;
        const uint8_t* t = tile_ptr(lane_tile(1, i), ok);
        dma_records<SW>(t, (rows > 0 && ok) ? uint32_t(rows * nw) * 4u : 0u, stage(i), voff16);
      } else {
        const int64_t w0 = rec_word(i);
        const int m = int(w0 & 3);                                 // block start within its 16 bytes
        dma_records<SW>(rbytes + uint64_t(w0 - m) * 4, rows > 0 ? uint32_t(m + rows * nw) * 4u : 0u, stage(i),
                        voff16);
      }
    }
  };
  // V pairs of tile i: one resource per tile, a fixed lane offset, and the
  // pair's rows as instruction offsets.
  const uint32_t lane_off = uint32_t(ts * kRowBytes + lane_row_offset<B>(cb));
  const uint32_t sel2 = (cb & 1) ? 0x07060302u : 0x05040100u;      // the lane's half of a 2-bit dword
  auto vrsrc = [&](int i) {
    if constexpr (kPaged) {
      bool ok;
      const uint8_t* t = tile_ptr(lane_tile(0, i), ok);
      return buffer_rsrc(t, ok ? uint32_t(tile_rows(i) * kRowBytes) : 0u);
    } else {
      return buffer_rsrc(vbase + int64_t(tile_row(i)) * kRowBytes, uint32_t(tile_rows(i) * kRowBytes));
    }
  };
  auto load_pair = [&](__amdgpu_buffer_rsrc_t r, int k) {
    return load_vpair_buf<B>(r, lane_off + 4 * k * kRowBytes, lane_off + (4 * k + 32) * kRowBytes);
  };
  auto load_pairs = [&](VPair<B> (&v)[kPairsPerLane], int i) {
    const __amdgpu_buffer_rsrc_t r = vrsrc(i);
#pragma unroll
    for (int k = 0; k < kPairsPerLane; ++k) v[k] = load_pair(r, k);
  };

  VPair<B> va[kPairsPerLane], vb[kPairsPerLane];
  if (use_ring) {
#pragma unroll
    for (int i = 0; i < kAhead; ++i) fetch_records(i);
  }
  if constexpr (PIPE) {
    if (n_tiles > 0) load_pairs(va, 0);
  }
  build_query_tables<G, SW>(si, pl, sm);
  __syncthreads();

  WaveState<GW> st;
  state_init(st);
  const int lane_rec = lane * nw;                                  // the lane's record in a stage
  auto tile = [&](int i, VPair<B> (&cur)[kPairsPerLane], VPair<B> (&nxt)[kPairsPerLane]) {
    const int b = tile_row(i);
    if constexpr (PIPE) load_pairs(nxt, i + 1);
    if constexpr (!PIPE && !kLateV) load_pairs(cur, i);
    if (use_ring) wait_vmem<(kWaitRec < 63 ? kWaitRec : 63)>();
    // (with SW > 0 and no record words, nothing is read from the stage)
    const uint32_t* my;
    if constexpr (SW > 0) {
      my = stage(i) + (kPaged ? 0 : int(rec_word(i) & 3)) + lane_rec;
    } else if constexpr (kPaged) {
      bool ok;   // (an entry outside the pool reads page 0: in memory, the segment's output is then wrong)
      my = reinterpret_cast<const uint32_t*>(tile_ptr(lane_tile(1, i), ok)) + (min(b + lane, pl.end - 1) - b) * nw;
    } else {
      my = reinterpret_cast<const uint32_t*>(rbytes) + pl.rec0 + int64_t(min(b + lane, pl.end - 1)) * nw;
    }
    float s[GW], vs, vz;
    record_logits<GW>(my, ks, nw, B < 16, sm, hb, s, vs, vz);
    // one softmax body for full and partial tiles (the validity test costs a
    // compare and a select per head; two bodies cost register moves to merge)
    softmax_tile<GW, G, SW, true>(st, s, b + lane < pl.end, vs, vz, sm, wave, lane);
    wave_lds_sync();
    __amdgpu_buffer_rsrc_t rl;
    if constexpr (kLateV) rl = vrsrc(i);
#pragma unroll
    for (int k = 0; k < kPairsPerLane; ++k) {
      uint32_t cf[GW];
      load_coefs<GW>(sm, wave, ts + 4 * k, cf);
      if constexpr (kLateV) {
        const VPair<B> v = load_pair(rl, k);
        pv_pair<GW, B>(st.acc, v, cf, sel2);
      } else {
        pv_pair<GW, B>(st.acc, cur[k], cf, sel2);
      }
    }
    wave_lds_sync();
    if (use_ring) fetch_records(i + kAhead);
  };
  for (int i = 0; i < n_tiles; i += 2) {
    tile(i, va, vb);
    if (i + 1 >= n_tiles) break;
    tile(i + 1, vb, va);
  }
  // The last steps copied (zero) blocks into ring stages that the partial
  // output below overwrites; those copies must land before it does.
  if (use_ring) wait_vmem<0>();
  wave_finish<GW, B>(st, sm, wave, lane);
}

// ---------------------------------------------------------------- zone C (fp16 rows, natural order)

// Zone-C rows [pl.start, pl.end); row c_len comes from k_new / v_new when
// `append` (this step's new token).  kPaged: rows are 64-row tiles on the
// segment's pages, one page lookup per tile.
template <int G, int SW, bool kPaged>
__device__ void run_zone_c(const DecodeParams& p, const SegInfo& si, int64_t seg, const Plan& pl, int c_len,
                           bool append, Smem<G, SW>& sm) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int cb = lane & 15, ts = lane >> 4;
  const int last = pl.end - 1;
  const uint8_t* kc = p.cache + si.off_kc;
  const uint8_t* vc = p.cache + si.off_vc;
  const uint8_t* knew = reinterpret_cast<const uint8_t*>(p.k_new + seg * kHeadDim);
  const uint8_t* vnew = reinterpret_cast<const uint8_t*>(p.v_new + seg * kHeadDim);
  constexpr uint32_t kTileBytes = uint32_t(kTile) * kHeadDim * 2;
  // Row 0 of the tile holding row `base` (a multiple of 64): every row a
  // tile step touches lies in that tile, so one lookup per tile; the zone-C
  // pages were checked when the segment was loaded.
  auto tile0 = [&](const uint8_t* flat, int vp0, int base) -> const uint8_t* {
    if constexpr (kPaged) {
      bool ok;
      return p.cache + paged_tile(p, si.table, vp0, base / kTile, kPageBytes / kTileBytes, kTileBytes, ok);
    } else {
      return flat + int64_t(base) * kHeadDim * 2;
    }
  };

  constexpr int GW = kHeadsPerWave<G>, kNS = kStreams<G>;
  const int hb = kNS == kWaves ? 0 : (wave / kNS) * GW;           // the wave's first query head
  build_query_tables<G, SW>(si, pl, sm);
  __syncthreads();
  WaveState<GW> st;
  state_init(st);
  for (int base = pl.start + kTile * (wave % kNS); base < pl.end; base += kTile * kNS) {
    const uint8_t* kt = tile0(kc, pl.vp_a, base);
    const uint8_t* vt = tile0(vc, pl.vp_b, base);
    auto vrow = [&](int r) {
      r = min(r, last);
      return (append && r == c_len) ? vnew : vt + int64_t(r - base) * kHeadDim * 2;
    };
    VPair<16> v[kPairsPerLane];
#pragma unroll
    for (int k = 0; k < kPairsPerLane; ++k) v[k] = load_vpair16(vrow(base + ts + 4 * k), vrow(base + ts + 4 * k + 32), cb);
    const int r = min(base + lane, last);
    const uint4* k4 = reinterpret_cast<const uint4*>((append && r == c_len) ? knew : kt + int64_t(r - base) * kHeadDim * 2);
    float s[GW];
#pragma unroll
    for (int g = 0; g < GW; ++g) s[g] = 0.f;
#pragma unroll 4
    for (int c = 0; c < 16; ++c) {
      const uint4 x = k4[c];
      const uint32_t ws[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t q[GW];
        load_qp<GW>(sm, 4 * c + j, hb, q);
#pragma unroll
        for (int g = 0; g < GW; ++g) s[g] = dot2(ws[j], q[g], s[g]);
      }
    }
    softmax_tile<GW, G, SW, true>(st, s, base + lane < pl.end, 1.f, 0.f, sm, wave, lane);
    wave_lds_sync();
#pragma unroll
    for (int k = 0; k < kPairsPerLane; ++k) {
      uint32_t cf[GW];
      load_coefs<GW>(sm, wave, ts + 4 * k, cf);
      pv_pair<GW, 16>(st.acc, v[k], cf, 0u);
    }
    wave_lds_sync();
  }
  wave_finish<GW, 16>(st, sm, wave, lane);
}

// ---------------------------------------------------------------- kernels

// out[seg][g][c] = sum_k e^{m_k - M} o_k[c] / sum_k e^{m_k - M} l_k over the
// segment's chunks; a segment with nothing to attend to gives 0.  One
// workgroup of Q * 128 threads per (segment, query head): thread t owns
// channel t mod 128 and, of each round of up to 32 Q chunk slots, the slots
// t / 128 + Q j.  A round issues all its reads (the slots' (m, l) in the
// first waves, 32 slots of its channel per thread) before it uses any, so it
// costs one memory round trip; Q = 4 when a segment has more than 32 chunk
// slots (one round up to 128), else 1.  The Q partial sums are added in a
// fixed order at the end, so the result does not depend on scheduling.
// Every slot up to max_chunks was written by the chunk kernel; slots past the
// segment's last chunk hold (-inf, 0, 0...), so the merge needs nothing from
// the blob.
constexpr int kMergeLoads = 32;
template <int Q> constexpr int kMergeThreads = Q * kHeadDim;
template <int Q> constexpr int kMergeRound = Q * kMergeLoads;

// With kAccum (rdkv_decode_accumulate), the workgroup of (segment, head g)
// then adds the step's final softmax probability of every zone-C row j < n_c,
// exp2(t_j - M) / L with t_j = q_g.k_j log2(e) / sqrt(d) recomputed from the
// zone-C key (fp32 products of the fp16 values), to zc_stats[seg][g][j], and
// q_g[c]^2 to zc_stats[seg][g][cap + c]; one thread per element, so no
// atomics and a fixed order.
template <int G, bool kAccum, int Q>
__global__ __launch_bounds__(kMergeThreads<Q>) void decode_merge_kernel(DecodeParams p) {
  constexpr int kRound = kMergeRound<Q>, kRoundWaves = (kRound + 63) / 64;
  __shared__ float s_w[kRound];
  __shared__ float s_red[2][kRoundWaves];
  __shared__ float s_o[Q][kHeadDim];
  const int64_t seg = blockIdx.x / G;
  const int g = int(blockIdx.x % G);
  const int t = threadIdx.x, c = t % kHeadDim, qd = t / kHeadDim;
  const int n = p.max_chunks;
  const float* part = p.partials + int64_t(seg) * n * G * kPartialFloats + g * kPartialFloats;
  const int64_t stride = int64_t(G) * kPartialFloats;
  float M = -INFINITY, L = 0.f, O = 0.f;
  for (int k0 = 0; k0 < n; k0 += kRound) {
    const int kn = min(kRound, n - k0);
    const float* pr = part + k0 * stride;
    float mc = -INFINITY, lc = 0.f;
    if (t < kn) {
      mc = pr[t * stride];
      lc = pr[t * stride + 1];
    }
    float o[kMergeLoads];
#pragma unroll
    for (int j = 0; j < kMergeLoads; ++j) {
      const int k = qd + Q * j;   // (uniform over a wave)
      o[j] = k < kn ? pr[k * stride + 4 + c] : 0.f;
    }
    // the round's largest m (the first kRoundWaves waves hold its slots)
    if (t < 64 * kRoundWaves) {
      const float wm = wave_reduce<true>(mc);
      if ((t & 63) == 0) s_red[0][t >> 6] = wm;
    }
    __syncthreads();
    float mb = M;
#pragma unroll
    for (int i = 0; i < kRoundWaves; ++i) mb = fmaxf(mb, s_red[0][i]);
    if (t < 64 * kRoundWaves) {
      const float w = mc == -INFINITY ? 0.f : exp2f(mc - mb);
      if (t < kRound) s_w[t] = w;
      const float lw = wave_reduce<false>(lc * w);
      if ((t & 63) == 0) s_red[1][t >> 6] = lw;
    }
    __syncthreads();
    if (mb != -INFINITY) {
      const float a = exp2f(M - mb);   // (0 while nothing was merged)
      float lsum = 0.f;
#pragma unroll
      for (int i = 0; i < kRoundWaves; ++i) lsum += s_red[1][i];
      L = fmaf(L, a, lsum);
      O *= a;
#pragma unroll
      for (int j = 0; j < kMergeLoads; ++j) O = fmaf(o[j], s_w[qd + Q * j], O);
      M = mb;
    }
    __syncthreads();
  }
  s_o[qd][c] = O;
  __syncthreads();
  if (t < kHeadDim) {
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < Q; ++i) sum += s_o[i][c];
    p.out[(seg * G + g) * kHeadDim + c] = L > 0.f ? sum / L : 0.f;
  }
  if constexpr (kAccum) {
    float* st = p.zc_stats + (seg * G + g) * int64_t(p.zc_cap + kHeadDim);
    float* s_q = s_o[0];           // free once every thread has read its sums
    __syncthreads();
    if (t < kHeadDim) {
      const float qc = __half2float(p.q[(seg * G + g) * kHeadDim + c]);
      st[p.zc_cap + c] += qc * qc;
      s_q[c] = qc;
    }
    __syncthreads();
    const uint8_t* d = p.cache + kHeaderBytes + uint64_t(seg) * kDescBytes;
    const uint64_t off_kc = *reinterpret_cast<const uint64_t*>(d + kDescOffKc);
    if (L > 0.f && off_kc + uint64_t(p.n_c) * kHeadDim * 2 <= p.main_bytes) {
      for (int j = t; j < p.n_c; j += kMergeThreads<Q>) {
        const uint4* kr = reinterpret_cast<const uint4*>(p.cache + off_kc + uint64_t(j) * kHeadDim * 2);
        float tj = 0.f;
#pragma unroll 4
        for (int i = 0; i < kHeadDim / 8; ++i) {
          const uint4 x = kr[i];
          const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            tj = fmaf(s_q[8 * i + 2 * e], half_lo(w4[e]), tj);
            tj = fmaf(s_q[8 * i + 2 * e + 1], half_hi(w4[e]), tj);
          }
        }
        st[j] += exp2f(tj * kLog2eOverSqrtD - M) / L;
      }
    }
  }
}

// The zone-C lengths of a paged cache's sequences (a contiguous cache has
// one, in DecodeParams).
struct NoSeqLens {};
template <typename Lens> constexpr bool kIsPaged = std::is_same<Lens, PagedSeqLens>::value;

template <int G, int SW, typename Lens>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void decode_chunk_kernel(DecodeParams p,
                                                                                                       Lens lens) {
  constexpr bool kPaged = kIsPaged<Lens>;
  __shared__ Smem<G, SW> sm;
  __shared__ uint32_t pg_lds[kPgLdsWords<G, kPaged>];
  // Chunk-major order: every segment's first chunk, then every second chunk,
  // ...  The full 2-bit chunks come first and the short tails, fp16 and zone-C
  // chunks last, so the dispatcher's in-order fill ends on light work; and
  // with n_seg a multiple of 8 all chunks of a segment land on one XCD (whose
  // L2 then holds the segment's descriptor and query).
  // (n_seg < 2^24: 32-bit division)
  const uint32_t n_seg = uint32_t(p.n_seg);
  const int64_t seg = blockIdx.x % n_seg;
  const int k = int(blockIdx.x / n_seg);
  // this step's zone C: rows before it and whether it appends one
  int c_len = p.c_len;
  bool append = p.append != 0;
  if constexpr (kPaged) c_len = lens.c_len[seg / p.seg_per_seq];
  // slot k: the prefill tokens' chunks, the generations' chunks, zone C
  const int gen_end = p.token_slots + p.n_gen * p.gen_slots;
  {
    // the descriptor this slot reads: the prefill blob's, or a generation blob's
    uint64_t desc = kHeaderBytes + uint64_t(seg) * kDescBytes;
    if (!kPaged && k >= p.token_slots && k < gen_end) desc += gen_blob(p, (k - p.token_slots) / p.gen_slots).base;
    stage_query(p, seg, desc, sm);
  }
  SegInfo si;
  Plan pl;
  if constexpr (kPaged) {
    si = load_segment_paged(p, seg, c_len + int(append));
    if (k < p.token_slots) pl = plan_tokens(si, p.chunk_tok2, k);
    else pl = plan_zone_c(si, si.zc_ok ? c_len + int(append) : 0, k - gen_end);
  } else if (k < p.token_slots) {
    si = load_segment(p, main_blob(p), seg, 0);
    pl = plan_tokens(si, p.chunk_tok2, k);
  } else if (k < gen_end) {
    const int g = (k - p.token_slots) / p.gen_slots;
    const int n_used = *reinterpret_cast<const int32_t*>(p.cache + kHdrNGenUsed);
    if (g < n_used) {
      const BlobRef b = gen_blob(p, g);
      si = load_segment(p, b, seg, 0);
      pl = plan_tokens(si, b.chunk_tok2, k - p.token_slots - g * p.gen_slots);
    } else {
      pl.kind = -1;
    }
  } else {
    si = load_segment(p, main_blob(p), seg, p.n_c);
    pl = plan_zone_c(si, si.zc_ok ? p.n_c : 0, k - gen_end);
  }
  const int tid = threadIdx.x;
  float* out = p.partials + (int64_t(seg) * p.max_chunks + k) * G * kPartialFloats;
  if (pl.kind < 0) {   // a slot past the segment's last chunk: (m, l, o) = (-inf, 0, 0)
    for (int i = tid; i < G * kPartialFloats; i += kThreads) out[i] = i % kPartialFloats == 0 ? -INFINITY : 0.f;
    return;
  }

  // append the new token to zone C (only the chunk holding row c_len does it)
  if (pl.kind == 4 && append && c_len >= pl.start && c_len < pl.end) {
    uint32_t *kc, *vc;
    if constexpr (kPaged) {
      constexpr uint32_t kTileBytes = uint32_t(kTile) * kHeadDim * 2;
      bool ok;
      const uint64_t row = uint64_t(c_len % kTile) * kHeadDim * 2;
      kc = reinterpret_cast<uint32_t*>(p.cache + row +
                                       paged_tile(p, si.table, pl.vp_a, c_len / kTile, kPageBytes / kTileBytes,
                                                  kTileBytes, ok));
      vc = reinterpret_cast<uint32_t*>(p.cache + row +
                                       paged_tile(p, si.table, pl.vp_b, c_len / kTile, kPageBytes / kTileBytes,
                                                  kTileBytes, ok));
    } else {
      kc = reinterpret_cast<uint32_t*>(p.cache + si.off_kc) + int64_t(c_len) * (kHeadDim / 2);
      vc = reinterpret_cast<uint32_t*>(p.cache + si.off_vc) + int64_t(c_len) * (kHeadDim / 2);
    }
    if (tid < 64) kc[tid] = reinterpret_cast<const uint32_t*>(p.k_new + seg * kHeadDim)[tid];
    else if (tid < 128) vc[tid - 64] = reinterpret_cast<const uint32_t*>(p.v_new + seg * kHeadDim)[tid - 64];
  }

  switch (pl.kind) {
    case 0: run_group<G, 2, SW, true, kPaged>(p, si, pl, seg, sm, pg_lds); break;
    case 1: run_group<G, 4, SW, true, kPaged>(p, si, pl, seg, sm, pg_lds); break;
    case 2: run_group<G, 8, SW, false, kPaged>(p, si, pl, seg, sm, pg_lds); break;
    case 3: run_group<G, 16, SW, false, kPaged>(p, si, pl, seg, sm, pg_lds); break;
    default: run_zone_c<G, SW, kPaged>(p, si, seg, pl, c_len, append, sm); break;
  }
  __syncthreads();

  // merge the waves' partials into the chunk's partial: head g was carried
  // by the kNS waves (g / GW) * kNS ... as their head g % GW
  constexpr int GW = kHeadsPerWave<G>, kNS = kStreams<G>;
  for (int i = tid; i < G * kHeadDim; i += kThreads) {
    const int g = i / kHeadDim, c = i % kHeadDim;
    const int w0 = (g / GW) * kNS, gl = g % GW;
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < kNS; ++j) M = fmaxf(M, sm.part_ml[w0 + j][gl][0]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int j = 0; j < kNS; ++j) {
      const float f = exp2f(sm.part_ml[w0 + j][gl][0] - M);
      L = fmaf(sm.part_ml[w0 + j][gl][1], f, L);
      O = fmaf(sm.wv[w0 + j].o[gl][c], f, O);
    }
    out[g * kPartialFloats + 4 + c] = O;
    if (c == 0) {
      out[g * kPartialFloats + 0] = M;
      out[g * kPartialFloats + 1] = L;
    }
  }
}

template <int G, int SW, typename Lens>
hipError_t launch_chunks_gs(const DecodeParams& p, const Lens& lens, hipStream_t stream) {
  const uint64_t grid = uint64_t(p.n_seg) * p.max_chunks;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((decode_chunk_kernel<G, SW, Lens>), dim3(unsigned(grid)), dim3(kThreads), 0, stream, p, lens);
  return hipGetLastError();
}

template <int G>
hipError_t launch_chunks_g(const DecodeParams& p, hipStream_t stream) {
  // K record words staged through LDS, from the layout's bound on a record
  const int words = (max(p.rec_max, p.gen_rec_max) + 3) / 4;
  const NoSeqLens none;
  if (words <= 8) return launch_chunks_gs<G, 8>(p, none, stream);
  if (words <= 10) return launch_chunks_gs<G, 10>(p, none, stream);
  if (words <= 12) return launch_chunks_gs<G, 12>(p, none, stream);
  if (words <= 16) return launch_chunks_gs<G, 16>(p, none, stream);
  if (words <= 20) return launch_chunks_gs<G, 20>(p, none, stream);
  if (words <= 24) return launch_chunks_gs<G, 24>(p, none, stream);
  if (words <= kMaxStagedWords) return launch_chunks_gs<G, 32>(p, none, stream);
  return launch_chunks_gs<G, 0>(p, none, stream);
}

// Paged caches: fewer record-stage variants (a layout's record bound is set
// by the largest budget it admits).
template <int G>
hipError_t launch_chunks_paged_g(const DecodeParams& p, const PagedSeqLens& lens, hipStream_t stream) {
  const int words = (p.rec_max + 3) / 4;
  if (words <= 10) return launch_chunks_gs<G, 10>(p, lens, stream);
  if (words <= 16) return launch_chunks_gs<G, 16>(p, lens, stream);
  if (words <= 24) return launch_chunks_gs<G, 24>(p, lens, stream);
  if (words <= kMaxStagedWords) return launch_chunks_gs<G, 32>(p, lens, stream);
  return launch_chunks_gs<G, 0>(p, lens, stream);
}

template <int G, int Q>
hipError_t launch_merge_gq(const DecodeParams& p, hipStream_t stream) {
  if (p.zc_stats)
    hipLaunchKernelGGL((decode_merge_kernel<G, true, Q>), dim3(unsigned(p.n_seg * G)), dim3(kMergeThreads<Q>), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((decode_merge_kernel<G, false, Q>), dim3(unsigned(p.n_seg * G)), dim3(kMergeThreads<Q>), 0,
                       stream, p);
  return hipGetLastError();
}

template <int G>
hipError_t launch_merge_g(const DecodeParams& p, hipStream_t stream) {
  if (p.n_seg == 0) return hipSuccess;
  return p.max_chunks > kMergeRound<1> ? launch_merge_gq<G, 4>(p, stream) : launch_merge_gq<G, 1>(p, stream);
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

hipError_t launch_decode_chunks_paged(const DecodeParams& p, const PagedSeqLens& lens, hipStream_t stream) {
  switch (p.group) {
    case 1: return launch_chunks_paged_g<1>(p, lens, stream);
    case 2: return launch_chunks_paged_g<2>(p, lens, stream);
    case 4: return launch_chunks_paged_g<4>(p, lens, stream);
    case 8: return launch_chunks_paged_g<8>(p, lens, stream);
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
