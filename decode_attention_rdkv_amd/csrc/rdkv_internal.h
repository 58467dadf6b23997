// Internal declarations shared by the RDKV HIP translation units.
//
// Format constants follow the packed-cache specification (header, 256-byte
// descriptors, fixed-size slots; see the TriZone zones of the RDKV summary,
// section 2.3).  Nothing here is exported from the library.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "rdkv.h"

namespace rdkv {

constexpr int kHeadDim = 128;
constexpr int64_t kMaxTokens = int64_t(1) << 19;   // prefill tokens per sequence
constexpr int64_t kMaxSegments = int64_t(1) << 24;  // sequences x layers x KV heads of one layout
// A layout (blob, generation blobs or decode workspace) above this many bytes
// is refused: with the bounds on tokens, segments, zone C and generations no
// size computation overflows before this test.
constexpr uint64_t kMaxCacheBytes = uint64_t(1) << 50;
constexpr uint32_t kMagic = 0x564B4452u;  // "RDKV" little-endian
constexpr int kFormatVersion = 2;
constexpr int kHeaderBytes = 256;
constexpr int kDescBytes = 256;
constexpr int kAlign = 256;

// Descriptor field byte offsets.
constexpr int kDescNTok = 0;      // i32[4]: kept tokens at 2, 4, 8, 16 bits
constexpr int kDescNKept = 16;    // i32
constexpr int kDescNChan = 20;    // i32[4]: channels at 16, 8, 4, 2 bits
constexpr int kDescRec = 36;      // i32: K record bytes of a 2/4/8-bit token
constexpr int kDescCap = 40;      // i32: zone C capacity
constexpr int kDescFlags = 44;    // i32: bit 0 = allocation did not fit, packed empty
constexpr int kDescOffV = 48;     // u64[4]
constexpr int kDescOffKrec = 80;  // u64
constexpr int kDescOffPos = 88;   // u64
constexpr int kDescOffKc = 96;    // u64
constexpr int kDescOffVc = 104;   // u64
constexpr int kDescPerm = 128;    // u8[128]

// Split-K chunking of decode: a chunk holds chunk_tok2 >> g tokens of V group
// g (2, 4, 8, 16 bits: equal V bytes per chunk), or kChunkRowsC zone-C rows.
// chunk_tok2 is a power of two in [kChunkTok2Min, kChunkTok2Max], chosen per
// layout so that one launch has about kDecodeTargetChunks chunks.
#ifndef RDKV_DECODE_TARGET_CHUNKS
#define RDKV_DECODE_TARGET_CHUNKS 512
#endif
constexpr int64_t kDecodeTargetChunks = RDKV_DECODE_TARGET_CHUNKS;
#ifndef RDKV_CHUNK_TOK2_MIN
#define RDKV_CHUNK_TOK2_MIN 512
#endif
constexpr int kChunkTok2Min = RDKV_CHUNK_TOK2_MIN;
#ifndef RDKV_CHUNK_TOK2_MAX
#define RDKV_CHUNK_TOK2_MAX 16384
#endif
constexpr int kChunkTok2Max = RDKV_CHUNK_TOK2_MAX;
__host__ __device__ constexpr int chunk_tokens(int chunk_tok2, int group) { return chunk_tok2 >> group; }
// log2 of chunk_tokens (chunk_tok2 is a power of two): chunk counts and
// indices by shifts rather than divisions.
__host__ __device__ inline int chunk_shift(int chunk_tok2, int group) { return __builtin_ctz(uint32_t(chunk_tok2)) - group; }
constexpr int kChunkRowsC = 256;
// Floats per (chunk, query head) partial: m, l, 2 pad, o[128].
constexpr int kPartialFloats = 4 + kHeadDim;

__host__ __device__ inline uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }
__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Word counts of a K record from the channel counts (n16, n8, n4, n2).
struct RecordShape {
  int w16, w8, w4, w2, n_meta;
  __host__ __device__ int words_a() const { return w16 + w8 + w4 + w2 + n_meta + 1; }
};
__host__ __device__ inline RecordShape record_shape(int n16, int n8, int n4, int n2) {
  RecordShape r;
  r.w16 = (n16 + 1) / 2;
  r.w8 = (n8 + 3) / 4;
  r.w4 = (n4 + 7) / 8;
  r.w2 = (n2 + 15) / 16;
  r.n_meta = (n8 > 0) + (n4 > 0) + (n2 > 0);
  return r;
}

// Bitwidth of token group g (0..3 -> 2, 4, 8, 16).
__host__ __device__ constexpr int group_bits(int g) { return 2 << g; }
// Token group of a bitwidth, -1 for anything that is not 2, 4, 8 or 16.
__host__ __device__ inline int bits_group(int b) {
  return b == 2 ? 0 : b == 4 ? 1 : b == 8 ? 2 : b == 16 ? 3 : -1;
}

// ------------------------------------------------------------ device helpers

__device__ inline float half_lo(uint32_t w) { return __half2float(__ushort_as_half((unsigned short)(w & 0xffffu))); }
__device__ inline float half_hi(uint32_t w) { return __half2float(__ushort_as_half((unsigned short)(w >> 16))); }

template <typename T>
__device__ inline T wave_shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, 64);
}
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ inline float wave_min(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fminf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}
__device__ inline int wave_sum_i(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// ------------------------------------------------------------ launchers
// Each returns hipSuccess or the launch error; arguments are already validated.

// Zone-C rollover: generation blobs reserved per layout, at most.
constexpr int kMaxGenerations = 4096;
// Blob header fields of the generations (bytes): count reserved, count in
// use, offset of generation 0, stride, V and K budgets per generation.
constexpr int kHdrNGen = 88;
constexpr int kHdrNGenUsed = 92;
constexpr int kHdrGenOffset = 96;
constexpr int kHdrGenBytes = 104;
constexpr int kHdrGenBudgetV = 112;
constexpr int kHdrGenBudgetK = 120;

// ------------------------------------------------------------ paged cache
// Pages of RDKV_PAGE_BYTES; each region of a segment is an array of 64-row
// tiles laid page after page, a page holding kPageBytes / tile-bytes tiles.
constexpr int kPageBytes = RDKV_PAGE_BYTES;
constexpr int kMaxPagedSeqs = RDKV_MAX_PAGED_SEQS;
constexpr uint32_t kPagedMagic = 0x504B4452u;  // "RDKP"
constexpr int kPagedTile = 64;
// A paged cache stays below 1 TiB, so decode can hold a tile's offset in 32
// bits as a count of 256-byte units (every tile starts on such a boundary).
constexpr uint64_t kPagedMaxCacheBytes = uint64_t(1) << 40;
// regions: V rows of groups 0..3, K records of groups 0..3, zone-C K, zone-C V, positions
constexpr int kRegions = 11;
constexpr int kRegV = 0, kRegRec = 4, kRegKC = 8, kRegVC = 9, kRegPos = 10;
// paged descriptor: the first 48 bytes as the contiguous descriptor, then
// i32 vpage[11] (first virtual page of each region) and i32 n_pages
constexpr int kPDescVpage = 48;
constexpr int kPDescNPages = 92;
// paged header: i64 table_offset, pool_offset, max_pages, n_pages, page bytes
constexpr int kPHdrTable = 72;

// Bytes of a 64-row tile of region r; rec = bytes of a zone-A K record.
__host__ __device__ inline uint32_t paged_tile_bytes(int r, int rec) {
  if (r < kRegRec) return uint32_t(kPagedTile) * (kHeadDim * (2 << r) / 8);
  if (r < kRegKC) return uint32_t(kPagedTile) * uint32_t(rec - 4 * (r - kRegRec == 3));
  if (r < kRegPos) return uint32_t(kPagedTile) * kHeadDim * 2;
  return uint32_t(kPagedTile) * 4;
}
__host__ __device__ inline int paged_region_pages(int64_t rows, uint32_t tile_bytes) {
  if (rows <= 0 || tile_bytes == 0) return 0;
  const int64_t tiles = (rows + kPagedTile - 1) / kPagedTile;
  const int64_t tpp = kPageBytes / tile_bytes;
  return int((tiles + tpp - 1) / tpp);
}

// Split-K chunk slots of a segment in decode: [0, token_slots) the prefill
// tokens' chunks, then n_gen * gen_slots for the generation blobs (empty
// while a generation is not in use), then the zone-C chunks.
struct DecodeParams {
  uint8_t* cache;
  uint64_t cache_bytes;    // whole blob, generations included
  uint64_t main_bytes;     // the prefill generation's part (descriptors, slots)
  int64_t n_seg;
  int64_t nk_max;
  int32_t max_chunks;
  int32_t token_slots;
  int32_t chunk_tok2;
  int32_t rec_max;
  int32_t group;           // G = Hq / Hkv
  int32_t zc_cap;          // zone-C capacity (stride of the zone-C statistics)
  int32_t c_len;           // zone-C rows present before this step
  int32_t n_c;             // zone-C rows attended this step
  int32_t append;          // 1: row c_len comes from k_new/v_new and is written
  // generation blobs (all 0 without rollover)
  int32_t n_gen, gen_slots, gen_chunk_tok2, gen_rec_max;
  int64_t gen_nk_max;
  uint64_t gen_offset, gen_bytes, gen_cache_bytes;
  const __half* q;         // [n_seg][G][128]
  const __half* k_new;     // [n_seg][128] or null
  const __half* v_new;
  float* partials;         // [n_seg][max_chunks][G][kPartialFloats]
  float* out;              // [n_seg][G][128]
  float* zc_stats;         // merge: [n_seg][G][zc_cap + 128] statistics to accumulate, or null
  // paged cache (paged = 0 for a contiguous blob): descriptors at 256, the
  // block table [n_seg][max_pages] at table_offset, pages at pool_offset
  int32_t paged;
  int32_t seg_per_seq;     // L * Hkv (the sequence of a segment is seg / seg_per_seq)
  int32_t max_pages;
  int64_t pool_pages;
  uint64_t table_offset, pool_offset;
};
// Zone-C rows of each sequence slot before a paged decode step.
struct PagedSeqLens {
  int32_t c_len[kMaxPagedSeqs];
};
hipError_t launch_decode_chunks_paged(const DecodeParams& p, const PagedSeqLens& lens, hipStream_t stream);
hipError_t launch_decode_chunks(const DecodeParams& p, hipStream_t stream);
// Device address (on the current device) of the library-owned decode scratch
// of kStaticScratchBytes bytes used by rdkv_decode_static.
constexpr uint64_t kStaticScratchBytes = RDKV_STATIC_SCRATCH_BYTES;
hipError_t static_scratch(void** out);
hipError_t launch_decode_merge(const DecodeParams& p, hipStream_t stream);

struct PackParams {
  uint8_t* cache;
  uint64_t cache_bytes;
  const rdkv_layout* lay;  // host copy, fields are read on the host only
  int32_t layer_begin, n_layers_in;
  const __half* K;         // [S][n_layers_in][Hkv][N][128]
  const __half* V;
  const uint8_t* bits_tok; // [S][n_layers_in][Hkv][N]
  const uint8_t* bits_chan;// [S][n_layers_in][Hkv][128]
};
// gen: the layout of each generation blob (rollover layouts), else null
hipError_t launch_cache_init(uint8_t* cache, const rdkv_layout& lay, const rdkv_layout* gen, hipStream_t stream);
hipError_t launch_pack(const PackParams& p, hipStream_t stream);
hipError_t launch_pack_status(const uint8_t* cache, int64_t n_seg, int32_t* out, hipStream_t stream);

struct PagedPackParams {
  uint8_t* cache;          // the paged cache
  const rdkv_paged_layout* play;   // host copy
  const uint8_t* staging;  // a contiguous one-sequence blob packed by launch_pack
  uint64_t staging_bytes;
  int32_t seq;             // slot
  const int32_t* pages;    // [L*Hkv][max_pages]
  int32_t* pages_needed;   // [L*Hkv]
};
hipError_t launch_paged_init(uint8_t* cache, const rdkv_paged_layout& play, hipStream_t stream);
hipError_t launch_paged_plan(const PagedPackParams& p, hipStream_t stream);
hipError_t launch_paged_commit(const PagedPackParams& p, hipStream_t stream);
hipError_t launch_paged_release(uint8_t* cache, const rdkv_paged_layout& play, int32_t seq, hipStream_t stream);
// The decode launch shape of a cache's segments in use (a paged cache's
// committed slots, or every segment of a contiguous blob's prefill part).
struct ShapeGeom {
  int64_t n_seg;
  int32_t zone_c_capacity, chunk_tok2, token_slots, rec_max, group;
};
// out[0] = the most prefill-token chunks, out[1] = the longest K record
// (bytes) over the segments in use (device int32[2]).
hipError_t launch_shape_scan(const uint8_t* cache, const ShapeGeom& g, int32_t* out, hipStream_t stream);
// NaN outputs for the segments in use that a shape does not cover.
hipError_t launch_shape_check(const uint8_t* cache, const ShapeGeom& g, int32_t token_slots, int32_t rec_max,
                              float* out, hipStream_t stream);
hipError_t launch_unpack(const uint8_t* cache, uint64_t cache_bytes, const rdkv_layout& lay, int64_t seg,
                         float* k_hat, float* v_hat, hipStream_t stream);

struct RolloverParams {
  uint8_t* cache;
  uint64_t main_bytes;     // bytes of the prefill generation's part (zone-C offsets are checked against it)
  int64_t n_seg;
  int32_t G, cap, n_layers;
  uint64_t gen_offset, gen_bytes;
  int64_t gen_budget_v, gen_budget_k;
  const float* stats;      // [n_seg][G][cap + 128]
  float* w_tok;            // [n_seg][cap]
  float* var_tok;          // [n_seg][cap]
  float* w_chan;           // [n_seg][128]
};
// Workspace of a rollover: zone-C rows gathered per segment, weights, bits.
uint64_t rollover_workspace_bytes(int64_t n_seg, int64_t cap);
hipError_t launch_rollover_score(const RolloverParams& r, hipStream_t stream);
// Score (into the workspace), allocate, pack into generation blob `gen`
// (laid out by `gen_layout`), clear zone C and the statistics.
hipError_t launch_rollover(RolloverParams r, const rdkv_layout& gen_layout, int32_t gen, uint8_t* workspace,
                           hipStream_t stream);

struct AllocParams {
  int64_t n_seg, n_tokens;
  int32_t group;           // consecutive segments sharing one budget (divides n_seg)
  const float* w_tok;
  const float* var_tok;
  const float* w_chan;
  const __half* K;         // [n_seg][N][128]
  int64_t budget_v, budget_k;
  uint8_t* bits_tok;
  uint8_t* bits_chan;
  float* var_chan;
  double* lambda;
  uint8_t* workspace;      // alloc_plan(n_seg, n_tokens, group).total bytes, 256-byte aligned
};
hipError_t launch_allocate(const AllocParams& p, hipStream_t stream);

// The first error of a sequence of kernel launches: hipGetLastError after each
// launch, since a later successful call can leave success as the last status.
class LaunchErrors {
 public:
  void check() {
    const hipError_t l = hipGetLastError();
    if (e_ == hipSuccess) e_ = l;
  }
  hipError_t status() const { return e_; }

 private:
  hipError_t e_ = hipSuccess;
};
// The allocation's workspace: per group its radix-selection histogram and
// state, per (segment, token block) the exact K sums; byte offsets.
struct AllocPlan {
  int32_t v_blocks, k_blocks;   // workgroups per group (V tokens), per segment (K sums)
  uint64_t hist, state, s1, s2, cnt, total;
};
AllocPlan alloc_plan(int64_t n_seg, int64_t n_tokens, int32_t group);

struct ScoreParams {
  int64_t n_tokens;
  int32_t S, L, Hq, Hkv;
  const __half* Q;
  const __half* K;
  const __half* V;
  float* w_tok;
  float* var_tok;
  float* w_chan;
  float* lse;              // workspace [S][L][Hq][N], base-2 log-sum-exp of the scaled scores
  const float* lse_in;     // launch_score_from_lse: natural-log LSE given by the caller
};
// The two passes and the bandwidth kernels (launch_score), pass 1 alone
// writing p.lse in natural log (launch_score_lse), or everything but pass 1
// from p.lse_in (launch_score_from_lse).
hipError_t launch_score(const ScoreParams& p, hipStream_t stream);
hipError_t launch_score_lse(const ScoreParams& p, hipStream_t stream);
hipError_t launch_score_from_lse(const ScoreParams& p, hipStream_t stream);
size_t score_workspace_bytes(int64_t S, int64_t L, int64_t Hq, int64_t N);

}  // namespace rdkv
