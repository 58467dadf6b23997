// Stage-1 scoring after prefill (RDKV summary, section 2.1 weights, section
// 2.2 stage 1: computed once on the full uncompressed cache).
//
//   w_tok[h][t] = sum_{g in group(h)} sum_{tau >= t} exp(s_{g,tau,t} - LSE_{g,tau})
//   with s = Q_g[tau].K_h[t] / sqrt(d) and LSE the causal row log-sum-exp.
//
// Two passes over the causal score matrix on MFMA (v_mfma_f32_16x16x32_f16,
// fp16 inputs, fp32 accumulation):
//   score_lse_kernel     workgroup = 128 query rows of one query head; walks
//                        the key tiles up to its last row, keeps a per-lane
//                        online (max, sum), then merges across lanes.
//   score_colsum_kernel  workgroup = 128 keys of one KV head; walks every
//                        query tile at or after the keys (last tile first,
//                        the G query heads innermost, so the workgroups of a
//                        KV head read the same tiles at the same time),
//                        summing exp2(s' - LSE') down each key column.  A
//                        key block is owned by one workgroup, so no atomics
//                        and the summation order is fixed.
// Each wave keeps 32 rows of its resident operand (Q rows, or K rows) in
// registers as two 16-row MFMA fragments, so every fragment of the streamed
// 64-row tile it reads from LDS feeds two products.  The streamed tiles go
// straight from memory into a three-stage LDS ring (no registers), two tiles
// ahead of the one being multiplied.  Masks are applied only on diagonal and
// ragged tiles; tiles entirely outside a wave's triangle are skipped by that
// wave.  Plus two bandwidth kernels: var_tok (one wave per token) and the
// column norms behind w_chan (partial sums in fp64, reduced in a fixed order).
#include "lds_dma.h"
#include "rdkv_internal.h"

namespace rdkv {
namespace {

using dma::buffer_rsrc4;
using dma::lds_addr;
using dma::rsrc4;
using dma::wait_vmem;

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kKT = 64;                     // rows of the streamed LDS tile (keys, or query rows)
constexpr int kWaveRows = 32;               // rows of the resident operand per wave (two 16-row fragments)
constexpr int kBlockRows = 4 * kWaveRows;   // per workgroup
constexpr int kThreads = 256;
constexpr float kLog2eOverSqrtD = 1.4426950408889634f / 11.313708498984761f;
constexpr int kNormSplits = 64;
constexpr int kRunTiles = 8;   // pass-2 tiles summed in fp32 before moving into fp64 (<= 32 terms of at most 1)

struct ScoreArgs {
  int64_t N;
  int32_t Hq, Hkv, G;
  const __half* Q;
  const __half* K;
  float* lse;      // [S*L][Hq][N], log-sum-exp of the scaled scores: base 2, times lse_scale on output
  float* w_tok;    // [S*L][Hkv][N]
  float lse_scale; // pass 1 writes (base-2 LSE) * lse_scale: 1, or ln 2 for a natural-log LSE
};

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- LDS tiles
// A streamed tile is 64 rows x 128 halves (16 KiB) in LDS without padding;
// the 16-byte piece c of row r sits at piece c ^ (r % 16) of its row, so the
// 16 rows one fragment read touches fall in 16 distinct bank groups.  Tiles
// are copied global -> LDS by buffer_load_dwordx4 ... lds (no registers), in
// a ring of kStages tiles issued kStages - 1 tiles ahead: each wave copies
// 16 rows with 4 instructions.  The copies are inline assembly, so the
// compiler's memory-counter bookkeeping does not see them; the loops wait for
// them explicitly.
constexpr int kStages = 3;
constexpr int kTileBytes = kKT * kHeadDim * 2;
// Per-lane range offsets of a wave's 4 copies: copy j fills LDS bytes
// 1024 j + 16 lane of the wave's quarter, i.e. row 4 j + lane / 16, piece
// p = lane % 16, which holds the row's piece p ^ (row % 16).  The instruction
// offset (1024 j) moves the range offset too, so it is taken out here.
struct CopyOffsets {
  uint32_t v[4];
};
__device__ inline CopyOffsets copy_offsets() {
  const int lane = threadIdx.x & 63;
  CopyOffsets o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * j + (lane >> 4), c = (lane & 15) ^ (r & 15);
    o.v[j] = uint32_t(256 * (lane >> 4) + 16 * c);
  }
  return o;
}

// The wave's 16 rows (row0 .. row0 + 15 of src, each 256 bytes) into LDS at
// byte lds; rows at or past N arrive as zeros without being read.
__device__ inline void copy_rows16(const __half* src, int64_t row0, int64_t N, const CopyOffsets& o, uint32_t lds) {
  const int64_t left = N - row0;
  const uint32_t bytes = left <= 0 ? 0u : left >= 16 ? 4096u : uint32_t(left) * 256u;
  const rsrc4 r = buffer_rsrc4(src + row0 * kHeadDim, bytes);
  lds = __builtin_amdgcn_readfirstlane(lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %6\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %1, %5, 0 offen offset:0 lds\n\t"
      "buffer_load_dwordx4 %2, %5, 0 offen offset:1024 lds\n\t"
      "buffer_load_dwordx4 %3, %5, 0 offen offset:2048 lds\n\t"
      "buffer_load_dwordx4 %4, %5, 0 offen offset:3072 lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(o.v[0]), "v"(o.v[1]), "v"(o.v[2]), "v"(o.v[3]), "s"(r), "s"(lds)
      : "memory");
}

// 64 fp32 values (src[row0 .. row0 + 63], zeros at or past N) into LDS at
// byte lds, one dword per lane.
__device__ inline void copy_floats64(const float* src, int64_t row0, int64_t N, uint32_t lds) {
  const int64_t left = N - row0;
  const uint32_t bytes = left <= 0 ? 0u : left >= 64 ? 256u : uint32_t(left) * 4u;
  const rsrc4 r = buffer_rsrc4(src + row0, bytes);
  const uint32_t voff = 4u * (threadIdx.x & 63);
  lds = __builtin_amdgcn_readfirstlane(lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
      "buffer_load_dword %1, %2, 0 offen offset:0 lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(r), "s"(lds)
      : "memory");
}

// A-operand fragments of 16 rows for the 16x16x32 MFMA: lane holds row
// (lane % 16), halves 32*kk + 8*(lane/16) .. +7 for kk = 0..3.
__device__ inline void load_rows_frag(h8 (&a)[4], const __half* src, int64_t row, int64_t N) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < N) v = *reinterpret_cast<const uint4*>(src + row * kHeadDim + 32 * kk + 8 * (lane >> 4));
    a[kk] = __builtin_bit_cast(h8, v);
  }
}

// B-operand fragments of rows 16*sub .. 16*sub + 15 of an LDS tile, in the
// same k order as the A fragments (piece 4 kk + lane / 16 of the row).
__device__ inline void load_tile_frag(h8 (&b)[4], const _Float16 (*tile)[kHeadDim], int sub) {
  const int lane = threadIdx.x & 63;
  const _Float16* trow = &tile[16 * sub + (lane & 15)][0];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) b[kk] = *reinterpret_cast<const h8*>(trow + 8 * (((lane >> 4) + 4 * kk) ^ (lane & 15)));
}

// C[i][j] = sum_k A[i][k] * B[j][k] over k = 0..127 for 16 rows of A and 16 of
// B.  Lane holds C[4*(lane/16) + r][lane % 16].
__device__ inline f4 mfma_16x16x128(const h8 (&a)[4], const h8 (&b)[4]) {
  f4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[kk], b[kk], c, 0, 0, 0);
  return c;
}

// max(a, b, c) in one instruction (inputs are finite or -inf).
__device__ inline float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// One key tile of pass 1 for a wave's 32 rows: scores c by MFMA, then per
// row the running sum s = sum exp2(c * k - mk) (k = log2(e) / sqrt(d)) over a
// reference mk, a maximum of the row's scores (times k) seen so far.  The
// reference is raised only when a tile's terms for some row sum past 2^64,
// which after the first tile needs a score 64 base-2 units above it: the tile
// is then redone over the raised reference (the branch is wave-uniform and
// rare).  Terms below the reference's own scale lose nothing that matters, and
// s stays far below the fp32 range.  mk starts at -FLT_MAX, not -inf, so a
// visible score always overflows the first tile's sum and masked scores (-inf)
// give exact zeros.  kEdge: keys after a row, or at or past N, are masked.
constexpr float kRaiseBound = 18446744073709551616.0f;   // 2^64
template <bool kEdge>
__device__ inline void lse_tile(const h8 (&qa)[2][4], const _Float16 (*cur)[kHeadDim], int key0, int wrow0, int N,
                                float (&mk)[2][4], float (&s)[2][4]) {
  const int lane = threadIdx.x & 63;
  float c[2][4][4];   // [fragment][sub][r]
  // The products at raised wave priority: a wave with MFMAs to issue goes
  // ahead of the waves busy with exponentials, which keeps the matrix pipe
  // fed.  (The priority changes also bound the compiler's reordering: the
  // tile then fits 136 registers instead of spilling at 168.)
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int sub = 0; sub < 4; ++sub) {
    h8 b[4];
    load_tile_frag(b, cur, sub);
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const f4 v = mfma_16x16x128(qa[f], b);
#pragma unroll
      for (int r = 0; r < 4; ++r) c[f][sub][r] = v[r];
    }
  }
  __builtin_amdgcn_s_setprio(0);
  if constexpr (kEdge) {
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int sub = 0; sub < 4; ++sub)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = key0 + 16 * sub + (lane & 15);
          const int row = wrow0 + 16 * f + 4 * (lane >> 4) + r;
          if (key > row || key >= N) c[f][sub][r] = -INFINITY;
        }
  }
  float t[2][4];
  bool big = false;
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float e[4];
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) e[sub] = __builtin_amdgcn_exp2f(fmaf(c[f][sub][r], kLog2eOverSqrtD, -mk[f][r]));
      t[f][r] = (e[0] + e[1]) + (e[2] + e[3]);
      big = big || !(t[f][r] <= kRaiseBound);
    }
  if (__builtin_amdgcn_ballot_w64(big) != 0) {
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float cm = fmaxf(fmaxf(c[f][0][r], c[f][1][r]), fmaxf(c[f][2][r], c[f][3][r]));
        const float mnew = fmaxf(mk[f][r], cm * kLog2eOverSqrtD);
        s[f][r] *= __builtin_amdgcn_exp2f(mk[f][r] - mnew);
        mk[f][r] = mnew;
        float e[4];
#pragma unroll
        for (int sub = 0; sub < 4; ++sub) e[sub] = __builtin_amdgcn_exp2f(fmaf(c[f][sub][r], kLog2eOverSqrtD, -mnew));
        t[f][r] = (e[0] + e[1]) + (e[2] + e[3]);
      }
  }
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) s[f][r] += t[f][r];
}

// Pass 1: workgroup = 128 query rows of one query head (32 per wave, two
// 16-row fragments sharing every K fragment read from LDS); walks the key
// tiles up to the block's last row.  Per lane and row an online (max, sum),
// merged across the 16 lanes of a row at the end in base 2.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void score_lse_kernel(ScoreArgs a) {
  __shared__ _Float16 ks[kStages][kKT][kHeadDim];
  const int64_t N = a.N;
  const int nqb = int(cdiv(N, kBlockRows));
  const int qb = nqb - 1 - int(blockIdx.x);   // long rows first
  const int hq = blockIdx.y;
  const int64_t sl = blockIdx.z;
  const int h = hq / a.G;
  const __half* Qh = a.Q + ((sl * a.Hq + hq) * N) * kHeadDim;
  const __half* Kh = a.K + ((sl * a.Hkv + h) * N) * kHeadDim;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t wrow0 = int64_t(qb) * kBlockRows + kWaveRows * wave;       // the wave's first row
  const int n_kt = int(cdiv(min(N, int64_t(qb + 1) * kBlockRows), kKT));   // key tiles the block needs

  h8 qa[2][4];
  load_rows_frag(qa[0], Qh, wrow0 + (lane & 15), N);
  load_rows_frag(qa[1], Qh, wrow0 + 16 + (lane & 15), N);
  float mk[2][4], s[2][4];   // reference (base 2), sum
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      mk[f][r] = -__FLT_MAX__;
      s[f][r] = 0.f;
    }
  const CopyOffsets co = copy_offsets();
  const uint32_t lds0 = lds_addr(&ks[0][0][0]) + uint32_t(kTileBytes / 4) * wave;
  auto issue = [&](int kt) {
    copy_rows16(Kh, int64_t(kt) * kKT + 16 * wave, N, co, lds0 + uint32_t(kTileBytes) * (kt % kStages));
  };
  issue(0);
  if (n_kt > 1) issue(1);
  for (int kt = 0; kt < n_kt; ++kt) {
    if (kt + 1 < n_kt) wait_vmem<4>();   // this wave's copies of tile kt have landed
    else wait_vmem<0>();
    __syncthreads();                     // ... and every wave's; tile kt - 1 is no longer read
    if (kt + 2 < n_kt) issue(kt + 2);
    const int64_t key0 = int64_t(kt) * kKT;
    // (wave-uniform) skip a tile whose keys all lie after the wave's rows
    if (key0 <= wrow0 + kWaveRows - 1 && wrow0 < N) {
      const _Float16 (*cur)[kHeadDim] = ks[kt % kStages];
      // diagonal or ragged tile: masks; otherwise every key precedes every row
      if (key0 + kKT - 1 > wrow0 || key0 + kKT > N) {
        lse_tile<true>(qa, cur, int(key0), int(wrow0), int(N), mk, s);
      } else {
        lse_tile<false>(qa, cur, int(key0), int(wrow0), int(N), mk, s);
      }
    }
  }
  // merge the 16 lanes that hold the same rows
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float mm = mk[f][r], ss = s[f][r];
#pragma unroll
      for (int x = 1; x < 16; x <<= 1) {
        const float mo = __shfl_xor(mm, x, 64), so = __shfl_xor(ss, x, 64);
        const float mn = fmaxf(mm, mo);   // (references are finite)
        ss = ss * exp2f(mm - mn) + so * exp2f(mo - mn);
        mm = mn;
      }
      const int64_t row = wrow0 + 16 * f + 4 * (lane >> 4) + r;
      if ((lane & 15) == 0 && row < N) a.lse[(sl * a.Hq + hq) * N + row] = (mm + log2f(ss)) * a.lse_scale;
    }
}

// One query tile of pass 2 for a wave's 32 keys: scores by MFMA and
// exp2(t - LSE) summed per key into fp32 run sums (each term is at most 1; the
// caller moves them into fp64 totals every few tiles).  kEdge: queries before
// a key, or at or past N, are masked.
template <bool kEdge>
__device__ inline void colsum_tile(const h8 (&ka)[2][4], const _Float16 (*cur)[kHeadDim], const float* lse, int qrow0,
                                   int wkey0, int N, float (&run)[2][4]) {
  const int lane = threadIdx.x & 63;
  f4 c[4][2];   // [sub][fragment]: every product of the tile first, then the exponentials
  __builtin_amdgcn_s_setprio(1);   // (as in pass 1)
#pragma unroll
  for (int sub = 0; sub < 4; ++sub) {
    h8 b[4];
    load_tile_frag(b, cur, sub);
#pragma unroll
    for (int f = 0; f < 2; ++f) c[sub][f] = mfma_16x16x128(ka[f], b);
  }
  __builtin_amdgcn_s_setprio(0);
#pragma unroll
  for (int sub = 0; sub < 4; ++sub) {
    const int query = qrow0 + 16 * sub + (lane & 15);
    const float lq = lse[16 * sub + (lane & 15)];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(c[sub][f][r], kLog2eOverSqrtD, -lq));
        if constexpr (kEdge) {
          const int key = wkey0 + 16 * f + 4 * (lane >> 4) + r;
          run[f][r] += (query < key || query >= N) ? 0.f : e;
        } else {
          run[f][r] += e;
        }
      }
  }
}

// Pass 2: workgroup = 128 keys of one KV head (32 per wave, two 16-key
// fragments sharing every Q fragment read from LDS); walks the G query heads
// and every 64-row query tile at or after the block's first key, summing
// exp2(t - LSE) down each key column.  A key block is owned by one
// workgroup, so no atomics and the summation order is fixed.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void score_colsum_kernel(ScoreArgs a) {
  __shared__ _Float16 qs[kStages][kKT][kHeadDim];
  __shared__ float ls[kStages][kKT];
  const int64_t N = a.N;
  const int nqt = int(cdiv(N, kKT));
  const int kb = blockIdx.x;                  // short key indices have the most rows: first
  const int h = blockIdx.y;
  const int64_t sl = blockIdx.z;
  const __half* Kh = a.K + ((sl * a.Hkv + h) * N) * kHeadDim;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t wkey0 = int64_t(kb) * kBlockRows + kWaveRows * wave;     // the wave's first key

  h8 ka[2][4];
  load_rows_frag(ka[0], Kh, wkey0 + (lane & 15), N);
  load_rows_frag(ka[1], Kh, wkey0 + 16 + (lane & 15), N);
  double tot[2][4] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
  float run[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  int n_run = 0;   // tiles summed into run since the last move into tot
  auto flush = [&]() {
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        tot[f][r] += double(run[f][r]);
        run[f][r] = 0.f;
      }
    n_run = 0;
  };
  const int qt0 = int(int64_t(kb) * kBlockRows / kKT);
  const int n_steps = a.G * (nqt - qt0);
  // steps walk the query tiles from the last one back to qt0, the G heads
  // innermost, so the workgroups of one KV head read the same tiles together
  int f_g = 0, f_qt = nqt - 1;   // the next tile to copy
  const CopyOffsets co = copy_offsets();
  const uint32_t q_lds0 = lds_addr(&qs[0][0][0]) + uint32_t(kTileBytes / 4) * wave;
  const uint32_t l_lds0 = lds_addr(&ls[0][0]);
  // copies of step f into stage f % kStages: 4 per wave, plus the 64 LSE
  // values by wave 0
  auto issue = [&](int f) {
    const int64_t hq = int64_t(h) * a.G + f_g;
    const __half* Qh = a.Q + ((sl * a.Hq + hq) * N) * kHeadDim;
    const int64_t row0 = int64_t(f_qt) * kKT;
    copy_rows16(Qh, row0 + 16 * wave, N, co, q_lds0 + uint32_t(kTileBytes) * (f % kStages));
    if (wave == 0) copy_floats64(a.lse + (sl * a.Hq + hq) * N, row0, N, l_lds0 + uint32_t(kKT * 4) * (f % kStages));
    if (++f_g == a.G) {
      f_g = 0;
      --f_qt;
    }
  };
  issue(0);
  if (n_steps > 1) issue(1);
  int qt = nqt - 1, g_cur = 0;   // the current tile
  for (int st = 0; st < n_steps; ++st) {
    // this wave's copies of step st have landed (wave 0 issues 5 per step)
    if (st + 1 < n_steps) {
      if (wave == 0) wait_vmem<5>();
      else wait_vmem<4>();
    } else {
      wait_vmem<0>();
    }
    __syncthreads();   // ... and every wave's; step st - 1 is no longer read
    if (st + 2 < n_steps) issue(st + 2);
    const int buf = st % kStages;
    const int64_t qrow0 = int64_t(qt) * kKT;
    if (++g_cur == a.G) {
      g_cur = 0;
      --qt;
    }
    // (wave-uniform) skip a tile whose rows all lie before the wave's keys
    if (qrow0 + kKT - 1 >= wkey0 && wkey0 < N) {
      // diagonal or ragged tile: masks; otherwise every row follows every key
      if (qrow0 < wkey0 + kWaveRows - 1 || qrow0 + kKT > N) {
        colsum_tile<true>(ka, qs[buf], ls[buf], int(qrow0), int(wkey0), int(N), run);
      } else {
        colsum_tile<false>(ka, qs[buf], ls[buf], int(qrow0), int(wkey0), int(N), run);
      }
      if (++n_run == kRunTiles) flush();
    }
  }
  flush();
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      double v = tot[f][r];
#pragma unroll
      for (int x = 1; x < 16; x <<= 1) v += __shfl_xor(v, x, 64);
      const int64_t key = wkey0 + 16 * f + 4 * (lane >> 4) + r;
      if ((lane & 15) == 0 && key < N) a.w_tok[(sl * a.Hkv + h) * N + key] = float(v);
    }
}

// A natural-log LSE (as a prefill attention forward returns it) in base 2.
__global__ __launch_bounds__(kThreads) void lse_to_base2_kernel(const float* in, float* out, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i < n) out[i] = in[i] * 1.4426950408889634f;
}

// Population variance of each V row: one wave per token, two passes in registers.
__global__ __launch_bounds__(kThreads) void var_tok_kernel(const __half* V, float* var, int64_t rows) {
  const int64_t row = int64_t(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const uint32_t w = reinterpret_cast<const uint32_t*>(V + row * kHeadDim)[lane];
  const float v0 = half_lo(w), v1 = half_hi(w);
  const float mean = wave_sum(v0 + v1) * (1.0f / kHeadDim);
  const float d0 = v0 - mean, d1 = v1 - mean;
  const float ss = wave_sum(fmaf(d0, d0, d1 * d1));
  if (lane == 0) var[row] = ss * (1.0f / kHeadDim);
}

// Partial column sums of squares of the group's Q rows and of K, per split of
// the token range: part[seg][split][0][c] (Q) and [1][c] (K), fp64.
__global__ __launch_bounds__(kThreads) void chan_norm_partial_kernel(ScoreArgs a, double* part) {
  const int64_t seg = blockIdx.y;              // (s*L + l)*Hkv + h
  const int split = blockIdx.x;
  const int64_t N = a.N;
  const int h = int(seg % a.Hkv);
  const int64_t sl = seg / a.Hkv;
  const int c = threadIdx.x & (kHeadDim - 1), tr = threadIdx.x / kHeadDim;   // 2 row lanes
  constexpr int kRowLanes = kThreads / kHeadDim;
  const int64_t per = cdiv(N, kNormSplits);
  const int64_t t0 = split * per, t1 = min(N, t0 + per);
  double sq = 0.0, sk = 0.0;
  const __half* Kh = a.K + ((sl * a.Hkv + h) * N) * kHeadDim;
  for (int64_t t = t0 + tr; t < t1; t += kRowLanes) {
    const float k = __half2float(Kh[t * kHeadDim + c]);
    sk += double(k) * k;
  }
  for (int g = 0; g < a.G; ++g) {
    const __half* Qh = a.Q + ((sl * a.Hq + h * a.G + g) * N) * kHeadDim;
    for (int64_t t = t0 + tr; t < t1; t += kRowLanes) {
      const float q = __half2float(Qh[t * kHeadDim + c]);
      sq += double(q) * q;
    }
  }
  __shared__ double s_q[kRowLanes][kHeadDim], s_k[kRowLanes][kHeadDim];
  s_q[tr][c] = sq;
  s_k[tr][c] = sk;
  __syncthreads();
  if (tr == 0) {
    for (int r = 1; r < kRowLanes; ++r) {
      sq += s_q[r][c];
      sk += s_k[r][c];
    }
    double* out = part + ((seg * kNormSplits + split) * 2) * kHeadDim;
    out[c] = sq;
    out[kHeadDim + c] = sk;
  }
}

__global__ void chan_norm_final_kernel(const double* part, float* w_chan) {
  const int64_t seg = blockIdx.x;
  const int c = threadIdx.x;
  double sq = 0.0, sk = 0.0;
  for (int s = 0; s < kNormSplits; ++s) {
    sq += part[((seg * kNormSplits + s) * 2) * kHeadDim + c];
    sk += part[((seg * kNormSplits + s) * 2 + 1) * kHeadDim + c];
  }
  w_chan[seg * kHeadDim + c] = float(sqrt(sq) * sqrt(sk) / sqrt(double(kHeadDim)));
}

}  // namespace

size_t score_workspace_bytes(int64_t S, int64_t L, int64_t Hq, int64_t N) {
  // LSE per query row, then fp64 partial norms per (segment, split); the
  // segment count is at most S*L*Hq.
  const size_t lse = align_up(uint64_t(S * L * Hq * N) * sizeof(float), kAlign);
  return lse + size_t(S * L * Hq) * kNormSplits * 2 * kHeadDim * sizeof(double);
}

namespace {

ScoreArgs score_args(const ScoreParams& p, float lse_scale) {
  return ScoreArgs{p.n_tokens, p.Hq, p.Hkv, p.Hq / p.Hkv, p.Q, p.K, p.lse, p.w_tok, lse_scale};
}

void launch_pass1(const ScoreParams& p, float lse_scale, hipStream_t stream, LaunchErrors& le) {
  const unsigned nb = unsigned(cdiv(p.n_tokens, kBlockRows));
  hipLaunchKernelGGL(score_lse_kernel, dim3(nb, unsigned(p.Hq), unsigned(int64_t(p.S) * p.L)), dim3(kThreads), 0,
                     stream, score_args(p, lse_scale));
  le.check();
}

// Pass 2 from the base-2 LSE in p.lse, then var_tok and w_chan.
hipError_t launch_rest(const ScoreParams& p, hipStream_t stream, LaunchErrors& le) {
  const ScoreArgs a = score_args(p, 1.0f);
  const int64_t SL = int64_t(p.S) * p.L;
  const unsigned nb = unsigned(cdiv(p.n_tokens, kBlockRows));
  hipLaunchKernelGGL(score_colsum_kernel, dim3(nb, unsigned(p.Hkv), unsigned(SL)), dim3(kThreads), 0, stream, a);
  le.check();
  const int64_t rows = SL * p.Hkv * p.n_tokens;
  hipLaunchKernelGGL(var_tok_kernel, dim3(unsigned(cdiv(rows, kThreads / 64))), dim3(kThreads), 0, stream, p.V,
                     p.var_tok, rows);
  le.check();
  double* part = reinterpret_cast<double*>(reinterpret_cast<uint8_t*>(p.lse) +
                                           align_up(uint64_t(SL * p.Hq * p.n_tokens) * sizeof(float), kAlign));
  const int64_t n_seg = SL * p.Hkv;
  hipLaunchKernelGGL(chan_norm_partial_kernel, dim3(kNormSplits, unsigned(n_seg)), dim3(kThreads), 0, stream, a, part);
  le.check();
  hipLaunchKernelGGL(chan_norm_final_kernel, dim3(unsigned(n_seg)), dim3(kHeadDim), 0, stream, part, p.w_chan);
  le.check();
  return le.status();
}

}  // namespace

hipError_t launch_score(const ScoreParams& p, hipStream_t stream) {
  LaunchErrors le;
  launch_pass1(p, 1.0f, stream, le);
  return launch_rest(p, stream, le);
}

hipError_t launch_score_lse(const ScoreParams& p, hipStream_t stream) {
  LaunchErrors le;
  launch_pass1(p, 0.69314718055994531f, stream, le);
  return le.status();
}

hipError_t launch_score_from_lse(const ScoreParams& p, hipStream_t stream) {
  LaunchErrors le;
  const int64_t n = int64_t(p.S) * p.L * p.Hq * p.n_tokens;
  if (n > 0) {
    hipLaunchKernelGGL(lse_to_base2_kernel, dim3(unsigned(cdiv(n, kThreads))), dim3(kThreads), 0, stream, p.lse_in,
                       p.lse, n);
    le.check();
  }
  return launch_rest(p, stream, le);
}

}  // namespace rdkv
