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
//   score_colsum_kernel  workgroup = 128 keys of one KV head; walks the G
//                        query heads and every query tile at or after the
//                        keys, summing exp2(s' - LSE') down each key column.
//                        A key block is owned by one workgroup, so no atomics
//                        and the summation order is fixed.
// Each wave keeps 32 rows of its resident operand (Q rows, or K rows) in
// registers as two 16-row MFMA fragments, so every fragment of the streamed
// 64-row tile it reads from LDS feeds two products.  The streamed tile is
// double buffered in LDS: the next tile's global loads are in flight while the
// current one is multiplied.  Masks are applied only on diagonal and ragged
// tiles; tiles entirely outside a wave's triangle are skipped by that wave.
// Plus two bandwidth kernels: var_tok (one wave per token) and the column
// norms behind w_chan (partial sums in fp64, reduced in a fixed order).
#include "rdkv_internal.h"

namespace rdkv {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kKT = 64;                     // rows of the streamed LDS tile (keys, or query rows)
constexpr int kWaveRows = 32;               // rows of the resident operand per wave (two 16-row fragments)
constexpr int kBlockRows = 4 * kWaveRows;   // per workgroup
constexpr int kPad = kHeadDim + 8;  // LDS row stride in halves (272 bytes)
constexpr int kThreads = 256;
constexpr float kLog2eOverSqrtD = 1.4426950408889634f / 11.313708498984761f;
constexpr int kNormSplits = 64;

struct ScoreArgs {
  int64_t N;
  int32_t Hq, Hkv, G;
  const __half* Q;
  const __half* K;
  float* lse;      // [S*L][Hq][N], base-2 log-sum-exp of the scaled scores
  float* w_tok;    // [S*L][Hkv][N]
};

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

// A 64 x 128 fp16 tile moving global -> registers -> LDS: each thread holds
// 4 of its 1024 16-byte pieces; rows >= N are 0.
struct TileRegs {
  uint4 v[4];
};
__device__ inline void tile_fetch(TileRegs& t, const __half* src, int64_t row0, int64_t N) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = threadIdx.x + kThreads * i, r = idx >> 4, c = idx & 15;
    t.v[i] = row0 + r < N ? reinterpret_cast<const uint4*>(src + (row0 + r) * kHeadDim)[c] : make_uint4(0, 0, 0, 0);
  }
}
__device__ inline void tile_store(const TileRegs& t, _Float16 (*tile)[kPad]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = threadIdx.x + kThreads * i, r = idx >> 4, c = idx & 15;
    *reinterpret_cast<uint4*>(&tile[r][c * 8]) = t.v[i];
  }
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
// same k order as the A fragments.
__device__ inline void load_tile_frag(h8 (&b)[4], const _Float16 (*tile)[kPad], int sub) {
  const int lane = threadIdx.x & 63;
  const _Float16* trow = &tile[16 * sub + (lane & 15)][8 * (lane >> 4)];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) b[kk] = *reinterpret_cast<const h8*>(trow + 32 * kk);
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
// reference mk = m * k.  The reference m is the row's maximum score when it was
// last raised; it is raised (and s rescaled) only when a score exceeds it by
// more than kSlack / k, so the terms stay below 2^kSlack and, after the first
// tiles, most tiles rescale nothing.  kEdge: keys after a row, or at or past
// N, are masked.
constexpr float kSlack = 8.0f;   // base-2 headroom of a term above the reference
template <bool kEdge>
__device__ inline void lse_tile(const h8 (&qa)[2][4], const _Float16 (*cur)[kPad], int key0, int wrow0, int N,
                                float (&thr)[2][4], float (&mk)[2][4], float (&s)[2][4]) {
  const int lane = threadIdx.x & 63;
  float c[2][4][4];   // [fragment][sub][r]
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
  float cm[2][4];
  bool up = false;
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      cm[f][r] = fmaxf(max3f(c[f][0][r], c[f][1][r], c[f][2][r]), c[f][3][r]);
      up = up || cm[f][r] > thr[f][r];
    }
  if (__builtin_amdgcn_ballot_w64(up) != 0) {   // (wave-uniform; rare after the first tiles)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (cm[f][r] > thr[f][r]) {
          const float mnew = cm[f][r] * kLog2eOverSqrtD;
          s[f][r] *= __builtin_amdgcn_exp2f(mk[f][r] - mnew);   // (0 while nothing was seen)
          mk[f][r] = mnew;
          thr[f][r] = cm[f][r] + kSlack / kLog2eOverSqrtD;
        }
  }
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (kEdge) {
        if (mk[f][r] == -INFINITY) continue;   // nothing visible to this row yet
      }
      float acc = s[f][r];
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) acc += __builtin_amdgcn_exp2f(fmaf(c[f][sub][r], kLog2eOverSqrtD, -mk[f][r]));
      s[f][r] = acc;
    }
}

// Pass 1: workgroup = 128 query rows of one query head (32 per wave, two
// 16-row fragments sharing every K fragment read from LDS); walks the key
// tiles up to the block's last row.  Per lane and row an online (max, sum),
// merged across the 16 lanes of a row at the end in base 2.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void score_lse_kernel(ScoreArgs a) {
  __shared__ _Float16 ks[2][kKT][kPad];
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
  float thr[2][4], mk[2][4], s[2][4];   // raise threshold (raw units), reference (base 2), sum
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      thr[f][r] = -INFINITY;
      mk[f][r] = -INFINITY;
      s[f][r] = 0.f;
    }
  TileRegs nxt;
  tile_fetch(nxt, Kh, 0, N);
  tile_store(nxt, ks[0]);
  for (int kt = 0; kt < n_kt; ++kt) {
    if (kt + 1 < n_kt) tile_fetch(nxt, Kh, int64_t(kt + 1) * kKT, N);
    __syncthreads();
    const int64_t key0 = int64_t(kt) * kKT;
    // (wave-uniform) skip a tile whose keys all lie after the wave's rows
    if (key0 <= wrow0 + kWaveRows - 1 && wrow0 < N) {
      const _Float16 (*cur)[kPad] = ks[kt & 1];
      // diagonal or ragged tile: masks; otherwise every key precedes every row
      if (key0 + kKT - 1 > wrow0 || key0 + kKT > N) {
        lse_tile<true>(qa, cur, int(key0), int(wrow0), int(N), thr, mk, s);
      } else {
        lse_tile<false>(qa, cur, int(key0), int(wrow0), int(N), thr, mk, s);
      }
    }
    if (kt + 1 < n_kt) tile_store(nxt, ks[(kt + 1) & 1]);
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
        const float mn = fmaxf(mm, mo);
        if (mn != -INFINITY) {
          ss = (mm == -INFINITY ? 0.f : ss * exp2f(mm - mn)) + (mo == -INFINITY ? 0.f : so * exp2f(mo - mn));
          mm = mn;
        }
      }
      const int64_t row = wrow0 + 16 * f + 4 * (lane >> 4) + r;
      if ((lane & 15) == 0 && row < N) a.lse[(sl * a.Hq + hq) * N + row] = mm + log2f(ss);
    }
}

// One query tile of pass 2 for a wave's 32 keys: scores by MFMA and
// exp2(t - LSE) summed per key, added to the fp64 totals.  kEdge: queries
// before a key, or at or past N, are masked.
template <bool kEdge>
__device__ inline void colsum_tile(const h8 (&ka)[2][4], const _Float16 (*cur)[kPad], const float* lse, int qrow0,
                                   int wkey0, int N, double (&tot)[2][4]) {
  const int lane = threadIdx.x & 63;
  float part[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int sub = 0; sub < 4; ++sub) {
    h8 b[4];
    load_tile_frag(b, cur, sub);
    const int query = qrow0 + 16 * sub + (lane & 15);
    const float lq = lse[16 * sub + (lane & 15)];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const f4 c = mfma_16x16x128(ka[f], b);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(c[r], kLog2eOverSqrtD, -lq));
        if constexpr (kEdge) {
          const int key = wkey0 + 16 * f + 4 * (lane >> 4) + r;
          part[f][r] += (query < key || query >= N) ? 0.f : e;
        } else {
          part[f][r] += e;
        }
      }
    }
  }
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) tot[f][r] += double(part[f][r]);
}

// Pass 2: workgroup = 128 keys of one KV head (32 per wave, two 16-key
// fragments sharing every Q fragment read from LDS); walks the G query heads
// and every 64-row query tile at or after the block's first key, summing
// exp2(t - LSE) down each key column.  A key block is owned by one
// workgroup, so no atomics and the summation order is fixed.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void score_colsum_kernel(ScoreArgs a) {
  __shared__ _Float16 qs[2][kKT][kPad];
  __shared__ float ls[2][kKT];
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
  // steps: (g, qt) for g in heads, qt in [qt0, nqt)
  const int qt0 = int(int64_t(kb) * kBlockRows / kKT);
  const int per = nqt - qt0, n_steps = a.G * per;
  auto step_src = [&](int st, const __half*& Qh, const float*& lse, int& qt) {
    const int g = st / per;
    qt = qt0 + st % per;
    const int hq = h * a.G + g;
    Qh = a.Q + ((sl * a.Hq + hq) * N) * kHeadDim;
    lse = a.lse + (sl * a.Hq + hq) * N;
  };
  TileRegs nxt;
  float lnext = 0.f;
  auto fetch = [&](int st) {
    const __half* Qh;
    const float* lse;
    int qt;
    step_src(st, Qh, lse, qt);
    tile_fetch(nxt, Qh, int64_t(qt) * kKT, N);
    if (threadIdx.x < kKT) {
      const int64_t row = int64_t(qt) * kKT + threadIdx.x;
      lnext = row < N ? lse[row] : 0.f;
    }
  };
  auto store = [&](int buf) {
    tile_store(nxt, qs[buf]);
    if (threadIdx.x < kKT) ls[buf][threadIdx.x] = lnext;
  };
  fetch(0);
  store(0);
  for (int st = 0; st < n_steps; ++st) {
    if (st + 1 < n_steps) fetch(st + 1);
    __syncthreads();
    const int buf = st & 1;
    const int64_t qrow0 = int64_t(qt0 + st % per) * kKT;
    // (wave-uniform) skip a tile whose rows all lie before the wave's keys
    if (qrow0 + kKT - 1 >= wkey0 && wkey0 < N) {
      // diagonal or ragged tile: masks; otherwise every row follows every key
      if (qrow0 < wkey0 + kWaveRows - 1 || qrow0 + kKT > N) {
        colsum_tile<true>(ka, qs[buf], ls[buf], int(qrow0), int(wkey0), int(N), tot);
      } else {
        colsum_tile<false>(ka, qs[buf], ls[buf], int(qrow0), int(wkey0), int(N), tot);
      }
    }
    if (st + 1 < n_steps) store((st + 1) & 1);
  }
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

hipError_t launch_score(const ScoreParams& p, hipStream_t stream) {
  const int G = p.Hq / p.Hkv;
  ScoreArgs a{p.n_tokens, p.Hq, p.Hkv, G, p.Q, p.K, p.lse, p.w_tok};
  const int64_t SL = int64_t(p.S) * p.L;
  const unsigned nb = unsigned(cdiv(p.n_tokens, kBlockRows));
  hipLaunchKernelGGL(score_lse_kernel, dim3(nb, unsigned(p.Hq), unsigned(SL)), dim3(kThreads), 0, stream, a);
  hipLaunchKernelGGL(score_colsum_kernel, dim3(nb, unsigned(p.Hkv), unsigned(SL)), dim3(kThreads), 0, stream, a);
  const int64_t rows = SL * p.Hkv * p.n_tokens;
  hipLaunchKernelGGL(var_tok_kernel, dim3(unsigned(cdiv(rows, kThreads / 64))), dim3(kThreads), 0, stream, p.V,
                     p.var_tok, rows);
  double* part = reinterpret_cast<double*>(reinterpret_cast<uint8_t*>(p.lse) +
                                           align_up(uint64_t(SL * p.Hq * p.n_tokens) * sizeof(float), kAlign));
  const int64_t n_seg = SL * p.Hkv;
  hipLaunchKernelGGL(chan_norm_partial_kernel, dim3(kNormSplits, unsigned(n_seg)), dim3(kThreads), 0, stream, a, part);
  hipLaunchKernelGGL(chan_norm_final_kernel, dim3(unsigned(n_seg)), dim3(kHeadDim), 0, stream, part, p.w_chan);
  return hipGetLastError();
}

}  // namespace rdkv
