// Stage-1 scoring after prefill (RDKV summary, section 2.1 weights, section
// 2.2 stage 1: computed once on the full uncompressed cache).
//
//   w_tok[h][t] = sum_{g in group(h)} sum_{tau >= t} exp(s_{g,tau,t} - LSE_{g,tau})
//   with s = Q_g[tau].K_h[t] / sqrt(d) and LSE the causal row log-sum-exp.
//
// Two passes over the causal score matrix on MFMA (v_mfma_f32_16x16x32_f16,
// fp16 inputs, fp32 accumulation):
//   score_lse_kernel     workgroup = 64 query rows of one query head; walks the
//                        key blocks 0..diagonal, keeps a per-lane online
//                        (max, sum) in base 2, then merges across lanes.
//   score_colsum_kernel  workgroup = 64 keys of one KV head; walks the G query
//                        heads and every query block at or after the keys,
//                        summing exp2(s' - LSE') down each key column.  A key
//                        block is owned by one workgroup, so no atomics and the
//                        summation order is fixed.
// The streamed 64x128 tile (K rows, or Q rows and their LSE) is double
// buffered in LDS: the next tile's global loads are in flight while the
// current one is multiplied.  Masks are applied only on the diagonal block
// and the ragged last block.
// Plus two bandwidth kernels: var_tok (one wave per token) and the column
// norms behind w_chan (partial sums in fp64, reduced in a fixed order).
#include "rdkv_internal.h"

namespace rdkv {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kB = 64;           // rows per block (queries or keys)
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

// C[i][j] = sum_k A[i][k] * T[16*sub + j][k] for the wave's 16 rows of A and
// 16 rows of the LDS tile T (B fragments in the same k order as A).  Lane
// holds C[4*(lane/16) + r][lane % 16].
__device__ inline f4 tile_product(const h8 (&a)[4], const _Float16 (*tile)[kPad], int sub) {
  const int lane = threadIdx.x & 63;
  f4 c = {0.f, 0.f, 0.f, 0.f};
  const _Float16* trow = &tile[16 * sub + (lane & 15)][8 * (lane >> 4)];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const h8 b = *reinterpret_cast<const h8*>(trow + 32 * kk);
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[kk], b, c, 0, 0, 0);
  }
  return c;
}

__global__ __launch_bounds__(kThreads) void score_lse_kernel(ScoreArgs a) {
  __shared__ _Float16 ks[2][kB][kPad];
  const int64_t N = a.N;
  const int nqb = int(cdiv(N, kB));
  const int qb = nqb - 1 - int(blockIdx.x);   // long rows first
  const int hq = blockIdx.y;
  const int64_t sl = blockIdx.z;
  const int h = hq / a.G;
  const __half* Qh = a.Q + ((sl * a.Hq + hq) * N) * kHeadDim;
  const __half* Kh = a.K + ((sl * a.Hkv + h) * N) * kHeadDim;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row0 = int64_t(qb) * kB + 16 * wave;

  h8 qa[4];
  load_rows_frag(qa, Qh, row0 + (lane & 15), N);
  float m[4], s[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m[r] = -INFINITY;
    s[r] = 0.f;
  }
  TileRegs nxt;
  tile_fetch(nxt, Kh, 0, N);
  tile_store(nxt, ks[0]);
  for (int kb = 0; kb <= qb; ++kb) {
    if (kb < qb) tile_fetch(nxt, Kh, int64_t(kb + 1) * kB, N);
    __syncthreads();
    const _Float16 (*cur)[kPad] = ks[kb & 1];
    const bool edge = kb == qb || int64_t(kb + 1) * kB > N;   // diagonal or ragged block
    float t[4][4];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const f4 c = tile_product(qa, cur, sub);
      const int64_t key = int64_t(kb) * kB + 16 * sub + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = row0 + 4 * (lane >> 4) + r;
        t[sub][r] = (edge && (key > row || key >= N)) ? -INFINITY : c[r] * kLog2eOverSqrtD;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float mb = fmaxf(fmaxf(t[0][r], t[1][r]), fmaxf(t[2][r], t[3][r]));
      const float mn = fmaxf(m[r], mb);
      if (mn == -INFINITY) continue;
      float acc = s[r];
      if (mn > m[r]) acc = m[r] == -INFINITY ? 0.f : acc * __builtin_amdgcn_exp2f(m[r] - mn);
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) acc += __builtin_amdgcn_exp2f(t[sub][r] - mn);
      s[r] = acc;
      m[r] = mn;
    }
    if (kb < qb) tile_store(nxt, ks[(kb + 1) & 1]);
  }
  // merge the 16 lanes that hold the same rows
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int x = 1; x < 16; x <<= 1) {
      const float mo = __shfl_xor(m[r], x, 64), so = __shfl_xor(s[r], x, 64);
      const float mn = fmaxf(m[r], mo);
      if (mn != -INFINITY) {
        s[r] = (m[r] == -INFINITY ? 0.f : s[r] * exp2f(m[r] - mn)) + (mo == -INFINITY ? 0.f : so * exp2f(mo - mn));
        m[r] = mn;
      }
    }
    const int64_t row = row0 + 4 * (lane >> 4) + r;
    if ((lane & 15) == 0 && row < N) a.lse[(sl * a.Hq + hq) * N + row] = m[r] + log2f(s[r]);
  }
}

__global__ __launch_bounds__(kThreads) void score_colsum_kernel(ScoreArgs a) {
  __shared__ _Float16 qs[2][kB][kPad];
  __shared__ float ls[2][kB];
  const int64_t N = a.N;
  const int nqb = int(cdiv(N, kB));
  const int kb = blockIdx.x;                  // short key indices have the most rows: first
  const int h = blockIdx.y;
  const int64_t sl = blockIdx.z;
  const __half* Kh = a.K + ((sl * a.Hkv + h) * N) * kHeadDim;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t key0 = int64_t(kb) * kB + 16 * wave;

  h8 ka[4];
  load_rows_frag(ka, Kh, key0 + (lane & 15), N);
  double tot[4] = {0.0, 0.0, 0.0, 0.0};
  // steps: (g, qb) for g in heads, qb in [kb, nqb)
  const int per = nqb - kb, n_steps = a.G * per;
  auto step_src = [&](int st, const __half*& Qh, const float*& lse, int& qb) {
    const int g = st / per;
    qb = kb + st % per;
    const int hq = h * a.G + g;
    Qh = a.Q + ((sl * a.Hq + hq) * N) * kHeadDim;
    lse = a.lse + (sl * a.Hq + hq) * N;
  };
  TileRegs nxt;
  float lnext = 0.f;
  auto fetch = [&](int st) {
    const __half* Qh;
    const float* lse;
    int qb;
    step_src(st, Qh, lse, qb);
    tile_fetch(nxt, Qh, int64_t(qb) * kB, N);
    if (threadIdx.x < kB) {
      const int64_t row = int64_t(qb) * kB + threadIdx.x;
      lnext = row < N ? lse[row] : 0.f;
    }
  };
  auto store = [&](int buf) {
    tile_store(nxt, qs[buf]);
    if (threadIdx.x < kB) ls[buf][threadIdx.x] = lnext;
  };
  fetch(0);
  store(0);
  for (int st = 0; st < n_steps; ++st) {
    if (st + 1 < n_steps) fetch(st + 1);
    __syncthreads();
    const int buf = st & 1;
    const int qb = kb + st % per;
    const bool edge = qb == kb || int64_t(qb + 1) * kB > N;
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const f4 c = tile_product(ka, qs[buf], sub);
      const int64_t query = int64_t(qb) * kB + 16 * sub + (lane & 15);
      const float lq = ls[buf][16 * sub + (lane & 15)];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t key = key0 + 4 * (lane >> 4) + r;
        const float e = __builtin_amdgcn_exp2f(fmaf(c[r], kLog2eOverSqrtD, -lq));
        part[r] += (edge && (query < key || query >= N)) ? 0.f : e;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) tot[r] += double(part[r]);
    if (st + 1 < n_steps) store((st + 1) & 1);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    double v = tot[r];
#pragma unroll
    for (int x = 1; x < 16; x <<= 1) v += __shfl_xor(v, x, 64);
    const int64_t key = key0 + 4 * (lane >> 4) + r;
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
  const unsigned nb = unsigned(cdiv(p.n_tokens, kB));
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
