// Lagrangian bit allocation (RDKV summary, section 2.1 objective, section 2.2
// "reverse water-filling", stages 2 and 3).
//
// For one segment and one problem (V tokens, or K channels) with unit costs
// c_u = fl32(w_u * sigma_u), unit u takes step j of the staircase
// 0 -> 2 -> 4 -> 8 -> 16 bits iff c_u * k_j > lambda, k = (3/8, 3/32, 15/1024,
// 255/524288); those are the exact per-bit gains of c * 2^-b, all five
// bitwidths lie on the unit's lower convex hull, and the rule is the per-unit
// argmin of c 2^-b + lambda b with ties at the lower bitwidth.  lambda* is the
// smallest value whose total bits fit the budget.  The total is a step
// function of lambda that only changes at the products c_u * k_j, which are
// exact in fp64, so a bisection over the ordered bit patterns of non-negative
// doubles (at most 63 halvings) lands exactly on lambda*.
//
// A budget may be shared by a group of consecutive segments (the heads of a
// layer, or all of a sequence): the group's units then form one problem with
// one lambda, the same rule over their union.
//
// Stage 3's unit variance is the exact population variance of a K channel over
// the kept tokens: fp16 values are integers times 2^-24, so the sums are done
// in 64- and 128-bit integers and the quotient is rounded once to fp32.
#include "rdkv_internal.h"

namespace rdkv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__device__ inline int64_t block_sum64(int v, int64_t* s_red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_i(v);
  __syncthreads();
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  int64_t t = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t += s_red[w];
  return t;
}

__device__ inline float block_max(float v, float* s_red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  float t = s_red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) t = fmaxf(t, s_red[w]);
  return t;
}

// Bits of one unit for a multiplier lambda: sum of the steps with c*k_j > lambda.
__device__ inline int unit_bits(float c, double lam) {
  const double cd = double(c);
  return 2 * (cd * 0.375 > lam) + 2 * (cd * 0.09375 > lam) + 4 * (cd * (15.0 / 1024.0) > lam) +
         8 * (cd * (255.0 / 524288.0) > lam);
}

// lambda* for the units this thread sees through `cost_of`, shared by the block.
template <typename CostFn>
__device__ double find_lambda(float cmax, int64_t budget, CostFn cost_of) {
  if (cost_of(0.0) <= budget) return 0.0;
  // invariant: cost(pattern lo) > budget >= cost(pattern hi)
  uint64_t lo = 0;
  uint64_t hi = __double_as_longlong(double(cmax) * 0.375);
  while (hi - lo > 1) {
    const uint64_t mid = lo + (hi - lo) / 2;
    if (cost_of(__longlong_as_double(mid)) <= budget)
      hi = mid;
    else
      lo = mid;
  }
  return __longlong_as_double(hi);
}

// The same lambda* found by radix selection instead of bisection, for
// problems of many units.  The total bits at lambda is W(> lambda), the
// weighted count (weights 2, 2, 4, 8) of the products p = c_u * k_j above it,
// and lambda* is the product p* with W(> p*) <= budget < W(>= p*).  Non-negative
// doubles order as their bit patterns, so p* is fixed one digit of its pattern
// at a time, top down: a weighted histogram of the digit over the products
// that match the digits fixed so far, then the digit where the count from
// above crosses the budget.  The first digit is the whole exponent (products
// then spread over many buckets, so the LDS atomics seldom collide), then
// 8-bit digits of the mantissa: 8 passes over the units instead of up to 63.
// cost0 is the total at lambda = 0 (every product of a positive cost).
constexpr int kSelBuckets = 2048;
constexpr int kUnitBatch = 4;   // units a thread loads together
template <typename CostAt>
__device__ double select_lambda(int64_t n, int64_t budget, int64_t cost0, CostAt cost_at,
                                unsigned long long* s_hist, unsigned long long* s_state) {
  if (cost0 <= budget) return 0.0;
  const unsigned long long B = (unsigned long long)budget;
  if (threadIdx.x == 0) s_state[0] = 0, s_state[1] = 0;   // weight above the prefix, prefix
  // digits: bits 52-63 (sign and exponent), then 44-51, ..., 4-11, then 0-3
#pragma unroll 1
  for (int pass = 0; pass < 8; ++pass) {
    const int width = pass == 0 ? 12 : pass == 7 ? 4 : 8;
    const int shift = pass == 0 ? 52 : pass == 7 ? 0 : 52 - 8 * pass;
    const int nb = 1 << width;
    for (int i = threadIdx.x; i < nb; i += kThreads) s_hist[i] = 0;
    __syncthreads();
    const unsigned long long prefix = s_state[1];
    const unsigned long long fixed = pass == 0 ? 0ull : ~0ull << (shift + width);
    const unsigned long long dmask = (unsigned long long)(nb - 1);
    for (int64_t t0 = threadIdx.x; t0 < n; t0 += int64_t(kThreads) * kUnitBatch) {
      float c[kUnitBatch];
#pragma unroll
      for (int u = 0; u < kUnitBatch; ++u) {
        const int64_t t = t0 + int64_t(u) * kThreads;
        c[u] = t < n ? cost_at(t) : 0.0f;   // (a zero cost has no positive product: never counted)
      }
#pragma unroll
      for (int u = 0; u < kUnitBatch; ++u) {
        if (!(c[u] > 0.0f)) continue;
        const double cd = double(c[u]);
        const double pj[4] = {cd * 0.375, cd * 0.09375, cd * (15.0 / 1024.0), cd * (255.0 / 524288.0)};
        const unsigned wj[4] = {2, 2, 4, 8};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const unsigned long long pat = __double_as_longlong(pj[j]);
          if ((pat & fixed) == (prefix & fixed)) atomicAdd(&s_hist[(pat >> shift) & dmask], (unsigned long long)wj[j]);
        }
      }
    }
    __syncthreads();
    // wave 0: lane L sums buckets [L C, L C + C); the lane where the weight
    // from above crosses the budget scans its buckets top down
    if (threadIdx.x < 64) {
      const int L = threadIdx.x, C = nb >= 64 ? nb / 64 : 1;
      unsigned long long sl = 0;
      if (L * C < nb)
        for (int i = 0; i < C; ++i) sl += s_hist[L * C + i];
      unsigned long long incl = sl;   // weight of lanes >= L
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const unsigned long long o = __shfl_down(incl, off);
        if (L + off < 64) incl += o;
      }
      const unsigned long long above = s_state[0], strictly = above + (incl - sl);
      if (strictly <= B && above + incl > B) {   // exactly one lane (weights are non-negative)
        unsigned long long acc = strictly;
        int d = L * C + C - 1;
        for (; d > L * C; --d) {
          if (acc + s_hist[d] > B) break;
          acc += s_hist[d];
        }
        s_state[0] = acc;
        s_state[1] = prefix | ((unsigned long long)d << shift);
      }
    }
    __syncthreads();
  }
  return __longlong_as_double(s_state[1]);
}

struct AllocVArgs {
  int64_t N;
  int32_t group;       // consecutive segments sharing the budget
  const float* w_tok;
  const float* var_tok;
  int64_t budget;
  uint8_t* bits_tok;
  double* lambda;
};

// One workgroup per group of segments: its group * N tokens are one problem.
// (A thread's bit count stays far below 2^31; the block total is 64-bit.)
__global__ __launch_bounds__(kThreads) void alloc_v_kernel(AllocVArgs a) {
  __shared__ int64_t s_i[kWaves];
  __shared__ unsigned long long s_hist[kSelBuckets], s_state[2];
  const int64_t n = a.N * a.group;
  const int64_t base = int64_t(blockIdx.x) * n;
  const float* w = a.w_tok + base;
  const float* v = a.var_tok + base;
  int k0 = 0;   // bits at lambda = 0: 16 per unit of positive cost
#pragma unroll 4
  for (int64_t t = threadIdx.x; t < n; t += kThreads) k0 += __fmul_rn(w[t], v[t]) > 0.0f ? 16 : 0;
  const int64_t cost0 = block_sum64(k0, s_i);
  const double lam = select_lambda(n, a.budget, cost0, [&](int64_t t) { return __fmul_rn(w[t], v[t]); }, s_hist,
                                   s_state);
  for (int64_t t = threadIdx.x; t < n; t += kThreads) a.bits_tok[base + t] = uint8_t(unit_bits(__fmul_rn(w[t], v[t]), lam));
  for (int s = threadIdx.x; s < a.group; s += kThreads) a.lambda[2 * (int64_t(blockIdx.x) * a.group + s)] = lam;
}

// ---------------------------------------------------------------- exact variance

struct U128 {
  uint64_t hi, lo;
};
__device__ inline U128 add128(U128 a, U128 b) {
  U128 r;
  r.lo = a.lo + b.lo;
  r.hi = a.hi + b.hi + (r.lo < a.lo);
  return r;
}
__device__ inline U128 sub128(U128 a, U128 b) {
  U128 r;
  r.lo = a.lo - b.lo;
  r.hi = a.hi - b.hi - (a.lo < b.lo);
  return r;
}
__device__ inline U128 mul64(uint64_t a, uint64_t b) { return U128{__umul64hi(a, b), a * b}; }
__device__ inline U128 mul128_64(U128 a, uint64_t b) {   // low 128 bits of a*b
  U128 r = mul64(a.lo, b);
  r.hi += a.hi * b;
  return r;
}
__device__ inline int bitlen64(uint64_t x) { return x ? 64 - __clzll(x) : 0; }

// Nearest-even fp32 of (M / D) * 2^e2 for M < 2^127, 1 <= D < 2^62; the result
// must be a normal fp32 (true for every variance of fp16 data).
__device__ float round_div_to_f32(U128 M, uint64_t D, int e2) {
  if (M.hi == 0 && M.lo == 0) return 0.0f;
  const int mb = M.hi ? 64 + bitlen64(M.hi) : bitlen64(M.lo);
  const int db = bitlen64(D);
  const int s = 26 - (mb - db);   // floor(M 2^s / D) lies in [2^25, 2^27)
  uint64_t num;
  bool sticky = false;
  if (s >= 0) {
    num = M.lo << s;               // M < 2^(db + 26 - s) <= 2^64 here
  } else {
    const int r = -s;
    if (r >= 64) {
      num = M.hi >> (r - 64);
      sticky = M.lo != 0 || (r > 64 && (M.hi & ((uint64_t(1) << (r - 64)) - 1)) != 0);
    } else {
      num = (M.lo >> r) | (M.hi << (64 - r));
      sticky = (M.lo & ((uint64_t(1) << r) - 1)) != 0;
    }
  }
  uint64_t q = num / D;
  sticky = sticky || (num - q * D) != 0;
  const int drop = bitlen64(q) - 24;
  uint64_t m = q >> drop;
  const uint64_t rb = q & ((uint64_t(1) << drop) - 1), half = uint64_t(1) << (drop - 1);
  if (rb > half || (rb == half && (sticky || (m & 1)))) ++m;
  int e = drop - s + e2;
  if (m == (uint64_t(1) << 24)) {
    m >>= 1;
    ++e;
  }
  return ldexpf(float(m), e);
}

struct AllocKArgs {
  int64_t N;
  int32_t group;       // consecutive segments sharing the budget
  const __half* K;
  const uint8_t* bits_tok;
  const float* w_chan;
  int64_t budget;
  uint8_t* bits_chan;
  float* var_chan;
  double* lambda;
};

// One workgroup per segment: the exact variance of each K channel over the
// segment's kept tokens.  A thread takes 8 channels of a row with one 16-byte
// load (16 threads per row, 64 rows in flight); the integer sums are merged
// across the rows' threads by shuffles, then across waves in LDS (exact, so
// the order does not matter).
__global__ __launch_bounds__(kThreads) void alloc_kvar_kernel(AllocKArgs a) {
  constexpr int kCB = kHeadDim / 8;            // 8-channel blocks per row
  constexpr int kRowLanes = kThreads / kCB;    // rows in flight
  __shared__ int64_t s_i[kWaves];
  __shared__ int64_t s_s1[kWaves][kHeadDim];
  __shared__ U128 s_s2[kWaves][kHeadDim];
  const int64_t seg = blockIdx.x;
  const int cb = threadIdx.x % kCB, tr = threadIdx.x / kCB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint4* Kseg = reinterpret_cast<const uint4*>(a.K + seg * a.N * kHeadDim);
  const uint8_t* bt = a.bits_tok + seg * a.N;

  // exact sums of X = x * 2^24 and X^2 over kept tokens, channels 8 cb + e
  int64_t s1[8];
  U128 s2[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    s1[e] = 0;
    s2[e] = U128{0, 0};
  }
  int n = 0;
  for (int64_t t = tr; t < a.N; t += kRowLanes) {
    if (bits_group(bt[t]) < 0) continue;
    const uint4 v = Kseg[t * kCB + cb];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = (e & 1) ? half_hi(w[e >> 1]) : half_lo(w[e >> 1]);
      const int64_t X = int64_t(double(x) * 16777216.0);
      s1[e] += X;
      const uint64_t ax = uint64_t(X < 0 ? -X : X);
      s2[e] = add128(s2[e], mul64(ax, ax));
    }
    ++n;
  }
  // the wave's 4 row lanes of each channel block: lanes cb, cb + 16, cb + 32, cb + 48
#pragma unroll
  for (int x = 16; x < 64; x <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s1[e] += __shfl_xor(s1[e], x, 64);
      const U128 o{__shfl_xor(s2[e].hi, x, 64), __shfl_xor(s2[e].lo, x, 64)};
      s2[e] = add128(s2[e], o);
    }
  if (lane < kCB) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s_s1[wave][8 * cb + e] = s1[e];
      s_s2[wave][8 * cb + e] = s2[e];
    }
  }
  n = int(block_sum64(n, s_i) / kCB);   // every kept row counted by its kCB threads
  __syncthreads();
  if (threadIdx.x < kHeadDim) {
    const int c = threadIdx.x;
    int64_t S1 = 0;
    U128 S2{0, 0};
    for (int w = 0; w < kWaves; ++w) {
      S1 += s_s1[w][c];
      S2 = add128(S2, s_s2[w][c]);
    }
    float var = 0.0f;
    if (n > 0) {
      const uint64_t a1 = uint64_t(S1 < 0 ? -S1 : S1);
      const U128 M = sub128(mul128_64(S2, uint64_t(n)), mul64(a1, a1));   // n*S2 - S1^2 >= 0
      var = round_div_to_f32(M, uint64_t(n) * uint64_t(n), -48);
    }
    a.var_chan[seg * kHeadDim + c] = var;
  }
}

// One workgroup per group of segments: the group * 128 channels are one
// problem with unit costs fl32(w_chan * var_chan).
__global__ __launch_bounds__(kThreads) void alloc_kbits_kernel(AllocKArgs a) {
  __shared__ int64_t s_i[kWaves];
  __shared__ float s_f[kWaves];
  const int64_t n = int64_t(kHeadDim) * a.group;
  const int64_t base = int64_t(blockIdx.x) * n;
  auto cost_at = [&](int64_t u) { return __fmul_rn(a.w_chan[base + u], a.var_chan[base + u]); };
  float cmax = 0.0f;
  for (int64_t u = threadIdx.x; u < n; u += kThreads) {
    const float cc = cost_at(u);
    if (cc > cmax) cmax = cc;
  }
  cmax = block_max(cmax, s_f);
  auto cost = [&](double lam) {
    int k = 0;
    for (int64_t u = threadIdx.x; u < n; u += kThreads) k += unit_bits(cost_at(u), lam);
    return block_sum64(k, s_i);
  };
  const double lam = find_lambda(cmax, a.budget, cost);
  for (int64_t u = threadIdx.x; u < n; u += kThreads) a.bits_chan[base + u] = uint8_t(unit_bits(cost_at(u), lam));
  for (int s = threadIdx.x; s < a.group; s += kThreads) a.lambda[2 * (int64_t(blockIdx.x) * a.group + s) + 1] = lam;
}

}  // namespace

hipError_t launch_allocate(const AllocParams& p, hipStream_t stream) {
  const unsigned n_groups = unsigned(p.n_seg / p.group);
  AllocVArgs va{p.n_tokens, p.group, p.w_tok, p.var_tok, p.budget_v, p.bits_tok, p.lambda};
  hipLaunchKernelGGL(alloc_v_kernel, dim3(n_groups), dim3(kThreads), 0, stream, va);
  AllocKArgs ka{p.n_tokens, p.group, p.K, p.bits_tok, p.w_chan, p.budget_k, p.bits_chan, p.var_chan, p.lambda};
  hipLaunchKernelGGL(alloc_kvar_kernel, dim3(unsigned(p.n_seg)), dim3(kThreads), 0, stream, ka);
  hipLaunchKernelGGL(alloc_kbits_kernel, dim3(n_groups), dim3(kThreads), 0, stream, ka);
  return hipGetLastError();
}

}  // namespace rdkv
