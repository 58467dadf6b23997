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
// exact in fp64, so a radix selection over the ordered bit patterns of
// non-negative doubles lands exactly on lambda*.
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

// Bits of one unit for a multiplier lambda: sum of the steps with c*k_j > lambda.
__device__ inline int unit_bits(float c, double lam) {
  const double cd = double(c);
  return 2 * (cd * 0.375 > lam) + 2 * (cd * 0.09375 > lam) + 4 * (cd * (15.0 / 1024.0) > lam) +
         8 * (cd * (255.0 / 524288.0) > lam);
}

// lambda* by radix selection.  The total bits at lambda is W(> lambda), the
// weighted count (weights 2, 2, 4, 8) of the products p = c_u * k_j above it,
// and lambda* is the product p* with W(> p*) <= budget < W(>= p*), or 0 when
// every product fits.  Non-negative doubles order as their bit patterns, so p*
// is fixed one digit of its pattern at a time, top down: a weighted histogram
// of the digit over the products that match the digits fixed so far, then the
// digit where the weight from above crosses the budget.  The first digit is
// the exponent, then six 8-bit digits of the mantissa and a last 4-bit one:
// 8 passes over the units.  A problem that fits one workgroup runs all passes
// in it (alloc_one_kernel: the K channels, and short V problems); a long V
// problem takes one launch per pass (sel_pass_kernel): its units are split
// over many workgroups, each adding its LDS histogram to the group's
// histogram in the workspace (integer sums, so the order of the additions does
// not matter); the next launch's workgroups fix that digit from it.
constexpr int kSelBuckets = 2048;
constexpr int kSelPasses = 8;
constexpr int kSelThreads = 256;
constexpr int kUnitBatch = 8;   // units a thread loads together: their loads are all in flight at once

// Digit `pass`: bits [shift, shift + width) of the pattern.  Bit 63 (the
// sign) is 0 for every product, so the first digit is the 11-bit exponent.
__host__ __device__ constexpr int sel_width(int pass) { return pass == 0 ? 11 : pass == kSelPasses - 1 ? 4 : 8; }
__host__ __device__ constexpr int sel_shift(int pass) {
  return pass == 0 ? 52 : pass == kSelPasses - 1 ? 0 : 52 - 8 * pass;
}
static_assert(sel_shift(kSelPasses - 1) == 0 && sel_shift(kSelPasses - 2) == sel_width(kSelPasses - 1) &&
                  sel_shift(0) + sel_width(0) == 63 && sel_shift(1) + sel_width(1) == sel_shift(0),
              "the digits tile bits 0-62 of the pattern");
static_assert((1 << sel_width(0)) == kSelBuckets && (1 << sel_width(1)) <= kSelBuckets, "a digit's buckets fit");

// A group's selection state: weight of the products above the prefix, the
// prefix (the digits fixed so far), and a flag for "every product fits".
enum { kStAbove = 0, kStPrefix = 1, kStDone = 2, kStWords = 4 };

struct SelArgs {
  int64_t n;                   // units per group (group * N tokens, or group * 128 channels)
  int32_t blocks;              // workgroups per group
  int32_t pass;
  const float* w;              // unit weights [groups][n]: w_tok, or w_chan
  const float* sigma;          // unit variances [groups][n]: var_tok, or var_chan
  unsigned long long* hist;    // [groups][kSelBuckets]
  unsigned long long* state;   // [groups][kStWords]
};

// Units [lo, hi) of workgroup blk of a problem of n units split over `blocks`.
__device__ inline void block_range(int64_t n, int blocks, int blk, int64_t& lo, int64_t& hi) {
  lo = n * blk / blocks;
  hi = n * (blk + 1) / blocks;
}

// c[u] = fl32(w * sigma) of unit t0 + u * kSelThreads (0 at or past hi: a zero
// cost has no positive product, so it is never counted).
__device__ inline void load_costs(const float* w, const float* v, int64_t t0, int64_t hi, float (&c)[kUnitBatch]) {
#pragma unroll
  for (int u = 0; u < kUnitBatch; ++u) {
    const int64_t t = t0 + int64_t(u) * kSelThreads;
    c[u] = t < hi ? __fmul_rn(w[t], v[t]) : 0.0f;
  }
}

__global__ __launch_bounds__(256) void fill_u64_kernel(unsigned long long* p, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x) p[i] = 0;
}

// Adds to s_hist (LDS, zero on entry for the digit's buckets) the weights of
// the products of units [lo, hi) (this thread: lo + threadIdx.x, then every
// kSelThreads-th) whose higher digits match `prefix`.
__device__ void histogram_digit(const float* w, const float* v, int64_t lo, int64_t hi, int pass,
                                unsigned long long prefix, unsigned long long* s_hist) {
  const int width = sel_width(pass), shift = sel_shift(pass);
  const unsigned long long fixed = pass == 0 ? 0ull : ~0ull << (shift + width);
  const unsigned long long dmask = (1ull << width) - 1;
  for (int64_t t0 = lo + threadIdx.x; t0 < hi; t0 += int64_t(kSelThreads) * kUnitBatch) {
    float c[kUnitBatch];
    load_costs(w, v, t0, hi, c);
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
}

// Called by one whole wave with a group's complete histogram h of digit
// `pass` and its state before that digit, st_in (LDS or global memory):
// writes to st_out the state with the digit fixed.  Lane L sums buckets
// [L C, L C + C); the lane where the weight from above crosses the budget B
// scans its buckets top down.  With `clear`, each lane then zeroes its own
// buckets for the next pass.  st_out may be st_in.
__device__ void pick_digit(unsigned long long* h, const unsigned long long* st_in, unsigned long long* st_out,
                           int pass, unsigned long long B, bool clear) {
  const int shift = sel_shift(pass), nb = 1 << sel_width(pass);
  const int L = threadIdx.x & 63, C = nb >= 64 ? nb / 64 : 1;
  const bool mine = L * C < nb;
  unsigned long long sl = 0;
  if (mine)
    for (int i = 0; i < C; ++i) sl += h[L * C + i];
  unsigned long long incl = sl;   // weight of lanes >= L
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long o = __shfl_down(incl, off);
    if (L + off < 64) incl += o;
  }
  const unsigned long long above = st_in[kStAbove], prefix = st_in[kStPrefix], done = st_in[kStDone];
  const unsigned long long total = __shfl(incl, 0);
  if (L == 0) {
    st_out[kStAbove] = above;
    st_out[kStPrefix] = prefix;
    st_out[kStDone] = done;
  }
  if (done) {
    // nothing left to fix
  } else if (pass == 0 && total <= B) {   // every product fits: lambda* = 0 (the prefix stays 0)
    if (L == 0) st_out[kStDone] = 1;
  } else {
    const unsigned long long strictly = above + (incl - sl);
    if (strictly <= B && above + incl > B) {   // exactly one lane (weights are non-negative)
      unsigned long long acc = strictly;
      int d = L * C + C - 1;
      for (; d > L * C; --d) {
        if (acc + h[d] > B) break;
        acc += h[d];
      }
      st_out[kStAbove] = acc;
      st_out[kStPrefix] = prefix | ((unsigned long long)d << shift);
    }
  }
  if (clear && mine)   // (after this lane's own reads of its buckets)
    for (int i = 0; i < C; ++i) h[L * C + i] = 0;
}

// Bits of units [lo, hi) of a group for its lambda*.
__device__ void write_bits(const float* w, const float* v, int64_t lo, int64_t hi, double lam, uint8_t* bt) {
  for (int64_t t0 = lo + threadIdx.x; t0 < hi; t0 += int64_t(kSelThreads) * kUnitBatch) {
    float c[kUnitBatch];
    load_costs(w, v, t0, hi, c);
#pragma unroll
    for (int u = 0; u < kUnitBatch; ++u) {
      const int64_t t = t0 + int64_t(u) * kSelThreads;
      if (t < hi) bt[t] = uint8_t(unit_bits(c[u], lam));
    }
  }
}

// The group's histograms and states in the workspace: three histogram
// buffers in rotation (pass p fills buffer p mod 3, reads buffer p - 1 mod 3
// and clears buffer p + 1 mod 3, which pass p - 1 read), and two state slots
// (the state after digit d in slot d mod 2).
constexpr int kHistBufs = 3, kStSlots = 2;

// Pass p over many workgroups per group.  Every workgroup first fixes digit
// p - 1 itself from the complete histogram of the previous launch (the same
// integer arithmetic everywhere, so the same digit), and its first workgroup
// stores that state for the next launch; then each histograms its share of
// the group's units for digit p and adds it to the group's buffer.
__global__ __launch_bounds__(kSelThreads) void sel_pass_kernel(SelArgs a, int64_t budget) {
  __shared__ unsigned long long s_hist[kSelBuckets];
  __shared__ unsigned long long s_st[kStWords];
  const int64_t g = blockIdx.x / a.blocks;
  const int blk = int(blockIdx.x % a.blocks);
  const int p = a.pass;
  unsigned long long* hist = a.hist + g * kHistBufs * kSelBuckets;
  unsigned long long* state = a.state + g * kStSlots * kStWords;
  if (p == 0) {
    if (threadIdx.x < kStWords) s_st[threadIdx.x] = 0;
  } else if (threadIdx.x < 64) {
    pick_digit(hist + ((p - 1) % kHistBufs) * kSelBuckets, state + ((p - 2) & 1) * kStWords, s_st, p - 1,
               (unsigned long long)budget, false);
  }
  __syncthreads();
  if (blk == 0 && p > 0 && threadIdx.x < kStWords) state[((p - 1) & 1) * kStWords + threadIdx.x] = s_st[threadIdx.x];
  if (s_st[kStDone]) return;   // (uniform)
  unsigned long long* next = hist + ((p + 1) % kHistBufs) * kSelBuckets;
  for (int i = blk * kSelThreads + threadIdx.x; i < kSelBuckets; i += a.blocks * kSelThreads) next[i] = 0;
  const int nb = 1 << sel_width(p);
  for (int i = threadIdx.x; i < nb; i += kSelThreads) s_hist[i] = 0;
  __syncthreads();
  int64_t lo, hi;
  block_range(a.n, a.blocks, blk, lo, hi);
  histogram_digit(a.w + g * a.n, a.sigma + g * a.n, lo, hi, p, s_st[kStPrefix], s_hist);
  __syncthreads();
  unsigned long long* gh = hist + (p % kHistBufs) * kSelBuckets;
  for (int i = threadIdx.x; i < nb; i += kSelThreads)
    if (s_hist[i]) atomicAdd(&gh[i], s_hist[i]);
}

// After the last pass: every workgroup fixes the last digit (lambda*), writes
// the bits of its share of the V tokens, and the first one lambda_V of the
// group's segments.
__global__ __launch_bounds__(kSelThreads) void alloc_v_bits_kernel(SelArgs a, int64_t budget, int32_t group,
                                                                   uint8_t* bits_tok, double* lambda) {
  __shared__ unsigned long long s_st[kStWords];
  const int64_t g = blockIdx.x / a.blocks;
  const int blk = int(blockIdx.x % a.blocks);
  constexpr int kLast = kSelPasses - 1;
  if (threadIdx.x < 64)
    pick_digit(a.hist + (g * kHistBufs + kLast % kHistBufs) * kSelBuckets,
               a.state + (g * kStSlots + ((kLast - 1) & 1)) * kStWords, s_st, kLast, (unsigned long long)budget,
               false);
  __syncthreads();
  const double lam = __longlong_as_double((long long)s_st[kStPrefix]);
  int64_t lo, hi;
  block_range(a.n, a.blocks, blk, lo, hi);
  write_bits(a.w + g * a.n, a.sigma + g * a.n, lo, hi, lam, bits_tok + g * a.n);
  if (blk == 0)
    for (int s = threadIdx.x; s < group; s += kSelThreads) lambda[2 * (g * group + s)] = lam;
}

// A whole problem of a group in one workgroup (small problems: the histogram
// and state stay in LDS, one launch instead of 17): the V tokens, or the K
// channels (units c = fl32(w_chan * var_chan), the same rule), whose lambda
// goes to lambda[2 seg + lam_slot].
__global__ __launch_bounds__(kSelThreads) void alloc_one_kernel(SelArgs a, int64_t budget, int32_t group,
                                                                uint8_t* bits, double* lambda, int32_t lam_slot) {
  __shared__ unsigned long long s_hist[kSelBuckets];
  __shared__ unsigned long long s_st[kStWords];
  const int64_t g = blockIdx.x;
  const float* w = a.w + g * a.n;
  const float* v = a.sigma + g * a.n;
  for (int i = threadIdx.x; i < kSelBuckets; i += kSelThreads) s_hist[i] = 0;
  if (threadIdx.x < kStWords) s_st[threadIdx.x] = 0;
  __syncthreads();
  for (int pass = 0; pass < kSelPasses; ++pass) {
    if (s_st[kStDone]) break;   // (uniform)
    histogram_digit(w, v, 0, a.n, pass, s_st[kStPrefix], s_hist);
    __syncthreads();
    if (threadIdx.x < 64) pick_digit(s_hist, s_st, s_st, pass, (unsigned long long)budget, true);
    __syncthreads();
  }
  const double lam = __longlong_as_double((long long)s_st[kStPrefix]);
  write_bits(w, v, 0, a.n, lam, bits + g * a.n);
  for (int s = threadIdx.x; s < group; s += kSelThreads) lambda[2 * (g * group + s) + lam_slot] = lam;
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

// Population variance (n S2 - S1^2) / n^2 of n values X 2^-24 with sums S1 of
// X and S2 of X^2, rounded once to fp32 (0 for n = 0).
__device__ inline float channel_variance(int64_t S1, U128 S2, int64_t n) {
  if (n <= 0) return 0.0f;
  const uint64_t a1 = uint64_t(S1 < 0 ? -S1 : S1);
  const U128 M = sub128(mul128_64(S2, uint64_t(n)), mul64(a1, a1));   // n*S2 - S1^2 >= 0
  return round_div_to_f32(M, uint64_t(n) * uint64_t(n), -48);
}

struct AllocKArgs {
  int64_t N;
  int32_t group;       // consecutive segments sharing the budget
  int32_t blocks;      // workgroups per segment for the sums
  const __half* K;
  const uint8_t* bits_tok;
  const float* w_chan;
  int64_t budget;
  uint8_t* bits_chan;
  float* var_chan;
  double* lambda;
  int64_t* s1;         // [n_seg][blocks][128] partial sums of X
  U128* s2;            // [n_seg][blocks][128] partial sums of X^2
  int64_t* cnt;        // [n_seg][blocks] kept tokens
};

// Exact sums of each K channel over a segment's kept tokens, the segment's
// tokens split over `blocks` workgroups by 64-token tiles dealt round robin
// (tile i to workgroup i mod blocks), so a run of kept tokens (the recent
// window, the sinks) is spread over many workgroups.  A workgroup takes its
// tiles kTilesPerBatch at a time: their bit widths are read with all loads in
// flight and the kept tokens listed in LDS (list order is free: the sums are
// exact), then a thread takes 8 channels of a listed row with one 16-byte load
// (16 threads per row, 16 rows in flight, kRowBatch rows per thread loaded
// together).  The sums are merged across the rows' threads by shuffles, then
// across waves in LDS, and written as the workgroup's partial sums.
constexpr int kKThreads = 256;
constexpr int kKWaves = kKThreads / 64;
constexpr int kKeepPerThread = 8;
constexpr int kKeepBatch = kKThreads * kKeepPerThread;
constexpr int kKTile = 64;
constexpr int kTilesPerBatch = kKeepBatch / kKTile;
static_assert(kKTile == 64 && kTilesPerBatch == kKWaves * kKeepPerThread, "a wave reads whole tiles");
constexpr int kRowBatch = 4;
__global__ __launch_bounds__(kKThreads) void kvar_sums_kernel(AllocKArgs a) {
  constexpr int kCB = kHeadDim / 8;            // 8-channel blocks per row
  constexpr int kRowLanes = kKThreads / kCB;   // rows in flight
  __shared__ int64_t s_s1[kKWaves][kHeadDim];
  __shared__ U128 s_s2[kKWaves][kHeadDim];
  __shared__ int32_t s_list[kKeepBatch];
  __shared__ int32_t s_count;
  const int64_t seg = blockIdx.x / a.blocks;
  const int blk = int(blockIdx.x % a.blocks);
  const int cb = threadIdx.x % kCB, tr = threadIdx.x / kCB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint4* Kseg = reinterpret_cast<const uint4*>(a.K + seg * a.N * kHeadDim);
  const uint8_t* bt = a.bits_tok + seg * a.N;
  const int64_t n_tiles = (a.N + kKTile - 1) / kKTile;
  const int64_t my_tiles = n_tiles > blk ? (n_tiles - blk + a.blocks - 1) / a.blocks : 0;

  // exact sums of X = x * 2^24 and X^2 over kept tokens, channels 8 cb + e
  int64_t s1[8];
  U128 s2[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    s1[e] = 0;
    s2[e] = U128{0, 0};
  }
  const auto add_row = [&](const uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = (e & 1) ? half_hi(w[e >> 1]) : half_lo(w[e >> 1]);
      const int64_t X = int64_t(double(x) * 16777216.0);
      s1[e] += X;
      const uint64_t ax = uint64_t(X < 0 ? -X : X);
      s2[e] = add128(s2[e], mul64(ax, ax));
    }
  };
  int64_t n = 0;   // kept tokens (the same in every thread)
  for (int64_t b0 = 0; b0 < my_tiles; b0 += kTilesPerBatch) {
    if (threadIdx.x == 0) s_count = 0;
    __syncthreads();
    // thread: token lane of local tiles b0 + wave + kKWaves j (a wave reads a tile's 64 bytes)
    uint8_t b[kKeepPerThread];
    int32_t tok[kKeepPerThread];
#pragma unroll
    for (int j = 0; j < kKeepPerThread; ++j) {
      const int64_t lt = b0 + wave + kKWaves * j;
      const int64_t t = (blk + lt * a.blocks) * kKTile + lane;
      const bool in = lt < my_tiles && t < a.N;
      b[j] = in ? bt[t] : 0;
      tok[j] = int32_t(t);   // (< 2^19)
    }
#pragma unroll
    for (int j = 0; j < kKeepPerThread; ++j)
      if (bits_group(b[j]) >= 0) s_list[atomicAdd(&s_count, 1)] = tok[j];
    __syncthreads();
    const int cnt = s_count;
    for (int r0 = tr; r0 < cnt; r0 += kRowLanes * kRowBatch) {
      uint4 v[kRowBatch];
#pragma unroll
      for (int i = 0; i < kRowBatch; ++i) {
        const int r = r0 + i * kRowLanes;
        v[i] = r < cnt ? Kseg[int64_t(s_list[r]) * kCB + cb] : make_uint4(0, 0, 0, 0);   // (a zero row adds 0)
      }
#pragma unroll
      for (int i = 0; i < kRowBatch; ++i) add_row(v[i]);
    }
    n += cnt;
    __syncthreads();   // (s_list and s_count are rewritten by the next batch)
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
  __syncthreads();
  if (threadIdx.x < kHeadDim) {
    const int c = threadIdx.x;
    int64_t S1 = 0;
    U128 S2{0, 0};
#pragma unroll
    for (int w = 0; w < kKWaves; ++w) {
      S1 += s_s1[w][c];
      S2 = add128(S2, s_s2[w][c]);
    }
    if (a.blocks == 1) {   // the whole segment: its variances directly
      a.var_chan[seg * kHeadDim + c] = channel_variance(S1, S2, n);
    } else {
      const int64_t slot = seg * a.blocks + blk;
      a.s1[slot * kHeadDim + c] = S1;
      a.s2[slot * kHeadDim + c] = S2;
      if (c == 0) a.cnt[slot] = n;
    }
  }
}

// var_chan of each (segment, channel): the partial sums added up (exact), and
// the population variance n S2 - S1^2 over n^2 rounded once to fp32.
__global__ __launch_bounds__(kHeadDim) void kvar_final_kernel(AllocKArgs a) {
  const int64_t seg = blockIdx.x;
  const int c = threadIdx.x;
  constexpr int kLoads = 8;   // blocks whose partial sums are loaded together
  int64_t S1 = 0, n = 0;
  U128 S2{0, 0};
  for (int b0 = 0; b0 < a.blocks; b0 += kLoads) {
    int64_t s1[kLoads], cn[kLoads];
    U128 s2[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int64_t slot = seg * a.blocks + b0 + j;
      const bool in = b0 + j < a.blocks;
      s1[j] = in ? a.s1[slot * kHeadDim + c] : 0;
      s2[j] = in ? a.s2[slot * kHeadDim + c] : U128{0, 0};
      cn[j] = in ? a.cnt[slot] : 0;
    }
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      S1 += s1[j];
      S2 = add128(S2, s2[j]);
      n += cn[j];
    }
  }
  a.var_chan[seg * kHeadDim + c] = channel_variance(S1, S2, n);
}

}  // namespace

hipError_t launch_allocate(const AllocParams& p, hipStream_t stream) {
  const int64_t n_groups = p.n_seg / p.group;
  if (n_groups == 0) return hipSuccess;
  const AllocPlan w = alloc_plan(p.n_seg, p.n_tokens, p.group);
  auto* hist = reinterpret_cast<unsigned long long*>(p.workspace + w.hist);
  auto* state = reinterpret_cast<unsigned long long*>(p.workspace + w.state);
  LaunchErrors le;
  SelArgs sa{p.n_tokens * p.group, w.v_blocks, 0, p.w_tok, p.var_tok, hist, state};
  if (w.v_blocks == 1) {
    hipLaunchKernelGGL(alloc_one_kernel, dim3(unsigned(n_groups)), dim3(kSelThreads), 0, stream, sa, p.budget_v,
                       p.group, p.bits_tok, p.lambda, 0);
    le.check();
  } else {
    // the histograms and states start at zero (a fill kernel, so a captured graph replays it)
    const int64_t words = (w.state + n_groups * kStSlots * kStWords * 8 - w.hist) / 8;
    hipLaunchKernelGGL(fill_u64_kernel, dim3(unsigned(std::min<int64_t>(cdiv(words, 256), 1024))), dim3(256), 0,
                       stream, hist, words);
    le.check();
    const unsigned v_grid = unsigned(n_groups * w.v_blocks);
    for (int pass = 0; pass < kSelPasses; ++pass) {
      sa.pass = pass;
      hipLaunchKernelGGL(sel_pass_kernel, dim3(v_grid), dim3(kSelThreads), 0, stream, sa, p.budget_v);
      le.check();
    }
    hipLaunchKernelGGL(alloc_v_bits_kernel, dim3(v_grid), dim3(kSelThreads), 0, stream, sa, p.budget_v, p.group,
                       p.bits_tok, p.lambda);
    le.check();
  }
  AllocKArgs ka{p.n_tokens, p.group, w.k_blocks, p.K, p.bits_tok, p.w_chan, p.budget_k, p.bits_chan, p.var_chan,
                p.lambda, reinterpret_cast<int64_t*>(p.workspace + w.s1), reinterpret_cast<U128*>(p.workspace + w.s2),
                reinterpret_cast<int64_t*>(p.workspace + w.cnt)};
  hipLaunchKernelGGL(kvar_sums_kernel, dim3(unsigned(p.n_seg * w.k_blocks)), dim3(kKThreads), 0, stream, ka);
  le.check();
  if (w.k_blocks > 1) {
    hipLaunchKernelGGL(kvar_final_kernel, dim3(unsigned(p.n_seg)), dim3(kHeadDim), 0, stream, ka);
    le.check();
  }
  // the K channels: group * 128 units per problem, always one workgroup
  const SelArgs sk{int64_t(kHeadDim) * p.group, 1, 0, p.w_chan, p.var_chan, nullptr, nullptr};
  hipLaunchKernelGGL(alloc_one_kernel, dim3(unsigned(n_groups)), dim3(kSelThreads), 0, stream, sk, p.budget_k,
                     p.group, p.bits_chan, p.lambda, 1);
  le.check();
  return le.status();
}

AllocPlan alloc_plan(int64_t n_seg, int64_t n_tokens, int32_t group) {
  // workgroups per problem: enough to fill the chip (about kFill in all),
  // none with fewer than kMinUnits V tokens or kMinTokens tokens for the sums
  constexpr int64_t kFill = 2048, kMinUnits = 2048, kMinTokens = 2048;
  AllocPlan w{};
  if (n_seg <= 0 || n_tokens <= 0 || group < 1) return w;
  const int64_t n_groups = n_seg / group, n = n_tokens * group;
  w.v_blocks = int32_t(std::max<int64_t>(1, std::min(cdiv(kFill, n_groups), cdiv(n, kMinUnits))));
  w.k_blocks = int32_t(std::max<int64_t>(1, std::min(cdiv(kFill, n_seg), cdiv(n_tokens, kMinTokens))));
  uint64_t o = 0;
  const auto take = [&](uint64_t bytes) {
    const uint64_t at = o;
    o += (bytes + 255) / 256 * 256;
    return at;
  };
  // (one workgroup per problem keeps its histogram in LDS and its sums in registers)
  const uint64_t vg = w.v_blocks > 1 ? uint64_t(n_groups) : 0, ks = w.k_blocks > 1 ? uint64_t(n_seg) * w.k_blocks : 0;
  w.hist = take(vg * kHistBufs * kSelBuckets * 8);
  w.state = take(vg * kStSlots * kStWords * 8);
  w.s1 = take(ks * kHeadDim * 8);
  w.s2 = take(ks * kHeadDim * 16);
  w.cnt = take(ks * 8);
  w.total = o;
  return w;
}

}  // namespace rdkv
