// Zone-C rollover (RDKV summary section 2.3: zone C holds the new tokens'
// fp16 rows).  When zone C is full its tokens are scored from what the
// decode steps accumulated (the attention each row received from every query
// that saw it, summed over the heads -- section 2.1's token weight over the
// decode queries, the accumulated attention score of the aistudio.id
// article's "Solusi 2"; the queries' channel sums of squares for the channel
// weight), allocated by the allocation kernels (section 2.2, with the
// generation budgets) and packed by the packing kernels into the next
// generation blob, a complete blob of the packed format for cap tokens per
// segment.  Then zone C and the statistics are cleared.
//
//   rollover_rows_kernel   one wave per (segment, zone-C row): gathers the K
//                          and V row into a contiguous [n_seg][cap][128]
//                          workspace, w_tok = sum over heads of the mass,
//                          var_tok = population variance of the V row
//   rollover_chan_kernel   one workgroup per segment: w_chan from the
//                          accumulated query squares and the zone-C K column
//                          norms (fp64 sums, rounded once)
//   rollover_reset_kernel  zone C and the statistics to zero, the header's
//                          generations-in-use count to gen + 1
#include "rdkv_internal.h"

namespace rdkv {
namespace {

constexpr int kThreads = 256;

__device__ inline void zone_c_offsets(const RolloverParams& r, int64_t seg, uint64_t& kc, uint64_t& vc, bool& ok) {
  const uint8_t* d = r.cache + kHeaderBytes + uint64_t(seg) * kDescBytes;
  kc = *reinterpret_cast<const uint64_t*>(d + kDescOffKc);
  vc = *reinterpret_cast<const uint64_t*>(d + kDescOffVc);
  const uint64_t rows = uint64_t(r.cap) * kHeadDim * 2;
  ok = kc + rows <= r.main_bytes && vc + rows <= r.main_bytes;
}

struct RowsArgs {
  RolloverParams r;
  __half* Kg;   // [n_seg][cap][128] or null
  __half* Vg;
};

__global__ __launch_bounds__(kThreads) void rollover_rows_kernel(RowsArgs a) {
  const RolloverParams& r = a.r;
  const int64_t row = int64_t(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= r.n_seg * r.cap) return;
  const int64_t seg = row / r.cap;
  const int j = int(row % r.cap);
  const int lane = threadIdx.x & 63;
  uint64_t kc, vc;
  bool ok;
  zone_c_offsets(r, seg, kc, vc, ok);
  uint32_t kw = 0, vw = 0;
  if (ok) {
    kw = reinterpret_cast<const uint32_t*>(r.cache + kc + uint64_t(j) * kHeadDim * 2)[lane];
    vw = reinterpret_cast<const uint32_t*>(r.cache + vc + uint64_t(j) * kHeadDim * 2)[lane];
  }
  if (a.Kg) {
    reinterpret_cast<uint32_t*>(a.Kg + row * kHeadDim)[lane] = kw;
    reinterpret_cast<uint32_t*>(a.Vg + row * kHeadDim)[lane] = vw;
  }
  // population variance of the V row, two passes in registers
  const float v0 = half_lo(vw), v1 = half_hi(vw);
  const float mean = wave_sum(v0 + v1) * (1.0f / kHeadDim);
  const float d0 = v0 - mean, d1 = v1 - mean;
  const float ss = wave_sum(fmaf(d0, d0, d1 * d1));
  if (lane == 0) {
    r.var_tok[row] = ss * (1.0f / kHeadDim);
    float w = 0.f;
    for (int g = 0; g < r.G; ++g) w += r.stats[(seg * r.G + g) * int64_t(r.cap + kHeadDim) + j];
    r.w_tok[row] = w;
  }
}

__global__ __launch_bounds__(kHeadDim) void rollover_chan_kernel(RolloverParams r) {
  const int64_t seg = blockIdx.x;
  const int c = threadIdx.x;
  uint64_t kc, vc;
  bool ok;
  zone_c_offsets(r, seg, kc, vc, ok);
  double sk = 0.0, sq = 0.0;
  if (ok) {
    const __half* K = reinterpret_cast<const __half*>(r.cache + kc);
    for (int j = 0; j < r.cap; ++j) {
      const double k = __half2float(K[int64_t(j) * kHeadDim + c]);
      sk += k * k;
    }
  }
  for (int g = 0; g < r.G; ++g) sq += double(r.stats[(seg * r.G + g) * int64_t(r.cap + kHeadDim) + r.cap + c]);
  r.w_chan[seg * kHeadDim + c] = float(sqrt(sq) * sqrt(sk) / sqrt(double(kHeadDim)));
}

__global__ __launch_bounds__(kThreads) void rollover_reset_kernel(RolloverParams r, float* stats, int32_t gen) {
  const int64_t seg = blockIdx.x;
  uint64_t kc, vc;
  bool ok;
  zone_c_offsets(r, seg, kc, vc, ok);
  if (ok) {
    const int n16 = r.cap * kHeadDim * 2 / 16;
    for (int i = threadIdx.x; i < n16; i += kThreads) {
      reinterpret_cast<uint4*>(r.cache + kc)[i] = make_uint4(0, 0, 0, 0);
      reinterpret_cast<uint4*>(r.cache + vc)[i] = make_uint4(0, 0, 0, 0);
    }
  }
  const int64_t n = int64_t(r.G) * (r.cap + kHeadDim);
  for (int64_t i = threadIdx.x; i < n; i += kThreads) stats[seg * n + i] = 0.f;
  if (seg == 0 && threadIdx.x == 0) *reinterpret_cast<int32_t*>(r.cache + kHdrNGenUsed) = gen + 1;
}

// Workspace regions of a rollover, each 256-byte aligned.
struct Workspace {
  uint64_t kg, vg, w_tok, var_tok, w_chan, var_chan, bits_tok, bits_chan, lambda, alloc, total;
};
Workspace workspace_plan(int64_t n_seg, int64_t cap) {
  Workspace w;
  uint64_t o = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t at = o;
    o = align_up(o + bytes, kAlign);
    return at;
  };
  w.kg = take(uint64_t(n_seg) * cap * kHeadDim * 2);
  w.vg = take(uint64_t(n_seg) * cap * kHeadDim * 2);
  w.w_tok = take(uint64_t(n_seg) * cap * 4);
  w.var_tok = take(uint64_t(n_seg) * cap * 4);
  w.w_chan = take(uint64_t(n_seg) * kHeadDim * 4);
  w.var_chan = take(uint64_t(n_seg) * kHeadDim * 4);
  w.bits_tok = take(uint64_t(n_seg) * cap);
  w.bits_chan = take(uint64_t(n_seg) * kHeadDim);
  w.lambda = take(uint64_t(n_seg) * 2 * 8);
  w.alloc = take(alloc_plan(n_seg, cap, 1).total);
  w.total = o;
  return w;
}

}  // namespace

uint64_t rollover_workspace_bytes(int64_t n_seg, int64_t cap) { return workspace_plan(n_seg, cap).total; }

hipError_t launch_rollover_score(const RolloverParams& r, hipStream_t stream) {
  LaunchErrors le;
  const int64_t rows = r.n_seg * r.cap;
  if (rows > 0) {
    hipLaunchKernelGGL(rollover_rows_kernel, dim3(unsigned(cdiv(rows, kThreads / 64))), dim3(kThreads), 0, stream,
                       RowsArgs{r, nullptr, nullptr});
    le.check();
  }
  if (r.n_seg > 0) {
    hipLaunchKernelGGL(rollover_chan_kernel, dim3(unsigned(r.n_seg)), dim3(kHeadDim), 0, stream, r);
    le.check();
  }
  return le.status();
}

hipError_t launch_rollover(RolloverParams r, const rdkv_layout& gen_layout, int32_t gen, uint8_t* ws,
                           hipStream_t stream) {
  const Workspace w = workspace_plan(r.n_seg, r.cap);
  __half* Kg = reinterpret_cast<__half*>(ws + w.kg);
  __half* Vg = reinterpret_cast<__half*>(ws + w.vg);
  r.w_tok = reinterpret_cast<float*>(ws + w.w_tok);
  r.var_tok = reinterpret_cast<float*>(ws + w.var_tok);
  r.w_chan = reinterpret_cast<float*>(ws + w.w_chan);
  const int64_t rows = r.n_seg * r.cap;
  LaunchErrors le;
  hipLaunchKernelGGL(rollover_rows_kernel, dim3(unsigned(cdiv(rows, kThreads / 64))), dim3(kThreads), 0, stream,
                     RowsArgs{r, Kg, Vg});
  le.check();
  hipLaunchKernelGGL(rollover_chan_kernel, dim3(unsigned(r.n_seg)), dim3(kHeadDim), 0, stream, r);
  le.check();
  hipError_t e = le.status();
  if (e != hipSuccess) return e;

  AllocParams ap;
  ap.n_seg = r.n_seg;
  ap.n_tokens = r.cap;
  ap.group = 1;
  ap.w_tok = r.w_tok;
  ap.var_tok = r.var_tok;
  ap.w_chan = r.w_chan;
  ap.K = Kg;
  ap.budget_v = r.gen_budget_v;
  ap.budget_k = r.gen_budget_k;
  ap.bits_tok = ws + w.bits_tok;
  ap.bits_chan = ws + w.bits_chan;
  ap.var_chan = reinterpret_cast<float*>(ws + w.var_chan);
  ap.lambda = reinterpret_cast<double*>(ws + w.lambda);
  ap.workspace = ws + w.alloc;
  e = launch_allocate(ap, stream);
  if (e != hipSuccess) return e;

  PackParams pp;
  pp.cache = r.cache + r.gen_offset + uint64_t(gen) * r.gen_bytes;
  pp.cache_bytes = gen_layout.cache_bytes;
  pp.lay = &gen_layout;
  pp.layer_begin = 0;
  pp.n_layers_in = r.n_layers;
  pp.K = Kg;
  pp.V = Vg;
  pp.bits_tok = ap.bits_tok;
  pp.bits_chan = ap.bits_chan;
  e = launch_pack(pp, stream);
  if (e != hipSuccess) return e;

  hipLaunchKernelGGL(rollover_reset_kernel, dim3(unsigned(r.n_seg)), dim3(kThreads), 0, stream, r,
                     const_cast<float*>(r.stats), gen);
  return hipGetLastError();
}

}  // namespace rdkv
