// C ABI of the RDKV library: host-side validation, layout arithmetic and
// dispatch to the kernels.  Every entry point validates before enqueueing
// anything; on an error nothing is enqueued and no output is touched.
#include <algorithm>
#include <cstring>

#include "rdkv_internal.h"

using namespace rdkv;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

rdkv_status check_dims(const rdkv_dims* d) {
  if (!d) return RDKV_ERR_NULL;
  if (d->reserved != 0) return RDKV_ERR_SHAPE;
  if (d->n_tokens < 1 || d->n_seq < 1 || d->n_layers < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1)
    return RDKV_ERR_SHAPE;
  if (d->n_q_heads % d->n_kv_heads != 0) return RDKV_ERR_SHAPE;
  // at most kMaxSegments segments, so every size below fits 64 bits
  const int64_t sl = int64_t(d->n_seq) * d->n_layers;   // < 2^62
  if (sl > kMaxSegments || sl * d->n_kv_heads > kMaxSegments) return RDKV_ERR_SHAPE;
  if (d->head_dim != kHeadDim) return RDKV_ERR_UNSUPPORTED;
  const int G = d->n_q_heads / d->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return RDKV_ERR_UNSUPPORTED;
  // the exact channel variance keeps |sum X| < 2^63 and n^2 < 2^38 in integers
  if (d->n_tokens > kMaxTokens) return RDKV_ERR_SHAPE;
  return RDKV_OK;
}

rdkv_status layout_init(const rdkv_dims* dims, int64_t budget_v, int64_t budget_k, int32_t zone_c_capacity,
                        int32_t n_gen, int64_t gen_budget_v, int64_t gen_budget_k, rdkv_layout* out);

rdkv_status check_layout(const rdkv_layout* lay) {
  if (!lay) return RDKV_ERR_NULL;
  rdkv_layout ref;
  rdkv_status st = layout_init(&lay->dims, lay->budget_v, lay->budget_k, lay->zone_c_capacity, lay->n_generations,
                               lay->gen_budget_v, lay->gen_budget_k, &ref);
  if (st != RDKV_OK) return st;
  if (std::memcmp(&ref, lay, sizeof(ref)) != 0) return RDKV_ERR_SHAPE;  // not from rdkv_layout_init*
  return RDKV_OK;
}

// The layout of one generation blob of a rollover layout: the same format
// for zone_c_capacity tokens per segment, the generation budgets, no zone C.
// (Called on layouts that passed check_layout, whose generation layout was
// built by layout_init; a zeroed layout if it cannot be built.)
rdkv_layout generation_layout(const rdkv_layout& lay) {
  rdkv_dims d = lay.dims;
  d.n_tokens = lay.zone_c_capacity;
  rdkv_layout g;
  if (layout_init(&d, lay.gen_budget_v, lay.gen_budget_k, 0, 0, 0, 0, &g) != RDKV_OK) std::memset(&g, 0, sizeof(g));
  return g;
}

rdkv_status hip_status(hipError_t e) { return e == hipSuccess ? RDKV_OK : RDKV_ERR_HIP; }

DecodeParams base_params(const rdkv_layout* layout, void* cache, int n_c, int c_len, int append) {
  DecodeParams p{};
  p.cache = static_cast<uint8_t*>(cache);
  p.cache_bytes = layout->cache_bytes;
  p.main_bytes = layout->n_generations > 0 ? layout->gen_offset : layout->cache_bytes;
  p.n_seg = layout->n_seg;
  p.nk_max = layout->nk_max;
  p.max_chunks = layout->max_chunks;
  p.token_slots = layout->token_slots;
  p.chunk_tok2 = layout->chunk_tok2;
  p.rec_max = layout->rec_max;
  p.group = layout->dims.n_q_heads / layout->dims.n_kv_heads;
  p.zc_cap = layout->zone_c_capacity;
  p.c_len = c_len;
  p.n_c = n_c;
  p.append = append;
  if (layout->n_generations > 0) {
    const rdkv_layout g = generation_layout(*layout);
    p.n_gen = layout->n_generations;
    p.gen_slots = g.max_chunks;
    p.gen_chunk_tok2 = g.chunk_tok2;
    p.gen_rec_max = g.rec_max;
    p.gen_nk_max = g.nk_max;
    p.gen_offset = layout->gen_offset;
    p.gen_bytes = layout->gen_bytes;
    p.gen_cache_bytes = g.cache_bytes;
  }
  return p;
}

RolloverParams rollover_params(const rdkv_layout& lay, void* cache, float* zc_stats) {
  RolloverParams r{};
  r.cache = static_cast<uint8_t*>(cache);
  r.main_bytes = lay.gen_offset;
  r.n_seg = lay.n_seg;
  r.G = lay.dims.n_q_heads / lay.dims.n_kv_heads;
  r.cap = lay.zone_c_capacity;
  r.n_layers = lay.dims.n_layers;
  r.gen_offset = lay.gen_offset;
  r.gen_bytes = lay.gen_bytes;
  r.gen_budget_v = lay.gen_budget_v;
  r.gen_budget_k = lay.gen_budget_k;
  r.stats = zc_stats;
  return r;
}

// Validation shared by the decode entry points.  With own_workspace (the
// library's static scratch, set by the caller afterwards) the workspace
// arguments are not checked.
rdkv_status decode_params(const rdkv_layout* layout, void* cache, size_t cache_bytes, int32_t c_len, const void* q,
                          const void* k_new, const void* v_new, void* workspace, size_t workspace_bytes,
                          DecodeParams* out, bool own_workspace = false, uint64_t workspace_need = ~uint64_t(0)) {
  rdkv_status st = check_layout(layout);
  if (st != RDKV_OK) return st;
  if (!cache || !q || (!workspace && !own_workspace)) return RDKV_ERR_NULL;
  if ((k_new == nullptr) != (v_new == nullptr)) return RDKV_ERR_NULL;
  if (!aligned16(cache) || !aligned16(q) || (!own_workspace && !aligned16(workspace))) return RDKV_ERR_ALIGN;
  if (k_new && (!aligned16(k_new) || !aligned16(v_new))) return RDKV_ERR_ALIGN;
  const uint64_t ws_need = workspace_need == ~uint64_t(0) ? layout->decode_workspace_bytes : workspace_need;
  if (cache_bytes < layout->cache_bytes || (!own_workspace && workspace_bytes < ws_need)) return RDKV_ERR_WORKSPACE;
  const int append = k_new != nullptr;
  if (c_len < 0 || int64_t(c_len) + append > layout->zone_c_capacity) return RDKV_ERR_CAPACITY;
  DecodeParams p = base_params(layout, cache, c_len + append, c_len, append);
  p.q = static_cast<const __half*>(q);
  p.k_new = static_cast<const __half*>(k_new);
  p.v_new = static_cast<const __half*>(v_new);
  p.partials = static_cast<float*>(workspace);
  *out = p;
  return RDKV_OK;
}

}  // namespace

extern "C" {

int32_t rdkv_version(void) { return (kFormatVersion << 16) | 1; }

const char* rdkv_status_string(int32_t s) {
  switch (s) {
    case RDKV_OK: return "ok";
    case RDKV_ERR_NULL: return "null pointer";
    case RDKV_ERR_SHAPE: return "bad shape";
    case RDKV_ERR_UNSUPPORTED: return "unsupported shape";
    case RDKV_ERR_BUDGET: return "negative budget";
    case RDKV_ERR_ALIGN: return "pointer not 16-byte aligned";
    case RDKV_ERR_WORKSPACE: return "buffer too small";
    case RDKV_ERR_CAPACITY: return "zone C capacity exceeded";
    case RDKV_ERR_HIP: return "HIP runtime error";
    case RDKV_ERR_OVERFLOW: return "allocation exceeds the layout's budget bounds";
  }
  return "unknown status";
}

}  // extern "C"

namespace {

rdkv_status layout_init(const rdkv_dims* dims, int64_t budget_v, int64_t budget_k, int32_t zone_c_capacity,
                        int32_t n_gen, int64_t gen_budget_v, int64_t gen_budget_k, rdkv_layout* out) {
  if (!out) return RDKV_ERR_NULL;
  rdkv_status st = check_dims(dims);
  if (st != RDKV_OK) return st;
  if (budget_v < 0 || budget_k < 0) return RDKV_ERR_BUDGET;
  if (zone_c_capacity < 0 || zone_c_capacity > (1 << 20)) return RDKV_ERR_SHAPE;
  if (budget_v > (int64_t(1) << 40) || budget_k > (int64_t(1) << 40)) return RDKV_ERR_BUDGET;
  rdkv_layout L;
  std::memset(&L, 0, sizeof(L));
  L.dims = *dims;
  L.budget_v = budget_v;
  L.budget_k = budget_k;
  L.zone_c_capacity = zone_c_capacity;
  const int64_t N = dims->n_tokens;
  const int64_t cap = zone_c_capacity;
  L.n_seg = int64_t(dims->n_seq) * dims->n_layers * dims->n_kv_heads;
  L.nk_max = std::min<int64_t>(N, budget_v / 2);
  const int64_t bk = std::min<int64_t>(budget_k, 16 * kHeadDim);
  // each of the four record parts pads to a word: words <= bk/32 + 3.0625
  L.rec_max = int32_t(4 * ((bk + 98) / 32 + 4));
  const uint64_t zone_c = uint64_t(cap) * kHeadDim * 2;           // one of K_C, V_C
  L.slot_off_v = align_up(2 * zone_c, kAlign);
  const uint64_t v_res = align_up(uint64_t(std::min<int64_t>(16 * budget_v, 2 * kHeadDim * N)) + 768, kAlign);
  L.slot_off_krec = L.slot_off_v + v_res;
  L.slot_off_pos = L.slot_off_krec + align_up(uint64_t(L.nk_max) * L.rec_max, kAlign);
  L.slot_bytes = L.slot_off_pos + align_up(uint64_t(4) * L.nk_max, kAlign);
  L.slots_offset = align_up(kHeaderBytes + uint64_t(kDescBytes) * L.n_seg, kAlign);
  L.cache_bytes = L.slots_offset + uint64_t(L.n_seg) * L.slot_bytes;
  // Split-K granularity.  A chunk of group g holds chunk_tok2 >> g tokens, so
  // sum_g ceil(n_g / (chunk_tok2 >> g)) <= sum_g n_g 2^g / chunk_tok2 + 4, and
  // sum_g n_g 2^g <= min(B_V / 2, 8 N) because a g-group token costs 2^(g+1) bits.
  const int64_t v_units = std::min<int64_t>(budget_v / 2, 8 * N);
  int64_t t2 = kChunkTok2Min;
  while (t2 < kChunkTok2Max && L.n_seg * v_units / (2 * t2) >= kDecodeTargetChunks) t2 *= 2;
  L.chunk_tok2 = int32_t(t2);
  const int64_t tok_chunks = v_units / t2 + 4;
  L.token_slots = int32_t(tok_chunks);
  L.max_chunks = int32_t(tok_chunks + cdiv(cap, kChunkRowsC));
  const int G = dims->n_q_heads / dims->n_kv_heads;
  if (n_gen != 0) {
    // generation blobs after the main blob, one per rollover of zone C
    if (n_gen < 0 || n_gen > kMaxGenerations || cap < 1) return RDKV_ERR_SHAPE;
    if (gen_budget_v < 0 || gen_budget_k < 0) return RDKV_ERR_BUDGET;
    if (gen_budget_v > (int64_t(1) << 40) || gen_budget_k > (int64_t(1) << 40)) return RDKV_ERR_BUDGET;
    L.n_generations = n_gen;
    L.gen_budget_v = gen_budget_v;
    L.gen_budget_k = gen_budget_k;
    rdkv_dims gd = L.dims;
    gd.n_tokens = cap;
    rdkv_layout g;
    st = layout_init(&gd, gen_budget_v, gen_budget_k, 0, 0, 0, 0, &g);
    if (st != RDKV_OK) return st;
    L.gen_offset = L.cache_bytes;
    L.gen_bytes = align_up(g.cache_bytes, kAlign);
    if (L.gen_bytes > kMaxCacheBytes / uint64_t(n_gen)) return RDKV_ERR_SHAPE;
    L.cache_bytes = L.gen_offset + uint64_t(n_gen) * L.gen_bytes;
    L.max_chunks = int32_t(tok_chunks + int64_t(n_gen) * g.max_chunks + cdiv(cap, kChunkRowsC));
    L.zc_stats_bytes = uint64_t(L.n_seg) * G * (cap + kHeadDim) * sizeof(float);
    L.rollover_workspace_bytes = rollover_workspace_bytes(L.n_seg, cap);
  }
  L.decode_workspace_bytes = uint64_t(L.n_seg) * L.max_chunks * G * kPartialFloats * sizeof(float);
  if (L.cache_bytes > kMaxCacheBytes || L.decode_workspace_bytes > kMaxCacheBytes) return RDKV_ERR_SHAPE;
  *out = L;
  return RDKV_OK;
}

}  // namespace

extern "C" {

rdkv_status rdkv_layout_init(const rdkv_dims* dims, int64_t budget_v, int64_t budget_k,
                             int32_t zone_c_capacity, rdkv_layout* out) {
  return layout_init(dims, budget_v, budget_k, zone_c_capacity, 0, 0, 0, out);
}

rdkv_status rdkv_layout_init_rollover(const rdkv_dims* dims, int64_t budget_v, int64_t budget_k,
                                      int32_t zone_c_capacity, int32_t n_generations, int64_t gen_budget_v,
                                      int64_t gen_budget_k, rdkv_layout* out) {
  if (n_generations < 1) return RDKV_ERR_SHAPE;
  return layout_init(dims, budget_v, budget_k, zone_c_capacity, n_generations, gen_budget_v, gen_budget_k, out);
}

size_t rdkv_score_workspace_bytes(const rdkv_dims* dims) {
  if (check_dims(dims) != RDKV_OK) return 0;
  return score_workspace_bytes(dims->n_seq, dims->n_layers, dims->n_q_heads, dims->n_tokens);
}

rdkv_status rdkv_score(const rdkv_dims* dims, const void* Q, const void* K, const void* V,
                       float* w_tok, float* var_tok, float* w_chan,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  rdkv_status st = check_dims(dims);
  if (st != RDKV_OK) return st;
  if (!Q || !K || !V || !w_tok || !var_tok || !w_chan || !workspace) return RDKV_ERR_NULL;
  for (const void* p : {Q, K, V, (const void*)w_tok, (const void*)var_tok, (const void*)w_chan, (const void*)workspace})
    if (!aligned16(p)) return RDKV_ERR_ALIGN;
  if (workspace_bytes < rdkv_score_workspace_bytes(dims)) return RDKV_ERR_WORKSPACE;
  ScoreParams p{};
  p.n_tokens = dims->n_tokens;
  p.S = dims->n_seq;
  p.L = dims->n_layers;
  p.Hq = dims->n_q_heads;
  p.Hkv = dims->n_kv_heads;
  p.Q = static_cast<const __half*>(Q);
  p.K = static_cast<const __half*>(K);
  p.V = static_cast<const __half*>(V);
  p.w_tok = w_tok;
  p.var_tok = var_tok;
  p.w_chan = w_chan;
  p.lse = static_cast<float*>(workspace);
  return hip_status(launch_score(p, stream));
}

rdkv_status rdkv_score_lse(const rdkv_dims* dims, const void* Q, const void* K, float* lse, hipStream_t stream) {
  rdkv_status st = check_dims(dims);
  if (st != RDKV_OK) return st;
  if (!Q || !K || !lse) return RDKV_ERR_NULL;
  for (const void* p : {Q, K, (const void*)lse})
    if (!aligned16(p)) return RDKV_ERR_ALIGN;
  ScoreParams p{};
  p.n_tokens = dims->n_tokens;
  p.S = dims->n_seq;
  p.L = dims->n_layers;
  p.Hq = dims->n_q_heads;
  p.Hkv = dims->n_kv_heads;
  p.Q = static_cast<const __half*>(Q);
  p.K = static_cast<const __half*>(K);
  p.lse = lse;
  return hip_status(launch_score_lse(p, stream));
}

rdkv_status rdkv_score_from_lse(const rdkv_dims* dims, const void* Q, const void* K, const void* V,
                                const float* lse, float* w_tok, float* var_tok, float* w_chan,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  rdkv_status st = check_dims(dims);
  if (st != RDKV_OK) return st;
  if (!Q || !K || !V || !lse || !w_tok || !var_tok || !w_chan || !workspace) return RDKV_ERR_NULL;
  for (const void* p : {Q, K, V, (const void*)lse, (const void*)w_tok, (const void*)var_tok, (const void*)w_chan,
                        (const void*)workspace})
    if (!aligned16(p)) return RDKV_ERR_ALIGN;
  if (workspace_bytes < rdkv_score_workspace_bytes(dims)) return RDKV_ERR_WORKSPACE;
  ScoreParams p{};
  p.n_tokens = dims->n_tokens;
  p.S = dims->n_seq;
  p.L = dims->n_layers;
  p.Hq = dims->n_q_heads;
  p.Hkv = dims->n_kv_heads;
  p.Q = static_cast<const __half*>(Q);
  p.K = static_cast<const __half*>(K);
  p.V = static_cast<const __half*>(V);
  p.w_tok = w_tok;
  p.var_tok = var_tok;
  p.w_chan = w_chan;
  p.lse = static_cast<float*>(workspace);
  p.lse_in = lse;
  return hip_status(launch_score_from_lse(p, stream));
}

size_t rdkv_allocate_workspace_bytes(const rdkv_dims* dims, int32_t group) {
  if (check_dims(dims) != RDKV_OK) return 0;
  const int64_t n_seg = int64_t(dims->n_seq) * dims->n_layers * dims->n_kv_heads;
  if (group < 1 || n_seg % group != 0) return 0;
  return size_t(alloc_plan(n_seg, dims->n_tokens, group).total);
}

rdkv_status rdkv_allocate_shared(const rdkv_dims* dims, const float* w_tok, const float* var_tok,
                                 const float* w_chan, const void* K, int64_t budget_v, int64_t budget_k,
                                 int32_t group, uint8_t* bits_tok, uint8_t* bits_chan, float* var_chan,
                                 double* lambda, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  rdkv_status st = check_dims(dims);
  if (st != RDKV_OK) return st;
  if (!w_tok || !var_tok || !w_chan || !K || !bits_tok || !bits_chan || !var_chan || !lambda) return RDKV_ERR_NULL;
  for (const void* p : {(const void*)w_tok, (const void*)var_tok, (const void*)w_chan, K, (const void*)bits_tok,
                        (const void*)bits_chan, (const void*)var_chan, (const void*)lambda, (const void*)workspace})
    if (!aligned16(p)) return RDKV_ERR_ALIGN;
  if (budget_v < 0 || budget_k < 0) return RDKV_ERR_BUDGET;
  AllocParams p;
  p.n_seg = int64_t(dims->n_seq) * dims->n_layers * dims->n_kv_heads;
  if (group < 1 || p.n_seg % group != 0) return RDKV_ERR_SHAPE;
  const uint64_t need = alloc_plan(p.n_seg, dims->n_tokens, group).total;
  if (need > 0 && !workspace) return RDKV_ERR_NULL;
  if (workspace_bytes < need) return RDKV_ERR_WORKSPACE;
  p.group = group;
  p.n_tokens = dims->n_tokens;
  p.w_tok = w_tok;
  p.var_tok = var_tok;
  p.w_chan = w_chan;
  p.K = static_cast<const __half*>(K);
  p.budget_v = budget_v;
  p.budget_k = budget_k;
  p.bits_tok = bits_tok;
  p.bits_chan = bits_chan;
  p.var_chan = var_chan;
  p.lambda = lambda;
  p.workspace = static_cast<uint8_t*>(workspace);
  return hip_status(launch_allocate(p, stream));
}

rdkv_status rdkv_allocate(const rdkv_dims* dims, const float* w_tok, const float* var_tok,
                          const float* w_chan, const void* K, int64_t budget_v, int64_t budget_k,
                          uint8_t* bits_tok, uint8_t* bits_chan, float* var_chan, double* lambda,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return rdkv_allocate_shared(dims, w_tok, var_tok, w_chan, K, budget_v, budget_k, 1, bits_tok, bits_chan, var_chan,
                              lambda, workspace, workspace_bytes, stream);
}

rdkv_status rdkv_cache_init(const rdkv_layout* layout, void* cache, size_t cache_bytes, hipStream_t stream) {
  rdkv_status st = check_layout(layout);
  if (st != RDKV_OK) return st;
  if (!cache) return RDKV_ERR_NULL;
  if (!aligned16(cache)) return RDKV_ERR_ALIGN;
  if (cache_bytes < layout->cache_bytes) return RDKV_ERR_WORKSPACE;
  if (layout->n_generations > 0) {
    const rdkv_layout g = generation_layout(*layout);
    return hip_status(launch_cache_init(static_cast<uint8_t*>(cache), *layout, &g, stream));
  }
  return hip_status(launch_cache_init(static_cast<uint8_t*>(cache), *layout, nullptr, stream));
}

rdkv_status rdkv_pack(const rdkv_layout* layout, int32_t layer_begin, int32_t n_layers,
                      const void* K, const void* V, const uint8_t* bits_tok, const uint8_t* bits_chan,
                      void* cache, size_t cache_bytes, hipStream_t stream) {
  rdkv_status st = check_layout(layout);
  if (st != RDKV_OK) return st;
  if (!K || !V || !bits_tok || !bits_chan || !cache) return RDKV_ERR_NULL;
  for (const void* p : {K, V, (const void*)bits_tok, (const void*)bits_chan, (const void*)cache})
    if (!aligned16(p)) return RDKV_ERR_ALIGN;
  if (layer_begin < 0 || n_layers < 1 || int64_t(layer_begin) + n_layers > layout->dims.n_layers)
    return RDKV_ERR_SHAPE;
  if (cache_bytes < layout->cache_bytes) return RDKV_ERR_WORKSPACE;
  PackParams p;
  p.cache = static_cast<uint8_t*>(cache);
  p.cache_bytes = cache_bytes;
  p.lay = layout;
  p.layer_begin = layer_begin;
  p.n_layers_in = n_layers;
  p.K = static_cast<const __half*>(K);
  p.V = static_cast<const __half*>(V);
  p.bits_tok = bits_tok;
  p.bits_chan = bits_chan;
  return hip_status(launch_pack(p, stream));
}

rdkv_status rdkv_pack_status(const rdkv_layout* layout, const void* cache, size_t cache_bytes, int32_t* n_dropped,
                             hipStream_t stream) {
  rdkv_status st = check_layout(layout);
  if (st != RDKV_OK) return st;
  if (!cache || !n_dropped) return RDKV_ERR_NULL;
  if (!aligned16(cache)) return RDKV_ERR_ALIGN;
  if (cache_bytes < layout->cache_bytes) return RDKV_ERR_WORKSPACE;
  return hip_status(launch_pack_status(static_cast<const uint8_t*>(cache), layout->n_seg, n_dropped, stream));
}

rdkv_status rdkv_decode_partials(const rdkv_layout* layout, void* cache, size_t cache_bytes, int32_t c_len,
                                 const void* q, const void* k_new, const void* v_new,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  DecodeParams p;
  rdkv_status st = decode_params(layout, cache, cache_bytes, c_len, q, k_new, v_new, workspace, workspace_bytes, &p);
  if (st != RDKV_OK) return st;
  if (!q) return RDKV_ERR_NULL;
  return hip_status(launch_decode_chunks(p, stream));
}

rdkv_status rdkv_decode_merge(const rdkv_layout* layout, const void* cache, size_t cache_bytes,
                              int32_t zone_c_rows, float* out, const void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  rdkv_status st = check_layout(layout);
  if (st != RDKV_OK) return st;
  if (!cache || !out || !workspace) return RDKV_ERR_NULL;
  for (const void* ptr : {cache, (const void*)out, workspace})
    if (!aligned16(ptr)) return RDKV_ERR_ALIGN;
  if (cache_bytes < layout->cache_bytes || workspace_bytes < layout->decode_workspace_bytes)
    return RDKV_ERR_WORKSPACE;
  if (zone_c_rows < 0 || zone_c_rows > layout->zone_c_capacity) return RDKV_ERR_CAPACITY;
  DecodeParams p = base_params(layout, const_cast<void*>(cache), zone_c_rows, 0, 0);
  p.partials = static_cast<float*>(const_cast<void*>(workspace));
  p.out = out;
  return hip_status(launch_decode_merge(p, stream));
}

rdkv_status rdkv_decode(const rdkv_layout* layout, void* cache, size_t cache_bytes, int32_t c_len,
                        const void* q, const void* k_new, const void* v_new, float* out,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  DecodeParams p;
  rdkv_status st = decode_params(layout, cache, cache_bytes, c_len, q, k_new, v_new, workspace, workspace_bytes, &p);
  if (st != RDKV_OK) return st;
  if (!out) return RDKV_ERR_NULL;
  if (!aligned16(out)) return RDKV_ERR_ALIGN;
  p.out = out;
  hipError_t e = launch_decode_chunks(p, stream);
  if (e == hipSuccess) e = launch_decode_merge(p, stream);
  return hip_status(e);
}

rdkv_status rdkv_decode_static(const rdkv_layout* layout, void* cache, size_t cache_bytes, int32_t c_len,
                               const void* q, const void* k_new, const void* v_new, float* out,
                               hipStream_t stream) {
  rdkv_status st = check_layout(layout);
  if (st != RDKV_OK) return st;
  if (layout->decode_workspace_bytes > kStaticScratchBytes) return RDKV_ERR_WORKSPACE;
  if (!out) return RDKV_ERR_NULL;
  if (!aligned16(out)) return RDKV_ERR_ALIGN;
  // every argument is validated before the device is touched
  DecodeParams p;
  st = decode_params(layout, cache, cache_bytes, c_len, q, k_new, v_new, nullptr, 0, &p, true);
  if (st != RDKV_OK) return st;
  void* scratch = nullptr;
  if (static_scratch(&scratch) != hipSuccess) return RDKV_ERR_HIP;
  p.partials = static_cast<float*>(scratch);
  p.out = out;
  hipError_t e = launch_decode_chunks(p, stream);
  if (e == hipSuccess) e = launch_decode_merge(p, stream);
  return hip_status(e);
}

rdkv_status rdkv_decode_accumulate(const rdkv_layout* layout, void* cache, size_t cache_bytes, int32_t c_len,
                                   const void* q, const void* k_new, const void* v_new, float* out,
                                   float* zc_stats, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  DecodeParams p;
  rdkv_status st = decode_params(layout, cache, cache_bytes, c_len, q, k_new, v_new, workspace, workspace_bytes, &p);
  if (st != RDKV_OK) return st;
  if (layout->n_generations < 1) return RDKV_ERR_SHAPE;
  if (!out || !zc_stats) return RDKV_ERR_NULL;
  if (!aligned16(out) || !aligned16(zc_stats)) return RDKV_ERR_ALIGN;
  p.out = out;
  p.zc_stats = zc_stats;
  hipError_t e = launch_decode_chunks(p, stream);
  if (e == hipSuccess) e = launch_decode_merge(p, stream);
  return hip_status(e);
}

rdkv_status rdkv_rollover_score(const rdkv_layout* layout, const void* cache, size_t cache_bytes,
                                const float* zc_stats, float* w_tok, float* var_tok, float* w_chan,
                                hipStream_t stream) {
  rdkv_status st = check_layout(layout);
  if (st != RDKV_OK) return st;
  if (layout->n_generations < 1) return RDKV_ERR_SHAPE;
  if (!cache || !zc_stats || !w_tok || !var_tok || !w_chan) return RDKV_ERR_NULL;
  for (const void* ptr : {cache, (const void*)zc_stats, (const void*)w_tok, (const void*)var_tok, (const void*)w_chan})
    if (!aligned16(ptr)) return RDKV_ERR_ALIGN;
  if (cache_bytes < layout->cache_bytes) return RDKV_ERR_WORKSPACE;
  RolloverParams r = rollover_params(*layout, const_cast<void*>(cache), const_cast<float*>(zc_stats));
  r.w_tok = w_tok;
  r.var_tok = var_tok;
  r.w_chan = w_chan;
  return hip_status(launch_rollover_score(r, stream));
}

rdkv_status rdkv_rollover(const rdkv_layout* layout, void* cache, size_t cache_bytes, int32_t generation,
                          float* zc_stats, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  rdkv_status st = check_layout(layout);
  if (st != RDKV_OK) return st;
  if (layout->n_generations < 1) return RDKV_ERR_SHAPE;
  if (!cache || !zc_stats || !workspace) return RDKV_ERR_NULL;
  for (const void* ptr : {(const void*)cache, (const void*)zc_stats, (const void*)workspace})
    if (!aligned16(ptr)) return RDKV_ERR_ALIGN;
  if (cache_bytes < layout->cache_bytes || workspace_bytes < layout->rollover_workspace_bytes)
    return RDKV_ERR_WORKSPACE;
  if (generation < 0 || generation >= layout->n_generations) return RDKV_ERR_CAPACITY;
  RolloverParams r = rollover_params(*layout, cache, zc_stats);
  const rdkv_layout g = generation_layout(*layout);
  return hip_status(launch_rollover(r, g, generation, static_cast<uint8_t*>(workspace), stream));
}

// ------------------------------------------------------------------ paged cache

rdkv_status rdkv_paged_layout_init(const rdkv_dims* dims_max, int64_t budget_v_max, int64_t budget_k_max,
                                   int32_t zone_c_capacity, int64_t n_pages, rdkv_paged_layout* out) {
  if (!out) return RDKV_ERR_NULL;
  rdkv_layout b;   // the bounds, as a contiguous layout of the same shape
  rdkv_status st = layout_init(dims_max, budget_v_max, budget_k_max, zone_c_capacity, 0, 0, 0, &b);
  if (st != RDKV_OK) return st;
  if (dims_max->n_seq > kMaxPagedSeqs || n_pages < 1 || n_pages > (int64_t(1) << 30)) return RDKV_ERR_SHAPE;
  rdkv_paged_layout P;
  std::memset(&P, 0, sizeof(P));
  P.dims = *dims_max;
  P.budget_v_max = budget_v_max;
  P.budget_k_max = budget_k_max;
  P.n_seg = b.n_seg;
  P.n_pages = n_pages;
  P.nk_max = b.nk_max;
  P.zone_c_capacity = zone_c_capacity;
  P.rec_max = b.rec_max;
  // Split-K granularity: the contiguous rule sizes chunks for every segment
  // holding its whole bound, which a budget shared across segments (bounds of
  // the group's budget) makes several times what they hold together.  The
  // pool bounds that total: at most n_pages * kPageBytes / 32 2-bit V rows, so
  // the chunk size is the smaller of the two rules' (equal to the contiguous
  // layout's whenever the pool is at least what the bounds need).
  const int64_t v_units = std::min<int64_t>(budget_v_max / 2, 8 * dims_max->n_tokens);
  const uint64_t pool_units = uint64_t(n_pages) * kPageBytes / 32;
  int64_t t2 = kChunkTok2Min;
  while (t2 < b.chunk_tok2 && pool_units / uint64_t(2 * t2) >= uint64_t(kDecodeTargetChunks)) t2 *= 2;
  P.chunk_tok2 = int32_t(t2);
  P.token_slots = int32_t(v_units / t2 + 4);
  P.max_chunks = int32_t(P.token_slots + cdiv(zone_c_capacity, kChunkRowsC));
  // block-table width: every region at its own worst case within the bounds
  const int64_t N = dims_max->n_tokens;
  int64_t pages = 0;
  for (int g = 0; g < 4; ++g) {
    const int64_t rows = std::min<int64_t>(N, budget_v_max / (int64_t(2) << g));
    pages += paged_region_pages(rows, paged_tile_bytes(kRegV + g, 0));
    pages += paged_region_pages(rows, uint32_t(kPagedTile) * uint32_t(b.rec_max));
  }
  pages += 2 * paged_region_pages(zone_c_capacity, paged_tile_bytes(kRegKC, 0));
  pages += paged_region_pages(b.nk_max, paged_tile_bytes(kRegPos, 0));
  P.max_pages = std::max<int64_t>(pages, 1);
  P.table_offset = align_up(kHeaderBytes + uint64_t(kDescBytes) * P.n_seg, kAlign);
  P.pool_offset = align_up(P.table_offset + 4 * uint64_t(P.n_seg) * P.max_pages, 4096);
  P.cache_bytes = P.pool_offset + uint64_t(n_pages) * kPageBytes;
  if (P.cache_bytes >= kPagedMaxCacheBytes) return RDKV_ERR_SHAPE;   // tile offsets fit 32 bits in 256-byte units
  const int G = dims_max->n_q_heads / dims_max->n_kv_heads;
  P.decode_workspace_bytes = uint64_t(P.n_seg) * P.max_chunks * G * kPartialFloats * sizeof(float);
  *out = P;
  return RDKV_OK;
}

}  // extern "C"

namespace {

rdkv_status check_paged(const rdkv_paged_layout* pl) {
  if (!pl) return RDKV_ERR_NULL;
  rdkv_paged_layout ref;
  rdkv_status st = rdkv_paged_layout_init(&pl->dims, pl->budget_v_max, pl->budget_k_max, pl->zone_c_capacity,
                                          pl->n_pages, &ref);
  if (st != RDKV_OK) return st;
  if (std::memcmp(&ref, pl, sizeof(ref)) != 0) return RDKV_ERR_SHAPE;
  return RDKV_OK;
}

// The contiguous layout one sequence is staged in: its own length and
// budgets, within the paged layout's bounds, no zone C.
rdkv_status staging_layout(const rdkv_paged_layout* pl, int64_t n_tokens, int64_t budget_v, int64_t budget_k,
                           rdkv_layout* out) {
  if (n_tokens < 1 || n_tokens > pl->dims.n_tokens) return RDKV_ERR_SHAPE;
  if (budget_v < 0 || budget_k < 0 || budget_v > pl->budget_v_max || budget_k > pl->budget_k_max)
    return RDKV_ERR_BUDGET;
  rdkv_dims d = pl->dims;
  d.n_seq = 1;
  d.n_tokens = n_tokens;
  return layout_init(&d, budget_v, budget_k, 0, 0, 0, 0, out);
}

}  // namespace

extern "C" {

rdkv_status rdkv_paged_cache_init(const rdkv_paged_layout* layout, void* cache, size_t cache_bytes,
                                  hipStream_t stream) {
  rdkv_status st = check_paged(layout);
  if (st != RDKV_OK) return st;
  if (!cache) return RDKV_ERR_NULL;
  if (!aligned16(cache)) return RDKV_ERR_ALIGN;
  if (cache_bytes < layout->cache_bytes) return RDKV_ERR_WORKSPACE;
  return hip_status(launch_paged_init(static_cast<uint8_t*>(cache), *layout, stream));
}

size_t rdkv_paged_staging_bytes(const rdkv_paged_layout* layout, int64_t n_tokens, int64_t budget_v,
                                int64_t budget_k) {
  if (check_paged(layout) != RDKV_OK) return 0;
  rdkv_layout s;
  if (staging_layout(layout, n_tokens, budget_v, budget_k, &s) != RDKV_OK) return 0;
  return s.cache_bytes;
}

rdkv_status rdkv_paged_stage(const rdkv_paged_layout* layout, int64_t n_tokens, int64_t budget_v,
                             int64_t budget_k, const void* K, const void* V, const uint8_t* bits_tok,
                             const uint8_t* bits_chan, void* staging, size_t staging_bytes,
                             int32_t* pages_needed, hipStream_t stream) {
  rdkv_status st = check_paged(layout);
  if (st != RDKV_OK) return st;
  rdkv_layout sl;
  st = staging_layout(layout, n_tokens, budget_v, budget_k, &sl);
  if (st != RDKV_OK) return st;
  if (!K || !V || !bits_tok || !bits_chan || !staging || !pages_needed) return RDKV_ERR_NULL;
  for (const void* ptr : {K, V, (const void*)bits_tok, (const void*)bits_chan, (const void*)staging,
                          (const void*)pages_needed})
    if (!aligned16(ptr)) return RDKV_ERR_ALIGN;
  if (staging_bytes < sl.cache_bytes) return RDKV_ERR_WORKSPACE;
  hipError_t e = launch_cache_init(static_cast<uint8_t*>(staging), sl, nullptr, stream);
  if (e != hipSuccess) return RDKV_ERR_HIP;
  PackParams pp;
  pp.cache = static_cast<uint8_t*>(staging);
  pp.cache_bytes = staging_bytes;
  pp.lay = &sl;
  pp.layer_begin = 0;
  pp.n_layers_in = sl.dims.n_layers;
  pp.K = static_cast<const __half*>(K);
  pp.V = static_cast<const __half*>(V);
  pp.bits_tok = bits_tok;
  pp.bits_chan = bits_chan;
  e = launch_pack(pp, stream);
  if (e != hipSuccess) return RDKV_ERR_HIP;
  PagedPackParams q{nullptr, layout, static_cast<const uint8_t*>(staging), sl.cache_bytes, 0, nullptr, pages_needed};
  return hip_status(launch_paged_plan(q, stream));
}

rdkv_status rdkv_paged_commit(const rdkv_paged_layout* layout, int32_t seq, int64_t n_tokens, int64_t budget_v,
                              int64_t budget_k, const void* staging, size_t staging_bytes, const int32_t* pages,
                              void* cache, size_t cache_bytes, hipStream_t stream) {
  rdkv_status st = check_paged(layout);
  if (st != RDKV_OK) return st;
  rdkv_layout sl;
  st = staging_layout(layout, n_tokens, budget_v, budget_k, &sl);
  if (st != RDKV_OK) return st;
  if (!staging || !pages || !cache) return RDKV_ERR_NULL;
  for (const void* ptr : {staging, (const void*)pages, (const void*)cache})
    if (!aligned16(ptr)) return RDKV_ERR_ALIGN;
  if (staging_bytes < sl.cache_bytes || cache_bytes < layout->cache_bytes) return RDKV_ERR_WORKSPACE;
  if (seq < 0 || seq >= layout->dims.n_seq) return RDKV_ERR_SHAPE;
  PagedPackParams q{static_cast<uint8_t*>(cache), layout, static_cast<const uint8_t*>(staging), sl.cache_bytes, seq,
                    pages, nullptr};
  return hip_status(launch_paged_commit(q, stream));
}

rdkv_status rdkv_paged_release(const rdkv_paged_layout* layout, int32_t seq, void* cache, size_t cache_bytes,
                               hipStream_t stream) {
  rdkv_status st = check_paged(layout);
  if (st != RDKV_OK) return st;
  if (!cache) return RDKV_ERR_NULL;
  if (!aligned16(cache)) return RDKV_ERR_ALIGN;
  if (cache_bytes < layout->cache_bytes) return RDKV_ERR_WORKSPACE;
  if (seq < 0 || seq >= layout->dims.n_seq) return RDKV_ERR_SHAPE;
  return hip_status(launch_paged_release(static_cast<uint8_t*>(cache), *layout, seq, stream));
}

}  // extern "C"

namespace {

ShapeGeom shape_geom(const rdkv_paged_layout& pl) {
  return ShapeGeom{pl.n_seg, pl.zone_c_capacity, pl.chunk_tok2, pl.token_slots, pl.rec_max,
                   pl.dims.n_q_heads / pl.dims.n_kv_heads};
}
ShapeGeom shape_geom(const rdkv_layout& l) {   // the prefill blob's segments
  return ShapeGeom{l.n_seg, l.zone_c_capacity, l.chunk_tok2, l.token_slots, l.rec_max,
                   l.dims.n_q_heads / l.dims.n_kv_heads};
}

// A launch shape read back from the device: the most prefill-token chunks
// and the longest record over the segments in use, within the bounds.
rdkv_status measure_shape(const uint8_t* cache, const ShapeGeom& g, int32_t zc_and_gen_slots, void* workspace,
                          hipStream_t stream, rdkv_launch_shape* out) {
  int32_t* dev = static_cast<int32_t*>(workspace);
  hipError_t e = launch_shape_scan(cache, g, dev, stream);
  int32_t host[2] = {0, 0};
  if (e == hipSuccess) e = hipMemcpyAsync(host, dev, sizeof(host), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_status(e);
  rdkv_launch_shape sh{};
  sh.token_slots = std::min(host[0], g.token_slots);
  sh.rec_max = std::min((host[1] + 3) / 4 * 4, g.rec_max);
  sh.max_chunks = sh.token_slots + zc_and_gen_slots;
  sh.decode_workspace_bytes = uint64_t(g.n_seg) * sh.max_chunks * g.group * kPartialFloats * sizeof(float);
  *out = sh;
  return RDKV_OK;
}

// A caller's shape against the bounds it must stay within.
bool shape_ok(const rdkv_launch_shape& sh, int32_t token_slots, int32_t rec_max) {
  return sh.reserved == 0 && sh.token_slots >= 0 && sh.token_slots <= token_slots && sh.rec_max >= 0 &&
         sh.rec_max <= rec_max && sh.rec_max % 4 == 0;
}

// One paged decode step with the launch shape (prefill chunk slots, record
// bound) of the layout or of a rdkv_paged_decode_shape result.
rdkv_status paged_decode(const rdkv_paged_layout* layout, const rdkv_launch_shape* shape, void* cache,
                         size_t cache_bytes, const int32_t* c_len, const void* q, const void* k_new, const void* v_new,
                         float* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  rdkv_status st = check_paged(layout);
  if (st != RDKV_OK) return st;
  if (!cache || !c_len || !q || !out || !workspace) return RDKV_ERR_NULL;
  if ((k_new == nullptr) != (v_new == nullptr)) return RDKV_ERR_NULL;
  for (const void* ptr : {(const void*)cache, q, (const void*)out, (const void*)workspace})
    if (!aligned16(ptr)) return RDKV_ERR_ALIGN;
  if (k_new && (!aligned16(k_new) || !aligned16(v_new))) return RDKV_ERR_ALIGN;
  const int G = layout->dims.n_q_heads / layout->dims.n_kv_heads;
  const int zc_slots = layout->max_chunks - layout->token_slots;
  int32_t token_slots = layout->token_slots, rec_max = layout->rec_max;
  if (shape) {
    if (!shape_ok(*shape, layout->token_slots, layout->rec_max)) return RDKV_ERR_SHAPE;
    token_slots = shape->token_slots;
    rec_max = shape->rec_max;
  }
  const int32_t max_chunks = token_slots + zc_slots;
  const uint64_t ws_need = uint64_t(layout->n_seg) * max_chunks * G * kPartialFloats * sizeof(float);
  if (cache_bytes < layout->cache_bytes || workspace_bytes < ws_need) return RDKV_ERR_WORKSPACE;
  const int append = k_new != nullptr;
  PagedSeqLens lens;
  std::memset(&lens, 0, sizeof(lens));
  for (int s = 0; s < layout->dims.n_seq; ++s) {
    if (c_len[s] < 0 || int64_t(c_len[s]) + append > layout->zone_c_capacity) return RDKV_ERR_CAPACITY;
    lens.c_len[s] = c_len[s];
  }
  DecodeParams p{};
  p.cache = static_cast<uint8_t*>(cache);
  p.cache_bytes = layout->cache_bytes;
  p.main_bytes = layout->cache_bytes;
  p.n_seg = layout->n_seg;
  p.nk_max = layout->nk_max;
  p.max_chunks = max_chunks;
  p.token_slots = token_slots;
  p.chunk_tok2 = layout->chunk_tok2;
  p.rec_max = rec_max;
  p.group = G;
  p.zc_cap = layout->zone_c_capacity;
  p.append = append;
  p.q = static_cast<const __half*>(q);
  p.k_new = static_cast<const __half*>(k_new);
  p.v_new = static_cast<const __half*>(v_new);
  p.partials = static_cast<float*>(workspace);
  p.out = out;
  p.paged = 1;
  p.seg_per_seq = layout->dims.n_layers * layout->dims.n_kv_heads;
  p.max_pages = int32_t(layout->max_pages);
  p.pool_pages = layout->n_pages;
  p.table_offset = layout->table_offset;
  p.pool_offset = layout->pool_offset;
  hipError_t e = launch_decode_chunks_paged(p, lens, stream);
  if (e == hipSuccess) e = launch_decode_merge(p, stream);
  if (e == hipSuccess && shape)
    e = launch_shape_check(p.cache, shape_geom(*layout), token_slots, rec_max, out, stream);
  return hip_status(e);
}

}  // namespace

extern "C" {

rdkv_status rdkv_paged_decode(const rdkv_paged_layout* layout, void* cache, size_t cache_bytes,
                              const int32_t* c_len, const void* q, const void* k_new, const void* v_new,
                              float* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return paged_decode(layout, nullptr, cache, cache_bytes, c_len, q, k_new, v_new, out, workspace, workspace_bytes,
                      stream);
}

rdkv_status rdkv_paged_decode_shape(const rdkv_paged_layout* layout, const void* cache, size_t cache_bytes,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream,
                                    rdkv_launch_shape* out) {
  rdkv_status st = check_paged(layout);
  if (st != RDKV_OK) return st;
  if (!cache || !workspace || !out) return RDKV_ERR_NULL;
  if (!aligned16(cache) || !aligned16(workspace)) return RDKV_ERR_ALIGN;
  if (cache_bytes < layout->cache_bytes || workspace_bytes < 8) return RDKV_ERR_WORKSPACE;
  return measure_shape(static_cast<const uint8_t*>(cache), shape_geom(*layout),
                       layout->max_chunks - layout->token_slots, workspace, stream, out);
}

rdkv_status rdkv_paged_decode_shaped(const rdkv_paged_layout* layout, const rdkv_launch_shape* shape, void* cache,
                                     size_t cache_bytes, const int32_t* c_len, const void* q, const void* k_new,
                                     const void* v_new, float* out, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  if (!shape) return RDKV_ERR_NULL;
  return paged_decode(layout, shape, cache, cache_bytes, c_len, q, k_new, v_new, out, workspace, workspace_bytes,
                      stream);
}

rdkv_status rdkv_unpack(const rdkv_layout* layout, const void* cache, size_t cache_bytes, int64_t seg,
                        float* k_hat, float* v_hat, hipStream_t stream) {
  rdkv_status st = check_layout(layout);
  if (st != RDKV_OK) return st;
  if (!cache || !k_hat || !v_hat) return RDKV_ERR_NULL;
  for (const void* p : {cache, (const void*)k_hat, (const void*)v_hat})
    if (!aligned16(p)) return RDKV_ERR_ALIGN;
  if (seg < 0 || seg >= layout->n_seg) return RDKV_ERR_SHAPE;
  if (cache_bytes < layout->cache_bytes) return RDKV_ERR_WORKSPACE;
  return hip_status(launch_unpack(static_cast<const uint8_t*>(cache), layout->cache_bytes, *layout, seg,
                                  k_hat, v_hat, stream));
}

rdkv_status rdkv_decode_shape(const rdkv_layout* layout, const void* cache, size_t cache_bytes, void* workspace,
                              size_t workspace_bytes, hipStream_t stream, rdkv_launch_shape* out) {
  rdkv_status st = check_layout(layout);
  if (st != RDKV_OK) return st;
  if (!cache || !workspace || !out) return RDKV_ERR_NULL;
  if (!aligned16(cache) || !aligned16(workspace)) return RDKV_ERR_ALIGN;
  if (cache_bytes < layout->cache_bytes || workspace_bytes < 8) return RDKV_ERR_WORKSPACE;
  return measure_shape(static_cast<const uint8_t*>(cache), shape_geom(*layout),
                       layout->max_chunks - layout->token_slots, workspace, stream, out);
}

rdkv_status rdkv_decode_shaped(const rdkv_layout* layout, const rdkv_launch_shape* shape, void* cache,
                               size_t cache_bytes, int32_t c_len, const void* q, const void* k_new, const void* v_new,
                               float* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  rdkv_status st = check_layout(layout);
  if (st != RDKV_OK) return st;
  if (!shape || !out) return RDKV_ERR_NULL;
  if (!shape_ok(*shape, layout->token_slots, layout->rec_max)) return RDKV_ERR_SHAPE;
  const int G = layout->dims.n_q_heads / layout->dims.n_kv_heads;
  const int32_t max_chunks = shape->token_slots + (layout->max_chunks - layout->token_slots);
  const uint64_t ws_need = uint64_t(layout->n_seg) * max_chunks * G * kPartialFloats * sizeof(float);
  DecodeParams p;
  st = decode_params(layout, cache, cache_bytes, c_len, q, k_new, v_new, workspace, workspace_bytes, &p, false,
                     ws_need);
  if (st != RDKV_OK) return st;
  if (!aligned16(out)) return RDKV_ERR_ALIGN;
  p.out = out;
  p.token_slots = shape->token_slots;   // the prefill blob's chunks; generations and zone C follow them
  p.max_chunks = max_chunks;
  p.rec_max = shape->rec_max;
  hipError_t e = launch_decode_chunks(p, stream);
  if (e == hipSuccess) e = launch_decode_merge(p, stream);
  if (e == hipSuccess) e = launch_shape_check(p.cache, shape_geom(*layout), p.token_slots, p.rec_max, out, stream);
  return hip_status(e);
}

}  // extern "C"
