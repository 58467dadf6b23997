// Host-side checks of the C ABI's validation and layout arithmetic, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code (the
// kernels are not in this build: a launch fails, which the entry points
// report as RDKV_ERR_HIP).  Device pointers are addresses of a host array that
// no host code reads or writes.  Every entry point is called with valid
// arguments, with each pointer NULL or misaligned, with short buffers and with
// tampered layouts; then random and extreme shapes, budgets and lengths are
// thrown at the layout functions and the entry points.  Exit status 0: every
// expectation held and the sanitizers reported nothing (they abort on the
// first finding).
#include "rdkv.h"

#include <cinttypes>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>

namespace {

alignas(4096) unsigned char g_dev[1 << 12];
void* const D = g_dev;
void* const M = g_dev + 4;  // misaligned
int g_fail = 0, g_checks = 0;

#define EXPECT(cond, ...)                                      \
  do {                                                         \
    ++g_checks;                                                \
    if (!(cond)) {                                             \
      ++g_fail;                                                \
      std::printf("FAIL line %d: ", __LINE__);                 \
      std::printf(__VA_ARGS__);                                \
      std::printf("\n");                                       \
    }                                                          \
  } while (0)

bool ok_or_hip(rdkv_status s) { return s == RDKV_OK || s == RDKV_ERR_HIP; }
float* F(void* p) { return static_cast<float*>(p); }
uint8_t* U(void* p) { return static_cast<uint8_t*>(p); }

rdkv_dims dims(int64_t N, int32_t S, int32_t L, int32_t Hq, int32_t Hkv) {
  rdkv_dims d;
  std::memset(&d, 0, sizeof(d));
  d.n_tokens = N;
  d.n_seq = S;
  d.n_layers = L;
  d.n_q_heads = Hq;
  d.n_kv_heads = Hkv;
  d.head_dim = 128;
  return d;
}

void scoring(const rdkv_dims& d) {
  const size_t ws = rdkv_score_workspace_bytes(&d);
  EXPECT(ok_or_hip(rdkv_score(&d, D, D, D, F(D), F(D), F(D), D, ws, nullptr)), "score");
  EXPECT(rdkv_score(&d, nullptr, D, D, F(D), F(D), F(D), D, ws, nullptr) == RDKV_ERR_NULL, "score null Q");
  EXPECT(rdkv_score(&d, D, D, D, F(M), F(D), F(D), D, ws, nullptr) == RDKV_ERR_ALIGN, "score misaligned");
  if (ws > 0) EXPECT(rdkv_score(&d, D, D, D, F(D), F(D), F(D), D, ws - 1, nullptr) == RDKV_ERR_WORKSPACE, "score ws");
  EXPECT(ok_or_hip(rdkv_score_lse(&d, D, D, F(D), nullptr)), "score_lse");
  EXPECT(rdkv_score_lse(&d, D, nullptr, F(D), nullptr) == RDKV_ERR_NULL, "score_lse null K");
  EXPECT(ok_or_hip(rdkv_score_from_lse(&d, D, D, D, F(D), F(D), F(D), F(D), D, ws, nullptr)), "score_from_lse");
  EXPECT(rdkv_score_from_lse(&d, D, D, D, nullptr, F(D), F(D), F(D), D, ws, nullptr) == RDKV_ERR_NULL, "lse null");
  const size_t aw = rdkv_allocate_workspace_bytes(&d, 1);
  EXPECT(ok_or_hip(rdkv_allocate(&d, F(D), F(D), F(D), D, 100, 50, U(D), U(D), F(D), (double*)D, D, aw, nullptr)),
         "alloc");
  EXPECT(rdkv_allocate(&d, F(D), F(D), F(D), D, -1, 50, U(D), U(D), F(D), (double*)D, D, aw, nullptr) ==
             RDKV_ERR_BUDGET,
         "alloc negative budget");
  EXPECT(rdkv_allocate(&d, F(D), F(D), F(D), D, 100, 50, nullptr, U(D), F(D), (double*)D, D, aw, nullptr) ==
             RDKV_ERR_NULL,
         "alloc null out");
  if (aw > 0)
    EXPECT(rdkv_allocate(&d, F(D), F(D), F(D), D, 100, 50, U(D), U(D), F(D), (double*)D, D, aw - 1, nullptr) ==
               RDKV_ERR_WORKSPACE,
           "alloc small workspace");
  EXPECT(ok_or_hip(rdkv_allocate_shared(&d, F(D), F(D), F(D), D, 100, 50, 1, U(D), U(D), F(D), (double*)D, D, aw,
                                        nullptr)),
         "alloc shared");
  EXPECT(rdkv_allocate_shared(&d, F(D), F(D), F(D), D, 100, 50, 0, U(D), U(D), F(D), (double*)D, D, aw, nullptr) !=
             RDKV_OK,
         "alloc shared group 0");
}

void contiguous(const rdkv_layout& lay) {
  const size_t cb = lay.cache_bytes, wb = lay.decode_workspace_bytes;
  const int32_t L = lay.dims.n_layers, cap = lay.zone_c_capacity;
  EXPECT(ok_or_hip(rdkv_cache_init(&lay, D, cb, nullptr)), "cache_init");
  EXPECT(rdkv_cache_init(&lay, nullptr, cb, nullptr) == RDKV_ERR_NULL, "cache_init null");
  EXPECT(rdkv_cache_init(&lay, M, cb, nullptr) == RDKV_ERR_ALIGN, "cache_init misaligned");
  EXPECT(rdkv_cache_init(&lay, D, cb - 1, nullptr) == RDKV_ERR_WORKSPACE, "cache_init short");
  EXPECT(ok_or_hip(rdkv_pack(&lay, 0, L, D, D, U(D), U(D), D, cb, nullptr)), "pack");
  EXPECT(rdkv_pack(&lay, L, 1, D, D, U(D), U(D), D, cb, nullptr) == RDKV_ERR_SHAPE, "pack layer past end");
  EXPECT(rdkv_pack(&lay, 0, L, D, nullptr, U(D), U(D), D, cb, nullptr) == RDKV_ERR_NULL, "pack null V");
  int32_t dropped = 0;
  EXPECT(ok_or_hip(rdkv_pack_status(&lay, D, cb, &dropped, nullptr)), "pack_status");
  EXPECT(ok_or_hip(rdkv_decode(&lay, D, cb, 0, D, D, D, F(D), D, wb, nullptr)), "decode");
  {
    rdkv_launch_shape sh{};
    EXPECT(ok_or_hip(rdkv_decode_shape(&lay, D, cb, D, wb, nullptr, &sh)), "decode shape");
    EXPECT(rdkv_decode_shape(&lay, D, cb, D, 7, nullptr, &sh) == RDKV_ERR_WORKSPACE, "decode shape workspace");
    sh = rdkv_launch_shape{lay.token_slots, lay.rec_max, lay.max_chunks, 0, 0};
    EXPECT(ok_or_hip(rdkv_decode_shaped(&lay, &sh, D, cb, 0, D, D, D, F(D), D, wb, nullptr)), "shaped decode");
    sh.rec_max = lay.rec_max + 4;
    EXPECT(rdkv_decode_shaped(&lay, &sh, D, cb, 0, D, D, D, F(D), D, wb, nullptr) == RDKV_ERR_SHAPE,
           "shaped decode past the bounds");
    EXPECT(rdkv_decode_shaped(&lay, nullptr, D, cb, 0, D, D, D, F(D), D, wb, nullptr) == RDKV_ERR_NULL,
           "shaped decode without a shape");
  }
  EXPECT(ok_or_hip(rdkv_decode(&lay, D, cb, cap, D, nullptr, nullptr, F(D), D, wb, nullptr)), "decode full zone C");
  EXPECT(rdkv_decode(&lay, D, cb, cap, D, D, D, F(D), D, wb, nullptr) == RDKV_ERR_CAPACITY, "decode over capacity");
  EXPECT(rdkv_decode(&lay, D, cb, -1, D, D, D, F(D), D, wb, nullptr) != RDKV_OK, "decode negative c_len");
  EXPECT(rdkv_decode(&lay, D, cb, 0, D, D, nullptr, F(D), D, wb, nullptr) == RDKV_ERR_NULL, "decode half append");
  if (wb > 0) EXPECT(rdkv_decode(&lay, D, cb, 0, D, D, D, F(D), D, wb - 1, nullptr) == RDKV_ERR_WORKSPACE, "decode ws");
  EXPECT(ok_or_hip(rdkv_decode_partials(&lay, D, cb, 0, D, D, D, D, wb, nullptr)), "partials");
  EXPECT(ok_or_hip(rdkv_decode_merge(&lay, D, cb, 1, F(D), D, wb, nullptr)), "merge");
  EXPECT(rdkv_decode_merge(&lay, D, cb, cap + 1, F(D), D, wb, nullptr) != RDKV_OK, "merge rows past capacity");
  rdkv_status s = rdkv_decode_static(&lay, D, cb, 0, D, D, D, F(D), nullptr);
  EXPECT(ok_or_hip(s) || s == RDKV_ERR_WORKSPACE, "decode_static");
  EXPECT(ok_or_hip(rdkv_unpack(&lay, D, cb, 0, F(D), F(D), nullptr)), "unpack");
  EXPECT(rdkv_unpack(&lay, D, cb, lay.n_seg, F(D), F(D), nullptr) == RDKV_ERR_SHAPE, "unpack segment past end");
  if (lay.n_generations > 0) {
    EXPECT(ok_or_hip(rdkv_decode_accumulate(&lay, D, cb, 0, D, D, D, F(D), F(D), D, wb, nullptr)), "accumulate");
    EXPECT(rdkv_decode_accumulate(&lay, D, cb, 0, D, D, D, F(D), nullptr, D, wb, nullptr) == RDKV_ERR_NULL,
           "accumulate null stats");
    EXPECT(ok_or_hip(rdkv_rollover_score(&lay, D, cb, F(D), F(D), F(D), F(D), nullptr)), "rollover_score");
    const size_t rb = lay.rollover_workspace_bytes;
    EXPECT(ok_or_hip(rdkv_rollover(&lay, D, cb, 0, F(D), D, rb, nullptr)), "rollover");
    EXPECT(rdkv_rollover(&lay, D, cb, lay.n_generations, F(D), D, rb, nullptr) == RDKV_ERR_CAPACITY,
           "rollover generation past end");
    EXPECT(rdkv_rollover(&lay, D, cb, 0, F(D), D, rb - 1, nullptr) == RDKV_ERR_WORKSPACE, "rollover ws");
  }
  // a layout not made by rdkv_layout_init*: every field changed in turn
  for (size_t i = 0; i < sizeof(rdkv_layout); i += 4) {
    rdkv_layout bad = lay;
    reinterpret_cast<unsigned char*>(&bad)[i] ^= 0x5A;
    const rdkv_status st = rdkv_decode(&bad, D, cb, 0, D, D, D, F(D), D, wb, nullptr);
    EXPECT(st != RDKV_OK, "tampered layout byte %zu accepted", i);
  }
}

void paged(const rdkv_paged_layout& pl) {
  const size_t cb = pl.cache_bytes, wb = pl.decode_workspace_bytes;
  const int64_t N = pl.dims.n_tokens, bv = pl.budget_v_max, bk = pl.budget_k_max;
  EXPECT(ok_or_hip(rdkv_paged_cache_init(&pl, D, cb, nullptr)), "paged init");
  EXPECT(rdkv_paged_cache_init(&pl, D, cb - 1, nullptr) == RDKV_ERR_WORKSPACE, "paged init short");
  const size_t sb = rdkv_paged_staging_bytes(&pl, N, bv, bk);
  EXPECT(sb > 0, "staging bytes");
  EXPECT(rdkv_paged_staging_bytes(&pl, N + 1, bv, bk) == 0, "staging bytes past the length bound");
  int32_t need[4096];
  EXPECT(ok_or_hip(rdkv_paged_stage(&pl, N, bv, bk, D, D, U(D), U(D), D, sb, need, nullptr)), "stage");
  EXPECT(rdkv_paged_stage(&pl, N, bv, bk, D, D, U(D), U(D), D, sb - 1, need, nullptr) == RDKV_ERR_WORKSPACE,
         "stage short");
  EXPECT(rdkv_paged_stage(&pl, N, bv, bk, D, D, U(D), U(D), D, sb, nullptr, nullptr) == RDKV_ERR_NULL, "stage null");
  EXPECT(ok_or_hip(rdkv_paged_commit(&pl, 0, N, bv, bk, D, sb, static_cast<const int32_t*>(D), D, cb, nullptr)),
         "commit");
  EXPECT(rdkv_paged_commit(&pl, pl.dims.n_seq, N, bv, bk, D, sb, static_cast<const int32_t*>(D), D, cb, nullptr) ==
             RDKV_ERR_SHAPE, "commit slot past end");
  EXPECT(ok_or_hip(rdkv_paged_release(&pl, 0, D, cb, nullptr)), "release");
  EXPECT(rdkv_paged_release(&pl, -1, D, cb, nullptr) == RDKV_ERR_SHAPE, "release negative slot");
  int32_t c_len[RDKV_MAX_PAGED_SEQS] = {0};
  EXPECT(ok_or_hip(rdkv_paged_decode(&pl, D, cb, c_len, D, D, D, F(D), D, wb, nullptr)), "paged decode");
  c_len[pl.dims.n_seq - 1] = pl.zone_c_capacity;
  EXPECT(rdkv_paged_decode(&pl, D, cb, c_len, D, D, D, F(D), D, wb, nullptr) == RDKV_ERR_CAPACITY,
         "paged decode over capacity");
  c_len[pl.dims.n_seq - 1] = -3;
  EXPECT(rdkv_paged_decode(&pl, D, cb, c_len, D, nullptr, nullptr, F(D), D, wb, nullptr) != RDKV_OK,
         "paged decode negative length");
  EXPECT(rdkv_paged_decode(&pl, D, cb, nullptr, D, nullptr, nullptr, F(D), D, wb, nullptr) == RDKV_ERR_NULL,
         "paged decode null lengths");
  {
    c_len[pl.dims.n_seq - 1] = 0;
    rdkv_launch_shape sh{};
    EXPECT(ok_or_hip(rdkv_paged_decode_shape(&pl, D, cb, D, wb, nullptr, &sh)), "decode shape");
    EXPECT(rdkv_paged_decode_shape(&pl, D, cb, D, 4, nullptr, &sh) == RDKV_ERR_WORKSPACE, "decode shape workspace");
    sh = rdkv_launch_shape{pl.token_slots, pl.rec_max, pl.max_chunks, 0, 0};
    EXPECT(ok_or_hip(rdkv_paged_decode_shaped(&pl, &sh, D, cb, c_len, D, D, D, F(D), D, wb, nullptr)),
           "shaped decode");
    sh.token_slots = pl.token_slots + 1;
    EXPECT(rdkv_paged_decode_shaped(&pl, &sh, D, cb, c_len, D, D, D, F(D), D, wb, nullptr) == RDKV_ERR_SHAPE,
           "shaped decode past the bounds");
    sh = rdkv_launch_shape{0, 0, 0, 0, 0};
    EXPECT(ok_or_hip(rdkv_paged_decode_shaped(&pl, &sh, D, cb, c_len, D, D, D, F(D), D, wb, nullptr)),
           "shaped decode, no prefill chunks");
  }
  for (size_t i = 0; i < sizeof(rdkv_paged_layout); i += 4) {
    rdkv_paged_layout bad = pl;
    reinterpret_cast<unsigned char*>(&bad)[i] ^= 0x21;
    EXPECT(rdkv_paged_cache_init(&bad, D, cb, nullptr) != RDKV_OK, "tampered paged layout byte %zu accepted", i);
  }
}

// Random and extreme arguments: only "no crash, no undefined behaviour" and
// internal consistency are checked.
void fuzz(unsigned seed, int rounds) {
  std::mt19937_64 r(seed);
  const int64_t big64[] = {0, 1, 63, 64, 65, 1000, 131072, 262144, int64_t(1) << 31, int64_t(1) << 40,
                           int64_t(1) << 62, INT64_MAX, -1, INT64_MIN};
  const int32_t big32[] = {0, 1, 2, 3, 4, 8, 16, 64, 129, 256, 257, 1 << 20, (1 << 20) + 1, INT32_MAX, -1, INT32_MIN};
  auto pick64 = [&]() { return (r() & 3) ? int64_t(r() % 300000) : big64[r() % (sizeof(big64) / 8)]; };
  auto pick32 = [&](int32_t hi) { return (r() & 3) ? int32_t(r() % hi) : big32[r() % (sizeof(big32) / 4)]; };
  int accepted = 0;
  for (int i = 0; i < rounds; ++i) {
    rdkv_dims d = dims(pick64(), pick32(5), pick32(100), pick32(65), pick32(9));
    if (r() % 8 == 0) d.head_dim = pick32(300);
    rdkv_layout lay;
    const int32_t cap = pick32(400);
    rdkv_status s = (r() & 1) ? rdkv_layout_init(&d, pick64(), pick64(), cap, &lay)
                              : rdkv_layout_init_rollover(&d, pick64(), pick64(), cap, pick32(6), pick64(), pick64(), &lay);
    (void)rdkv_score_workspace_bytes(&d);
    (void)rdkv_allocate_workspace_bytes(&d, pick32(700));
    if (s == RDKV_OK) {
      ++accepted;
      EXPECT(lay.cache_bytes > 0 && lay.n_seg > 0, "accepted layout with no bytes");
      const int32_t c = pick32(600);
      (void)rdkv_decode(&lay, D, lay.cache_bytes, c, D, D, D, F(D), D, lay.decode_workspace_bytes, nullptr);
      (void)rdkv_decode_merge(&lay, D, lay.cache_bytes, c, F(D), D, lay.decode_workspace_bytes, nullptr);
      const rdkv_launch_shape sh{pick32(lay.token_slots + 2), pick32(lay.rec_max + 8) & ~3, 0, 0, 0};
      (void)rdkv_decode_shaped(&lay, &sh, D, lay.cache_bytes, c, D, D, D, F(D), D, lay.decode_workspace_bytes,
                               nullptr);
      (void)rdkv_pack(&lay, pick32(100), pick32(100), D, D, U(D), U(D), D, lay.cache_bytes, nullptr);
      (void)rdkv_unpack(&lay, D, lay.cache_bytes, pick64(), F(D), F(D), nullptr);
      if (lay.n_generations > 0) (void)rdkv_rollover(&lay, D, lay.cache_bytes, pick32(8), F(D), D, lay.rollover_workspace_bytes, nullptr);
    }
    rdkv_paged_layout pl;
    d.n_seq = pick32(300);
    if (rdkv_paged_layout_init(&d, pick64(), pick64(), pick32(400), pick64(), &pl) == RDKV_OK) {
      ++accepted;
      const int64_t n = pick64(), bv = pick64(), bk = pick64();
      const size_t sb = rdkv_paged_staging_bytes(&pl, n, bv, bk);
      int32_t need[1024];
      if (pl.dims.n_layers * int64_t(pl.dims.n_kv_heads) <= 1024)
        (void)rdkv_paged_stage(&pl, n, bv, bk, D, D, U(D), U(D), D, sb, need, nullptr);
      (void)rdkv_paged_commit(&pl, pick32(300), n, bv, bk, D, sb, static_cast<const int32_t*>(D), D, pl.cache_bytes,
                              nullptr);
      int32_t c_len[RDKV_MAX_PAGED_SEQS];
      for (int k = 0; k < RDKV_MAX_PAGED_SEQS; ++k) c_len[k] = pick32(600);
      (void)rdkv_paged_decode(&pl, D, pl.cache_bytes, c_len, D, D, D, F(D), D, pl.decode_workspace_bytes, nullptr);
      const rdkv_launch_shape sh{pick32(pl.token_slots + 2), pick32(pl.rec_max + 8) & ~3, 0, 0, 0};
      (void)rdkv_paged_decode_shaped(&pl, &sh, D, pl.cache_bytes, c_len, D, D, D, F(D), D,
                                     pl.decode_workspace_bytes, nullptr);
    }
  }
  std::printf("fuzz seed %u: %d rounds, %d layouts accepted\n", seed, rounds, accepted);
}

}  // namespace

int main() {
  EXPECT(rdkv_version() > 0, "version");
  for (int32_t s : {-2, 0, 1, 9, 10, 11, 12345, INT32_MIN, INT32_MAX})
    EXPECT(rdkv_status_string(s) != nullptr, "status string %d", s);
  const rdkv_dims shapes[] = {dims(1000, 2, 2, 8, 2), dims(1024, 1, 1, 4, 1), dims(32768, 1, 1, 32, 8),
                              dims(131072, 1, 32, 32, 8), dims(262144, 1, 80, 64, 8), dims(65, 3, 2, 2, 2)};
  for (const rdkv_dims& d : shapes) {
    scoring(d);
    rdkv_layout lay;
    EXPECT(rdkv_layout_init(&d, 2 * d.n_tokens, 256, 128, &lay) == RDKV_OK, "layout");
    contiguous(lay);
    EXPECT(rdkv_layout_init_rollover(&d, 2 * d.n_tokens, 256, 64, 3, 128, 256, &lay) == RDKV_OK, "rollover layout");
    contiguous(lay);
    rdkv_paged_layout pl;
    EXPECT(rdkv_paged_layout_init(&d, 2 * d.n_tokens, 256, 64, 1000, &pl) == RDKV_OK, "paged layout");
    paged(pl);
  }
  rdkv_layout lay;
  EXPECT(rdkv_layout_init(nullptr, 1, 1, 1, &lay) == RDKV_ERR_NULL, "null dims");
  rdkv_dims d = dims(1000, 1, 1, 12, 4);
  EXPECT(rdkv_layout_init(&d, 1, 1, 1, &lay) == RDKV_ERR_UNSUPPORTED, "G = 3");
  d = dims(1000, 1, 1, 8, 2);
  d.head_dim = 64;
  EXPECT(rdkv_layout_init(&d, 1, 1, 1, &lay) == RDKV_ERR_UNSUPPORTED, "head_dim 64");
  fuzz(1, 20000);
  fuzz(2, 20000);
  std::printf("%d checks, %d failed\n", g_checks, g_fail);
  return g_fail == 0 ? 0 : 1;
}
