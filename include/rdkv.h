/*
 * rdkv.h -- C ABI of the RDKV hot path on MI355X (gfx950).
 *
 * RDKV compresses a KV cache after prefill by rate-distortion bit allocation:
 * every V token and every K channel of a (sequence, layer, KV head) "segment"
 * gets a bitwidth in {0, 2, 4, 8, 16}, 0 meaning eviction, chosen to minimise
 * sum_u w_u sigma_u 2^-b_u under a bit budget.  Sources, cited by page and
 * section: the gist.science technical summary "RDKV - KV 캐시 공동 추방 및 양자화를
 * 위한 왜곡-비트 할당" (paper 2605.08317), sections 2.1 (weights and objective),
 * 2.2 (allocation pipeline), 2.3 (TriZone packed decode); the aistudio.id article
 * "Matematika KV Cache Compression", section "Solusi 3" (asymmetric quantizer).
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Tensor arguments are DEVICE pointers into memory the caller owns; struct
 *   arguments (rdkv_dims, rdkv_layout) are HOST pointers read during the call.
 *   The library allocates nothing, keeps no global state and is reentrant.
 * - Tensors are dense row-major; fp16 tensors are passed as const void*.
 *   Every device pointer must be 16-byte aligned (else RDKV_ERR_ALIGN).
 * - A call validates its arguments on the host, then enqueues kernels on
 *   `stream` and returns without waiting.  On any error status nothing has
 *   been enqueued and no output has been touched.  Inputs must stay alive
 *   and unmodified until the enqueued work has finished.
 * - Only head_dim == 128 and n_q_heads / n_kv_heads in {1, 2, 4, 8} are
 *   supported (else RDKV_ERR_UNSUPPORTED).  n_tokens <= 2^19 and
 *   n_seq * n_layers * n_kv_heads <= 2^24, and a layout whose blob or decode
 *   workspace would pass 2^50 bytes is refused (else RDKV_ERR_SHAPE).
 * - Segment index: seg = (s * n_layers + l) * n_kv_heads + h.  Query head g
 *   belongs to KV head g / (n_q_heads / n_kv_heads).
 */
#ifndef RDKV_H
#define RDKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rdkv_status {
  RDKV_OK = 0,
  RDKV_ERR_NULL = 1,         /* a required pointer is NULL                          */
  RDKV_ERR_SHAPE = 2,        /* a size is out of range or sizes are inconsistent    */
  RDKV_ERR_UNSUPPORTED = 3,  /* head_dim != 128 or an unsupported GQA group size     */
  RDKV_ERR_BUDGET = 4,       /* a bit budget is negative                             */
  RDKV_ERR_ALIGN = 5,        /* a device pointer is not 16-byte aligned              */
  RDKV_ERR_WORKSPACE = 6,    /* a workspace or cache buffer is smaller than required */
  RDKV_ERR_CAPACITY = 7,     /* zone C has no room for the requested rows            */
  RDKV_ERR_HIP = 8,          /* a HIP runtime call failed                            */
  RDKV_ERR_OVERFLOW = 9      /* an allocation exceeded the layout's budget bounds     */
                             /* (reported by the binding from rdkv_pack_status)       */
} rdkv_status;

/* Shapes.  Q is [S][L][Hq][N][d], K and V are [S][L][Hkv][N][d]. */
typedef struct rdkv_dims {
  int64_t n_tokens;          /* N: prefill tokens per sequence, 1..524288          */
  int32_t n_seq;             /* S >= 1                                              */
  int32_t n_layers;          /* L >= 1                                              */
  int32_t n_q_heads;         /* Hq, a multiple of Hkv                               */
  int32_t n_kv_heads;        /* Hkv >= 1                                            */
  int32_t head_dim;          /* d, must be 128                                      */
  int32_t reserved;          /* must be 0                                           */
} rdkv_dims;

/* Sizes of a packed cache, all derived on the host from the dimensions and the
 * budgets (section 2.2 "sum_u b_u <= B" bounds every region), so no size ever
 * has to be read back from the device.  Filled by rdkv_layout_init; treat as
 * read-only. */
typedef struct rdkv_layout {
  rdkv_dims dims;
  int64_t budget_v;              /* B_V: bits per segment for the V-token problem   */
  int64_t budget_k;              /* B_K: bits per segment for the K-channel problem */
  int64_t n_seg;                 /* S * L * Hkv                                     */
  int64_t nk_max;                /* bound on kept tokens per segment, min(N, B_V/2) */
  uint64_t cache_bytes;          /* bytes of the packed cache blob                  */
  uint64_t slots_offset;         /* blob offset of segment 0's slot                 */
  uint64_t slot_bytes;           /* bytes per segment slot                          */
  uint64_t slot_off_v;           /* slot-relative offset of the V rows              */
  uint64_t slot_off_krec;        /* slot-relative offset of the K records           */
  uint64_t slot_off_pos;         /* slot-relative offset of the kept positions      */
  uint64_t decode_workspace_bytes; /* workspace rdkv_decode needs                   */
  int32_t zone_c_capacity;       /* rows of zone C per segment                      */
  int32_t rec_max;               /* bound on K record bytes                         */
  int32_t max_chunks;            /* split-K partial slots per segment in decode     */
  int32_t chunk_tok2;            /* decode split-K chunk: tokens of the 2-bit group */
                                 /* (4/8/16-bit groups: 1/2, 1/4, 1/8 of it)        */
  /* zone-C rollover (rdkv_layout_init_rollover; all 0 from rdkv_layout_init) */
  int32_t n_generations;         /* generation blobs reserved for rollovers         */
  int32_t token_slots;           /* chunk slots per segment of the prefill tokens    */
  int64_t gen_budget_v;          /* bits per segment per generation, V tokens       */
  int64_t gen_budget_k;          /* bits per segment per generation, K channels     */
  uint64_t gen_offset;           /* blob offset of generation blob 0                */
  uint64_t gen_bytes;            /* bytes from one generation blob to the next      */
  uint64_t zc_stats_bytes;       /* rdkv_decode_accumulate statistics buffer        */
  uint64_t rollover_workspace_bytes; /* workspace rdkv_rollover needs               */
} rdkv_layout;

/* Library version (format version in the high 16 bits, build in the low 16). */
int32_t rdkv_version(void);

/* Human-readable name of a status code (static string); any other value,
 * negative ones included, gives "unknown status".  The argument is a plain
 * int32_t so that every value a caller may hold is a valid argument. */
const char* rdkv_status_string(int32_t status);

/* Fill *out for a cache of the given dimensions and budgets.  budget_v and
 * budget_k are bits per segment (the "B" of section 2.1), >= 0; zone_c_capacity
 * >= 0 rows.  Host only; touches no device. */
rdkv_status rdkv_layout_init(const rdkv_dims* dims, int64_t budget_v, int64_t budget_k,
                             int32_t zone_c_capacity, rdkv_layout* out);

/* The same layout, plus room for the cache to grow past its zone C: when
 * zone C is full, rdkv_rollover scores its zone_c_capacity tokens, allocates
 * them with gen_budget_v / gen_budget_k bits per segment (the budgets of
 * section 2.1 for the new tokens) and packs them, like the prefill tokens,
 * into the next of n_generations generation blobs (n_generations >= 1,
 * zone_c_capacity >= 1), after which zone C is empty again.  Each generation
 * blob is a complete blob of this format for zone_c_capacity tokens per
 * segment and no zone C of its own, placed at gen_offset + g * gen_bytes in
 * the cache; decode attends over every generation in use.  Host only.
 * Errors: as rdkv_layout_init; RDKV_ERR_SHAPE for n_generations < 1 (or above
 * 4096) or zone_c_capacity < 1, RDKV_ERR_BUDGET for a negative budget. */
rdkv_status rdkv_layout_init_rollover(const rdkv_dims* dims, int64_t budget_v, int64_t budget_k,
                                      int32_t zone_c_capacity, int32_t n_generations, int64_t gen_budget_v,
                                      int64_t gen_budget_k, rdkv_layout* out);

/* ---------------------------------------------------------------- stage 1
 * Distortion weights after prefill (section 2.1, section 2.2 stage 1).
 *   w_tok[seg][t]  = sum over the G query heads g of KV head h and query rows
 *                    tau >= t of softmax_{t' <= tau}(Q[g,tau].K[t']/sqrt(d))[t]
 *                    (causal prefill attention);              fp32 [S][L][Hkv][N]
 *   var_tok[seg][t]= population variance of V[h,t,0:128];      fp32 [S][L][Hkv][N]
 *   w_chan[seg][c] = ||Q[group,:,c]||_2 * ||K[h,:,c]||_2 / sqrt(d), the query
 *                    rows of the G heads stacked;               fp32 [S][L][Hkv][128]
 * Inputs Q, K, V are fp16 as above.  `workspace` must hold
 * rdkv_score_workspace_bytes(dims) bytes (device). */
size_t rdkv_score_workspace_bytes(const rdkv_dims* dims);
rdkv_status rdkv_score(const rdkv_dims* dims, const void* Q, const void* K, const void* V,
                       float* w_tok, float* var_tok, float* w_chan,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Stage 1 in two halves, for callers that already have the row log-sum-exp of
 * their causal prefill attention (section 2.2 stage 1 runs after prefill, whose
 * attention forward computes it): rdkv_score = rdkv_score_lse, then
 * rdkv_score_from_lse, up to rounding.
 *   rdkv_score_lse: lse[s][l][hq][tau] = ln sum_{t <= tau} exp(Q[hq,tau].K[h,t]/sqrt(d)),
 *     h = hq / G, natural log, fp32 [S][L][Hq][N] (device, caller-owned); Q, K
 *     fp16 as for rdkv_score.  No workspace.
 *   rdkv_score_from_lse: w_tok, var_tok, w_chan as rdkv_score, from that lse
 *     (read only) instead of recomputing it: half of rdkv_score's matrix work.
 *     `workspace` as for rdkv_score.
 * Errors as rdkv_score (RDKV_ERR_NULL, _ALIGN for pointers not 16-byte
 * aligned, _WORKSPACE, _SHAPE / _UNSUPPORTED for dims). */
rdkv_status rdkv_score_lse(const rdkv_dims* dims, const void* Q, const void* K, float* lse, hipStream_t stream);
rdkv_status rdkv_score_from_lse(const rdkv_dims* dims, const void* Q, const void* K, const void* V,
                                const float* lse, float* w_tok, float* var_tok, float* w_chan,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- stages 2-3
 * Lagrangian bit allocation (section 2.1 objective, section 2.2 stages 2 and 3).
 * Per segment, V tokens first: unit cost c_t = fl32(w_tok*var_tok); token t gets
 * the sum of the steps j (2,2,4,8 bits) with c_t*k_j > lambda_V, k = (3/8, 3/32,
 * 15/1024, 255/524288), lambda_V the smallest value in {0} U {c_t*k_j} whose
 * total is <= budget_v.  Then var_chan[c] = fl32(exact population variance of
 * K[h,t,c] over the kept tokens b_t > 0) (0 if none), and the same rule over the
 * 128 channels with c_c = fl32(w_chan*var_chan) and budget_k.
 *   bits_tok  u8 [S][L][Hkv][N], bits_chan u8 [S][L][Hkv][128] (values 0,2,4,8,16)
 *   var_chan  fp32 [S][L][Hkv][128]; lambda fp64 [S][L][Hkv][2] (lambda_V, lambda_K)
 * K is the fp16 prefill K [S][L][Hkv][N][128].  Budgets are bits per segment.
 * workspace: device scratch of rdkv_allocate_workspace_bytes(dims, 1) bytes
 * (group for rdkv_allocate_shared), 16-byte aligned, owned by the caller (may
 * be NULL when that size is 0: problems small enough for one workgroup each);
 * its contents need no initialisation and mean nothing afterwards; two calls
 * in flight at once need two workspaces.  The allocation is exact: same inputs
 * give the same bits on every run.  Errors: RDKV_ERR_NULL, _ALIGN (any pointer
 * not 16-byte aligned), _BUDGET (a negative budget), _WORKSPACE (too small),
 * _SHAPE / _UNSUPPORTED for dims; nothing is enqueued on an error. */
size_t rdkv_allocate_workspace_bytes(const rdkv_dims* dims, int32_t group);   /* 0 for invalid dims or group */
rdkv_status rdkv_allocate(const rdkv_dims* dims, const float* w_tok, const float* var_tok,
                          const float* w_chan, const void* K, int64_t budget_v, int64_t budget_k,
                          uint8_t* bits_tok, uint8_t* bits_chan, float* var_chan, double* lambda,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The same allocation with one budget shared by each group of `group`
 * consecutive segments (section 2.1 states B as the total bit budget; segments
 * are ordered [S][L][Hkv], so group = Hkv shares a layer's budget across its
 * KV heads and group = L*Hkv a sequence's across all layers and heads).  Each
 * group's V tokens form one problem with one lambda_V and budget_v bits, then
 * its K channels (variances still per segment over that segment's kept
 * tokens) one problem with one lambda_K and budget_k bits; lambda is written
 * for every segment of the group.  rdkv_allocate is group = 1.  A segment may
 * now receive up to its group's whole budget, so a blob packed from this
 * allocation needs a layout made with the group budgets as the per-segment
 * budgets (rdkv_pack marks a segment that does not fit as empty).
 * group must be >= 1 and divide S*L*Hkv, else RDKV_ERR_SHAPE. */
rdkv_status rdkv_allocate_shared(const rdkv_dims* dims, const float* w_tok, const float* var_tok,
                                 const float* w_chan, const void* K, int64_t budget_v, int64_t budget_k,
                                 int32_t group, uint8_t* bits_tok, uint8_t* bits_chan, float* var_chan,
                                 double* lambda, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- packing
 * TriZone packing (section 2.3; quantizer of "Solusi 3").  The blob format is
 * specified in the repository's design notes; every offset inside the blob is
 * relative to its base, so a blob may be copied to another address.
 *
 * rdkv_cache_init: zero `cache` and write the header and an empty descriptor
 * for every segment (no kept tokens; zone C empty).  cache_bytes must be
 * >= layout->cache_bytes.
 *
 * rdkv_pack: quantize and pack the segments of layers [layer_begin,
 * layer_begin + n_layers) of every sequence.  K, V are fp16 [S][n_layers][Hkv]
 * [N][128]; bits_tok u8 [S][n_layers][Hkv][N]; bits_chan u8 [S][n_layers][Hkv]
 * [128].  A value other than 2, 4, 8 or 16 counts as 0 (token evicted,
 * channel dropped).  The allocation must respect the layout's budgets (per
 * segment, sum of bits_tok <= budget_v and sum of bits_chan <= budget_k); a
 * segment whose allocation does not fit its slot is written empty with bit 0
 * of its descriptor's flags word set, never past its slot; rdkv_pack_status
 * counts such segments.  Zone C of every packed segment is cleared. */
rdkv_status rdkv_cache_init(const rdkv_layout* layout, void* cache, size_t cache_bytes,
                            hipStream_t stream);
rdkv_status rdkv_pack(const rdkv_layout* layout, int32_t layer_begin, int32_t n_layers,
                      const void* K, const void* V, const uint8_t* bits_tok,
                      const uint8_t* bits_chan, void* cache, size_t cache_bytes,
                      hipStream_t stream);

/* How many segments of the cache were packed empty because their allocation
 * did not fit the layout (descriptor flag bit 0): more kept tokens than
 * nk_max, V payload or V units (sum over kept tokens of b_t / 2) above what
 * budget_v bounds, or a K record longer than rec_max -- section 2.2's
 * "sum_u b_u <= B" violated for the layout's B.  rdkv_pack cannot report this
 * itself without waiting for the device; this call enqueues one small kernel
 * that writes the count to n_dropped (device int32[1], caller-owned), which
 * the caller reads once the stream has reached it.  Errors: RDKV_ERR_NULL,
 * _ALIGN (cache), _WORKSPACE (cache_bytes below the layout's), _SHAPE (a
 * layout rdkv_layout_init did not produce). */
rdkv_status rdkv_pack_status(const rdkv_layout* layout, const void* cache, size_t cache_bytes,
                             int32_t* n_dropped, hipStream_t stream);

/* ---------------------------------------------------------------- decode
 * One decode step over every segment of the cache (section 2.3: fused
 * dequantization inside attention over zones A, B and C).
 *   q      fp16 [S][L][Hq][128]   the step's queries
 *   k_new, v_new fp16 [S][L][Hkv][128] or both NULL.  When given they are
 *          written to zone-C row c_len of every segment and attended to, so
 *          the step sees c_len + 1 zone-C rows; when NULL it sees c_len rows.
 *          The caller advances its c_len after an appending step.
 *   out    fp32 [S][L][Hq][128]   softmax(q.k_hat/sqrt(128)) v_hat over the kept
 *          tokens and zone-C rows; evicted tokens are absent; 0-bit K channels
 *          contribute 0; a segment with nothing to attend to gives 0.
 * c_len + (append ? 1 : 0) must be <= zone_c_capacity (else RDKV_ERR_CAPACITY).
 * `workspace` must hold layout->decode_workspace_bytes bytes.  The cache must
 * have been initialised and packed with the same layout. */
rdkv_status rdkv_decode(const rdkv_layout* layout, void* cache, size_t cache_bytes, int32_t c_len,
                        const void* q, const void* k_new, const void* v_new, float* out,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- zone-C rollover
 * Decode-time scoring of the new tokens, for caches made with
 * rdkv_layout_init_rollover.  Section 2.1's token weight is the attention a
 * token receives from the queries that see it; for a token of zone C these
 * are the decode steps' query heads from its own step on (the accumulated
 * attention score of the aistudio.id article's "Solusi 2").
 *
 * rdkv_decode_accumulate: rdkv_decode, plus, after the step's softmax over
 * the whole cache is known, for every segment, query head g and zone-C row
 * j < n_c (the rows this step attended):
 *   zc_stats[seg][g][j]       += exp(q_g.k_j / sqrt(d) - LSE_g)  (its attention mass)
 *   zc_stats[seg][g][cap + c] += q_g[c]^2                        (c = 0..127)
 * zc_stats is fp32 [n_seg][G][cap + 128] (layout->zc_stats_bytes, device,
 * caller-owned), all zero before the first step after rdkv_cache_init
 * (rdkv_rollover zeroes it again).  Arguments and errors otherwise as
 * rdkv_decode; RDKV_ERR_SHAPE if the layout has no generations. */
rdkv_status rdkv_decode_accumulate(const rdkv_layout* layout, void* cache, size_t cache_bytes, int32_t c_len,
                                   const void* q, const void* k_new, const void* v_new, float* out,
                                   float* zc_stats, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* rdkv_rollover_score: stage 1 (section 2.1) for the cap zone-C tokens of
 * every segment, from zc_stats:
 *   w_tok[seg][j]   = sum over g of zc_stats[seg][g][j]           fp32 [n_seg][cap]
 *   var_tok[seg][j] = population variance of zone-C V row j        fp32 [n_seg][cap]
 *   w_chan[seg][c]  = sqrt(sum_g zc_stats[seg][g][cap + c]) * ||K_C[:, c]||_2 / sqrt(d)
 *                                                                  fp32 [n_seg][128]
 * Rows never appended are zero (weight 0, variance 0).  Reads only. */
rdkv_status rdkv_rollover_score(const rdkv_layout* layout, const void* cache, size_t cache_bytes,
                                const float* zc_stats, float* w_tok, float* var_tok, float* w_chan,
                                hipStream_t stream);

/* rdkv_rollover: roll zone C into generation blob `generation`: the weights
 * of rdkv_rollover_score, the allocation of rdkv_allocate (section 2.2: V
 * tokens with gen_budget_v, then K channels over the kept ones with
 * gen_budget_k; 0 bits = evicted), the packing of rdkv_pack into that blob;
 * then zone C and zc_stats are zeroed and the blob header counts
 * generation + 1 generations in use.  Call it when zone C is full (the
 * caller's c_len == zone_c_capacity) and continue decoding with c_len = 0.
 * `generation` is the number of rollovers done so far (0, 1, ...), which the
 * caller tracks like c_len; generation >= layout->n_generations gives
 * RDKV_ERR_CAPACITY.  `workspace` must hold layout->rollover_workspace_bytes.
 * Other errors: RDKV_ERR_NULL, _ALIGN, _WORKSPACE, _SHAPE (no generations). */
rdkv_status rdkv_rollover(const rdkv_layout* layout, void* cache, size_t cache_bytes, int32_t generation,
                          float* zc_stats, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* rdkv_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): no
 * workspace argument; the split-K partials go to a library-owned device array
 * of RDKV_STATIC_SCRATCH_BYTES bytes per GPU, part of the library's code
 * object and held by every GPU the library runs on until the process ends.
 * Results are those of rdkv_decode, bit for bit (same kernels).  Allocates
 * nothing: the first call on a device only looks up that device's array
 * address.  Every call on one GPU uses the same array, so calls that overlap
 * on one GPU (other streams, or other host threads without ordering) race;
 * nothing in the array needs to start at zero.  Errors: as rdkv_decode, and
 * RDKV_ERR_WORKSPACE when layout->decode_workspace_bytes exceeds
 * RDKV_STATIC_SCRATCH_BYTES. */
#define RDKV_STATIC_SCRATCH_BYTES (64u << 20)
rdkv_status rdkv_decode_static(const rdkv_layout* layout, void* cache, size_t cache_bytes, int32_t c_len,
                               const void* q, const void* k_new, const void* v_new, float* out,
                               hipStream_t stream);

/* The two split-K phases of rdkv_decode, for callers that time them, or that
 * exchange the per-chunk partials between devices before merging.
 *
 * rdkv_decode_partials: the append and the per-chunk partial softmax state
 * (running max m, sum l, unnormalised o[128] per query head and chunk) into
 * `workspace`; arguments as rdkv_decode.
 * rdkv_decode_merge: out = sum_k e^{m_k-M} o_k / sum_k e^{m_k-M} l_k over each
 * segment's chunks, in a fixed order.  The partials phase writes every chunk
 * slot of the workspace (slots past a segment's last chunk are marked empty),
 * so the merge needs nothing else from the blob.  zone_c_rows is the number of
 * zone-C rows the partials phase attended (its c_len, plus 1 if it appended);
 * it is checked, 0 <= zone_c_rows <= zone_c_capacity, else RDKV_ERR_CAPACITY. */
rdkv_status rdkv_decode_partials(const rdkv_layout* layout, void* cache, size_t cache_bytes, int32_t c_len,
                                 const void* q, const void* k_new, const void* v_new,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);
rdkv_status rdkv_decode_merge(const rdkv_layout* layout, const void* cache, size_t cache_bytes,
                              int32_t zone_c_rows, float* out, const void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* ---------------------------------------------------------------- paged zones
 * A paged cache for batched serving: the packed zones of every segment live
 * in fixed-size pages of one shared pool, found through a block table per
 * segment (the aistudio.id article's "Solusi 1": KV blocks, non-contiguous,
 * mapped per sequence), so sequences of different lengths take exactly the
 * pages they need, and the pages of a finished sequence go to the next one.
 * The caller owns the pages (its own allocator hands them out and takes them
 * back, as a serving block manager does); the library writes and reads them.
 *
 * Layout of the buffer: 256-byte header; a 256-byte descriptor per segment
 * slot (sequence slot s < n_seq, layer, KV head: seg = (s*L + l)*Hkv + h);
 * the block table int32 [n_seg][max_pages] (physical page of each virtual
 * page of a segment, -1 unused); the pool of n_pages pages of
 * RDKV_PAGE_BYTES.  A segment's regions -- V rows of its 2/4/8/16-bit token
 * groups, their K records, zone-C keys, zone-C values, kept positions -- are
 * each an array of 64-row tiles laid page after page (a tile never straddles
 * a page), starting at a fresh virtual page; the tiles' content is that of
 * the contiguous format.  A free slot has zone-C capacity 0. */
#define RDKV_PAGE_BYTES 32768
#define RDKV_MAX_PAGED_SEQS 256
typedef struct rdkv_paged_layout {
  rdkv_dims dims;                /* n_seq = sequence slots (<= 256), n_tokens = bound on a prefill length */
  int64_t budget_v_max;          /* bound on a sequence's V budget (bits per segment) */
  int64_t budget_k_max;          /* bound on a sequence's K budget                   */
  int64_t n_seg;                 /* n_seq * n_layers * n_kv_heads                    */
  int64_t n_pages;               /* pages in the pool                                */
  int64_t max_pages;             /* block-table entries per segment                  */
  int64_t nk_max;                /* bound on kept tokens per segment                 */
  uint64_t table_offset;         /* byte offset of the block table                   */
  uint64_t pool_offset;          /* byte offset of page 0                            */
  uint64_t cache_bytes;          /* bytes of the whole paged cache                   */
  uint64_t decode_workspace_bytes;
  int32_t zone_c_capacity;       /* zone-C rows of every sequence                     */
  int32_t rec_max, max_chunks, token_slots, chunk_tok2, reserved;
} rdkv_paged_layout;

/* Host only.  dims_max: sequence slots, layers, heads, and the bound on any
 * sequence's prefill length; budget bounds per segment; zone-C capacity;
 * n_pages >= 1.  Errors as rdkv_layout_init, RDKV_ERR_SHAPE for n_seq >
 * RDKV_MAX_PAGED_SEQS, n_pages < 1 or a cache of 1 TiB (2^40 bytes) or more. */
rdkv_status rdkv_paged_layout_init(const rdkv_dims* dims_max, int64_t budget_v_max, int64_t budget_k_max,
                                   int32_t zone_c_capacity, int64_t n_pages, rdkv_paged_layout* out);
/* Zero the buffer, write the header, every slot free, the table -1. */
rdkv_status rdkv_paged_cache_init(const rdkv_paged_layout* layout, void* cache, size_t cache_bytes,
                                  hipStream_t stream);
/* Adding a sequence, in two calls around the caller's page allocation:
 * rdkv_paged_stage packs one sequence -- its own prefill length n_tokens <=
 * the bound, its own budgets within the bounds -- with rdkv_pack into a
 * caller-provided staging buffer of rdkv_paged_staging_bytes bytes, and
 * writes to pages_needed (device int32 [L*Hkv]) how many pages each of its
 * segments takes (zone C included).  K, V fp16 [L][Hkv][n_tokens][128],
 * bits_tok u8 [L][Hkv][n_tokens], bits_chan u8 [L][Hkv][128], as for
 * rdkv_pack (an allocation over its budgets packs empty, see
 * rdkv_pack_status).  The caller then reads pages_needed, takes that many
 * pages from its pool and calls rdkv_paged_commit with them: pages is device
 * int32 [L*Hkv][max_pages], row i listing segment i's pages in order (row
 * entries past its count are ignored); entries outside [0, n_pages) make
 * that segment empty (descriptor flag bit 0).  The sequence lands in slot
 * `seq`, its zone C empty.  staging must still hold what rdkv_paged_stage
 * wrote.  rdkv_paged_release frees slot `seq` (descriptors empty, table -1);
 * the caller takes back the pages it gave. */
size_t rdkv_paged_staging_bytes(const rdkv_paged_layout* layout, int64_t n_tokens, int64_t budget_v,
                                int64_t budget_k);
rdkv_status rdkv_paged_stage(const rdkv_paged_layout* layout, int64_t n_tokens, int64_t budget_v,
                             int64_t budget_k, const void* K, const void* V, const uint8_t* bits_tok,
                             const uint8_t* bits_chan, void* staging, size_t staging_bytes,
                             int32_t* pages_needed, hipStream_t stream);
rdkv_status rdkv_paged_commit(const rdkv_paged_layout* layout, int32_t seq, int64_t n_tokens, int64_t budget_v,
                              int64_t budget_k, const void* staging, size_t staging_bytes, const int32_t* pages,
                              void* cache, size_t cache_bytes, hipStream_t stream);
rdkv_status rdkv_paged_release(const rdkv_paged_layout* layout, int32_t seq, void* cache, size_t cache_bytes,
                               hipStream_t stream);
/* One decode step over every sequence slot (section 2.3 decode, as
 * rdkv_decode): c_len is a HOST array [n_seq] of each slot's zone-C rows
 * before the step (0 for free slots); with k_new/v_new every slot in use
 * appends its token at its own row c_len[s] (so c_len[s] < capacity) and
 * attends c_len[s] + 1 rows; the caller then advances its c_len.  q, k_new,
 * v_new, out as rdkv_decode over [n_seq][L]...; free slots give 0.
 * workspace: layout->decode_workspace_bytes.  Errors: RDKV_ERR_CAPACITY for a
 * c_len out of range, others as rdkv_decode. */
rdkv_status rdkv_paged_decode(const rdkv_paged_layout* layout, void* cache, size_t cache_bytes,
                              const int32_t* c_len, const void* q, const void* k_new, const void* v_new,
                              float* out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Decode launch shape of the segments in use.  rdkv_paged_decode (and
 * rdkv_decode) size their launch from the layout's bounds: chunk slots per
 * segment for the largest V budget a segment may hold, and an LDS record ring
 * for the longest K record it may have.  With one budget shared by a layer's
 * heads (rdkv_allocate_shared) those bounds are those of the whole layer's
 * budget, several times what the segments actually hold, and the launch pays
 * for empty slots and a larger ring.  rdkv_paged_decode_shape (rdkv_decode_shape
 * for a contiguous cache: its prefill blob's segments) measures the segments
 * in use instead: it reads every segment's descriptor on `stream` and WAITS
 * for the result (a synchronous call, like reading pages_needed after
 * rdkv_paged_stage); `workspace` is any device buffer of >= 8 bytes, e.g. the
 * decode workspace.  rdkv_paged_decode_shaped (rdkv_decode_shaped) is
 * rdkv_paged_decode (rdkv_decode) launched with that shape; its workspace
 * needs shape->decode_workspace_bytes (<= the layout's).  A shape covers the
 * segments as they were when it was made: make a new one after a commit or a
 * pack (a release leaves it valid).  A segment in use that the shape does not
 * cover (more chunks or longer records than it allows) is not decoded and
 * takes no appended token: its outputs are set to NaN.  The shaped calls read
 * token_slots, rec_max and reserved from the shape; max_chunks and
 * decode_workspace_bytes are what they derive from them, for the caller.
 * Errors: RDKV_ERR_SHAPE for a shape outside the layout's bounds (or a
 * nonzero reserved field), others as the unshaped call. */
typedef struct rdkv_launch_shape {
  int32_t token_slots;              /* prefill-token chunk slots per segment (<= layout->token_slots) */
  int32_t rec_max;                  /* bytes of the longest K record, a multiple of 4 (<= layout->rec_max) */
  int32_t max_chunks;               /* token_slots + the other chunk slots (generations, zone C) */
  int32_t reserved;                 /* 0 */
  uint64_t decode_workspace_bytes;  /* split-K partials of a launch of this shape */
} rdkv_launch_shape;
rdkv_status rdkv_paged_decode_shape(const rdkv_paged_layout* layout, const void* cache, size_t cache_bytes,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream,
                                    rdkv_launch_shape* out);
rdkv_status rdkv_paged_decode_shaped(const rdkv_paged_layout* layout, const rdkv_launch_shape* shape, void* cache,
                                     size_t cache_bytes, const int32_t* c_len, const void* q, const void* k_new,
                                     const void* v_new, float* out, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);
rdkv_status rdkv_decode_shape(const rdkv_layout* layout, const void* cache, size_t cache_bytes, void* workspace,
                              size_t workspace_bytes, hipStream_t stream, rdkv_launch_shape* out);
rdkv_status rdkv_decode_shaped(const rdkv_layout* layout, const rdkv_launch_shape* shape, void* cache,
                               size_t cache_bytes, int32_t c_len, const void* q, const void* k_new, const void* v_new,
                               float* out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Test support: dequantized kept rows of one segment, in kept order, with the
 * fused multiply-add dequantization x_hat = fmaf(code, scale, zero).
 *   k_hat, v_hat fp32 [nk_max][128] (rows past the segment's kept count are
 *   not written); K channels with 0 bits are written as 0, in original channel
 *   order. */
rdkv_status rdkv_unpack(const rdkv_layout* layout, const void* cache, size_t cache_bytes,
                        int64_t seg, float* k_hat, float* v_hat, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RDKV_H */
