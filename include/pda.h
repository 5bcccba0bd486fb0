/*
 * pda.h — C ABI of libpda.so: FP8 (OCP e4m3) paged decode attention for
 * AMD Instinct MI355X (gfx950).
 *
 * Sources for what the calls compute (four web pages about Cloudflare's
 * Workers AI serving of Kimi K2.6 and GLM 5.2):
 *   [SK]  aifeed.sk, "Cloudflare zrýchľuje inferenciu modelov Kimi a GLM
 *         kompresiou cache a váh"
 *   [VN]  manulx.blog, "Công thức của Cloudflare để phục vụ Kimi và GLM:
 *         lượng tử hóa bộ nhớ đệm KV, nén trọng số, xác minh bộ nhớ đệm"
 *   [DE]  remio.ai, "Cloudflare: Kleinere Modellbereitstellung senkt
 *         Speicherbedarf, doch Sicherheit wird zum Prüfstein"
 *   [JA]  agentlenshq.com, "Cloudflare Workers AI: Kimi および GLM の推論を
 *         大規模に最適化する"
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All array pointers are DEVICE pointers owned by the caller. The library
 *    never allocates, retains or frees memory.
 *  - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *    NULL = the default stream). Nothing synchronises the device.
 *  - Return value: PDA_OK, or a PDA_ERR_* code from host-side argument checks
 *    made before anything is enqueued, or PDA_ERR_LAUNCH when the HIP runtime
 *    refuses a launch. Faults in device DATA (stale page tags, bad block ids,
 *    malformed sequence lengths) are never return codes: validate_page_tags
 *    reports them per sequence, and paged_decode_attn writes NaN rows for
 *    sequences it cannot read safely (see below).
 *  - Re-entrant; no global mutable state beyond a per-device cache of the
 *    compute-unit count.
 *  - Intended order on one stream per decode step:
 *        kv_write_fp8 -> validate_page_tags -> paged_decode_attn,
 *    or kv_write_check (the first two in one launch) -> paged_decode_attn.
 *
 * Physical KV-cache format ("page" = `page_size` consecutive token slots of
 * one sequence; slot = page * page_size + offset). Element size is 1 byte for
 * FP8 caches and 2 bytes for BF16 caches; indices below are in elements.
 *
 *  K cache, logical shape [num_pages][Hkv][Dk/16][S][16]:
 *    element (page p, kv head h, offset o, dim d) is at
 *      (((p*Hkv + h)*(Dk/16) + d/16)*S + o)*16 + d%16
 *    i.e. each (page, head) block holds 16-dim column groups, token-major
 *    inside a group, so one token's 16 dims are 16 contiguous elements.
 *    Requires Dk % 16 == 0.
 *
 *  V cache, logical shape [num_pages][Hkv][S/2][Dv/8][8][2]:
 *    element (p, h, o, d) is at
 *      ((((p*Hkv + h)*(S/2) + o/2)*(Dv/8) + d/8)*8 + d%8)*2 + o%2
 *    i.e. the two tokens of an even/odd slot pair sit next to each other for
 *    every dim. Requires S even and Dv % 8 == 0.
 *
 *  Latent caches (v_in_k = 1) have no V cache: the value vector of a token is
 *  the first Dv dims of its K entry.
 *
 *  FP8 element = OCP FP8 E4M3 ("E4M3FN": bias 7, no infinities, NaN =
 *  S.1111.111, largest finite magnitude 448). Stored value = code * scale.
 *  Scales: PER_HEAD keeps one fp32 scale per kv head for K and one for V;
 *  PER_TOKEN keeps one fp32 scale per slot, shared by K and V of that token,
 *  in token_scale[num_pages * page_size].
 */
#ifndef PDA_H
#define PDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum pda_status {
  PDA_OK = 0,
  PDA_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, bad ratio   */
  PDA_ERR_UNSUPPORTED = 2, /* valid but not built: (dtype, dims, page size) */
  PDA_ERR_LAUNCH = 3,      /* the HIP runtime rejected a kernel launch      */
  PDA_ERR_WORKSPACE = 4,   /* workspace smaller than the minimum           */
  PDA_ERR_POOL_EXHAUSTED = 5, /* fewer free pages than an allocation asks for */
  PDA_ERR_SCRATCH = 6      /* shape needs more than the fixed scratch of
                              paged_decode_attn_noalloc                     */
};

enum pda_kv_dtype { PDA_KV_BF16 = 0, PDA_KV_FP8_E4M3 = 1 };

enum pda_scale_mode {
  PDA_SCALE_NONE = 0,      /* BF16 caches                                   */
  PDA_SCALE_PER_HEAD = 1,  /* k_scale[Hkv], v_scale[Hkv]                    */
  PDA_SCALE_PER_TOKEN = 2  /* token_scale[num_pages*page_size], K and V     */
};

/* Shape of one paged_decode_attn call. */
typedef struct pda_attn_shape {
  int32_t num_seqs;           /* B                                          */
  int32_t num_q_heads;        /* Hq; query head h reads kv head h/(Hq/Hkv)  */
  int32_t num_kv_heads;       /* Hkv; Hq % Hkv == 0                         */
  int32_t head_dim_qk;        /* Dk                                         */
  int32_t head_dim_v;         /* Dv                                         */
  int32_t page_size;          /* S                                          */
  int32_t num_pages;          /* P, physical pages in the pool              */
  int32_t max_blocks_per_seq; /* row length of block_table                  */
  int32_t kv_dtype;           /* enum pda_kv_dtype                          */
  int32_t scale_mode;         /* enum pda_scale_mode                        */
  int32_t v_in_k;             /* 1: V = first Dv dims of each K entry       */
  int32_t split_tokens;       /* split-K chunk in tokens; 0 = automatic     */
  float sm_scale;             /* softmax scale, usually 1/sqrt(Dk)          */
} pda_attn_shape;

/*
 * kv_write_fp8 — quantise new K/V rows to FP8 e4m3 and scatter them into
 * their cache slots. The pages state that keys and values are kept as 8-bit
 * e4m3 instead of 16-bit BF16, halving the cache ([SK] § "Dve odlišné úzke
 * miesta v pamäti GPU"; [VN] § "Bộ nhớ đệm KV FP8 tăng gấp đôi dung lượng
 * ngữ cảnh"; [JA] § "並行性を高めるための KV キャッシュ量子化").
 *
 *  k_new        bf16 [num_tokens][Hkv][Dk], row-major.
 *  v_new        bf16 [num_tokens][Hkv][Dv]; NULL iff the cache is latent
 *               (v_in_k: then v_cache must be NULL too and Dv is ignored).
 *  slot_mapping int64 [num_tokens]: slot = page*page_size + offset. Tokens
 *               with slot < 0 or slot >= num_pages*page_size write nothing.
 *               Duplicate slots in one call are undefined.
 *  scale_mode   PER_HEAD: k_scale[Hkv], v_scale[Hkv] are fp32 inputs and
 *               token_scale must be NULL.
 *               PER_TOKEN (latent caches only: Hkv == 1, v_new == NULL):
 *               the call computes sc = amax/448 (fp32 division; amax = max
 *               |x| over the token's Dk values, NaN values (quiet or
 *               signaling) ignored; 1.0 when amax == 0) and writes
 *               it to token_scale[slot]; k_scale/v_scale must be NULL.
 *  Per element: code = e4m3(fp32(x) / scale), the division correctly rounded
 *               in fp32, then round-to-nearest-even with saturation to ±448
 *               (±inf -> ±448), sign of zero kept, NaN -> 0x7F|sign.
 *  k_cache, v_cache  FP8 caches in the format above. Bytes of slots not
 *               addressed by this call are left unchanged.
 */
int kv_write_fp8(const void* k_new, const void* v_new,
                 const int64_t* slot_mapping, int32_t num_tokens,
                 int32_t num_kv_heads, int32_t head_dim_k, int32_t head_dim_v,
                 int32_t page_size, int32_t num_pages, int32_t scale_mode,
                 const float* k_scale, const float* v_scale,
                 float* token_scale,
                 uint8_t* k_cache, uint8_t* v_cache, void* stream);

/*
 * kv_write_bf16 — the BF16-cache variant of kv_write_fp8: same arguments
 * minus scales, and the stored element is the BF16 input, bit for bit. It is
 * the comparison path the pages measure FP8 against ([DE] § "Warum kleinere
 * Cloudflare-Caches reine Geschwindigkeit schlagen").
 */
int kv_write_bf16(const void* k_new, const void* v_new,
                  const int64_t* slot_mapping, int32_t num_tokens,
                  int32_t num_kv_heads, int32_t head_dim_k, int32_t head_dim_v,
                  int32_t page_size, int32_t num_pages,
                  void* k_cache, void* v_cache, void* stream);

/*
 * kv_write_check — the kv write and the page-tag check of one decode step in
 * a single launch: exactly the effect of kv_write_fp8 (kv_dtype
 * PDA_KV_FP8_E4M3) or kv_write_bf16 (PDA_KV_BF16, scale_mode PDA_SCALE_NONE,
 * all scale pointers NULL) followed by validate_page_tags on the same
 * stream, with the arguments of both (num_pages and page_size serve both).
 * The check stays a batch step of its own, outside attention, as the pages
 * describe it ([SK] § "Kvalita odpovedí a integrita spoločnej cache"; [DE]
 * § "Sicherheit gemeinsamer KV-Caches wird zum Produktionsthema"); it only
 * shares the launch with the write, which it does not depend on: the write
 * changes cache bytes, the check reads tags, the block table and lengths.
 * Workgroups [0, num_tokens) write one token each and workgroups
 * [num_tokens, num_tokens + num_seqs) check one sequence each, so the
 * launch costs one kernel start instead of two.
 *
 *  Write arguments as kv_write_fp8 / kv_write_bf16 (k_cache and v_cache
 *  point at uint8 codes or uint16 BF16 elements); check arguments as
 *  validate_page_tags. num_tokens == 0 runs the check alone and reads
 *  none of the write's arguments (empty inputs may be NULL); num_seqs == 0
 *  runs the write alone and reads none of the check's pointers; both zero
 *  is a no-op.
 *  The caches must not overlap page_tags, block_table, expected_tags,
 *  seq_lens or verdict.
 *  Errors: those of the two calls it replaces; PDA_ERR_INVALID_ARG for an
 *  unknown kv_dtype; PDA_ERR_UNSUPPORTED when num_tokens + num_seqs exceeds
 *  2^31 - 1.
 */
int kv_write_check(const void* k_new, const void* v_new,
                   const int64_t* slot_mapping, int32_t num_tokens,
                   int32_t num_kv_heads, int32_t head_dim_k, int32_t head_dim_v,
                   int32_t page_size, int32_t num_pages, int32_t kv_dtype,
                   int32_t scale_mode, const float* k_scale,
                   const float* v_scale, float* token_scale, void* k_cache,
                   void* v_cache, const uint32_t* page_tags,
                   const int32_t* block_table, const uint32_t* expected_tags,
                   int32_t max_blocks_per_seq, const int32_t* seq_lens,
                   int32_t num_seqs, int32_t* verdict, void* stream);

/*
 * kv_transcode_bf16_to_fp8 — re-encode pages of a BF16 cache as pages of an
 * FP8 e4m3 cache. The pages describe separate GPU pools for prefill and
 * decode, the prefill pool keeping its cache in BF16 and the decode pool in
 * FP8 ([SK] § "Kompresia sa oplatí inde pri vstupe a inde pri výstupe"; [VN]
 * § "Bộ nhớ đệm KV FP8 tăng gấp đôi dung lượng ngữ cảnh"; [DE] § "Was
 * Cloudflare für Kimi und GLM geändert hat"; [JA] § "並行性を高めるための KV
 * キャッシュ量子化"), so a request's pages change format when it moves from
 * the first pool to the second. They do not say how; the reading taken
 * here is that every token is quantised exactly as kv_write_fp8 would have
 * quantised the same BF16 rows in the decode pool.
 *
 *  k_src, v_src BF16 caches (uint16 elements) in the format above, with
 *               src_num_pages pages; v_src NULL iff the caches are latent
 *               (then v_dst must be NULL too and Dv is ignored).
 *  src_pages, dst_pages, valid  int32 [num_pairs] device arrays: pair i
 *               re-encodes slots [0, valid[i]) of BF16 page src_pages[i]
 *               into the same slots of FP8 page dst_pages[i]. A pair whose
 *               page ids fall outside [0, src_num_pages) / [0, dst_num_pages)
 *               or whose valid lies outside [0, page_size] writes nothing.
 *               Two pairs with the same destination page are undefined.
 *  scale_mode   PER_HEAD: k_scale[Hkv], v_scale[Hkv] fp32 inputs, token_scale
 *               NULL. PER_TOKEN (latent, Hkv == 1): the per-token scale of
 *               every re-encoded slot is computed as kv_write_fp8 computes it
 *               and written to token_scale[dst_page*page_size + slot].
 *  k_dst, v_dst FP8 caches with dst_num_pages pages. Slots at or past
 *               valid[i], and pages no pair names, are left unchanged.
 *  Errors as kv_write_fp8: PDA_ERR_UNSUPPORTED unless Dk % 16 == 0, the
 *  page size is even and Dv % 8 == 0 (non-latent); PER_TOKEN also needs a
 *  page size dividing 256. Caches must be 16-byte aligned (v_dst 8).
 */
int kv_transcode_bf16_to_fp8(const void* k_src, const void* v_src,
                             const int32_t* src_pages, const int32_t* dst_pages,
                             const int32_t* valid, int32_t num_pairs,
                             int32_t num_kv_heads, int32_t head_dim_k,
                             int32_t head_dim_v, int32_t page_size,
                             int32_t src_num_pages, int32_t dst_num_pages,
                             int32_t scale_mode, const float* k_scale,
                             const float* v_scale, float* token_scale,
                             uint8_t* k_dst, uint8_t* v_dst, void* stream);

/*
 * validate_page_tags — the separate batched check of cache-page tags that
 * runs before decode attention reads the cache. Every physical page carries
 * a tag that changes whenever the page is handed out again; each request
 * keeps the pages and tags it expects; a mismatch aborts the request instead
 * of letting it read another request's data ([SK] § "Kvalita odpovedí a
 * integrita spoločnej cache"; [VN] § "Bảo vệ bộ nhớ đệm dùng chung"; [DE]
 * § "Sicherheit gemeinsamer KV-Caches wird zum Produktionsthema"; [JA]
 * § "KV キャッシュ整合性チェック").
 *
 *  page_tags     uint32 [num_pages]: current tag of each physical page.
 *  block_table   int32  [num_seqs][max_blocks_per_seq]: physical page of
 *                logical block j of sequence s.
 *  expected_tags uint32 [num_seqs][max_blocks_per_seq]: the tag sequence s
 *                recorded for block j when it was given that page.
 *  seq_lens      int32  [num_seqs].
 *  verdict       int32  [num_seqs], written:
 *                   0     every block j < ceil(len/page_size) has
 *                         0 <= block_table[s][j] < num_pages and
 *                         page_tags[block_table[s][j]] == expected_tags[s][j];
 *                   j+1   j is the first block that fails that test;
 *                  -1     len < 0 or len > max_blocks_per_seq*page_size.
 *                Entries beyond ceil(len/page_size) are never read.
 *  A passing verdict covers page identity and generation only, never the
 *  contents of the page.
 */
int validate_page_tags(const uint32_t* page_tags, int32_t num_pages,
                       const int32_t* block_table,
                       const uint32_t* expected_tags,
                       int32_t max_blocks_per_seq, const int32_t* seq_lens,
                       int32_t num_seqs, int32_t page_size, int32_t* verdict,
                       void* stream);

/*
 * paged_decode_attn_workspace_bytes — device scratch needed by
 * paged_decode_attn for `shape` when no sequence is longer than
 * max_seq_len tokens. Vector-ALU path: a header plus one split-K partial
 * (G rows of Dv fp32 accumulators, a running max and a running sum per row)
 * per (sequence, unit of up to four consecutive chunks, kv head), i.e. the
 * chunk count of a sequence divided by four and rounded up; a smaller
 * workspace down to one partial per (sequence, kv head) is still accepted,
 * and the device then widens the split chunk (by doubling) until the
 * partials fit, which changes results only within rounding. Latent path:
 * a header plus one partial (Hq rows of Dv + 4 fp32) per (compute unit +
 * sequence) of the current device; with less room
 * fewer workgroups are launched (at least one partial per sequence plus one
 * is required). Returns 0 for an invalid shape and for a valid one that
 * neither kernel supports (paged_decode_attn returns PDA_ERR_UNSUPPORTED
 * for it).
 */
size_t paged_decode_attn_workspace_bytes(const pda_attn_shape* shape,
                                         int32_t max_seq_len);

/*
 * paged_decode_attn — single-query-per-sequence attention over a paged KV
 * cache reached through a block table, converting FP8 codes to values as it
 * reads them ([SK] § "Dve odlišné úzke miesta v pamäti GPU"; [VN] § "Bộ nhớ
 * đệm KV FP8 tăng gấp đôi dung lượng ngữ cảnh"). For every sequence s and
 * query head h (kv head g = h / (Hq/Hkv)):
 *     z_t   = sm_scale * sum_d q[s][h][d] * K̂[t][d]      for t < len_s
 *     out   = sum_t softmax(z)_t * V̂[t]                   (fp32 result)
 * with K̂ = code*k_scale[g] (PER_HEAD) or code*token_scale[slot] (PER_TOKEN),
 * V̂ likewise with v_scale[g] (or the token scale), and BF16 values as
 * stored. Long contexts are split into page-aligned chunks whose partial
 * results are merged by a log-sum-exp combine step.
 *
 *  q            bf16 [num_seqs][Hq][Dk].
 *  k_cache, v_cache  caches in the format above (v_cache NULL if v_in_k).
 *  k_scale, v_scale  PER_HEAD: fp32 [Hkv] each. PER_TOKEN: k_scale is the
 *               token_scale array [num_pages*page_size], v_scale NULL.
 *               NONE (BF16): both NULL.
 *  block_table  int32 [num_seqs][max_blocks_per_seq].
 *  seq_lens     int32 [num_seqs]; token t of s lives in slot
 *               block_table[s][t/S]*S + t%S. Tokens >= len are never read.
 *  max_seq_len  host-side upper bound of seq_lens, used to size the launch.
 *  verdict      int32 [num_seqs] from validate_page_tags, or NULL for the
 *               no-op tracker (no check, no extra work). A sequence with
 *               verdict != 0 is aborted: none of its KV bytes are read and
 *               its output rows are written as zeros.
 *  workspace    device scratch of workspace_bytes (see above); its contents
 *               need no initialisation and are clobbered.
 *  out          fp32 [num_seqs][Hq][Dv]. Rows of sequences with len == 0
 *               are zero. Rows of a sequence that is not aborted but whose
 *               len is negative or exceeds max_blocks_per_seq*page_size, or
 *               whose block table holds a page id outside [0, num_pages) in
 *               its first ceil(len/S) entries, are NaN (no out-of-range
 *               address is ever formed).
 *  Supported: FP8 or BF16, PER_HEAD/NONE, Dk == Dv == 128, Hq/Hkv in
 *  {1,2,4,8}, S in {16, 32, 64}, num_seqs <= 16384 (vector-ALU kernel);
 *  and latent FP8 PER_TOKEN, Hkv == 1, Dk == 576, Dv == 512, v_in_k,
 *  S == 64, Hq in {32, 64, 96, 128}, num_seqs <= 2048 (matrix-core kernel;
 *  split_tokens is ignored there: the valid pages of all sequences are cut
 *  into one equal range per compute unit, and the workspace holds one
 *  partial per (range, sequence) pair that meets).
 */
int paged_decode_attn(const pda_attn_shape* shape, const void* q,
                      const void* k_cache, const void* v_cache,
                      const float* k_scale, const float* v_scale,
                      const int32_t* block_table, const int32_t* seq_lens,
                      int32_t max_seq_len, const int32_t* verdict,
                      void* workspace, size_t workspace_bytes, float* out,
                      void* stream);

/*
 * paged_decode_attn_noalloc — paged_decode_attn for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments minus the workspace,
 * the same kernels and results, with the partials in a fixed scratch array
 * that the library keeps in device memory (one copy per device, 96 MiB,
 * see paged_decode_attn_noalloc_scratch_bytes, held until the process ends).
 * The call itself allocates and frees nothing; its first call on a device
 * looks up that device's copy.
 *  - Every call on one device shares that device's scratch, and each call
 *    overwrites it (nothing in it needs to start at zero): calls that may
 *    overlap on one device (several streams, several host threads) race and
 *    must be serialised by the caller.
 *  - PDA_ERR_SCRATCH if the shape cannot run in the scratch even at its
 *    smallest workspace (vector-ALU path: a header of 4*(num_seqs + 65)
 *    bytes rounded up to 256 plus num_seqs * Hkv * G*(Dv+2)*4 bytes; latent
 *    path: num_seqs + 1 partials of Hq*516*4 bytes plus its header). Shapes
 *    whose full workspace is larger than the scratch run with the split
 *    chunk widened (vector-ALU) or fewer workgroups (latent), as
 *    paged_decode_attn does with a small workspace.
 *  Other arguments, results and errors: as paged_decode_attn.
 */
int paged_decode_attn_noalloc(const pda_attn_shape* shape, const void* q,
                              const void* k_cache, const void* v_cache,
                              const float* k_scale, const float* v_scale,
                              const int32_t* block_table, const int32_t* seq_lens,
                              int32_t max_seq_len, const int32_t* verdict,
                              float* out, void* stream);

/* Bytes of the fixed scratch paged_decode_attn_noalloc runs in. */
size_t paged_decode_attn_noalloc_scratch_bytes(void);

/* Human-readable name of a status code (static storage). */
const char* pda_status_string(int status);

/*
 * Host page pool and tag tracker — the host side of the tag check. The
 * pages say every physical page carries a tag that changes when the page is
 * handed out again, that each request records the pages and tags it
 * expects, and that a no-op tracker costs nothing when the check is off
 * ([VN] § "Bảo vệ bộ nhớ đệm dùng chung"; [DE] § "Sicherheit gemeinsamer
 * KV-Caches wird zum Produktionsthema"; [JA] § "KV キャッシュ整合性チェック").
 * Host memory only; no GPU call is made. A pool is not thread-safe: calls
 * on one pool must not overlap.
 *
 * pda_pool_create  num_pages > 0 pages, all free. initial_order: NULL hands
 *                  pages out as 0, 1, 2, ...; else a permutation of
 *                  [0, num_pages) giving the order of the first hand-outs
 *                  (rejected if it is not one). tag_start: the counter's
 *                  start value. track_tags == 0 makes the no-op tracker: no
 *                  tag is ever stamped (tags stay 0) and the caller passes
 *                  verdict NULL to paged_decode_attn. *out receives the pool.
 * pda_pool_alloc   hands out n pages, the most recently freed first
 *                  (free pages form a stack); with tracking each hand-out
 *                  stamps the page with ++counter (32-bit, wrapping), so a
 *                  page handed out again carries a new tag. pages[n] and
 *                  tags[n] receive the page ids and their new tags (tags may
 *                  be NULL). PDA_ERR_POOL_EXHAUSTED, with nothing handed
 *                  out, if fewer than n pages are free.
 * pda_pool_free    returns n pages, pushed in array order (so the last one
 *                  is handed out first). PDA_ERR_INVALID_ARG, with nothing
 *                  freed, if an id is out of range, not in use, or repeated.
 * pda_pool_tags    the current tag of every page, [num_pages] uint32 (valid
 *                  until the next call on the pool); the array to upload as
 *                  validate_page_tags' page_tags.
 * pda_pool_num_free  free page count (-1 for a NULL pool).
 */
typedef struct pda_page_pool pda_page_pool;
int pda_pool_create(int32_t num_pages, const int32_t* initial_order, uint32_t tag_start,
                    int32_t track_tags, pda_page_pool** out);
void pda_pool_destroy(pda_page_pool* pool);
int pda_pool_alloc(pda_page_pool* pool, int32_t n, int32_t* pages, uint32_t* tags);
int pda_pool_free(pda_page_pool* pool, const int32_t* pages, int32_t n);
const uint32_t* pda_pool_tags(const pda_page_pool* pool);
int32_t pda_pool_num_free(const pda_page_pool* pool);

#ifdef __cplusplus
}
#endif

#endif /* PDA_H */
