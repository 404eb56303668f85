/*
 * prkv.h -- pre-RoPE KV injection with Chunked RoPE into a paged KV cache.
 *
 * C ABI of libprkv.so (gfx950 / MI355X).  The operation is the serving-time
 * step of "InferScale: GPU-Native KV Injection for Personalized LLM Serving"
 * (Pith review of arXiv 2607.27090): facts' keys and values are precomputed
 * once and kept GPU-resident with keys BEFORE rotary position encoding; at
 * serving time the top-k retrieved facts are resolved to their KV by fact_id,
 * the keys are rotated to the facts' serving-time positions (Chunked RoPE),
 * and K and V are scatter-copied into the engine's paged KV cache so that
 * only the query needs prefill ("The pith"; "Referee Report", Summary;
 * Figure 2 caption; "Axiom & Free-Parameter Ledger", KV-connector axiom,
 * section 3.4).
 *
 * Conventions
 *  - bf16 values are passed as raw 16-bit patterns (uint16_t storage).
 *  - Every call returns PRKV_OK (0) or a negative PRKV_ERR_* code; the text
 *    of the last error on the calling thread is last_error_string().
 *  - Validation is complete before anything is enqueued: on error nothing is
 *    enqueued and no output is modified.
 *  - Device memory is always owned by the caller.  The library never
 *    allocates device memory; it keeps host-side metadata only.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Enqueued work is asynchronous with respect to the host unless stated.
 *  - Device pointers must be 16-byte aligned.
 *
 * Layouts
 *  - Store arenas (K and V separately): [L][capacity_rows][H][D] bf16,
 *    layer-major; a fact owns the same contiguous row range in every layer.
 *  - Paged cache, one K and one V tensor per layer, slot = block *
 *    block_size + offset, in one of two layouts (prkv_cache_layout):
 *    NHD [num_blocks][block_size][H][D] bf16 (vLLM's paged layout: a slot's
 *    heads are contiguous) or HND [num_blocks][H][block_size][D] bf16 (each
 *    head's part of a block is contiguous).
 *  - RoPE: pair j (j = 0 .. D/2-1) is the complex number z_j = x_a + i x_b
 *    with (a, b) = (j, j + D/2) for half-split pairing (GPT-NeoX style) or
 *    (2j, 2j + 1) for interleaved pairing (GPT-J style); rotation to position
 *    p is z_j' = z_j * exp(+i p f_j) with f_j = rope_theta^(-2j/D), or f_j
 *    rescaled by the Llama 3.1 long-context rule when the descriptor asks for
 *    it (see prkv_store_desc).
 *  - Keys in the store are either pre-RoPE (rotated at injection to their
 *    serving position) or already rotated at chunk-local positions 0, 1, ...
 *    within their fact (relocated at injection by R(s), s = the fact's
 *    serving start; R_a^T R_b = R_{b-a}, Theorem 6).
 */
#ifndef PRKV_H
#define PRKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum prkv_status {
  PRKV_OK = 0,
  PRKV_ERR_INVALID_ARG = -1,    /* bad size, null pointer, bad descriptor   */
  PRKV_ERR_ALIGNMENT = -2,      /* device pointer not 16-byte aligned       */
  PRKV_ERR_UNKNOWN_FACT = -3,   /* fact id never put                        */
  PRKV_ERR_DUPLICATE_FACT = -4, /* fact id put twice                        */
  PRKV_ERR_CAPACITY = -5,       /* arena rows exhausted / id >= max_facts   */
  PRKV_ERR_OUT_OF_RANGE = -6,   /* position, block index or block id        */
  PRKV_ERR_DUPLICATE_SLOT = -7, /* two injected tokens map to one slot      */
  PRKV_ERR_BUFFER_TOO_SMALL = -8,
  PRKV_ERR_NO_DEVICE = -9,      /* metadata-only store used for device work */
  PRKV_ERR_HIP = -10,           /* a HIP runtime call failed                */
  PRKV_ERR_NO_MEMORY = -11      /* host allocation failed                   */
};

/* Pairing of the head dimensions into rotated pairs. */
enum prkv_rope_style {
  PRKV_ROPE_HALF_SPLIT = 0,   /* (j, j + D/2): GPT-NeoX / Hugging Face Llama  */
  PRKV_ROPE_INTERLEAVED = 1   /* (2j, 2j + 1): GPT-J / original Llama          */
};

/* Frequency rule.  LLAMA3 is the long-context rescaling published with
 * Llama 3.1 (one of the models the InferScale review evaluates, "Referee
 * Report" Summary): with wavelength w_j = 2 pi / f_j, W = original_max_position,
 * f_j is kept where w_j < W / high_freq_factor, divided by scaling_factor
 * where w_j > W / low_freq_factor, and in between blended as
 * (1 - m) f_j / scaling_factor + m f_j, m = (W / w_j - low_freq_factor) /
 * (high_freq_factor - low_freq_factor).  Llama 3.1 uses factor 8, low 1,
 * high 4, W = 8192, rope_theta = 5e5. */
enum prkv_rope_scaling { PRKV_SCALING_NONE = 0, PRKV_SCALING_LLAMA3 = 1 };

/* What the store's K rows hold.  PRE_ROPE: keys before rotary encoding
 * (InferScale review, "What carries the argument").  CHUNK_LOCAL: keys
 * already rotated at positions 0 .. len-1 of their own fact (a fact encoded
 * on its own); injection applies the relocation R(s), s = the fact's first
 * serving position, which equals rotating the pre-RoPE key to s + t in exact
 * arithmetic (Theorem 6) but not bit for bit, since the stored key was
 * already rounded to bf16 once. */
enum prkv_key_layout { PRKV_KEYS_PRE_ROPE = 0, PRKV_KEYS_CHUNK_LOCAL = 1 };

/* Element order inside one block of the paged cache (the same for every
 * layer, K and V).  NHD: [block_size][H][D], the paged layout of vLLM that
 * the InferScale review scatters into ("Referee Report", Summary); element
 * (block b, offset o, head h, dim d) is at ((b * block_size + o) * H + h) * D
 * + d.  HND: [H][block_size][D]; the same element is at ((b * H + h) *
 * block_size + o) * D + d, so one head's keys of a block are contiguous
 * (block_size * D * 2 bytes), which suits per-head attention reads.  Slots
 * and block tables mean the same in both. */
enum prkv_cache_layout { PRKV_CACHE_NHD = 0, PRKV_CACHE_HND = 1 };

/* Shape of a store and of the model it serves.  Zero-initialised trailing
 * fields select the defaults (pre-RoPE keys, no frequency scaling, NHD
 * cache). */
typedef struct prkv_store_desc {
  int32_t num_layers;    /* L, 1..128                                         */
  int32_t num_kv_heads;  /* H >= 1                                            */
  int32_t head_dim;      /* D in {16, 32, 64, 128, 256, 512, 1024}            */
  int32_t max_facts;     /* fact ids are 0 .. max_facts-1                     */
  int64_t capacity_rows; /* rows per layer in each arena, <= 2^31-1           */
  int32_t max_position;  /* positions must be < max_position                  */
  int32_t rope_style;    /* prkv_rope_style                                   */
  double rope_theta;     /* RoPE base, > 1                                    */
  int32_t key_layout;    /* prkv_key_layout                                   */
  int32_t rope_scaling;  /* prkv_rope_scaling                                 */
  double scaling_factor;   /* LLAMA3: >= 1                                    */
  double low_freq_factor;  /* LLAMA3: > 0                                     */
  double high_freq_factor; /* LLAMA3: > low_freq_factor                       */
  int32_t original_max_position; /* LLAMA3: W >= 1                            */
  int32_t cache_layout;  /* prkv_cache_layout of the paged caches this store
                            injects into (inject_topk, inject_topk_device) and
                            attend_paged reads                                 */
} prkv_store_desc;

typedef struct prkv_store prkv_store; /* opaque host-side store handle */

/* Bytes the caller must allocate on the device for ONE arena (K or V) and for
 * the RoPE table that store_create fills:
 *   arena = L * capacity_rows * H * D * 2,
 *   rope  = max_position * (D/2) * 16   (cos, sin as float32 hi/lo pairs). */
int store_required_bytes(const prkv_store_desc* desc, size_t* arena_bytes_each,
                         size_t* rope_table_bytes);

/* Create a store over caller-owned device memory.
 * Source: InferScale review, "Referee Report" Summary ("stored pre-RoPE
 * alongside semantic embeddings", GPU-resident) and Figure 2 (one fact_id
 * names the fact's embedding and its pre-RoPE K/V).
 * k_arena, v_arena: arena_bytes_each each, in device memory, or in pinned
 * host memory mapped for the device (hipHostMalloc) to keep the store in host
 * DRAM ("If this is right" bullet 4: offloading the store to host DRAM costs
 * milliseconds); the inject kernel then reads only the retrieved rows, over
 * PCIe, directly from host memory.  rope_table: device,
 * rope_table_bytes; filled here (float64 angles split into float32 hi + lo)
 * with a copy on `stream` that this call waits for.  Passing all three
 * pointers as NULL creates a metadata-only store: facts can be reserved and
 * build_slot_mapping works, device calls return PRKV_ERR_NO_DEVICE.
 * On success *out receives the handle (free with store_destroy). */
int store_create(const prkv_store_desc* desc, void* k_arena, void* v_arena,
                 void* rope_table, void* stream, prkv_store** out);

/* Append one fact: `len` rows in every layer, the same row range in K and V.
 * Source: InferScale review, Figure 2 caption (offline, each fact is encoded
 * once under a shared fact_id) and the ledger's read-mostly-store axiom
 * (Proposition 5; online updates are future work, so the store is
 * append-only and has no delete).
 * k_src, v_src: [L][len][H][D] bf16, contiguous, device memory or pinned host
 * memory; copied on `stream` (asynchronous: keep them alive until the stream
 * passes).  With both NULL the rows are only reserved (another producer may
 * write them; see store_fact_info).  Errors: INVALID_ARG, CAPACITY (id >=
 * max_facts or not enough rows), DUPLICATE_FACT, NO_DEVICE (sources given to a
 * metadata-only store), HIP. */
int store_put_fact(prkv_store* st, int32_t fact_id, int32_t len, const void* k_src,
                   const void* v_src, void* stream);

/* Copy facts from one store into another: K and V rows of every listed
 * fact, all layers, with one hipMemcpy2DAsync per fact and tensor on
 * `stream`.  For a store kept in host DRAM ("If this is right" bullet 4 of
 * the InferScale review: the store can live in host memory at a cost of
 * milliseconds; Figure 1: only the retrieved facts' KV cross PCIe) this
 * stages the retrieved facts into an HBM store before injecting from it, as
 * an alternative to the kernel reading host memory directly; staging a
 * batch in chunks on a second stream overlaps the copies with the injection
 * of earlier chunks.
 * src, dst: two different device-backed stores with equal num_layers,
 * num_kv_heads, head_dim and key_layout (arenas may be device or pinned
 * host memory).
 * fact_ids: host int32[n_facts].  A fact already in dst (same length) has
 * its rows overwritten in place; an absent one is appended (once, if listed
 * twice).  Errors, all before anything is enqueued: INVALID_ARG (shapes,
 * lengths), UNKNOWN_FACT (not in src), CAPACITY (dst rows or fact ids),
 * NO_DEVICE, NO_MEMORY; HIP if a copy cannot be enqueued (copies enqueued
 * before it stay enqueued, and dst records none of this call's appends).
 * Asynchronous: src and dst must stay valid until the stream passes. */
int store_stage_facts(const prkv_store* src, prkv_store* dst, int32_t n_facts,
                      const int32_t* fact_ids, void* stream);

/* Row range of a fact: *first_row and *len (UNKNOWN_FACT if never put). */
int store_fact_info(const prkv_store* st, int32_t fact_id, int64_t* first_row,
                    int32_t* len);

/* Release the host-side handle.  Device memory stays the caller's. */
void store_destroy(prkv_store* st);

/* Flatten a batch of requests into per-token (arena row, position, slot).
 * Source: InferScale review, "If this is right" bullet 2 and "invented
 * entities: Chunked RoPE" (facts encoded once are placed at arbitrary prompt
 * positions, dynamically ordered), and the KV-connector axiom (section 3.4:
 * the prefix is marked externally available, blocks are allocated without
 * prefill, then K/V are scatter-copied).
 * Host-only; makes no HIP call.
 *   Request r has facts fact_ids[req_fact_ptr[r] .. req_fact_ptr[r+1]) in
 *   rank order and a prefix of start_pos[r] tokens.  Its facts occupy
 *   positions start_pos[r], start_pos[r]+1, ... contiguously, in list order;
 *   position p lives in slot block_tables[r*bt_stride + p/block_size] *
 *   block_size + p % block_size, for p/block_size < bt_len[r].
 * Outputs (host int32, `capacity` entries each), in request, fact, token
 * order: src_row (arena row), pos (rotation position: the token's serving
 * position for a PRE_ROPE store, its fact's first serving position, i.e. the
 * relocation offset, for a CHUNK_LOCAL store), slot (cache slot); *n_tokens
 * is the token count.  If capacity is too small, BUFFER_TOO_SMALL is returned
 * with *n_tokens set to the count needed and the outputs untouched.
 * Errors: INVALID_ARG, UNKNOWN_FACT, OUT_OF_RANGE (position >= max_position,
 * block table too short, block id outside [0, num_blocks)), DUPLICATE_SLOT
 * (two tokens of this call in one slot; the same fact twice in one request is
 * legal, at two positions).  Safe to call concurrently on one store. */
int build_slot_mapping(const prkv_store* st, int32_t n_req, const int32_t* req_fact_ptr,
                       const int32_t* fact_ids, const int32_t* start_pos,
                       const int32_t* block_tables, int32_t bt_stride,
                       const int32_t* bt_len, int32_t block_size, int64_t num_blocks,
                       int32_t* src_row, int32_t* pos, int32_t* slot, int64_t capacity,
                       int64_t* n_tokens);

/* Gather, rotate and scatter: for every token t and layer l,
 *   Kcache_l[slot[t]] = R(pos[t]) applied to Karena[l][src_row[t]]
 *   Vcache_l[slot[t]] = Varena[l][src_row[t]]            (bit copy)
 * Source: InferScale review, "What carries the argument" (keys stored
 * pre-RoPE are re-rotated to serving-time positions on injection into the
 * paged cache) and "Referee Report" Summary (scatter-copy into vLLM's paged
 * KV cache); Theorem 6 (rotation at injection is an exact relocation).
 * One kernel launch covers every token, layer and KV head.  K is rotated in
 * float32 with compensated (hi/lo) cos/sin and rounded to nearest-even bf16.
 * d_src_row, d_pos, d_slot: device int32[n_tokens] (from build_slot_mapping).
 * k_cache_layers, v_cache_layers: HOST arrays of L device pointers, each a
 * bf16 tensor of num_blocks blocks in the store's cache_layout
 * ([num_blocks][block_size][H][D] for NHD, [num_blocks][H][block_size][D]
 * for HND).  d_status: optional device
 * int32; if non-NULL the kernel ORs 1 (row out of range), 2 (position out of
 * range) or 4 (slot out of range) into it for any token it skipped; tokens
 * out of range are never read or written, and a row of -1 skips a token
 * silently.  n_tokens == 0 is a no-op.
 * Asynchronous on `stream`; never synchronizes.  Slots must be distinct
 * (build_slot_mapping guarantees it); otherwise the result is undefined. */
int inject_topk(const prkv_store* st, int64_t n_tokens, const int32_t* d_src_row,
                const int32_t* d_pos, const int32_t* d_slot,
                void* const* k_cache_layers, void* const* v_cache_layers,
                int32_t block_size, int64_t num_blocks, int32_t* d_status,
                void* stream);

/* Device-resident description of a batch of requests (all pointers are
 * device memory, int32): request r has facts fact_ids[req_fact_ptr[r] ..
 * req_fact_ptr[r+1]) in rank order, a prefix of start_pos[r] tokens, and
 * block table block_tables[r*bt_stride .. + bt_len[r]).  max_facts bounds
 * req_fact_ptr[n_req]; max_tokens bounds the injected token count and sizes
 * the workspace.  flags: 0, or PRKV_BATCH_CHECK_SLOTS (see
 * inject_topk_device). */
#define PRKV_BATCH_CHECK_SLOTS 1
typedef struct prkv_device_batch {
  int32_t n_req;
  int32_t bt_stride;
  int32_t max_facts;
  int32_t flags;
  int64_t max_tokens;
  const int32_t* req_fact_ptr;  /* [n_req + 1] */
  const int32_t* fact_ids;      /* [req_fact_ptr[n_req]] */
  const int32_t* start_pos;     /* [n_req] */
  const int32_t* block_tables;  /* [n_req][bt_stride] */
  const int32_t* bt_len;        /* [n_req] */
} prkv_device_batch;

/* Copy the store's fact table into caller-owned device memory for
 * inject_topk_device: [max_facts] x (int32 first row or -1 when absent,
 * int32 length), table_bytes >= 8 * max_facts, 8-byte aligned.  The copy is
 * complete when the call returns.  Call again after further puts.
 * Source: InferScale review, Figure 2 caption (top-k ids resolved to their
 * KV by fact_id on the GPU). */
int store_upload_fact_table(const prkv_store* st, void* d_table, size_t table_bytes,
                            void* stream);

/* Workspace bytes inject_topk_device needs for the given bounds.  Layout
 * (all offsets 256-byte aligned): int64 token count at 0, int32 fact count
 * at 8; per-fact plan (16 bytes each) at 256; then the per-token arrays
 * src_row, pos, slot (int32 [max_tokens] each) -- the same mapping
 * build_slot_mapping produces on the host, valid after the call's kernels
 * have run (a row of -1 marks a token that failed validation or, with
 * PRKV_BATCH_CHECK_SLOTS, whose slot another token also maps to); then the
 * duplicate-slot set used by PRKV_BATCH_CHECK_SLOTS: uint32 entries, as many
 * as the smallest power of two >= max(64, 2 * max_tokens). */
int inject_device_workspace_bytes(int32_t max_facts, int64_t max_tokens, size_t* bytes);

/* The whole retrieve-and-inject step on the device, from a batch resident in
 * HBM: resolve fact ids through the device fact table, place each request's
 * facts after its prefix in rank order, map positions to slots through its
 * block table, then gather, rotate and scatter exactly as inject_topk.
 * Source: as build_slot_mapping and inject_topk (InferScale review, "If this
 * is right" bullet 2, KV-connector axiom of section 3.4, "What carries the
 * argument", "Referee Report" Summary).
 * Kernels on `stream`: when batch->max_facts <= 256, n_req <= 256 and the
 * expected token count (max_facts x the store's mean stored fact length,
 * + 10 %) is <= 4096, one launch (every inject workgroup maps its own tokens
 * from the batch); other batches take three (plan, per-token mapping,
 * inject).  Both fill the
 * workspace and d_status identically.  The launch is sized for max_facts
 * facts of the store's mean stored length; any count up to max_tokens is
 * handled, a larger one with more work per workgroup.  Asynchronous, never
 * synchronizes.  d_workspace: caller-owned device memory of
 * inject_device_workspace_bytes(batch->max_facts, batch->max_tokens), 256-byte
 * aligned; d_fact_table from store_upload_fact_table.  Invalid input found on
 * the device never faults: the token is skipped and d_status (optional) gets
 * 2 (position out of range), 4 (block table too short or block id out of
 * range), 8 (unknown fact id), 16 (more than max_tokens tokens; the excess is
 * dropped) or 32 (more than max_facts facts).
 * Duplicate slots (two tokens of the batch mapped to one cache slot, e.g.
 * block tables that share a block; the result would depend on write order)
 * are detected only when batch->flags has PRKV_BATCH_CHECK_SLOTS: every
 * token whose slot another token of the batch also maps to is skipped (none
 * of them is written, the rest of the batch is) and d_status gets 128.  The
 * check always takes the separate kernels, plus a clear of the workspace's
 * slot set and a pass that marks the colliding tokens (KV-connector axiom,
 * section 3.4: blocks are allocated to the request, then scatter-copied;
 * build_slot_mapping rejects such a batch on the host with DUPLICATE_SLOT).
 * Without the flag duplicate slots are not detected (block tables from one
 * allocator never overlap) and the colliding writes race.
 * Host-side argument errors (including unknown flags) return INVALID_ARG /
 * ALIGNMENT / BUFFER_TOO_SMALL / NO_DEVICE with nothing enqueued. */
int inject_topk_device(const prkv_store* st, const void* d_fact_table,
                       const prkv_device_batch* batch, void* const* k_cache_layers,
                       void* const* v_cache_layers, int32_t block_size, int64_t num_blocks,
                       void* d_workspace, size_t workspace_bytes, int32_t* d_status,
                       void* stream);

/* inject_topk_device without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, kernels, results and
 * d_status bits as inject_topk_device; the workspace is instead a static
 * array of PRKV_NOALLOC_SCRATCH_BYTES in this library's device code, one per
 * GPU, held until the process ends.  The call allocates nothing (no
 * hipMalloc, no host-side allocation on success).  Limits: the batch bounds
 * must fit the array, i.e. inject_device_workspace_bytes(batch->max_facts,
 * batch->max_tokens) <= PRKV_NOALLOC_SCRATCH_BYTES (16 MiB: e.g. 4,096 facts
 * and 690,000 tokens), else PRKV_ERR_BUFFER_TOO_SMALL with nothing
 * enqueued.  Every call on one GPU shares that GPU's array and leaves the
 * last call's mapping in it; nothing in it needs to start at zero.  Calls
 * that overlap on one GPU (several streams, several threads or processes'
 * streams at once) race on the array: serialize them, or use
 * inject_topk_device with separate workspaces.  The array used is the one
 * of the device that runs `stream` (the current device for the null
 * stream); the first call on a device looks up its address
 * (hipGetSymbolAddress) with that device current, then restores the
 * caller's current device. */
#define PRKV_NOALLOC_SCRATCH_BYTES (16u << 20)
int inject_topk_device_noalloc(const prkv_store* st, const void* d_fact_table,
                               const prkv_device_batch* batch, void* const* k_cache_layers,
                               void* const* v_cache_layers, int32_t block_size,
                               int64_t num_blocks, int32_t* d_status, void* stream);

/* Exact top-k retrieval by inner product, the step before injection.
 * Source: InferScale review, "Referee Report" Summary (facts retrieved at
 * serving time through a GPU index, then resolved to their KV) and Figure 2
 * caption (each fact has a retrieval embedding in the GPU vector store under
 * its fact_id); "Circularity Check": the index backend changes latency, not
 * the facts found -- exact search stands in for the approximate index.
 * d_fact_emb: device bf16 [n_stores][facts_per_store][dim]; d_query_emb:
 * device bf16 [n_req][dim]; d_req_store: device int32 [n_req], the store each
 * request searches.  dim: multiple of 8 in [8, 4096]; 1 <= k <= 64 and
 * k <= facts_per_store.  Scores are inner products of the bf16 values
 * accumulated in float64 (products are exact).  Output d_fact_ids: device
 * int32 [n_req][k], global ids store * facts_per_store + fact, best first
 * (higher score, then smaller id; a NaN score ranks below every number);
 * d_scores: optional device double
 * [n_req][k].  A request with an out-of-range store gets ids -1 and sets
 * bit 64 in d_status.  d_workspace: device, retrieve_workspace_bytes
 * (scores, plus partial top-64 lists when few requests have many facts),
 * 8-byte aligned.  Two kernels on `stream` (scores, top-k), three when the
 * top-k of a request is split over several workgroups; asynchronous.  The ids can be
 * passed straight to inject_topk_device (req_fact_ptr[r] = r * k). */
int retrieve_workspace_bytes(int32_t n_req, int32_t facts_per_store, size_t* bytes);
int retrieve_topk(const void* d_fact_emb, int32_t n_stores, int32_t facts_per_store,
                  int32_t dim, const void* d_query_emb, const int32_t* d_req_store,
                  int32_t n_req, int32_t k, int32_t* d_fact_ids, double* d_scores,
                  void* d_workspace, size_t workspace_bytes, int32_t* d_status, void* stream);

/* Query-prefill attention over the paged cache, the step after injection:
 * only the query is prefilled and it attends to the prefix, the injected
 * facts and itself.  Source: InferScale review, "The pith" (only the query
 * is prefilled), "Core claim" / Theorem 3 (KV injected at the intended
 * positions is equivalent to prompt-injecting the same tokens), reference
 * [1] (grouped-query attention).
 * For every layer l, request r, query token i (position q_start[r] + i) and
 * query head h (KV head h / (num_q_heads / H)):
 *   out[l][r][i][h] = softmax_j(scale * <RoPE(q), K_l[j]>) V_l[j] over the
 *   positions j <= q_start[r] + i, K/V read from the paged cache (in the
 *   store's cache_layout) through the request's block table (every such
 *   position must have been written: prefix, injected facts and the query's
 *   own K/V).
 * q: pre-RoPE, rotated in the kernel with the store's table.  K and V of the
 * cache are bf16; q and the probabilities are carried as bf16 hi + lo pairs
 * into the matrix cores, so the result is accurate to fp32 rounding.
 * Limits: head_dim 64 or 128; q_len <= max_position.  A block table of up
 * to 2048 entries is staged in LDS, a longer one read from device memory.
 * Rows (query token, query head) are taken 64 at a time per (layer,
 * request, KV head): a query of q_len * (num_q_heads / H) <= 64 rows reads
 * its context once, a longer one once per 64 rows.
 * Status (d_status, optional): positions whose block is missing from the
 * table are masked and set bit 4; a request whose query positions do not
 * lie in [0, max_position) sets bit 2 and gets output 0; a q_lens value
 * outside [0, q_len] sets bit 8 and is clamped.
 * One kernel launch on `stream`, asynchronous. */
typedef struct prkv_attn_batch {
  int32_t n_req;
  int32_t q_len;               /* query tokens per request */
  int32_t num_q_heads;         /* multiple of the store's num_kv_heads */
  int32_t bt_stride;
  const uint16_t* q;           /* device [n_req][q_len][num_q_heads][D] bf16 */
  const int32_t* q_start;      /* device [n_req]: position of the first query token */
  const int32_t* block_tables; /* device [n_req][bt_stride] */
  const int32_t* bt_len;       /* device [n_req] */
  float* out;                  /* device [L][n_req][q_len][num_q_heads][D] */
  const int32_t* q_lens;       /* device [n_req] or NULL: request r's query is its
                                  first q_lens[r] <= q_len tokens (positions
                                  q_start[r] ..); the rows past it get output 0 */
} prkv_attn_batch;

int attend_paged(const prkv_store* st, const prkv_attn_batch* batch,
                 void* const* k_cache_layers, void* const* v_cache_layers, int32_t block_size,
                 int64_t num_blocks, float softmax_scale, int32_t* d_status, void* stream);

/* Fill a HOST buffer with the RoPE table store_create would upload:
 * [max_position][D/2][4] float32 = (cos_hi, cos_lo, sin_hi, sin_lo) with
 * cos_hi = fl32(cos a), cos_lo = fl32(cos a - cos_hi), a = pos * f_j in
 * float64 (f_j after the descriptor's frequency rule).  out_bytes must be
 * >= rope_table_bytes. */
int rope_table_fill(const prkv_store_desc* desc, float* out, size_t out_bytes);

/* Text of the last error on this thread ("" if none). */
const char* last_error_string(void);

#ifdef __cplusplus
}
#endif

#endif /* PRKV_H */
