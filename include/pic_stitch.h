/*
 * pic_stitch.h -- C ABI of the position-independent KV stitching library
 * (libpic_stitch.so, HIP for gfx950).
 *
 * Position-independent caching keeps the KV cache of every reusable chunk
 * (a document, a tool schema, a system prompt) computed once at virtual
 * offset 0 and places it at any logical offset of a later request (EPIC
 * Guide: Position-Independent Caching for LLM Serving, "Position-Independent
 * Caching (PIC): Formalization & Core Challenges" and "Algorithmic
 * Architecture: The EPIC Serving Runtime").  Placing a chunk needs:
 *   - the keys' rotary part turned by delta = p_target - p_source on every
 *     RoPE plane i, by the angle delta * theta_i with theta_i = b^(-2i/d)
 *     (EPIC Guide, "Mathematical Foundations", sections 1 and 2; Irminsul:
 *     MLA-Native Position-Independent Caching for Agentic LLM Serving,
 *     Technical Summary section 2.2, delta-rotation rule);
 *   - the values, and for MLA the 512-dim content latent, copied unchanged
 *     (EPIC Guide section 2, values untouched; Irminsul section 2.1);
 *   - the first recompute_k tokens of a chunk left out, for a recompute
 *     pass to fill (Irminsul section 2.2, first-chunk carve-out).
 *
 * Conventions for every call:
 *   - All sizes, offsets and strides are in elements of the storage type
 *     unless stated otherwise; positions and token indices are int64.
 *   - KV memory is device memory owned by the caller.  Views are borrowed
 *     until the work enqueued on `stream` has finished.
 *   - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *     Calls return once the work is enqueued; device faults surface at the
 *     caller's next synchronisation.
 *   - Every argument is validated before anything is enqueued: a call that
 *     returns an error has written nothing.  Nothing aborts the process.
 *   - Device pointers and every row start must be 16-byte aligned, i.e. all
 *     strides and the rotary offset are multiples of 16 bytes' worth of
 *     elements (4 for f32, 8 for bf16).
 *   - pic_last_error() returns a thread-local message for the last failure
 *     on the calling thread.
 */
#ifndef PIC_STITCH_H
#define PIC_STITCH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pic_status {
    PIC_OK = 0,
    PIC_ERR_INVALID_ARG = 1, /* malformed shape, rope config, view or layer range */
    PIC_ERR_RANGE = 2,       /* index or length outside what it refers to */
    PIC_ERR_OVERLAP = 3,     /* two placements claim one position or one row */
    PIC_ERR_ALIGN = 4,       /* pointer, stride or slice not 16-byte aligned */
    PIC_ERR_DEVICE = 5,      /* HIP runtime error (launch, copy, allocation) */
    PIC_ERR_NOMEM = 6,       /* host allocation failed */
    PIC_ERR_STATE = 7        /* plan used on another device, or destroyed */
} pic_status;

enum { PIC_DTYPE_F32 = 0, PIC_DTYPE_BF16 = 1 };

/* Pairing of the rotated dimensions into planes. */
enum {
    PIC_ROPE_HALF = 0,       /* plane i = dims (i, i + rope_dim/2): rotate-half models */
    PIC_ROPE_INTERLEAVED = 1 /* plane i = dims (2i, 2i + 1), as the EPIC Guide writes it */
};

/* RoPE of the model (EPIC Guide, "RoPE Mathematical Structure"). */
typedef struct pic_rope_config {
    int32_t rope_dim;        /* rotated dims per head row: even, >= 2 */
    int32_t style;           /* PIC_ROPE_HALF | PIC_ROPE_INTERLEAVED */
    double theta;            /* base b; theta_i = b^(-2i/rope_dim) */
    const double *inv_freq;  /* optional host table of rope_dim/2 values replacing the
                                formula (scaled RoPE variants); NULL = formula */
} pic_rope_config;

/*
 * Per-layer KV geometry.  Every token has num_heads K rows of row_dim
 * elements (and as many V rows when has_v); the rotary slice of each K row
 * is [rope_offset, rope_offset + rope_dim).
 *   GQA (Llama-style):  num_heads 8, row_dim 128, rope_offset 0, has_v 1
 *   MLA (DeepSeek-V3):  num_heads 1, row_dim 576, rope_offset 512, has_v 0
 *                       (Irminsul section 2.1: cKV 512 + k_r 64)
 */
typedef struct pic_kv_shape {
    int32_t dtype; /* PIC_DTYPE_F32 | PIC_DTYPE_BF16 */
    int32_t num_layers;
    int32_t num_heads;
    int32_t row_dim;
    int32_t rope_offset;
    int32_t has_v; /* 0 or 1 */
} pic_kv_shape;

/*
 * A cached chunk.  Its keys were rotated for positions base_pos, base_pos +
 * 1, ... (EPIC caches at virtual offset 0, so base_pos is normally 0;
 * Irminsul's registry stores it explicitly, section 2.2).
 *   Contiguous pool (geometry src_page_size 0): the chunk's tokens are pool
 *     rows [token_start, token_start + length); n_pages 0, page_table NULL.
 *   Paged pool (src_page_size > 0: the PagedAttention block pool of the EPIC
 *     Guide's runtime figure, chunks kept at virtual offset 0 in physical
 *     blocks): token t of the chunk is at slot (token_start + t) %
 *     src_page_size of physical page page_table[(token_start + t) /
 *     src_page_size]; token_start is the chunk's offset inside its first
 *     page (normally 0) and page_table (host memory, read during pic_plan
 *     only) holds n_pages entries.
 */
typedef struct pic_chunk {
    int64_t token_start;
    int64_t base_pos;
    int32_t length;
    int32_t n_pages;
    const int32_t *page_table;
} pic_chunk;

/* One placement: chunk tokens [0, length) go to logical positions
 * [dst_offset, dst_offset + length) of the request; tokens [0, recompute_k)
 * are not written. */
typedef struct pic_entry {
    int64_t dst_offset;
    int32_t chunk_id;
    int32_t length;
    int32_t recompute_k;
    int32_t reserved; /* must be 0 */
} pic_entry;

/* A request's placement table (host memory, read during pic_plan only).
 * page_table maps logical page j to a physical page of the paged
 * destination; it is ignored for a contiguous destination.  context_len is
 * the request's context for pic_attend: positions [0, context_len); 0 means
 * up to the end of its last entry. */
typedef struct pic_request {
    const pic_entry *entries;
    const int32_t *page_table;
    int32_t n_entries;
    int32_t n_pages;
    int64_t context_len;
} pic_request;

/* Pool and destination geometry.  Destination: dst_page_size 0 =
 * contiguous (each request owns dst_capacity positions), else paged with
 * dst_num_pages pages of dst_page_size tokens shared by all requests.
 * Pool: src_page_size 0 = contiguous rows, else src_num_pages pages of
 * src_page_size tokens. */
typedef struct pic_geom {
    int32_t dst_page_size;
    int32_t src_page_size;
    int64_t dst_capacity;
    int64_t dst_num_pages;
    int64_t src_num_pages;
} pic_geom;

/*
 * A device view of K (and V) memory.  Element (layer l, token row t, head
 * h, dim d) of K is k[l*layer_stride + t*token_stride + h*head_stride + d],
 * V the same with v; K and V share the strides.
 *   contiguous pool / in-place buffer: t is the token index.
 *   paged pool: the row of slot s of physical page g starts at
 *     l*layer_stride + g*page_stride + s*token_stride.
 *   contiguous destination: t = r*request_stride/token_stride + position,
 *     i.e. the row of request r's position p starts at
 *     l*layer_stride + r*request_stride + p*token_stride.
 *   paged destination: the row of a position p of a request starts at
 *     l*layer_stride + page_table[p / page_size]*page_stride
 *     + (p % page_size)*token_stride.
 * Unused strides are ignored.  v is ignored when has_v is 0.
 */
typedef struct pic_kv_view {
    void *k;
    void *v;
    int64_t layer_stride;
    int64_t token_stride;
    int64_t head_stride;
    int64_t page_stride;
    int64_t request_stride;
} pic_kv_view;

/* In-place mode: rotate tokens [token_start + recompute_k, token_start +
 * length) of a buffer by delta positions. */
typedef struct pic_segment {
    int64_t token_start;
    int64_t delta;
    int32_t length;
    int32_t recompute_k;
} pic_segment;

typedef struct pic_plan_info_t {
    int64_t n_requests;
    int64_t n_entries;
    int64_t n_tiles;              /* work items of one layer */
    int64_t tokens_written;       /* per layer */
    int64_t tokens_masked;        /* per layer: sum of recompute_k */
    int64_t pool_tokens_required; /* contiguous pool: max token_start + length over chunks;
                                     paged pool: src_num_pages * src_page_size */
    int64_t bytes_read_per_layer; /* algorithmic: rows read */
    int64_t bytes_written_per_layer;
    int64_t tile_tokens;          /* most tokens of one work tile (paged tiles also stop at
                                     page ends) */
    int64_t context_tokens;       /* pic_attend: sum of context_len over requests */
    int64_t attend_blocks;        /* pic_attend: (request, block of positions) work items */
    int64_t attend_block_tokens;  /* pic_attend: positions per block at most (256, 128 or 64:
                                     shorter when few blocks would leave the GPU idle) */
} pic_plan_info_t;

typedef struct pic_plan pic_plan_t;

/*
 * pic_plan -- validate a stitch problem and build its execution plan
 * (EPIC Guide, "Modular Prompt Composer": the composer computes the shift of
 * every hit chunk; SemPIC: Learning Semantic Position-Independent KV Caches,
 * cache-hit serving: final logical positions are assigned, then keys are
 * re-rotated).
 *
 * For every entry, delta = dst_offset - chunk.base_pos; cos/sin of
 * delta*theta_i are computed in fp64 on the host; tokens [recompute_k,
 * length) are cut into work tiles.  Host only: no HIP call is made, so the
 * plan can be built without a GPU.  All input arrays are copied; the
 * caller may free them on return.  The attention map (pic_attend*) is not
 * built here but by the first call that needs it.
 *
 * Valid input (else PIC_ERR_RANGE unless noted):
 *   0 <= chunk_id < n_chunks; 1 <= length <= chunk.length;
 *   0 <= recompute_k <= length; dst_offset >= 0;
 *   dst_offset + length <= dst_capacity (contiguous) or
 *     <= n_pages * dst_page_size (paged), and < 2^31 (positions are int32
 *     on the device);
 *   chunk.token_start >= 0, chunk.length >= 1, |chunk.base_pos| <= 2^62
 *     (so delta = dst_offset - base_pos fits int64); in a paged pool
 *     token_start + length <= n_pages * src_page_size;
 *   every destination page written is in [0, dst_num_pages) and every
 *     pool page read in [0, src_num_pages);
 *   entries of one request do not overlap, and no destination row is
 *     written twice (PIC_ERR_OVERLAP);
 *   duplicate chunk_ids and negative deltas are allowed.
 * Shape/rope errors are PIC_ERR_INVALID_ARG; a rotary slice or unit count
 * that does not fit 16-byte vectors is PIC_ERR_ALIGN.
 *
 * On success *out owns a plan released by pic_plan_destroy.
 */
pic_status pic_plan(const pic_kv_shape *shape, const pic_rope_config *rope,
                    const pic_chunk *chunks, int32_t n_chunks, const pic_request *requests,
                    int32_t n_requests, const pic_geom *geom, pic_plan_t **out);

/*
 * pic_stitch -- run a plan for layers [layer_begin, layer_end) of the views:
 * one kernel launch reads each placed chunk row once from `pool`, turns the
 * rotary slice of every K row by its entry's delta (fp64 arithmetic, one
 * round-to-nearest-even into the storage type; delta 0 copies the bits),
 * copies V rows and the rest of K unchanged, and writes them to `dst`
 * (EPIC Guide, "The In-Place Shift Transformation"; Irminsul section 2.2).
 * Destination rows not covered (prefixes, gaps, masked tokens) are not
 * touched.  Layer indices address the views directly (0 <= layer_begin <=
 * layer_end <= num_layers), so a view holding a group of layers is run with
 * a range inside that group; every layer has the plan's geometry.
 *
 * The first call uploads the plan's metadata to the current device,
 * ordered on `stream`; later calls on any stream wait for that upload.
 * A plan is bound to the device of its first call (PIC_ERR_STATE after).
 * pool and dst must not overlap.
 */
pic_status pic_stitch(pic_plan_t *plan, const pic_kv_view *pool, const pic_kv_view *dst,
                      int32_t layer_begin, int32_t layer_end, void *stream);

/*
 * pic_rotate_inplace -- turn the rotary slice of K, in place, for tokens
 * [token_start + recompute_k, token_start + length) of every segment by the
 * segment's delta, for layers [layer_begin, layer_end) of `buf` (EPIC
 * Guide, "The In-Place Shift Transformation" and the runtime's in-place key
 * rotation step).  V and the non-rotary dims are not touched.  Segments
 * must lie in [0, buf_tokens) and must not overlap (PIC_ERR_RANGE,
 * PIC_ERR_OVERLAP).  Per call, the library builds the shift tables on the
 * host and stages them in stream-ordered device memory that it frees on
 * the same stream.
 */
pic_status pic_rotate_inplace(const pic_kv_shape *shape, const pic_rope_config *rope,
                              const pic_kv_view *buf, int64_t buf_tokens,
                              const pic_segment *segments, int32_t n_segments,
                              int32_t layer_begin, int32_t layer_end, void *stream);

/*
 * pic_rotate_inplace_noalloc -- pic_rotate_inplace for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments, the same kernels
 * and the same result, with nothing allocated by the call.  The tiles and
 * shift tables, which pic_rotate_inplace stages in stream-ordered device
 * memory, are written by small fill kernels (their bytes carried in the
 * kernel arguments) into a static device array of 4 MiB that each device
 * holds until the process ends; its address is taken once per device, on
 * the first call with that device current.
 * Limit: the staged metadata (32 bytes per tile of at most 16 tokens, plus
 * rope_dim * 8 bytes per distinct nonzero delta, each part padded to 256
 * bytes) must fit in 4 MiB, else PIC_ERR_RANGE before anything is enqueued
 * (e.g. 64 segments of 2032 turned tokens with rope_dim 128 stage 318 KiB).
 * Every call on a device shares that array: calls ordered on one stream
 * are safe; calls that may overlap on one device (different streams) race.
 * Errors otherwise as pic_rotate_inplace.
 */
pic_status pic_rotate_inplace_noalloc(const pic_kv_shape *shape, const pic_rope_config *rope,
                                      const pic_kv_view *buf, int64_t buf_tokens,
                                      const pic_segment *segments, int32_t n_segments,
                                      int32_t layer_begin, int32_t layer_end, void *stream);

/*
 * One segment of a paged KV buffer for pic_rotate_paged.  Token t of the
 * segment (t in [0, length)) sits at logical position first + t of the
 * segment's block table: slot (first + t) % page_size of physical page
 * pages[(first + t) / page_size]; n_pages = ceil((first + length) /
 * page_size).  cow, when given, holds for every logical page the physical
 * page a shared page is copied to, or -1 for a page the caller owns.
 */
typedef struct pic_page_segment {
    const int32_t *pages;  /* host, n_pages physical page ids */
    const int32_t *cow;    /* host, n_pages entries, or NULL: every page owned */
    int64_t delta;
    int32_t n_pages;
    int32_t first;         /* 0 <= first < page_size */
    int32_t length;        /* >= 1 */
    int32_t recompute_k;   /* tokens [0, recompute_k) are not turned */
} pic_page_segment;

/*
 * pic_rotate_paged -- the in-place turn on a paged buffer whose physical
 * pages (blocks) may be shared by several requests, with copy-on-write
 * (EPIC Guide, "Algorithmic Architecture: The EPIC Serving Runtime": chunk
 * KV kept at virtual offset 0 in physical blocks of a pool and reused
 * through block tables, and the runtime's in-place key rotation; turning a
 * block in place that another request maps would change that request's
 * keys).  For every segment and token t in [recompute_k, length) the
 * rotary slice of K is turned by the segment's delta, layers [layer_begin,
 * layer_end):
 *   - a page the caller owns (cow NULL or cow[i] < 0) is turned in place:
 *     only the rotary slice of those tokens' K rows is written;
 *   - a shared page (cow[i] >= 0) is left unchanged and its complete
 *     content -- every slot, K and (when the shape has V) V, all dims -- is
 *     written to physical page cow[i], with the segment's tokens on it
 *     turned there; the caller then maps logical page i to cow[i].
 * buf is a paged view (k, v, layer_stride, token_stride = slot stride,
 * head_stride, page_stride) of n_phys_pages pages of page_size slots; v may
 * be NULL when no segment copies a page or the shape has no V.
 * Errors, all before any launch: PIC_ERR_INVALID_ARG (NULL arrays, bad
 * counts, page_size < 1, n_pages not ceil((first + length) / page_size)),
 * PIC_ERR_RANGE (first, length, recompute_k or a page id out of range, or
 * n_pages * page_size above 2^31 - 1: logical positions are int32),
 * PIC_ERR_OVERLAP (two segments turn the same slot of a page in place; a
 * copy target is used twice, or is also a page some segment reads or
 * turns; a page is copied by one segment and turned in place by another).
 * Per call the library stages the tiles and shift tables in stream-ordered
 * device memory that it frees on the same stream.
 */
pic_status pic_rotate_paged(const pic_kv_shape *shape, const pic_rope_config *rope,
                            const pic_kv_view *buf, int32_t page_size, int64_t n_phys_pages,
                            const pic_page_segment *segments, int32_t n_segments,
                            int32_t layer_begin, int32_t layer_end, void *stream);

/*
 * Decode attention over a request's context without writing the stitched
 * cache (Irminsul, Technical Summary sections 2.2 and 4: the delta-rotation
 * applied in the attention kernel's HBM-to-on-chip load path).  For every
 * request r and query head j (KV head j / (num_q_heads / num_heads)):
 *   out[r][j] = sum_p w_p V_p / sum_p w_p,  w_p = exp(scale * q . K_p + b_p)
 * over positions p in [0, context_len).  Positions an entry writes (tokens
 * [recompute_k, length)) read the chunk's pool row and turn its rotary slice
 * by the entry's delta on load (fp32); every other position (prefix, gaps,
 * tokens left for recompute) reads the request's own cache `cache` (the
 * plan's destination geometry) unrotated.  b_p = sink_bias for the first
 * sink_tokens positions of every entry placed after position 0 (the EPIC
 * Guide's LegoLink pseudo-sink damping, section "1. Identifying and
 * Neutralizing Pseudo-Sinks" and its listing: 4 tokens, -15), else 0.
 * Query rows are post-RoPE (rotated for the query's own position).
 */
typedef struct pic_attend_args {
    const void *q;        /* device [request][q head][row_dim], the plan's dtype */
    int64_t q_request_stride, q_head_stride;
    float *out;           /* device [request][q head][row_dim], fp32 */
    int64_t out_request_stride, out_head_stride;
    int32_t num_q_heads;  /* a multiple of the plan's num_heads */
    int32_t layer;        /* layer of the views */
    float scale;          /* logit scale, e.g. 1/sqrt(row_dim) */
    int32_t sink_tokens;  /* LegoLink damping: tokens per chunk start (0 = off) */
    float sink_bias;      /* LegoLink damping: logit offset (the EPIC listing: -15) */
    int32_t reserved;
} pic_attend_args;

/*
 * pic_attend -- enqueue decode attention for every request of a plan at one
 * layer (see above).  GQA rows only (has_v = 1, rope_offset 0 or any slice);
 * row_dim / (16 / element size) must be a power of two and row_dim <= 256
 * (else PIC_ERR_ALIGN); q rows 16-byte aligned (PIC_ERR_ALIGN);
 * num_q_heads a multiple of num_heads, at most 8x (PIC_ERR_INVALID_ARG).
 * Each request's context must be non-empty and, in a paged cache, every
 * page it covers must be in [0, dst_num_pages) (PIC_ERR_RANGE).  In-place
 * plans are refused (PIC_ERR_STATE).
 *
 * The partial results go to a workspace that the plan keeps per stream
 * for its whole life (allocated by the first call on that stream, replaced
 * by a larger one when a call needs more, freed by pic_plan_destroy), so
 * calls on one stream reuse it in stream order and calls on one plan from
 * several streams may overlap.  A stream handle is taken to name one stream
 * for the plan's life.  The plan's attention map is built on
 * the host by the first call that needs it, and its device metadata for a
 * launch shape is uploaded once, ordered on the stream of the call that
 * first needs it; calls on other streams wait for that upload on their own
 * stream.  Nothing waits for the device.
 */
pic_status pic_attend(pic_plan_t *plan, const pic_kv_view *pool, const pic_kv_view *cache,
                      const pic_attend_args *args, void *stream);

/*
 * Decode attention over MLA latent rows (Irminsul, Technical Summary
 * sections 2.1, 2.2 and 4): the plan's rows are 576-wide bf16 latent rows
 * (pic_kv_shape num_heads 1, row_dim 576, rope_offset 512, rope_dim 64,
 * has_v 0).  In the absorbed form of MLA decode every query head j has a
 * 576-wide query row (content part already in the latent space, rotary part
 * post-RoPE); for every request r and query head j:
 *   out[r][j] = sum_p w_p row_p[0, 512) / sum_p w_p,
 *   w_p = exp(scale * q_j . row_p + b_p)
 * over positions p in [0, context_len).  row_p is the row the stitch of
 * this plan would leave at position p: for positions an entry writes, the
 * chunk's pool row with its rotary key turned by the entry's delta (fp64,
 * rounded to bf16 as pic_stitch stores it) while it is loaded; for every
 * other position the request's own cache row.  b_p is the LegoLink damping
 * of pic_attend.  Products on the matrix cores with fp32 accumulation; the
 * softmax weights enter the value product as two bf16 terms (hi + lo).
 */
typedef struct pic_attend_latent_args {
    const void *q;        /* device bf16 [request][q head][576] */
    int64_t q_request_stride, q_head_stride;
    float *out;           /* device fp32 [request][q head][512] */
    int64_t out_request_stride, out_head_stride;
    int32_t num_q_heads;  /* a multiple of 16, at most 1024 */
    int32_t layer;        /* layer of the views */
    float scale;          /* logit scale (DeepSeek-V2/V3: 1/sqrt(192)) */
    int32_t sink_tokens;  /* LegoLink damping: tokens per chunk start (0 = off) */
    float sink_bias;      /* LegoLink damping: logit offset */
    int32_t reserved;
} pic_attend_latent_args;

/*
 * pic_attend_latent -- enqueue latent decode attention for every request of
 * a plan at one layer (see above).  The plan must be a bf16 MLA plan of the
 * shape above (PIC_ERR_INVALID_ARG); q rows 16-byte aligned
 * (PIC_ERR_ALIGN); contexts and pages as for pic_attend (PIC_ERR_RANGE);
 * in-place plans are refused (PIC_ERR_STATE).  Workspace and metadata as
 * for pic_attend: calls on one plan from several streams may overlap.
 */
pic_status pic_attend_latent(pic_plan_t *plan, const pic_kv_view *pool, const pic_kv_view *cache,
                             const pic_attend_latent_args *args, void *stream);

/*
 * LegoLink's boundary reconnection (EPIC Guide, "2. Sparse Cross-Block
 * Reconnection"): the boundary tokens of relocated chunks attend across the
 * chunk boundary.  By default (rows NULL) boundary row b is token j <
 * min(boundary_k, length) of an entry placed after position 0 (entries
 * request by request, in each request's order; pic_plan_ranges lists them).
 * The page leaves open how the "top-k" boundary tokens are chosen, so a
 * caller may instead name them: rows[b] = {entry, j}, entry indexed in plan
 * order (request by request, as pic_plan_ranges lists them), j < its
 * length.  Either way row b attends causally to positions
 * [0, dst_offset + j] of its request:
 *   out[b][jq] = sum_p w_p V_p / sum_p w_p,  w_p = exp(scale * q[b][jq] . K_p + b_p)
 * with the rows pic_attend reads (chunk keys turned by the entry's delta on
 * load, rounded to bf16 as pic_stitch stores them; other positions from the
 * request's own cache), query head jq reading KV head jq / (num_q_heads /
 * num_heads), and b_p the LegoLink damping of pic_attend.  Products on the
 * matrix cores with fp32 accumulation, weights as two bf16 terms.
 */
typedef struct pic_attend_boundary_args {
    const void *q;          /* device bf16 [boundary row][q head][row_dim], post-RoPE */
    int64_t q_row_stride, q_head_stride;
    float *out;             /* device fp32 [boundary row][q head][row_dim] */
    int64_t out_row_stride, out_head_stride;
    int32_t num_q_heads;    /* a multiple of num_heads, at most 8x */
    int32_t layer;
    float scale;
    int32_t boundary_k;     /* boundary tokens per relocated entry, >= 1 (the EPIC
                               listing: 16) */
    int32_t sink_tokens;    /* LegoLink damping (0 = off) */
    float sink_bias;
    const int32_t *rows;    /* host [n_rows][2] {entry, token}, or NULL: the first
                               boundary_k tokens of every relocated entry */
    int32_t n_rows;         /* rows given (ignored when rows is NULL) */
    int32_t reserved;       /* must be 0 */
} pic_attend_boundary_args;

/*
 * pic_attend_boundary -- enqueue the boundary reconnection of a plan at one
 * layer, for the first boundary_k tokens of every relocated entry or for
 * the rows the caller names (see above).  All boundary rows of a request
 * read its context together.
 * Requirements: bf16 plans with K and V head rows of 128 dims and a rotary
 * slice on 8-dim pieces (PIC_ERR_INVALID_ARG, PIC_ERR_ALIGN); q rows
 * 16-byte aligned (PIC_ERR_ALIGN); every boundary row's positions inside
 * its request's context and mapped pages (PIC_ERR_RANGE; also for more
 * than 65535 requests with boundary rows or a launch beyond 2^31 threads);
 * in-place plans refused (PIC_ERR_STATE).
 * Without rows: boundary_k >= 1 (PIC_ERR_INVALID_ARG); a plan without
 * relocated entries enqueues nothing; the work items for a launch shape
 * (boundary_k and the device's CU count) are built on the host and uploaded
 * once per plan.
 * With rows: n_rows >= 0 and reserved 0 (PIC_ERR_INVALID_ARG); rows come
 * request by request -- the rows of one request together, requests in
 * ascending order, any order and repeats within a request -- else
 * PIC_ERR_INVALID_ARG; an entry outside the plan or a token outside its
 * entry is PIC_ERR_RANGE; boundary_k is ignored.  The rows' work items are
 * built and uploaded per call (stream-ordered memory filled from pinned
 * staging), since a selection usually changes from call to call.
 * Workspace and metadata as for pic_attend: calls on one plan from several
 * streams may overlap.
 */
pic_status pic_attend_boundary(pic_plan_t *plan, const pic_kv_view *pool, const pic_kv_view *cache,
                               const pic_attend_boundary_args *args, void *stream);

/* pic_plan_info -- sizes and algorithmic byte counts of a plan.  Host only.
 * The attention counts (attend_blocks, attend_block_tokens) need the plan's
 * attention map: the first call builds it if no attention call has. */
pic_status pic_plan_info(const pic_plan_t *plan, pic_plan_info_t *info);

/*
 * pic_plan_ranges -- chunk boundaries and recompute ranges, entry by entry
 * in request order (EPIC Guide, the chunk boundaries a LegoLink pass
 * consumes; Irminsul section 2.2, the recompute carve-out).  Either output
 * may be NULL; each must hold n_entries rows:
 *   boundaries[e] = {request, dst_offset, dst_offset + length}
 *   recompute[e]  = {request, dst_offset, dst_offset + recompute_k}
 */
pic_status pic_plan_ranges(const pic_plan_t *plan, int64_t *boundaries, int64_t *recompute);

/* pic_plan_destroy -- wait for the work enqueued with the plan (its last
 * use on every stream it ran on, and its uploads; not the whole device),
 * then release it and its device memory.  NULL is a no-op. */
void pic_plan_destroy(pic_plan_t *plan);

/* ------------------------------------------------------------------------
 * Content-defined chunking of a token stream and the chunk registry: how a
 * request's prompt is cut into chunks whose caches can be found again
 * (Irminsul, Technical Summary, "Content-Hash Keying with CDC" and the S1
 * "detect and recover" strategy; EPIC Guide, the content hash registry of
 * the serving runtime, SHA-256 keyed).
 *
 * Definitions (every one of them is computed on the GPU by pic_match):
 *   G(t)   = xxHash64 of token t's 4 little-endian bytes, seed gear_seed
 *            (the Gear value of a token; the pages give no Gear table);
 *   h_i    = 2 h_{i-1} + G(t_i) mod 2^64, h_{-1} = 0: a rolling hash whose
 *            value depends on tokens i-63 .. i only (a 64-token window);
 *   a chunk ends after token i when h_i < threshold, and at the stream end;
 *   fingerprint of tokens [s, s+len) = SHA-256 of their little-endian int32
 *            bytes, or their xxHash64 (seed fp_seed) as 8 little-endian bytes
 *            followed by 24 zero bytes;
 *   a segment is registered when the registry holds an entry with the
 *            same fingerprint and the same length.
 * ------------------------------------------------------------------------ */
enum { PIC_FP_XXH64 = 0, PIC_FP_SHA256 = 1 };

typedef struct pic_cdc_config {
    uint64_t threshold;   /* chunk ends after token i when h_i < threshold; the mean chunk
                             length of random text is about 2^64 / threshold */
    uint64_t gear_seed;   /* seed of the Gear values */
    uint64_t fp_seed;     /* xxHash64 seed of the fingerprints (unused for SHA-256) */
    int32_t fingerprint;  /* PIC_FP_XXH64 | PIC_FP_SHA256 */
    int32_t window;       /* fallback window (Irminsul S1: 128 tokens); 0 = no fallback */
} pic_cdc_config;

/* One segment of a stream.  level 0: a content-defined chunk; level 1: a
 * window of a chunk the registry does not hold (consecutive windows of
 * `window` tokens from the chunk start, the last one shorter). */
typedef struct pic_match_t {
    int64_t start;      /* first token */
    int32_t length;
    int32_t level;
    int32_t chunk_id;   /* id of the registered entry, -1: not registered */
    int32_t reserved;
    uint8_t fp[32];     /* fingerprint */
} pic_match_t;

typedef struct pic_registry pic_registry_t;

/* pic_registry_create -- an empty registry for one fingerprint kind. */
pic_status pic_registry_create(int32_t fingerprint, pic_registry_t **out);

/* pic_registry_add -- register a segment (host call; fp is 32 host bytes).
 * length >= 1, chunk_id >= 0 (PIC_ERR_RANGE); an entry with the same
 * fingerprint and length is refused (PIC_ERR_OVERLAP).  The next pic_match
 * uploads a new version of the registry's device table, ordered on its
 * stream; earlier pic_match calls on any stream keep reading the version
 * they were given, which is freed once they have run (no call waits for the
 * device).  A registry is bound to the device of its first pic_match
 * (PIC_ERR_STATE after).
 * Adding while a pic_match runs on another host thread is serialised by the
 * registry's lock. */
pic_status pic_registry_add(pic_registry_t *reg, const uint8_t *fp, int32_t length,
                            int32_t chunk_id);

/* pic_registry_destroy -- wait for the pic_match calls that read the
 * registry's tables, release it and its per-stream temporaries.  NULL is a
 * no-op. */
void pic_registry_destroy(pic_registry_t *reg);

/*
 * pic_match -- cut tokens[0, n_tokens) (device, int32) into content-defined
 * chunks, fingerprint every chunk and look it up in `reg` (NULL: an empty
 * registry).  A chunk that is not registered is replaced, when window > 0,
 * by its windows, each fingerprinted and looked up.  The segments, in
 * stream order, tile the stream; the first max_out are written to `out`
 * (device, max_out records) and their total count to *n_out (device int64),
 * so a count above max_out means the output was cut short (a stream of n
 * tokens never yields more than n segments).
 * n_tokens in [0, 2^31) and window >= 0 and max_out >= 0 (PIC_ERR_RANGE);
 * tokens (when n_tokens > 0), out (when max_out > 0) and n_out non-NULL
 * (PIC_ERR_INVALID_ARG); tokens 4-byte, out and n_out 8-byte aligned
 * (PIC_ERR_ALIGN).  The registry's fingerprint kind must equal
 * cfg->fingerprint (PIC_ERR_INVALID_ARG).
 * Work is enqueued on `stream` and the call does not wait for it: counts
 * stay on the device.  Temporaries take about 8 bytes per token plus 36
 * bytes per kept record (min(n_tokens, max_out)) of device memory: with a
 * registry, from a buffer the registry keeps per stream until
 * pic_registry_destroy (replaced by a larger one when a call needs more;
 * a stream handle is taken to name one stream for the registry's life);
 * without one, allocated and freed on `stream` (stream-ordered).
 */
pic_status pic_match(pic_registry_t *reg, const pic_cdc_config *cfg, const int32_t *tokens,
                     int64_t n_tokens, pic_match_t *out, int64_t max_out, int64_t *n_out,
                     void *stream);

/*
 * pic_stream_copy -- the measurement reference of the library, not a step
 * of the method: copy nbytes from src to dst (device memory, 16-byte
 * aligned, nbytes a multiple of 16, else PIC_ERR_ALIGN; overlapping buffers
 * PIC_ERR_OVERLAP; NULL pointers PIC_ERR_INVALID_ARG; nbytes < 0
 * PIC_ERR_RANGE) with the 16-byte non-temporal loads and stores the stitch
 * kernel uses, every byte read once and written once.  Its rate is the
 * practical HBM ceiling of a 1:1 read/write stream, against which the
 * stitch's rate is read.  Enqueued on `stream`; nothing is allocated.
 */
pic_status pic_stream_copy(void *dst, const void *src, int64_t nbytes, void *stream);

/* Thread-local message for the last failed call on this thread ("" if none). */
const char *pic_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PIC_STITCH_H */
