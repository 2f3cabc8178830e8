/*
 * pic_oracle.c -- plain, slow, fp64 reference for position-independent KV
 * chunk stitching.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check
 * and the benchmark's CPU-baseline leg may load or call this library.  It
 * shares no code, header, table or constant with the HIP library it checks,
 * and it includes nothing from it.
 *
 * What is computed, and where the pages state it:
 *
 *  - RoPE on one 2-D plane i (EPIC Guide, "Mathematical Foundations",
 *    section 1 "RoPE Mathematical Structure"): the pair (x, y) at angle phi
 *    becomes (x cos phi - y sin phi, x sin phi + y cos phi), and the
 *    frequency of plane i is theta_i = b^(-2i/d), b the RoPE base, d the
 *    number of rotated dimensions.
 *
 *  - Relocation by a shift (same page, section 2 "The In-Place Shift
 *    Transformation"; Irminsul, Technical Summary section 2.2, the
 *    delta-rotation rule): rotation angles add, so a key cached at position
 *    n and moved by delta = p_target - p_source is the cached key rotated by
 *    delta * theta_i on every plane.  delta is one constant per chunk.
 *
 *  - Values are never rotated (EPIC Guide, section 2, the note that RoPE is
 *    not applied to V), and in the MLA row only the 64-dim rotary slice k_r
 *    is rotated while the 512-dim content latent cKV is reused verbatim
 *    (Irminsul, Technical Summary section 2.1).
 *
 *  - Chunks are cached at virtual offset 0 and placed at arbitrary logical
 *    offsets of a request, into a contiguous or a paged KV cache (EPIC
 *    Guide, "Algorithmic Architecture: The EPIC Serving Runtime", the
 *    virtual block mapping and the modular prompt composer).
 *
 *  - The first recompute_k tokens of each placed chunk are not written:
 *    a recompute pass overwrites them (Irminsul section 2.2, first-chunk
 *    carve-out; EPIC Guide, LegoLink).
 *
 * Readings taken where the pages are silent (each is listed with its
 * reason in the design notes of the repository):
 *  - pairing: "half" pairs (i, i + R/2), "interleaved" pairs (2i, 2i+1);
 *    plane i uses theta_i in both;
 *  - arithmetic: angles, cos/sin and the rotation in fp64 (libm), then one
 *    round-to-nearest-even into the storage type;
 *  - delta == 0 copies the row bits unchanged (R(0) is the identity);
 *  - destination rows not written keep their prior contents.
 *
 * Layouts are dense and row-major (elements):
 *   pool       [n_layers][pool_tokens][n_heads][row_dim], or, paged,
 *              [n_layers][src_num_pages][src_page_size][n_heads][row_dim]
 *   contiguous [n_layers][n_requests][capacity][n_heads][row_dim]
 *   paged      [n_layers][n_phys_pages][page_size][n_heads][row_dim]
 *   in-place   [n_layers][n_tokens][n_heads][row_dim]
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (see build.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* storage types of the oracle (its own numbering) */
#define ORC_F32 0
#define ORC_BF16 1
#define ORC_F64 2 /* oracle-only: lets the self-checks run without rounding */

/* pairing of the rotated dimensions */
#define ORC_HALF 0
#define ORC_INTERLEAVED 1

/* results */
#define ORC_OK 0
#define ORC_BAD_ARG 1 /* malformed shape, rope config or layer range */
#define ORC_RANGE 2   /* an index or a length outside what it refers to */
#define ORC_OVERLAP 3 /* two placements claim the same position or row */

typedef struct {
    int32_t dtype, n_layers, n_heads, row_dim, rope_offset, rope_dim, style, has_v;
    double theta;
    const double *inv_freq; /* optional, rope_dim/2 values; NULL = theta formula */
    int64_t pool_tokens;
    int32_t src_page_size;      /* 0 = contiguous pool */
    int64_t src_num_pages;      /* paged pool: pages in the pool */
    const int32_t *chunk_pages; /* paged pool: pages per chunk */
    const int32_t *chunk_page_table; /* paged pool: tables listed chunk by chunk */
    int32_t n_chunks;
    const int64_t *chunk_start; /* contiguous: first pool row; paged: offset in its pages */
    const int64_t *chunk_base;  /* position the chunk's keys were cached at */
    const int32_t *chunk_len;
    int32_t n_requests;
    const int32_t *req_entries; /* entries per request, listed request by request */
    const int32_t *ent_chunk;
    const int64_t *ent_dst; /* logical position of the entry's first token */
    const int32_t *ent_len;
    const int32_t *ent_k;    /* recompute_k */
    int32_t page_size;       /* 0 = contiguous destination */
    int64_t capacity;        /* contiguous: positions per request */
    int64_t n_phys_pages;    /* paged: pages in the destination pool */
    const int32_t *req_pages; /* paged: logical pages per request */
    const int32_t *page_table; /* paged: tables listed request by request */
} orc_stitch_problem;

typedef struct {
    int32_t dtype, n_layers, n_heads, row_dim, rope_offset, rope_dim, style, pad_;
    double theta;
    const double *inv_freq;
    int64_t n_tokens;
    int32_t n_segments, pad2_;
    const int64_t *seg_start;
    const int64_t *seg_delta;
    const int32_t *seg_len;
    const int32_t *seg_k;
} orc_inplace_problem;

/* ---------------------------------------------------------------- values */

static size_t orc_elem_size(int dtype)
{
    if (dtype == ORC_F32) return 4;
    if (dtype == ORC_BF16) return 2;
    return 8;
}

/* bf16 is the upper half of an IEEE binary32: widening is exact. */
static double orc_bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * One rounding from double to bf16, to nearest, ties to even.  bf16 keeps 8
 * significant bits and the binary32 exponent range (subnormal quantum
 * 2^-133).  The value is scaled so that one bf16 quantum is 1, rounded to an
 * integer with nearbyint (ties to even in the default rounding mode), and
 * scaled back; every step but the rounding is exact.
 */
uint16_t orc_round_bf16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return (uint16_t)(sign | 0x7FC0u);
    double ax = fabs(x);
    if (isinf(ax)) return (uint16_t)(sign | 0x7F80u);
    if (ax == 0.0) return sign;
    int e;
    frexp(ax, &e); /* ax = m * 2^e with m in [0.5, 1) */
    int lead = e - 1; /* exponent of the leading bit */
    if (lead < -126) lead = -126;
    double quantum = ldexp(1.0, lead - 7);
    double y = nearbyint(ax / quantum) * quantum;
    const double bf16_max = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
    if (y > bf16_max) return (uint16_t)(sign | 0x7F80u);
    float f = (float)y; /* exact: y has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)(u >> 16));
}

static double orc_load(const void *base, int dtype, int64_t i)
{
    if (dtype == ORC_F32) return (double)((const float *)base)[i];
    if (dtype == ORC_BF16) return orc_bf16_to_double(((const uint16_t *)base)[i]);
    return ((const double *)base)[i];
}

static void orc_store(void *base, int dtype, int64_t i, double x)
{
    if (dtype == ORC_F32) ((float *)base)[i] = (float)x; /* RNE */
    else if (dtype == ORC_BF16) ((uint16_t *)base)[i] = orc_round_bf16(x);
    else ((double *)base)[i] = x;
}

/* ------------------------------------------------------------------ rope */

/* theta_i = b^(-2i/d) (EPIC Guide, section 1), unless the caller gives a table. */
double orc_inv_freq(double theta, int rope_dim, int i)
{
    return pow(theta, -(2.0 * (double)i) / (double)rope_dim);
}

/* indices, inside the row, of the two members of plane i */
static void orc_pair(int style, int rope_offset, int rope_dim, int i, int *a, int *b)
{
    if (style == ORC_HALF) {
        *a = rope_offset + i;
        *b = rope_offset + i + rope_dim / 2;
    } else {
        *a = rope_offset + 2 * i;
        *b = rope_offset + 2 * i + 1;
    }
}

/* cos/sin of delta * theta_i for every plane, in fp64 */
static void orc_shift_table(double theta, const double *inv_freq, int rope_dim, int64_t delta,
                            double *c, double *s)
{
    for (int i = 0; i < rope_dim / 2; i++) {
        double f = inv_freq ? inv_freq[i] : orc_inv_freq(theta, rope_dim, i);
        double phi = (double)delta * f;
        c[i] = cos(phi);
        s[i] = sin(phi);
    }
}

/*
 * Rotate the rotary slice of one head row (element index `row` of its first
 * element) of `src` by the table (c, s) and store into `dst` at `drow`.
 */
static void orc_rotate_row(const void *src, int64_t row, void *dst, int64_t drow, int dtype,
                           int style, int rope_offset, int rope_dim, const double *c,
                           const double *s)
{
    for (int i = 0; i < rope_dim / 2; i++) {
        int a, b;
        orc_pair(style, rope_offset, rope_dim, i, &a, &b);
        double x = orc_load(src, dtype, row + a);
        double y = orc_load(src, dtype, row + b);
        double xr = x * c[i] - y * s[i];
        double yr = x * s[i] + y * c[i];
        orc_store(dst, dtype, drow + a, xr);
        orc_store(dst, dtype, drow + b, yr);
    }
}

/* ------------------------------------------------------------ validation */

static int orc_check_shape(int dtype, int n_layers, int n_heads, int row_dim, int rope_offset,
                           int rope_dim, int style, double theta, const double *inv_freq,
                           int layer_begin, int layer_end)
{
    if (dtype != ORC_F32 && dtype != ORC_BF16 && dtype != ORC_F64) return ORC_BAD_ARG;
    if (style != ORC_HALF && style != ORC_INTERLEAVED) return ORC_BAD_ARG;
    if (n_layers < 1 || n_heads < 1 || row_dim < 1) return ORC_BAD_ARG;
    if (rope_dim < 2 || rope_dim % 2 != 0) return ORC_BAD_ARG;
    if (rope_offset < 0 || rope_offset + rope_dim > row_dim) return ORC_BAD_ARG;
    if (!inv_freq && !(theta > 0.0)) return ORC_BAD_ARG;
    if (layer_begin < 0 || layer_begin > layer_end || layer_end > n_layers) return ORC_BAD_ARG;
    return ORC_OK;
}

/* paged pool: physical page holding offset `at` of chunk c's page list */
static int32_t orc_src_page(const orc_stitch_problem *p, int c, int64_t at)
{
    int64_t first = 0;
    for (int i = 0; i < c; i++) first += p->chunk_pages[i];
    return p->chunk_page_table[first + at / p->src_page_size];
}

/* pool row (within a layer) of token t of chunk c */
static int64_t orc_src_row(const orc_stitch_problem *p, int c, int64_t t)
{
    if (p->src_page_size == 0) return p->chunk_start[c] + t;
    int64_t at = p->chunk_start[c] + t;
    return (int64_t)orc_src_page(p, c, at) * p->src_page_size + at % p->src_page_size;
}

/*
 * A problem is valid when every chunk lies in the pool, every entry names
 * an existing chunk, places 1..chunk_len of its tokens with 0 <= k <= length
 * at a position >= 0 that fits its request, the pages it writes exist, no
 * two entries of a request cover the same logical position, and no
 * destination row is written twice.  Overlaps are found by brute force:
 * every claimed position and every written row is marked in a map.
 */
int orc_validate_stitch(const orc_stitch_problem *p, int layer_begin, int layer_end)
{
    int st = orc_check_shape(p->dtype, p->n_layers, p->n_heads, p->row_dim, p->rope_offset,
                             p->rope_dim, p->style, p->theta, p->inv_freq, layer_begin,
                             layer_end);
    if (st) return st;
    if (p->has_v != 0 && p->has_v != 1) return ORC_BAD_ARG;
    if (p->pool_tokens < 0 || p->n_chunks < 0 || p->n_requests < 0) return ORC_BAD_ARG;
    if (p->page_size < 0 || p->src_page_size < 0) return ORC_BAD_ARG;
    if (p->src_page_size > 0 && p->src_num_pages < 0) return ORC_BAD_ARG;
    if (p->src_page_size > 0)
        for (int c = 0; c < p->n_chunks; c++)
            if (p->chunk_pages[c] < 0) return ORC_BAD_ARG;
    if (p->page_size == 0 && p->capacity < 0) return ORC_BAD_ARG;
    if (p->page_size > 0 && p->n_phys_pages < 0) return ORC_BAD_ARG;
    for (int r = 0; r < p->n_requests; r++) {
        if (p->req_entries[r] < 0) return ORC_BAD_ARG;
        if (p->page_size > 0 && p->req_pages[r] < 0) return ORC_BAD_ARG;
    }

    for (int c = 0; c < p->n_chunks; c++) {
        if (p->chunk_start[c] < 0 || p->chunk_len[c] < 1) return ORC_RANGE;
        /* |base_pos| <= 2^62: delta = dst - base_pos stays inside int64 */
        if (p->chunk_base[c] < -((int64_t)1 << 62) || p->chunk_base[c] > ((int64_t)1 << 62))
            return ORC_RANGE;
        int64_t room = p->src_page_size > 0 ? (int64_t)p->chunk_pages[c] * p->src_page_size
                                            : p->pool_tokens;
        if (p->chunk_start[c] + p->chunk_len[c] > room) return ORC_RANGE;
    }
    int64_t e0 = 0, pt0 = 0;
    for (int r = 0; r < p->n_requests; r++) {
        int64_t span = p->page_size > 0 ? (int64_t)p->req_pages[r] * p->page_size : p->capacity;
        for (int j = 0; j < p->req_entries[r]; j++) {
            int64_t e = e0 + j;
            int32_t c = p->ent_chunk[e];
            if (c < 0 || c >= p->n_chunks) return ORC_RANGE;
            if (p->ent_len[e] < 1 || p->ent_len[e] > p->chunk_len[c]) return ORC_RANGE;
            if (p->ent_k[e] < 0 || p->ent_k[e] > p->ent_len[e]) return ORC_RANGE;
            if (p->ent_dst[e] < 0 || p->ent_dst[e] + p->ent_len[e] > span) return ORC_RANGE;
            if (p->ent_dst[e] + p->ent_len[e] > 2147483647) return ORC_RANGE; /* positions < 2^31 */
            if (p->page_size > 0) {
                for (int t = p->ent_k[e]; t < p->ent_len[e]; t++) {
                    int64_t pos = p->ent_dst[e] + t;
                    int32_t page = p->page_table[pt0 + pos / p->page_size];
                    if (page < 0 || page >= p->n_phys_pages) return ORC_RANGE;
                }
            }
            if (p->src_page_size > 0) {
                for (int t = p->ent_k[e]; t < p->ent_len[e]; t++) {
                    int32_t page = orc_src_page(p, c, p->chunk_start[c] + t);
                    if (page < 0 || page >= p->src_num_pages) return ORC_RANGE;
                }
            }
        }
        e0 += p->req_entries[r];
        if (p->page_size > 0) pt0 += p->req_pages[r];
    }

    /* logical overlap inside each request (whole entry intervals) */
    e0 = 0;
    for (int r = 0; r < p->n_requests; r++) {
        int64_t span = p->page_size > 0 ? (int64_t)p->req_pages[r] * p->page_size : p->capacity;
        unsigned char *seen = calloc((size_t)(span > 0 ? span : 1), 1);
        if (!seen) return ORC_BAD_ARG;
        for (int j = 0; j < p->req_entries[r]; j++) {
            int64_t e = e0 + j;
            for (int t = 0; t < p->ent_len[e]; t++) {
                int64_t pos = p->ent_dst[e] + t;
                if (seen[pos]) {
                    free(seen);
                    return ORC_OVERLAP;
                }
                seen[pos] = 1;
            }
        }
        free(seen);
        e0 += p->req_entries[r];
    }

    /* physical overlap of written rows across requests (paged) */
    if (p->page_size > 0) {
        int64_t rows = p->n_phys_pages * p->page_size;
        unsigned char *written = calloc((size_t)(rows > 0 ? rows : 1), 1);
        if (!written) return ORC_BAD_ARG;
        e0 = 0;
        pt0 = 0;
        for (int r = 0; r < p->n_requests; r++) {
            for (int j = 0; j < p->req_entries[r]; j++) {
                int64_t e = e0 + j;
                for (int t = p->ent_k[e]; t < p->ent_len[e]; t++) {
                    int64_t pos = p->ent_dst[e] + t;
                    int64_t page = p->page_table[pt0 + pos / p->page_size];
                    int64_t row = page * p->page_size + pos % p->page_size;
                    if (written[row]) {
                        free(written);
                        return ORC_OVERLAP;
                    }
                    written[row] = 1;
                }
            }
            e0 += p->req_entries[r];
            pt0 += p->req_pages[r];
        }
        free(written);
    }
    return ORC_OK;
}

int orc_validate_inplace(const orc_inplace_problem *p, int layer_begin, int layer_end)
{
    int st = orc_check_shape(p->dtype, p->n_layers, p->n_heads, p->row_dim, p->rope_offset,
                             p->rope_dim, p->style, p->theta, p->inv_freq, layer_begin,
                             layer_end);
    if (st) return st;
    if (p->n_tokens < 0 || p->n_segments < 0) return ORC_BAD_ARG;
    for (int g = 0; g < p->n_segments; g++) {
        if (p->seg_start[g] < 0 || p->seg_len[g] < 1) return ORC_RANGE;
        if (p->seg_start[g] + p->seg_len[g] > p->n_tokens) return ORC_RANGE;
        if (p->seg_k[g] < 0 || p->seg_k[g] > p->seg_len[g]) return ORC_RANGE;
    }
    unsigned char *seen = calloc((size_t)(p->n_tokens > 0 ? p->n_tokens : 1), 1);
    if (!seen) return ORC_BAD_ARG;
    for (int g = 0; g < p->n_segments; g++) {
        for (int64_t t = 0; t < p->seg_len[g]; t++) {
            if (seen[p->seg_start[g] + t]) {
                free(seen);
                return ORC_OVERLAP;
            }
            seen[p->seg_start[g] + t] = 1;
        }
    }
    free(seen);
    return ORC_OK;
}

/* ----------------------------------------------------------------- stitch */

/*
 * Stitch layers [layer_begin, layer_end): for every request and entry, the
 * tokens t in [k, length) of the entry's chunk are written at logical
 * position dst + t: the V row and the non-rotary part of the K row as
 * copies, the rotary slice of K rotated by delta = dst - base_pos.
 * Nothing is written unless the whole problem is valid.
 */
int orc_stitch(const orc_stitch_problem *p, const void *pool_k, const void *pool_v, void *dst_k,
               void *dst_v, int layer_begin, int layer_end)
{
    int st = orc_validate_stitch(p, layer_begin, layer_end);
    if (st) return st;

    const int64_t row = (int64_t)p->n_heads * p->row_dim; /* elements per token */
    const size_t es = orc_elem_size(p->dtype);
    const int npairs = p->rope_dim / 2;
    double *c = malloc(sizeof(double) * (size_t)npairs);
    double *s = malloc(sizeof(double) * (size_t)npairs);
    if (!c || !s) {
        free(c);
        free(s);
        return ORC_BAD_ARG;
    }
    const int64_t dst_rows_per_layer = p->page_size > 0
                                           ? p->n_phys_pages * p->page_size
                                           : (int64_t)p->n_requests * p->capacity;
    const int64_t src_rows_per_layer =
        p->src_page_size > 0 ? p->src_num_pages * p->src_page_size : p->pool_tokens;

    for (int layer = layer_begin; layer < layer_end; layer++) {
        int64_t e0 = 0, pt0 = 0;
        for (int r = 0; r < p->n_requests; r++) {
            for (int j = 0; j < p->req_entries[r]; j++) {
                int64_t e = e0 + j;
                int32_t ch = p->ent_chunk[e];
                int64_t delta = p->ent_dst[e] - p->chunk_base[ch];
                if (delta != 0)
                    orc_shift_table(p->theta, p->inv_freq, p->rope_dim, delta, c, s);
                for (int t = p->ent_k[e]; t < p->ent_len[e]; t++) {
                    int64_t src_tok = orc_src_row(p, ch, t);
                    int64_t pos = p->ent_dst[e] + t;
                    int64_t dst_tok; /* destination row within the layer */
                    if (p->page_size > 0) {
                        int64_t page = p->page_table[pt0 + pos / p->page_size];
                        dst_tok = page * p->page_size + pos % p->page_size;
                    } else {
                        dst_tok = (int64_t)r * p->capacity + pos;
                    }
                    int64_t src_off = ((int64_t)layer * src_rows_per_layer + src_tok) * row;
                    int64_t dst_off = ((int64_t)layer * dst_rows_per_layer + dst_tok) * row;
                    /* values and the K row: bit copies */
                    if (p->has_v)
                        memcpy((char *)dst_v + dst_off * es,
                               (const char *)pool_v + src_off * es, (size_t)row * es);
                    memcpy((char *)dst_k + dst_off * es, (const char *)pool_k + src_off * es,
                           (size_t)row * es);
                    /* the rotary slice of every head, rotated by delta */
                    if (delta != 0) {
                        for (int h = 0; h < p->n_heads; h++) {
                            int64_t hoff = (int64_t)h * p->row_dim;
                            orc_rotate_row(pool_k, src_off + hoff, dst_k, dst_off + hoff,
                                           p->dtype, p->style, p->rope_offset, p->rope_dim, c,
                                           s);
                        }
                    }
                }
            }
            e0 += p->req_entries[r];
            if (p->page_size > 0) pt0 += p->req_pages[r];
        }
    }
    free(c);
    free(s);
    return ORC_OK;
}

/*
 * Rotate, in place, the rotary slice of K for tokens [k, length) of every
 * segment by the segment's delta (EPIC Guide, section 2: keys are shifted
 * in place, values untouched).  Nothing is written unless the problem is
 * valid.
 */
int orc_rotate_inplace(const orc_inplace_problem *p, void *buf_k, int layer_begin, int layer_end)
{
    int st = orc_validate_inplace(p, layer_begin, layer_end);
    if (st) return st;
    const int64_t row = (int64_t)p->n_heads * p->row_dim;
    const int npairs = p->rope_dim / 2;
    double *c = malloc(sizeof(double) * (size_t)npairs);
    double *s = malloc(sizeof(double) * (size_t)npairs);
    if (!c || !s) {
        free(c);
        free(s);
        return ORC_BAD_ARG;
    }
    for (int layer = layer_begin; layer < layer_end; layer++) {
        for (int g = 0; g < p->n_segments; g++) {
            if (p->seg_delta[g] == 0) continue; /* R(0) is the identity */
            orc_shift_table(p->theta, p->inv_freq, p->rope_dim, p->seg_delta[g], c, s);
            for (int t = p->seg_k[g]; t < p->seg_len[g]; t++) {
                int64_t off = ((int64_t)layer * p->n_tokens + p->seg_start[g] + t) * row;
                for (int h = 0; h < p->n_heads; h++) {
                    int64_t hoff = off + (int64_t)h * p->row_dim;
                    orc_rotate_row(buf_k, hoff, buf_k, hoff, p->dtype, p->style,
                                   p->rope_offset, p->rope_dim, c, s);
                }
            }
        }
    }
    free(c);
    free(s);
    return ORC_OK;
}

/* vector helper for the self-checks: round n doubles to bf16 bit patterns */
void orc_round_bf16_array(const double *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++) out[i] = orc_round_bf16(x[i]);
}
