/*
 * cdc_oracle.c -- plain reference for content-defined chunking of a token
 * stream, chunk fingerprints and the chunk-registry lookup.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check
 * and the benchmark's CPU-baseline leg may load or call this library.  It
 * shares no code, header, table or constant with the HIP library it checks.
 *
 * What is computed, and where the pages state it:
 *
 *  - Content-defined chunking (Irminsul: MLA-Native Position-Independent
 *    Caching for Agentic LLM Serving, Technical Summary, "Content-Hash
 *    Keying with CDC"): a rolling Gear hash over 64-token windows; a chunk
 *    ends where the hash falls below a threshold, so boundaries follow the
 *    content rather than fixed offsets.
 *  - Each chunk is fingerprinted with xxHash64 (same section); the EPIC
 *    runtime keys its chunk registry by SHA-256 (EPIC Guide: Position-
 *    Independent Caching for LLM Serving, "Algorithmic Architecture: The
 *    EPIC Serving Runtime", the content hash registry and section 1).
 *  - A chunk the registry does not hold is split into fixed 128-token
 *    windows that are looked up again (Irminsul, the S1 "detect and
 *    recover" strategy).
 *
 * Readings taken where the pages are silent:
 *  - the Gear value of a token is the xxHash64 of its 4 little-endian bytes
 *    under a gear seed (the pages give no Gear table);
 *  - the rolling hash is h_i = 2 h_{i-1} + G(t_i) mod 2^64 with h_{-1} = 0,
 *    so h_i depends on tokens i-63 .. i only: a 64-token window;
 *  - a chunk ends after token i when h_i < threshold, and at the end of the
 *    stream; there is no minimum or maximum length;
 *  - fingerprints hash the chunk's token ids as little-endian int32 bytes; a
 *    fingerprint is 32 bytes (SHA-256), or the 8 little-endian bytes of the
 *    xxHash64 value followed by 24 zero bytes;
 *  - a registry hit needs an equal fingerprint and an equal length;
 *  - with fallback window W > 0 a missed chunk becomes consecutive windows
 *    of W tokens from its start, the last one shorter if W does not divide
 *    its length, and each window is looked up; with W = 0 the chunk stays
 *    one missed segment.
 *
 * xxHash64 and SHA-256 follow their published specifications (Y. Collet's
 * xxHash specification; FIPS 180-4).  The SHA-256 round constants and
 * initial state are computed here from their definitions (fractional parts
 * of cube and square roots of the first primes), not copied.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------ xxHash64 */

static const uint64_t XP1 = 0x9E3779B185EBCA87ull;
static const uint64_t XP2 = 0xC2B2AE3D27D4EB4Full;
static const uint64_t XP3 = 0x165667B19E3779F9ull;
static const uint64_t XP4 = 0x85EBCA77C2B2AE63ull;
static const uint64_t XP5 = 0x27D4EB2F165667C5ull;

static uint64_t rotl64(uint64_t x, int r) { return (x << r) | (x >> (64 - r)); }

static uint64_t read_le64(const uint8_t *p)
{
    uint64_t v = 0;
    for (int i = 7; i >= 0; i--) v = (v << 8) | p[i];
    return v;
}

static uint32_t read_le32(const uint8_t *p)
{
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) |
           ((uint32_t)p[3] << 24);
}

/* one accumulator step: add input * P2, rotate by 31, multiply by P1 */
static uint64_t xxh_round(uint64_t acc, uint64_t input)
{
    acc += input * XP2;
    acc = rotl64(acc, 31);
    return acc * XP1;
}

static uint64_t xxh_merge(uint64_t h, uint64_t acc)
{
    h ^= xxh_round(0, acc);
    return h * XP1 + XP4;
}

uint64_t orc_xxh64(const uint8_t *p, int64_t len, uint64_t seed)
{
    const uint8_t *end = p + len;
    uint64_t h;
    if (len >= 32) {
        uint64_t v1 = seed + XP1 + XP2, v2 = seed + XP2, v3 = seed, v4 = seed - XP1;
        while (end - p >= 32) { /* 32-byte stripes, four lanes */
            v1 = xxh_round(v1, read_le64(p));
            v2 = xxh_round(v2, read_le64(p + 8));
            v3 = xxh_round(v3, read_le64(p + 16));
            v4 = xxh_round(v4, read_le64(p + 24));
            p += 32;
        }
        h = rotl64(v1, 1) + rotl64(v2, 7) + rotl64(v3, 12) + rotl64(v4, 18);
        h = xxh_merge(h, v1);
        h = xxh_merge(h, v2);
        h = xxh_merge(h, v3);
        h = xxh_merge(h, v4);
    } else {
        h = seed + XP5;
    }
    h += (uint64_t)len;
    while (end - p >= 8) {
        h ^= xxh_round(0, read_le64(p));
        h = rotl64(h, 27) * XP1 + XP4;
        p += 8;
    }
    if (end - p >= 4) {
        h ^= (uint64_t)read_le32(p) * XP1;
        h = rotl64(h, 23) * XP2 + XP3;
        p += 4;
    }
    while (p < end) {
        h ^= (uint64_t)(*p) * XP5;
        h = rotl64(h, 11) * XP1;
        p++;
    }
    /* final avalanche */
    h ^= h >> 33;
    h *= XP2;
    h ^= h >> 29;
    h *= XP3;
    h ^= h >> 32;
    return h;
}

/* ------------------------------------------------------------- SHA-256 */

static uint32_t SK[64], SH0[8];
static int sha_ready = 0;

static int is_prime(int n)
{
    if (n < 2) return 0;
    for (int d = 2; d * d <= n; d++)
        if (n % d == 0) return 0;
    return 1;
}

/* first 32 bits of the fractional part of x */
static uint32_t frac32(long double x)
{
    long double f = x - floorl(x);
    return (uint32_t)floorl(f * 4294967296.0L);
}

static void sha_init_constants(void)
{
    int n = 0;
    for (int p = 2; n < 64; p++) {
        if (!is_prime(p)) continue;
        if (n < 8) SH0[n] = frac32(sqrtl((long double)p));
        SK[n] = frac32(cbrtl((long double)p));
        n++;
    }
    sha_ready = 1;
}

static uint32_t rotr32(uint32_t x, int r) { return (x >> r) | (x << (32 - r)); }

static void sha_block(uint32_t st[8], const uint8_t *blk)
{
    uint32_t w[64];
    for (int t = 0; t < 16; t++)
        w[t] = ((uint32_t)blk[4 * t] << 24) | ((uint32_t)blk[4 * t + 1] << 16) |
               ((uint32_t)blk[4 * t + 2] << 8) | (uint32_t)blk[4 * t + 3];
    for (int t = 16; t < 64; t++) {
        uint32_t s0 = rotr32(w[t - 15], 7) ^ rotr32(w[t - 15], 18) ^ (w[t - 15] >> 3);
        uint32_t s1 = rotr32(w[t - 2], 17) ^ rotr32(w[t - 2], 19) ^ (w[t - 2] >> 10);
        w[t] = w[t - 16] + s0 + w[t - 7] + s1;
    }
    uint32_t a = st[0], b = st[1], c = st[2], d = st[3], e = st[4], f = st[5], g = st[6],
             h = st[7];
    for (int t = 0; t < 64; t++) {
        uint32_t S1 = rotr32(e, 6) ^ rotr32(e, 11) ^ rotr32(e, 25);
        uint32_t ch = (e & f) ^ (~e & g);
        uint32_t T1 = h + S1 + ch + SK[t] + w[t];
        uint32_t S0 = rotr32(a, 2) ^ rotr32(a, 13) ^ rotr32(a, 22);
        uint32_t maj = (a & b) ^ (a & c) ^ (b & c);
        uint32_t T2 = S0 + maj;
        h = g;
        g = f;
        f = e;
        e = d + T1;
        d = c;
        c = b;
        b = a;
        a = T1 + T2;
    }
    st[0] += a;
    st[1] += b;
    st[2] += c;
    st[3] += d;
    st[4] += e;
    st[5] += f;
    st[6] += g;
    st[7] += h;
}

void orc_sha256(const uint8_t *p, int64_t len, uint8_t out[32])
{
    if (!sha_ready) sha_init_constants();
    uint32_t st[8];
    memcpy(st, SH0, sizeof(st));
    int64_t i = 0;
    for (; i + 64 <= len; i += 64) sha_block(st, p + i);
    /* padding: 0x80, zeros, then the bit length big-endian in the last 8 bytes */
    uint8_t tail[128];
    memset(tail, 0, sizeof(tail));
    int64_t rem = len - i;
    memcpy(tail, p + i, (size_t)rem);
    tail[rem] = 0x80;
    int64_t tl = rem + 1 + 8 <= 64 ? 64 : 128;
    uint64_t bits = (uint64_t)len * 8u;
    for (int k = 0; k < 8; k++) tail[tl - 1 - k] = (uint8_t)(bits >> (8 * k));
    for (int64_t o = 0; o < tl; o += 64) sha_block(st, tail + o);
    for (int k = 0; k < 8; k++) {
        out[4 * k] = (uint8_t)(st[k] >> 24);
        out[4 * k + 1] = (uint8_t)(st[k] >> 16);
        out[4 * k + 2] = (uint8_t)(st[k] >> 8);
        out[4 * k + 3] = (uint8_t)st[k];
    }
}

/* ------------------------------------------------------- chunking, lookup */

enum { ORC_FP_XXH64 = 0, ORC_FP_SHA256 = 1 };

static void tokens_le(const int32_t *t, int64_t n, uint8_t *b)
{
    for (int64_t i = 0; i < n; i++) {
        uint32_t u = (uint32_t)t[i];
        b[4 * i] = (uint8_t)u;
        b[4 * i + 1] = (uint8_t)(u >> 8);
        b[4 * i + 2] = (uint8_t)(u >> 16);
        b[4 * i + 3] = (uint8_t)(u >> 24);
    }
}

uint64_t orc_gear_value(int32_t token, uint64_t gear_seed)
{
    uint8_t b[4];
    tokens_le(&token, 1, b);
    return orc_xxh64(b, 4, gear_seed);
}

/* h[i] for every position: the rolling Gear hash */
void orc_gear(const int32_t *tokens, int64_t n, uint64_t gear_seed, uint64_t *h)
{
    uint64_t x = 0;
    for (int64_t i = 0; i < n; i++) {
        x = (x << 1) + orc_gear_value(tokens[i], gear_seed);
        h[i] = x;
    }
}

/* Exclusive end positions of the content-defined chunks; returns their count. */
int64_t orc_cdc_ends(const int32_t *tokens, int64_t n, uint64_t threshold, uint64_t gear_seed,
                     int64_t *ends)
{
    int64_t count = 0;
    uint64_t x = 0;
    for (int64_t i = 0; i < n; i++) {
        x = (x << 1) + orc_gear_value(tokens[i], gear_seed);
        if (x < threshold || i == n - 1) ends[count++] = i + 1;
    }
    return count;
}

int orc_fingerprint(const int32_t *tokens, int64_t start, int64_t len, int kind, uint64_t seed,
                    uint8_t out[32])
{
    uint8_t *b = malloc((size_t)(4 * len + 1));
    if (!b) return 1;
    tokens_le(tokens + start, len, b);
    memset(out, 0, 32);
    if (kind == ORC_FP_SHA256) {
        orc_sha256(b, 4 * len, out);
    } else {
        uint64_t v = orc_xxh64(b, 4 * len, seed);
        for (int k = 0; k < 8; k++) out[k] = (uint8_t)(v >> (8 * k));
    }
    free(b);
    return 0;
}

/* first registered entry with this fingerprint and length, else -1 */
static int32_t reg_find(const uint8_t *reg_fp, const int32_t *reg_len, const int32_t *reg_id,
                        int64_t n_reg, const uint8_t fp[32], int64_t len)
{
    for (int64_t r = 0; r < n_reg; r++)
        if (reg_len[r] == len && memcmp(reg_fp + 32 * r, fp, 32) == 0) return reg_id[r];
    return -1;
}

/*
 * Segments of a stream, in order: every content-defined chunk the registry
 * holds, and in place of every other chunk its fallback windows (window > 0)
 * or the chunk itself as a miss (window == 0).  Per segment: start, length,
 * level (0 chunk, 1 window), registry id (-1: none) and fingerprint.
 * Returns the number of segments (written up to max_out), or -1 on an
 * allocation failure.
 */
int64_t orc_match(const int32_t *tokens, int64_t n, uint64_t threshold, uint64_t gear_seed,
                  int kind, uint64_t fp_seed, int32_t window, const uint8_t *reg_fp,
                  const int32_t *reg_len, const int32_t *reg_id, int64_t n_reg,
                  int64_t *out_start, int32_t *out_len, int32_t *out_level, int32_t *out_id,
                  uint8_t *out_fp, int64_t max_out)
{
    if (n == 0) return 0;
    int64_t *ends = malloc(sizeof(int64_t) * (size_t)n);
    if (!ends) return -1;
    int64_t nc = orc_cdc_ends(tokens, n, threshold, gear_seed, ends);
    int64_t m = 0, s = 0;
    uint8_t fp[32];
    for (int64_t c = 0; c < nc; c++) {
        int64_t len = ends[c] - s;
        if (orc_fingerprint(tokens, s, len, kind, fp_seed, fp)) {
            free(ends);
            return -1;
        }
        int32_t id = reg_find(reg_fp, reg_len, reg_id, n_reg, fp, len);
        if (id >= 0 || window <= 0) {
            if (m < max_out) {
                out_start[m] = s;
                out_len[m] = (int32_t)len;
                out_level[m] = 0;
                out_id[m] = id;
                memcpy(out_fp + 32 * m, fp, 32);
            }
            m++;
        } else {
            for (int64_t w = s; w < ends[c]; w += window) {
                int64_t wl = ends[c] - w < window ? ends[c] - w : window;
                if (orc_fingerprint(tokens, w, wl, kind, fp_seed, fp)) {
                    free(ends);
                    return -1;
                }
                if (m < max_out) {
                    out_start[m] = w;
                    out_len[m] = (int32_t)wl;
                    out_level[m] = 1;
                    out_id[m] = reg_find(reg_fp, reg_len, reg_id, n_reg, fp, wl);
                    memcpy(out_fp + 32 * m, fp, 32);
                }
                m++;
            }
        }
        s = ends[c];
    }
    free(ends);
    return m;
}
