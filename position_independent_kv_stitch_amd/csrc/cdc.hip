// cdc.hip -- content-defined chunking of token streams, chunk fingerprints
// and the chunk-registry lookup, on the GPU (pic_match and the registry
// calls of the C ABI).
//
// What is computed (Irminsul: MLA-Native Position-Independent Caching for
// Agentic LLM Serving, Technical Summary, "Content-Hash Keying with CDC" and
// the S1 "detect and recover" strategy; EPIC Guide: Position-Independent
// Caching for LLM Serving, the runtime's content hash registry):
//   - the Gear value of a token is the xxHash64 of its 4 little-endian bytes
//     under a gear seed; the rolling hash is h_i = 2 h_{i-1} + G(t_i) mod
//     2^64, so h_i is a weighted sum over the 64-token window ending at i;
//   - a chunk ends after token i when h_i < threshold, and at the stream end;
//   - a chunk's fingerprint is the SHA-256 of its tokens' little-endian
//     int32 bytes, or their xxHash64 as 8 little-endian bytes and 24 zeros;
//   - a chunk is a hit when the registry holds the same fingerprint with the
//     same length; a missed chunk is replaced, when a fallback window W > 0
//     is given, by its consecutive W-token windows, each looked up again.
//
// GPU decomposition (integer work on a few bytes per token: no MFMA, no
// HBM pressure; the cost is ALU work and its balance over lanes):
//   1. cdc_flag_kernel: a workgroup takes 1024 positions, computes the Gear
//      values of those positions and of the 64 before them into LDS, and
//      every lane rolls the hash over 16 consecutive positions (64 steps to
//      enter the window, then one shift-add per position).  Boundaries
//      become a bit mask and a count per workgroup.
//   2. scan_top_kernel: exclusive scan of the per-workgroup counts.
//   3. cdc_ends_kernel: every boundary writes its chunk's end position.
//   4. cdc_chunk_kernel: one lane per chunk (four for xxHash64, one per
//      accumulator) hashes it, looks it up and counts the segments it
//      becomes (1, or its number of windows).
//   5. scan of the segment counts (reduce, top, apply) gives every chunk's
//      first output slot and the total, which is written to *n_out; the
//      apply step also marks the chunk of every output slot.
//   6. cdc_emit_kernel: one lane per output segment writes its record,
//      hashing and looking up a window.
// Every lane's hash is a serial chain, so the longest chunk sets the time
// of step 4: loads are issued a block (or stripe) ahead of the arithmetic.
// The stream length and every count stay on the device: no call waits for
// the GPU, and later kernels run grid-stride loops bounded by counts they
// read from device memory.
//
// Hashes follow their published definitions: xxHash64 (Y. Collet's xxHash
// specification) and SHA-256 (FIPS 180-4).  SHA-256's round constants and
// initial state are the first 32 fractional bits of the cube roots of the
// first 64 primes and of the square roots of the first 8; they are computed
// at compile time below as exact integer roots.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <memory>
#include <mutex>
#include <new>
#include <string>
#include <unordered_set>
#include <vector>

#include "pic_internal.hpp"

namespace pic {
pic_status hip_fail(hipError_t e, const char *what);  // stitch.hip

// Registry table (device and host).

// Open-addressing table, linear probing, at most half full; an empty slot
// has chunk_id -1.
struct RegSlot {
    uint64_t fp[4];
    int32_t length;
    int32_t chunk_id;
};
static_assert(sizeof(RegSlot) == 40, "slot layout");

__host__ __device__ __forceinline__ uint64_t slot_hash(uint64_t fp0, int32_t length) {
    uint64_t x = fp0 ^ (static_cast<uint64_t>(static_cast<uint32_t>(length)) * 0x9E3779B97F4A7C15ull);
    x ^= x >> 31;
    x *= 0xD6E8FEB86659FD93ull;
    return x ^ (x >> 32);
}

namespace {

constexpr int kThreads = 256;                  // workgroup of the block kernels
constexpr int kPerThread = 16;                 // positions (or items) per lane
constexpr int kBlockItems = kThreads * kPerThread;  // 4096
constexpr int kWindow = 64;                    // Gear window
constexpr int kFlagThreads = 64;              // boundary kernels: one wave per workgroup
constexpr int kFlagItems = kFlagThreads * kPerThread;  // 1024 positions per workgroup
constexpr int kFlagWords = kFlagItems / 64;
constexpr int kLaneThreads = 64;               // workgroup of the lane-per-item kernels

// ------------------------------------------------------------- xxHash64

constexpr uint64_t kP1 = 0x9E3779B185EBCA87ull;
constexpr uint64_t kP2 = 0xC2B2AE3D27D4EB4Full;
constexpr uint64_t kP3 = 0x165667B19E3779F9ull;
constexpr uint64_t kP4 = 0x85EBCA77C2B2AE63ull;
constexpr uint64_t kP5 = 0x27D4EB2F165667C5ull;

__device__ __forceinline__ uint64_t rotl64(uint64_t x, int r) { return (x << r) | (x >> (64 - r)); }

__device__ __forceinline__ uint64_t xx_round(uint64_t acc, uint64_t lane) {
    return rotl64(acc + lane * kP2, 31) * kP1;
}

__device__ __forceinline__ uint64_t xx_avalanche(uint64_t h) {
    h = (h ^ (h >> 33)) * kP2;
    h = (h ^ (h >> 29)) * kP3;
    return h ^ (h >> 32);
}

// An empty asm that claims to change x: the compiler cannot see through it,
// so a value loaded for the next block stays a load issued in this one
// (without it, the load is re-formed at its use, and the lane stalls on it).
__device__ __forceinline__ void opaque(uint32_t &x) { asm volatile("" : "+v"(x)); }

// Two consecutive tokens as one little-endian 64-bit word.
__device__ __forceinline__ uint64_t tok_pair(const int32_t *t) {
    return static_cast<uint64_t>(static_cast<uint32_t>(t[0])) |
           (static_cast<uint64_t>(static_cast<uint32_t>(t[1])) << 32);
}

// Seed of accumulator q (0..3) of xxHash64's 32-byte stripe phase.
__device__ __forceinline__ uint64_t xx_acc_seed(uint64_t seed, int q) {
    return q == 0 ? seed + kP1 + kP2 : q == 1 ? seed + kP2 : q == 2 ? seed : seed - kP1;
}

// The phase after the stripes: merge the accumulators (when there were
// stripes), add the length, mix the remaining 8- and 4-byte words of
// t[i, n) and avalanche.  The input is a whole number of 4-byte words, so
// the specification's single-byte tail never occurs.
__device__ uint64_t xx_finish(const int32_t *t, int64_t i, int64_t n, uint64_t seed,
                              const uint64_t a[4]) {
    uint64_t h;
    if (n >= 8) {
        h = rotl64(a[0], 1) + rotl64(a[1], 7) + rotl64(a[2], 12) + rotl64(a[3], 18);
#pragma unroll
        for (int q = 0; q < 4; ++q) h = (h ^ xx_round(0, a[q])) * kP1 + kP4;
    } else {
        h = seed + kP5;
    }
    h += static_cast<uint64_t>(n) * 4u;
    for (; i + 2 <= n; i += 2) h = rotl64(h ^ xx_round(0, tok_pair(t + i)), 27) * kP1 + kP4;
    if (i < n) h = rotl64(h ^ (static_cast<uint64_t>(static_cast<uint32_t>(t[i])) * kP1), 23) * kP2 + kP3;
    return xx_avalanche(h);
}

// xxHash64 of the 4 n bytes of tokens t[0, n), one lane.  Stripes are taken
// four at a time; the next group is loaded (addresses clamped to the last
// stripe, so every load is in bounds) before the current group is mixed.
__device__ uint64_t xxh64_tokens(const int32_t *t, int64_t n, uint64_t seed) {
    constexpr int kG = 4;
    const int64_t stripes = n / 8;
    uint64_t a[4] = {xx_acc_seed(seed, 0), xx_acc_seed(seed, 1), xx_acc_seed(seed, 2),
                     xx_acc_seed(seed, 3)};
    if (stripes > 0) {
        uint32_t cur[8 * kG];
#pragma unroll
        for (int k = 0; k < kG; ++k) {
            const int32_t *p = t + 8 * min(static_cast<int64_t>(k), stripes - 1);
#pragma unroll
            for (int j = 0; j < 8; ++j) cur[8 * k + j] = static_cast<uint32_t>(p[j]);
        }
        for (int64_t g = 0; g < stripes; g += kG) {
            uint32_t nxt[8 * kG];
#pragma unroll
            for (int k = 0; k < kG; ++k) {
                const int32_t *p = t + 8 * min(g + kG + k, stripes - 1);
#pragma unroll
                for (int j = 0; j < 8; ++j) nxt[8 * k + j] = static_cast<uint32_t>(p[j]);
            }
            asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]) : : "memory");
#pragma unroll
            for (int k = 0; k < kG; ++k) {
                const bool live = g + k < stripes;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint64_t r = xx_round(a[q], cur[8 * k + 2 * q] |
                                       (static_cast<uint64_t>(cur[8 * k + 2 * q + 1]) << 32));
                    a[q] = live ? r : a[q];
                }
            }
#pragma unroll
            for (int j = 0; j < 8 * kG; ++j) {
                opaque(nxt[j]);
                cur[j] = nxt[j];
            }
        }
    }
    return xx_finish(t, 8 * stripes, n, seed, a);
}

// xxHash64 of t[0, n) by a group of four consecutive lanes (q = lane % 4):
// lane q runs accumulator q over the 8-byte word q of every stripe, kG
// stripes per load group, then the group's accumulators meet in lane q = 0,
// which alone returns the hash.  All four lanes must call it together.
template <int kG>
__device__ uint64_t xxh64_tokens_x4(const int32_t *t, int64_t n, uint64_t seed, int q) {
    const int64_t stripes = n / 8;
    uint64_t acc = xx_acc_seed(seed, q);
    const int32_t *base = t + 2 * q;
    if (stripes > 0) {
        uint32_t cur[2 * kG];
#pragma unroll
        for (int k = 0; k < kG; ++k) {
            const int32_t *p = base + 8 * min(static_cast<int64_t>(k), stripes - 1);
            cur[2 * k] = static_cast<uint32_t>(p[0]);
            cur[2 * k + 1] = static_cast<uint32_t>(p[1]);
        }
        for (int64_t g = 0; g < stripes; g += kG) {
            uint32_t nxt[2 * kG];
#pragma unroll
            for (int k = 0; k < kG; ++k) {
                const int32_t *p = base + 8 * min(g + kG + k, stripes - 1);
                nxt[2 * k] = static_cast<uint32_t>(p[0]);
                nxt[2 * k + 1] = static_cast<uint32_t>(p[1]);
            }
            asm volatile("" : "+v"(acc) : : "memory");
#pragma unroll
            for (int k = 0; k < kG; ++k) {
                const uint64_t r = xx_round(acc, cur[2 * k] | (static_cast<uint64_t>(cur[2 * k + 1]) << 32));
                acc = g + k < stripes ? r : acc;
            }
#pragma unroll
            for (int j = 0; j < 2 * kG; ++j) {
                opaque(nxt[j]);
                cur[j] = nxt[j];
            }
        }
    }
    const int lead = (threadIdx.x & 63) & ~3;
    uint64_t a[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = __shfl(acc, lead + k, 64);
    return q == 0 ? xx_finish(t, 8 * stripes, n, seed, a) : 0;
}

// Gear value: xxHash64 of one token's 4 bytes (the short-input form).
__device__ __forceinline__ uint64_t gear_value(int32_t token, uint64_t seed) {
    uint64_t h = seed + kP5 + 4u;
    h = rotl64(h ^ (static_cast<uint64_t>(static_cast<uint32_t>(token)) * kP1), 23) * kP2 + kP3;
    return xx_avalanche(h);
}

// -------------------------------------------------------------- SHA-256

struct ShaConstants {
    uint32_t k[64];
    uint32_t h0[8];
};

constexpr bool is_prime(uint32_t v) {
    if (v < 2) return false;
    for (uint32_t d = 2; d * d <= v; ++d)
        if (v % d == 0) return false;
    return true;
}

// Largest r with r^e <= x (e = 2 or 3), by bisection on exact integers.
constexpr uint64_t iroot(unsigned __int128 x, int e) {
    uint64_t lo = 0, hi = 1ull << 40;
    while (hi - lo > 1) {
        const uint64_t mid = lo + (hi - lo) / 2;
        unsigned __int128 p = mid;
        p *= mid;
        if (e == 3) p *= mid;
        if (p <= x) lo = mid; else hi = mid;
    }
    return lo;
}

// floor(root(p) * 2^32) = floor(root(p * 2^(32 e))); its low 32 bits are the
// first 32 fractional bits of root(p).
constexpr ShaConstants make_sha_constants() {
    ShaConstants c{};
    int n = 0;
    for (uint32_t p = 2; n < 64; ++p) {
        if (!is_prime(p)) continue;
        c.k[n] = static_cast<uint32_t>(iroot(static_cast<unsigned __int128>(p) << 96, 3));
        if (n < 8) c.h0[n] = static_cast<uint32_t>(iroot(static_cast<unsigned __int128>(p) << 64, 2));
        ++n;
    }
    return c;
}

constexpr ShaConstants kSha = make_sha_constants();

__device__ __forceinline__ uint32_t rotr32(uint32_t x, int r) { return (x >> r) | (x << (32 - r)); }

__device__ __forceinline__ uint32_t bswap32(uint32_t x) { return __builtin_bswap32(x); }

// x ^ y ^ z in one instruction (gfx950's three-input bit operation; 0x96 is
// the truth table of a three-way exclusive or).
__device__ __forceinline__ uint32_t xor3(uint32_t x, uint32_t y, uint32_t z) {
    return __builtin_amdgcn_bitop3_b32(x, y, z, 0x96);
}


// One compression of a 16-word block; w is consumed as the schedule's ring.
__device__ __forceinline__ void sha_compress(uint32_t st[8], uint32_t w[16]) {
    uint32_t a = st[0], b = st[1], c = st[2], d = st[3], e = st[4], f = st[5], g = st[6],
             h = st[7];
#pragma unroll
    for (int t = 0; t < 64; ++t) {
        if (t >= 16) {
            const uint32_t x = w[(t + 1) & 15], y = w[(t + 14) & 15];
            const uint32_t s0 = xor3(rotr32(x, 7), rotr32(x, 18), x >> 3);
            const uint32_t s1 = xor3(rotr32(y, 17), rotr32(y, 19), y >> 10);
            w[t & 15] += s0 + w[(t + 9) & 15] + s1;
        }
        // Ch picks f where e is set, else g; Maj picks c where a and b differ,
        // else b: both written as bit selects (one v_bfi each).
        const uint32_t ab = a ^ b;
        const uint32_t t1 = h + xor3(rotr32(e, 6), rotr32(e, 11), rotr32(e, 25)) +
                            ((e & f) | (~e & g)) + kSha.k[t] + w[t & 15];
        const uint32_t t2 = xor3(rotr32(a, 2), rotr32(a, 13), rotr32(a, 22)) +
                            ((ab & c) | (~ab & b));
        h = g;
        g = f;
        f = e;
        e = d + t1;
        d = c;
        c = b;
        b = a;
        a = t1 + t2;
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

// SHA-256 of the 4 n bytes of tokens t[0, n).  The message is word-aligned,
// so message word q is the byte swap of token q, the 0x80 padding byte
// starts word n, and the bit length fills words 14 and 15 of the last block.
// Over the full 16-word blocks the next block is loaded (unconditionally:
// the last iteration reloads its own block) before the current one is
// compressed, so a lane's loads overlap its rounds.  The one or two padded
// blocks follow.
__device__ void sha256_tokens(const int32_t *t, int64_t n, uint32_t st[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) st[j] = kSha.h0[j];
    const int64_t full = n / 16;
    uint32_t cur[16];
    if (full > 0) {
#pragma unroll
        for (int j = 0; j < 16; ++j) cur[j] = static_cast<uint32_t>(t[j]);
    }
    for (int64_t b = 0; b < full; ++b) {
        const int32_t *p = t + 16 * (b + 1 < full ? b + 1 : b);
        uint32_t nxt[16], w[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) nxt[j] = static_cast<uint32_t>(p[j]);
        // The loads stay above this point, and the rounds below it: the
        // state passes through the (empty) asm.
        asm volatile("" : "+v"(st[0]), "+v"(st[1]), "+v"(st[2]), "+v"(st[3]), "+v"(st[4]),
                     "+v"(st[5]), "+v"(st[6]), "+v"(st[7]) : : "memory");
#pragma unroll
        for (int j = 0; j < 16; ++j) w[j] = bswap32(cur[j]);
        sha_compress(st, w);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            opaque(nxt[j]);
            cur[j] = nxt[j];
        }
    }
    const int r = static_cast<int>(n - 16 * full);  // words left: 0..15
    const int32_t *p = t + 16 * full;
    const uint64_t bits = static_cast<uint64_t>(n) * 32u;
    const int tail_blocks = r <= 13 ? 1 : 2;
    for (int tb = 0; tb < tail_blocks; ++tb) {
        uint32_t w[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int q = 16 * tb + j;
            w[j] = q < r ? bswap32(static_cast<uint32_t>(p[q])) : (q == r ? 0x80000000u : 0u);
        }
        if (tb == tail_blocks - 1) {
            w[14] = static_cast<uint32_t>(bits >> 32);
            w[15] = static_cast<uint32_t>(bits);
        }
        sha_compress(st, w);
    }
}

// Fingerprint as four little-endian 64-bit words of its 32 bytes.
__device__ void fingerprint(const int32_t *t, int64_t n, int32_t kind, uint64_t seed,
                            uint64_t fp[4]) {
    if (kind == PIC_FP_SHA256) {
        uint32_t st[8];
        sha256_tokens(t, n, st);
#pragma unroll
        for (int j = 0; j < 4; ++j)  // digest bytes are the state words, big-endian
            fp[j] = static_cast<uint64_t>(bswap32(st[2 * j])) |
                    (static_cast<uint64_t>(bswap32(st[2 * j + 1])) << 32);
    } else {
        fp[0] = xxh64_tokens(t, n, seed);
        fp[1] = fp[2] = fp[3] = 0;
    }
}

// ------------------------------------------------------- registry lookup

__device__ int32_t reg_lookup(const RegSlot *tab, uint32_t mask, const uint64_t fp[4],
                              int32_t length) {
    if (!tab) return -1;
    uint32_t i = static_cast<uint32_t>(slot_hash(fp[0], length)) & mask;
    for (uint32_t probe = 0; probe <= mask; ++probe) {
        const RegSlot &s = tab[i];
        if (s.chunk_id < 0) return -1;
        if (s.length == length && s.fp[0] == fp[0] && s.fp[1] == fp[1] && s.fp[2] == fp[2] &&
            s.fp[3] == fp[3])
            return s.chunk_id;
        i = (i + 1) & mask;
    }
    return -1;
}

// ------------------------------------------------------------ scan helper

// Exclusive scan of one int32 per lane over a workgroup of kThreads lanes;
// *total receives the sum.  `lds` holds kThreads / 64 + 1 ints.
__device__ int32_t block_exclusive_scan(int32_t v, int32_t *lds, int32_t *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int32_t x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) lds[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t run = 0;
        for (int w = 0; w < kThreads / 64; ++w) {
            const int32_t s = lds[w];
            lds[w] = run;
            run += s;
        }
        lds[kThreads / 64] = run;
    }
    __syncthreads();
    const int32_t r = lds[wave] + x - v;
    *total = lds[kThreads / 64];
    __syncthreads();
    return r;
}

// --------------------------------------------------------------- kernels

// Padded LDS index of Gear slot j (slots 0..63 are the 64 positions before
// the workgroup's first): one 8-byte pad per 16 slots puts the 16-position
// runs of consecutive lanes in different banks.
__device__ __forceinline__ int gpad(int j) { return j + (j >> 4); }

__global__ __launch_bounds__(kFlagThreads) void cdc_flag_kernel(const int32_t *__restrict__ tok,
                                                                int64_t n, uint64_t gear_seed,
                                                                uint64_t threshold,
                                                                uint64_t *__restrict__ flags,
                                                                int32_t *__restrict__ bcnt) {
    constexpr int kSlots = kFlagItems + kWindow;
    __shared__ uint64_t g[kSlots + kSlots / 16];
    __shared__ uint32_t bits[kFlagThreads];
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kFlagItems;
    for (int j = threadIdx.x; j < kSlots; j += kFlagThreads) {
        const int64_t pos = base - kWindow + j;
        g[gpad(j)] = (pos >= 0 && pos < n) ? gear_value(tok[pos], gear_seed) : 0;
    }
    __syncthreads();
    const int first = threadIdx.x * kPerThread;
    uint64_t h = 0;  // after this loop: h at the position before the lane's first
    for (int j = 0; j < kWindow; ++j) h = (h << 1) + g[gpad(first + j)];
    uint32_t b = 0;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
        const int64_t pos = base + first + j;
        h = (h << 1) + g[gpad(first + kWindow + j)];
        if (pos < n && (h < threshold || pos == n - 1)) b |= 1u << j;
    }
    bits[threadIdx.x] = b;
    int32_t c = __popc(b);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) c += __shfl_xor(c, d, 64);
    __syncthreads();
    if (threadIdx.x < kFlagWords) {
        const int t = 4 * threadIdx.x;
        flags[static_cast<int64_t>(blockIdx.x) * kFlagWords + threadIdx.x] =
            static_cast<uint64_t>(bits[t]) | (static_cast<uint64_t>(bits[t + 1]) << 16) |
            (static_cast<uint64_t>(bits[t + 2]) << 32) | (static_cast<uint64_t>(bits[t + 3]) << 48);
    }
    if (threadIdx.x == 0) bcnt[blockIdx.x] = c;
}

// Exclusive scan, in place, of v[0, len) where len = n_host, or, when
// items_dev is given, the number of kBlockItems-blocks covering *items_dev
// items.  The sum goes to *total (and to *total64 when given).  One
// workgroup of 1024 lanes; lane l scans a contiguous slice.
__global__ __launch_bounds__(1024) void scan_top_kernel(int32_t *__restrict__ v, int64_t n_host,
                                                        const int32_t *__restrict__ items_dev,
                                                        int32_t *__restrict__ total,
                                                        int64_t *__restrict__ total64) {
    __shared__ int32_t part[1024];
    const int64_t len =
        items_dev ? (static_cast<int64_t>(*items_dev) + kBlockItems - 1) / kBlockItems : n_host;
    const int64_t per = (len + 1023) / 1024;
    const int64_t lo = min(len, per * threadIdx.x), hi = min(len, lo + per);
    int32_t s = 0;
    for (int64_t i = lo; i < hi; ++i) s += v[i];
    part[threadIdx.x] = s;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {  // inclusive Hillis-Steele scan of the slices
        const int32_t y = threadIdx.x >= d ? part[threadIdx.x - d] : 0;
        __syncthreads();
        part[threadIdx.x] += y;
        __syncthreads();
    }
    int32_t run = part[threadIdx.x] - s;
    for (int64_t i = lo; i < hi; ++i) {
        const int32_t x = v[i];
        v[i] = run;
        run += x;
    }
    if (threadIdx.x == 1023) {
        *total = part[1023];
        if (total64) *total64 = part[1023];
    }
}

// End position (exclusive) of every chunk, in stream order.  One wave per
// workgroup, the boundary kernel's partition.
__global__ __launch_bounds__(kFlagThreads) void cdc_ends_kernel(const uint64_t *__restrict__ flags,
                                                               const int32_t *__restrict__ boff,
                                                               int32_t *__restrict__ ends) {
    const uint64_t word =
        flags[static_cast<int64_t>(blockIdx.x) * kFlagWords + (threadIdx.x >> 2)];
    uint32_t b = static_cast<uint32_t>(word >> (16 * (threadIdx.x & 3))) & 0xFFFFu;
    const int32_t cnt = __popc(b);
    int32_t x = cnt;  // inclusive scan over the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t y = __shfl_up(x, d, 64);
        if (static_cast<int>(threadIdx.x) >= d) x += y;
    }
    int32_t slot = boff[blockIdx.x] + x - cnt;
    const int64_t first = static_cast<int64_t>(blockIdx.x) * kFlagItems + threadIdx.x * kPerThread;
    while (b) {
        const int j = __ffs(b) - 1;
        ends[slot++] = static_cast<int32_t>(first + j + 1);
        b &= b - 1;
    }
}

struct MatchArgs {
    const int32_t *tok;
    const int32_t *ends;    // [nc]
    int32_t *seg;           // [nc]: segment count, then first output slot
    const int32_t *counts;  // [0] chunks nc, [1] segments m
    uint64_t *cfp;          // [keep][4] chunk fingerprints
    int32_t *cid;           // [keep] chunk registry ids
    int32_t *owner;         // [keep] chunk of every output slot
    const RegSlot *tab;
    uint32_t mask;
    int32_t kind;
    uint64_t fp_seed;
    int32_t window;
    int32_t keep;           // chunks whose fingerprint is kept: min(n, max_out)
    pic_match_t *out;
    int64_t max_out;
    int64_t n;              // stream length: bounds every count read back
};

__device__ __forceinline__ int64_t chunk_start(const int32_t *ends, int64_t c) {
    return c ? ends[c - 1] : 0;
}

// G lanes per chunk (G = 4: xxHash64's four accumulators on four lanes; G =
// 1: SHA-256, which is serial): fingerprint, lookup, number of output
// segments.  The lanes of a group share their chunk index, so a group is
// active or idle as a whole.
template <int G>
__global__ __launch_bounds__(kLaneThreads) void cdc_chunk_kernel(MatchArgs a) {
    const int64_t nc = min(static_cast<int64_t>(a.counts[0]), a.n);
    const int q = threadIdx.x % G;
    for (int64_t c = (static_cast<int64_t>(blockIdx.x) * kLaneThreads + threadIdx.x) / G; c < nc;
         c += static_cast<int64_t>(gridDim.x) * (kLaneThreads / G)) {
        const int64_t s = chunk_start(a.ends, c), len = a.ends[c] - s;
        uint64_t fp[4] = {0, 0, 0, 0};
        if constexpr (G == 4) {
            fp[0] = xxh64_tokens_x4<8>(a.tok + s, len, a.fp_seed, q);
        } else {
            fingerprint(a.tok + s, len, a.kind, a.fp_seed, fp);
        }
        if (q != 0) continue;
        const int32_t id = reg_lookup(a.tab, a.mask, fp, static_cast<int32_t>(len));
        a.seg[c] = (id >= 0 || a.window <= 0) ? 1
                                              : static_cast<int32_t>((len + a.window - 1) / a.window);
        if (c < a.keep) {
#pragma unroll
            for (int j = 0; j < 4; ++j) a.cfp[4 * c + j] = fp[j];
            a.cid[c] = id;
        }
    }
}

// Per-block sums of v[0, *len_dev) (blocks past the end write nothing).
__global__ __launch_bounds__(kThreads) void scan_reduce_kernel(const int32_t *__restrict__ v,
                                                               const int32_t *__restrict__ len_dev,
                                                               int32_t *__restrict__ bsum) {
    __shared__ int32_t cnt;
    const int64_t len = *len_dev, base = static_cast<int64_t>(blockIdx.x) * kBlockItems;
    if (base >= len) return;
    if (threadIdx.x == 0) cnt = 0;
    __syncthreads();
    int32_t s = 0;
    for (int j = 0; j < kPerThread; ++j) {
        const int64_t i = base + j * kThreads + threadIdx.x;
        if (i < len) s += v[i];
    }
    atomicAdd(&cnt, s);
    __syncthreads();
    if (threadIdx.x == 0) bsum[blockIdx.x] = cnt;
}

// In-place exclusive scan of v[0, *len_dev), block b offset by boff[b].
// With `owner`, item i also marks the slots [v'[i], v'[i] + v[i]) below
// `keep` as its own (v' the scanned value): the chunk of every output slot.
__global__ __launch_bounds__(kThreads) void scan_apply_kernel(int32_t *__restrict__ v,
                                                              const int32_t *__restrict__ len_dev,
                                                              const int32_t *__restrict__ boff,
                                                              int32_t *__restrict__ owner,
                                                              int64_t keep) {
    __shared__ int32_t lds[kThreads / 64 + 1];
    const int64_t len = *len_dev, base = static_cast<int64_t>(blockIdx.x) * kBlockItems;
    if (base >= len) return;  // uniform over the workgroup
    const int64_t first = base + threadIdx.x * kPerThread;
    int32_t x[kPerThread];
    int32_t s = 0;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
        x[j] = first + j < len ? v[first + j] : 0;
        s += x[j];
    }
    int32_t total;
    int32_t run = boff[blockIdx.x] + block_exclusive_scan(s, lds, &total);
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
        if (first + j < len) {
            v[first + j] = run;
            if (owner)
                for (int64_t k = run; k < run + x[j] && k < keep; ++k)
                    owner[k] = static_cast<int32_t>(first + j);
        }
        run += x[j];
    }
}

// G lanes per output record (the first max_out segments; G = 4 for
// xxHash64, whose windows are hashed like chunks, 1 for SHA-256); the owner
// map names each slot's chunk, and lane q = 0 of the group writes the record.
template <int G>
__global__ __launch_bounds__(kLaneThreads) void cdc_emit_kernel(MatchArgs a) {
    const int64_t m = min(static_cast<int64_t>(a.counts[1]), a.n);
    const int64_t lim = m < a.max_out ? m : a.max_out;
    const int q = threadIdx.x % G;
    for (int64_t s = (static_cast<int64_t>(blockIdx.x) * kLaneThreads + threadIdx.x) / G; s < lim;
         s += static_cast<int64_t>(gridDim.x) * (kLaneThreads / G)) {
        const int64_t c = a.owner[s], k = s - a.seg[c];
        const int64_t cs = chunk_start(a.ends, c), ce = a.ends[c];
        pic_match_t r;
        uint64_t fp[4];
        if (a.cid[c] >= 0 || a.window <= 0) {
            r.start = cs;
            r.length = static_cast<int32_t>(ce - cs);
            r.level = 0;
            r.chunk_id = a.cid[c];
#pragma unroll
            for (int j = 0; j < 4; ++j) fp[j] = a.cfp[4 * c + j];
        } else {
            // (uniform over the group: its lanes share s)
            const int64_t ws = cs + k * a.window;
            const int64_t wl = ce - ws < a.window ? ce - ws : a.window;
            if constexpr (G == 4) {
                fp[0] = xxh64_tokens_x4<16>(a.tok + ws, wl, a.fp_seed, q);
                fp[1] = fp[2] = fp[3] = 0;
            } else {
                fingerprint(a.tok + ws, wl, a.kind, a.fp_seed, fp);
            }
            r.start = ws;
            r.length = static_cast<int32_t>(wl);
            r.level = 1;
            r.chunk_id = q == 0 ? reg_lookup(a.tab, a.mask, fp, static_cast<int32_t>(wl)) : -1;
        }
        if (q != 0) continue;
        r.reserved = 0;
        memcpy(r.fp, fp, 32);
        a.out[s] = r;
    }
}

__global__ void write_zero_kernel(int64_t *p) { *p = 0; }

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace
}  // namespace pic

namespace pic {
// One uploaded version of a registry's device table.  A version is never
// written after its upload: a changed registry uploads a new one, and the
// old one is freed once every pic_match that read it has run (its last-use
// event per stream has completed).
struct RegTable {
    RegSlot *dev = nullptr;
    std::vector<RegSlot> host;  // the uploaded slots (alive for the copy)
    uint32_t mask = 0;
    hipEvent_t ready = nullptr;
    std::vector<std::pair<hipStream_t, hipEvent_t>> uses;
};
}  // namespace pic

// The opaque registry handle of the C ABI.
struct pic_registry {
    uint32_t magic = 0x52454753u;
    int32_t kind = 0;
    std::mutex mu;
    std::vector<pic::RegSlot> entries;    // in registration order
    std::unordered_set<std::string> keys;  // fingerprint bytes + length, for duplicates
    bool dirty = true;
    int device = -1;
    std::unique_ptr<pic::RegTable> table;                 // the current version
    std::vector<std::unique_ptr<pic::RegTable>> retired;  // older versions still in use
    // pic_match's temporaries, one buffer per stream kept between calls (the
    // calls on one stream reuse it in stream order), and outgrown buffers
    // with an event recorded after their last use; all freed by destroy
    struct Scratch {
        hipStream_t stream;
        void *ptr;
        size_t bytes;
    };
    std::vector<Scratch> scratch;
    std::vector<std::pair<void *, hipEvent_t>> retired_scratch;
};

namespace pic {
namespace {

constexpr uint32_t kRegMagic = 0x52454753u;

std::string reg_key(const uint64_t fp[4], int32_t length) {
    std::string k(reinterpret_cast<const char *>(fp), 32);
    k.append(reinterpret_cast<const char *>(&length), 4);
    return k;
}

// Whether every launch that read table t has run (host check, no wait).
bool table_idle(const RegTable &t) {
    if (t.ready && hipEventQuery(t.ready) == hipErrorNotReady) return false;
    for (const auto &u : t.uses)
        if (hipEventQuery(u.second) == hipErrorNotReady) return false;
    return true;
}

// Release table t; with `wait`, first wait for the launches that read it.
void free_table(RegTable &t, bool wait) {
    for (auto &u : t.uses) {
        if (wait) (void)hipEventSynchronize(u.second);
        (void)hipEventDestroy(u.second);
    }
    if (t.ready) {
        if (wait) (void)hipEventSynchronize(t.ready);
        (void)hipEventDestroy(t.ready);
    }
    if (t.dev) (void)hipFree(t.dev);
    t = RegTable{};
}

// Bring the device table up to date on the current device, ordered on
// `stream`.  A changed registry uploads a new version (earlier calls on any
// stream may still read the old one, which is retired, not overwritten);
// an unchanged one makes `stream` wait for the current version's upload.
pic_status sync_registry(pic_registry *reg, hipStream_t stream, const RegSlot **tab,
                         uint32_t *mask) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (reg->device >= 0 && dev != reg->device)
        return fail(PIC_ERR_STATE, "registry lives on device %d, current device is %d",
                    reg->device, dev);
    for (size_t i = 0; i < reg->retired.size();) {  // versions no call reads any more
        if (table_idle(*reg->retired[i])) {
            free_table(*reg->retired[i], false);
            reg->retired.erase(reg->retired.begin() + static_cast<std::ptrdiff_t>(i));
        } else {
            i++;
        }
    }
    if (reg->dirty || !reg->table) {
        std::unique_ptr<RegTable> t(new (std::nothrow) RegTable);
        if (!t) return fail(PIC_ERR_NOMEM, "out of host memory");
        size_t slots = 16;
        while (slots < 2 * reg->entries.size()) slots *= 2;
        t->host.assign(slots, RegSlot{{0, 0, 0, 0}, 0, -1});
        const uint32_t m = static_cast<uint32_t>(slots - 1);
        for (const RegSlot &sl : reg->entries) {
            uint32_t i = static_cast<uint32_t>(slot_hash(sl.fp[0], sl.length)) & m;
            while (t->host[i].chunk_id >= 0) i = (i + 1) & m;
            t->host[i] = sl;
        }
        t->mask = m;
        e = hipMalloc(&t->dev, slots * sizeof(RegSlot));
        if (e != hipSuccess) {
            t->dev = nullptr;
            return hip_fail(e, "hipMalloc (registry table)");
        }
        e = hipMemcpyAsync(t->dev, t->host.data(), slots * sizeof(RegSlot), hipMemcpyHostToDevice,
                           stream);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&t->ready, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventRecord(t->ready, stream);
        if (e != hipSuccess) {
            (void)hipStreamSynchronize(stream);
            free_table(*t, false);
            return hip_fail(e, "registry table upload");
        }
        if (reg->table) reg->retired.push_back(std::move(reg->table));
        reg->table = std::move(t);
        reg->device = dev;
        reg->dirty = false;
    } else {
        e = hipStreamWaitEvent(stream, reg->table->ready, 0);
        if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
    }
    *tab = reg->table->dev;
    *mask = reg->table->mask;
    return PIC_OK;
}

// Record that launches on `stream` read the registry's current table.
pic_status note_table_use(pic_registry *reg, hipStream_t stream) {
    RegTable &t = *reg->table;
    hipEvent_t ev = nullptr;
    for (auto &u : t.uses)
        if (u.first == stream) ev = u.second;
    if (!ev) {
        // completion is all that is waited for: no system-scope fence
        const hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming | hipEventDisableSystemFence);
        if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
        t.uses.emplace_back(stream, ev);
    }
    const hipError_t e = hipEventRecord(ev, stream);
    return e == hipSuccess ? PIC_OK : hip_fail(e, "hipEventRecord");
}

// At least `bytes` of pic_match temporaries for launches on `stream`, from
// the registry's buffer for that stream (reg->mu held).  A buffer too small
// is replaced by a larger one (at least 1.5 times the size) and kept, with an
// event recorded after the work already queued on the stream, until destroy.
pic_status registry_scratch(pic_registry *reg, hipStream_t stream, size_t bytes, void **out) {
    *out = nullptr;
    pic_registry::Scratch *w = nullptr;
    for (auto &x : reg->scratch)
        if (x.stream == stream) w = &x;
    if (w && w->bytes >= bytes) {
        *out = w->ptr;
        return PIC_OK;
    }
    if (w) {
        hipEvent_t ev = nullptr;
        hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming | hipEventDisableSystemFence);
        if (e == hipSuccess) e = hipEventRecord(ev, stream);
        if (e != hipSuccess) {
            if (ev) (void)hipEventDestroy(ev);
            return hip_fail(e, "pic_match temporaries retirement");
        }
        reg->retired_scratch.emplace_back(w->ptr, ev);
        bytes = std::max(bytes, w->bytes + w->bytes / 2);
        w->ptr = nullptr;
        w->bytes = 0;
    }
    void *p = nullptr;
    const hipError_t e = hipMalloc(&p, bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return hip_fail(e, "hipMalloc (pic_match temporaries)");
    }
    if (w) {
        w->ptr = p;
        w->bytes = bytes;
    } else {
        reg->scratch.push_back(pic_registry::Scratch{stream, p, bytes});
    }
    *out = p;
    return PIC_OK;
}

}  // namespace
}  // namespace pic

extern "C" {

pic_status pic_registry_create(int32_t fingerprint, pic_registry_t **out) {
    pic::clear_error();
    if (!out) return pic::fail(PIC_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (fingerprint != PIC_FP_XXH64 && fingerprint != PIC_FP_SHA256)
        return pic::fail(PIC_ERR_INVALID_ARG, "unknown fingerprint kind %d", fingerprint);
    pic_registry *r = new (std::nothrow) pic_registry;
    if (!r) return pic::fail(PIC_ERR_NOMEM, "out of host memory");
    r->kind = fingerprint;
    *out = r;
    return PIC_OK;
}

pic_status pic_registry_add(pic_registry_t *reg, const uint8_t *fp, int32_t length,
                            int32_t chunk_id) {
    pic::clear_error();
    if (!reg || reg->magic != pic::kRegMagic)
        return pic::fail(PIC_ERR_STATE, "invalid or destroyed registry");
    if (!fp) return pic::fail(PIC_ERR_INVALID_ARG, "fingerprint is NULL");
    if (length < 1) return pic::fail(PIC_ERR_RANGE, "length %d < 1", length);
    if (chunk_id < 0) return pic::fail(PIC_ERR_RANGE, "chunk_id %d < 0", chunk_id);
    pic::RegSlot s{};
    std::memcpy(s.fp, fp, 32);
    s.length = length;
    s.chunk_id = chunk_id;
    std::lock_guard<std::mutex> lock(reg->mu);
    try {
        if (!reg->keys.insert(pic::reg_key(s.fp, length)).second)
            return pic::fail(PIC_ERR_OVERLAP, "a segment with this fingerprint and length %d "
                             "is already registered", length);
        reg->entries.push_back(s);
    } catch (const std::bad_alloc &) {
        return pic::fail(PIC_ERR_NOMEM, "out of host memory");
    }
    reg->dirty = true;
    return PIC_OK;
}

void pic_registry_destroy(pic_registry_t *reg) {
    if (!reg || reg->magic != pic::kRegMagic) return;
    reg->magic = 0;
    // the registry's own work only: the launches that read any table version
    if (reg->table) pic::free_table(*reg->table, true);
    for (auto &t : reg->retired) pic::free_table(*t, true);
    // every pic_match that used the temporaries recorded a use of some table
    // version after its launches, and those have all completed now
    for (auto &r : reg->retired_scratch) {
        (void)hipEventSynchronize(r.second);
        (void)hipEventDestroy(r.second);
        (void)hipFree(r.first);
    }
    for (auto &x : reg->scratch) (void)hipFree(x.ptr);
    delete reg;
}

pic_status pic_match(pic_registry_t *reg, const pic_cdc_config *cfg, const int32_t *tokens,
                     int64_t n_tokens, pic_match_t *out, int64_t max_out, int64_t *n_out,
                     void *stream_) {
    using namespace pic;
    clear_error();
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    if (!cfg) return fail(PIC_ERR_INVALID_ARG, "cfg is NULL");
    if (cfg->fingerprint != PIC_FP_XXH64 && cfg->fingerprint != PIC_FP_SHA256)
        return fail(PIC_ERR_INVALID_ARG, "unknown fingerprint kind %d", cfg->fingerprint);
    if (reg && reg->magic != kRegMagic) return fail(PIC_ERR_STATE, "invalid or destroyed registry");
    if (reg && reg->kind != cfg->fingerprint)
        return fail(PIC_ERR_INVALID_ARG, "registry holds fingerprint kind %d, cfg asks for %d",
                    reg->kind, cfg->fingerprint);
    if (n_tokens < 0 || n_tokens >= (int64_t{1} << 31))
        return fail(PIC_ERR_RANGE, "n_tokens %lld outside [0, 2^31)",
                    static_cast<long long>(n_tokens));
    if (cfg->window < 0) return fail(PIC_ERR_RANGE, "window %d < 0", cfg->window);
    if (max_out < 0) return fail(PIC_ERR_RANGE, "max_out < 0");
    if (!n_out) return fail(PIC_ERR_INVALID_ARG, "n_out is NULL");
    if (n_tokens > 0 && !tokens) return fail(PIC_ERR_INVALID_ARG, "tokens is NULL");
    if (max_out > 0 && !out) return fail(PIC_ERR_INVALID_ARG, "out is NULL");
    if ((reinterpret_cast<uintptr_t>(tokens) & 3u) || (reinterpret_cast<uintptr_t>(out) & 7u) ||
        (reinterpret_cast<uintptr_t>(n_out) & 7u))
        return fail(PIC_ERR_ALIGN, "tokens must be 4-byte, out and n_out 8-byte aligned");

    const RegSlot *tab = nullptr;
    uint32_t mask = 0;
    std::unique_lock<std::mutex> lock;
    if (reg) {
        lock = std::unique_lock<std::mutex>(reg->mu);
        pic_status st = sync_registry(reg, stream, &tab, &mask);
        if (st != PIC_OK) return st;
    }
    hipError_t e;
    if (n_tokens == 0) {
        write_zero_kernel<<<1, 1, 0, stream>>>(n_out);
        e = hipGetLastError();
        return e == hipSuccess ? PIC_OK : hip_fail(e, "pic_match launch");
    }

    // Temporary device memory (stream-ordered).
    const int64_t n = n_tokens;
    const int64_t nb = (n + kBlockItems - 1) / kBlockItems;  // scan blocks
    const int64_t nbf = (n + kFlagItems - 1) / kFlagItems;   // boundary workgroups
    const int64_t keep = max_out < n ? max_out : n;
    size_t off = 0;
    const size_t o_flags = off; off = align256(off + sizeof(uint64_t) * nbf * kFlagWords);
    const size_t o_bcnt = off;  off = align256(off + sizeof(int32_t) * (nbf + 1));
    const size_t o_ends = off;  off = align256(off + sizeof(int32_t) * n);
    const size_t o_seg = off;   off = align256(off + sizeof(int32_t) * n);
    const size_t o_ssum = off;  off = align256(off + sizeof(int32_t) * (nb + 1));
    const size_t o_cnt = off;   off = align256(off + sizeof(int32_t) * 2);
    const size_t o_cfp = off;   off = align256(off + sizeof(uint64_t) * 4 * keep);
    const size_t o_cid = off;   off = align256(off + sizeof(int32_t) * keep);
    const size_t o_own = off;   off = align256(off + sizeof(int32_t) * keep);
    // temporaries: the registry's buffer for this stream, or stream-ordered
    // memory when there is no registry
    void *mem = nullptr;
    if (reg) {
        pic_status st = registry_scratch(reg, stream, off, &mem);
        if (st != PIC_OK) return st;
    } else {
        e = hipMallocAsync(&mem, off, stream);
        if (e != hipSuccess) return hip_fail(e, "hipMallocAsync (pic_match temporaries)");
    }
    uint8_t *base = static_cast<uint8_t *>(mem);
    auto *flags = reinterpret_cast<uint64_t *>(base + o_flags);
    auto *bcnt = reinterpret_cast<int32_t *>(base + o_bcnt);
    auto *ssum = reinterpret_cast<int32_t *>(base + o_ssum);
    auto *counts = reinterpret_cast<int32_t *>(base + o_cnt);

    MatchArgs a{};
    a.tok = tokens;
    a.ends = reinterpret_cast<int32_t *>(base + o_ends);
    a.seg = reinterpret_cast<int32_t *>(base + o_seg);
    a.counts = counts;
    a.cfp = reinterpret_cast<uint64_t *>(base + o_cfp);
    a.cid = reinterpret_cast<int32_t *>(base + o_cid);
    a.owner = reinterpret_cast<int32_t *>(base + o_own);
    a.tab = tab;
    a.mask = mask;
    a.kind = cfg->fingerprint;
    a.fp_seed = cfg->fp_seed;
    a.window = cfg->window;
    a.keep = static_cast<int32_t>(keep);
    a.out = out;
    a.max_out = max_out;
    a.n = n;

    // Lane-per-item kernels stride over at most this many workgroups.
    auto lane_grid = [](int64_t bound) {
        const int64_t g = (bound + kLaneThreads - 1) / kLaneThreads;
        return static_cast<unsigned>(g < 1 ? 1 : (g > 16384 ? 16384 : g));
    };
    const unsigned gb = static_cast<unsigned>(nb);
    const unsigned gf = static_cast<unsigned>(nbf);
    cdc_flag_kernel<<<gf, kFlagThreads, 0, stream>>>(tokens, n, cfg->gear_seed, cfg->threshold,
                                                    flags, bcnt);
    scan_top_kernel<<<1, 1024, 0, stream>>>(bcnt, nbf, nullptr, &counts[0], nullptr);
    cdc_ends_kernel<<<gf, kFlagThreads, 0, stream>>>(flags, bcnt, const_cast<int32_t *>(a.ends));
    if (cfg->fingerprint == PIC_FP_XXH64)
        cdc_chunk_kernel<4><<<lane_grid(4 * n), kLaneThreads, 0, stream>>>(a);
    else
        cdc_chunk_kernel<1><<<lane_grid(n), kLaneThreads, 0, stream>>>(a);
    scan_reduce_kernel<<<gb, kThreads, 0, stream>>>(a.seg, &counts[0], ssum);
    scan_top_kernel<<<1, 1024, 0, stream>>>(ssum, 0, &counts[0], &counts[1], n_out);
    scan_apply_kernel<<<gb, kThreads, 0, stream>>>(a.seg, &counts[0], ssum, a.owner, keep);
    if (keep > 0) {
        if (cfg->fingerprint == PIC_FP_XXH64)
            cdc_emit_kernel<4><<<lane_grid(4 * keep), kLaneThreads, 0, stream>>>(a);
        else
            cdc_emit_kernel<1><<<lane_grid(keep), kLaneThreads, 0, stream>>>(a);
    }
    e = hipGetLastError();
    const hipError_t e2 = reg ? hipSuccess : hipFreeAsync(mem, stream);
    if (e != hipSuccess) return hip_fail(e, "pic_match launch");
    if (e2 != hipSuccess) return hip_fail(e2, "hipFreeAsync (pic_match temporaries)");
    if (reg) return note_table_use(reg, stream);  // the lock is still held
    return PIC_OK;
}

}  // extern "C"
