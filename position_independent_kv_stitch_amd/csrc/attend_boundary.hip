// attend_boundary.hip -- LegoLink's boundary reconnection (pic_attend_boundary).
//
// A chunk prefilled on its own never saw the chunks placed before it.  The
// EPIC Guide (Position-Independent Caching for LLM Serving, "2. Sparse
// Cross-Block Reconnection") repairs this by letting only the first tokens
// of every relocated chunk (its boundary tokens; the EPIC listing's sparse
// k is 16) attend across the chunk boundary to what precedes it.  Here
// boundary token j of an entry placed at d > 0 attends causally to every
// position up to its own, d + j: the preceding chunks and prefix (rows read
// as pic_attend reads them: chunk keys turned by the entry's shift on load
// and rounded to bf16 as the stitch stores them, everything else from the
// request's own cache) and its own chunk's earlier tokens.  The LegoLink
// damping of pseudo-sinks is the same optional logit bias as in pic_attend.
//
// Work: per relocated entry, its boundary rows (tokens j < min(k, length) x
// the GQA group's query heads) form up to 8 row tiles of 16; a workgroup is
// one wave per row tile, for one KV head and one work item (a run of the
// entry's context [0, d + k)).  Items are cut per launch so that every
// workgroup has about the same number of positions.  Per step of 32
// positions (the latent kernel's scheme, attend_mla.hip):
//   - the step's K and V rows of the KV head (16 KB) go from HBM straight
//     into LDS (global_load_lds_dwordx4), in the MFMA A-fragment layout,
//     double-buffered across steps;
//   - rotary pieces of moved chunk rows are turned in LDS (fp64, rounded
//     to bf16 by the stitch's own code, rotate.hpp);
//   - S^T = K Q^T (v_mfma_f32_16x16x32_bf16, queries in registers), causal
//     limit per row, online softmax per row;
//   - O^T += V^T P^T with the weights from the S^T D registers (hi + lo
//     bf16) and V^T by transposing LDS reads (ds_read_b64_tr_b16).
// A partial (max, sum, accumulator) per (item, KV head, row) is merged by
// bnd_combine_kernel.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "pic_internal.hpp"
#include "rotate.hpp"

namespace pic {

pic_status hip_fail(hipError_t e, const char *what);  // stitch.hip

namespace {

constexpr int kDim = 128;                 // head row
constexpr int kKSteps = kDim / 32;        // MFMA k-steps
constexpr int kDTiles = kDim / 16;        // output tiles of 16 dims
constexpr int kStepPos = 32;              // positions per step: two 16-position tiles
constexpr int kKSlabs = 2 * kKSteps;      // 1 KB slabs of K per step (then as many of V)
constexpr int kSlabs = 2 * kKSlabs;
constexpr int kMaxWaves = 8;              // row tiles (of 16 rows) per entry at most
constexpr int kItemTiles = 64;            // map tiles per block at most
constexpr int kBlockPos = 4096;           // positions per block at most
constexpr int kCombineThreads = 128;

constexpr uint32_t kMetaDamp = 1u << 31;      // LegoLink bias applies
constexpr uint32_t kMetaCs = (1u << 30) - 1;  // shift table + 1 (0: row not turned)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef const void __attribute__((address_space(1))) *gptr_t;
typedef void __attribute__((address_space(3))) *lptr_t;

// One relocated entry: its boundary rows start at row0 (n_tok tokens), its
// token j sits at position pos0 + j of request `request`, its work items
// are [item0, item1).
struct BndEntry {
    int32_t request;
    int32_t row0;
    int32_t n_tok;
    int32_t pos0;
    int32_t item0;
    int32_t item1;
    int32_t pad[2];
};

// A work item: blocks [block0, block1) of entry `entry`.
struct BndItem {
    int32_t entry;
    int32_t block0;
    int32_t block1;
    int32_t pad;
};

struct BndArgs {
    const AttnTile *tiles;    // blocks' tiles (tok0: position in the block)
    const AttnBlock *blocks;  // request, tile0, ntiles, ntok
    const int32_t *block_pos; // context position of every block's first token
    const BndItem *items;
    const BndEntry *entries;
    const double *cs;
    const uint16_t *pool_k, *pool_v, *cache_k, *cache_v;
    int64_t s_layer, s_tok, s_head, s_page;
    int64_t c_layer, c_tok, c_head, c_page, c_req;
    const uint16_t *q;
    int64_t q_row, q_head;
    float *out;
    int64_t o_row, o_head;
    float *part_acc;  // [item][kv head][kMaxWaves * 16 rows][kDim]
    float *part_ml;   // [item][kv head][kMaxWaves * 16 rows][2]
    int32_t n_items, n_kv_heads, group, num_q_heads;
    int32_t rope_offset, half_r;
    float scale;
    int32_t sink_tokens;
    float sink_bias;
};

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &v) {
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Row offset (elements, layer and head included) and meta of position pi of
// a block whose tiles are s_tiles[0, ntiles); *pool tells the source.
__device__ __forceinline__ int64_t bnd_row(const BndArgs &a, const AttnTile *s_tiles, int ntiles,
                                           int pi, int32_t layer, int h, uint32_t *meta,
                                           bool *pool) {
    int lo = 0, hi = ntiles - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_tiles[mid].tok0 <= pi) lo = mid;
        else hi = mid - 1;
    }
    const AttnTile &T = s_tiles[lo];
    const int t = pi - T.tok0;
    const int64_t L = layer;
    uint32_t m = T.cs_idx >= 0 ? static_cast<uint32_t>(T.cs_idx + 1) : 0u;
    if (T.sink_dist + t < a.sink_tokens) m |= kMetaDamp;
    *meta = m;
    switch (T.kind) {
        case kPoolRows:
            *pool = true;
            return L * a.s_layer + (T.a + t) * a.s_tok + h * a.s_head;
        case kPoolPages:
            *pool = true;
            return L * a.s_layer + T.a * a.s_page + static_cast<int64_t>(T.b + t) * a.s_tok +
                   h * a.s_head;
        case kCacheRows:
            *pool = false;
            return L * a.c_layer + T.a * a.c_req + static_cast<int64_t>(T.b + t) * a.c_tok +
                   h * a.c_head;
        default:
            *pool = false;
            return L * a.c_layer + T.a * a.c_page + static_cast<int64_t>(T.b + t) * a.c_tok +
                   h * a.c_head;
    }
}

template <int STYLE>
__global__ void __launch_bounds__(64 * kMaxWaves) bnd_block_kernel(const BndArgs a, int32_t layer) {
    // staged step: slab j < kKSlabs is K, k-step j >> 1, position tile j & 1;
    // slab kKSlabs + j the same for V.  Slot 16 g + p holds dims 32 s + 8 g ..
    // + 8 of position 16 tau + p (the A fragment of lane 16 g + p).
    __shared__ __attribute__((aligned(16))) uint4 s_stage[2][kSlabs * 64];
    __shared__ AttnTile s_tiles[kItemTiles];
    __shared__ uint32_t s_pmeta[2][kStepPos];

    const int item = blockIdx.x / a.n_kv_heads;
    const int h = blockIdx.x - item * a.n_kv_heads;
    const BndItem I = a.items[item];
    const BndEntry E = a.entries[I.entry];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r16 = lane & 15, g = lane >> 4;
    const int W = blockDim.x >> 6;
    const int n_rows = E.n_tok * a.group;  // rows: token j, query head h G + gh at j G + gh
    const int my_row = 16 * wave + r16;    // this lane's row (as a D column)
    const bool row_live = my_row < n_rows;
    const int my_tok = row_live ? my_row / a.group : 0;
    const int my_limit = E.pos0 + my_tok;  // last position the row sees
    const bool wave_live = 16 * wave < n_rows;

    // query fragments (B of S^T): row r16 of the wave's tile, dims 32 s + 8 g
    bf16x8 qf[kKSteps];
    {
        const uint16_t *qr =
            a.q + static_cast<int64_t>(E.row0 + my_tok) * a.q_row +
            static_cast<int64_t>(h * a.group + (row_live ? my_row % a.group : 0)) * a.q_head;
#pragma unroll
        for (int s = 0; s < kKSteps; s++)
            qf[s] = as_bf16x8(row_live ? *reinterpret_cast<const uint4 *>(qr + 32 * s + 8 * g)
                                       : make_uint4(0u, 0u, 0u, 0u));
    }
    f32x4 acc[kDTiles];
#pragma unroll
    for (int t = 0; t < kDTiles; t++) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    for (int b = I.block0; b < I.block1; b++) {
        const AttnBlock B = a.blocks[b];
        const int bpos = a.block_pos[b];
        __syncthreads();
        if (tid < B.ntiles) s_tiles[tid] = a.tiles[B.tile0 + tid];
        __syncthreads();

        auto stage = [&](int p0, int bf) {
#pragma unroll
            for (int tau = 0; tau < 2; tau++) {
                int pi = p0 + 16 * tau + r16;
                const bool valid = pi < B.ntok;
                if (!valid) pi = p0;
                uint32_t meta;
                bool pool;
                const int64_t off = bnd_row(a, s_tiles, B.ntiles, pi, layer, h, &meta, &pool);
                if (wave == 0 && g == 0) s_pmeta[bf][16 * tau + r16] = valid ? meta : 0u;
                const uint16_t *kr = (pool ? a.pool_k : a.cache_k) + off + 8 * g;
                const uint16_t *vr = (pool ? a.pool_v : a.cache_v) + off + 8 * g;
                for (int j = 2 * wave + tau; j < kSlabs; j += 2 * W) {
                    const int s = (j % kKSlabs) >> 1;
                    const uint16_t *src = (j < kKSlabs ? kr : vr) + 32 * s;
                    __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)(&s_stage[bf][j * 64]),
                                                     16, 0, 0);
                }
            }
        };

        stage(0, 0);
        int bf = 0;
        for (int p0 = 0; p0 < B.ntok; p0 += kStepPos, bf ^= 1) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (p0 + kStepPos < B.ntok) stage(p0 + kStepPos, bf ^ 1);

            // ---- turn the rotary pieces of moved chunk rows (K slabs)
            const int pieces = a.half_r / 8;  // (x, y) piece pairs per position
            for (int t = tid; t < pieces * kStepPos; t += 64 * W) {
                const int pos = t / pieces, m = t - pos * pieces;
                const uint32_t cs1 = s_pmeta[bf][pos] & kMetaCs;
                if (cs1 == 0u) continue;
                const double *tab = a.cs + static_cast<int64_t>(cs1 - 1) * a.half_r * 2;
                const int tau = pos >> 4, pp = pos & 15;
                if constexpr (STYLE == PIC_ROPE_HALF) {
                    // x of planes 8 m .. 8 m + 7 in piece (ro + 8 m) / 8, y in
                    // piece (ro + half_r + 8 m) / 8
                    const int px = (a.rope_offset + 8 * m) >> 3, py = px + (a.half_r >> 3);
                    uint4 &kx = s_stage[bf][(2 * (px >> 2) + tau) * 64 + 16 * (px & 3) + pp];
                    uint4 &ky = s_stage[bf][(2 * (py >> 2) + tau) * 64 + 16 * (py & 3) + pp];
                    uint32_t xw[4] = {kx.x, kx.y, kx.z, kx.w}, yw[4] = {ky.x, ky.y, ky.z, ky.w};
#pragma unroll
                    for (int q = 0; q < 8; q++) {
                        const double c = tab[2 * (8 * m + q)], sn = tab[2 * (8 * m + q) + 1];
                        uint32_t &wx = xw[q >> 1], &wy = yw[q >> 1];
                        const int sh = 16 * (q & 1);
                        const double x = static_cast<double>(__uint_as_float(((wx >> sh) & 0xFFFFu) << 16));
                        const double y = static_cast<double>(__uint_as_float(((wy >> sh) & 0xFFFFu) << 16));
                        const uint32_t nx = f64_to_bf16(x * c - y * sn), ny = f64_to_bf16(x * sn + y * c);
                        wx = (wx & ~(0xFFFFu << sh)) | (nx << sh);
                        wy = (wy & ~(0xFFFFu << sh)) | (ny << sh);
                    }
                    kx = make_uint4(xw[0], xw[1], xw[2], xw[3]);
                    ky = make_uint4(yw[0], yw[1], yw[2], yw[3]);
                } else {
                    // whole pairs: piece (ro / 8) + 2 m and the next hold
                    // planes 8 m .. 8 m + 7
#pragma unroll
                    for (int half = 0; half < 2; half++) {
                        const int pc = (a.rope_offset >> 3) + 2 * m + half;
                        uint4 &kw = s_stage[bf][(2 * (pc >> 2) + tau) * 64 + 16 * (pc & 3) + pp];
                        uint32_t w[4] = {kw.x, kw.y, kw.z, kw.w};
#pragma unroll
                        for (int q = 0; q < 4; q++) {
                            const int plane = 8 * m + 4 * half + q;
                            const double c = tab[2 * plane], sn = tab[2 * plane + 1];
                            const double x = bf16_lo(w[q]), y = bf16_hi(w[q]);
                            w[q] = f64_to_bf16(x * c - y * sn) | (f64_to_bf16(x * sn + y * c) << 16);
                        }
                        kw = make_uint4(w[0], w[1], w[2], w[3]);
                    }
                }
            }
            __syncthreads();
            if (!wave_live) continue;  // (the wave still joins every barrier)

            // ---- logits S^T (16 positions x the wave's 16 rows) per tile
            const uint4 *stg = s_stage[bf];
            f32x4 st[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int s = 0; s < kKSteps; s++)
#pragma unroll
                for (int tau = 0; tau < 2; tau++)
                    st[tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        as_bf16x8(stg[(2 * s + tau) * 64 + lane]), qf[s], st[tau], 0, 0, 0);
            float sc[8];
#pragma unroll
            for (int tau = 0; tau < 2; tau++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int pos = 16 * tau + 4 * g + i;
                    const int ctx = bpos + p0 + pos;  // context position
                    float x = st[tau][i] * a.scale;
                    if (s_pmeta[bf][pos] & kMetaDamp) x += a.sink_bias;
                    const bool ok = row_live && p0 + pos < B.ntok && ctx <= my_limit;
                    sc[4 * tau + i] = ok ? x : -INFINITY;
                }
            float mx = sc[0];
#pragma unroll
            for (int k = 1; k < 8; k++) mx = fmaxf(mx, sc[k]);
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float m_new = fmaxf(m_run, mx);
            // a row may have no position yet (all masked): keep it empty
            const float alpha = m_new == -INFINITY ? 1.f : __expf(m_run - m_new);
            float pw[8], psum = 0.f;
#pragma unroll
            for (int k = 0; k < 8; k++) {
                pw[k] = m_new == -INFINITY ? 0.f : __expf(sc[k] - m_new);
                psum += pw[k];
            }
            l_run = l_run * alpha + psum;
            m_run = m_new;
#pragma unroll
            for (int t = 0; t < kDTiles; t++) acc[t] *= alpha;
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const uint32_t h0 = f32_to_bf16(pw[2 * k]), h1 = f32_to_bf16(pw[2 * k + 1]);
                const float r0 = pw[2 * k] - __uint_as_float(h0 << 16);
                const float r1 = pw[2 * k + 1] - __uint_as_float(h1 << 16);
                hi[k] = h0 | (h1 << 16);
                lo[k] = f32_to_bf16(r0) | (f32_to_bf16(r1) << 16);
            }
            const bf16x8 phi = as_bf16x8(make_uint4(hi[0], hi[1], hi[2], hi[3]));
            const bf16x8 plo = as_bf16x8(make_uint4(lo[0], lo[1], lo[2], lo[3]));

            // ---- A = V^T by transposing LDS reads (see attend_mla.hip): lane
            // i of group g addresses position 4 g + i / 4 (+ 16), dims 16 t +
            // 4 (i % 4) .. + 4 of the V slabs
            const char *stg8 = reinterpret_cast<const char *>(stg + kKSlabs * 64);
            const int pq = r16 >> 2, dq = r16 & 3;
#pragma unroll
            for (int t = 0; t < kDTiles; t++) {
                const int gq = 2 * (t & 1) + (dq >> 1);
                const int base = ((2 * (t >> 1)) * 64 + 16 * gq + 4 * g + pq) * 16 + 8 * (dq & 1);
                const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(stg8 + base));
                const s16x4 v1 =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(stg8 + base + 64 * 16));
                const uint2 w0 = __builtin_bit_cast(uint2, v0), w1 = __builtin_bit_cast(uint2, v1);
                const bf16x8 va = as_bf16x8(make_uint4(w0.x, w0.y, w1.x, w1.y));
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi, acc[t], 0, 0, 0);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, plo, acc[t], 0, 0, 0);
            }
        }
    }

    // ---- partial results: O^T D registers hold dims 16 t + 4 g + i of row r16
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
    const int64_t slot = (static_cast<int64_t>(item) * a.n_kv_heads + h) * (kMaxWaves * 16) + my_row;
    float *pa = a.part_acc + slot * kDim;
#pragma unroll
    for (int t = 0; t < kDTiles; t++)
        *reinterpret_cast<float4 *>(pa + 16 * t + 4 * g) =
            make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
    if (g == 0) {
        a.part_ml[2 * slot] = m_run;
        a.part_ml[2 * slot + 1] = l_run;
    }
}

// out[row][q head] = merge of the entry's items (flash-decoding rescaling);
// one workgroup per (entry, local row), a thread per dim.
__global__ void __launch_bounds__(kCombineThreads) bnd_combine_kernel(const BndArgs a) {
    const int e = blockIdx.x;
    const int row = blockIdx.y;  // j G + gh within the KV head's rows
    const int h = blockIdx.z;
    const BndEntry E = a.entries[e];
    if (row >= E.n_tok * a.group) return;
    const int d = threadIdx.x;
    float M = -INFINITY;
    for (int it = E.item0; it < E.item1; it++) {
        const int64_t slot = (static_cast<int64_t>(it) * a.n_kv_heads + h) * (kMaxWaves * 16) + row;
        M = fmaxf(M, a.part_ml[2 * slot]);
    }
    float L = 0.f, O = 0.f;
    for (int it = E.item0; it < E.item1; it++) {
        const int64_t slot = (static_cast<int64_t>(it) * a.n_kv_heads + h) * (kMaxWaves * 16) + row;
        const float m = a.part_ml[2 * slot];
        if (m == -INFINITY) continue;  // the item held no position of this row
        const float f = __expf(m - M);
        L += a.part_ml[2 * slot + 1] * f;
        O += a.part_acc[slot * kDim + d] * f;
    }
    const int tok = row / a.group, gh = row - tok * a.group;
    a.out[static_cast<int64_t>(E.row0 + tok) * a.o_row + (h * a.group + gh) * a.o_head + d] = O / L;
}

// ------------------------------------------------------------------ host

AttnTile advance(AttnTile t, int32_t k) {
    if (t.kind == kPoolRows) t.a += k;
    else t.b += k;
    if (t.sink_dist < kNoSink)
        t.sink_dist = static_cast<int32_t>(std::min<int64_t>(int64_t{t.sink_dist} + k, kNoSink));
    t.ntok -= k;
    return t;
}

struct BndMap {
    std::vector<uint8_t> bytes;
    size_t off_blocks = 0, off_bpos = 0, off_items = 0, off_entries = 0;
    int32_t n_items = 0, n_entries = 0, n_rows = 0;
};

// Relocated entries (dst_offset > 0) of every request in order; entry e
// reads context [0, d_e + n_e) of its request, cut into ceil(L_e / S) items
// of equal length, S the total context over `target`: long prefixes are
// split, short ones stay whole.
// A relocated entry: request, dst_offset, length.
struct Reloc {
    int32_t request;
    int64_t dst;
    int32_t length;
};

BndMap build_bnd_map(const Problem &p, const std::vector<Reloc> &order, int32_t k,
                     int64_t target) {
    std::vector<AttnTile> tiles;
    std::vector<AttnBlock> blocks;
    std::vector<int32_t> bpos;
    std::vector<BndItem> items;
    std::vector<BndEntry> ents;
    int64_t total = 0;
    for (const Reloc &e : order) total += e.dst + std::min(k, e.length);
    int32_t row0 = 0;
    for (const Reloc &e : order) {
        const int32_t r = e.request;
        const int32_t nt = std::min(k, e.length);
        const int64_t L = e.dst + nt;  // context of the entry's rows
        const int64_t per = std::max<int64_t>(kStepPos, (total + target - 1) / target);
        const int64_t n = (L + per - 1) / per;
        const int64_t S = (L + n - 1) / n;
        BndEntry E{r, row0, nt, static_cast<int32_t>(e.dst),
                   static_cast<int32_t>(items.size()), 0, {0, 0}};
        row0 += nt;
        int64_t pos = 0, left = L, item_left = 0;
        AttnBlock blk{r, 0, 0, 0};
        int32_t blk_pos = 0;
        auto close_block = [&]() {
            if (blk.ntiles > 0) {
                blocks.push_back(blk);
                bpos.push_back(blk_pos);
            }
            blk = AttnBlock{r, static_cast<int32_t>(tiles.size()), 0, 0};
            blk_pos = static_cast<int32_t>(pos);
        };
        for (int32_t t = p.req_tile0[r]; t < p.req_tile0[r + 1] && left > 0; t++) {
            AttnTile T = p.atiles[t];
            while (T.ntok > 0 && left > 0) {
                if (item_left == 0) {
                    close_block();
                    if (!items.empty() && items.back().block1 < 0)
                        items.back().block1 = static_cast<int32_t>(blocks.size());
                    items.push_back(BndItem{static_cast<int32_t>(ents.size()),
                                            static_cast<int32_t>(blocks.size()), -1, 0});
                    item_left = std::min(S, left);
                }
                if (blk.ntok == kBlockPos || blk.ntiles == kItemTiles) close_block();
                const int32_t take = static_cast<int32_t>(
                    std::min<int64_t>({int64_t{T.ntok}, item_left, int64_t{kBlockPos - blk.ntok}}));
                AttnTile piece = T;
                piece.ntok = take;
                piece.tok0 = blk.ntok;
                tiles.push_back(piece);
                blk.ntiles++;
                blk.ntok += take;
                item_left -= take;
                left -= take;
                pos += take;
                T = advance(T, take);
                if (item_left == 0) close_block();
            }
        }
        close_block();
        if (!items.empty() && items.back().block1 < 0)
            items.back().block1 = static_cast<int32_t>(blocks.size());
        E.item1 = static_cast<int32_t>(items.size());
        ents.push_back(E);
    }
    BndMap m;
    auto put = [&](const void *src, size_t n) {
        const size_t at = (m.bytes.size() + 15) & ~size_t{15};
        m.bytes.resize(at + n);
        if (n) std::memcpy(m.bytes.data() + at, src, n);
        return at;
    };
    put(tiles.data(), tiles.size() * sizeof(AttnTile));
    m.off_blocks = put(blocks.data(), blocks.size() * sizeof(AttnBlock));
    m.off_bpos = put(bpos.data(), bpos.size() * sizeof(int32_t));
    m.off_items = put(items.data(), items.size() * sizeof(BndItem));
    m.off_entries = put(ents.data(), ents.size() * sizeof(BndEntry));
    m.n_items = static_cast<int32_t>(items.size());
    m.n_entries = static_cast<int32_t>(ents.size());
    m.n_rows = row0;
    return m;
}

int cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    return n;
}

}  // namespace
}  // namespace pic

extern "C" pic_status pic_attend_boundary(pic_plan_t *plan, const pic_kv_view *pool,
                                          const pic_kv_view *cache,
                                          const pic_attend_boundary_args *args, void *stream_) {
    using namespace pic;
    clear_error();
    if (!plan || plan->magic != kPlanMagic) return fail(PIC_ERR_STATE, "invalid or destroyed plan");
    const Problem &p = plan->prob;
    if (!args || !args->q || !args->out)
        return fail(PIC_ERR_INVALID_ARG, "attend arguments, q and out must not be NULL");
    if (p.mode == kInPlace) return fail(PIC_ERR_STATE, "in-place plans have no attention map");
    if (p.shape.dtype != PIC_DTYPE_BF16 || !p.shape.has_v || p.shape.row_dim != kDim)
        return fail(PIC_ERR_INVALID_ARG, "pic_attend_boundary needs a bf16 plan with K and V "
                    "head rows of %d dims", kDim);
    if (p.shape.rope_offset % 8 || p.u.half_r % 8)
        return fail(PIC_ERR_ALIGN, "rotary slice must start and split on 8-dim pieces");
    const int H = p.shape.num_heads;
    if (args->num_q_heads < H || args->num_q_heads % H != 0 || args->num_q_heads / H > 8)
        return fail(PIC_ERR_INVALID_ARG, "num_q_heads %d: need a multiple of %d, at most 8x",
                    args->num_q_heads, H);
    const int G = args->num_q_heads / H;
    if (args->boundary_k < 1 || args->boundary_k * G > kMaxWaves * 16)
        return fail(PIC_ERR_INVALID_ARG, "boundary_k %d: need 1 <= boundary_k x %d <= %d",
                    args->boundary_k, G, kMaxWaves * 16);
    if (args->layer < 0 || args->layer >= p.shape.num_layers)
        return fail(PIC_ERR_INVALID_ARG, "layer %d outside [0, %d)", args->layer,
                    p.shape.num_layers);
    if (args->q_row_stride % 8 || args->q_head_stride % 8 ||
        (reinterpret_cast<uintptr_t>(args->q) & 15u))
        return fail(PIC_ERR_ALIGN, "q rows must be 16-byte aligned");
    if (args->sink_tokens < 0) return fail(PIC_ERR_INVALID_ARG, "negative sink_tokens");
    pic_status st = check_view(pool, 8, true, "pool");
    if (st) return st;
    st = check_view(cache, 8, true, "cache");
    if (st) return st;

    // relocated entries (dst_offset > 0), request by request, in each
    // request's order: the plan's boundaries [request, begin, end]
    std::vector<Reloc> order;
    for (size_t i = 0; i + 2 < p.bounds.size(); i += 3)
        if (p.bounds[i + 1] > 0)
            order.push_back(Reloc{static_cast<int32_t>(p.bounds[i]), p.bounds[i + 1],
                                  static_cast<int32_t>(p.bounds[i + 2] - p.bounds[i + 1])});
    for (const Reloc &e : order) {
        const int32_t r = e.request;
        const int64_t need = e.dst + std::min(args->boundary_k, e.length);
        if (need > p.context[r])
            return fail(PIC_ERR_RANGE, "request %d: boundary rows beyond its context", r);
        if (p.context_bad_page[r] >= 0 &&
            p.context_bad_page[r] * static_cast<int64_t>(p.page_size) < need)
            return fail(PIC_ERR_RANGE, "request %d: context page %d maps outside the cache", r,
                        p.context_bad_page[r]);
    }
    if (order.empty()) return PIC_OK;

    hipStream_t stream = static_cast<hipStream_t>(stream_);
    st = ensure_device_plan(plan, stream_);
    if (st) return st;
    // items: about four rounds of the CU slots (four workgroups of 35 KB LDS
    // per CU, one per KV head and item)
    const int64_t target = std::max<int64_t>(1, 16 * static_cast<int64_t>(cu_count()) / H);
    const int64_t key = (target << 20) | args->boundary_k;
    {
        std::lock_guard<std::mutex> lock(plan->mu);
        hipError_t e;
        if (plan->bnd_key != key) {
            BndMap m = build_bnd_map(p, order, args->boundary_k, target);
            if (plan->d_bnd) {
                e = hipDeviceSynchronize();  // earlier launches may read the old items
                if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
            }
            if (m.bytes.size() > plan->bnd_bytes) {
                if (plan->d_bnd) (void)hipFree(plan->d_bnd);
                plan->d_bnd = nullptr;
                plan->bnd_bytes = 0;
                e = hipMalloc(&plan->d_bnd, m.bytes.size());
                if (e != hipSuccess) {
                    plan->d_bnd = nullptr;
                    return hip_fail(e, "hipMalloc (boundary work items)");
                }
                plan->bnd_bytes = m.bytes.size();
            }
            plan->bnd_host = std::move(m.bytes);
            e = hipMemcpyAsync(plan->d_bnd, plan->bnd_host.data(), plan->bnd_host.size(),
                               hipMemcpyHostToDevice, stream);
            if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (boundary work items)");
            e = hipEventRecord(static_cast<hipEvent_t>(plan->upload_event), stream);
            if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
            plan->bnd_off[0] = m.off_blocks;
            plan->bnd_off[1] = m.off_bpos;
            plan->bnd_off[2] = m.off_items;
            plan->bnd_off[3] = m.off_entries;
            plan->bnd_n_items = m.n_items;
            plan->bnd_n_entries = m.n_entries;
            plan->bnd_key = key;
        }
        const size_t need = static_cast<size_t>(plan->bnd_n_items) * H * (kMaxWaves * 16) *
                            (static_cast<size_t>(kDim) + 2) * sizeof(float);
        if (plan->work_bytes < need) {
            if (plan->d_work) {
                e = hipDeviceSynchronize();
                if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
                (void)hipFree(plan->d_work);
                plan->d_work = nullptr;
                plan->work_bytes = 0;
            }
            e = hipMalloc(&plan->d_work, need);
            if (e != hipSuccess) {
                plan->d_work = nullptr;
                return hip_fail(e, "hipMalloc (attention workspace)");
            }
            plan->work_bytes = need;
        }
    }
    const uint8_t *dm = static_cast<const uint8_t *>(plan->d_mem);
    const uint8_t *bm = static_cast<const uint8_t *>(plan->d_bnd);
    BndArgs a{};
    a.tiles = reinterpret_cast<const AttnTile *>(bm);
    a.blocks = reinterpret_cast<const AttnBlock *>(bm + plan->bnd_off[0]);
    a.block_pos = reinterpret_cast<const int32_t *>(bm + plan->bnd_off[1]);
    a.items = reinterpret_cast<const BndItem *>(bm + plan->bnd_off[2]);
    a.entries = reinterpret_cast<const BndEntry *>(bm + plan->bnd_off[3]);
    a.cs = reinterpret_cast<const double *>(dm + plan->staged.off_cs);
    a.pool_k = static_cast<const uint16_t *>(pool->k);
    a.pool_v = static_cast<const uint16_t *>(pool->v);
    a.cache_k = static_cast<const uint16_t *>(cache->k);
    a.cache_v = static_cast<const uint16_t *>(cache->v);
    a.s_layer = pool->layer_stride;
    a.s_tok = pool->token_stride;
    a.s_head = pool->head_stride;
    a.s_page = pool->page_stride;
    a.c_layer = cache->layer_stride;
    a.c_tok = cache->token_stride;
    a.c_head = cache->head_stride;
    a.c_page = cache->page_stride;
    a.c_req = cache->request_stride;
    a.q = static_cast<const uint16_t *>(args->q);
    a.q_row = args->q_row_stride;
    a.q_head = args->q_head_stride;
    a.out = args->out;
    a.o_row = args->out_row_stride;
    a.o_head = args->out_head_stride;
    const size_t acc_elems =
        static_cast<size_t>(plan->bnd_n_items) * H * (kMaxWaves * 16) * static_cast<size_t>(kDim);
    a.part_acc = static_cast<float *>(plan->d_work);
    a.part_ml = static_cast<float *>(plan->d_work) + acc_elems;
    a.n_items = plan->bnd_n_items;
    a.n_kv_heads = H;
    a.group = G;
    a.num_q_heads = args->num_q_heads;
    a.rope_offset = p.shape.rope_offset;
    a.half_r = p.u.half_r;
    a.scale = args->scale;
    a.sink_tokens = args->sink_tokens;
    a.sink_bias = args->sink_bias;
    const int waves = (args->boundary_k * G + 15) / 16;
    const dim3 grid(static_cast<unsigned>(a.n_items) * static_cast<unsigned>(H));
    if (p.style == PIC_ROPE_HALF)
        hipLaunchKernelGGL(bnd_block_kernel<PIC_ROPE_HALF>, grid, dim3(64 * waves), 0, stream, a,
                           args->layer);
    else
        hipLaunchKernelGGL(bnd_block_kernel<PIC_ROPE_INTERLEAVED>, grid, dim3(64 * waves), 0,
                           stream, a, args->layer);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "boundary attention kernel launch");
    hipLaunchKernelGGL(bnd_combine_kernel,
                       dim3(static_cast<unsigned>(plan->bnd_n_entries),
                            static_cast<unsigned>(args->boundary_k * G), static_cast<unsigned>(H)),
                       dim3(kCombineThreads), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "boundary attention combine launch");
    return PIC_OK;
}
