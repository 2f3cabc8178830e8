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
// Work: all boundary rows of a request (tokens x the GQA group's query heads)
// share one pass over the request's context.  A workgroup of 8 waves takes
// one KV head, one work item (a run of positions of the request, cut on the
// host per launch shape) and up to 256 rows: each wave holds two row tiles of
// 16 adjacent rows (more rows take more row sets, which read the same rows
// on the same XCD at about the same time).  Per step of 64 positions:
//   - the step's K and V rows of the KV head (32 KB) go from HBM straight
//     into LDS (global_load_lds_dwordx4), in the MFMA A-fragment layout,
//     double-buffered across steps; each wave stages one 16-position tile's
//     K or V, its row addresses from per-tile records built once per block;
//   - rotary pieces of moved chunk rows are turned in LDS (fp64, rounded to
//     bf16 by the stitch's own code, rotate.hpp), with the block's shift
//     tables copied to LDS once;
//   - S^T = K Q^T (v_mfma_f32_16x16x32_bf16): each K fragment is read once
//     and used for both of the wave's row tiles; causal limit per row;
//   - online softmax per row in log2 units, with a lazy running max (the
//     accumulator is rescaled only when a logit passes the reference by
//     2^12), weights split into hi + lo bf16;
//   - O^T += V^T P^T with the weights taken from the S^T D registers and
//     each V^T fragment (transposing LDS reads) used for both row tiles.
// Steps past every row of a wave are skipped by that wave.  A partial (max,
// sum, accumulator) per (item, KV head, row) is merged by bnd_combine_kernel.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "lds_load.hpp"
#include "pic_internal.hpp"
#include "rotate.hpp"

namespace pic {

pic_status hip_fail(hipError_t e, const char *what);  // stitch.hip

namespace {

constexpr int kDim = 128;                 // head row
constexpr int kKSteps = kDim / 32;        // MFMA k-steps
constexpr int kDTiles = kDim / 16;        // output tiles of 16 dims
#ifndef PIC_BND_POS_TILES
#define PIC_BND_POS_TILES 4
#endif
constexpr int kPT = PIC_BND_POS_TILES;   // 16-position tiles per step (2 or 4)
constexpr int kStepPos = 16 * kPT;        // positions per step
constexpr int kSlabs = 2 * kKSteps * kPT; // 1 KB slabs per step: K, then V
static_assert(kPT == 2 || kPT == 4, "position tiles per step");
constexpr int kNBuf = 4;                  // staging buffers (computed, turned, two loading)
#ifndef PIC_BND_WAVES
#define PIC_BND_WAVES 8
#endif
constexpr int kWaves = PIC_BND_WAVES;     // waves per workgroup
constexpr int kMaxTT = 2;                 // row tiles per wave at most (registers)
constexpr int kItemTiles = 64;            // map tiles per block at most
constexpr int kBlockPos = 4096;           // positions per block at most
constexpr int kBlockTabs = 4;             // shift tables per block at most (kept in LDS)
constexpr int kMaxHalf = kDim / 2;        // rotary planes at most
constexpr float kLazy = 12.f;             // running-max slack of the online softmax (log2 units)
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxItems = 64;            // work items per request at most (one combine wave)


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef const void __attribute__((address_space(1))) *gptr_t;
typedef void __attribute__((address_space(3))) *lptr_t;

// A request with boundary rows: its boundary tokens are global rows [row0,
// row0 + n_tok) (entry by entry, token by token), the last position each
// sees is limit[row0 + i]; its work items are [item0, item1).
struct BndReq {
    int32_t row0;
    int32_t n_tok;
    int32_t item0;
    int32_t item1;
};

// A work item: blocks [block0, block1) of request `req` (index into the
// request table), covering context positions [pos_a, pos_b).
struct BndItem {
    int32_t req;
    int32_t block0;
    int32_t block1;
    int32_t pos_a;
};

struct BndArgs {
    const AttnTile *tiles;    // blocks' tiles (tok0: position in the block)
    const AttnBlock *blocks;  // request, tile0, ntiles, ntok
    const int32_t *block_pos; // context position of every block's first token
    const int32_t *block_tabs;  // [block][kBlockTabs] shift tables its tiles use (-1: none)
    const BndItem *items;
    const BndReq *reqs;
    const int32_t *limit;     // last position every boundary token sees
    const double *cs;
    const uint16_t *pool_k, *pool_v, *cache_k, *cache_v;
    int64_t s_layer, s_tok, s_head, s_page;
    int64_t c_layer, c_tok, c_head, c_page, c_req;
    const uint16_t *q;
    int64_t q_row, q_head;
    float *out;
    int64_t o_row, o_head;
    float *part_acc;  // [item][kv head][row slots][kDim]
    float *part_ml;   // [item][kv head][row slots][2]
    int32_t n_items, n_kv_heads, group, num_q_heads;
    int32_t row_slots;  // rows per (item, KV head): the most rows of a request, in tiles
    int32_t n_sets;     // row sets per item
    int32_t rope_offset, half_r;
    float scale;
    int32_t sink_tokens;
    float sink_bias;
};

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &v) {
    return __builtin_bit_cast(bf16x8, v);
}

// max over the four lanes of a row (lanes r, r + 16, r + 32, r + 48): the
// 32-lane swap pairs lane i with i ^ 32, the 16-lane swap i with i ^ 16
__device__ __forceinline__ float row_max(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// A map tile as the staging reads it: the row of block position pi is
// off0 + pi * token stride (elements, layer and head included) in the pool
// (info bit kInfoPool) or the cache; info also holds the tile's shift-table
// slot + 1 (bits 0-2, 0: rows not turned) and how many of its first
// positions take the damping bias (bits 8-31).
struct StageTile {
    int64_t off0;
    int32_t tok0;
    uint32_t info;
};
constexpr uint32_t kInfoPool = 1u << 3;

__device__ __forceinline__ StageTile stage_tile(const BndArgs &a, const AttnTile &T, int slot,
                                                int32_t layer, int h) {
    const int64_t L = layer;
    int64_t off0;
    bool pool = true;
    switch (T.kind) {
        case kPoolRows:
            off0 = L * a.s_layer + h * a.s_head + (T.a - T.tok0) * a.s_tok;
            break;
        case kPoolPages:
            off0 = L * a.s_layer + h * a.s_head + T.a * a.s_page +
                   static_cast<int64_t>(T.b - T.tok0) * a.s_tok;
            break;
        case kCacheRows:
            pool = false;
            off0 = L * a.c_layer + h * a.c_head + T.a * a.c_req +
                   static_cast<int64_t>(T.b - T.tok0) * a.c_tok;
            break;
        default:
            pool = false;
            off0 = L * a.c_layer + h * a.c_head + T.a * a.c_page +
                   static_cast<int64_t>(T.b - T.tok0) * a.c_tok;
            break;
    }
    // positions tok0 .. tok0 + damp - 1 lie within sink_tokens of their chunk's start
    const int64_t damp = std::min<int64_t>(std::max<int64_t>(int64_t{a.sink_tokens} - T.sink_dist, 0),
                                           (1 << 24) - 1);
    const uint32_t info = static_cast<uint32_t>(slot + 1) | (pool ? kInfoPool : 0u) |
                          (static_cast<uint32_t>(damp) << 8);
    return StageTile{off0, T.tok0, info};
}

// Rows per workgroup: 8 waves x TT tiles x 16.
template <int STYLE, int TT>
__global__ void __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2)))
bnd_block_kernel(const BndArgs a, int32_t layer) {
    // staged step: slab kind * kKSteps * kPT + s * kPT + tau (kind 0: K, 1:
    // V) holds dims 32 s .. 32 s + 31 of positions 16 tau .. 16 tau + 15; its
    // slot 16 g + p holds dims 32 s + 8 g .. + 8 of position 16 tau + p (the
    // A fragment of lane 16 g + p)
    __shared__ __attribute__((aligned(16))) uint4 s_stage[kNBuf][kSlabs * 64];
    __shared__ __attribute__((aligned(16))) double2 s_cs[kBlockTabs][kMaxHalf];  // block's shift tables
    __shared__ __attribute__((aligned(8))) float2 s_cs32[kBlockTabs][kMaxHalf];  // the same, fp32
    __shared__ StageTile s_tiles[kItemTiles];
    __shared__ uint8_t s_tile_of[kBlockPos];  // map tile of every block position
    __shared__ uint32_t s_pslot[kNBuf][kStepPos];                       // shift-table slot + 1 (0: not turned)
    __shared__ __attribute__((aligned(16))) float s_pbias[kNBuf][kStepPos];  // damping, -inf past the block
    __shared__ __attribute__((aligned(4))) uint8_t s_pflag[kNBuf][4];  // position tile has a nonzero bias

    // grid: runs of 8 (item, KV head) pairs c, each run once per row set;
    // workgroup w goes to XCD w % 8, so every set of one pair shares an XCD
    // (and its L2) and reads the same rows close together in time
    const int w = blockIdx.x;
    const int c = (w / (8 * a.n_sets)) * 8 + (w & 7);
    const int set = (w >> 3) % a.n_sets;
    if (c >= a.n_items * a.n_kv_heads) return;
    const int h = c % a.n_kv_heads;
    const int item = c / a.n_kv_heads;
    const BndItem I = a.items[item];
    const BndReq Q = a.reqs[I.req];
    const int n_rows = Q.n_tok * a.group;  // row = token i x G + query head gh of KV head h
    const int set_row0 = set * (kWaves * TT * 16);
    if (set_row0 >= n_rows) return;  // uniform over the workgroup
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r16 = lane & 15, g = lane >> 4;

    // the wave's row tiles: rows set_row0 + 16 (TT wave + k) + r16, adjacent
    // rows (mostly one entry) so that they end at about the same step
    bf16x8 qf[TT][kKSteps];
    int limit[TT];  // the row's last position (rows past the request's: none)
#pragma unroll
    for (int k = 0; k < TT; k++) {
        const int row = set_row0 + 16 * (TT * wave + k) + r16;
        const bool live = row < n_rows;
        const int tok = live ? row / a.group : 0;
        limit[k] = live ? a.limit[Q.row0 + tok] : -1;
        const uint16_t *qr = a.q + static_cast<int64_t>(Q.row0 + tok) * a.q_row +
                             static_cast<int64_t>(h * a.group + (live ? row % a.group : 0)) *
                                 a.q_head;
#pragma unroll
        for (int s = 0; s < kKSteps; s++)
            qf[k][s] = as_bf16x8(live ? *reinterpret_cast<const uint4 *>(qr + 32 * s + 8 * g)
                                      : make_uint4(0u, 0u, 0u, 0u));
    }
    // per tile, the latest last position of its rows: a step past it is
    // skipped (rows past the request: -1)
    int tile_last[TT];
    // and the earliest last position of its live rows: a step that ends by
    // then needs no causal mask for the tile
    int tile_first[TT];
#pragma unroll
    for (int k = 0; k < TT; k++) {
        int x = limit[k], y = limit[k] < 0 ? INT32_MAX : limit[k];
        for (int m = 1; m < 16; m <<= 1) {
            x = max(x, __shfl_xor(x, m, 64));
            y = min(y, __shfl_xor(y, m, 64));
        }
        tile_last[k] = x;
        tile_first[k] = y;
    }
    const float scale2 = a.scale * kLog2e;  // logits in log2 units (exp2 weights)
    const float bias2 = a.sink_bias * kLog2e;
    // the last position any row of the workgroup sees: later positions are
    // neither staged nor turned, and a workgroup whose rows all end before
    // its item returns at once (the merge never reads its partial results)
    __shared__ int s_last[kWaves];
    if (lane == 0) {
        int x = tile_last[0];
#pragma unroll
        for (int k = 1; k < TT; k++) x = max(x, tile_last[k]);
        s_last[wave] = x;
    }
    __syncthreads();
    int wg_last = s_last[0];
#pragma unroll
    for (int v = 1; v < kWaves; v++) wg_last = max(wg_last, s_last[v]);
    if (wg_last < I.pos_a) return;  // uniform over the workgroup

    f32x4 acc[TT][kDTiles];
    float m_run[TT], l_run[TT];
#pragma unroll
    for (int k = 0; k < TT; k++) {
#pragma unroll
        for (int t = 0; t < kDTiles; t++) acc[k][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run[k] = -INFINITY;
        l_run[k] = 0.f;
    }
    const int half_r = a.half_r;
    // staging roles: the wave loads position tile my_tau of every step, the
    // slabs my_j0 .. my_j0 + kSlabsPerWave - 1 of that tile's K then V slabs
    constexpr int kWavesPerTau = kWaves / kPT;
    constexpr int kSlabsPerWave = 2 * kKSteps / kWavesPerTau;
    const int my_tau = wave / kWavesPerTau;
    const int my_j0 = (wave % kWavesPerTau) * kSlabsPerWave;

    for (int b = I.block0; b < I.block1; b++) {
        const AttnBlock B = a.blocks[b];
        const int bpos = a.block_pos[b];
        if (bpos > wg_last) break;  // uniform
        const int ntok = min(B.ntok, wg_last + 1 - bpos);  // positions some row sees
        __syncthreads();
        if (tid < B.ntiles) {
            const AttnTile T = a.tiles[B.tile0 + tid];
            int sl = -1;
#pragma unroll
            for (int j = 0; j < kBlockTabs; j++)
                if (T.cs_idx >= 0 && a.block_tabs[kBlockTabs * b + j] == T.cs_idx) sl = j;
            s_tiles[tid] = stage_tile(a, T, sl, layer, h);
        }
        for (int i = tid; i < kBlockTabs * half_r; i += 64 * kWaves) {
            const int j = i / half_r, pl = i - j * half_r;
            const int tab = a.block_tabs[kBlockTabs * b + j];
            if (tab >= 0) {
                const double *src = a.cs + (static_cast<int64_t>(tab) * half_r + pl) * 2;
                s_cs[j][pl] = make_double2(src[0], src[1]);
                s_cs32[j][pl] = make_float2(static_cast<float>(src[0]), static_cast<float>(src[1]));
            }
        }
        __syncthreads();
        // the map tile of every position the block stages (the last tile
        // starting at or before it; tiles are in position order), so that a
        // staging lane finds its tile with one LDS read
        static_assert(kItemTiles <= 256, "tile index in a byte");
        for (int pp = tid; pp < ntok; pp += 64 * kWaves) {
            int lo = 0, hi = B.ntiles - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (s_tiles[mid].tok0 <= pp) lo = mid;
                else hi = mid - 1;
            }
            s_tile_of[pp] = static_cast<uint8_t>(lo);
        }
        __syncthreads();

        auto stage = [&](int p0, int bf) {
            int pi = p0 + 16 * my_tau + r16;
            const bool valid = pi < ntok;
            if (!valid) pi = p0;
            const StageTile T = s_tiles[s_tile_of[pi]];
            const bool pool = T.info & kInfoPool;
            const int64_t off = T.off0 + static_cast<int64_t>(pi) * (pool ? a.s_tok : a.c_tok);
            if (my_j0 == 0) {
                const bool damp = static_cast<uint32_t>(pi - T.tok0) < (T.info >> 8);
                const uint64_t biased = __ballot(g == 0 && (!valid || damp));
                if (g == 0) {
                    s_pslot[bf][16 * my_tau + r16] = valid ? (T.info & 7u) : 0u;
                    s_pbias[bf][16 * my_tau + r16] = valid ? (damp ? bias2 : 0.f) : -INFINITY;
                }
                if (lane == 0) s_pflag[bf][my_tau] = biased != 0;
            }
            const uint16_t *kr = (pool ? a.pool_k : a.cache_k) + off + 8 * g;
            const uint16_t *vr = (pool ? a.pool_v : a.cache_v) + off + 8 * g;
#pragma unroll
            for (int i = 0; i < kSlabsPerWave; i++) {
                const int jl = my_j0 + i;  // kind * kKSteps + s
                const int kind = jl / kKSteps, s = jl % kKSteps;
                const uint16_t *src = (kind == 0 ? kr : vr) + 32 * s;
                const int slab = kind * kKSteps * kPT + s * kPT + my_tau;
                load_lds16(src, &s_stage[bf][slab * 64]);
            }
        };

        // turn the rotary pieces of moved chunk rows (K slabs) of buffer bb:
        // unit (position, 8-plane group m, half hh) turns 4 planes
        auto turn = [&](int bb) {
            // unit (position, 8-plane group m): the lanes of a wave take one
            // group of consecutive positions, so their 16-byte LDS pieces are
            // contiguous (no bank conflicts) and their cos/sin reads coincide
            const int units = (half_r / 8) * kStepPos;
            for (int u = tid; u < units; u += 64 * kWaves) {
                const int pos = u % kStepPos, m = u / kStepPos;
                const uint32_t slot1 = s_pslot[bb][pos];
                if (slot1 == 0u) continue;
                const double2 *tab = s_cs[slot1 - 1] + 8 * m;
                const float2 *tab32 = s_cs32[slot1 - 1] + 8 * m;
                const int tau = pos >> 4, pp = pos & 15;
                // the unit's two 16-byte pieces: half pairing, x of planes
                // 8 m .. + 8 in piece (ro + 8 m) / 8 and their y half_r dims on;
                // interleaved, whole pairs in pieces ro / 8 + 2 m and the next
                int pa, pb;
                if constexpr (STYLE == PIC_ROPE_HALF) {
                    pa = (a.rope_offset + 8 * m) >> 3;
                    pb = pa + (half_r >> 3);
                } else {
                    pa = (a.rope_offset >> 3) + 2 * m;
                    pb = pa + 1;
                }
                uint4 &ka = s_stage[bb][((pa >> 2) * kPT + tau) * 64 + 16 * (pa & 3) + pp];
                uint4 &kb = s_stage[bb][((pb >> 2) * kPT + tau) * 64 + 16 * (pb & 3) + pp];
                const uint4 va = ka, vb = kb;
                const uint32_t wa[4] = {va.x, va.y, va.z, va.w}, wb[4] = {vb.x, vb.y, vb.z, vb.w};
                // fp32 first; the fp64 turn only for the planes where it could
                // round otherwise (redo[p]: the lanes whose plane p needs it),
                // each plane under its own branch so that a wave pays for the
                // planes some lane flagged, not for the whole unit
                uint32_t na[4], nb[4];
                uint64_t redo[8];
                if constexpr (STYLE == PIC_ROPE_HALF) {
#pragma unroll
                    for (int k = 0; k < 4; k++) {  // planes 2 k, 2 k + 1: word k of each piece
                        float rx0, ry0, rx1, ry1;
                        const float2 c0 = tab32[2 * k], c1 = tab32[2 * k + 1];
                        redo[2 * k] = __ballot(turn_f32(__uint_as_float(wa[k] << 16),
                                                        __uint_as_float(wb[k] << 16), c0.x, c0.y, &rx0, &ry0));
                        redo[2 * k + 1] = __ballot(turn_f32(__uint_as_float(wa[k] & 0xFFFF0000u),
                                                            __uint_as_float(wb[k] & 0xFFFF0000u), c1.x, c1.y,
                                                            &rx1, &ry1));
                        na[k] = pack2_bf16(rx0, rx1);
                        nb[k] = pack2_bf16(ry0, ry1);
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < 4; k++) {  // plane k: word k of piece a; plane 4 + k of piece b
                        float rx, ry;
                        const float2 ca = tab32[k], cb = tab32[4 + k];
                        redo[k] = __ballot(turn_f32(__uint_as_float(wa[k] << 16),
                                                    __uint_as_float(wa[k] & 0xFFFF0000u), ca.x, ca.y, &rx, &ry));
                        na[k] = pack2_bf16(rx, ry);
                        redo[4 + k] = __ballot(turn_f32(__uint_as_float(wb[k] << 16),
                                                        __uint_as_float(wb[k] & 0xFFFF0000u), cb.x, cb.y, &rx, &ry));
                        nb[k] = pack2_bf16(rx, ry);
                    }
                }
                uint64_t any_redo = 0;
#pragma unroll
                for (int pl = 0; pl < 8; pl++) any_redo |= redo[pl];
                if (any_redo != 0) {  // uniform
#pragma unroll
                    for (int pl = 0; pl < 8; pl++) {
                        if (!((redo[pl] >> lane) & 1)) continue;
                        const double2 cs = tab[pl];
                        if constexpr (STYLE == PIC_ROPE_HALF) {
                            // plane pl: half pl % 2 of word pl / 2 in both pieces
                            const int k = pl >> 1, sh = 16 * (pl & 1);
                            const double x = (pl & 1) ? bf16_hi(wa[k]) : bf16_lo(wa[k]);
                            const double y = (pl & 1) ? bf16_hi(wb[k]) : bf16_lo(wb[k]);
                            const uint32_t keep = 0xFFFF0000u >> sh;
                            na[k] = (na[k] & keep) | (f64_to_bf16(x * cs.x - y * cs.y) << sh);
                            nb[k] = (nb[k] & keep) | (f64_to_bf16(x * cs.y + y * cs.x) << sh);
                        } else {
                            // plane pl: word pl % 4 of piece a (pl < 4) or b
                            const uint32_t w = pl < 4 ? wa[pl & 3] : wb[pl & 3];
                            const double x = bf16_lo(w), y = bf16_hi(w);
                            const uint32_t r = pack_bf16(x * cs.x - y * cs.y, x * cs.y + y * cs.x);
                            if (pl < 4) na[pl & 3] = r;
                            else nb[pl & 3] = r;
                        }
                    }
                }
                ka = make_uint4(na[0], na[1], na[2], na[3]);
                kb = make_uint4(nb[0], nb[1], nb[2], nb[3]);
            }
        };

        // four buffers: step i is computed while step i + 1 is turned and
        // steps i + 2, i + 3 load, with one barrier per step.  Each stage call
        // issues kSlabsPerWave loads per wave, and they complete in order, so
        // waiting until at most n loads are outstanding leaves the newest n
        // (a later step's) in flight.
        auto wait_loads = [](int n) {
            if (n >= 2 * kSlabsPerWave) wait_vm<2 * kSlabsPerWave>();
            else if (n >= kSlabsPerWave) wait_vm<kSlabsPerWave>();
            else wait_vm<0>();
        };
        const int nsteps = (ntok + kStepPos - 1) / kStepPos;
        stage(0, 0);
        if (nsteps > 1) stage(kStepPos, 1);
        if (nsteps > 2) stage(2 * kStepPos, 2);
        wait_loads((nsteps > 1 ? kSlabsPerWave : 0) + (nsteps > 2 ? kSlabsPerWave : 0));
        __syncthreads();
        turn(0);
        for (int i = 0; i < nsteps; i++) {
            const int p0 = i * kStepPos;
            // step i + 1's loads are in (step i + 2's may not be); after the
            // barrier every wave's are, step i is turned, and step i - 1's
            // buffer is free
            wait_loads(i + 2 < nsteps ? kSlabsPerWave : 0);
            __syncthreads();
            const int cur_bf = i & (kNBuf - 1);
            if (i + 3 < nsteps) stage(p0 + 3 * kStepPos, (i + 3) & (kNBuf - 1));
            if (i + 1 < nsteps) turn((i + 1) & (kNBuf - 1));


            const int step_pos = bpos + p0;  // context position of the step's first row
            bool any = false;
#pragma unroll
            for (int k = 0; k < TT; k++) any = any || tile_last[k] >= step_pos;
            if (!any) continue;  // (the wave still joins every barrier)
            // every tile of an active wave is computed, without branches, so
            // that the matrix and vector work of its tiles interleave; rows
            // past their last position are masked to weight 0

            // ---- logits S^T: each K fragment serves every tile
            const uint4 *stg = s_stage[cur_bf];
            f32x4 st[TT][kPT];
#pragma unroll
            for (int k = 0; k < TT; k++)
#pragma unroll
                for (int tau = 0; tau < kPT; tau++) st[k][tau] = f32x4{0.f, 0.f, 0.f, 0.f};
            // (K fragments read one k-step ahead of their products, fenced so
            // that the compiler keeps two k-steps of them in registers, not four)
            bf16x8 kf[kPT];
#pragma unroll
            for (int tau = 0; tau < kPT; tau++) kf[tau] = as_bf16x8(stg[tau * 64 + lane]);
#pragma unroll
            for (int s = 0; s < kKSteps; s++) {
                bf16x8 kn[kPT];
                if (s + 1 < kKSteps) {
#pragma unroll
                    for (int tau = 0; tau < kPT; tau++)
                        kn[tau] = as_bf16x8(stg[((s + 1) * kPT + tau) * 64 + lane]);
                }
#pragma unroll
                for (int tau = 0; tau < kPT; tau++)
#pragma unroll
                    for (int k = 0; k < TT; k++)
                        st[k][tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[tau], qf[k][s], st[k][tau], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                if (s + 1 < kKSteps) {
#pragma unroll
                    for (int tau = 0; tau < kPT; tau++) kf[tau] = kn[tau];
                }
            }
            // ---- online softmax per row (log2 units).  The running max is
            // kept until a logit passes it by kLazy (weights stay below
            // 2^kLazy; the merge uses the same reference), so the accumulator
            // is seldom rescaled.
            // A step with no damped or missing position that ends before
            // every live row of the wave's tiles does (the usual case) needs
            // neither bias nor mask: its logits stay unscaled in st, the row
            // max is scaled after the reduction (exact: rounding is
            // monotonic and scale2 > 0), and the weights take the scale in
            // the exponent's fma.  Otherwise st becomes the scaled, biased,
            // masked logits and the weights multiply by 1.
            bool fast = (__builtin_amdgcn_readfirstlane(*reinterpret_cast<const uint32_t *>(s_pflag[cur_bf])) &
                         (0xFFFFFFFFu >> (32 - 8 * kPT))) == 0u;
#pragma unroll
            for (int k = 0; k < TT; k++) fast = fast && tile_first[k] >= step_pos + kStepPos - 1;
            const float wmul = fast ? scale2 : 1.f;
            float alpha[TT], m_use[TT];
            bool bump_any = false;
#pragma unroll
            for (int k = 0; k < TT; k++) {
                float mx = -INFINITY;
                if (fast) {
#pragma unroll
                    for (int tau = 0; tau < kPT; tau++)
#pragma unroll
                        for (int i = 0; i < 4; i++) mx = fmaxf(mx, st[k][tau][i]);
                    mx = row_max(mx) * scale2;
                } else {
                    // position terms (D registers: positions 16 tau + 4 g + i)
                    const int lim = limit[k] - step_pos - 4 * g;  // position 16 tau + i must be <= lim
#pragma unroll
                    for (int tau = 0; tau < kPT; tau++) {
                        const f32x4 pb = *reinterpret_cast<const f32x4 *>(&s_pbias[cur_bf][16 * tau + 4 * g]);
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            const float x = fmaf(st[k][tau][i], scale2, pb[i]);
                            st[k][tau][i] = 16 * tau + i <= lim ? x : -INFINITY;
                            mx = fmaxf(mx, st[k][tau][i]);
                        }
                    }
                    mx = row_max(mx);
                }
                // (-inf + kLazy stays -inf: a row's first finite logit bumps)
                const bool bump = mx > m_run[k] + kLazy;
                const float m_new = bump ? mx : m_run[k];
                alpha[k] = bump ? __builtin_amdgcn_exp2f(m_run[k] - m_new) : 1.f;
                m_use[k] = m_new == -INFINITY ? 0.f : m_new;  // all -inf: weights 0
                m_run[k] = m_new;
                bump_any = bump_any || bump;
            }
            if (__any(bump_any)) {
#pragma unroll
                for (int k = 0; k < TT; k++)
#pragma unroll
                    for (int t = 0; t < kDTiles; t++) acc[k][t] *= alpha[k];
            }
            // ---- weights as B fragments (hi + lo bf16) of the value product,
            // 32 positions (two position tiles) per k-step kk
            const char *stg8 = reinterpret_cast<const char *>(stg + kKSteps * kPT * 64);
            const int pq = r16 >> 2, dq = r16 & 3;
#pragma unroll
            for (int kk = 0; kk < kPT / 2; kk++) {
                bf16x8 phi[TT], plo[TT];
#pragma unroll
                for (int k = 0; k < TT; k++) {
                    float pw[8];
                    const float neg_m = -m_use[k];
#pragma unroll
                    for (int q = 0; q < 8; q++)
                        pw[q] = __builtin_amdgcn_exp2f(fmaf(st[k][2 * kk + (q >> 2)][q & 3], wmul, neg_m));
                    const float psum =
                        ((pw[0] + pw[1]) + (pw[2] + pw[3])) + ((pw[4] + pw[5]) + (pw[6] + pw[7]));
                    l_run[k] = (kk == 0 ? l_run[k] * alpha[k] : l_run[k]) + psum;
                    uint32_t hi[4], lo[4];
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        const f32x2 pr = {pw[2 * q], pw[2 * q + 1]};
                        hi[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
                        const f32x2 rr = {pw[2 * q] - __uint_as_float(hi[q] << 16),
                                          pw[2 * q + 1] - __uint_as_float(hi[q] & 0xFFFF0000u)};
                        lo[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(rr, bf16x2));
                    }
                    phi[k] = as_bf16x8(make_uint4(hi[0], hi[1], hi[2], hi[3]));
                    plo[k] = as_bf16x8(make_uint4(lo[0], lo[1], lo[2], lo[3]));
                }
                // ---- A = V^T by transposing LDS reads (see attend_mla.hip),
                // each fragment used for every tile
#pragma unroll
                for (int t = 0; t < kDTiles; t++) {
                    const int gq = 2 * (t & 1) + (dq >> 1);
                    const int base =
                        (((t >> 1) * kPT + 2 * kk) * 64 + 16 * gq + 4 * g + pq) * 16 + 8 * (dq & 1);
                    const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(stg8 + base));
                    const s16x4 v1 =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(stg8 + base + 64 * 16));
                    const uint2 w0 = __builtin_bit_cast(uint2, v0), w1 = __builtin_bit_cast(uint2, v1);
                    const bf16x8 va = as_bf16x8(make_uint4(w0.x, w0.y, w1.x, w1.y));
#pragma unroll
                    for (int k = 0; k < TT; k++) {
                        acc[k][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi[k], acc[k][t], 0, 0, 0);
                        acc[k][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, plo[k], acc[k][t], 0, 0, 0);
                    }
                }
            }
        }
    }

    // ---- partial results of the tiles with rows that reach this item:
    // O^T D registers hold dims 16 t + 4 g + i of row r16
#pragma unroll
    for (int k = 0; k < TT; k++) {
        if (tile_last[k] < I.pos_a) continue;
        float l = l_run[k];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        const int row = set_row0 + 16 * (TT * wave + k) + r16;
        const int64_t slot = (static_cast<int64_t>(item) * a.n_kv_heads + h) * a.row_slots + row;
        float *pa = a.part_acc + slot * kDim;
#pragma unroll
        for (int t = 0; t < kDTiles; t++)
            *reinterpret_cast<float4 *>(pa + 16 * t + 4 * g) =
                make_float4(acc[k][t][0], acc[k][t][1], acc[k][t][2], acc[k][t][3]);
        if (g == 0) {
            a.part_ml[2 * slot] = m_run[k];
            a.part_ml[2 * slot + 1] = l;
        }
    }
}

// out[token][q head] = merge of the request's items that the token's row
// reaches (flash-decoding rescaling).  One wave per (request, row, KV head):
// lane t holds item t's max and sum (a request has at most 64 items), then
// every lane merges two dims.
__global__ void __launch_bounds__(64) bnd_combine_kernel(const BndArgs a) {
    const BndReq Q = a.reqs[blockIdx.y];
    const int row = blockIdx.x;  // token i x G + gh
    const int h = blockIdx.z;
    if (row >= Q.n_tok * a.group) return;
    const int lane = threadIdx.x;
    const int tok = row / a.group, gh = row - tok * a.group;
    const int lim = a.limit[Q.row0 + tok];
    const int it = Q.item0 + lane;
    const int64_t slot = (static_cast<int64_t>(it) * a.n_kv_heads + h) * a.row_slots + row;
    // items are in position order; those past the row's limit hold nothing
    const bool mine = it < Q.item1 && a.items[it].pos_a <= lim;
    const float m = mine ? a.part_ml[2 * slot] : -INFINITY;
    const float lsum = mine ? a.part_ml[2 * slot + 1] : 0.f;
    float M = m;
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    const float f = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M);  // log2 units
    float L = lsum * f;
    for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o, 64);
    const int n = Q.item1 - Q.item0;
    float2 O = make_float2(0.f, 0.f);
    for (int t = 0; t < n; t++) {
        const float ft = __shfl(f, t, 64);
        if (ft == 0.f) continue;  // uniform: an item the row does not reach, or empty
        const int64_t st = (static_cast<int64_t>(Q.item0 + t) * a.n_kv_heads + h) * a.row_slots + row;
        const float2 v = *reinterpret_cast<const float2 *>(a.part_acc + st * kDim + 2 * lane);
        O.x += v.x * ft;
        O.y += v.y * ft;
    }
    float *o = a.out + static_cast<int64_t>(Q.row0 + tok) * a.o_row +
               static_cast<int64_t>(h * a.group + gh) * a.o_head + 2 * lane;
    o[0] = O.x / L;
    o[1] = O.y / L;
}

// ------------------------------------------------------------------ host

struct BndMap {
    std::vector<uint8_t> bytes;
    size_t off_blocks = 0, off_bpos = 0, off_items = 0, off_reqs = 0, off_limit = 0, off_tabs = 0;
    int32_t n_items = 0, n_reqs = 0, n_rows = 0, max_req_rows = 0;
};

// The boundary rows of one request, in the caller's row order: the last
// context position each row sees.
struct ReqRows {
    int32_t request;
    std::vector<int32_t> limit;
};

// Requests with boundary rows, in order; each request's context [0, L),
// L = its last boundary position + 1, is cut into ceil(L / S) items of
// about equal length, S the total over `target` (at least one step, at most
// kMaxItems items per request).  Boundary rows are numbered request by
// request in the order given: the order of the caller's q.
BndMap build_bnd_map(const Problem &p, const std::vector<ReqRows> &groups, int64_t target) {
    std::vector<AttnTile> tiles;
    std::vector<AttnBlock> blocks;
    std::vector<int32_t> bpos;
    std::vector<int32_t> btabs;  // kBlockTabs per block
    std::vector<BndItem> items;
    std::vector<BndReq> reqs;
    std::vector<int32_t> limit;
    auto ctx_of = [&](const ReqRows &gr) {
        int64_t L = 0;
        for (int32_t x : gr.limit) L = std::max<int64_t>(L, int64_t{x} + 1);
        return L;
    };
    int64_t total = 0;
    for (const auto &gr : groups) total += ctx_of(gr);
    const int64_t per = std::max<int64_t>(kStepPos, (total + target - 1) / target);
    int32_t max_rows = 0;
    for (const auto &gr : groups) {
        const int32_t r = gr.request;
        BndReq R{static_cast<int32_t>(limit.size()), 0, static_cast<int32_t>(items.size()), 0};
        limit.insert(limit.end(), gr.limit.begin(), gr.limit.end());
        R.n_tok = static_cast<int32_t>(limit.size()) - R.row0;
        max_rows = std::max(max_rows, R.n_tok);
        const int64_t L = ctx_of(gr);
        const int64_t n = std::min<int64_t>(kMaxItems, (L + per - 1) / per);
        const int64_t S = (L + n - 1) / n;
        int64_t pos = 0, left = L, item_left = 0;
        AttnBlock blk{r, 0, 0, 0};
        int32_t blk_pos = 0;
        std::vector<int32_t> tabs;  // the open block's shift tables
        auto close_block = [&]() {
            if (blk.ntiles > 0) {
                blocks.push_back(blk);
                bpos.push_back(blk_pos);
                for (int j = 0; j < kBlockTabs; j++)
                    btabs.push_back(j < static_cast<int>(tabs.size()) ? tabs[j] : -1);
            }
            blk = AttnBlock{r, static_cast<int32_t>(tiles.size()), 0, 0};
            blk_pos = static_cast<int32_t>(pos);
            tabs.clear();
        };
        for (int32_t t = p.req_tile0[r]; t < p.req_tile0[r + 1] && left > 0; t++) {
            AttnTile T = p.atiles[t];
            while (T.ntok > 0 && left > 0) {
                if (item_left == 0) {
                    close_block();
                    if (!items.empty() && items.back().block1 < 0)
                        items.back().block1 = static_cast<int32_t>(blocks.size());
                    items.push_back(BndItem{static_cast<int32_t>(reqs.size()),
                                            static_cast<int32_t>(blocks.size()), -1,
                                            static_cast<int32_t>(pos)});
                    item_left = std::min(S, left);
                }
                const bool new_tab = T.cs_idx >= 0 &&
                                     std::find(tabs.begin(), tabs.end(), T.cs_idx) == tabs.end();
                if (blk.ntok == kBlockPos || blk.ntiles == kItemTiles ||
                    (new_tab && static_cast<int>(tabs.size()) == kBlockTabs))
                    close_block();
                if (T.cs_idx >= 0 && std::find(tabs.begin(), tabs.end(), T.cs_idx) == tabs.end())
                    tabs.push_back(T.cs_idx);
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
                T = advance_tile(T, take);
                if (item_left == 0) close_block();
            }
        }
        close_block();
        if (!items.empty() && items.back().block1 < 0)
            items.back().block1 = static_cast<int32_t>(blocks.size());
        R.item1 = static_cast<int32_t>(items.size());
        reqs.push_back(R);
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
    m.off_reqs = put(reqs.data(), reqs.size() * sizeof(BndReq));
    m.off_limit = put(limit.data(), limit.size() * sizeof(int32_t));
    m.off_tabs = put(btabs.data(), btabs.size() * sizeof(int32_t));
    m.n_items = static_cast<int32_t>(items.size());
    m.n_reqs = static_cast<int32_t>(reqs.size());
    m.n_rows = static_cast<int32_t>(limit.size());
    m.max_req_rows = max_rows;
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
    {
        const pic_status st0 = ensure_attention(plan);
        if (st0) return st0;
    }
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
    if (args->reserved != 0) return fail(PIC_ERR_INVALID_ARG, "reserved must be 0");
    if (!args->rows && args->boundary_k < 1)
        return fail(PIC_ERR_INVALID_ARG, "boundary_k %d < 1", args->boundary_k);
    if (args->rows && args->n_rows < 0) return fail(PIC_ERR_INVALID_ARG, "n_rows %d < 0", args->n_rows);
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

    // the boundary rows, request by request: the last position each row
    // sees.  Default: tokens j < k of every relocated entry (dst_offset > 0),
    // in each request's entry order; else the caller's (entry, token) rows.
    // The plan's boundaries are [request, begin, end] per entry.
    std::vector<ReqRows> groups;
    try {
        const int64_t n_entries = static_cast<int64_t>(p.bounds.size() / 3);
        auto add = [&](int32_t r, int64_t pos) {
            if (groups.empty() || groups.back().request != r) groups.push_back(ReqRows{r, {}});
            groups.back().limit.push_back(static_cast<int32_t>(pos));
        };
        if (args->rows) {
            for (int32_t b = 0; b < args->n_rows; b++) {
                const int32_t e = args->rows[2 * b], j = args->rows[2 * b + 1];
                if (e < 0 || e >= n_entries)
                    return fail(PIC_ERR_RANGE, "row %d: entry %d outside the plan's %lld entries", b, e,
                                static_cast<long long>(n_entries));
                const int32_t r = static_cast<int32_t>(p.bounds[3 * e]);
                const int64_t dst = p.bounds[3 * e + 1], len = p.bounds[3 * e + 2] - dst;
                if (j < 0 || j >= len)
                    return fail(PIC_ERR_RANGE, "row %d: token %d outside entry %d of length %lld", b, j,
                                e, static_cast<long long>(len));
                if (!groups.empty() && r < groups.back().request)
                    return fail(PIC_ERR_INVALID_ARG, "row %d: request %d after request %d (rows must "
                                "come request by request)", b, r, groups.back().request);
                add(r, dst + j);
            }
        } else {
            for (int64_t e = 0; e < n_entries; e++) {
                const int64_t dst = p.bounds[3 * e + 1], len = p.bounds[3 * e + 2] - dst;
                if (dst <= 0) continue;
                for (int64_t j = 0; j < std::min<int64_t>(args->boundary_k, len); j++)
                    add(static_cast<int32_t>(p.bounds[3 * e]), dst + j);
            }
        }
    } catch (const std::bad_alloc &) {
        return fail(PIC_ERR_NOMEM, "out of host memory");
    }
    for (const ReqRows &gr : groups) {
        const int32_t r = gr.request;
        const int64_t need = int64_t{*std::max_element(gr.limit.begin(), gr.limit.end())} + 1;
        if (need > p.context[r])
            return fail(PIC_ERR_RANGE, "request %d: boundary rows beyond its context", r);
        if (p.context_bad_page[r] >= 0 &&
            p.context_bad_page[r] * static_cast<int64_t>(p.page_size) < need)
            return fail(PIC_ERR_RANGE, "request %d: context page %d maps outside the cache", r,
                        p.context_bad_page[r]);
    }
    if (groups.empty()) return PIC_OK;

    hipStream_t stream = static_cast<hipStream_t>(stream_);
    st = ensure_device_plan(plan, stream_);
    if (st) return st;
    // items: about two rounds of the CU slots (one workgroup of 8 waves per
    // CU and KV head at a time)
    const int64_t target = std::max<int64_t>(1, 2 * static_cast<int64_t>(cu_count()) / H);
    int TT = 1, n_sets = 1, row_slots = 0;
    auto fill_blob = [&](DevBlob &b, BndMap &m) {
        b.off[0] = m.off_blocks;
        b.off[1] = m.off_bpos;
        b.off[2] = m.off_items;
        b.off[3] = m.off_reqs;
        b.off[4] = m.off_limit;
        b.off[5] = m.off_tabs;
        b.n[0] = m.n_items;
        b.n[1] = m.n_reqs;
        b.n[2] = m.max_req_rows;
    };
    const DevBlob *blob = nullptr;
    DevBlob call_blob;       // the caller's rows: metadata of this call only
    void *call_dev = nullptr;
    if (args->rows) {
        BndMap m;
        try {
            m = build_bnd_map(p, groups, target);
        } catch (const std::bad_alloc &) {
            return fail(PIC_ERR_NOMEM, "out of host memory");
        }
        fill_blob(call_blob, m);
        st = stage_per_call(std::max<size_t>(m.bytes.size(), 16),
                            [&](uint8_t *host) { std::memcpy(host, m.bytes.data(), m.bytes.size()); },
                            stream_, &call_dev, "boundary rows");
        if (st) return st;
        call_blob.dev = call_dev;
        blob = &call_blob;
    } else {
        const int64_t key = (target << 32) | static_cast<uint32_t>(args->boundary_k);
        st = plan_blob(plan, blob_key(kBlobBoundary, key), stream_, [&](DevBlob &b) {
            BndMap m = build_bnd_map(p, groups, target);
            b.host = std::move(m.bytes);
            fill_blob(b, m);
        }, &blob);
        if (st) return st;
    }
    auto release_call = [&]() {
        if (call_dev) (void)hipFreeAsync(call_dev, stream);
        call_dev = nullptr;
    };
    const int32_t n_items = blob->n[0], n_reqs = blob->n[1], max_rows = blob->n[2];
    // rows of a request's KV head: tokens x G, in as few sets of 8 waves x TT
    // tiles as the registers allow, TT as small as they then permit
    const int64_t rows = static_cast<int64_t>(max_rows) * G;
    const int64_t max_set = int64_t{kWaves} * kMaxTT * 16;
    n_sets = static_cast<int>((rows + max_set - 1) / max_set);
    TT = static_cast<int>((rows + int64_t{n_sets} * kWaves * 16 - 1) / (int64_t{n_sets} * kWaves * 16));
    row_slots = n_sets * kWaves * TT * 16;
    if ((static_cast<int64_t>(n_items) * H + 7) / 8 * 8 * n_sets >= (int64_t{1} << 31) / (64 * kWaves) ||
        static_cast<int64_t>(n_reqs) * rows * H >= (int64_t{1} << 31) / 64 || n_reqs > 65535) {
        release_call();
        return fail(PIC_ERR_RANGE, "boundary rows x context too large for one launch");
    }
    const size_t need = static_cast<size_t>(n_items) * H * row_slots *
                        (static_cast<size_t>(kDim) + 2) * sizeof(float);
    void *work = nullptr;
    st = call_workspace(plan, need, stream_, &work);
    if (st) {
        release_call();
        return st;
    }
    const uint8_t *dm = static_cast<const uint8_t *>(plan->d_mem);
    const uint8_t *bm = static_cast<const uint8_t *>(blob->dev);
    BndArgs a{};
    a.tiles = reinterpret_cast<const AttnTile *>(bm);
    a.blocks = reinterpret_cast<const AttnBlock *>(bm + blob->off[0]);
    a.block_pos = reinterpret_cast<const int32_t *>(bm + blob->off[1]);
    a.items = reinterpret_cast<const BndItem *>(bm + blob->off[2]);
    a.reqs = reinterpret_cast<const BndReq *>(bm + blob->off[3]);
    a.limit = reinterpret_cast<const int32_t *>(bm + blob->off[4]);
    a.block_tabs = reinterpret_cast<const int32_t *>(bm + blob->off[5]);
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
    const size_t acc_elems = static_cast<size_t>(n_items) * H * row_slots * static_cast<size_t>(kDim);
    a.part_acc = static_cast<float *>(work);
    a.part_ml = static_cast<float *>(work) + acc_elems;
    a.n_items = n_items;
    a.n_kv_heads = H;
    a.group = G;
    a.num_q_heads = args->num_q_heads;
    a.row_slots = row_slots;
    a.n_sets = n_sets;
    a.rope_offset = p.shape.rope_offset;
    a.half_r = p.u.half_r;
    a.scale = args->scale;
    a.sink_tokens = args->sink_tokens;
    a.sink_bias = args->sink_bias;
    const dim3 grid(static_cast<unsigned>((static_cast<int64_t>(a.n_items) * H + 7) / 8 * 8 * n_sets));
    const bool half = p.style == PIC_ROPE_HALF;
    switch (TT) {
#define PIC_BND_LAUNCH(T)                                                                          \
    case T:                                                                                        \
        if (half)                                                                                  \
            hipLaunchKernelGGL((bnd_block_kernel<PIC_ROPE_HALF, T>), grid, dim3(64 * kWaves), 0,  \
                               stream, a, args->layer);                                            \
        else                                                                                       \
            hipLaunchKernelGGL((bnd_block_kernel<PIC_ROPE_INTERLEAVED, T>), grid,                  \
                               dim3(64 * kWaves), 0, stream, a, args->layer);                      \
        break;
        PIC_BND_LAUNCH(1)
        PIC_BND_LAUNCH(2)
#undef PIC_BND_LAUNCH
        default:
            release_call();
            return fail(PIC_ERR_INVALID_ARG, "internal: row tiles per wave %d", TT);
    }
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) {
        hipLaunchKernelGGL(bnd_combine_kernel,
                           dim3(static_cast<unsigned>(max_rows * G), static_cast<unsigned>(n_reqs),
                                static_cast<unsigned>(H)),
                           dim3(64), 0, stream, a);
        e = hipGetLastError();
    }
    release_call();
    if (e != hipSuccess) return hip_fail(e, "boundary attention kernel launch");
    return note_use(plan, stream_);
}
