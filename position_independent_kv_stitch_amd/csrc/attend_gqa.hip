// attend_gqa.hip -- decode attention over stitched GQA requests on the
// matrix cores: the bf16 path of pic_attend for 128-dim head rows.
//
// What is computed is pic_attend's definition (attend.hip): every query head
// of a request attends over the request's context at one layer; positions a
// placed chunk writes read the chunk's pool row with its key turned by the
// chunk's shift (cos/sin the plan's fp64 values rounded to fp32), every other
// position reads the request's own cache; the EPIC Guide's LegoLink damping
// is an optional logit bias on the first tokens of every chunk placed after
// position 0.
//
// The turn is moved to the query.  For a chunk turned by R (plane i:
// x' = x c - y s, y' = x s + y c), q . (R k) = (R^T q) . k, so the keys are
// used exactly as stored and each chunk's query is turned once instead of
// every key (Irminsul: MLA-Native Position-Independent Caching for Agentic
// LLM Serving, Technical Summary section 4, the delta-rotation moved out of
// the stored rows).  The turned query is held as the sum of three bf16 terms
// (the residual of each rounding rounded again), which carries it to about
// 2^-24 of its size, so the products on the matrix cores lose nothing
// against fp32.
//
// Work: one wave per work item (a run of positions of one request, cut on
// the host per launch shape) and KV head; waves do not share data, so there
// is no barrier.  Per step of 32 positions:
//   - the K and V rows of the KV head (16 KB) go from HBM straight into the
//     wave's ring of LDS stages (global_load_lds_dwordx4), in the MFMA
//     A-fragment layout, several steps ahead of their use;
//   - S^T = K Q'^T (v_mfma_f32_16x16x32_bf16) with Q' the query of the
//     positions' chunk: one product per term (for groups of 1, 2 or 4 query
//     heads the terms share one product in the spare rows and DPP row shifts
//     add them up), a position tile that mixes chunks is computed once per
//     chunk and selected per position;
//   - online softmax over the query heads (rows), in log2 units with a lazy
//     running max;
//   - O^T += V^T P^T with the weights straight from the S^T D registers
//     (hi + lo bf16) and V^T by transposing LDS reads.
// A partial (max, sum, accumulator) per (item, query head) is merged by
// gqa_combine_kernel.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <type_traits>

#include "lds_load.hpp"
#include "pic_internal.hpp"

namespace pic {

pic_status hip_fail(hipError_t e, const char *what);  // stitch.hip

namespace {

constexpr int kDim = 128;                  // head row
constexpr int kKSteps = kDim / 32;         // MFMA k-steps
constexpr int kDTiles = kDim / 16;         // output tiles of 16 dims
#ifndef PIC_GQA_PT
#define PIC_GQA_PT 2
#endif
constexpr int kPT = PIC_GQA_PT;            // 16-position tiles per step (1 or 2)
constexpr int kStepPos = 16 * kPT;         // positions per step
constexpr int kSlabs = 2 * kKSteps * kPT;  // 1 KB slabs per step: K (s, tau), then V
#ifndef PIC_GQA_STAGES
#define PIC_GQA_STAGES 3
#endif
constexpr int kStages = PIC_GQA_STAGES;    // LDS stages per wave (steps in flight + 1)
// waves whose rings (and ~3 KB of tables) fit a CU's 160 KB of LDS
constexpr int kWavesPerCu = 160 * 1024 / (kStages * kSlabs * 1024 + 3 * 1024);
constexpr int kMaxHalf = kDim / 2;         // rotary planes at most
constexpr int kMaxItems = 128;             // items per request (the merge keeps 64 per lane round)
constexpr float kLazy = 12.f;              // running-max slack of the online softmax (log2 units)
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

struct CosSin {
    float c, s;
};

struct GqaArgs {
    const AttnTile *tiles;      // blocks' tiles (tok0: position in the block)
    const AttnBlock *blocks;
    const int32_t *item_block0; // first block of every item (+ end)
    const int32_t *req_item0;   // first item of every request (+ end)
    const int32_t *block_tabs;  // [block][kItemBlockTabs] shift tables (-1: none)
    const double *cs;
    const uint16_t *pool_k, *pool_v, *cache_k, *cache_v;
    int64_t s_layer, s_tok, s_head, s_page;
    int64_t c_layer, c_tok, c_head, c_page, c_req;
    const uint16_t *q;
    int64_t q_req, q_head;
    float *out;
    int64_t o_req, o_head;
    float *part_acc;  // [item][q head][kDim]
    float *part_ml;   // [item][q head][2]
    int32_t n_items, n_kv_heads, group, num_q_heads;
    int32_t rope_offset, half_r;
    float scale;
    int32_t sink_tokens;
    float sink_bias;
};

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &v) {
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float bf16_to_f32(__bf16 v) {
    return __uint_as_float(static_cast<uint32_t>(__builtin_bit_cast(uint16_t, v)) << 16);
}

// max over the four lanes of a row (lanes r, r + 16, r + 32, r + 48): the
// 32-lane swap pairs lane i with i ^ 32, the 16-lane swap i with i ^ 16
__device__ __forceinline__ float row_max(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// lane i of every 16-lane row takes lane i + K's value (DPP row_shl; lanes
// whose source lies past the row take 0)
template <int K>
__device__ __forceinline__ float row_shl(float v) {
    static_assert(K >= 1 && K < 16, "DPP row shift");
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x100 + K, 0xF, 0xF, true));
}

// the same with bitwise or
__device__ __forceinline__ uint32_t row_or(uint32_t v) {
    const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    v = a[0] | a[1];
    const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return b[0] | b[1];
}

// A map tile as the staging reads it: the row of block position pi starts at
// element off0 + pi * token stride (layer and head included) of the pool
// (info bit kInfoPool) or the cache; info also holds the tile's shift-table
// slot + 1 (bits 0-2, 0: rows not turned) and how many of its first
// positions take the damping bias (bits 8-31).
struct StageTile {
    int64_t off0;
    int32_t tok0;
    uint32_t info;
};
constexpr uint32_t kInfoPool = 1u << 3;

__device__ __forceinline__ StageTile stage_tile(const GqaArgs &a, const AttnTile &T, int slot,
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
    const int64_t damp = std::min<int64_t>(std::max<int64_t>(int64_t{a.sink_tokens} - T.sink_dist, 0),
                                           (1 << 24) - 1);
    const uint32_t info = static_cast<uint32_t>(slot + 1) | (pool ? kInfoPool : 0u) |
                          (static_cast<uint32_t>(damp) << 8);
    return StageTile{off0, T.tok0, info};
}

// The query fragment of this lane (row r16, dims 32 s + 8 g + e) turned by
// the inverse of a chunk's rotation, as three bf16 terms.  Half pairing: the
// pieces of a lane are wholly x (plane d - ro), wholly y (its partner half_r
// dims on, the same lane since half_r is a multiple of 32) or outside the
// rotary slice; interleaved pairing: a piece inside the slice holds 4 pairs.
template <int STYLE>
__device__ __forceinline__ void turn_query(const bf16x8 (&qf)[kKSteps], bf16x8 (&qt)[3][kKSteps],
                                           const CosSin *cs, int ro, int hr, int g) {
    float v[kKSteps][8], o[kKSteps][8];
#pragma unroll
    for (int s = 0; s < kKSteps; s++)
#pragma unroll
        for (int e = 0; e < 8; e++) o[s][e] = v[s][e] = bf16_to_f32(qf[s][e]);
#pragma unroll
    for (int s = 0; s < kKSteps; s++) {
        const int d0 = 32 * s + 8 * g;
        if constexpr (STYLE == PIC_ROPE_HALF) {
#pragma unroll
            for (int sy = s + 1; sy < kKSteps; sy++) {
                if (d0 >= ro && d0 < ro + hr && 32 * (sy - s) == hr) {
#pragma unroll
                    for (int e = 0; e < 8; e++) {
                        const CosSin t = cs[d0 - ro + e];
                        const float x = v[s][e], y = v[sy][e];
                        o[s][e] = fmaf(x, t.c, y * t.s);
                        o[sy][e] = fmaf(y, t.c, -(x * t.s));
                    }
                }
            }
        } else {
            if (d0 >= ro && d0 < ro + 2 * hr) {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const CosSin t = cs[(d0 - ro) / 2 + e];
                    const float x = v[s][2 * e], y = v[s][2 * e + 1];
                    o[s][2 * e] = fmaf(x, t.c, y * t.s);
                    o[s][2 * e + 1] = fmaf(y, t.c, -(x * t.s));
                }
            }
        }
    }
#pragma unroll
    for (int s = 0; s < kKSteps; s++) {
        uint32_t w[3][4];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            f32x2 r = {o[s][2 * k], o[s][2 * k + 1]};
#pragma unroll
            for (int term = 0; term < 3; term++) {
                const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
                w[term][k] = b;
                r = f32x2{r[0] - __uint_as_float(b << 16), r[1] - __uint_as_float(b & 0xFFFF0000u)};
            }
        }
#pragma unroll
        for (int term = 0; term < 3; term++)
            qt[term][s] = as_bf16x8(make_uint4(w[term][0], w[term][1], w[term][2], w[term][3]));
    }
}

// The packed form for groups of PG <= 5 query heads: row n of the products
// holds term n / PG of head n % PG (rows from 3 PG on: zero), so one product
// per k-step computes all three terms and row_shl folds them into rows
// 0 .. PG - 1.  qr holds the lane's raw query (head n % PG).
template <int STYLE>
__device__ __forceinline__ void turn_query_packed(const bf16x8 (&qr)[kKSteps], bf16x8 (&qp)[kKSteps],
                                                  const CosSin *cs, int ro, int hr, int g, int term) {
    bf16x8 qt[3][kKSteps];
    turn_query<STYLE>(qr, qt, cs, ro, hr, g);
#pragma unroll
    for (int s = 0; s < kKSteps; s++) {
        const uint4 t0 = __builtin_bit_cast(uint4, qt[0][s]), t1 = __builtin_bit_cast(uint4, qt[1][s]),
                    t2 = __builtin_bit_cast(uint4, qt[2][s]);
        const uint4 z = make_uint4(0u, 0u, 0u, 0u);
        qp[s] = as_bf16x8(term == 0 ? t0 : term == 1 ? t1 : term == 2 ? t2 : z);
    }
}

// Wait until the stage calls issued after the oldest one (`newer` of them,
// kSlabs loads each) are the only ones outstanding.
template <int N>
__device__ __forceinline__ void wait_newer(int newer) {
    if constexpr (N > 0) {
        if (newer >= N) {
            wait_vm<N * kSlabs>();
            return;
        }
        wait_newer<N - 1>(newer);
    } else {
        wait_vm<0>();
    }
}

// PG: the group size when it is packed (1, 2 or 4 query heads), else 0.
template <int STYLE, int PG>
__global__ void __launch_bounds__(64) gqa_tile_kernel(const GqaArgs a, int32_t layer) {
    static_assert(PG >= 0 && 3 * PG <= 16, "packed terms fit the 16 rows");
    // stage slab (kind, s, tau) = kind * 2 kKSteps + 2 s + tau (kind 0: K,
    // 1: V) holds dims 32 s .. + 31 of positions 16 tau .. + 15; its slot
    // 16 g + p holds dims 32 s + 8 g .. + 8 of position 16 tau + p
    __shared__ __attribute__((aligned(16))) uint4 s_stage[kStages][kSlabs * 64];
    __shared__ CosSin s_cs[kItemBlockTabs][kMaxHalf];  // the block's tables, fp32
    __shared__ StageTile s_tiles[kItemBlockTiles];
    __shared__ __attribute__((aligned(16))) uint32_t s_pslot[kStages][kStepPos];
    __shared__ __attribute__((aligned(16))) float s_pbias[kStages][kStepPos];

    const int item = blockIdx.x / a.n_kv_heads;
    const int h = blockIdx.x - item * a.n_kv_heads;
    const int lane = threadIdx.x, r16 = lane & 15, g = lane >> 4;
    const int G = a.group;
    const int b_lo = a.item_block0[item], b_hi = a.item_block0[item + 1];
    const int request = a.blocks[b_lo].request;
    const float scale2 = a.scale * kLog2e;  // logits in log2 units (exp2 weights)
    const float bias2 = a.sink_bias * kLog2e;
    const int ro = a.rope_offset, hr = a.half_r;

    // query fragments (B of S^T = K Q^T): row r16 = query head h G + r16
    // (rows past the group are zero), dims 32 s + 8 g .. + 8.  Packed, the
    // lane also keeps the raw query of its term row's head r16 % PG.
    bf16x8 qf[kKSteps];
    bf16x8 qr[PG ? kKSteps : 1];
    {
        const int qh = PG ? r16 % PG : r16;
        const bool live = PG ? r16 < 3 * PG : r16 < G;
        const uint16_t *qrow = a.q + request * a.q_req + (h * G + (live ? qh : 0)) * a.q_head;
#pragma unroll
        for (int s = 0; s < kKSteps; s++) {
            const uint4 v = live ? *reinterpret_cast<const uint4 *>(qrow + 32 * s + 8 * g)
                                 : make_uint4(0u, 0u, 0u, 0u);
            if constexpr (PG) {
                qr[s] = as_bf16x8(v);
                qf[s] = as_bf16x8(r16 < PG ? v : make_uint4(0u, 0u, 0u, 0u));
            } else {
                qf[s] = as_bf16x8(v);
            }
        }
    }
    // the query turned for table cur_tab: three terms, or packed
    bf16x8 qt[PG ? 1 : 3][kKSteps];
    int cur_tab = -1;

    f32x4 acc[kDTiles];
#pragma unroll
    for (int t = 0; t < kDTiles; t++) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    for (int b = b_lo; b < b_hi; b++) {
        const AttnBlock B = a.blocks[b];
        int btab[kItemBlockTabs];  // the block's tables (read here: no memory load in the steps)
#pragma unroll
        for (int j = 0; j < kItemBlockTabs; j++)
            btab[j] = __builtin_amdgcn_readfirstlane(a.block_tabs[kItemBlockTabs * b + j]);
        // the previous block's loads are all consumed; its tables and tiles
        // may be replaced (one wave: program order)
        if (lane < B.ntiles) {
            const AttnTile T = a.tiles[B.tile0 + lane];
            int sl = -1;
#pragma unroll
            for (int j = 0; j < kItemBlockTabs; j++)
                if (T.cs_idx >= 0 && btab[j] == T.cs_idx) sl = j;
            s_tiles[lane] = stage_tile(a, T, sl, layer, h);
        }
        for (int i = lane; i < kItemBlockTabs * hr; i += 64) {
            const int j = i / hr, pl = i - j * hr;
            int tab = btab[0];
#pragma unroll
            for (int jj = 1; jj < kItemBlockTabs; jj++)
                if (j == jj) tab = btab[jj];
            if (tab >= 0) {
                const double *src = a.cs + (static_cast<int64_t>(tab) * hr + pl) * 2;
                s_cs[j][pl] = CosSin{static_cast<float>(src[0]), static_cast<float>(src[1])};
            }
        }
        __syncthreads();  // one wave: orders the LDS writes above before their reads

        // stage step p0 into ring slot st: lane (g, r16) loads piece g of
        // position 16 tau + r16 for every k-step, K and V; lanes past the
        // block's end repeat position p0 (their weights are 0)
        int cur[2] = {0, 0};
        auto stage = [&](int p0, int st) {
#pragma unroll
            for (int tau = 0; tau < kPT; tau++) {
                int pi = p0 + 16 * tau + r16;
                const bool valid = pi < B.ntok;
                if (!valid) pi = p0;
                while (cur[tau] + 1 < B.ntiles && s_tiles[cur[tau] + 1].tok0 <= pi) cur[tau]++;
                const StageTile T = s_tiles[cur[tau]];
                const bool pool = T.info & kInfoPool;
                const int64_t off = T.off0 + static_cast<int64_t>(pi) * (pool ? a.s_tok : a.c_tok);
                if (g == 0) {
                    const bool damp = static_cast<uint32_t>(pi - T.tok0) < (T.info >> 8);
                    s_pslot[st][16 * tau + r16] = valid ? (T.info & 7u) : 0u;
                    s_pbias[st][16 * tau + r16] = valid ? (damp ? bias2 : 0.f) : -INFINITY;
                }
                const uint16_t *kr = (pool ? a.pool_k : a.cache_k) + off + 8 * g;
                const uint16_t *vr = (pool ? a.pool_v : a.cache_v) + off + 8 * g;
                // k-step s of the row is 64 s bytes on (the load's offset field)
                load_lds16<0>(kr, &s_stage[st][(0 * kPT + tau) * 64]);
                load_lds16<64>(kr, &s_stage[st][(1 * kPT + tau) * 64]);
                load_lds16<128>(kr, &s_stage[st][(2 * kPT + tau) * 64]);
                load_lds16<192>(kr, &s_stage[st][(3 * kPT + tau) * 64]);
                load_lds16<0>(vr, &s_stage[st][(kKSteps * kPT + 0 * kPT + tau) * 64]);
                load_lds16<64>(vr, &s_stage[st][(kKSteps * kPT + 1 * kPT + tau) * 64]);
                load_lds16<128>(vr, &s_stage[st][(kKSteps * kPT + 2 * kPT + tau) * 64]);
                load_lds16<192>(vr, &s_stage[st][(kKSteps * kPT + 3 * kPT + tau) * 64]);
            }
        };

        const int nsteps = (B.ntok + kStepPos - 1) / kStepPos;
        for (int i = 0; i < kStages - 1 && i < nsteps; i++) stage(i * kStepPos, i);
        for (int i = 0; i < nsteps; i++) {
            const int p0 = i * kStepPos;
            const int slot = i % kStages;
            // step i's loads are in; the ones of the steps after it may not be
            wait_newer<kStages - 2>(min(kStages - 2, nsteps - 1 - i));
            // the slot freed by step i - 1 takes step i + kStages - 1
            if (i + kStages - 1 < nsteps) stage(p0 + (kStages - 1) * kStepPos, (i + kStages - 1) % kStages);

            // ---- logits S^T, position tile by tile; the positions' chunk
            // classes (0: not turned, j + 1: block table j) pick the query
            const uint4 *stg = s_stage[slot];
            f32x4 st[kPT];
#pragma unroll
            for (int tau = 0; tau < kPT; tau++) {
                const uint4 cl4 = *reinterpret_cast<const uint4 *>(&s_pslot[slot][16 * tau + 4 * g]);
                const uint32_t cls[4] = {cl4.x, cl4.y, cl4.z, cl4.w};
                uint32_t present = (1u << cls[0]) | (1u << cls[1]) | (1u << cls[2]) | (1u << cls[3]);
                present = __builtin_amdgcn_readfirstlane(row_or(present));
                st[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
                const bool single = (present & (present - 1)) == 0;
                while (present) {
                    const int c = __builtin_ctz(present);
                    present &= present - 1;
                    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
                    if (c == 0) {
#pragma unroll
                        for (int s = 0; s < kKSteps; s++)
                            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                as_bf16x8(stg[(s * kPT + tau) * 64 + lane]), qf[s], sc, 0, 0, 0);
                    } else {
                        int tab = btab[0];
#pragma unroll
                        for (int jj = 1; jj < kItemBlockTabs; jj++)
                            if (c - 1 == jj) tab = btab[jj];
                        if (tab != cur_tab) {
                            if constexpr (PG)
                                turn_query_packed<STYLE>(qr, qt[0], s_cs[c - 1], ro, hr, g, r16 / PG);
                            else
                                turn_query<STYLE>(qf, qt, s_cs[c - 1], ro, hr, g);
                            cur_tab = tab;
                        }
                        if constexpr (PG) {
#pragma unroll
                            for (int s = 0; s < kKSteps; s++)
                                sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    as_bf16x8(stg[(s * kPT + tau) * 64 + lane]), qt[0][s], sc, 0, 0, 0);
                            // rows 0 .. PG - 1 gather their terms from rows + PG, + 2 PG
#pragma unroll
                            for (int e = 0; e < 4; e++)
                                sc[e] = (sc[e] + row_shl<PG>(sc[e])) + row_shl<2 * PG>(sc[e]);
                        } else {
#pragma unroll
                            for (int s = 0; s < kKSteps; s++) {
                                const bf16x8 kf = as_bf16x8(stg[(s * kPT + tau) * 64 + lane]);
#pragma unroll
                                for (int term = 0; term < 3; term++)
                                    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qt[term][s], sc, 0, 0, 0);
                            }
                        }
                    }
                    if (single) {
                        st[tau] = sc;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            if (cls[e] == static_cast<uint32_t>(c)) st[tau][e] = sc[e];
                    }
                }
            }

            // ---- online softmax per row (log2 units); lane holds positions
            // 16 tau + 4 g + e.  The running max is kept until a logit passes
            // it by kLazy (weights stay below 2^kLazy; the merge uses the same
            // reference), so the accumulator is seldom rescaled
            constexpr int NV = 4 * kPT;  // positions of this lane: 16 tau + 4 g + e
            float x[NV];
#pragma unroll
            for (int tau = 0; tau < kPT; tau++) {
                const f32x4 pb = *reinterpret_cast<const f32x4 *>(&s_pbias[slot][16 * tau + 4 * g]);
#pragma unroll
                for (int e = 0; e < 4; e++) x[4 * tau + e] = fmaf(st[tau][e], scale2, pb[e]);
            }
            float mx = x[0];
#pragma unroll
            for (int k = 1; k < NV; k++) mx = fmaxf(mx, x[k]);
            mx = row_max(mx);  // finite: position p0 is in the block
            const bool bump = mx > m_run + kLazy;  // (-inf + kLazy stays -inf)
            const float m_new = bump ? mx : m_run;
            const float alpha = bump ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
            float pw[NV], psum = 0.f;
#pragma unroll
            for (int k = 0; k < NV; k++) {
                pw[k] = __builtin_amdgcn_exp2f(x[k] - m_new);
                psum += pw[k];
            }
            l_run = l_run * alpha + psum;
            m_run = m_new;
            if (__any(bump)) {
#pragma unroll
                for (int t = 0; t < kDTiles; t++) acc[t] *= alpha;
            }
            // weights as B of O^T += V^T P^T (hi + lo bf16): k index 8 g + j is
            // position 4 g + j (j < 4) or 16 + 4 g + j - 4 with two position
            // tiles, 4 g + j with one -- the order of pw
            uint32_t hi[NV / 2], lo[NV / 2];
#pragma unroll
            for (int k = 0; k < NV / 2; k++) {
                const f32x2 pr = {pw[2 * k], pw[2 * k + 1]};
                hi[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
                const f32x2 rr = {pw[2 * k] - __uint_as_float(hi[k] << 16),
                                  pw[2 * k + 1] - __uint_as_float(hi[k] & 0xFFFF0000u)};
                lo[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(rr, bf16x2));
            }

            // ---- A = V^T by transposing LDS reads: within each 16-lane
            // group, lane i receives element i % 4 of the 8-byte rows that
            // lanes 4 j + i / 4 address (j = 0..3), so lane i of group g
            // addresses position 4 g + i / 4 of a position tile, dims
            // 16 t + 4 (i % 4) .. + 4, and receives dim 16 t + i of positions
            // 4 g .. 4 g + 3
            const char *stg8 = reinterpret_cast<const char *>(stg + kKSteps * kPT * 64);
            const int pq = r16 >> 2, dq = r16 & 3;
#pragma unroll
            for (int t = 0; t < kDTiles; t++) {
                const int gq = 2 * (t & 1) + (dq >> 1);
                const int base = (((t >> 1) * kPT) * 64 + 16 * gq + 4 * g + pq) * 16 + 8 * (dq & 1);
                const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(stg8 + base));
                if constexpr (kPT == 2) {
                    const s16x4 v1 =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(stg8 + base + 64 * 16));
                    const uint2 w0 = __builtin_bit_cast(uint2, v0), w1 = __builtin_bit_cast(uint2, v1);
                    const bf16x8 va = as_bf16x8(make_uint4(w0.x, w0.y, w1.x, w1.y));
                    const bf16x8 phi = as_bf16x8(make_uint4(hi[0], hi[1], hi[2], hi[3]));
                    const bf16x8 plo = as_bf16x8(make_uint4(lo[0], lo[1], lo[2], lo[3]));
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi, acc[t], 0, 0, 0);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, plo, acc[t], 0, 0, 0);
                } else {
                    const s16x4 phi = __builtin_bit_cast(s16x4, make_uint2(hi[0], hi[1]));
                    const s16x4 plo = __builtin_bit_cast(s16x4, make_uint2(lo[0], lo[1]));
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v0, phi, acc[t], 0, 0, 0);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v0, plo, acc[t], 0, 0, 0);
                }
            }
        }
        __syncthreads();  // (one wave) the block's LDS reads are done before the next block's writes
    }

    // ---- partial results of the group's heads: O^T D registers hold dims
    // 16 t + 4 g + e of row r16
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
    if (r16 < G) {
        const int64_t slot_id = static_cast<int64_t>(item) * a.num_q_heads + h * G + r16;
        float *pa = a.part_acc + slot_id * kDim;
#pragma unroll
        for (int t = 0; t < kDTiles; t++)
            *reinterpret_cast<float4 *>(pa + 16 * t + 4 * g) =
                make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
        if (g == 0) {
            a.part_ml[2 * slot_id] = m_run;
            a.part_ml[2 * slot_id + 1] = l_run;
        }
    }
}

// out[request][q head] = merge of the request's items (flash-decoding
// rescaling, log2 units): one wave per (request, query head).  Lane l holds
// the max and sum of items l, l + 64, ... (kMaxItems / 64 rounds); then
// every lane merges two dims of the items' rows, reading them eight at a
// time with all eight loads in flight before the first is used (the wave
// alone sums its request, so the loop is latency-bound otherwise).  A slot
// past the last item repeats it with weight 0, which adds exactly zero.
__global__ void __launch_bounds__(64) gqa_combine_kernel(const GqaArgs a) {
    constexpr int kRounds = kMaxItems / 64;
    constexpr int kInFlight = 8;
    static_assert(kMaxItems % 64 == 0 && 64 % kInFlight == 0, "item rounds of a wave");
    const int r = blockIdx.x, j = blockIdx.y, lane = threadIdx.x;
    const int i0 = a.req_item0[r], n = a.req_item0[r + 1] - i0;
    const int64_t hq = a.num_q_heads;
    float m[kRounds], lsum[kRounds], f[kRounds];
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < kRounds; q++) {
        const int t = 64 * q + lane;
        const bool mine = t < n;
        const int64_t slot = (static_cast<int64_t>(i0) + (mine ? t : 0)) * hq + j;
        m[q] = mine ? a.part_ml[2 * slot] : -INFINITY;
        lsum[q] = mine ? a.part_ml[2 * slot + 1] : 0.f;
        M = fmaxf(M, m[q]);
    }
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    float L = 0.f;
#pragma unroll
    for (int q = 0; q < kRounds; q++) {
        f[q] = 64 * q + lane < n ? __builtin_amdgcn_exp2f(m[q] - M) : 0.f;
        L += lsum[q] * f[q];
    }
    for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o, 64);
    const float *acc = a.part_acc + (static_cast<int64_t>(i0) * hq + j) * kDim + 2 * lane;
    const int64_t item_stride = hq * kDim;
    float2 O = make_float2(0.f, 0.f);
#pragma unroll
    for (int q = 0; q < kRounds; q++) {
        for (int t0 = 64 * q; t0 < min(n, 64 * q + 64); t0 += kInFlight) {
            float2 v[kInFlight];
            float ft[kInFlight];
#pragma unroll
            for (int k = 0; k < kInFlight; k++) {
                const int t = min(t0 + k, n - 1);
                ft[k] = __shfl(f[q], (t0 + k) & 63, 64);
                if (t0 + k >= n) ft[k] = 0.f;
                v[k] = *reinterpret_cast<const float2 *>(acc + t * item_stride);
            }
#pragma unroll
            for (int k = 0; k < kInFlight; k++) {
                O.x += v[k].x * ft[k];
                O.y += v[k].y * ft[k];
            }
        }
    }
    float *o = a.out + r * a.o_req + j * a.o_head + 2 * lane;
    o[0] = O.x / L;
    o[1] = O.y / L;
}

int cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    return n;
}

}  // namespace

// Whether pic_attend takes the matrix-core path for this plan and group.
bool gqa_tile_path(const Problem &p, int group) {
    if (p.shape.dtype != PIC_DTYPE_BF16 || p.shape.row_dim != kDim || !p.shape.has_v) return false;
    if (group < 1 || group > 16) return false;
    const int ro = p.shape.rope_offset, hr = p.u.half_r;
    if (ro % 8) return false;
    if (hr == 0) return true;
    if (p.style == PIC_ROPE_HALF) return hr % 32 == 0 && ro + 2 * hr <= kDim;
    return hr % 4 == 0 && ro + 2 * hr <= kDim;
}

// The matrix-core path of pic_attend (arguments checked by the caller).
pic_status attend_gqa(struct ::pic_plan *plan, const pic_kv_view *pool, const pic_kv_view *cache,
                      const pic_attend_args *args, hipStream_t stream) {
    const Problem &p = plan->prob;
    const int H = p.shape.num_heads;
    const int64_t slots = static_cast<int64_t>(cu_count()) * kWavesPerCu;
    const int64_t target = std::max<int64_t>(1, 2 * slots / H);  // about two rounds
    // a request alone in the batch gets at most one round of items: two
    // rounds of short items cost more in set-up than they gain
    const int64_t per_request = std::min<int64_t>(kMaxItems, std::max<int64_t>(1, slots / H));
    const DevBlob *blob = nullptr;
    pic_status st = plan_blob(plan, blob_key(kBlobGqa, target), stream, [&](DevBlob &b) {
        ItemMap m = build_item_map(p, target, per_request);
        b.host = std::move(m.bytes);
        b.off[0] = m.off_blocks;
        b.off[1] = m.off_items;
        b.off[2] = m.off_reqs;
        b.off[3] = m.off_tabs;
        b.n[0] = m.n_items;
    }, &blob);
    if (st) return st;
    const int32_t n_items = blob->n[0];
    const size_t need = static_cast<size_t>(n_items) * static_cast<size_t>(args->num_q_heads) *
                        (static_cast<size_t>(kDim) + 2) * sizeof(float);
    void *work = nullptr;
    st = call_workspace(plan, need, stream, &work);
    if (st) return st;
    const uint8_t *dm = static_cast<const uint8_t *>(plan->d_mem);
    const uint8_t *gm = static_cast<const uint8_t *>(blob->dev);
    GqaArgs a{};
    a.tiles = reinterpret_cast<const AttnTile *>(gm);
    a.blocks = reinterpret_cast<const AttnBlock *>(gm + blob->off[0]);
    a.item_block0 = reinterpret_cast<const int32_t *>(gm + blob->off[1]);
    a.req_item0 = reinterpret_cast<const int32_t *>(gm + blob->off[2]);
    a.block_tabs = reinterpret_cast<const int32_t *>(gm + blob->off[3]);
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
    a.q_req = args->q_request_stride;
    a.q_head = args->q_head_stride;
    a.out = args->out;
    a.o_req = args->out_request_stride;
    a.o_head = args->out_head_stride;
    const size_t acc_elems =
        static_cast<size_t>(n_items) * static_cast<size_t>(args->num_q_heads) * kDim;
    a.part_acc = static_cast<float *>(work);
    a.part_ml = static_cast<float *>(work) + acc_elems;
    a.n_items = n_items;
    a.n_kv_heads = H;
    a.group = args->num_q_heads / H;
    a.num_q_heads = args->num_q_heads;
    a.rope_offset = p.shape.rope_offset;
    a.half_r = p.u.half_r;
    a.scale = args->scale;
    a.sink_tokens = args->sink_tokens;
    a.sink_bias = args->sink_bias;
    const dim3 grid(static_cast<unsigned>(a.n_items) * static_cast<unsigned>(H));
    auto launch = [&](auto style_tag, auto pg_tag) {
        constexpr int S = decltype(style_tag)::value, PG = decltype(pg_tag)::value;
        hipLaunchKernelGGL((gqa_tile_kernel<S, PG>), grid, dim3(64), 0, stream, a, args->layer);
    };
    auto with_style = [&](auto pg_tag) {
        if (p.style == PIC_ROPE_HALF) launch(std::integral_constant<int, PIC_ROPE_HALF>{}, pg_tag);
        else launch(std::integral_constant<int, PIC_ROPE_INTERLEAVED>{}, pg_tag);
    };
    switch (a.group) {  // packed terms for groups of 1, 2 or 4 query heads
        case 1: with_style(std::integral_constant<int, 1>{}); break;
        case 2: with_style(std::integral_constant<int, 2>{}); break;
        case 4: with_style(std::integral_constant<int, 4>{}); break;
        default: with_style(std::integral_constant<int, 0>{}); break;
    }
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) {
        hipLaunchKernelGGL(gqa_combine_kernel,
                           dim3(static_cast<unsigned>(p.context.size()),
                                static_cast<unsigned>(args->num_q_heads)),
                           dim3(64), 0, stream, a);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
    return note_use(plan, stream);
}

}  // namespace pic
