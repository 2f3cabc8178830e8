// attend_mla.hip -- decode attention over MLA latent rows with the chunks'
// delta-rotation done on load (pic_attend_latent).
//
// An MLA cache row is a 512-dim content latent followed by a 64-dim rotary
// key (Irminsul: MLA-Native Position-Independent Caching for Agentic LLM
// Serving, Technical Summary section 2.1).  In the absorbed form of MLA
// decode the query of head h is a 576-dim row as well (its content part
// already multiplied into the latent space, its rotary part post-RoPE), the
// logit is scale * q_h . row_p, and the value of position p is the content
// latent row_p[0, 512): every query head attends over the same rows.
// Positions a placed chunk writes read the chunk's pool row, whose rotary
// key is turned by the chunk's shift once it is on chip (Irminsul sections
// 2.2 and 4: the delta-rotation fused into the attention kernel's load
// path); the turned key is rounded to bf16 exactly as the stitch would store
// it, so the result is attention over the stitched cache.  Every other
// position reads the request's own cache.  The EPIC Guide's LegoLink damping
// is the same optional logit bias as in pic_attend.
//
// Work: a workgroup takes one work item (a run of positions of one request)
// for a set of query-head groups of 16: W waves of one group each, or, for
// 128 heads, four waves of two groups each (one wave per SIMD, so that a
// wave holds 512 registers and each fragment it reads from LDS feeds two
// heads' groups of products).  The
// items are cut for the launch: each request gets a share of the CU slots in
// proportion to its context, so every workgroup has about the same number
// of positions and the launch is one round.  An item's positions come in
// steps of 32 (16 for a one-wave workgroup, which then double-buffers in
// the LDS that one 32-position step took and still shares a CU with three
// others):
//   - staging: the step's rows (36 KB for 32) go from HBM straight into LDS
//     (global_load_lds_dwordx4, no registers), spread over the W waves, into
//     a later buffer while an earlier one is computed on;
//   - the rotary slots of moved chunk rows are turned in LDS (fp64, rounded
//     to bf16 by the stitch's own code, rotate.hpp);
//   - S^T = K Q^T on the matrix cores (v_mfma_f32_16x16x32_bf16): A = 16
//     positions x 32 dims of K, one contiguous 1 KB LDS read per wave (the
//     staging layout is the A-fragment layout); B = the wave's head groups'
//     queries, in registers for the whole item;
//   - online softmax over each of the wave's groups of 16 heads;
//   - O^T += V^T P^T: B = the weights straight from the D registers of the
//     two S^T tiles (the product's k order is permuted to match), split into
//     bf16 hi + lo so the weights lose nothing; A = V^T, eight 2-byte LDS
//     reads per fragment from the same staged rows.
// All W waves read the one staged copy of the rows, so with 128 heads the
// rows leave HBM once.  A partial (max, sum, accumulator) per (item, head)
// is merged by mla_combine_kernel.  Lane layouts of the MFMA and of the
// direct-to-LDS load were checked on the GPU.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "acc_scale.hpp"
#include "lds_load.hpp"
#include "pic_internal.hpp"
#include "rotate.hpp"

namespace pic {

pic_status hip_fail(hipError_t e, const char *what);  // stitch.hip

namespace {

constexpr int kRow = 576;                 // latent row: content 512 + rotary 64
constexpr int kRopeOff = 512;
constexpr int kRopeDim = 64;
constexpr int kVDim = 512;                // value = the content latent
constexpr int kKSteps = kRow / 32;        // MFMA k-steps of 32 dims
constexpr int kRopeStep = kRopeOff / 32;  // first rotary k-step (x half; y in the next)
constexpr int kDTiles = kVDim / 16;       // output tiles of 16 dims
constexpr int kGroupHeads = 16;           // query heads per wave
constexpr int kItemTiles = kItemBlockTiles;  // map tiles per block at most
constexpr int kCombineThreads = 256;
constexpr int kSDepth = 4;  // logit fragments read ahead (two-group waves)
constexpr int kVDepth = 3;  // V^T fragments read ahead (two-group waves)
constexpr int kTurnAt0 = 8, kTurnAt1 = 20;  // value tiles that carry the next step's turn

constexpr int kBlockTabs = kItemBlockTabs;  // shift tables per block at most (kept in LDS)
constexpr int kHalfR = kRopeDim / 2;      // rotary planes
constexpr float kLazy = 12.f;             // running-max slack of the online softmax (log2 units)
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct MlaArgs {
    const AttnTile *tiles;     // latent blocks' tiles (tok0: position in the block)
    const AttnBlock *blocks;   // latent blocks (<= kBlockPos positions, <= kItemTiles tiles)
    const int32_t *block_tabs; // [block][kBlockTabs] shift tables its tiles use (-1: none)
    const int32_t *item_block0;  // first block of every item (+ end)
    const int32_t *req_item0;    // first item of every request (+ end)
    const double *cs;
    const uint16_t *pool_k, *cache_k;
    int64_t s_layer, s_tok, s_page;
    int64_t c_layer, c_tok, c_page, c_req;
    const uint16_t *q;
    int64_t q_req, q_head;
    float *out;
    int64_t o_req, o_head;
    float *part_acc;  // [item][q head][kVDim]
    float *part_ml;   // [item][q head][2]
    int32_t n_items, n_sets, num_q_heads;
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

// A map tile as the staging reads it: the row of block position pi starts at
// element off0 + pi * token stride (layer included) of the pool (info bit
// kInfoPool) or the cache; info also holds the tile's shift-table slot + 1
// (bits 0-2, 0: rows not turned) and how many of its first positions take
// the damping bias (bits 8-31).
struct StageTile {
    int64_t off0;
    int32_t tok0;
    uint32_t info;
};
constexpr uint32_t kInfoPool = 1u << 3;

__device__ __forceinline__ StageTile stage_tile(const MlaArgs &a, const AttnTile &T, int slot,
                                                int32_t layer) {
    const int64_t L = layer;
    int64_t off0;
    bool pool = true;
    switch (T.kind) {
        case kPoolRows:
            off0 = L * a.s_layer + (T.a - T.tok0) * a.s_tok;
            break;
        case kPoolPages:
            off0 = L * a.s_layer + T.a * a.s_page + static_cast<int64_t>(T.b - T.tok0) * a.s_tok;
            break;
        case kCacheRows:
            pool = false;
            off0 = L * a.c_layer + T.a * a.c_req + static_cast<int64_t>(T.b - T.tok0) * a.c_tok;
            break;
        default:
            pool = false;
            off0 = L * a.c_layer + T.a * a.c_page + static_cast<int64_t>(T.b - T.tok0) * a.c_tok;
            break;
    }
    const int64_t damp = std::min<int64_t>(std::max<int64_t>(int64_t{a.sink_tokens} - T.sink_dist, 0),
                                           (1 << 24) - 1);
    const uint32_t info = static_cast<uint32_t>(slot + 1) | (pool ? kInfoPool : 0u) |
                          (static_cast<uint32_t>(damp) << 8);
    return StageTile{off0, T.tok0, info};
}

// S^T = K Q^T of two-group waves on the matrix cores with VGPR results:
// their 256 output accumulators fill the AGPRs, where the compiler would
// otherwise also place these logits (it picks one register kind for every
// product of a kernel) and then copy accumulators back and forth at every
// step.  An accumulation into the same registers as the previous product's
// result needs no wait states; a vector ALU read of the result does, which
// vgpr_mfma_guard provides (its operands tie the logits, so no read of them
// is scheduled before it).  The first k-step starts from zero.
template <bool FIRST>
__device__ __forceinline__ void mfma_v(f32x4 &c, const bf16x8 &a, const bf16x8 &b) {
    if constexpr (FIRST)
        asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
    else
        asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void vgpr_mfma_guard(f32x4 &a, f32x4 &b, f32x4 &c, f32x4 &d) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}

// A map tile as the two-group staging reads it: the byte address of the row
// of block position 0 (pool or cache, layer included) and the token stride in
// bytes, so that position pi's row starts at addr0 + pi * stride.
struct StageRow {
    uint64_t addr0;
    int64_t stride;
};

__device__ __forceinline__ StageRow stage_row(const MlaArgs &a, const AttnTile &T, int32_t layer) {
    const StageTile S = stage_tile(a, T, 0, layer);
    const bool pool = S.info & kInfoPool;
    const uint64_t base = reinterpret_cast<uint64_t>(pool ? a.pool_k : a.cache_k);
    return StageRow{base + 2 * static_cast<uint64_t>(S.off0), 2 * (pool ? a.s_tok : a.c_tok)};
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef const void __attribute__((address_space(1))) *gptr_t;
typedef void __attribute__((address_space(3))) *lptr_t;

// HT head groups of 16 per wave.  HT = 1 (two waves per SIMD): the register
// budget is 256 per lane (72 for the queries, 128 accumulators, the rest for
// fragments in flight).  HT = 2 (one wave per SIMD, 512 registers): 144 for
// the queries, 256 accumulators (in AGPRs), and every staged fragment read
// from LDS feeds twice the matrix-core work, which halves the LDS traffic
// per product.  Scheduling barriers keep the compiler from hoisting every
// LDS read of a phase ahead.  NB staging buffers: 4 keep three steps in
// flight; 2 overlap a step's loads with the previous step's work inside the
// workgroup; 1 halves the LDS so that twice as many workgroups share a CU
// and overlap each other instead.  TPS 16-position tiles per step: 2 (the
// value product on 16x16x32 tiles), or 1 (on 16x16x16 tiles), which halves a
// step's LDS so that a one-wave workgroup can hold two steps and still share
// a CU with three others.
template <int STYLE, int W, int NB, int TPS, int HT>
__device__ __forceinline__ void mla_block_body(const MlaArgs &a, int32_t layer) {
    static_assert(TPS == 1 || TPS == 2, "position tiles per step");
    static_assert(HT == 1 || (HT == 2 && TPS == 2 && NB == 4), "head groups per wave");
    constexpr int kStepPos = 16 * TPS;      // positions per step
    constexpr int kSlabs = TPS * kKSteps;   // 1 KB slabs of a staged step
    // staged step: slab j = (k-step j / TPS, position tile j % TPS); slot
    // 16 g + p of a slab holds dims 32 s + 8 g .. + 8 of position 16 tau + p,
    // i.e. the A fragment of lane 16 g + p
    __shared__ __attribute__((aligned(16))) uint4 s_stage[NB][kSlabs * 64];
    __shared__ __attribute__((aligned(16))) double2 s_cs[kBlockTabs][kHalfR];  // block's shift tables
    __shared__ StageTile s_tiles[HT == 1 ? kItemTiles : 1];
    // two-group waves: every block position's tile (bits 0-5) and damping
    // (bit 6), every tile's row address and stride and its table slot + 1
    __shared__ uint8_t s_pinfo[HT == 2 ? kItemBlockPos : 1];
    __shared__ __attribute__((aligned(16))) StageRow s_rows[HT == 2 ? kItemTiles : 1];
    __shared__ uint8_t s_tslot[HT == 2 ? kItemTiles : 1];
    static_assert(kItemTiles <= 64, "tile index in 6 bits");
    __shared__ uint32_t s_pslot[NB][kStepPos];                        // table slot + 1 (0: not turned)
    __shared__ __attribute__((aligned(16))) float s_pbias[NB][kStepPos];  // damping, -inf past the block

    // the head-group sets of an item sit on one XCD: workgroup w runs on XCD w % 8
    const int wid = blockIdx.x;
    const int slot = wid >> 3;
    const int set = slot % a.n_sets;
    const int item = (slot / a.n_sets) * 8 + (wid & 7);
    if (item >= a.n_items) return;  // uniform over the workgroup
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r16 = lane & 15, g = lane >> 4;
    const int hg0 = (set * W + wave) * HT;  // the wave's first head group
    const int b_lo = a.item_block0[item], b_hi = a.item_block0[item + 1];
    const int request = a.blocks[b_lo].request;
    const float scale2 = a.scale * kLog2e;  // logits in log2 units (exp2 weights)
    const float bias2 = a.sink_bias * kLog2e;

    // ---- query fragments (B of S^T = K Q^T): head r16 of group hg0 + h,
    // dims 32 s + 8 g .. + 8 of k-step s
    bf16x8 qf[HT][kKSteps];
#pragma unroll
    for (int h = 0; h < HT; h++) {
        const uint16_t *qrow = a.q + request * a.q_req + ((hg0 + h) * kGroupHeads + r16) * a.q_head;
#pragma unroll
        for (int s = 0; s < kKSteps; s++)
            qf[h][s] = as_bf16x8(*reinterpret_cast<const uint4 *>(qrow + 32 * s + 8 * g));
    }

    f32x4 acc[HT][kDTiles];
#pragma unroll
    for (int h = 0; h < HT; h++)
#pragma unroll
        for (int t = 0; t < kDTiles; t++) acc[h][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[HT], l_run[HT];
#pragma unroll
    for (int h = 0; h < HT; h++) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.f;
    }
    // lane part of the transposing V^T reads (see the value product)
    const int pq = r16 >> 2, dq = r16 & 3;
    const int vt_lane = ((16 * (dq >> 1) + 4 * g + pq) * 16 + 8 * (dq & 1));

    for (int b = b_lo; b < b_hi; b++) {
        const AttnBlock B = a.blocks[b];
        __syncthreads();  // the previous block's steps are done with s_tiles and s_stage
        if constexpr (HT == 1) {
            if (tid < B.ntiles) {
                const AttnTile T = a.tiles[B.tile0 + tid];
                int sl = -1;
#pragma unroll
                for (int j = 0; j < kBlockTabs; j++)
                    if (T.cs_idx >= 0 && a.block_tabs[kBlockTabs * b + j] == T.cs_idx) sl = j;
                s_tiles[tid] = stage_tile(a, T, sl, layer);
            }
        } else {
            // four threads per tile fill its positions' bytes
            const int t = tid >> 2;
            if (t < B.ntiles) {
                const AttnTile T = a.tiles[B.tile0 + t];
                if ((tid & 3) == 0) {
                    int sl = -1;
#pragma unroll
                    for (int j = 0; j < kBlockTabs; j++)
                        if (T.cs_idx >= 0 && a.block_tabs[kBlockTabs * b + j] == T.cs_idx) sl = j;
                    s_rows[t] = stage_row(a, T, layer);
                    s_tslot[t] = static_cast<uint8_t>(sl + 1);
                }
                const int damp = static_cast<int>(std::min<int64_t>(
                    std::max<int64_t>(int64_t{a.sink_tokens} - T.sink_dist, 0), T.ntok));
                for (int k = tid & 3; k < T.ntok; k += 4)
                    s_pinfo[T.tok0 + k] = static_cast<uint8_t>(t | (k < damp ? 64 : 0));
            }
        }
        for (int i = tid; i < kBlockTabs * kHalfR; i += 64 * W) {
            const int j = i / kHalfR, pl = i - j * kHalfR;
            const int tab = a.block_tabs[kBlockTabs * b + j];
            if (tab >= 0) {
                const double *src = a.cs + (static_cast<int64_t>(tab) * kHalfR + pl) * 2;
                s_cs[j][pl] = make_double2(src[0], src[1]);
            }
        }
        __syncthreads();
        // stage step p0 into buffer bf: wave w loads slabs TPS w + tau,
        // + TPS W, ... of position tile tau; lanes past the block's end repeat position p0
        // (their weights are 0).  The tile holding a lane's position is found
        // by a forward search (positions only grow within a block).
        int cur[2] = {0, 0};
        const int wave_u = __builtin_amdgcn_readfirstlane(wave);
        auto stage = [&](int p0, int bf) {
            if constexpr (HT == 2) {
                // wave w loads k-steps w, w + 4, ... (slabs 2 w + tau + 8 k) of
                // both position tiles: one address per tile, the k-steps 256
                // bytes apart in the row (the instruction's offset)
                static_assert(TPS == 2 && W == 4 && kKSteps == 18, "two-group staging layout");
#pragma unroll
                for (int tau = 0; tau < TPS; tau++) {
                    int pi = p0 + 16 * tau + r16;
                    const bool valid = pi < B.ntok;
                    if (!valid) pi = p0;
                    const uint32_t info = s_pinfo[pi];
                    const uint32_t t = info & 63u;
                    const StageRow R = s_rows[t];
                    if (wave == 0 && g == 0) {
                        s_pslot[bf][16 * tau + r16] = valid ? s_tslot[t] : 0u;
                        s_pbias[bf][16 * tau + r16] = valid ? ((info & 64u) ? bias2 : 0.f) : -INFINITY;
                    }
                    const char *row = reinterpret_cast<const char *>(
                        R.addr0 + static_cast<uint64_t>(static_cast<int64_t>(pi) * R.stride)) +
                        16 * g + 64 * wave_u;
                    uint4 *slab = &s_stage[bf][(TPS * wave_u + tau) * 64];
                    load_lds16<0>(row, slab);
                    load_lds16<256>(row, slab + 8 * 64);
                    load_lds16<512>(row, slab + 16 * 64);
                    load_lds16<768>(row, slab + 24 * 64);
                    if (TPS * wave_u + tau + 32 < kSlabs) load_lds16<1024>(row, slab + 32 * 64);
                }
                return;
            }
#pragma unroll
            for (int tau = 0; tau < TPS; tau++) {
                int pi = p0 + 16 * tau + r16;
                const bool valid = pi < B.ntok;
                if (!valid) pi = p0;
                while (cur[tau] + 1 < B.ntiles && s_tiles[cur[tau] + 1].tok0 <= pi) cur[tau]++;
                const StageTile T = s_tiles[cur[tau]];
                const bool pool = T.info & kInfoPool;
                const int64_t off = T.off0 + static_cast<int64_t>(pi) * (pool ? a.s_tok : a.c_tok);
                if (wave == 0 && g == 0) {
                    const bool damp = static_cast<uint32_t>(pi - T.tok0) < (T.info >> 8);
                    s_pslot[bf][16 * tau + r16] = valid ? (T.info & 7u) : 0u;
                    s_pbias[bf][16 * tau + r16] = valid ? (damp ? bias2 : 0.f) : -INFINITY;
                }
                const uint16_t *row = (pool ? a.pool_k : a.cache_k) + off + 8 * g;
                if constexpr (W == 1 && TPS == 1) {
                    // the row's 18 k-steps with one base address: slab s at
                    // 1 KB s in LDS, k-step s 64 s bytes into the row
                    load_lds16_row18(row, &s_stage[bf][0]);
                } else {
                    for (int j = TPS * wave + tau; j < kSlabs; j += TPS * W) {
                        const int s = j / TPS;
                        load_lds16(row + 32 * s, &s_stage[bf][j * 64]);
                    }
                }
            }
        };

        // turn the rotary slots of moved chunk rows of buffer bb, in LDS: unit
        // u = (position, 8-plane group gg, pair qh) turns planes 2 qh, 2 qh + 1
        // of the group, with the stitch's fp64 turn and rounding.  A wave's
        // lanes take 16 positions of one 8-plane group, so its LDS words are
        // 256 contiguous bytes (no bank conflicts).  Without branches: a unit
        // of a row that is not turned writes its words back unchanged.
        auto turn_unit = [&](int bb, int u) {
            const int qh = u & 3, pos = (u >> 2) % kStepPos, gg = (u >> 2) / kStepPos;
            // (clamped: after a block's last step the buffer may hold any bits)
            const uint32_t slot1 = min(s_pslot[bb][pos], static_cast<uint32_t>(kBlockTabs));
            const bool on = slot1 != 0u;
            const double2 *tab = s_cs[on ? slot1 - 1 : 0];
            const int tau = pos >> 4, pp = pos & 15;
            uint32_t *kx = reinterpret_cast<uint32_t *>(
                &s_stage[bb][(TPS * kRopeStep + tau) * 64 + 16 * gg + pp]);
            uint32_t *ky = reinterpret_cast<uint32_t *>(
                &s_stage[bb][(TPS * (kRopeStep + 1) + tau) * 64 + 16 * gg + pp]);
            if constexpr (STYLE == PIC_ROPE_HALF) {
                // x of planes 8 gg + 2 qh, + 1 in word qh of the first rotary
                // k-step's piece, their y (32 planes later) in the second's
                const uint32_t ox = kx[qh], oy = ky[qh];
                uint32_t wx = ox, wy = oy;
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const double2 cs = tab[8 * gg + 2 * qh + h];
                    const int sh = 16 * h;
                    const double x = static_cast<double>(__uint_as_float(((ox >> sh) & 0xFFFFu) << 16));
                    const double y = static_cast<double>(__uint_as_float(((oy >> sh) & 0xFFFFu) << 16));
                    const uint32_t nx = f64_to_bf16(x * cs.x - y * cs.y);
                    const uint32_t ny = f64_to_bf16(x * cs.y + y * cs.x);
                    wx = (wx & ~(0xFFFFu << sh)) | (nx << sh);
                    wy = (wy & ~(0xFFFFu << sh)) | (ny << sh);
                }
                kx[qh] = on ? wx : ox;
                ky[qh] = on ? wy : oy;
            } else {
                // a whole pair per word: words 2 qh, 2 qh + 1 of the first
                // piece hold planes 4 gg + 2 qh, + 1 (qh < 2); of the second,
                // planes 16 + 4 gg + 2 qh - 4, + 1 (qh >= 2)
                uint32_t *wp = qh < 2 ? kx + 2 * qh : ky + 2 * qh - 4;
                const int plane0 = qh < 2 ? 4 * gg + 2 * qh : 16 + 4 * gg + 2 * qh - 4;
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const double2 cs = tab[plane0 + h];
                    const uint32_t w = wp[h];
                    const double x = bf16_lo(w), y = bf16_hi(w);
                    const uint32_t n = f64_to_bf16(x * cs.x - y * cs.y) |
                                       (f64_to_bf16(x * cs.y + y * cs.x) << 16);
                    wp[h] = on ? n : w;
                }
            }
        };
        // one-wave workgroups (steps of one 16-position tile): lane 16 g + p
        // turns the 8 planes of dim group g of position p, whose x and y (half
        // pairing) or pairs (interleaved) are its two pieces of the rotary
        // k-steps' slabs; in fp32 first, with the fp64 turn only for the
        // planes where fp32 could round otherwise (rotate.hpp: turn_f32), each
        // under its own branch, so a wave pays fp64 work for the planes some
        // lane flagged.  The fp32 cos and sin are the fp64 table's, rounded.
        auto turn8 = [&](int bb) {
            const int p = r16;
            const uint32_t slot1 = min(s_pslot[bb][p], static_cast<uint32_t>(kBlockTabs));
            const bool on = slot1 != 0u;
            const double2 *tab = s_cs[on ? slot1 - 1 : 0];
            uint4 &ka = s_stage[bb][kRopeStep * 64 + 16 * g + p];
            uint4 &kb = s_stage[bb][(kRopeStep + 1) * 64 + 16 * g + p];
            const uint4 va = ka, vb = kb;
            const uint32_t wa[4] = {va.x, va.y, va.z, va.w}, wb[4] = {vb.x, vb.y, vb.z, vb.w};
            // planes of the lane: half pairing 8 g + e (x in piece a, y in b);
            // interleaved 4 g + k (piece a, word k) and 16 + 4 g + k (piece b)
            auto plane = [&](int e) {
                return STYLE == PIC_ROPE_HALF ? 8 * g + e : (e < 4 ? 4 * g + e : 16 + 4 * g + e - 4);
            };
            uint32_t na[4], nb[4];
            uint64_t redo[8];
#pragma unroll
            for (int k = 0; k < 4; k++) {
                if constexpr (STYLE == PIC_ROPE_HALF) {
                    const double2 d0 = tab[plane(2 * k)], d1 = tab[plane(2 * k + 1)];
                    float rx0, ry0, rx1, ry1;
                    redo[2 * k] = __ballot(on && turn_f32(__uint_as_float(wa[k] << 16), __uint_as_float(wb[k] << 16),
                                                          static_cast<float>(d0.x), static_cast<float>(d0.y), &rx0, &ry0));
                    redo[2 * k + 1] = __ballot(on && turn_f32(__uint_as_float(wa[k] & 0xFFFF0000u),
                                                              __uint_as_float(wb[k] & 0xFFFF0000u),
                                                              static_cast<float>(d1.x), static_cast<float>(d1.y), &rx1, &ry1));
                    na[k] = pack2_bf16(rx0, rx1);
                    nb[k] = pack2_bf16(ry0, ry1);
                } else {
                    const double2 da = tab[plane(k)], db = tab[plane(4 + k)];
                    float rx, ry;
                    redo[k] = __ballot(on && turn_f32(__uint_as_float(wa[k] << 16), __uint_as_float(wa[k] & 0xFFFF0000u),
                                                      static_cast<float>(da.x), static_cast<float>(da.y), &rx, &ry));
                    na[k] = pack2_bf16(rx, ry);
                    redo[4 + k] = __ballot(on && turn_f32(__uint_as_float(wb[k] << 16), __uint_as_float(wb[k] & 0xFFFF0000u),
                                                          static_cast<float>(db.x), static_cast<float>(db.y), &rx, &ry));
                    nb[k] = pack2_bf16(rx, ry);
                }
            }
            uint64_t any_redo = 0;
#pragma unroll
            for (int e = 0; e < 8; e++) any_redo |= redo[e];
            if (any_redo != 0) {  // uniform
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    if (!((redo[e] >> lane) & 1)) continue;
                    const double2 cs = tab[plane(e)];
                    if constexpr (STYLE == PIC_ROPE_HALF) {
                        // plane e: half e % 2 of word e / 2 in both pieces
                        const int k = e >> 1, sh = 16 * (e & 1);
                        const double x = (e & 1) ? bf16_hi(wa[k]) : bf16_lo(wa[k]);
                        const double y = (e & 1) ? bf16_hi(wb[k]) : bf16_lo(wb[k]);
                        const uint32_t keep = 0xFFFF0000u >> sh;
                        na[k] = (na[k] & keep) | (f64_to_bf16(x * cs.x - y * cs.y) << sh);
                        nb[k] = (nb[k] & keep) | (f64_to_bf16(x * cs.y + y * cs.x) << sh);
                    } else {
                        // plane e: word e % 4 of piece a (e < 4) or b
                        const uint32_t w = e < 4 ? wa[e & 3] : wb[e & 3];
                        const double x = bf16_lo(w), y = bf16_hi(w);
                        const uint32_t r = pack_bf16(x * cs.x - y * cs.y, x * cs.y + y * cs.x);
                        if (e < 4) na[e & 3] = r;
                        else nb[e & 3] = r;
                    }
                }
            }
            if (on) {
                ka = make_uint4(na[0], na[1], na[2], na[3]);
                kb = make_uint4(nb[0], nb[1], nb[2], nb[3]);
            }
        };
        auto turn = [&](int bb) {
            if constexpr (W == 1 && TPS == 1) {
                turn8(bb);
                return;
            }
            for (int u = tid; u < 16 * kStepPos; u += 64 * W) {
                if (s_pslot[bb][(u >> 2) % kStepPos] == 0u) continue;
                turn_unit(bb, u);
            }
        };

        // NB = 4: step i is computed while step i + 1 is turned and steps
        // i + 2, i + 3 load, one barrier per step; NB = 2: the next step loads
        // while this one is turned and computed; NB = 1: it loads after.  A
        // stage call issues at least kMinLoads loads per wave (wave 0 may
        // issue more), which complete in order: waiting until at most n
        // kMinLoads are outstanding leaves the newest n stage calls in flight.
        constexpr int kMinLoads = TPS * ((kSlabs - TPS * W) / (TPS * W) + 1);
        const int nsteps = (B.ntok + kStepPos - 1) / kStepPos;
        stage(0, 0);
        if constexpr (NB == 4) {
            if (nsteps > 1) stage(kStepPos, 1);
            if (nsteps > 2) stage(2 * kStepPos, 2);
            const int newer = (nsteps > 1) + (nsteps > 2);
            if (newer == 2) wait_vm<2 * kMinLoads>();
            else if (newer == 1) wait_vm<kMinLoads>();
            else wait_vm<0>();
            __syncthreads();
            turn(0);
        }
        for (int i = 0; i < nsteps; i++) {
            const int p0 = i * kStepPos;
            int cb;  // the buffer computed on
            bf16x8 kq[kSDepth];  // two-group waves: the first logit fragments
            if constexpr (NB == 4) {
                // step i + 1's loads are in (i + 2's may not be); after the
                // barrier every wave's are, step i is turned, step i - 1's
                // buffer is free
                if (i + 2 < nsteps) wait_vm<kMinLoads>();
                else wait_vm<0>();
                __syncthreads();
                cb = i & 3;
                if constexpr (HT == 2) {
                    // read ahead of the staging and the turn, which hide their latency
#pragma unroll
                    for (int f = 0; f < kSDepth; f++) kq[f] = as_bf16x8(s_stage[cb][f * 64 + lane]);
                }
                if (i + 3 < nsteps) stage(p0 + 3 * kStepPos, (i + 3) & 3);
                // two-group waves turn step i + 1 among the value products
                if (HT == 1 && i + 1 < nsteps) turn((i + 1) & 3);
            } else {
                wait_vm<0>();
                __syncthreads();  // the step is in LDS (every wave's share) and its meta written
                cb = NB == 2 ? (i & 1) : 0;
                if (NB == 2 && i + 1 < nsteps) stage(p0 + kStepPos, cb ^ 1);
                turn(cb);
                __syncthreads();
            }

            // ---- logits S^T for the wave's heads
            const uint4 *stg = s_stage[cb];
            f32x4 st[HT][TPS];
#pragma unroll
            for (int h = 0; h < HT; h++)
#pragma unroll
                for (int tau = 0; tau < TPS; tau++) st[h][tau] = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (HT == 2) {
                // fragments f = TPS s + tau in slab order, the first kSDepth
                // read at the top of the step, later ones kSDepth ahead
                constexpr int kSFrags = TPS * kKSteps;
#pragma unroll
                for (int f = 0; f < kSFrags; f++) {
                    const int s = f / TPS, tau = f % TPS;
                    const bf16x8 kf = kq[f % kSDepth];
                    if (f + kSDepth < kSFrags) kq[f % kSDepth] = as_bf16x8(stg[(f + kSDepth) * 64 + lane]);
#pragma unroll
                    for (int h = 0; h < HT; h++) {
                        if (s == 0)
                            mfma_v<true>(st[h][tau], kf, qf[h][s]);
                        else
                            mfma_v<false>(st[h][tau], kf, qf[h][s]);
                    }
                    if (tau == TPS - 1) __builtin_amdgcn_sched_barrier(0);
                }
                vgpr_mfma_guard(st[0][0], st[0][1], st[1][0], st[1][1]);
            } else {
#pragma unroll
                for (int s = 0; s < kKSteps; s++) {
#pragma unroll
                    for (int tau = 0; tau < TPS; tau++)
                        st[0][tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            as_bf16x8(stg[(TPS * s + tau) * 64 + lane]), qf[0][s], st[0][tau], 0, 0, 0);
                    if (s % 6 == 5) __builtin_amdgcn_sched_barrier(0);
                }
            }

            // ---- online softmax over head r16 of each group (log2 units):
            // this lane holds positions p0 + 16 tau + 4 g + i.  The running max
            // is kept until a logit passes it by kLazy (weights stay below
            // 2^kLazy; the merge uses the same reference), so the accumulator
            // is seldom rescaled
            constexpr int NV = 4 * TPS;  // logits per lane and group
            float pb[NV];
#pragma unroll
            for (int tau = 0; tau < TPS; tau++) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(&s_pbias[cb][16 * tau + 4 * g]);
#pragma unroll
                for (int i = 0; i < 4; i++) pb[4 * tau + i] = v[i];
            }
            // the first V^T fragments (see the value product), read ahead of the softmax
            const char *vt = reinterpret_cast<const char *>(stg) + vt_lane;
            constexpr int kTileBytes = 64 * 16;  // one slab
            auto vt_frag = [&](int t) {
                const int tc = (TPS * (t >> 1)) * kTileBytes + 32 * 16 * (t & 1);
                const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vt + tc));
                const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4 *)(vt + tc + kTileBytes));  // tile 1: the next slab
                const uint2 w0 = __builtin_bit_cast(uint2, v0), w1 = __builtin_bit_cast(uint2, v1);
                return as_bf16x8(make_uint4(w0.x, w0.y, w1.x, w1.y));
            };
            bf16x8 vq[kVDepth];
            if constexpr (HT == 2) {
#pragma unroll
                for (int t = 0; t < kVDepth; t++) vq[t] = vt_frag(t);
            }
            // weights as B of O^T += V^T P^T: k index 8 g + j is position
            // 4 g + j (j < 4) or 16 + 4 g + j - 4 with two tiles, k index 4 g + j
            // position 4 g + j with one -- the order of pw; hi + lo bf16
            uint32_t hi[HT][NV / 2], lo[HT][NV / 2];
#pragma unroll
            for (int h = 0; h < HT; h++) {
                float sc[NV];
#pragma unroll
                for (int tau = 0; tau < TPS; tau++)
#pragma unroll
                    for (int i = 0; i < 4; i++) sc[4 * tau + i] = fmaf(st[h][tau][i], scale2, pb[4 * tau + i]);
                float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
                if constexpr (TPS == 2) mx = fmaxf(mx, fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
                mx = row_max(mx);  // finite: position p0 is in the block
                const bool bump = mx > m_run[h] + kLazy;  // (-inf + kLazy stays -inf)
                const float m_new = bump ? mx : m_run[h];
                const float alpha = bump ? __builtin_amdgcn_exp2f(m_run[h] - m_new) : 1.f;
                float pw[NV];
#pragma unroll
                for (int k = 0; k < NV; k++) pw[k] = __builtin_amdgcn_exp2f(sc[k] - m_new);
                float psum = (pw[0] + pw[1]) + (pw[2] + pw[3]);
                if constexpr (TPS == 2) psum += (pw[4] + pw[5]) + (pw[6] + pw[7]);
                l_run[h] = l_run[h] * alpha + psum;
                m_run[h] = m_new;
                if (__any(bump)) {
                    // one wave per SIMD: the accumulators live in AGPRs, and
                    // plain code paid their copies at every step
                    if constexpr (W <= 2 || HT == 2) {
                        acc_read_guard();
#pragma unroll
                        for (int t = 0; t < kDTiles; t++) scale_acc(acc[h][t], alpha);
                    } else {
#pragma unroll
                        for (int t = 0; t < kDTiles; t++) acc[h][t] *= alpha;
                    }
                }
#pragma unroll
                for (int k = 0; k < NV / 2; k++) {
                    const f32x2 pr = {pw[2 * k], pw[2 * k + 1]};
                    hi[h][k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
                    const f32x2 rr = {pw[2 * k] - __uint_as_float(hi[h][k] << 16),
                                      pw[2 * k + 1] - __uint_as_float(hi[h][k] & 0xFFFF0000u)};
                    lo[h][k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(rr, bf16x2));
                }
            }

            // ---- A = V^T (dim d = 16 t + r16; positions 4 g .. 4 g + 3, then
            // 16 + 4 g .. + 3) by transposing LDS reads: within each 16-lane
            // group, lane i receives element i % 4 of the 8-byte rows that
            // lanes 4 j + i / 4 address (j = 0..3).  So lane i of group g
            // addresses position 4 g + i / 4 (+ 16 for the second tile), dims
            // 16 t + 4 (i % 4) .. + 4: slab (t / 2, tile), slot 16 g' + position
            // % 16 with g' = 2 (t % 2) + (i % 4) / 2, second half when i is odd.
            // The lane's part of the address is vt_lane; tile t adds a constant.
            if constexpr (HT == 2) {
                // kVDepth fragments read ahead: tile t + kVDepth's reads are
                // issued with tile t's products (four per fragment)
#pragma unroll
                for (int t = 0; t < kDTiles; t++) {
                    const bf16x8 va = vq[t % kVDepth];
                    if (t + kVDepth < kDTiles) vq[t % kVDepth] = vt_frag(t + kVDepth);
#pragma unroll
                    for (int h = 0; h < HT; h++) {
                        const bf16x8 phi = as_bf16x8(make_uint4(hi[h][0], hi[h][1], hi[h][2], hi[h][3]));
                        const bf16x8 plo = as_bf16x8(make_uint4(lo[h][0], lo[h][1], lo[h][2], lo[h][3]));
                        acc[h][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi, acc[h][t], 0, 0, 0);
                        acc[h][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, plo, acc[h][t], 0, 0, 0);
                    }
                    // the turn of the next step's buffer, one unit per thread
                    // among tiles kTurnAt[k] .. + 3 (the vector work of a turn
                    // takes about as long as their 16 products).  After the
                    // block's last step it turns a buffer no step reads again.
                    if (t == kTurnAt0 || t == kTurnAt1)
                        turn_unit((i + 1) & 3, tid + (t == kTurnAt0 ? 0 : 64 * W));
                    if (!((t >= kTurnAt0 && t < kTurnAt0 + 3) || (t >= kTurnAt1 && t < kTurnAt1 + 3)))
                        __builtin_amdgcn_sched_barrier(0);
                }
            } else
#pragma unroll
            for (int t = 0; t < kDTiles; t++) {
                const int tc = (TPS * (t >> 1)) * kTileBytes + 32 * 16 * (t & 1);
                const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vt + tc));
                if constexpr (TPS == 2) {
                    const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4 *)(vt + tc + kTileBytes));  // tile 1: the next slab
                    const uint2 w0 = __builtin_bit_cast(uint2, v0), w1 = __builtin_bit_cast(uint2, v1);
                    const bf16x8 va = as_bf16x8(make_uint4(w0.x, w0.y, w1.x, w1.y));
#pragma unroll
                    for (int h = 0; h < HT; h++) {
                        const bf16x8 phi = as_bf16x8(make_uint4(hi[h][0], hi[h][1], hi[h][2], hi[h][3]));
                        const bf16x8 plo = as_bf16x8(make_uint4(lo[h][0], lo[h][1], lo[h][2], lo[h][3]));
                        acc[h][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi, acc[h][t], 0, 0, 0);
                        acc[h][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, plo, acc[h][t], 0, 0, 0);
                    }
                } else {
                    const s16x4 phi = __builtin_bit_cast(s16x4, make_uint2(hi[0][0], hi[0][1]));
                    const s16x4 plo = __builtin_bit_cast(s16x4, make_uint2(lo[0][0], lo[0][1]));
                    acc[0][t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v0, phi, acc[0][t], 0, 0, 0);
                    acc[0][t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v0, plo, acc[0][t], 0, 0, 0);
                }
                if (t % 4 == 3) __builtin_amdgcn_sched_barrier(0);
            }
            if (NB == 1 && i + 1 < nsteps) {
                __syncthreads();  // every wave is done with the buffer
                stage(p0 + kStepPos, 0);
            }
        }
    }

    // ---- partial results: O^T D registers hold dims 16 t + 4 g + i of head r16
#pragma unroll
    for (int h = 0; h < HT; h++) {
        float l = l_run[h];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        const int head = (hg0 + h) * kGroupHeads + r16;
        const int64_t slot_id = static_cast<int64_t>(item) * a.num_q_heads + head;
        float *pa = a.part_acc + slot_id * kVDim;
#pragma unroll
        for (int t = 0; t < kDTiles; t++)
            *reinterpret_cast<float4 *>(pa + 16 * t + 4 * g) =
                make_float4(acc[h][t][0], acc[h][t][1], acc[h][t][2], acc[h][t][3]);
        if (g == 0) {
            a.part_ml[2 * slot_id] = m_run[h];
            a.part_ml[2 * slot_id + 1] = l;
        }
    }
}

template <int STYLE, int W, int NB, int TPS>
__global__ void __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2)))
mla_block_kernel(const MlaArgs a, int32_t layer) {
    mla_block_body<STYLE, W, NB, TPS, 1>(a, layer);
}

// 128 query heads per workgroup: four waves of two head groups, one wave per
// SIMD
template <int STYLE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_wide_kernel(const MlaArgs a, int32_t layer) {
    mla_block_body<STYLE, 4, 4, 2, 2>(a, layer);
}

// out[r][j][d] = sum_b acc_b[d] e^{m_b - M} / sum_b l_b e^{m_b - M} over the
// request's items b.  Wave w takes items b0 + w, b0 + w + 4, ...; lane i holds
// dims 4 i .. 4 i + 3 and 256 + 4 i .. + 3, so each item's 2 KB row is one
// coalesced read per wave, and four items per wave are in flight.  The waves'
// sums meet in LDS; thread t writes dims t and t + 256.
__global__ void __launch_bounds__(kCombineThreads) mla_combine_kernel(const MlaArgs a) {
    constexpr int kWaves = kCombineThreads / 64;
    static_assert(kVDim == 2 * kCombineThreads && kCombineThreads % 64 == 0,
                  "a lane holds two float4 of the value row");
    __shared__ __attribute__((aligned(16))) float s_o[kWaves][kVDim];
    __shared__ float s_red[kWaves];
    __shared__ float s_l[kWaves];
    const int r = blockIdx.x;
    const int j = blockIdx.y;
    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const int b0 = a.req_item0[r], b1 = a.req_item0[r + 1];
    const int64_t hq = a.num_q_heads;
    float M = -INFINITY;
    for (int b = b0 + t; b < b1; b += kCombineThreads) M = fmaxf(M, a.part_ml[(b * hq + j) * 2]);
    for (int x = 1; x < 64; x <<= 1) M = fmaxf(M, __shfl_xor(M, x, 64));
    if (lane == 0) s_red[w] = M;
    __syncthreads();
    M = s_red[0];
#pragma unroll
    for (int v = 1; v < kWaves; v++) M = fmaxf(M, s_red[v]);
    float L = 0.f;
    float4 o0 = make_float4(0.f, 0.f, 0.f, 0.f), o1 = o0;
#pragma unroll 4
    for (int b = b0 + w; b < b1; b += kWaves) {
        const int64_t slot = static_cast<int64_t>(b) * hq + j;
        const float2 ml = *reinterpret_cast<const float2 *>(a.part_ml + 2 * slot);
        const float4 *row = reinterpret_cast<const float4 *>(a.part_acc + slot * kVDim);
        const float4 x0 = row[lane], x1 = row[64 + lane];
        const float f = __builtin_amdgcn_exp2f(ml.x - M);  // log2 units
        L += ml.y * f;
        o0.x += x0.x * f; o0.y += x0.y * f; o0.z += x0.z * f; o0.w += x0.w * f;
        o1.x += x1.x * f; o1.y += x1.y * f; o1.z += x1.z * f; o1.w += x1.w * f;
    }
    *reinterpret_cast<float4 *>(&s_o[w][4 * lane]) = o0;
    *reinterpret_cast<float4 *>(&s_o[w][256 + 4 * lane]) = o1;
    if (lane == 0) s_l[w] = L;
    __syncthreads();
    float Lt = s_l[0], O0 = s_o[0][t], O1 = s_o[0][t + kCombineThreads];
#pragma unroll
    for (int v = 1; v < kWaves; v++) {
        Lt += s_l[v];
        O0 += s_o[v][t];
        O1 += s_o[v][t + kCombineThreads];
    }
    float *o = a.out + r * a.o_req + j * a.o_head;
    o[t] = O0 / Lt;
    o[t + kCombineThreads] = O1 / Lt;
}

// ------------------------------------------------------------------ host

int cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    return n;
}

#ifndef PIC_MLA_NB1
#define PIC_MLA_NB1 2
#endif
#ifndef PIC_MLA_TPS1
#define PIC_MLA_TPS1 1
#endif
// staging buffers and position tiles per step of the one-wave workgroup
constexpr int kNb1 = PIC_MLA_NB1;
constexpr int kTps1 = PIC_MLA_TPS1;
// one-wave workgroups per CU: LDS holds kNb1 steps of 16 kTps1 rows (18 KB a
// tile) plus about 3 KB of tables; registers allow eight waves
constexpr int kPerCu1 = std::min(8, 160 / (18 * kNb1 * kTps1 + 3));

template <int STYLE>
hipError_t launch_block(int w, dim3 grid, hipStream_t stream, const MlaArgs &a, int32_t layer) {
    switch (w) {
        case 8: hipLaunchKernelGGL((mla_wide_kernel<STYLE>), grid, dim3(256), 0, stream, a, layer); break;
        case 4: hipLaunchKernelGGL((mla_block_kernel<STYLE, 4, 2, 2>), grid, dim3(256), 0, stream, a, layer); break;
        case 2: hipLaunchKernelGGL((mla_block_kernel<STYLE, 2, 2, 2>), grid, dim3(128), 0, stream, a, layer); break;
        default:
            hipLaunchKernelGGL((mla_block_kernel<STYLE, 1, kNb1, kTps1>), grid, dim3(64), 0, stream, a, layer);
            break;
    }
    return hipGetLastError();
}

}  // namespace
}  // namespace pic

extern "C" pic_status pic_attend_latent(pic_plan_t *plan, const pic_kv_view *pool,
                                        const pic_kv_view *cache,
                                        const pic_attend_latent_args *args, void *stream_) {
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
    if (p.shape.dtype != PIC_DTYPE_BF16 || p.shape.num_heads != 1 || p.shape.has_v ||
        p.shape.row_dim != kRow || p.shape.rope_offset != kRopeOff || p.rope_dim != kRopeDim)
        return fail(PIC_ERR_INVALID_ARG, "pic_attend_latent needs a bf16 MLA plan: one 576-wide "
                    "row per token (512 content dims, 64 rotary dims at 512), no V rows");
    if (args->num_q_heads < kGroupHeads || args->num_q_heads % kGroupHeads != 0 ||
        args->num_q_heads > 1024)
        return fail(PIC_ERR_INVALID_ARG, "num_q_heads %d: need a multiple of %d, at most 1024",
                    args->num_q_heads, kGroupHeads);
    if (args->layer < 0 || args->layer >= p.shape.num_layers)
        return fail(PIC_ERR_INVALID_ARG, "layer %d outside [0, %d)", args->layer,
                    p.shape.num_layers);
    if (args->q_request_stride % 8 || args->q_head_stride % 8 ||
        (reinterpret_cast<uintptr_t>(args->q) & 15u))
        return fail(PIC_ERR_ALIGN, "q rows must be 16-byte aligned");
    if (args->sink_tokens < 0) return fail(PIC_ERR_INVALID_ARG, "negative sink_tokens");
    pic_status st = check_view(pool, 8, false, "pool");
    if (st) return st;
    st = check_view(cache, 8, false, "cache");
    if (st) return st;
    for (size_t r = 0; r < p.context.size(); r++) {
        if (p.context[r] <= 0)
            return fail(PIC_ERR_RANGE, "request %zu has an empty context", r);
        if (p.context_bad_page[r] >= 0)
            return fail(PIC_ERR_RANGE, "request %zu: context page %d maps outside the cache", r,
                        p.context_bad_page[r]);
    }
    if (p.ablocks.empty()) return PIC_OK;

    hipStream_t stream = static_cast<hipStream_t>(stream_);
    st = ensure_device_plan(plan, stream_);
    if (st) return st;

    // head groups per workgroup (W = 8: four waves of two groups, the rest
    // one wave per group) and workgroups per item
    const int G = args->num_q_heads / kGroupHeads;
    const int W = G % 8 == 0 ? 8 : G % 4 == 0 ? 4 : G % 2 == 0 ? 2 : 1;
    const int sets = G / W;
    // concurrent workgroups per CU: one of four 512-register waves (four
    // 37 KB staging buffers), two with two staging buffers each, kPerCu1
    // one-wave workgroups
    const int per_cu = W == 8 ? 1 : W == 1 ? kPerCu1 : 2;
    const int64_t slots = static_cast<int64_t>(cu_count()) * per_cu;
    const int64_t target = std::max<int64_t>(1, slots / sets);
    const DevBlob *blob = nullptr;
    st = plan_blob(plan, blob_key(kBlobLatent, target), stream_, [&](DevBlob &b) {
        ItemMap m = build_item_map(p, target, int64_t{1} << 30);
        b.host = std::move(m.bytes);
        b.off[0] = m.off_blocks;
        b.off[1] = m.off_items;
        b.off[2] = m.off_reqs;
        b.off[3] = m.off_tabs;
        b.n[0] = m.n_items;
        b.n[1] = m.n_blocks;
    }, &blob);
    if (st) return st;
    const int32_t n_items = blob->n[0];
    const size_t need = static_cast<size_t>(n_items) * static_cast<size_t>(args->num_q_heads) *
                        (static_cast<size_t>(kVDim) + 2) * sizeof(float);
    void *work = nullptr;
    st = call_workspace(plan, need, stream_, &work);
    if (st) return st;
    const uint8_t *dm = static_cast<const uint8_t *>(plan->d_mem);
    const uint8_t *lm = static_cast<const uint8_t *>(blob->dev);
    MlaArgs a{};
    a.tiles = reinterpret_cast<const AttnTile *>(lm);
    a.blocks = reinterpret_cast<const AttnBlock *>(lm + blob->off[0]);
    a.item_block0 = reinterpret_cast<const int32_t *>(lm + blob->off[1]);
    a.req_item0 = reinterpret_cast<const int32_t *>(lm + blob->off[2]);
    a.block_tabs = reinterpret_cast<const int32_t *>(lm + blob->off[3]);
    a.cs = reinterpret_cast<const double *>(dm + plan->staged.off_cs);
    a.pool_k = static_cast<const uint16_t *>(pool->k);
    a.cache_k = static_cast<const uint16_t *>(cache->k);
    a.s_layer = pool->layer_stride;
    a.s_tok = pool->token_stride;
    a.s_page = pool->page_stride;
    a.c_layer = cache->layer_stride;
    a.c_tok = cache->token_stride;
    a.c_page = cache->page_stride;
    a.c_req = cache->request_stride;
    a.q = static_cast<const uint16_t *>(args->q);
    a.q_req = args->q_request_stride;
    a.q_head = args->q_head_stride;
    a.out = args->out;
    a.o_req = args->out_request_stride;
    a.o_head = args->out_head_stride;
    const size_t acc_elems =
        static_cast<size_t>(n_items) * static_cast<size_t>(args->num_q_heads) * kVDim;
    a.part_acc = static_cast<float *>(work);
    a.part_ml = static_cast<float *>(work) + acc_elems;
    a.n_items = n_items;
    a.n_sets = sets;
    a.num_q_heads = args->num_q_heads;
    a.scale = args->scale;
    a.sink_tokens = args->sink_tokens;
    a.sink_bias = args->sink_bias;
    // items rounded up to a multiple of the 8 XCDs, times the head-group sets
    const dim3 grid(static_cast<unsigned>((a.n_items + 7) / 8 * 8) * static_cast<unsigned>(sets));
    hipError_t e = p.style == PIC_ROPE_HALF
                       ? launch_block<PIC_ROPE_HALF>(W, grid, stream, a, args->layer)
                       : launch_block<PIC_ROPE_INTERLEAVED>(W, grid, stream, a, args->layer);
    if (e == hipSuccess) {
        hipLaunchKernelGGL(mla_combine_kernel,
                           dim3(static_cast<unsigned>(p.context.size()),
                                static_cast<unsigned>(args->num_q_heads)),
                           dim3(kCombineThreads), 0, stream, a);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return hip_fail(e, "latent attention kernel launch");
    return note_use(plan, stream_);
}
