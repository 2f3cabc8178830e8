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
// key is turned by the chunk's shift while it is loaded (Irminsul sections
// 2.2 and 4: the delta-rotation fused into the attention kernel's load
// path); the turned key is rounded to bf16 exactly as the stitch would store
// it, so the result is attention over the stitched cache.  Every other
// position reads the request's own cache.  The EPIC Guide's LegoLink damping
// is the same optional logit bias as in pic_attend.
//
// 16 query heads share one row of 1,152 bytes: ~2,200 flops per head per row
// over 16 heads is ~30 flop/B, beyond the fp32 vector ALU at HBM speed, so
// both products run on the matrix cores (v_mfma_f32_16x16x32_bf16):
//   S^T = K Q^T: A = 16 positions x 32 dims of K (a lane holds one
//     position's 8 consecutive dims: one 16-byte load), B = the head group's
//     queries, held in registers for the whole block; D gives a lane 4
//     positions of one head.
//   O^T += V^T P^T: B = the weights straight from the D registers of two
//     S^T tiles (the k order of the product is permuted to match them), in
//     two bf16 terms (hi + lo, so the weights lose nothing to bf16); A = the
//     values transposed, which go through LDS: each lane writes the value
//     dims of the key fragments it loaded into a [dim][position] tile.
// Work item: one wave per (block of <= 256 positions of a request, group of
// 16 query heads).  The head groups of one block are mapped to the same XCD
// (workgroups are dealt round-robin over the 8 XCDs), so its rows are read
// from HBM once and from that XCD's L2 after.  Partial (max, sum,
// accumulator) per (block, head) are merged by mla_combine_kernel.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

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
constexpr int kVSteps = kVDim / 32;       // the k-steps holding value dims
constexpr int kRopeStep = kRopeOff / 32;  // first rotary k-step (x half; y in the next)
constexpr int kDTiles = kVDim / 16;       // output tiles of 16 dims
constexpr int kGroupHeads = 16;           // query heads per work item
constexpr int kStepPos = 32;              // positions per step: two 16-position tiles
constexpr int kVtStride = kStepPos + 4;   // LDS row of the transposed value tile
constexpr int kCombineThreads = 256;

constexpr uint32_t kMetaPool = 1u << 31;      // row read from the pool (else the cache)
constexpr uint32_t kMetaDamp = 1u << 30;      // LegoLink bias applies
constexpr uint32_t kMetaCs = (1u << 30) - 1;  // shift table + 1 (0: row not turned)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct MlaArgs {
    const AttnTile *tiles;
    const AttnBlock *blocks;
    const int32_t *req_block0;
    const double *cs;
    const uint16_t *pool_k, *cache_k;
    int64_t s_layer, s_tok, s_page;
    int64_t c_layer, c_tok, c_page, c_req;
    const uint16_t *q;
    int64_t q_req, q_head;
    float *out;
    int64_t o_req, o_head;
    float *part_acc;  // [block][q head][kVDim]
    float *part_ml;   // [block][q head][2]
    int32_t n_blocks, n_groups, num_q_heads;
    float scale;
    int32_t sink_tokens;
    float sink_bias;
};

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &v) {
    return __builtin_bit_cast(bf16x8, v);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int STYLE>
__global__ void __launch_bounds__(64) mla_block_kernel(const MlaArgs a, int32_t layer) {
    __shared__ AttnTile s_tiles[kAttnBlockTiles];
    __shared__ int64_t s_off[kAttnBlockTokens];
    __shared__ uint32_t s_meta[kAttnBlockTokens];
    __shared__ __attribute__((aligned(16))) uint16_t s_vt[kVDim * kVtStride];  // [dim][position]

    // the head groups of a block sit on one XCD: workgroup w runs on XCD w % 8
    const int wid = blockIdx.x;
    const int slot = wid >> 3;
    const int hg = slot % a.n_groups;
    const int block = (slot / a.n_groups) * 8 + (wid & 7);
    if (block >= a.n_blocks) return;  // uniform over the wave
    const AttnBlock B = a.blocks[block];
    const int lane = threadIdx.x;
    const int r16 = lane & 15, g = lane >> 4;

    // ---- the block's row table: element offset of every position's row
    if (lane < B.ntiles) s_tiles[lane] = a.tiles[B.tile0 + lane];
    __syncthreads();
    for (int pi = lane; pi < B.ntok; pi += 64) {
        int lo = 0, hi = B.ntiles - 1;  // the last tile starting at or before pi
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_tiles[mid].tok0 <= pi) lo = mid;
            else hi = mid - 1;
        }
        const AttnTile &T = s_tiles[lo];
        const int t = pi - T.tok0;
        const int64_t L = layer;
        int64_t off;
        uint32_t meta = 0;
        switch (T.kind) {
            case kPoolRows:
                off = L * a.s_layer + (T.a + t) * a.s_tok;
                meta = kMetaPool;
                break;
            case kPoolPages:
                off = L * a.s_layer + T.a * a.s_page + static_cast<int64_t>(T.b + t) * a.s_tok;
                meta = kMetaPool;
                break;
            case kCacheRows:
                off = L * a.c_layer + T.a * a.c_req + static_cast<int64_t>(T.b + t) * a.c_tok;
                break;
            default:
                off = L * a.c_layer + T.a * a.c_page + static_cast<int64_t>(T.b + t) * a.c_tok;
                break;
        }
        if (T.cs_idx >= 0) meta |= static_cast<uint32_t>(T.cs_idx + 1);
        if (T.sink_dist + t < a.sink_tokens) meta |= kMetaDamp;
        s_off[pi] = off;
        s_meta[pi] = meta;
    }

    // ---- query fragments (B of S^T = K Q^T): head r16 of the group, dims
    // 32 s + 8 g .. + 8 of k-step s
    bf16x8 qf[kKSteps];
    {
        const uint16_t *qrow = a.q + B.request * a.q_req + (hg * kGroupHeads + r16) * a.q_head;
#pragma unroll
        for (int s = 0; s < kKSteps; s++)
            qf[s] = as_bf16x8(*reinterpret_cast<const uint4 *>(qrow + 32 * s + 8 * g));
    }
    __syncthreads();

    f32x4 acc[kDTiles];
#pragma unroll
    for (int t = 0; t < kDTiles; t++) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    for (int p0 = 0; p0 < B.ntok; p0 += kStepPos) {
        // ---- key fragments of the step: tile tau, position p0 + 16 tau + r16
        uint4 kf[2][kKSteps];
        uint32_t meta[2];
#pragma unroll
        for (int tau = 0; tau < 2; tau++) {
            const int pi = p0 + 16 * tau + r16;
            const bool valid = pi < B.ntok;
            meta[tau] = valid ? s_meta[pi] : 0u;
            const uint16_t *row =
                ((meta[tau] & kMetaPool) ? a.pool_k : a.cache_k) + (valid ? s_off[pi] : 0);
#pragma unroll
            for (int s = 0; s < kKSteps; s++)
                kf[tau][s] = valid ? *reinterpret_cast<const uint4 *>(row + 32 * s + 8 * g)
                                   : make_uint4(0u, 0u, 0u, 0u);
        }
        // ---- turn the rotary key of pool rows whose chunk moved, rounding
        // to bf16 as the stitch stores it
#pragma unroll
        for (int tau = 0; tau < 2; tau++) {
            const uint32_t cs1 = meta[tau] & kMetaCs;
            if (cs1 == 0u) continue;
            const double *tab = a.cs + static_cast<int64_t>(cs1 - 1) * (kRopeDim / 2) * 2;
            uint4 &kx = kf[tau][kRopeStep], &ky = kf[tau][kRopeStep + 1];
            uint32_t xw[4] = {kx.x, kx.y, kx.z, kx.w}, yw[4] = {ky.x, ky.y, ky.z, ky.w};
            if constexpr (STYLE == PIC_ROPE_HALF) {
                // x of planes 8 g .. 8 g + 7 in the first rotary k-step, their
                // y (32 planes later) in the second
                double c[8], s[8];
#pragma unroll
                for (int p = 0; p < 8; p++) {
                    c[p] = tab[2 * (8 * g + p)];
                    s[p] = tab[2 * (8 * g + p) + 1];
                }
                rotate_unit<uint16_t, PIC_ROPE_HALF, 4>(xw, yw, c, s);
            } else {
                // whole pairs: planes 4 g .. 4 g + 3, then 16 + 4 g .. + 3
                double c0[4], s0[4], c1[4], s1[4];
#pragma unroll
                for (int p = 0; p < 4; p++) {
                    c0[p] = tab[2 * (4 * g + p)];
                    s0[p] = tab[2 * (4 * g + p) + 1];
                    c1[p] = tab[2 * (16 + 4 * g + p)];
                    s1[p] = tab[2 * (16 + 4 * g + p) + 1];
                }
                rotate_unit<uint16_t, PIC_ROPE_INTERLEAVED, 4>(xw, xw, c0, s0);
                rotate_unit<uint16_t, PIC_ROPE_INTERLEAVED, 4>(yw, yw, c1, s1);
            }
            kx = make_uint4(xw[0], xw[1], xw[2], xw[3]);
            ky = make_uint4(yw[0], yw[1], yw[2], yw[3]);
        }
        // ---- logits S^T for the group's heads
        f32x4 st[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int s = 0; s < kKSteps; s++)
#pragma unroll
            for (int tau = 0; tau < 2; tau++)
                st[tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[tau][s]), qf[s],
                                                                 st[tau], 0, 0, 0);
        // ---- the value dims into LDS, transposed: s_vt[dim][position in step]
#pragma unroll
        for (int tau = 0; tau < 2; tau++)
#pragma unroll
            for (int s = 0; s < kVSteps; s++) {
                const uint32_t w[4] = {kf[tau][s].x, kf[tau][s].y, kf[tau][s].z, kf[tau][s].w};
#pragma unroll
                for (int j = 0; j < 8; j++)
                    s_vt[(32 * s + 8 * g + j) * kVtStride + 16 * tau + r16] =
                        static_cast<uint16_t>((j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xFFFFu));
            }
        // ---- online softmax over head r16: this lane holds positions
        // p0 + 16 tau + 4 g + i
        float sc[8];
#pragma unroll
        for (int tau = 0; tau < 2; tau++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int pos = p0 + 16 * tau + 4 * g + i;
                float x = st[tau][i] * a.scale;
                if (pos < B.ntok && (s_meta[pos] & kMetaDamp)) x += a.sink_bias;
                sc[4 * tau + i] = pos < B.ntok ? x : -INFINITY;
            }
        float mx = sc[0];
#pragma unroll
        for (int k = 1; k < 8; k++) mx = fmaxf(mx, sc[k]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);  // finite: position p0 is in the block
        const float alpha = __expf(m_run - m_new);
        float pw[8], psum = 0.f;
#pragma unroll
        for (int k = 0; k < 8; k++) {
            pw[k] = __expf(sc[k] - m_new);
            psum += pw[k];
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int t = 0; t < kDTiles; t++) acc[t] *= alpha;
        // weights as B of O^T += V^T P^T: k index 8 g + j is position
        // 4 g + j (j < 4) or 16 + 4 g + j - 4, the order of pw; hi + lo bf16
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
        __syncthreads();  // the value tile is complete
#pragma unroll
        for (int t = 0; t < kDTiles; t++) {
            // A = V^T: dim 16 t + r16, positions 4 g .. 4 g + 3 and 16 + 4 g .. + 3
            const uint16_t *vr = s_vt + (16 * t + r16) * kVtStride;
            const uint2 v0 = *reinterpret_cast<const uint2 *>(vr + 4 * g);
            const uint2 v1 = *reinterpret_cast<const uint2 *>(vr + 16 + 4 * g);
            const bf16x8 va = as_bf16x8(make_uint4(v0.x, v0.y, v1.x, v1.y));
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi, acc[t], 0, 0, 0);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, plo, acc[t], 0, 0, 0);
        }
        __syncthreads();  // before the next step rewrites the tile
    }

    // ---- partial results: O^T D registers hold dims 16 t + 4 g + i of head r16
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
    const int head = hg * kGroupHeads + r16;
    const int64_t item = static_cast<int64_t>(block) * a.num_q_heads + head;
    float *pa = a.part_acc + item * kVDim;
#pragma unroll
    for (int t = 0; t < kDTiles; t++)
        *reinterpret_cast<float4 *>(pa + 16 * t + 4 * g) =
            make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
    if (g == 0) {
        a.part_ml[2 * item] = m_run;
        a.part_ml[2 * item + 1] = l_run;
    }
}

// out[r][j][d] = sum_b acc_b[d] e^{m_b - M} / sum_b l_b e^{m_b - M} over the
// request's blocks, in order, 256 at a time; a thread owns two dims.
__global__ void __launch_bounds__(kCombineThreads) mla_combine_kernel(const MlaArgs a) {
    __shared__ float s_f[kCombineThreads];
    __shared__ float s_lf[kCombineThreads];
    __shared__ float s_red[kCombineThreads / 64];
    const int r = blockIdx.x;
    const int j = blockIdx.y;
    const int d = threadIdx.x;
    const int b0 = a.req_block0[r], b1 = a.req_block0[r + 1];
    const int64_t hq = a.num_q_heads;
    float M = -INFINITY;
    for (int b = b0 + d; b < b1; b += kCombineThreads) M = fmaxf(M, a.part_ml[(b * hq + j) * 2]);
    for (int x = 1; x < 64; x <<= 1) M = fmaxf(M, __shfl_xor(M, x, 64));
    if ((d & 63) == 0) s_red[d >> 6] = M;
    __syncthreads();
    M = s_red[0];
#pragma unroll
    for (int w = 1; w < kCombineThreads / 64; w++) M = fmaxf(M, s_red[w]);
    float L = 0.f, O0 = 0.f, O1 = 0.f;
    for (int base = b0; base < b1; base += kCombineThreads) {
        const int nb = min(kCombineThreads, b1 - base);
        __syncthreads();
        if (d < nb) {
            const float *ml = a.part_ml + ((base + d) * hq + j) * 2;
            const float f = __expf(ml[0] - M);
            s_f[d] = f;
            s_lf[d] = ml[1] * f;
        }
        __syncthreads();
        for (int i = 0; i < nb; i++) L += s_lf[i];
        const float *acc = a.part_acc + (base * hq + j) * kVDim + d;
#pragma unroll 4
        for (int i = 0; i < nb; i++) {
            O0 += acc[i * hq * kVDim] * s_f[i];
            O1 += acc[i * hq * kVDim + kCombineThreads] * s_f[i];
        }
    }
    float *o = a.out + r * a.o_req + j * a.o_head;
    o[d] = O0 / L;
    o[d + kCombineThreads] = O1 / L;
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
    const size_t need = p.ablocks.size() * static_cast<size_t>(args->num_q_heads) *
                        (static_cast<size_t>(kVDim) + 2) * sizeof(float);
    {
        std::lock_guard<std::mutex> lock(plan->mu);
        if (plan->work_bytes < need) {
            if (plan->d_work) {
                hipError_t e = hipDeviceSynchronize();  // earlier calls may use it
                if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
                (void)hipFree(plan->d_work);
                plan->d_work = nullptr;
                plan->work_bytes = 0;
            }
            hipError_t e = hipMalloc(&plan->d_work, need);
            if (e != hipSuccess) {
                plan->d_work = nullptr;
                return hip_fail(e, "hipMalloc (attention workspace)");
            }
            plan->work_bytes = need;
        }
    }
    const uint8_t *dm = static_cast<const uint8_t *>(plan->d_mem);
    MlaArgs a{};
    a.tiles = reinterpret_cast<const AttnTile *>(dm + plan->staged.off_atiles);
    a.blocks = reinterpret_cast<const AttnBlock *>(dm + plan->staged.off_ablocks);
    a.req_block0 = reinterpret_cast<const int32_t *>(dm + plan->staged.off_rblock);
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
    const size_t acc_elems = p.ablocks.size() * static_cast<size_t>(args->num_q_heads) * kVDim;
    a.part_acc = static_cast<float *>(plan->d_work);
    a.part_ml = static_cast<float *>(plan->d_work) + acc_elems;
    a.n_blocks = static_cast<int32_t>(p.ablocks.size());
    a.n_groups = args->num_q_heads / kGroupHeads;
    a.num_q_heads = args->num_q_heads;
    a.scale = args->scale;
    a.sink_tokens = args->sink_tokens;
    a.sink_bias = args->sink_bias;
    // blocks rounded up to a multiple of the 8 XCDs, times the head groups
    const unsigned grid = static_cast<unsigned>((a.n_blocks + 7) / 8 * 8) *
                          static_cast<unsigned>(a.n_groups);
    if (p.style == PIC_ROPE_HALF)
        hipLaunchKernelGGL(mla_block_kernel<PIC_ROPE_HALF>, dim3(grid), dim3(64), 0, stream, a,
                           args->layer);
    else
        hipLaunchKernelGGL(mla_block_kernel<PIC_ROPE_INTERLEAVED>, dim3(grid), dim3(64), 0, stream,
                           a, args->layer);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "latent attention kernel launch");
    hipLaunchKernelGGL(mla_combine_kernel,
                       dim3(static_cast<unsigned>(p.context.size()),
                            static_cast<unsigned>(args->num_q_heads)),
                       dim3(kCombineThreads), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "latent attention combine launch");
    return PIC_OK;
}
