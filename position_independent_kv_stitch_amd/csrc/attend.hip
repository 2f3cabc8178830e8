// attend.hip -- decode attention over stitched requests without writing the
// stitched cache: the chunk keys' delta-rotation is done while they are
// loaded (Irminsul: MLA-Native Position-Independent Caching for Agentic LLM
// Serving, Technical Summary sections 2.2 and 4), with the EPIC Guide's
// LegoLink pseudo-sink damping as an optional logit bias on the first
// tokens of every chunk placed after position 0 (EPIC Guide: Position-
// Independent Caching for LLM Serving, "1. Identifying and Neutralizing
// Pseudo-Sinks" and its listing).
//
// Two kernels:
//   attend_block_kernel: one workgroup per (256-position block of a request,
//     KV head).  Pass 1 reads every key row of the block once (pool rows of
//     placed chunks turned by the chunk's shift on load; other positions from
//     the request's own cache), scores it against the GQA group's query
//     heads and keeps the logits in LDS; the block's softmax max and sum are
//     taken in LDS; pass 2 reads every value row once and accumulates the
//     weighted sum.  Partial (max, sum, accumulator) per (block, query head)
//     go to the plan's workspace.
//   attend_combine_kernel: one workgroup per (request, query head) merges
//     the request's blocks (flash-decoding style rescaling).
// A token's head row is split over LPT lanes, 16 bytes each; a wave step
// takes 64 / LPT tokens.  Arithmetic is fp32 (the rotation with fp32
// cos/sin rounded from the plan's fp64 tables).  Decode attention reads
// each K and V row once, so it is HBM-bound like the stitch.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "pic_internal.hpp"

namespace pic {

pic_status hip_fail(hipError_t e, const char *what);  // stitch.hip

namespace {

constexpr int kAttnThreads = 256;  // four wave64s
constexpr int kMaxDim = 256;       // head dims supported by the workspace layout

struct AttnArgs {
    const AttnTile *tiles;
    const AttnBlock *blocks;
    const int32_t *req_block0;
    const double *cs;
    const void *pool_k, *pool_v, *cache_k, *cache_v;
    int64_t s_layer, s_tok, s_head, s_page;          // pool view
    int64_t c_layer, c_tok, c_head, c_page, c_req;   // cache view
    const void *q;
    int64_t q_req, q_head;
    float *out;
    int64_t o_req, o_head;
    float *part_acc;  // [block][q head][row_dim]
    float *part_ml;   // [block][q head][2]
    int32_t n_kv_heads, group, row_dim, rope_offset, half_r, lpt_shift;
    int32_t num_q_heads;
    float scale;
    int32_t sink_tokens;
    float sink_bias;
};

template <typename E>
struct Elems;
template <>
struct Elems<float> {
    static constexpr int kVec = 4;
    __device__ static void widen(const uint4 &w, float (&x)[4]) {
        x[0] = __uint_as_float(w.x);
        x[1] = __uint_as_float(w.y);
        x[2] = __uint_as_float(w.z);
        x[3] = __uint_as_float(w.w);
    }
};
template <>
struct Elems<uint16_t> {
    static constexpr int kVec = 8;
    __device__ static void widen(const uint4 &w, float (&x)[8]) {
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; k++) {
            x[2 * k] = __uint_as_float(u[k] << 16);
            x[2 * k + 1] = __uint_as_float(u[k] & 0xFFFF0000u);
        }
    }
};

__device__ __forceinline__ uint4 load16(const void *base, int64_t elem, int esize) {
    return *reinterpret_cast<const uint4 *>(static_cast<const char *>(base) + elem * esize);
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// Element offset of the row of position `t` of a tile, at one layer.
__device__ __forceinline__ int64_t row_base(const AttnArgs &a, const AttnTile &T, int64_t layer,
                                            bool &from_pool) {
    switch (T.kind) {
        case kPoolRows:
            from_pool = true;
            return layer * a.s_layer + T.a * a.s_tok;
        case kPoolPages:
            from_pool = true;
            return layer * a.s_layer + T.a * a.s_page + static_cast<int64_t>(T.b) * a.s_tok;
        case kCacheRows:
            from_pool = false;
            return layer * a.c_layer + T.a * a.c_req + static_cast<int64_t>(T.b) * a.c_tok;
        default:
            from_pool = false;
            return layer * a.c_layer + T.a * a.c_page + static_cast<int64_t>(T.b) * a.c_tok;
    }
}

template <typename E, int STYLE, int GMAX>
__global__ void __launch_bounds__(kAttnThreads) attend_block_kernel(const AttnArgs a, int32_t layer) {
    constexpr int VEC = Elems<E>::kVec;
    constexpr int ES = sizeof(E);
    constexpr int kWaves = kAttnThreads / 64;
    __shared__ float s_w[kAttnBlockTokens * GMAX];   // logits, then weights
    __shared__ float s_acc[kWaves * GMAX * kMaxDim];  // per-wave accumulators
    __shared__ float s_ml[2 * GMAX];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int LPT = 1 << a.lpt_shift;      // lanes per token row
    const int TPW = 64 >> a.lpt_shift;     // tokens per wave step
    const int lj = lane & (LPT - 1);       // this lane's 16-byte piece of the row
    const int tg = lane >> a.lpt_shift;    // this lane's token in the step
    const int G = a.group;
    const int block = blockIdx.x / a.n_kv_heads;
    const int h = blockIdx.x - block * a.n_kv_heads;
    const AttnBlock B = a.blocks[block];
    const int d0 = lj * VEC;                // first dim of this lane's piece

    // this lane's piece of each query head of the group
    float q[GMAX][VEC];
#pragma unroll
    for (int g = 0; g < GMAX; g++) {
        if (g < G) {
            const int64_t qo = B.request * a.q_req + (h * G + g) * a.q_head + d0;
            Elems<E>::widen(load16(a.q, qo, ES), q[g]);
        } else {
#pragma unroll
            for (int e = 0; e < VEC; e++) q[g][e] = 0.f;
        }
    }

    // where this lane's piece sits in the rotary slice
    const int ro = a.rope_offset, hr = a.half_r;
    int role = 0;  // 0: not rotary, 1: x of (half) planes, 2: y of (half) planes, 3: interleaved
    int plane0 = 0, partner = lane;
    if (d0 >= ro && d0 < ro + 2 * hr) {
        if (STYLE == PIC_ROPE_HALF) {
            if (d0 < ro + hr) {
                role = 1;
                plane0 = d0 - ro;
                partner = lane + hr / VEC;
            } else {
                role = 2;
                plane0 = d0 - ro - hr;
                partner = lane - hr / VEC;
            }
        } else {
            role = 3;
            plane0 = (d0 - ro) / 2;
        }
    }
    constexpr int NCS = STYLE == PIC_ROPE_HALF ? VEC : VEC / 2;
    float c[NCS], s[NCS];
    int cur = -2;

    // ---- pass 1: logits
    int tok0 = 0;  // block position of the tile's first token
    for (int ti = 0; ti < B.ntiles; ti++) {
        const AttnTile T = a.tiles[B.tile0 + ti];
        bool from_pool;
        const int64_t base = row_base(a, T, layer, from_pool);
        const void *kbase = from_pool ? a.pool_k : a.cache_k;
        const int64_t tstride = from_pool ? a.s_tok : a.c_tok;
        const int64_t hstride = from_pool ? a.s_head : a.c_head;
        const bool turn = from_pool && T.cs_idx >= 0;
        if (turn && T.cs_idx != cur) {
            cur = T.cs_idx;
            if (role) {
                const double *t = a.cs + (static_cast<int64_t>(cur) * hr + plane0) * 2;
#pragma unroll
                for (int p = 0; p < NCS; p++) {
                    c[p] = static_cast<float>(t[2 * p]);
                    s[p] = static_cast<float>(t[2 * p + 1]);
                }
            }
        }
        for (int t0 = wave * TPW; t0 < T.ntok; t0 += kWaves * TPW) {
            const int t = t0 + tg;
            const bool live = t < T.ntok;
            uint4 w = make_uint4(0u, 0u, 0u, 0u);
            if (live) w = load16(kbase, base + t * tstride + h * hstride + d0, ES);
            float k[VEC];
            Elems<E>::widen(w, k);
            if (turn) {
                if (STYLE == PIC_ROPE_HALF) {
                    float o[VEC];
#pragma unroll
                    for (int e = 0; e < VEC; e++) o[e] = __shfl(k[e], partner, 64);
                    if (role == 1) {
#pragma unroll
                        for (int e = 0; e < VEC; e++) k[e] = k[e] * c[e] - o[e] * s[e];
                    } else if (role == 2) {
#pragma unroll
                        for (int e = 0; e < VEC; e++) k[e] = o[e] * s[e] + k[e] * c[e];
                    }
                } else if (role == 3) {
#pragma unroll
                    for (int e = 0; e < VEC / 2; e++) {
                        const float x = k[2 * e], y = k[2 * e + 1];
                        k[2 * e] = x * c[e] - y * s[e];
                        k[2 * e + 1] = x * s[e] + y * c[e];
                    }
                }
            }
            float dot[GMAX];
#pragma unroll
            for (int g = 0; g < GMAX; g++) {
                float acc = 0.f;
#pragma unroll
                for (int e = 0; e < VEC; e++) acc += q[g][e] * k[e];
                dot[g] = acc;
            }
            for (int m = 1; m < LPT; m <<= 1) {
#pragma unroll
                for (int g = 0; g < GMAX; g++) dot[g] += shfl_xor_f(dot[g], m);
            }
            if (live && lj == 0) {
                const int dist = T.sink_dist + t;
                const float bias = (dist < a.sink_tokens) ? a.sink_bias : 0.f;
#pragma unroll
                for (int g = 0; g < GMAX; g++)
                    if (g < G) s_w[(tok0 + t) * GMAX + g] = dot[g] * a.scale + bias;
            }
        }
        tok0 += T.ntok;
    }
    __syncthreads();

    // ---- block softmax: max and sum per query head
    for (int g = wave; g < G; g += kWaves) {
        float m = -INFINITY;
        for (int i = lane; i < B.ntok; i += 64) m = fmaxf(m, s_w[i * GMAX + g]);
        for (int x = 1; x < 64; x <<= 1) m = fmaxf(m, shfl_xor_f(m, x));
        float l = 0.f;
        for (int i = lane; i < B.ntok; i += 64) {
            const float p = __expf(s_w[i * GMAX + g] - m);
            s_w[i * GMAX + g] = p;
            l += p;
        }
        for (int x = 1; x < 64; x <<= 1) l += shfl_xor_f(l, x);
        if (lane == 0) {
            s_ml[2 * g] = m;
            s_ml[2 * g + 1] = l;
        }
    }
    __syncthreads();

    // ---- pass 2: weighted values
    float acc[GMAX][VEC];
#pragma unroll
    for (int g = 0; g < GMAX; g++)
#pragma unroll
        for (int e = 0; e < VEC; e++) acc[g][e] = 0.f;
    tok0 = 0;
    for (int ti = 0; ti < B.ntiles; ti++) {
        const AttnTile T = a.tiles[B.tile0 + ti];
        bool from_pool;
        const int64_t base = row_base(a, T, layer, from_pool);
        const void *vbase = from_pool ? a.pool_v : a.cache_v;
        const int64_t tstride = from_pool ? a.s_tok : a.c_tok;
        const int64_t hstride = from_pool ? a.s_head : a.c_head;
        for (int t0 = wave * TPW; t0 < T.ntok; t0 += kWaves * TPW) {
            const int t = t0 + tg;
            if (t < T.ntok) {
                float v[VEC];
                Elems<E>::widen(load16(vbase, base + t * tstride + h * hstride + d0, ES), v);
#pragma unroll
                for (int g = 0; g < GMAX; g++) {
                    if (g < G) {
                        const float p = s_w[(tok0 + t) * GMAX + g];
#pragma unroll
                        for (int e = 0; e < VEC; e++) acc[g][e] += p * v[e];
                    }
                }
            }
        }
        tok0 += T.ntok;
    }
    // sum the wave's token groups, then the waves
    for (int m = LPT; m < 64; m <<= 1) {
#pragma unroll
        for (int g = 0; g < GMAX; g++)
#pragma unroll
            for (int e = 0; e < VEC; e++) acc[g][e] += shfl_xor_f(acc[g][e], m);
    }
    if (tg == 0) {
#pragma unroll
        for (int g = 0; g < GMAX; g++)
            if (g < G)
#pragma unroll
                for (int e = 0; e < VEC; e++) s_acc[(wave * GMAX + g) * kMaxDim + d0 + e] = acc[g][e];
    }
    __syncthreads();
    const int D = a.row_dim;
    for (int idx = threadIdx.x; idx < G * D; idx += kAttnThreads) {
        const int g = idx / D, d = idx - g * D;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; w++) sum += s_acc[(w * GMAX + g) * kMaxDim + d];
        a.part_acc[(static_cast<int64_t>(block) * a.num_q_heads + h * G + g) * D + d] = sum;
    }
    if (threadIdx.x < G) {
        const int g = threadIdx.x;
        float *ml = a.part_ml + (static_cast<int64_t>(block) * a.num_q_heads + h * G + g) * 2;
        ml[0] = s_ml[2 * g];
        ml[1] = s_ml[2 * g + 1];
    }
}

// out[r][j][d] = sum_b acc_b[d] e^{m_b - M} / sum_b l_b e^{m_b - M}
__global__ void __launch_bounds__(kMaxDim) attend_combine_kernel(const AttnArgs a) {
    const int r = blockIdx.x;
    const int j = blockIdx.y;
    const int d = threadIdx.x;
    const int b0 = a.req_block0[r], b1 = a.req_block0[r + 1];
    float M = -INFINITY;
    for (int b = b0; b < b1; b++)
        M = fmaxf(M, a.part_ml[(static_cast<int64_t>(b) * a.num_q_heads + j) * 2]);
    float L = 0.f, O = 0.f;
    for (int b = b0; b < b1; b++) {
        const float *ml = a.part_ml + (static_cast<int64_t>(b) * a.num_q_heads + j) * 2;
        const float f = __expf(ml[0] - M);
        L += ml[1] * f;
        if (d < a.row_dim)
            O += a.part_acc[(static_cast<int64_t>(b) * a.num_q_heads + j) * a.row_dim + d] * f;
    }
    if (d < a.row_dim) a.out[r * a.o_req + j * a.o_head + d] = O / L;
}

template <typename E, int STYLE>
hipError_t launch_attend(const AttnArgs &a, int n_blocks, int n_requests, int layer,
                         hipStream_t stream) {
    dim3 grid(static_cast<unsigned>(n_blocks) * static_cast<unsigned>(a.n_kv_heads));
    if (a.group <= 4)
        hipLaunchKernelGGL((attend_block_kernel<E, STYLE, 4>), grid, dim3(kAttnThreads), 0, stream,
                           a, layer);
    else
        hipLaunchKernelGGL((attend_block_kernel<E, STYLE, 8>), grid, dim3(kAttnThreads), 0, stream,
                           a, layer);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attend_combine_kernel, dim3(static_cast<unsigned>(n_requests),
                                                   static_cast<unsigned>(a.num_q_heads)),
                       dim3(kMaxDim), 0, stream, a);
    return hipGetLastError();
}

}  // namespace
}  // namespace pic

extern "C" pic_status pic_attend(pic_plan_t *plan, const pic_kv_view *pool,
                                 const pic_kv_view *cache, const pic_attend_args *args,
                                 void *stream_) {
    using namespace pic;
    clear_error();
    if (!plan || plan->magic != kPlanMagic) return fail(PIC_ERR_STATE, "invalid or destroyed plan");
    const Problem &p = plan->prob;
    if (!args || !args->q || !args->out)
        return fail(PIC_ERR_INVALID_ARG, "attend arguments, q and out must not be NULL");
    if (p.mode == kInPlace) return fail(PIC_ERR_STATE, "in-place plans have no attention map");
    if (!p.shape.has_v) return fail(PIC_ERR_INVALID_ARG, "pic_attend needs K and V rows (has_v)");
    const int H = p.shape.num_heads, D = p.shape.row_dim;
    if (args->num_q_heads < H || args->num_q_heads % H != 0 || args->num_q_heads / H > 8)
        return fail(PIC_ERR_INVALID_ARG, "num_q_heads %d: need a multiple of %d, at most 8x",
                    args->num_q_heads, H);
    if (args->layer < 0 || args->layer >= p.shape.num_layers)
        return fail(PIC_ERR_INVALID_ARG, "layer %d outside [0, %d)", args->layer,
                    p.shape.num_layers);
    const int vec = p.u.vec;
    const int lpt = D / vec;
    if (D > kMaxDim || lpt > 64 || (lpt & (lpt - 1)) != 0)
        return fail(PIC_ERR_ALIGN, "pic_attend needs row_dim / %d a power of two, row_dim <= %d",
                    vec, kMaxDim);
    if (args->q_request_stride % vec || args->q_head_stride % vec ||
        (reinterpret_cast<uintptr_t>(args->q) & 15u))
        return fail(PIC_ERR_ALIGN, "q rows must be 16-byte aligned");
    if (args->sink_tokens < 0) return fail(PIC_ERR_INVALID_ARG, "negative sink_tokens");
    pic_status st = check_view(pool, vec, true, "pool");
    if (st) return st;
    st = check_view(cache, vec, true, "cache");
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
                        (static_cast<size_t>(D) + 2) * sizeof(float);
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
    AttnArgs a{};
    a.tiles = reinterpret_cast<const AttnTile *>(dm + plan->staged.off_atiles);
    a.blocks = reinterpret_cast<const AttnBlock *>(dm + plan->staged.off_ablocks);
    a.req_block0 = reinterpret_cast<const int32_t *>(dm + plan->staged.off_rblock);
    a.cs = reinterpret_cast<const double *>(dm + plan->staged.off_cs);
    a.pool_k = pool->k;
    a.pool_v = pool->v;
    a.cache_k = cache->k;
    a.cache_v = cache->v;
    a.s_layer = pool->layer_stride;
    a.s_tok = pool->token_stride;
    a.s_head = pool->head_stride;
    a.s_page = pool->page_stride;
    a.c_layer = cache->layer_stride;
    a.c_tok = cache->token_stride;
    a.c_head = cache->head_stride;
    a.c_page = cache->page_stride;
    a.c_req = cache->request_stride;
    a.q = args->q;
    a.q_req = args->q_request_stride;
    a.q_head = args->q_head_stride;
    a.out = args->out;
    a.o_req = args->out_request_stride;
    a.o_head = args->out_head_stride;
    const size_t acc_elems = p.ablocks.size() * static_cast<size_t>(args->num_q_heads) * D;
    a.part_acc = static_cast<float *>(plan->d_work);
    a.part_ml = static_cast<float *>(plan->d_work) + acc_elems;
    a.n_kv_heads = H;
    a.group = args->num_q_heads / H;
    a.row_dim = D;
    a.rope_offset = p.shape.rope_offset;
    a.half_r = p.u.half_r;
    a.lpt_shift = 0;
    while ((1 << a.lpt_shift) < lpt) a.lpt_shift++;
    a.num_q_heads = args->num_q_heads;
    a.scale = args->scale;
    a.sink_tokens = args->sink_tokens;
    a.sink_bias = args->sink_bias;
    const int nb = static_cast<int>(p.ablocks.size());
    const int nr = static_cast<int>(p.context.size());
    hipError_t e;
    if (p.shape.dtype == PIC_DTYPE_F32)
        e = p.style == PIC_ROPE_HALF ? launch_attend<float, PIC_ROPE_HALF>(a, nb, nr, args->layer, stream)
                                     : launch_attend<float, PIC_ROPE_INTERLEAVED>(a, nb, nr, args->layer, stream);
    else
        e = p.style == PIC_ROPE_HALF ? launch_attend<uint16_t, PIC_ROPE_HALF>(a, nb, nr, args->layer, stream)
                                     : launch_attend<uint16_t, PIC_ROPE_INTERLEAVED>(a, nb, nr, args->layer, stream);
    if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
    return PIC_OK;
}
