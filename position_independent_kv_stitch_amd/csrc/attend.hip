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
//   attend_block_kernel: one workgroup per (block of at most 256 positions
//     of a request, KV head).  The block's rows are first resolved into an
//     LDS table (element offset and source per position), so both passes
//     run one flat loop over positions whatever the mix of pool rows, pool
//     pages and cache pages.  Pass 1 reads every key row once (pool rows of
//     placed chunks turned by the chunk's shift on load), scores it against
//     the GQA group's query heads and keeps the logits in LDS; the block's
//     softmax max and sum are taken in LDS; pass 2 reads every value row
//     once and accumulates the weighted sum.  Partial (max, sum,
//     accumulator) per (block, query head) go to the plan's workspace.
//   attend_combine_kernel: one workgroup per (request, query head) merges
//     the request's blocks (flash-decoding style rescaling).
// Lanes: a token's head row is split over LPT = row_dim / (16 / element
// size) lanes; a wave step covers 64 / LPT tokens.  For keys a lane holds
// two 8-byte pieces chosen so that, with half pairing, the x and y halves
// of its planes are both in the lane (the rotation needs no lane exchange).
// Arithmetic is fp32 (the rotation with cos/sin rounded from the plan's
// fp64 tables).  Decode attention reads each K and V row once, so it is
// HBM-bound like the stitch.

#include <hip/hip_runtime.h>

#include <cstring>

#include <algorithm>
#include <cstdint>

#include "pic_internal.hpp"

namespace pic {

pic_status hip_fail(hipError_t e, const char *what);  // stitch.hip
pic_status attend_gqa(struct ::pic_plan *plan, const pic_kv_view *pool, const pic_kv_view *cache,
                      const pic_attend_args *args, hipStream_t stream);  // attend_gqa.hip

namespace {

constexpr int kAttnThreads = 256;  // four wave64s
constexpr int kWaves = kAttnThreads / 64;
constexpr int kMaxDim = 256;  // head dims supported by the LDS layout
#ifndef PIC_ATTN_UNROLL
#define PIC_ATTN_UNROLL 4
#endif
#ifndef PIC_ATTN_UNROLL_V
#define PIC_ATTN_UNROLL_V PIC_ATTN_UNROLL
#endif
// wave steps whose loads are issued together (keys, values)
constexpr int kUnroll = PIC_ATTN_UNROLL;
constexpr int kUnrollV = PIC_ATTN_UNROLL_V;
#ifndef PIC_ATTN_PIPE
#define PIC_ATTN_PIPE 0
#endif
constexpr bool kPipe = PIC_ATTN_PIPE != 0;  // next batch's loads issued before this one is used

// Per-position flags of the block's row table.
constexpr uint32_t kMetaPool = 1u << 31;      // row read from the pool (else the cache)
constexpr uint32_t kMetaDamp = 1u << 30;      // LegoLink bias applies
constexpr uint32_t kMetaCs = (1u << 30) - 1;  // shift table + 1 (0: row not turned)

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

// Element i of packed 32-bit words, widened to fp32.
template <typename E>
struct Elems;
template <>
struct Elems<float> {
    static constexpr int kVec = 4;  // elements per 16 bytes
    __device__ static float get(const uint32_t *w, int i) { return __uint_as_float(w[i]); }
};
template <>
struct Elems<uint16_t> {
    static constexpr int kVec = 8;
    __device__ static float get(const uint32_t *w, int i) {
        return __uint_as_float((i & 1) ? (w[i >> 1] & 0xFFFF0000u) : (w[i >> 1] << 16));
    }
};

__device__ __forceinline__ void load8(const void *base, int64_t elem, int esize, uint32_t (&w)[2]) {
    const uint2 v =
        *reinterpret_cast<const uint2 *>(static_cast<const char *>(base) + elem * esize);
    w[0] = v.x;
    w[1] = v.y;
}

__device__ __forceinline__ void load16(const void *base, int64_t elem, int esize,
                                       uint32_t (&w)[4]) {
    const uint4 v =
        *reinterpret_cast<const uint4 *>(static_cast<const char *>(base) + elem * esize);
    w[0] = v.x;
    w[1] = v.y;
    w[2] = v.z;
    w[3] = v.w;
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

template <int N>
struct Log2 {
    static constexpr int value = 1 + Log2<N / 2>::value;
};
template <>
struct Log2<1> {
    static constexpr int value = 0;
};

template <typename E, int STYLE, int GMAX>
__global__ void __launch_bounds__(kAttnThreads) attend_block_kernel(const AttnArgs a, int32_t layer) {
    constexpr int VEC = Elems<E>::kVec;
    constexpr int HV = VEC / 2;  // elements of one 8-byte piece
    constexpr int ES = sizeof(E);
    constexpr int NH = Log2<GMAX>::value;
    __shared__ AttnTile s_tiles[kAttnBlockTiles];
    __shared__ int64_t s_off[kAttnBlockTokens];
    __shared__ uint32_t s_meta[kAttnBlockTokens];
    // logits, then weights; after pass 2 the cross-wave sums
    __shared__ __attribute__((aligned(16))) float s_w[kAttnBlockTokens * GMAX];
    __shared__ float s_ml[2 * GMAX];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int LPT = 1 << a.lpt_shift;   // lanes per token row
    const int TPW = 64 >> a.lpt_shift;  // tokens per wave step
    const int lj = lane & (LPT - 1);
    const int tg = lane >> a.lpt_shift;
    const int G = a.group;
    const int block = blockIdx.x / a.n_kv_heads;
    const int h = blockIdx.x - block * a.n_kv_heads;
    const AttnBlock B = a.blocks[block];

    // ---- the block's row table
    if (threadIdx.x < B.ntiles) s_tiles[threadIdx.x] = a.tiles[B.tile0 + threadIdx.x];
    __syncthreads();
    for (int pi = threadIdx.x; pi < B.ntok; pi += kAttnThreads) {
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
                off = L * a.s_layer + (T.a + t) * a.s_tok + h * a.s_head;
                meta = kMetaPool;
                break;
            case kPoolPages:
                off = L * a.s_layer + T.a * a.s_page + static_cast<int64_t>(T.b + t) * a.s_tok +
                      h * a.s_head;
                meta = kMetaPool;
                break;
            case kCacheRows:
                off = L * a.c_layer + T.a * a.c_req + static_cast<int64_t>(T.b + t) * a.c_tok +
                      h * a.c_head;
                break;
            default:
                off = L * a.c_layer + T.a * a.c_page + static_cast<int64_t>(T.b + t) * a.c_tok +
                      h * a.c_head;
                break;
        }
        if (T.cs_idx >= 0) meta |= static_cast<uint32_t>(T.cs_idx + 1);
        if (T.sink_dist + t < a.sink_tokens) meta |= kMetaDamp;
        s_off[pi] = off;
        s_meta[pi] = meta;
    }

    // ---- this lane's two key pieces: first elements e0, e1 of the head row
    const int ro = a.rope_offset, hr = a.half_r;
    int e0, e1, plane0 = 0;
    bool rot = false;
    if (STYLE == PIC_ROPE_HALF) {
        const int nrl = hr / HV;  // lanes holding rotary planes
        if (lj < nrl) {
            rot = true;
            plane0 = lj * HV;
            e0 = ro + plane0;  // x of planes plane0 .. plane0 + HV - 1
            e1 = e0 + hr;      // their y
        } else {
            const int x = (lj - nrl) * VEC;  // index among the non-rotary dims
            e0 = x < ro ? x : x + 2 * hr;
            e1 = e0 + HV;
        }
    } else {
        e0 = lj * VEC;
        e1 = e0 + HV;
        rot = e0 >= ro && e0 < ro + 2 * hr;
        plane0 = (e0 - ro) / 2;
    }
    float q0[GMAX][HV], q1[GMAX][HV];
#pragma unroll
    for (int g = 0; g < GMAX; g++) {
        uint32_t w0[2] = {0u, 0u}, w1[2] = {0u, 0u};
        if (g < G) {
            const int64_t qo = B.request * a.q_req + (h * G + g) * a.q_head;
            load8(a.q, qo + e0, ES, w0);
            load8(a.q, qo + e1, ES, w1);
        }
#pragma unroll
        for (int e = 0; e < HV; e++) {
            q0[g][e] = Elems<E>::get(w0, e);
            q1[g][e] = Elems<E>::get(w1, e);
        }
    }
    __syncthreads();

    const int sub = LPT >> NH;  // lanes that end up holding one head's sum
    const bool writer = (lj & (sub - 1)) == 0;
    const int my_g = lj / sub;
    const int steps = (B.ntok + kWaves * TPW - 1) / (kWaves * TPW);
    uint32_t cur = 0;  // shift table (+1) whose cos/sin sit in c, s
    float c[HV], s[HV];
#pragma unroll
    for (int p = 0; p < HV; p++) c[p] = 1.f, s[p] = 0.f;

    // key loads of kUnroll wave steps starting at step s0
    struct KBatch {
        uint32_t w0[kUnroll][2], w1[kUnroll][2], mt[kUnroll];
    };
    auto issue_k = [&](KBatch &b, int s0) {
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int pi = ((s0 + u) * kWaves + wave) * TPW + tg;
            b.w0[u][0] = b.w0[u][1] = b.w1[u][0] = b.w1[u][1] = 0u;
            b.mt[u] = 0u;
            if (pi < B.ntok) {
                b.mt[u] = s_meta[pi];
                const int64_t off = s_off[pi];
                const void *base = (b.mt[u] & kMetaPool) ? a.pool_k : a.cache_k;
                load8(base, off + e0, ES, b.w0[u]);
                load8(base, off + e1, ES, b.w1[u]);
            }
        }
    };
    auto score = [&](const KBatch &b, int s0) {
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int pi = ((s0 + u) * kWaves + wave) * TPW + tg;
            float k0[HV], k1[HV];
#pragma unroll
            for (int e = 0; e < HV; e++) {
                k0[e] = Elems<E>::get(b.w0[u], e);
                k1[e] = Elems<E>::get(b.w1[u], e);
            }
            const uint32_t cs1 = b.mt[u] & kMetaCs;
            if (rot && cs1 != 0u) {
                if (cs1 != cur) {
                    cur = cs1;
                    const double *t =
                        a.cs + (static_cast<int64_t>(cs1 - 1) * hr + plane0) * 2;
#pragma unroll
                    for (int p = 0; p < HV; p++) {
                        c[p] = static_cast<float>(t[2 * p]);
                        s[p] = static_cast<float>(t[2 * p + 1]);
                    }
                }
                if (STYLE == PIC_ROPE_HALF) {
#pragma unroll
                    for (int p = 0; p < HV; p++) {
                        const float x = k0[p], y = k1[p];
                        k0[p] = x * c[p] - y * s[p];
                        k1[p] = x * s[p] + y * c[p];
                    }
                } else {
#pragma unroll
                    for (int p = 0; p < HV / 2; p++) {
                        float x = k0[2 * p], y = k0[2 * p + 1];
                        k0[2 * p] = x * c[p] - y * s[p];
                        k0[2 * p + 1] = x * s[p] + y * c[p];
                        x = k1[2 * p];
                        y = k1[2 * p + 1];
                        k1[2 * p] = x * c[HV / 2 + p] - y * s[HV / 2 + p];
                        k1[2 * p + 1] = x * s[HV / 2 + p] + y * c[HV / 2 + p];
                    }
                }
            }
            float v[GMAX];
#pragma unroll
            for (int g = 0; g < GMAX; g++) {
                float acc = 0.f;
#pragma unroll
                for (int e = 0; e < HV; e++) acc += q0[g][e] * k0[e] + q1[g][e] * k1[e];
                v[g] = acc;
            }
            // reduce-scatter over the token's lanes: each halving round keeps
            // half of the heads, so lane lj ends with head lj / sub
#pragma unroll
            for (int r = 0; r < NH; r++) {
                const int n = GMAX >> r;
                const int m = LPT >> (r + 1);
                const bool upper = (lane & m) != 0;
#pragma unroll
                for (int i = 0; i < n / 2; i++) {
                    const float send = upper ? v[i] : v[i + n / 2];
                    const float keep = upper ? v[i + n / 2] : v[i];
                    v[i] = keep + shfl_xor_f(send, m);
                }
            }
            for (int m = sub >> 1; m >= 1; m >>= 1) v[0] += shfl_xor_f(v[0], m);
            if (pi < B.ntok && writer && my_g < G)
                s_w[pi * GMAX + my_g] =
                    v[0] * a.scale + ((b.mt[u] & kMetaDamp) ? a.sink_bias : 0.f);
        }
    };

    // value loads of kUnrollV wave steps starting at step s0; this lane's
    // 16-byte piece of the row
    const int dv = lj * VEC;
    struct VBatch {
        uint32_t w[kUnrollV][4];
    };
    auto issue_v = [&](VBatch &b, int s0) {
#pragma unroll
        for (int u = 0; u < kUnrollV; u++) {
            const int pi = ((s0 + u) * kWaves + wave) * TPW + tg;
            b.w[u][0] = b.w[u][1] = b.w[u][2] = b.w[u][3] = 0u;
            if (pi < B.ntok) {
                const void *base = (s_meta[pi] & kMetaPool) ? a.pool_v : a.cache_v;
                load16(base, s_off[pi] + dv, ES, b.w[u]);
            }
        }
    };
    float acc[GMAX][VEC];
#pragma unroll
    for (int g = 0; g < GMAX; g++)
#pragma unroll
        for (int e = 0; e < VEC; e++) acc[g][e] = 0.f;
    auto accumulate = [&](const VBatch &b, int s0) {
#pragma unroll
        for (int u = 0; u < kUnrollV; u++) {
            const int pi = ((s0 + u) * kWaves + wave) * TPW + tg;
            if (pi < B.ntok) {
                float p[GMAX];
#pragma unroll
                for (int g = 0; g < GMAX; g++) p[g] = s_w[pi * GMAX + g];
#pragma unroll
                for (int e = 0; e < VEC; e++) {
                    const float x = Elems<E>::get(b.w[u], e);
#pragma unroll
                    for (int g = 0; g < GMAX; g++) acc[g][e] += p[g] * x;
                }
            }
        }
    };

    // ---- pass 1: logits.  With kPipe the next batch's loads are in flight
    // while the current one is scored.
    {
        KBatch kb;
        issue_k(kb, 0);
        for (int s0 = 0; s0 < steps; s0 += kUnroll) {
            if (kPipe) {
                KBatch next;
                if (s0 + kUnroll < steps) issue_k(next, s0 + kUnroll);
                score(kb, s0);
                kb = next;
            } else {
                score(kb, s0);
                if (s0 + kUnroll < steps) issue_k(kb, s0 + kUnroll);
            }
        }
    }
    // the first values are loaded while the softmax runs
    VBatch vb;
    issue_v(vb, 0);
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
    for (int s0 = 0; s0 < steps; s0 += kUnrollV) {
        if (kPipe) {
            VBatch next;
            if (s0 + kUnrollV < steps) issue_v(next, s0 + kUnrollV);
            accumulate(vb, s0);
            vb = next;
        } else {
            accumulate(vb, s0);
            if (s0 + kUnrollV < steps) issue_v(vb, s0 + kUnrollV);
        }
    }
    // sum the wave's token groups, then the waves in order (wave 0 first)
    for (int m = LPT; m < 64; m <<= 1) {
#pragma unroll
        for (int g = 0; g < GMAX; g++)
#pragma unroll
            for (int e = 0; e < VEC; e++) acc[g][e] += shfl_xor_f(acc[g][e], m);
    }
    const int D = a.row_dim;
    float *s_sum = s_w;  // [g][row_dim]; G * D <= GMAX * kMaxDim fits
    for (int w = 0; w < kWaves; w++) {
        __syncthreads();
        if (wave == w && tg == 0) {
#pragma unroll
            for (int g = 0; g < GMAX; g++)
                if (g < G)
#pragma unroll
                    for (int e = 0; e < VEC; e++) {
                        float *x = s_sum + g * D + dv + e;
                        *x = (w == 0 ? 0.f : *x) + acc[g][e];
                    }
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += kAttnThreads) {
        const int g = idx / D, d = idx - g * D;
        a.part_acc[(static_cast<int64_t>(block) * a.num_q_heads + h * G + g) * D + d] = s_sum[idx];
    }
    if (threadIdx.x < G) {
        const int g = threadIdx.x;
        float *ml = a.part_ml + (static_cast<int64_t>(block) * a.num_q_heads + h * G + g) * 2;
        ml[0] = s_ml[2 * g];
        ml[1] = s_ml[2 * g + 1];
    }
}

// out[r][j][d] = sum_b acc_b[d] e^{m_b - M} / sum_b l_b e^{m_b - M}, the
// blocks taken in order, 256 at a time.
__global__ void __launch_bounds__(kMaxDim) attend_combine_kernel(const AttnArgs a) {
    __shared__ float s_f[kMaxDim];   // e^{m_b - M} of a batch of blocks
    __shared__ float s_lf[kMaxDim];  // l_b e^{m_b - M}
    __shared__ float s_red[kMaxDim / 64];
    const int r = blockIdx.x;
    const int j = blockIdx.y;
    const int d = threadIdx.x;
    const int b0 = a.req_block0[r], b1 = a.req_block0[r + 1];
    const int64_t hq = a.num_q_heads;
    float M = -INFINITY;
    for (int b = b0 + d; b < b1; b += kMaxDim) M = fmaxf(M, a.part_ml[(b * hq + j) * 2]);
    for (int x = 1; x < 64; x <<= 1) M = fmaxf(M, shfl_xor_f(M, x));
    if ((d & 63) == 0) s_red[d >> 6] = M;
    __syncthreads();
    M = s_red[0];
#pragma unroll
    for (int w = 1; w < kMaxDim / 64; w++) M = fmaxf(M, s_red[w]);
    float L = 0.f, O = 0.f;
    for (int base = b0; base < b1; base += kMaxDim) {
        const int nb = min(kMaxDim, b1 - base);
        __syncthreads();
        if (d < nb) {
            const float *ml = a.part_ml + ((base + d) * hq + j) * 2;
            const float f = __expf(ml[0] - M);
            s_f[d] = f;
            s_lf[d] = ml[1] * f;
        }
        __syncthreads();
        for (int i = 0; i < nb; i++) L += s_lf[i];
        if (d < a.row_dim) {
            const float *acc = a.part_acc + (base * hq + j) * a.row_dim + d;
#pragma unroll 8
            for (int i = 0; i < nb; i++) O += acc[i * hq * a.row_dim] * s_f[i];
        }
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
    pic_status st0 = ensure_attention(plan);
    if (st0) return st0;
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
    const int gmax = args->num_q_heads / H <= 4 ? 4 : 8;  // query heads per kernel instance
    if (lpt < gmax)
        return fail(PIC_ERR_ALIGN, "pic_attend needs row_dim >= %d for %d query heads per KV head",
                    gmax * vec, args->num_q_heads / H);
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
    // bf16 128-dim rows: the matrix-core path (attend_gqa.hip)
    if (gqa_tile_path(p, args->num_q_heads / H)) return attend_gqa(plan, pool, cache, args, stream);
    // the map's work blocks, uploaded once per plan
    const DevBlob *blob = nullptr;
    st = plan_blob(plan, blob_key(kBlobAttnMap, 0), stream_, [&](DevBlob &b) {
        auto put = [&](const void *src, size_t n) {
            const size_t at = (b.host.size() + 255) & ~size_t{255};
            b.host.resize(at + n);
            if (n) std::memcpy(b.host.data() + at, src, n);
            return at;
        };
        b.off[0] = put(p.atiles.data(), p.atiles.size() * sizeof(AttnTile));
        b.off[1] = put(p.ablocks.data(), p.ablocks.size() * sizeof(AttnBlock));
        b.off[2] = put(p.req_block0.data(), p.req_block0.size() * sizeof(int32_t));
    }, &blob);
    if (st) return st;
    const size_t need = p.ablocks.size() * static_cast<size_t>(args->num_q_heads) *
                        (static_cast<size_t>(D) + 2) * sizeof(float);
    void *work = nullptr;
    st = call_workspace(plan, need, stream_, &work);
    if (st) return st;
    const uint8_t *dm = static_cast<const uint8_t *>(plan->d_mem);
    const uint8_t *bm = static_cast<const uint8_t *>(blob->dev);
    AttnArgs a{};
    a.tiles = reinterpret_cast<const AttnTile *>(bm + blob->off[0]);
    a.blocks = reinterpret_cast<const AttnBlock *>(bm + blob->off[1]);
    a.req_block0 = reinterpret_cast<const int32_t *>(bm + blob->off[2]);
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
    a.part_acc = static_cast<float *>(work);
    a.part_ml = static_cast<float *>(work) + acc_elems;
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
    return note_use(plan, stream_);
}
