// stitch.hip -- gfx950 kernels and launch code of the stitch library.
//
// One kernel serves the three operations of the path:
//   copy mode, contiguous or paged destination (pic_stitch): every placed
//     token row is read once from the pool and written once to its
//     destination row; the rotary slice of each K head row is turned by the
//     entry's shift, everything else is moved as raw 16-byte words;
//   MLA rows: the same kernel with one head, the 512-dim content latent as
//     copy units and the 64-dim rotary key as rotary units (Irminsul:
//     MLA-Native Position-Independent Caching for Agentic LLM Serving,
//     Technical Summary sections 2.1 and 2.2);
//   in-place mode (pic_rotate_inplace): rotary units only, read and written
//     at the same addresses by the same lane.
//
// The shift itself: a key cached at position n equals R_n k_raw, and the
// key it must become at n + delta is R_{n+delta} k_raw = R_delta (R_n k_raw),
// so every plane i of the cached key's rotary slice is turned by
// delta * theta_i (EPIC Guide: Position-Independent Caching for LLM Serving,
// "Mathematical Foundations", sections 1 and 2).  The pair (x, y) becomes
// (x c - y s, x s + y c) with c, s the cosine and sine of that angle.
//
// Work decomposition (the path is HBM-bound: a few flops per 16 bytes, no
// contraction, so no MFMA): a workgroup of four wave64s takes one tile of up
// to 64 tokens of one entry for one layer; each wave walks the tile's tokens,
// one token row per step.  A token row is split into 16-byte units: rotary
// units (HALF pairing: two 16-byte words, one from each half of the rotary
// slice; INTERLEAVED: one word holding whole pairs), and copy units (the
// non-rotary part of K, and V).  A lane owns the same units for every token,
// so its unit offsets and its planes' cos/sin are computed once per tile and
// kept in registers; all of a step's loads are issued before any store.
// Consecutive lanes cover consecutive 16-byte words of a row, so a wave's
// accesses are fully coalesced (a bf16 GQA token row is 2 KiB of K and
// 2 KiB of V).
//
// Arithmetic: storage values are widened exactly to fp64, the rotation is
// done in fp64 with fp64 cos/sin from the host planner, and the result is
// rounded once to the storage type, to nearest, ties to even.  fp64 is
// full-rate on CDNA vector ALUs and the kernel is memory-bound, so this
// costs no time and keeps the result within one storage rounding of the
// exact rotation.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <memory>

#include "pic_internal.hpp"

namespace pic {
namespace {

// ------------------------------------------------------------ kernel args

struct KArgs {
    const DevTile *tiles;
    const DevEntry *entries;
    const double *cs;
    const int32_t *pages;
    const void *src_k;
    const void *src_v;
    void *dst_k;
    void *dst_v;
    int64_t s_layer, s_tok, s_head;                  // source strides
    int64_t d_layer, d_tok, d_head, d_page, d_req;   // destination strides
    int32_t layer_begin;
    int32_t mode;  // DstMode
    int32_t page_size;
    int32_t page_shift;  // log2(page_size) when a power of two, else -1
    int32_t rope_offset;
    int32_t half_r;
    int32_t nr, uph_shift;  // rotary units
    int32_t nck, cph;       // K copy units
    int32_t nv, vph;        // V units
    int32_t nblk;           // unit blocks per token row
};

constexpr int kHalf = PIC_ROPE_HALF;

// ------------------------------------------------------ storage conversion

// bf16 -> fp32 is a 16-bit shift, exact; fp32 -> fp64 exact.
__device__ __forceinline__ double bf16_lo(uint32_t w) {
    return static_cast<double>(__uint_as_float(w << 16));
}
__device__ __forceinline__ double bf16_hi(uint32_t w) {
    return static_cast<double>(__uint_as_float(w & 0xFFFF0000u));
}

// fp64 -> bf16 with one round-to-nearest-even: first to fp32 with
// round-to-odd (truncate, then set the last bit when inexact), which keeps
// enough information for the final 8-bit rounding to be the correct one,
// then fp32 -> bf16 round-to-nearest-even on the bit pattern.
__device__ __forceinline__ uint32_t f64_to_bf16(double d) {
    const float f = static_cast<float>(d);  // nearest
    uint32_t u = __float_as_uint(f);
    const double back = static_cast<double>(f);
    if (back != d) {
        if (fabs(back) > fabs(d)) u -= 1u;  // step the magnitude down: truncation
        u |= 1u;                            // sticky bit: round-to-odd
    }
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16(double lo, double hi) {
    return f64_to_bf16(lo) | (f64_to_bf16(hi) << 16);
}

// ----------------------------------------------------------------- rotation

template <typename E>
struct Vec;

template <>
struct Vec<float> {
    static constexpr int kElems = 4;
};
template <>
struct Vec<uint16_t> {
    static constexpr int kElems = 8;
};

// HALF pairing: word a holds x of planes p0..p0+VEC-1, word b their y.
__device__ __forceinline__ void rotate_half(uint4 &a, uint4 &b, const double *c, const double *s,
                                            float) {
    double x[4] = {__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z),
                   __uint_as_float(a.w)};
    double y[4] = {__uint_as_float(b.x), __uint_as_float(b.y), __uint_as_float(b.z),
                   __uint_as_float(b.w)};
    float xo[4], yo[4];
#pragma unroll
    for (int e = 0; e < 4; e++) {
        xo[e] = static_cast<float>(x[e] * c[e] - y[e] * s[e]);
        yo[e] = static_cast<float>(x[e] * s[e] + y[e] * c[e]);
    }
    a = make_uint4(__float_as_uint(xo[0]), __float_as_uint(xo[1]), __float_as_uint(xo[2]),
                   __float_as_uint(xo[3]));
    b = make_uint4(__float_as_uint(yo[0]), __float_as_uint(yo[1]), __float_as_uint(yo[2]),
                   __float_as_uint(yo[3]));
}

__device__ __forceinline__ void rotate_half(uint4 &a, uint4 &b, const double *c, const double *s,
                                            uint16_t) {
    uint32_t aw[4] = {a.x, a.y, a.z, a.w};
    uint32_t bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const double x0 = bf16_lo(aw[k]), x1 = bf16_hi(aw[k]);
        const double y0 = bf16_lo(bw[k]), y1 = bf16_hi(bw[k]);
        const double c0 = c[2 * k], s0 = s[2 * k], c1 = c[2 * k + 1], s1 = s[2 * k + 1];
        aw[k] = pack_bf16(x0 * c0 - y0 * s0, x1 * c1 - y1 * s1);
        bw[k] = pack_bf16(x0 * s0 + y0 * c0, x1 * s1 + y1 * c1);
    }
    a = make_uint4(aw[0], aw[1], aw[2], aw[3]);
    b = make_uint4(bw[0], bw[1], bw[2], bw[3]);
}

// INTERLEAVED pairing: one word holds (x, y) of consecutive planes.
__device__ __forceinline__ void rotate_interleaved(uint4 &a, const double *c, const double *s,
                                                   float) {
    const double x0 = __uint_as_float(a.x), y0 = __uint_as_float(a.y);
    const double x1 = __uint_as_float(a.z), y1 = __uint_as_float(a.w);
    a = make_uint4(__float_as_uint(static_cast<float>(x0 * c[0] - y0 * s[0])),
                   __float_as_uint(static_cast<float>(x0 * s[0] + y0 * c[0])),
                   __float_as_uint(static_cast<float>(x1 * c[1] - y1 * s[1])),
                   __float_as_uint(static_cast<float>(x1 * s[1] + y1 * c[1])));
}

__device__ __forceinline__ void rotate_interleaved(uint4 &a, const double *c, const double *s,
                                                   uint16_t) {
    uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const double x = bf16_lo(w[k]), y = bf16_hi(w[k]);
        w[k] = pack_bf16(x * c[k] - y * s[k], x * s[k] + y * c[k]);
    }
    a = make_uint4(w[0], w[1], w[2], w[3]);
}

#ifndef PIC_NT_LOADS
#define PIC_NT_LOADS 0
#endif
#ifndef PIC_NT_STORES
#define PIC_NT_STORES 0
#endif
#ifndef PIC_TOKENS_PER_STEP
#define PIC_TOKENS_PER_STEP 1
#endif

// 16-byte global accesses; the pool is read once and the destination written
// once per launch, so both may bypass cache retention (non-temporal hints).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld16(const void *base, int64_t elem, int esize) {
    const char *p = static_cast<const char *>(base) + elem * esize;
#if PIC_NT_LOADS
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
#else
    return *reinterpret_cast<const uint4 *>(p);
#endif
}
__device__ __forceinline__ void st16(void *base, int64_t elem, int esize, const uint4 &v) {
    char *p = static_cast<char *>(base) + elem * esize;
#if PIC_NT_STORES
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p));
#else
    *reinterpret_cast<uint4 *>(p) = v;
#endif
}

// --------------------------------------------------------------- the kernel

// MAXR rotary units and MAXC copy units per lane per block of units.
template <typename E, int STYLE, int MAXR, int MAXC>
__global__ void __launch_bounds__(kBlockThreads) stitch_kernel(const KArgs a) {
    constexpr int VEC = Vec<E>::kElems;
    constexpr int ES = sizeof(E);
    constexpr int NCS = STYLE == kHalf ? VEC : VEC / 2;  // planes per rotary unit
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    constexpr int kWaves = kBlockThreads / 64;

    const DevTile tile = a.tiles[blockIdx.x];
    const DevEntry ent = a.entries[tile.entry];
    const int64_t layer = a.layer_begin + static_cast<int64_t>(blockIdx.y);
    const bool turn = ent.cs_idx >= 0;

    // cos/sin of the planes this lane's rotary units cover (uph divides 64,
    // so the plane group is the same for all of the lane's units)
    double c[NCS], s[NCS];
    if (turn) {
        const int j = lane & ((1 << a.uph_shift) - 1);
        const double *t = a.cs + (static_cast<int64_t>(ent.cs_idx) * a.half_r + j * NCS) * 2;
#pragma unroll
        for (int p = 0; p < NCS; p++) {
            c[p] = t[2 * p];
            s[p] = t[2 * p + 1];
        }
    } else {
#pragma unroll
        for (int p = 0; p < NCS; p++) {
            c[p] = 1.0;
            s[p] = 0.0;
        }
    }

    const void *sk = a.src_k;
    const void *sv = a.src_v;
    void *dk = a.dst_k;
    void *dv = a.dst_v;
    const int64_t s_base = layer * a.s_layer;
    const int64_t d_base = layer * a.d_layer;
    const int64_t half_off = STYLE == kHalf ? a.half_r : 0;

    for (int blk = 0; blk < a.nblk; blk++) {
        // this lane's unit offsets inside a source row (rs, cs_) and inside a
        // destination row (rd, cd); heads may be laid out differently
        int64_t rs[MAXR], rd[MAXR];
        bool rv[MAXR];
#pragma unroll
        for (int i = 0; i < MAXR; i++) {
            const int u = blk * 64 * MAXR + lane + 64 * i;
            rv[i] = u < a.nr;
            const int h = u >> a.uph_shift;
            const int j = u & ((1 << a.uph_shift) - 1);
            const int inner = a.rope_offset + j * VEC;
            rs[i] = h * a.s_head + inner;
            rd[i] = h * a.d_head + inner;
        }
        int64_t cs_[MAXC], cd[MAXC];
        bool cv[MAXC], isv[MAXC];
#pragma unroll
        for (int i = 0; i < MAXC; i++) {
            const int u = blk * 64 * MAXC + lane + 64 * i;
            cv[i] = u < a.nck + a.nv;
            isv[i] = u >= a.nck;
            int h, inner;
            if (!isv[i]) {
                h = a.cph ? u / a.cph : 0;
                inner = (u - h * a.cph) * VEC;
                if (inner >= a.rope_offset) inner += 2 * a.half_r;  // skip the rotary slice
            } else {
                const int u2 = u - a.nck;
                h = a.vph ? u2 / a.vph : 0;
                inner = (u2 - h * a.vph) * VEC;
            }
            cs_[i] = h * a.s_head + inner;
            cd[i] = h * a.d_head + inner;
        }

        constexpr int TPS = PIC_TOKENS_PER_STEP;
        const int t_end = tile.tok0 + tile.ntok;
        for (int t0 = tile.tok0 + wave * TPS; t0 < t_end; t0 += kWaves * TPS) {
            int64_t srow[TPS], drow[TPS];
            bool tv[TPS];
#pragma unroll
            for (int q = 0; q < TPS; q++) {
                const int t = t0 + q;
                tv[q] = t < t_end;
                srow[q] = s_base + (ent.src_tok + t) * a.s_tok;
                if (a.mode == kInPlace) {
                    drow[q] = srow[q];
                } else {
                    const int32_t pos = static_cast<int32_t>(ent.dst_pos) + t;
                    if (a.mode == kContiguous) {
                        drow[q] = d_base + ent.request * a.d_req +
                                  static_cast<int64_t>(pos) * a.d_tok;
                    } else {
                        int32_t lp, slot;
                        if (a.page_shift >= 0) {
                            lp = pos >> a.page_shift;
                            slot = pos & (a.page_size - 1);
                        } else {
                            lp = pos / a.page_size;
                            slot = pos - lp * a.page_size;
                        }
                        const int64_t phys = tv[q] ? a.pages[ent.page_base + lp] : 0;
                        drow[q] = d_base + phys * a.d_page + static_cast<int64_t>(slot) * a.d_tok;
                    }
                }
            }

            uint4 A[TPS][MAXR], B[TPS][MAXR], Cw[TPS][MAXC];
#pragma unroll
            for (int q = 0; q < TPS; q++) {
                if (!tv[q]) continue;
#pragma unroll
                for (int i = 0; i < MAXR; i++) {
                    if (rv[i]) {
                        A[q][i] = ld16(sk, srow[q] + rs[i], ES);
                        if (STYLE == kHalf) B[q][i] = ld16(sk, srow[q] + rs[i] + half_off, ES);
                    }
                }
#pragma unroll
                for (int i = 0; i < MAXC; i++)
                    if (cv[i]) Cw[q][i] = ld16(isv[i] ? sv : sk, srow[q] + cs_[i], ES);
            }

#pragma unroll
            for (int q = 0; q < TPS; q++) {
                if (!tv[q]) continue;
#pragma unroll
                for (int i = 0; i < MAXR; i++) {
                    if (rv[i]) {
                        if (STYLE == kHalf) {
                            if (turn) rotate_half(A[q][i], B[q][i], c, s, E{});
                            st16(dk, drow[q] + rd[i], ES, A[q][i]);
                            st16(dk, drow[q] + rd[i] + half_off, ES, B[q][i]);
                        } else {
                            if (turn) rotate_interleaved(A[q][i], c, s, E{});
                            st16(dk, drow[q] + rd[i], ES, A[q][i]);
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < MAXC; i++)
                    if (cv[i]) st16(isv[i] ? dv : dk, drow[q] + cd[i], ES, Cw[q][i]);
            }
        }
    }
}

// ----------------------------------------------------------------- launch

template <typename E, int STYLE>
hipError_t launch_typed(const KArgs &a, int n_tiles, int n_layers, hipStream_t stream) {
    constexpr int MAXR = sizeof(E) == 2 ? 1 : 2;
    constexpr int MAXC = sizeof(E) == 2 ? 2 : 4;
    dim3 grid(static_cast<unsigned>(n_tiles), static_cast<unsigned>(n_layers));
    hipLaunchKernelGGL((stitch_kernel<E, STYLE, MAXR, MAXC>), grid, dim3(kBlockThreads), 0,
                       stream, a);
    return hipGetLastError();
}

int max_rot_units(int dtype) { return dtype == PIC_DTYPE_BF16 ? 1 : 2; }
int max_copy_units(int dtype) { return dtype == PIC_DTYPE_BF16 ? 2 : 4; }

hipError_t launch(const Problem &p, const KArgs &base, int n_layers, hipStream_t stream) {
    KArgs a = base;
    const int n_tiles = static_cast<int>(p.tiles.size());
    const int mr = 64 * max_rot_units(p.shape.dtype);
    const int mc = 64 * max_copy_units(p.shape.dtype);
    const int rb = (p.u.nr + mr - 1) / mr;
    const int cb = (p.u.nck + p.u.nv + mc - 1) / mc;
    a.nblk = rb > cb ? rb : cb;
    if (p.shape.dtype == PIC_DTYPE_F32) {
        return p.style == PIC_ROPE_HALF ? launch_typed<float, PIC_ROPE_HALF>(a, n_tiles, n_layers, stream)
                                        : launch_typed<float, PIC_ROPE_INTERLEAVED>(a, n_tiles, n_layers, stream);
    }
    return p.style == PIC_ROPE_HALF ? launch_typed<uint16_t, PIC_ROPE_HALF>(a, n_tiles, n_layers, stream)
                                    : launch_typed<uint16_t, PIC_ROPE_INTERLEAVED>(a, n_tiles, n_layers, stream);
}

pic_status hip_fail(hipError_t e, const char *what) {
    return fail(PIC_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// Checks of a view against the plan's element size and needs.
pic_status check_view(const pic_kv_view *v, int vec, bool need_v, const char *name) {
    if (!v) return fail(PIC_ERR_INVALID_ARG, "%s view is NULL", name);
    if (!v->k || (need_v && !v->v))
        return fail(PIC_ERR_INVALID_ARG, "%s view: missing K or V pointer", name);
    const int es = 16 / vec;
    auto misaligned = [](const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) != 0; };
    if (misaligned(v->k) || (need_v && misaligned(v->v)))
        return fail(PIC_ERR_ALIGN, "%s view: base pointer not 16-byte aligned", name);
    const int64_t strides[5] = {v->layer_stride, v->token_stride, v->head_stride, v->page_stride,
                                v->request_stride};
    for (int64_t s : strides) {
        if (s < 0) return fail(PIC_ERR_INVALID_ARG, "%s view: negative stride", name);
        if (s % vec)
            return fail(PIC_ERR_ALIGN, "%s view: stride %lld not a multiple of %d elements (%d "
                        "bytes each)", name, static_cast<long long>(s), vec, es);
    }
    return PIC_OK;
}

int page_shift_of(int32_t ps) {
    if (ps <= 0 || (ps & (ps - 1))) return -1;
    int s = 0;
    while ((1 << s) < ps) s++;
    return s;
}

KArgs args_for(const Problem &p, const uint8_t *dmem, const Staged &stg) {
    KArgs a{};
    a.tiles = reinterpret_cast<const DevTile *>(dmem + stg.off_tiles);
    a.entries = reinterpret_cast<const DevEntry *>(dmem + stg.off_entries);
    a.cs = reinterpret_cast<const double *>(dmem + stg.off_cs);
    a.pages = reinterpret_cast<const int32_t *>(dmem + stg.off_pages);
    a.mode = p.mode;
    a.page_size = p.page_size;
    a.page_shift = page_shift_of(p.page_size);
    a.rope_offset = p.shape.rope_offset;
    a.half_r = p.u.half_r;
    a.nr = p.u.nr;
    a.uph_shift = p.u.uph_shift;
    a.nck = p.u.nck;
    a.cph = p.u.cph;
    a.nv = p.u.nv;
    a.vph = p.u.vph;
    return a;
}

struct HostBytes {
    std::vector<uint8_t> bytes;
};

void free_host_bytes(void *p) { delete static_cast<HostBytes *>(p); }

}  // namespace
}  // namespace pic

extern "C" {

pic_status pic_stitch(pic_plan_t *plan, const pic_kv_view *pool, const pic_kv_view *dst,
                      int32_t layer_begin, int32_t layer_end, void *stream_) {
    using namespace pic;
    clear_error();
    if (!plan || plan->magic != kPlanMagic) return fail(PIC_ERR_STATE, "invalid or destroyed plan");
    const Problem &p = plan->prob;
    if (layer_begin < 0 || layer_begin > layer_end || layer_end > p.shape.num_layers)
        return fail(PIC_ERR_INVALID_ARG, "layer range [%d, %d) outside [0, %d)", layer_begin,
                    layer_end, p.shape.num_layers);
    const bool need_v = p.shape.has_v != 0;
    pic_status st = check_view(pool, p.u.vec, need_v, "pool");
    if (st) return st;
    st = check_view(dst, p.u.vec, need_v, "dst");
    if (st) return st;
    if (p.mode == kContiguous && p.n_requests > 1 &&
        dst->request_stride < p.capacity * dst->token_stride)
        return fail(PIC_ERR_OVERLAP, "dst view: request_stride smaller than capacity rows, "
                    "requests would alias");
    if (p.tiles.empty() || layer_begin == layer_end) return PIC_OK;

    hipStream_t stream = static_cast<hipStream_t>(stream_);
    std::lock_guard<std::mutex> lock(plan->mu);
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (!plan->d_mem) {
        const size_t n = plan->staged.bytes.size();
        e = hipMalloc(&plan->d_mem, n);
        if (e != hipSuccess) {
            plan->d_mem = nullptr;
            return hip_fail(e, "hipMalloc (plan metadata)");
        }
        e = hipMemcpyAsync(plan->d_mem, plan->staged.bytes.data(), n, hipMemcpyHostToDevice,
                           stream);
        if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (plan metadata)");
        hipEvent_t ev;
        e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
        if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
        e = hipEventRecord(ev, stream);
        if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
        plan->upload_event = ev;
        plan->device = dev;
    } else {
        if (dev != plan->device)
            return fail(PIC_ERR_STATE, "plan was uploaded to device %d, current device is %d",
                        plan->device, dev);
        e = hipStreamWaitEvent(stream, static_cast<hipEvent_t>(plan->upload_event), 0);
        if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
    }

    KArgs a = args_for(p, static_cast<const uint8_t *>(plan->d_mem), plan->staged);
    a.src_k = pool->k;
    a.src_v = pool->v;
    a.dst_k = dst->k;
    a.dst_v = dst->v;
    a.s_layer = pool->layer_stride;
    a.s_tok = pool->token_stride;
    a.s_head = pool->head_stride;
    a.d_layer = dst->layer_stride;
    a.d_tok = dst->token_stride;
    a.d_head = dst->head_stride;
    a.d_page = dst->page_stride;
    a.d_req = dst->request_stride;
    a.layer_begin = layer_begin;
    e = launch(p, a, layer_end - layer_begin, stream);
    if (e != hipSuccess) return hip_fail(e, "stitch kernel launch");
    return PIC_OK;
}

pic_status pic_rotate_inplace(const pic_kv_shape *shape, const pic_rope_config *rope,
                              const pic_kv_view *buf, int64_t buf_tokens,
                              const pic_segment *segments, int32_t n_segments,
                              int32_t layer_begin, int32_t layer_end, void *stream_) {
    using namespace pic;
    clear_error();
    Problem p;
    pic_status st = build_inplace(shape, rope, buf_tokens, segments, n_segments, &p);
    if (st) return st;
    if (layer_begin < 0 || layer_begin > layer_end || layer_end > p.shape.num_layers)
        return fail(PIC_ERR_INVALID_ARG, "layer range [%d, %d) outside [0, %d)", layer_begin,
                    layer_end, p.shape.num_layers);
    st = check_view(buf, p.u.vec, false, "buf");
    if (st) return st;
    if (p.tiles.empty() || layer_begin == layer_end) return PIC_OK;

    hipStream_t stream = static_cast<hipStream_t>(stream_);
    Staged stg = stage(p);
    auto *host = new (std::nothrow) HostBytes{std::move(stg.bytes)};
    if (!host) return fail(PIC_ERR_NOMEM, "out of host memory");
    void *dmem = nullptr;
    hipError_t e = hipMallocAsync(&dmem, host->bytes.size(), stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();  // clear it
        delete host;
        return hip_fail(e, "hipMallocAsync (segment metadata)");
    }
    e = hipMemcpyAsync(dmem, host->bytes.data(), host->bytes.size(), hipMemcpyHostToDevice,
                       stream);
    if (e != hipSuccess) {
        (void)hipFreeAsync(dmem, stream);
        (void)hipStreamSynchronize(stream);
        delete host;
        return hip_fail(e, "hipMemcpyAsync (segment metadata)");
    }
    // the staging bytes live until the stream has consumed them
    e = hipLaunchHostFunc(stream, free_host_bytes, host);
    if (e != hipSuccess) {
        (void)hipStreamSynchronize(stream);
        delete host;
        (void)hipFreeAsync(dmem, stream);
        return hip_fail(e, "hipLaunchHostFunc");
    }
    KArgs a = args_for(p, static_cast<const uint8_t *>(dmem), stg);
    a.src_k = buf->k;
    a.dst_k = buf->k;
    a.s_layer = a.d_layer = buf->layer_stride;
    a.s_tok = a.d_tok = buf->token_stride;
    a.s_head = a.d_head = buf->head_stride;
    a.layer_begin = layer_begin;
    e = launch(p, a, layer_end - layer_begin, stream);
    hipError_t e2 = hipFreeAsync(dmem, stream);
    if (e != hipSuccess) return hip_fail(e, "rotate kernel launch");
    if (e2 != hipSuccess) return hip_fail(e2, "hipFreeAsync (segment metadata)");
    return PIC_OK;
}

void pic_plan_destroy(pic_plan_t *plan) {
    using namespace pic;
    if (!plan || plan->magic != kPlanMagic) return;
    if (plan->d_mem) {
        int cur = -1;
        (void)hipGetDevice(&cur);
        if (cur != plan->device) (void)hipSetDevice(plan->device);
        (void)hipDeviceSynchronize();
        (void)hipFree(plan->d_mem);
        if (plan->upload_event)
            (void)hipEventDestroy(static_cast<hipEvent_t>(plan->upload_event));
        if (cur != plan->device && cur >= 0) (void)hipSetDevice(cur);
    }
    plan->magic = kDeadMagic;
    delete plan;
}

}  // extern "C"
