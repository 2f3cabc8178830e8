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
// kept in registers.  A wave loads all of its steps of the tile first, each
// step into registers of its own, and then turns and stores them step by
// step, so its waits count down to the step they need instead of draining
// the stores of the step before.  Consecutive lanes cover consecutive
// 16-byte words of a row, so a wave's
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

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>

#include "pic_internal.hpp"
#include "rotate.hpp"

namespace pic {
namespace {

// ------------------------------------------------------------ kernel args

struct KArgs {
    const DevTile *tiles;
    const double *cs;
    const void *src_k;
    const void *src_v;
    void *dst_k;
    void *dst_v;
    int64_t s_layer, s_tok, s_head, s_page;         // source strides
    int64_t d_layer, d_tok, d_head, d_page, d_req;  // destination strides
    int32_t layer_begin;
    int32_t mode;         // DstMode
    int32_t src_paged;    // 1: the pool is paged (tile.src_row is a page)
    int32_t rope_offset;
    int32_t half_r;
    int32_t nr, uph_shift;  // rotary units per token, log2(units per head)
    int32_t nck, cph;       // K copy units per token / per head
    int32_t nv, vph;        // V units per token / per head
    int32_t g;              // tokens per wave step
    int32_t nblk;           // unit blocks per step (1 unless a row is very wide)
    int32_t wpt;            // waves per tile (1, 2 or 4): a workgroup takes 4 / wpt tiles
    int32_t n_tiles;
};

constexpr int kHalf = PIC_ROPE_HALF;

#ifndef PIC_NT_STORES
#define PIC_NT_STORES 1
#endif

// 16-byte global accesses.  The destination is written once per launch and
// not read back by it, so stores are non-temporal; loads are non-temporal
// (NTL) when the plan reads every pool row once, and cached otherwise, so a
// chunk placed into several requests can be served from L2/MALL.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int NTL>
__device__ __forceinline__ uint4 ld16(const void *base, int64_t elem, int esize) {
    const char *p = static_cast<const char *>(base) + elem * esize;
    if constexpr (NTL) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    } else {
        return *reinterpret_cast<const uint4 *>(p);
    }
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

// NW consecutive 32-bit words (NW = 4: one 16-byte access; NW = 1: one dword).
template <int NW, int NTL>
__device__ __forceinline__ void ldw(const void *base, int64_t elem, int esize, uint32_t (&w)[NW]) {
    if constexpr (NW == 4) {
        const uint4 v = ld16<NTL>(base, elem, esize);
        w[0] = v.x;
        w[1] = v.y;
        w[2] = v.z;
        w[3] = v.w;
    } else {
        static_assert(NW == 1, "rotary words are 16 or 4 bytes");
        const uint32_t *p = reinterpret_cast<const uint32_t *>(static_cast<const char *>(base) +
                                                               elem * esize);
        if constexpr (NTL)
            w[0] = __builtin_nontemporal_load(p);
        else
            w[0] = *p;
    }
}
template <int NW>
__device__ __forceinline__ void stw(void *base, int64_t elem, int esize, const uint32_t (&w)[NW]) {
    if constexpr (NW == 4) {
        st16(base, elem, esize, make_uint4(w[0], w[1], w[2], w[3]));
    } else {
        uint32_t *p = reinterpret_cast<uint32_t *>(static_cast<char *>(base) + elem * esize);
#if PIC_NT_STORES
        __builtin_nontemporal_store(w[0], p);
#else
        *p = w[0];
#endif
    }
}

// --------------------------------------------------------------- the kernel

#ifndef PIC_WAVES_PER_EU
#define PIC_WAVES_PER_EU 0
#endif
#if PIC_WAVES_PER_EU > 0
#define PIC_OCCUPANCY_HINT __attribute__((amdgpu_waves_per_eu(PIC_WAVES_PER_EU)))
#else
#define PIC_OCCUPANCY_HINT
#endif

// One workgroup of four wave64s per (4 / wpt tiles, layer): wpt waves take a
// tile of up to 4 wpt wave steps of consecutive tokens of one placed chunk
// landing in consecutive destination rows (wpt < 4 where rows are so narrow
// that a page of them fills fewer than four waves' steps); a wave step covers
// g tokens, whose rotary units (g * nr) and copy units (g * (nck + nv)) are
// dealt to the 64 lanes, MAXR and MAXC per lane.  Each lane's slot offsets
// and the cos/sin of its planes are set up once per tile; all of the wave's
// loads are issued before its stores.
template <typename E, int STYLE, int MAXR, int MAXC, int RB, int NTL>
__global__ void __launch_bounds__(kBlockThreads) PIC_OCCUPANCY_HINT stitch_kernel(const KArgs a) {
    constexpr int VEC = Vec<E>::kElems;              // elements per 16-byte copy unit
    constexpr int ES = sizeof(E);
    constexpr int NW = RB / 4;                       // 32-bit words per rotary word
    constexpr int RVEC = RB / ES;                    // elements per rotary word
    constexpr int NCS = STYLE == kHalf ? RVEC : RVEC / 2;  // planes per rotary unit
    constexpr int kWaves = kBlockThreads / 64;
    constexpr int kNone = 1 << 30;                       // slot token index: unused slot
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int ncv = a.nck + a.nv;
    const int half_off = STYLE == kHalf ? a.half_r : 0;

    // the wave's tile, and its place among the tile's waves
    const int tile = static_cast<int>(blockIdx.x) * (kWaves / a.wpt) + wave / a.wpt;
    if (tile >= a.n_tiles) return;  // the last workgroup's spare waves (no barriers here)
    const int wv = wave % a.wpt;
    const DevTile T = a.tiles[tile];
    const int64_t layer = a.layer_begin + static_cast<int64_t>(blockIdx.y);
    const bool turn = T.cs_idx >= 0;

    // cos/sin of this lane's planes: the same for all of its rotary units,
    // because the rotary units per head (a power of two) divide 64
    double c[NCS], s[NCS];
    if (turn) {
        const int plane0 = (lane & ((1 << a.uph_shift) - 1)) * NCS;
        const double *t = a.cs + (static_cast<int64_t>(T.cs_idx) * a.half_r + plane0) * 2;
#pragma unroll
        for (int p = 0; p < NCS; p++) {
            c[p] = t[2 * p];
            s[p] = t[2 * p + 1];
        }
    }

    const void *sk = a.src_k;
    const void *sv = a.src_v;
    void *dk = a.dst_k;
    void *dv = a.dst_v;
    const int64_t s0 = layer * a.s_layer +
                       (a.src_paged ? T.src_row * a.s_page + static_cast<int64_t>(T.src_slot) * a.s_tok
                                    : T.src_row * a.s_tok);
    int64_t d0;
    if (a.mode == kInPlace)
        d0 = s0;
    else
        d0 = layer * a.d_layer + T.dst_a * (a.mode == kPaged ? a.d_page : a.d_req) +
             static_cast<int64_t>(T.dst_b) * a.d_tok;

    // the unit blocks of a step (one unless a row is very wide); with one,
    // no loop, so that the compiler counts this step's memory operations
    // exactly instead of assuming another iteration's are pending
    auto do_blk = [&](const int blk) {
        int rs[MAXR], rd[MAXR];  // slot offsets from the step's first source/dest row
        int rq[MAXR];            // token of the step the slot belongs to
#pragma unroll
        for (int i = 0; i < MAXR; i++) {
            const int u = (blk * MAXR + i) * 64 + lane;
            rq[i] = kNone;
            rs[i] = rd[i] = 0;
            if (u < a.g * a.nr) {
                const int q = u / a.nr;
                const int r = u - q * a.nr;
                const int h = r >> a.uph_shift;
                const int inner = a.rope_offset + (r & ((1 << a.uph_shift) - 1)) * RVEC;
                rq[i] = q;
                rs[i] = static_cast<int>(q * a.s_tok + h * a.s_head + inner);
                rd[i] = static_cast<int>(q * a.d_tok + h * a.d_head + inner);
            }
        }
        int cs_[MAXC], cd[MAXC];
        int cq[MAXC];
        bool isv[MAXC];
#pragma unroll
        for (int i = 0; i < MAXC; i++) {
            const int u = (blk * MAXC + i) * 64 + lane;
            cq[i] = kNone;
            cs_[i] = cd[i] = 0;
            isv[i] = false;
            if (u < a.g * ncv) {
                const int q = u / ncv;
                const int r = u - q * ncv;
                int h, inner;
                if (r < a.nck) {
                    h = r / a.cph;
                    inner = (r - h * a.cph) * VEC;
                    if (inner >= a.rope_offset) inner += 2 * a.half_r;  // skip the rotary slice
                } else {
                    const int r2 = r - a.nck;
                    h = r2 / a.vph;
                    inner = (r2 - h * a.vph) * VEC;
                    isv[i] = true;
                }
                cq[i] = q;
                cs_[i] = static_cast<int>(q * a.s_tok + h * a.s_head + inner);
                cd[i] = static_cast<int>(q * a.d_tok + h * a.d_head + inner);
            }
        }

        // the wave's steps of the tile (at most kTileSteps: the planner cuts
        // tiles of kTileSteps x 4 waves x g tokens) loaded first, each into
        // registers of its own.  On gfx9 stores and loads share one counter,
        // and a load into registers that a pending store still reads must
        // wait for everything before it; with distinct registers every wait
        // only counts down to the step it needs.
        static_assert(kWaves >= 4, "a tile's steps per wave");
        uint32_t A[kTileSteps][MAXR][NW], B[kTileSteps][MAXR][NW];
        uint4 Cw[kTileSteps][MAXC];
        // Loads are not predicated: a slot with no live token loads the
        // tile's first row instead (always in bounds) and is not stored, so
        // every wave issues the same loads in the same order and the waits
        // can count them.
#pragma unroll
        for (int st = 0; st < kTileSteps; st++) {
            const int t0 = (wv + a.wpt * st) * a.g;
            const int lim = T.ntok - t0;  // slots of tokens q < lim are live
            const int64_t sb = s0 + static_cast<int64_t>(t0) * a.s_tok;
#pragma unroll
            for (int i = 0; i < MAXR; i++) {
                const int64_t o = rq[i] < lim ? sb + rs[i] : s0;
                ldw<NW, NTL>(sk, o, ES, A[st][i]);
                if (STYLE == kHalf) ldw<NW, NTL>(sk, rq[i] < lim ? o + half_off : s0, ES, B[st][i]);
            }
#pragma unroll
            for (int i = 0; i < MAXC; i++)
                Cw[st][i] = ld16<NTL>(isv[i] ? sv : sk, cq[i] < lim ? sb + cs_[i] : s0, ES);
        }
#pragma unroll
        for (int st = 0; st < kTileSteps; st++) {
            const int t0 = (wv + a.wpt * st) * a.g;
            const int lim = T.ntok - t0;
            const int64_t db = d0 + static_cast<int64_t>(t0) * a.d_tok;
#pragma unroll
            for (int i = 0; i < MAXR; i++) {
                if (rq[i] < lim) {
                    if (turn) rotate_unit<E, STYLE, NW>(A[st][i], B[st][i], c, s);
                    stw<NW>(dk, db + rd[i], ES, A[st][i]);
                    if (STYLE == kHalf) stw<NW>(dk, db + rd[i] + half_off, ES, B[st][i]);
                }
            }
#pragma unroll
            for (int i = 0; i < MAXC; i++)
                if (cq[i] < lim) st16(isv[i] ? dv : dk, db + cd[i], ES, Cw[st][i]);
        }
    };
    if (a.nblk == 1) {
        do_blk(0);
        return;
    }
    for (int blk = 0; blk < a.nblk; blk++) do_blk(blk);
}

// The bandwidth reference of the library: a plain copy with the stitch's
// 16-byte non-temporal loads and stores, one read and one write per byte.
// Each thread moves kCopyUnroll words per pass, all loads of a pass issued
// before its stores; passes stride over the whole buffer.
constexpr int kCopyThreads = 512;
constexpr int kCopyUnroll = 4;

__global__ void __launch_bounds__(kCopyThreads)
    stream_copy_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kCopyThreads;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x; base < n;
         base += stride * kCopyUnroll) {
        u32x4 w[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; u++) {
            const int64_t i = base + u * stride;
            if (i < n) w[u] = __builtin_nontemporal_load(src + i);
        }
#pragma unroll
        for (int u = 0; u < kCopyUnroll; u++) {
            const int64_t i = base + u * stride;
            if (i < n) __builtin_nontemporal_store(w[u], dst + i);
        }
    }
}

// ----------------------------------------------------------------- launch

// The kernel keeps a step's slot offsets in 32 bits: g token rows and all
// heads of a view must span fewer than 2^31 elements.
bool slot_offsets_fit(const Problem &p, int64_t tok, int64_t head) {
    const int64_t span = (p.launch.g - 1) * tok +
                         static_cast<int64_t>(p.shape.num_heads - 1) * head + p.shape.row_dim;
    return span <= INT32_MAX;
}

template <typename E, int STYLE, int MAXR, int MAXC, int RB, int NTL>
hipError_t launch_kernel(const KArgs &a, int n_tiles, int n_layers, hipStream_t stream) {
    const int per_group = (kBlockThreads / 64) / a.wpt;  // tiles per workgroup
    dim3 grid(static_cast<unsigned>((n_tiles + per_group - 1) / per_group),
              static_cast<unsigned>(n_layers));
    hipLaunchKernelGGL((stitch_kernel<E, STYLE, MAXR, MAXC, RB, NTL>), grid, dim3(kBlockThreads),
                       0, stream, a);
    return hipGetLastError();
}

template <typename E, int STYLE, int RB, int NTL>
hipError_t launch_shape(const Problem &p, const KArgs &a, int n_layers, hipStream_t stream) {
    const int n_tiles = static_cast<int>(p.tiles.size());
    const Launch &l = p.launch;
    if (l.maxr == 1 && l.maxc == 2)
        return launch_kernel<E, STYLE, 1, 2, RB, NTL>(a, n_tiles, n_layers, stream);
    if (l.maxr == 1) return launch_kernel<E, STYLE, 1, 4, RB, NTL>(a, n_tiles, n_layers, stream);
    return launch_kernel<E, STYLE, 2, 4, RB, NTL>(a, n_tiles, n_layers, stream);
}

template <typename E, int STYLE, int RB>
hipError_t launch_rb(const Problem &p, const KArgs &a, int n_layers, hipStream_t stream) {
    if (p.launch.stream_loads) return launch_shape<E, STYLE, RB, 1>(p, a, n_layers, stream);
    return launch_shape<E, STYLE, RB, 0>(p, a, n_layers, stream);
}

template <typename E, int STYLE>
hipError_t launch_style(const Problem &p, const KArgs &a, int n_layers, hipStream_t stream) {
    if constexpr (STYLE == PIC_ROPE_HALF) {
        if (p.launch.rb == 4) return launch_rb<E, STYLE, 4>(p, a, n_layers, stream);
    }
    return launch_rb<E, STYLE, 16>(p, a, n_layers, stream);
}

hipError_t launch(const Problem &p, KArgs a, int n_layers, hipStream_t stream) {
    a.g = p.launch.g;
    a.nblk = p.launch.nblk;
    a.wpt = p.launch.wpt;
    a.n_tiles = static_cast<int32_t>(p.tiles.size());
    a.nr = p.launch.nr;
    a.uph_shift = p.launch.uph_shift;
    if (p.shape.dtype == PIC_DTYPE_F32)
        return p.style == PIC_ROPE_HALF ? launch_style<float, PIC_ROPE_HALF>(p, a, n_layers, stream)
                                        : launch_style<float, PIC_ROPE_INTERLEAVED>(p, a, n_layers, stream);
    return p.style == PIC_ROPE_HALF ? launch_style<uint16_t, PIC_ROPE_HALF>(p, a, n_layers, stream)
                                    : launch_style<uint16_t, PIC_ROPE_INTERLEAVED>(p, a, n_layers, stream);
}

}  // namespace

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

KArgs args_for(const Problem &p, const uint8_t *dmem, const Staged &stg) {
    KArgs a{};
    a.tiles = reinterpret_cast<const DevTile *>(dmem + stg.off_tiles);
    a.cs = reinterpret_cast<const double *>(dmem + stg.off_cs);
    a.mode = p.mode;
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

// Upload the plan's metadata to the current device on first use, ordered on
// `stream`; later uses on any stream wait for that upload.  A plan stays on
// the device of its first use.  The copies read the plan's own tile and
// table vectors, which live as long as the plan.
pic_status ensure_device_plan(struct ::pic_plan *plan, void *stream_) {
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    std::lock_guard<std::mutex> lock(plan->mu);
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (!plan->d_mem) {
        const Problem &p = plan->prob;
        const Staged &stg = plan->staged;
        e = hipMalloc(&plan->d_mem, stg.total);
        if (e != hipSuccess) {
            plan->d_mem = nullptr;
            return hip_fail(e, "hipMalloc (plan metadata)");
        }
        uint8_t *d = static_cast<uint8_t *>(plan->d_mem);
        if (!p.tiles.empty())
            e = hipMemcpyAsync(d + stg.off_tiles, p.tiles.data(), p.tiles.size() * sizeof(DevTile),
                               hipMemcpyHostToDevice, stream);
        if (e == hipSuccess && !p.cs.empty())
            e = hipMemcpyAsync(d + stg.off_cs, p.cs.data(), p.cs.size() * sizeof(double),
                               hipMemcpyHostToDevice, stream);
        hipEvent_t ev = nullptr;
        if (e == hipSuccess) e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventRecord(ev, stream);
        if (e != hipSuccess) {
            if (ev) (void)hipEventDestroy(ev);
            (void)hipStreamSynchronize(stream);  // nothing may still read or write d_mem
            (void)hipFree(plan->d_mem);
            plan->d_mem = nullptr;
            return hip_fail(e, "plan metadata upload");
        }
        plan->upload_event = ev;
        plan->device = dev;
        return PIC_OK;
    }
    if (dev != plan->device)
        return fail(PIC_ERR_STATE, "plan was uploaded to device %d, current device is %d",
                    plan->device, dev);
    e = hipStreamWaitEvent(stream, static_cast<hipEvent_t>(plan->upload_event), 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
    return PIC_OK;
}

pic_status plan_blob(struct ::pic_plan *plan, int64_t key, void *stream_,
                     const std::function<void(DevBlob &)> &make, const DevBlob **out) {
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    std::lock_guard<std::mutex> lock(plan->mu);
    auto it = plan->blobs.find(key);
    if (it == plan->blobs.end()) {
        DevBlob b;
        try {
            make(b);
        } catch (const std::bad_alloc &) {
            return fail(PIC_ERR_NOMEM, "out of host memory (attention metadata)");
        }
        const size_t n = std::max<size_t>(b.host.size(), 16);
        b.host.resize(n);
        hipError_t e = hipMalloc(&b.dev, n);
        if (e != hipSuccess) return hip_fail(e, "hipMalloc (attention metadata)");
        hipEvent_t ev = nullptr;
        e = hipMemcpyAsync(b.dev, b.host.data(), n, hipMemcpyHostToDevice, stream);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventRecord(ev, stream);
        if (e != hipSuccess) {
            if (ev) (void)hipEventDestroy(ev);
            (void)hipStreamSynchronize(stream);
            (void)hipFree(b.dev);
            return hip_fail(e, "attention metadata upload");
        }
        b.ready = ev;
        it = plan->blobs.emplace(key, std::move(b)).first;
    }
    const hipError_t e = hipStreamWaitEvent(stream, static_cast<hipEvent_t>(it->second.ready), 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
    *out = &it->second;  // map nodes never move, and blobs are never erased before the plan
    return PIC_OK;
}

pic_status call_workspace(struct ::pic_plan *plan, size_t bytes, void *stream, void **out) {
    *out = nullptr;
    bytes = std::max<size_t>(bytes, 256);
    std::lock_guard<std::mutex> lock(plan->mu);
    Workspace *w = nullptr;
    for (auto &x : plan->work)
        if (x.stream == stream) w = &x;
    if (w && w->bytes >= bytes) {
        *out = w->ptr;
        return PIC_OK;
    }
    if (w) {
        // outgrown: the work already queued on the stream may still read it
        hipEvent_t ev = nullptr;
        hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming | hipEventDisableSystemFence);
        if (e == hipSuccess) e = hipEventRecord(ev, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) {
            if (ev) (void)hipEventDestroy(ev);
            return hip_fail(e, "attention workspace retirement");
        }
        plan->retired_work.emplace_back(w->ptr, ev);
        bytes = std::max(bytes, w->bytes + w->bytes / 2);
        w->ptr = nullptr;
        w->bytes = 0;
    }
    void *p = nullptr;
    const hipError_t e = hipMalloc(&p, bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return hip_fail(e, "hipMalloc (attention workspace)");
    }
    if (w) {
        w->ptr = p;
        w->bytes = bytes;
    } else {
        plan->work.push_back(Workspace{stream, p, bytes});
    }
    *out = p;
    return PIC_OK;
}

pic_status note_use(struct ::pic_plan *plan, void *stream) {
    std::lock_guard<std::mutex> lock(plan->mu);
    hipEvent_t ev = nullptr;
    for (auto &u : plan->uses)
        if (u.first == stream) ev = static_cast<hipEvent_t>(u.second);
    if (!ev) {
        // completion is all that destroy waits for: no system-scope fence
        hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming | hipEventDisableSystemFence);
        if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
        plan->uses.emplace_back(stream, ev);
    }
    const hipError_t e = hipEventRecord(ev, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    return PIC_OK;
}

namespace {

// Pinned staging for per-call metadata.  A copy from pageable memory makes
// hipMemcpyAsync wait for the stream to drain, so each call would stall its
// caller until earlier work finished; copies from pinned memory are truly
// asynchronous.  Each device keeps a ring of pinned slots, each guarded by
// an event recorded after the copy that reads it: a slot is refilled only
// once that copy has run (the wait blocks only with more calls in flight
// than slots).  Slots grow on demand and live until the process ends.
constexpr int kPinnedSlots = 4;

struct PinnedSlot {
    void *host = nullptr;
    size_t cap = 0;
    hipEvent_t done = nullptr;
};

struct PinnedRing {
    std::mutex mu;
    PinnedSlot slots[kPinnedSlots];
    int next = 0;
};

PinnedRing *pinned_ring(int device) {
    static std::mutex mu;
    static std::map<int, std::unique_ptr<PinnedRing>> rings;
    std::lock_guard<std::mutex> lock(mu);
    std::unique_ptr<PinnedRing> &r = rings[device];
    if (!r) r.reset(new (std::nothrow) PinnedRing);
    return r.get();
}

// Kernel arguments of a per-call problem whose metadata sits at dmem, with
// the pointers and strides of `views`.
KArgs with_views(const Problem &p, const KArgs &views, const uint8_t *dmem, const Staged &stg,
                 int32_t layer_begin) {
    KArgs a = args_for(p, dmem, stg);
    a.src_k = views.src_k;
    a.src_v = views.src_v;
    a.dst_k = views.dst_k;
    a.dst_v = views.dst_v;
    a.s_layer = views.s_layer;
    a.s_tok = views.s_tok;
    a.s_head = views.s_head;
    a.s_page = views.s_page;
    a.src_paged = views.src_paged;
    a.d_layer = views.d_layer;
    a.d_tok = views.d_tok;
    a.d_head = views.d_head;
    a.d_page = views.d_page;
    a.d_req = views.d_req;
    a.layer_begin = layer_begin;
    return a;
}

// ------------------------------------------------- the no-allocation path
//
// pic_rotate_inplace_noalloc stages its tiles and shift tables in this
// file-scope array instead of stream-ordered device memory.  In host code
// the name `scratch` is a host-side stand-in, not a device address: the
// device address is taken once per device with hipGetSymbolAddress (that
// device current) and used wherever host code needs the array.  Every call
// on a device shares its copy; calls that overlap on one device (different
// streams) race.
constexpr size_t kScratchBytes = size_t{4} << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// The metadata reaches the array through kernel arguments, kFillBytes per
// launch: the runtime copies arguments at launch, so no host buffer has to
// outlive the call and nothing is allocated.
constexpr int kFillBytes = 3584;
struct FillArgs {
    uint4 *dst;
    uint32_t n16;  // 16-byte words in `words`
    uint32_t pad;
    uint4 words[kFillBytes / 16];
};

__global__ void __launch_bounds__(256) scratch_fill_kernel(const FillArgs a) {
    for (uint32_t i = threadIdx.x; i < a.n16; i += 256) a.dst[i] = a.words[i];
}

constexpr int kMaxDevices = 64;

// The device address of `scratch` on device `dev` (current), taken once.
pic_status scratch_address(int dev, uint8_t **out) {
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    if (dev < 0 || dev >= kMaxDevices) return fail(PIC_ERR_DEVICE, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) return hip_fail(e, "hipGetSymbolAddress (scratch)");
        addr[dev] = ptr;
    }
    *out = static_cast<uint8_t *>(addr[dev]);
    return PIC_OK;
}

}  // namespace

pic_status stage_per_call(size_t n, const std::function<void(uint8_t *)> &fill, void *stream_,
                          void **dmem, const char *what) {
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    *dmem = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PIC_ERR_DEVICE, "%s: hipGetDevice: %s", what, hipGetErrorString(e));
    PinnedRing *ring = pinned_ring(dev);
    if (!ring) return fail(PIC_ERR_NOMEM, "out of host memory");
    std::lock_guard<std::mutex> lock(ring->mu);
    PinnedSlot &slot = ring->slots[ring->next];
    ring->next = (ring->next + 1) % kPinnedSlots;
    if (slot.done) {
        e = hipEventSynchronize(slot.done);  // the copy that last read the slot has run
        if (e != hipSuccess)
            return fail(PIC_ERR_DEVICE, "%s: hipEventSynchronize: %s", what, hipGetErrorString(e));
    } else {
        e = hipEventCreateWithFlags(&slot.done, hipEventDisableTiming);
        if (e != hipSuccess) {
            slot.done = nullptr;
            return fail(PIC_ERR_DEVICE, "%s: hipEventCreate: %s", what, hipGetErrorString(e));
        }
    }
    if (slot.cap < n) {
        if (slot.host) (void)hipHostFree(slot.host);
        slot.host = nullptr;
        slot.cap = 0;
        const size_t cap = std::max<size_t>(n, size_t{1} << 20);
        e = hipHostMalloc(&slot.host, cap, hipHostMallocDefault);
        if (e != hipSuccess) {
            slot.host = nullptr;
            return fail(PIC_ERR_NOMEM, "%s: hipHostMalloc (%zu bytes): %s", what, cap,
                        hipGetErrorString(e));
        }
        slot.cap = cap;
    }
    fill(static_cast<uint8_t *>(slot.host));
    e = hipMallocAsync(dmem, n, stream);
    if (e != hipSuccess) {
        *dmem = nullptr;
        (void)hipGetLastError();  // clear it
        return fail(PIC_ERR_DEVICE, "%s: hipMallocAsync (metadata): %s", what, hipGetErrorString(e));
    }
    e = hipMemcpyAsync(*dmem, slot.host, n, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipEventRecord(slot.done, stream);
    if (e != hipSuccess) {
        (void)hipFreeAsync(*dmem, stream);
        *dmem = nullptr;
        (void)hipStreamSynchronize(stream);
        return fail(PIC_ERR_DEVICE, "%s: hipMemcpyAsync (metadata): %s", what, hipGetErrorString(e));
    }
    return PIC_OK;
}

namespace {

// Stage a per-call problem's tiles and shift tables in stream-ordered device
// memory (freed on the same stream once the kernel has run) and launch it
// over n_layers layers from layer_begin; views holds the pointers and strides.
pic_status run_staged(const Problem &p, const KArgs &views, int32_t layer_begin, int32_t n_layers,
                      hipStream_t stream, const char *what) {
    if (p.tiles.empty() || n_layers == 0) return PIC_OK;
    const Staged stg = stage(p);
    void *dmem = nullptr;
    pic_status st = stage_per_call(stg.total, [&](uint8_t *host) { write_staged(p, stg, host); },
                                   stream, &dmem, what);
    if (st) return st;
    hipError_t e = launch(p, with_views(p, views, static_cast<const uint8_t *>(dmem), stg, layer_begin),
                          n_layers, stream);
    const hipError_t e2 = hipFreeAsync(dmem, stream);
    if (e != hipSuccess) return fail(PIC_ERR_DEVICE, "%s kernel launch: %s", what, hipGetErrorString(e));
    if (e2 != hipSuccess)
        return fail(PIC_ERR_DEVICE, "%s: hipFreeAsync (metadata): %s", what, hipGetErrorString(e2));
    return PIC_OK;
}

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
    if (!slot_offsets_fit(p, pool->token_stride, pool->head_stride) ||
        !slot_offsets_fit(p, dst->token_stride, dst->head_stride))
        return fail(PIC_ERR_RANGE, "a view's token/head strides span 2^31 elements or more "
                    "within one step");
    if (p.tiles.empty() || layer_begin == layer_end) return PIC_OK;

    hipStream_t stream = static_cast<hipStream_t>(stream_);
    st = ensure_device_plan(plan, stream_);
    if (st) return st;

    KArgs a = args_for(p, static_cast<const uint8_t *>(plan->d_mem), plan->staged);
    a.src_k = pool->k;
    a.src_v = pool->v;
    a.dst_k = dst->k;
    a.dst_v = dst->v;
    a.s_layer = pool->layer_stride;
    a.s_tok = pool->token_stride;
    a.s_head = pool->head_stride;
    a.s_page = pool->page_stride;
    a.src_paged = p.src_page_size > 0 ? 1 : 0;
    a.d_layer = dst->layer_stride;
    a.d_tok = dst->token_stride;
    a.d_head = dst->head_stride;
    a.d_page = dst->page_stride;
    a.d_req = dst->request_stride;
    a.layer_begin = layer_begin;
    const hipError_t e = launch(p, a, layer_end - layer_begin, stream);
    if (e != hipSuccess) return hip_fail(e, "stitch kernel launch");
    return note_use(plan, stream_);
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
    if (!slot_offsets_fit(p, buf->token_stride, buf->head_stride))
        return fail(PIC_ERR_RANGE, "the view's token/head strides span 2^31 elements or more "
                    "within one step");
    if (p.tiles.empty() || layer_begin == layer_end) return PIC_OK;

    KArgs v{};
    v.src_k = buf->k;
    v.dst_k = buf->k;
    v.s_layer = v.d_layer = buf->layer_stride;
    v.s_tok = v.d_tok = buf->token_stride;
    v.s_head = v.d_head = buf->head_stride;
    return run_staged(p, v, layer_begin, layer_end - layer_begin, static_cast<hipStream_t>(stream_),
                      "rotate");
}

pic_status pic_rotate_inplace_noalloc(const pic_kv_shape *shape, const pic_rope_config *rope,
                                      const pic_kv_view *buf, int64_t buf_tokens,
                                      const pic_segment *segments, int32_t n_segments,
                                      int32_t layer_begin, int32_t layer_end, void *stream_) {
    using namespace pic;
    clear_error();
    Problem p;
    pic_status st;
    try {
        st = build_inplace(shape, rope, buf_tokens, segments, n_segments, &p);
    } catch (const std::bad_alloc &) {
        return fail(PIC_ERR_NOMEM, "out of host memory");
    }
    if (st) return st;
    if (layer_begin < 0 || layer_begin > layer_end || layer_end > p.shape.num_layers)
        return fail(PIC_ERR_INVALID_ARG, "layer range [%d, %d) outside [0, %d)", layer_begin,
                    layer_end, p.shape.num_layers);
    st = check_view(buf, p.u.vec, false, "buf");
    if (st) return st;
    if (!slot_offsets_fit(p, buf->token_stride, buf->head_stride))
        return fail(PIC_ERR_RANGE, "the view's token/head strides span 2^31 elements or more "
                    "within one step");
    const Staged stg = stage(p);
    if (stg.total > kScratchBytes)
        return fail(PIC_ERR_RANGE, "%zu bytes of tiles and shift tables (%zu tiles, %zu tables) "
                    "exceed the %zu-byte static scratch", stg.total, p.tiles.size(),
                    p.cs.size() / std::max(1, p.rope_dim), kScratchBytes);
    if (p.tiles.empty() || layer_begin == layer_end) return PIC_OK;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    uint8_t *dmem = nullptr;
    st = scratch_address(dev, &dmem);
    if (st) return st;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    FillArgs fa{};
    for (size_t off = 0; off < stg.total; off += kFillBytes) {
        const size_t n = std::min<size_t>(kFillBytes, stg.total - off);  // a multiple of 16
        std::memset(fa.words, 0, sizeof fa.words);
        auto put = [&](size_t at, const void *src, size_t len) {  // [at, at + len) of the layout
            const size_t lo = std::max(at, off), hi = std::min(at + len, off + n);
            if (lo < hi)
                std::memcpy(reinterpret_cast<uint8_t *>(fa.words) + (lo - off),
                            static_cast<const uint8_t *>(src) + (lo - at), hi - lo);
        };
        put(stg.off_tiles, p.tiles.data(), p.tiles.size() * sizeof(DevTile));
        put(stg.off_cs, p.cs.data(), p.cs.size() * sizeof(double));
        fa.dst = reinterpret_cast<uint4 *>(dmem + off);
        fa.n16 = static_cast<uint32_t>(n / 16);
        hipLaunchKernelGGL(scratch_fill_kernel, dim3(1), dim3(256), 0, stream, fa);
        e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e, "scratch fill launch");
    }
    KArgs v{};
    v.src_k = buf->k;
    v.dst_k = buf->k;
    v.s_layer = v.d_layer = buf->layer_stride;
    v.s_tok = v.d_tok = buf->token_stride;
    v.s_head = v.d_head = buf->head_stride;
    e = launch(p, with_views(p, v, dmem, stg, layer_begin), layer_end - layer_begin, stream);
    if (e != hipSuccess) return hip_fail(e, "rotate kernel launch");
    return PIC_OK;
}

pic_status pic_rotate_paged(const pic_kv_shape *shape, const pic_rope_config *rope,
                            const pic_kv_view *buf, int32_t page_size, int64_t n_phys_pages,
                            const pic_page_segment *segments, int32_t n_segments,
                            int32_t layer_begin, int32_t layer_end, void *stream_) {
    using namespace pic;
    clear_error();
    Problem turn, copy;
    pic_status st = build_rotate_paged(shape, rope, page_size, n_phys_pages, segments, n_segments,
                                       &turn, &copy);
    if (st) return st;
    if (layer_begin < 0 || layer_begin > layer_end || layer_end > shape->num_layers)
        return fail(PIC_ERR_INVALID_ARG, "layer range [%d, %d) outside [0, %d)", layer_begin,
                    layer_end, shape->num_layers);
    const bool need_v = !copy.tiles.empty() && shape->has_v;
    st = check_view(buf, turn.u.vec, need_v, "buf");
    if (st) return st;
    if (!slot_offsets_fit(copy, buf->token_stride, buf->head_stride) ||
        !slot_offsets_fit(turn, buf->token_stride, buf->head_stride))
        return fail(PIC_ERR_RANGE, "the view's token/head strides span 2^31 elements or more "
                    "within one step");
    if (layer_begin == layer_end) return PIC_OK;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    KArgs v{};
    v.src_k = v.dst_k = buf->k;
    v.src_v = v.dst_v = need_v ? buf->v : nullptr;
    v.s_layer = v.d_layer = buf->layer_stride;
    v.s_tok = v.d_tok = buf->token_stride;
    v.s_head = v.d_head = buf->head_stride;
    v.s_page = v.d_page = buf->page_stride;
    v.src_paged = 1;
    // the copies read shared pages that no turn writes, and the turns write
    // pages that no copy reads or writes, so their order does not matter
    st = run_staged(copy, v, layer_begin, layer_end - layer_begin, stream, "copy-on-write");
    if (st) return st;
    return run_staged(turn, v, layer_begin, layer_end - layer_begin, stream, "paged rotate");
}

pic_status pic_stream_copy(void *dst, const void *src, int64_t nbytes, void *stream_) {
    using namespace pic;
    clear_error();
    if (nbytes < 0) return fail(PIC_ERR_RANGE, "nbytes %lld < 0", static_cast<long long>(nbytes));
    if (nbytes == 0) return PIC_OK;
    if (!dst || !src) return fail(PIC_ERR_INVALID_ARG, "dst and src must not be NULL");
    if ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src) |
         static_cast<uintptr_t>(nbytes)) & 15u)
        return fail(PIC_ERR_ALIGN, "dst, src and nbytes must be multiples of 16 bytes");
    const uintptr_t d0 = reinterpret_cast<uintptr_t>(dst), s0 = reinterpret_cast<uintptr_t>(src);
    if (d0 < s0 + static_cast<uintptr_t>(nbytes) && s0 < d0 + static_cast<uintptr_t>(nbytes))
        return fail(PIC_ERR_OVERLAP, "dst and src overlap");
    const int64_t n = nbytes / 16;
    const int64_t per_block = int64_t{kCopyThreads} * kCopyUnroll;
    const int64_t blocks = std::min<int64_t>(16384, (n + per_block - 1) / per_block);
    hipLaunchKernelGGL(stream_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kCopyThreads),
                       0, static_cast<hipStream_t>(stream_), static_cast<const u32x4 *>(src),
                       static_cast<u32x4 *>(dst), n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "copy kernel launch");
    return PIC_OK;
}

void pic_plan_destroy(pic_plan_t *plan) {
    using namespace pic;
    if (!plan || plan->magic != kPlanMagic) return;
    plan->magic = kDeadMagic;
    if (plan->d_mem) {
        int cur = -1;
        (void)hipGetDevice(&cur);
        if (cur != plan->device) (void)hipSetDevice(plan->device);
        // the plan's own work only: the last use on every stream it ran on
        for (auto &u : plan->uses) {
            (void)hipEventSynchronize(static_cast<hipEvent_t>(u.second));
            (void)hipEventDestroy(static_cast<hipEvent_t>(u.second));
        }
        for (auto &r : plan->retired_work) {
            (void)hipEventSynchronize(static_cast<hipEvent_t>(r.second));
            (void)hipEventDestroy(static_cast<hipEvent_t>(r.second));
            (void)hipFree(r.first);
        }
        for (auto &w : plan->work) (void)hipFree(w.ptr);
        for (auto &kv : plan->blobs) {
            (void)hipEventSynchronize(static_cast<hipEvent_t>(kv.second.ready));
            (void)hipEventDestroy(static_cast<hipEvent_t>(kv.second.ready));
            (void)hipFree(kv.second.dev);
        }
        if (plan->upload_event) {
            (void)hipEventSynchronize(static_cast<hipEvent_t>(plan->upload_event));
            (void)hipEventDestroy(static_cast<hipEvent_t>(plan->upload_event));
        }
        (void)hipFree(plan->d_mem);
        if (cur != plan->device && cur >= 0) (void)hipSetDevice(cur);
    }
    delete plan;
}

}  // extern "C"
