// pic_internal.hpp -- plan representation shared by the host planner
// (plan.cpp) and the HIP launch code (stitch.hip).
#pragma once

#include <cstdint>
#include <functional>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "attend_map.hpp"
#include "pic_stitch.h"

namespace pic {

constexpr uint32_t kPlanMagic = 0x50494350u;  // live plan
constexpr uint32_t kDeadMagic = 0x44454144u;  // destroyed plan
#ifndef PIC_TILE_TOKENS
#define PIC_TILE_TOKENS 16
#endif
#ifndef PIC_BLOCK_THREADS
#define PIC_BLOCK_THREADS 256
#endif
constexpr int kTileSteps = PIC_TILE_TOKENS / 4;  // wave steps per tile (4 waves)
constexpr int kBlockThreads = PIC_BLOCK_THREADS; // wave64s per workgroup x 64

// Destination addressing of a plan.
enum DstMode : int32_t { kContiguous = 0, kPaged = 1, kInPlace = 2 };

// One work tile: ntok consecutive tokens of one placed chunk that land in
// consecutive destination rows (a paged tile never crosses a page).  The
// kernel reads it for every layer of a launch.
struct DevTile {
    int64_t src_row;   // contiguous pool: row of the first token; paged pool: its page
    int64_t dst_a;     // contiguous: request; paged: physical page; in place: unused
    int32_t dst_b;     // contiguous: position; paged: slot in the page; in place: unused
    int32_t ntok;
    int32_t cs_idx;    // shift table, -1 = delta 0 (rows copied)
    int32_t src_slot;  // paged pool: slot of the first token in its page
};

// Host-side record of one placement (entry of a request, or in-place segment).
struct HostEntry {
    int64_t src_tok;
    int64_t dst_pos;
    int32_t request;
    int32_t page_base;
    int32_t cs_idx;
    int32_t pad;
};

// 16-byte work units of one token row, derived from the shape.
struct Units {
    int32_t vec;        // elements per 16 bytes
    int32_t half_r;     // rope_dim / 2
    int32_t nr, uph;    // rotary units per token / per head (uph: power of two dividing 64)
    int32_t uph_shift;  // log2(uph)
    int32_t ncs;        // cos/sin pairs one rotary unit needs
    int32_t interleaved;  // 1 for interleaved pairing
    int32_t nck, cph;   // K copy units per token / per head (non-rotary dims)
    int32_t nv, vph;    // V units per token / per head
};

// Per-lane slot shape of a launch: MAXR rotary and MAXC copy units per lane,
// g tokens per wave step, nblk unit blocks per step; rotary units are rb-byte
// words (16, or 4 when 16-byte rotary units would leave lanes of a step idle),
// nr of them per token, 2^uph_shift per head.
struct Launch {
    int32_t maxr = 1, maxc = 2, g = 1, nblk = 1;
    int32_t wpt = 4;  // waves per tile: a workgroup of 4 waves takes 4 / wpt tiles
    int32_t rb = 16, nr = 0, uph_shift = 0;
    int32_t stream_loads = 0;  // 1: no pool row is read twice in a launch (non-temporal loads)
};

// What a plan's attention map is built from, copied from the caller's arrays
// by pic_plan (pic_plan returns before the map exists; the first call that
// needs it builds it).  requests[r] and chunks[c] point into the vectors
// here.
struct AttnSource {
    std::vector<pic_chunk> chunks;
    std::vector<int32_t> chunk_pages;  // pool page tables, chunk after chunk (paged pool)
    std::vector<pic_entry> entries;    // request after request
    std::vector<int32_t> req_pages;    // destination page tables, request after request
    std::vector<pic_request> requests;
    std::vector<int32_t> cs_of_entry;  // shift table of every entry (-1: delta 0)
};

struct Problem {
    pic_kv_shape shape{};
    int32_t rope_dim = 0;
    int32_t style = 0;
    int32_t mode = kContiguous;
    int32_t page_size = 0;
    int32_t src_page_size = 0;  // 0: contiguous pool
    int64_t capacity = 0;
    int64_t num_phys_pages = 0;
    int32_t n_requests = 0;
    Units u{};
    Launch launch{};
    int32_t tile_tokens = 0;
    std::vector<HostEntry> entries;
    std::vector<DevTile> tiles;
    std::vector<double> cs;       // [table][rope_dim/2][cos, sin]
    std::vector<int64_t> bounds;  // [entry][request, begin, end]
    std::vector<int64_t> recompute;
    AttnSource attn_src;
    bool attn_built = false;       // the members below exist once this is set
    std::vector<AttnTile> atiles;  // pic_attend map, request after request
    std::vector<AttnBlock> ablocks;
    std::vector<int64_t> context;  // context_len per request
    std::vector<int32_t> req_block0;  // first attention block of each request (+ end)
    std::vector<int32_t> req_tile0;   // first attention tile of each request (+ end)
    int32_t attn_block_tokens = 0;    // positions per attention block at most
    std::vector<int32_t> context_bad_page;  // per request: a context page out of range (-1: none)
    pic_plan_info_t info{};
};

// Layout of a plan's stitch tiles and shift tables in one device buffer.
struct Staged {
    size_t off_tiles = 0, off_cs = 0, total = 0;
};

// Metadata of one attention launch shape (the map in work blocks, or work
// items of a kernel), packed for one upload: `host` stays alive with the
// plan (the copy reads it asynchronously), `ready` is recorded after the
// copy and every launch that reads `dev` waits for it on its own stream.
// Blobs are never rebuilt or freed before the plan, so launches on other
// streams can still read them.
struct DevBlob {
    std::vector<uint8_t> host;
    void *dev = nullptr;
    void *ready = nullptr;  // hipEvent_t
    size_t off[8] = {};
    int32_t n[4] = {};
};
enum BlobKind : int64_t { kBlobAttnMap = 1, kBlobGqa = 2, kBlobLatent = 3, kBlobBoundary = 4 };
inline int64_t blob_key(BlobKind kind, int64_t shape_key) { return (int64_t{kind} << 56) | shape_key; }

// Thread-local error reporting.
void clear_error();
pic_status fail(pic_status st, const char *fmt, ...);

// Shape/rope validation and work-unit derivation.
pic_status derive_units(const pic_kv_shape *shape, const pic_rope_config *rope, bool inplace,
                        Units *u);

// Slot shape of the kernel for a dtype and unit counts.
Launch launch_shape_of(int32_t dtype, const Units &u);

// The attention map of a copy-mode problem, from its AttnSource (host only).
void build_attention(Problem *p);

// Copy-mode and in-place problem builders (host only).
pic_status build_stitch(const pic_kv_shape *shape, const pic_rope_config *rope,
                        const pic_chunk *chunks, int32_t n_chunks, const pic_request *requests,
                        int32_t n_requests, const pic_geom *geom, Problem *out);
pic_status build_inplace(const pic_kv_shape *shape, const pic_rope_config *rope,
                         int64_t buf_tokens, const pic_segment *segments, int32_t n_segments,
                         Problem *out);

// pic_rotate_paged: the in-place turns (turn) and the copies of shared pages
// (copy) of a set of paged segments, validated.
pic_status build_rotate_paged(const pic_kv_shape *shape, const pic_rope_config *rope,
                              int32_t page_size, int64_t n_phys_pages,
                              const pic_page_segment *segments, int32_t n_segments,
                              Problem *turn, Problem *copy);
Staged stage(const Problem &p);
// The staged bytes of p written to `out` (stage(p).total bytes).
void write_staged(const Problem &p, const Staged &s, uint8_t *out);

// The matrix-core path of pic_attend (attend_gqa.hip): whether it takes a
// plan at a GQA group size, and its launch (arguments checked by pic_attend).
bool gqa_tile_path(const Problem &p, int group);

// The plan's attention map, built on first use (host only; thread-safe).
pic_status ensure_attention(struct ::pic_plan *plan);

// Device side (stitch.hip): first-use upload of a plan's metadata, ordered on
// `stream` (a hipStream_t); view checks shared by the launchers.
pic_status ensure_device_plan(struct ::pic_plan *plan, void *stream);
pic_status check_view(const pic_kv_view *v, int vec, bool need_v, const char *name);

// The plan's blob `key` on its device: built by `make` and uploaded ordered
// on `stream` the first time, and waited for on `stream` every time
// (ensure_device_plan must have succeeded first).
pic_status plan_blob(struct ::pic_plan *plan, int64_t key, void *stream,
                     const std::function<void(DevBlob &)> &make, const DevBlob **out);

// A workspace of at least `bytes` for a call's launches on `stream`: the
// plan keeps one buffer per stream for its whole life, so the calls on one
// stream reuse it in stream order and calls on different streams never share
// one.  A buffer too small is replaced by a larger one (at least 1.5 times
// the size); the old one is kept, with an event recorded on the stream after
// the work already queued there, until pic_plan_destroy frees it.
pic_status call_workspace(struct ::pic_plan *plan, size_t bytes, void *stream, void **out);

// One stream's workspace of a plan.
struct Workspace {
    void *stream;  // hipStream_t
    void *ptr;
    size_t bytes;
};

// n bytes written by `fill` into pinned staging, copied ordered on `stream`
// into fresh stream-ordered device memory *dmem (the caller frees it with
// hipFreeAsync on the same stream after the launches that read it).
pic_status stage_per_call(size_t n, const std::function<void(uint8_t *)> &fill, void *stream,
                          void **dmem, const char *what);

// Record that work reading the plan is enqueued on `stream` (the plan keeps
// one event per stream it was used on; pic_plan_destroy waits for them).
pic_status note_use(struct ::pic_plan *plan, void *stream);
}  // namespace pic

// The opaque plan handle of the C ABI.
struct pic_plan {
    uint32_t magic = pic::kPlanMagic;
    pic::Problem prob;
    pic::Staged staged;
    std::mutex mu;
    int device = -1;
    void *d_mem = nullptr;
    void *upload_event = nullptr;  // hipEvent_t
    std::map<int64_t, pic::DevBlob> blobs;
    std::vector<std::pair<void *, void *>> uses;  // (hipStream_t, hipEvent_t of its last use)
    std::vector<pic::Workspace> work;  // attention workspaces, one per stream
    std::vector<std::pair<void *, void *>> retired_work;  // (buffer, hipEvent_t after its last use)
};
