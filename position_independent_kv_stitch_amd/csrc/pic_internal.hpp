// pic_internal.hpp -- plan representation shared by the host planner
// (plan.cpp) and the HIP launch code (stitch.hip).
#pragma once

#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "pic_stitch.h"

namespace pic {

constexpr uint32_t kPlanMagic = 0x50494350u;  // live plan
constexpr uint32_t kDeadMagic = 0x44454144u;  // destroyed plan
#ifndef PIC_TILE_TOKENS
#define PIC_TILE_TOKENS 64
#endif
#ifndef PIC_BLOCK_THREADS
#define PIC_BLOCK_THREADS 256
#endif
constexpr int kTileTokens = PIC_TILE_TOKENS;     // tokens of one entry per work tile
constexpr int kBlockThreads = PIC_BLOCK_THREADS; // wave64s per workgroup x 64

// Destination addressing of a plan.
enum DstMode : int32_t { kContiguous = 0, kPaged = 1, kInPlace = 2 };

// One work tile: tokens [tok0, tok0 + ntok) of entry `entry`.
struct DevTile {
    int32_t entry;
    int32_t tok0;
    int32_t ntok;
    int32_t pad;
};

// One placement as the kernel reads it.  src_tok is the pool row of the
// entry's token 0, dst_pos its logical position (in place: unused);
// cs_idx selects the shift table (-1 = delta 0, rows are copied).
struct DevEntry {
    int64_t src_tok;
    int64_t dst_pos;
    int32_t request;
    int32_t page_base;  // first entry of the request's page table (paged)
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
    int32_t nck, cph;   // K copy units per token / per head (non-rotary dims)
    int32_t nv, vph;    // V units per token / per head
};

struct Problem {
    pic_kv_shape shape{};
    int32_t rope_dim = 0;
    int32_t style = 0;
    int32_t mode = kContiguous;
    int32_t page_size = 0;
    int64_t capacity = 0;
    int64_t num_phys_pages = 0;
    int32_t n_requests = 0;
    Units u{};
    std::vector<DevEntry> entries;
    std::vector<DevTile> tiles;
    std::vector<double> cs;       // [table][rope_dim/2][cos, sin]
    std::vector<int32_t> pages;   // page tables, request after request
    std::vector<int64_t> bounds;  // [entry][request, begin, end]
    std::vector<int64_t> recompute;
    pic_plan_info_t info{};
};

// Everything the device needs, packed into one upload.
struct Staged {
    std::vector<uint8_t> bytes;
    size_t off_tiles = 0, off_entries = 0, off_cs = 0, off_pages = 0;
};

// Thread-local error reporting.
void clear_error();
pic_status fail(pic_status st, const char *fmt, ...);

// Shape/rope validation and work-unit derivation.
pic_status derive_units(const pic_kv_shape *shape, const pic_rope_config *rope, bool inplace,
                        Units *u);

// Copy-mode and in-place problem builders (host only).
pic_status build_stitch(const pic_kv_shape *shape, const pic_rope_config *rope,
                        const pic_chunk *chunks, int32_t n_chunks, const pic_request *requests,
                        int32_t n_requests, const pic_dst_geom *dst, Problem *out);
pic_status build_inplace(const pic_kv_shape *shape, const pic_rope_config *rope,
                         int64_t buf_tokens, const pic_segment *segments, int32_t n_segments,
                         Problem *out);

Staged stage(const Problem &p);

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
};
