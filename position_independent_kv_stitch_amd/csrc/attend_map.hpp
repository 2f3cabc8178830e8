// attend_map.hpp -- the attention map of a plan: runs of context positions
// (tiles) grouped into work blocks, as the host planner builds them
// (attend_plan.cpp) and the attention kernels read them (attend.hip).
#pragma once

#include <cstdint>
#include <vector>

#include "pic_stitch.h"

namespace pic {

// pic_attend: a run of consecutive context positions of one request read from
// one source with consecutive rows.
enum AttnSrc : int32_t { kPoolRows = 0, kPoolPages = 1, kCacheRows = 2, kCachePages = 3 };
constexpr int kAttnTileTokens = 64;    // positions per attention tile at most
constexpr int kAttnBlockTokens = 256;  // positions per attention work item at most
constexpr int kAttnBlockTiles = 32;    // tiles per attention work item at most
constexpr int32_t kNoSink = 1 << 30;   // sink distance of runs not after a chunk start
#ifndef PIC_ATTN_MIN_ITEMS
#define PIC_ATTN_MIN_ITEMS 1024
#endif
// Work items (blocks x KV heads) below which the planner halves the block
// length, down to kAttnTileTokens positions, so that a launch fills the chip.
constexpr int64_t kAttnMinItems = PIC_ATTN_MIN_ITEMS;

struct AttnTile {
    int64_t a;          // pool row | pool page | request | destination page
    int32_t b;          // -      | pool slot | position | destination slot
    int32_t ntok;
    int32_t cs_idx;     // pool runs whose chunk moved: shift table; else -1
    int32_t kind;       // AttnSrc
    int32_t sink_dist;  // position of the first token minus the last chunk start (> 0 only)
    int32_t tok0;       // position of the first token within its block
};

struct AttnBlock {  // consecutive tiles [tile0, tile0 + ntiles) of one request
    int32_t request;
    int32_t tile0;
    int32_t ntiles;
    int32_t ntok;
};

struct Problem;

// Append request r's tiles (prefix, gaps, recompute tokens and trailing
// positions from the cache; placed chunk tokens from the pool) and its
// context length to the plan.  cs_of_entry holds the shift table of every
// entry of the plan; the request's entries start at entry0.
void build_attention_map(Problem *p, const pic_chunk *chunks, const pic_request &rq, int32_t r,
                         const std::vector<int32_t> &cs_of_entry, int32_t entry0);

// Group every request's tiles into work blocks (after the last request).
void build_attention_blocks(Problem *p);

// Work items of one launch of the latent and GQA tile kernels: request r gets
// a share of `target` items in proportion to its context (at least one, at
// most max_per_request), each of ceil(L / n) positions cut from its map tiles
// (tiles split where an item ends), stored as blocks of at most
// kItemBlockPos positions, kItemBlockTiles tiles and kItemBlockTabs shift
// tables.  Packed as [tiles][blocks][item -> first block (+ end)]
// [request -> first item (+ end)][block -> its shift tables, -1 padded].
constexpr int kItemBlockPos = 4096;
constexpr int kItemBlockTiles = 64;
constexpr int kItemBlockTabs = 4;
struct ItemMap {
    std::vector<uint8_t> bytes;
    size_t off_blocks = 0, off_items = 0, off_reqs = 0, off_tabs = 0;
    int32_t n_items = 0, n_blocks = 0;
};
ItemMap build_item_map(const Problem &p, int64_t target, int64_t max_per_request);

// A map tile moved k positions on (its rows are consecutive in its source).
AttnTile advance_tile(AttnTile t, int32_t k);

}  // namespace pic
