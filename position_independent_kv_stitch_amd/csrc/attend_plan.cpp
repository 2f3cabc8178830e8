// attend_plan.cpp -- host side of pic_attend: the attention map of a plan.
// Every context position of a request is read either from the pool (tokens
// an entry writes: the chunk's row, turned by the entry's shift on load;
// Irminsul: MLA-Native Position-Independent Caching for Agentic LLM Serving,
// Technical Summary sections 2.2 and 4) or from the request's own cache
// (prefix, gaps, tokens left for recompute).  Runs of positions with
// consecutive rows in one source become tiles; tiles are grouped into work
// blocks.  The distance of a run from the last chunk start placed after
// position 0 drives the LegoLink damping (EPIC Guide: Position-Independent
// Caching for LLM Serving, "1. Identifying and Neutralizing Pseudo-Sinks").

#include <algorithm>
#include <cstring>

#include "pic_internal.hpp"

namespace pic {

// The pic_attend map of one request: positions [0, L) in order, each run of
// positions with one source (a chunk's written tokens: the pool, turned by
// the chunk's shift; anything else: the request's own cache) cut into tiles
// of consecutive rows that stop at pool and cache page ends and at chunk
// starts.
void build_attention_map(Problem *p, const pic_chunk *chunks, const pic_request &rq, int32_t r,
                         const std::vector<int32_t> &cs_of_entry, int32_t entry0) {
    std::vector<int32_t> order(rq.n_entries);
    for (int j = 0; j < rq.n_entries; j++) order[j] = j;
    std::sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
        return rq.entries[x].dst_offset < rq.entries[y].dst_offset;
    });
    int64_t L = rq.context_len;
    for (int j = 0; j < rq.n_entries; j++)
        if (rq.context_len == 0) L = std::max(L, rq.entries[j].dst_offset + rq.entries[j].length);
    p->context.push_back(L);

    const bool paged = p->mode == kPaged;
    const int32_t tile_begin = static_cast<int32_t>(p->atiles.size());
    int32_t bad_page = -1;  // a context page no stitch writes may be unmapped; attend checks
    int64_t last_start = -1;  // last chunk start after position 0
    // cut [lo, hi) of one source into tiles
    auto emit = [&](int64_t lo, int64_t hi, const pic_entry *e, const pic_chunk *ch, int32_t cs) {
        hi = std::min(hi, L);
        while (lo < hi) {
            int64_t n = std::min<int64_t>(kAttnTileTokens, hi - lo);
            AttnTile t{};
            t.cs_idx = -1;
            if (e) {  // pool rows of the chunk's tokens
                const int64_t at = ch->token_start + (lo - e->dst_offset);
                if (p->src_page_size > 0) {
                    const int64_t slot = at % p->src_page_size;
                    n = std::min<int64_t>(n, p->src_page_size - slot);
                    t.kind = kPoolPages;
                    t.a = ch->page_table[at / p->src_page_size];
                    t.b = static_cast<int32_t>(slot);
                } else {
                    t.kind = kPoolRows;
                    t.a = at;
                }
                t.cs_idx = cs;
            } else if (paged) {
                const int64_t slot = lo % p->page_size;
                n = std::min<int64_t>(n, p->page_size - slot);
                t.kind = kCachePages;
                t.a = rq.page_table[lo / p->page_size];
                t.b = static_cast<int32_t>(slot);
                if ((t.a < 0 || t.a >= p->num_phys_pages) && bad_page < 0)
                    bad_page = static_cast<int32_t>(lo / p->page_size);
            } else {
                t.kind = kCacheRows;
                t.a = r;
                t.b = static_cast<int32_t>(lo);
            }
            t.ntok = static_cast<int32_t>(n);
            t.sink_dist = last_start >= 0 ? static_cast<int32_t>(std::min<int64_t>(lo - last_start, kNoSink)) : kNoSink;
            p->atiles.push_back(t);
            lo += n;
        }
    };
    int64_t pos = 0;
    for (int32_t j : order) {
        const pic_entry &e = rq.entries[j];
        if (pos >= L) break;
        emit(pos, e.dst_offset, nullptr, nullptr, -1);  // gap before the chunk
        if (e.dst_offset > 0) last_start = e.dst_offset;
        emit(e.dst_offset, e.dst_offset + e.recompute_k, nullptr, nullptr, -1);  // recomputed
        emit(e.dst_offset + e.recompute_k, e.dst_offset + e.length, &e, &chunks[e.chunk_id],
             cs_of_entry[entry0 + j]);
        pos = e.dst_offset + e.length;
    }
    emit(pos, L, nullptr, nullptr, -1);
    p->context_bad_page.push_back(bad_page);
    p->req_tile0.push_back(tile_begin);
}

// Group every request's attention tiles into work blocks of whole tiles, at
// most `bt` positions and kAttnBlockTiles tiles each.  bt is the longest of
// 256, 128, 64 positions that still gives kAttnMinItems (block, KV head)
// work items, so that small batches are split finer.
void build_attention_blocks(Problem *p) {
    const int32_t n_req = static_cast<int32_t>(p->context.size());
    p->req_tile0.push_back(static_cast<int32_t>(p->atiles.size()));
    int64_t ctx_blocks_256 = 0;
    for (int64_t L : p->context) ctx_blocks_256 += (L + kAttnBlockTokens - 1) / kAttnBlockTokens;
    int32_t bt = kAttnBlockTokens;
    while (bt > kAttnTileTokens && ctx_blocks_256 * (kAttnBlockTokens / bt) *
                                           p->shape.num_heads < kAttnMinItems)
        bt /= 2;
    p->attn_block_tokens = bt;
    for (int32_t r = 0; r < n_req; r++) {
        p->req_block0.push_back(static_cast<int32_t>(p->ablocks.size()));
        int32_t t = p->req_tile0[r];
        const int32_t tile_end = p->req_tile0[r + 1];
        while (t < tile_end) {
            AttnBlock b{r, t, 0, 0};
            while (t < tile_end && b.ntiles < kAttnBlockTiles &&
                   b.ntok + p->atiles[t].ntok <= bt) {
                p->atiles[t].tok0 = b.ntok;
                b.ntok += p->atiles[t].ntok;
                b.ntiles++;
                t++;
            }
            p->ablocks.push_back(b);
        }
    }
    p->req_block0.push_back(static_cast<int32_t>(p->ablocks.size()));
}

// A map tile moved k positions on (its rows are consecutive in its source).
AttnTile advance_tile(AttnTile t, int32_t k) {
    if (t.kind == kPoolRows) t.a += k;
    else t.b += k;
    if (t.sink_dist < kNoSink)
        t.sink_dist = static_cast<int32_t>(std::min<int64_t>(int64_t{t.sink_dist} + k, kNoSink));
    t.ntok -= k;
    return t;
}

ItemMap build_item_map(const Problem &p, int64_t target, int64_t max_per_request) {
    std::vector<AttnTile> tiles;
    std::vector<AttnBlock> blocks;
    std::vector<int32_t> item0, req0;
    std::vector<int32_t> btabs;  // kItemBlockTabs per block
    int64_t total = 0;
    for (int64_t L : p.context) total += L;
    const int32_t n_req = static_cast<int32_t>(p.context.size());
    for (int32_t r = 0; r < n_req; r++) {
        req0.push_back(static_cast<int32_t>(item0.size()));
        const int64_t L = p.context[r];
        const int64_t n = std::min<int64_t>(
            max_per_request,
            std::max<int64_t>(1, (target * L + total / 2) / std::max<int64_t>(total, 1)));
        const int64_t S = (L + n - 1) / n;  // positions per item
        int64_t left = L, item_left = 0;
        AttnBlock blk{r, 0, 0, 0};
        std::vector<int32_t> tabs;  // the open block's shift tables
        auto close_block = [&]() {
            if (blk.ntiles > 0) {
                blocks.push_back(blk);
                for (int j = 0; j < kItemBlockTabs; j++)
                    btabs.push_back(j < static_cast<int>(tabs.size()) ? tabs[j] : -1);
            }
            blk = AttnBlock{r, static_cast<int32_t>(tiles.size()), 0, 0};
            tabs.clear();
        };
        for (int32_t t = p.req_tile0[r]; t < p.req_tile0[r + 1] && left > 0; t++) {
            AttnTile T = p.atiles[t];
            while (T.ntok > 0 && left > 0) {
                if (item_left == 0) {  // a new item starts here
                    close_block();
                    item0.push_back(static_cast<int32_t>(blocks.size()));
                    item_left = std::min(S, left);
                }
                const bool new_tab = T.cs_idx >= 0 &&
                                     std::find(tabs.begin(), tabs.end(), T.cs_idx) == tabs.end();
                if (blk.ntok == kItemBlockPos || blk.ntiles == kItemBlockTiles ||
                    (new_tab && static_cast<int>(tabs.size()) == kItemBlockTabs))
                    close_block();
                if (T.cs_idx >= 0 && std::find(tabs.begin(), tabs.end(), T.cs_idx) == tabs.end())
                    tabs.push_back(T.cs_idx);
                const int32_t take = static_cast<int32_t>(std::min<int64_t>(
                    {int64_t{T.ntok}, item_left, int64_t{kItemBlockPos - blk.ntok}}));
                AttnTile piece = T;
                piece.ntok = take;
                piece.tok0 = blk.ntok;
                tiles.push_back(piece);
                blk.ntiles++;
                blk.ntok += take;
                item_left -= take;
                left -= take;
                T = advance_tile(T, take);
                if (item_left == 0) close_block();
            }
        }
        close_block();
    }
    req0.push_back(static_cast<int32_t>(item0.size()));
    item0.push_back(static_cast<int32_t>(blocks.size()));
    ItemMap m;
    auto put = [&](const void *src, size_t n) {
        const size_t at = (m.bytes.size() + 15) & ~size_t{15};
        m.bytes.resize(at + n);
        if (n) std::memcpy(m.bytes.data() + at, src, n);
        return at;
    };
    put(tiles.data(), tiles.size() * sizeof(AttnTile));
    m.off_blocks = put(blocks.data(), blocks.size() * sizeof(AttnBlock));
    m.off_items = put(item0.data(), item0.size() * sizeof(int32_t));
    m.off_reqs = put(req0.data(), req0.size() * sizeof(int32_t));
    m.off_tabs = put(btabs.data(), btabs.size() * sizeof(int32_t));
    m.n_items = static_cast<int32_t>(item0.size()) - 1;
    m.n_blocks = static_cast<int32_t>(blocks.size());
    return m;
}

}  // namespace pic
