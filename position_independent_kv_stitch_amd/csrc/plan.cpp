// plan.cpp -- host planner of the stitch library: validation, per-entry
// shifts and fp64 cos/sin tables, work tiles, boundary and recompute
// ranges.  No HIP call is made here, so plans can be built and inspected
// without a GPU.
//
// The shift of a placed chunk is delta = p_target - p_source (Irminsul:
// MLA-Native Position-Independent Caching for Agentic LLM Serving,
// Technical Summary section 2.2); the composer computes it for every hit
// chunk (EPIC Guide: Position-Independent Caching for LLM Serving,
// "Modular Prompt Composer").  Because 2-D rotations compose by adding
// angles (EPIC Guide, "The In-Place Shift Transformation"), one table of
// cos/sin(delta * theta_i) per distinct delta serves every token of the
// chunk, with theta_i = b^(-2i/d) ("RoPE Mathematical Structure").

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <unordered_map>

#include "pic_internal.hpp"

namespace pic {

namespace {
thread_local std::string g_error;

constexpr int64_t kMaxPosition = INT32_MAX;  // positions and in-chunk offsets fit int32
constexpr int64_t kMaxBase = int64_t{1} << 62;  // |base_pos|: delta = dst - base_pos fits int64
}  // namespace

void clear_error() { g_error.clear(); }

pic_status fail(pic_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return st;
}

pic_status derive_units(const pic_kv_shape *shape, const pic_rope_config *rope, bool inplace,
                        Units *u) {
    if (!shape || !rope) return fail(PIC_ERR_INVALID_ARG, "shape and rope must not be NULL");
    if (shape->dtype != PIC_DTYPE_F32 && shape->dtype != PIC_DTYPE_BF16)
        return fail(PIC_ERR_INVALID_ARG, "unknown dtype %d", shape->dtype);
    if (rope->style != PIC_ROPE_HALF && rope->style != PIC_ROPE_INTERLEAVED)
        return fail(PIC_ERR_INVALID_ARG, "unknown rope style %d", rope->style);
    if (shape->num_layers < 1 || shape->num_heads < 1 || shape->row_dim < 1)
        return fail(PIC_ERR_INVALID_ARG, "num_layers, num_heads and row_dim must be >= 1");
    if (rope->rope_dim < 2 || rope->rope_dim % 2 != 0)
        return fail(PIC_ERR_INVALID_ARG, "rope_dim %d must be even and >= 2", rope->rope_dim);
    if (shape->rope_offset < 0 || shape->rope_offset + rope->rope_dim > shape->row_dim)
        return fail(PIC_ERR_INVALID_ARG, "rotary slice [%d, %d) outside a row of %d",
                    shape->rope_offset, shape->rope_offset + rope->rope_dim, shape->row_dim);
    if (rope->inv_freq) {
        for (int i = 0; i < rope->rope_dim / 2; i++)
            if (!std::isfinite(rope->inv_freq[i]))
                return fail(PIC_ERR_INVALID_ARG, "inv_freq[%d] is not finite", i);
    } else if (!(rope->theta > 0.0) || !std::isfinite(rope->theta)) {
        return fail(PIC_ERR_INVALID_ARG, "theta must be finite and > 0");
    }
    if (shape->has_v != 0 && shape->has_v != 1)
        return fail(PIC_ERR_INVALID_ARG, "has_v must be 0 or 1");

    const int es = shape->dtype == PIC_DTYPE_F32 ? 4 : 2;
    const int vec = 16 / es;
    const int half_r = rope->rope_dim / 2;
    if (shape->row_dim % vec || shape->rope_offset % vec)
        return fail(PIC_ERR_ALIGN, "row_dim and rope_offset must be multiples of %d", vec);
    int uph, ncs;
    if (rope->style == PIC_ROPE_HALF) {
        if (half_r % vec)
            return fail(PIC_ERR_ALIGN, "rope_dim/2 must be a multiple of %d (half pairing)", vec);
        uph = half_r / vec;
        ncs = vec;
    } else {
        if (rope->rope_dim % vec)
            return fail(PIC_ERR_ALIGN, "rope_dim must be a multiple of %d (interleaved)", vec);
        uph = rope->rope_dim / vec;
        ncs = vec / 2;
    }
    if (uph > 64 || (64 % uph) != 0)
        return fail(PIC_ERR_ALIGN, "rotary slice of %d 16-byte units per head: need a power "
                    "of two <= 64", uph);
    u->vec = vec;
    u->half_r = half_r;
    u->uph = uph;
    u->uph_shift = 0;
    while ((1 << u->uph_shift) < uph) u->uph_shift++;
    u->ncs = ncs;
    u->interleaved = rope->style == PIC_ROPE_INTERLEAVED ? 1 : 0;
    u->nr = shape->num_heads * uph;
    u->cph = (shape->row_dim - rope->rope_dim) / vec;
    u->vph = shape->row_dim / vec;
    u->nck = inplace ? 0 : shape->num_heads * u->cph;
    u->nv = (inplace || !shape->has_v) ? 0 : shape->num_heads * u->vph;
    return PIC_OK;
}

// A wave step takes g consecutive tokens of a tile and deals their rotary
// units (g * nr) and copy units (g * (nck + nv)) to its 64 lanes, MAXR and
// MAXC per lane.  Rows with few copy units (MLA: 4 rotary + 64 copy units
// in bf16) take the wider copy shape, so one step spans several tokens and
// every lane still has several 16-byte words in flight.
Launch launch_shape_of(int32_t dtype, const Units &u) {
    Launch l;
    const int ncv = u.nck + u.nv;
    if (dtype == PIC_DTYPE_BF16) {
        l.maxr = 1;
        l.maxc = (ncv > 0 && ncv <= 64) ? 4 : 2;
    } else {
        l.maxr = u.nr <= 64 ? 1 : 2;
        l.maxc = 4;
    }
    auto tokens_per_step = [&](int nr) {
        int g = (64 * l.maxr) / nr;
        if (ncv > 0) g = std::min(g, (64 * l.maxc) / ncv);
        return std::max(1, std::min(g, 8));
    };
    l.rb = 16;
    l.nr = u.nr;
    l.uph_shift = u.uph_shift;
    l.g = tokens_per_step(l.nr);
    // A step that leaves lanes without rotary work (narrow rotary slices, as
    // in MLA rows) deals its planes in 4-byte words instead: four times the
    // units, a quarter of the fp64 work per lane.  Half pairing only: a
    // 4-byte word of an interleaved f32 row would hold half a plane.
    if (l.g * u.nr < 64 && u.uph <= 16 && u.interleaved == 0) {
        l.rb = 4;
        l.nr = u.nr * 4;
        l.uph_shift = u.uph_shift + 2;
        l.g = tokens_per_step(l.nr);
    }
    const int rb = (l.g * l.nr + 64 * l.maxr - 1) / (64 * l.maxr);
    const int cb = (l.g * ncv + 64 * l.maxc - 1) / (64 * l.maxc);
    l.nblk = std::max(rb, cb);
    return l;
}

namespace {

// Waves per tile.  A tile holds at most tile_tokens tokens and never crosses
// a page of a paged destination or pool (page_bound, 0 for none).  With
// narrow rows a wave step spans several tokens, and one or two waves' steps
// then cover the longest tile the plan can have: a workgroup of four waves
// takes 4 / wpt tiles, each wave every step of its share, instead of one
// tile whose page leaves most of its waves' steps empty.
void set_tile_waves(Problem *p, int64_t page_bound) {
    const int64_t per_wave = int64_t{kTileSteps} * p->launch.g;
    const int64_t longest =
        page_bound > 0 ? std::min<int64_t>(p->tile_tokens, page_bound) : p->tile_tokens;
    p->launch.wpt = longest <= per_wave ? 1 : longest <= 2 * per_wave ? 2 : 4;
    p->tile_tokens = static_cast<int32_t>(std::min<int64_t>(p->tile_tokens, p->launch.wpt * per_wave));
}

// theta_i = b^(-2i/d) for i < rope_dim/2 in fp64 (libm), or the caller's table.
std::vector<double> plane_frequencies(const pic_rope_config &rope) {
    const int half_r = rope.rope_dim / 2;
    std::vector<double> f(static_cast<size_t>(half_r));
    for (int i = 0; i < half_r; i++)
        f[i] = rope.inv_freq ? rope.inv_freq[i]
                             : std::pow(rope.theta, -(2.0 * i) / static_cast<double>(rope.rope_dim));
    return f;
}

// cos/sin of delta * theta_i for every plane i, in fp64 (libm), appended to cs.
void append_shift_table(const std::vector<double> &freq, int64_t delta, std::vector<double> &cs) {
    const size_t at = cs.size();
    cs.resize(at + 2 * freq.size());
    double *out = cs.data() + at;
    for (size_t i = 0; i < freq.size(); i++) {
        const double phi = static_cast<double>(delta) * freq[i];
        sincos(phi, &out[2 * i + 1], &out[2 * i]);
    }
}

struct Interval {
    int64_t key;  // sort key (physical page or request)
    int64_t lo, hi;
};

bool any_overlap(std::vector<Interval> &v) {
    std::sort(v.begin(), v.end(), [](const Interval &a, const Interval &b) {
        return a.key != b.key ? a.key < b.key : a.lo < b.lo;
    });
    for (size_t i = 1; i < v.size(); i++)
        if (v[i].key == v[i - 1].key && v[i].lo < v[i - 1].hi) return true;
    return false;
}

// Claims on the slots of a pool of pages (a flat range of rows is one page),
// for the checks that no slot is written twice or read twice.  A bit per
// slot while the pool is not much larger than the claimed slots (about 1.5 M
// bits for the batched-RAG destination), else the claimed runs, sorted once.
class SlotClaims {
  public:
    SlotClaims(int64_t n_pages, int64_t page_size, int64_t expected_slots) : ps_(page_size) {
        constexpr int64_t kMaxBits = int64_t{1} << 30;
        use_bits_ = page_size > 0 && n_pages >= 0 && n_pages <= kMaxBits / page_size &&
                    n_pages * page_size <= 64 * expected_slots + (int64_t{1} << 22);
        if (use_bits_) words_.assign(static_cast<size_t>((n_pages * page_size + 63) / 64), 0);
    }
    void claim(int64_t page, int64_t lo, int64_t hi) {
        if (!use_bits_) {
            runs_.push_back(Interval{page, lo, hi});
            return;
        }
        int64_t a = page * ps_ + lo;
        const int64_t b = page * ps_ + hi;
        while (a < b) {
            const int sh = static_cast<int>(a & 63);
            const int64_t n = std::min<int64_t>(64 - sh, b - a);
            const uint64_t m = (n == 64 ? ~uint64_t{0} : ((uint64_t{1} << n) - 1)) << sh;
            uint64_t &w = words_[static_cast<size_t>(a >> 6)];
            clash_ |= (w & m) != 0;
            w |= m;
            a += n;
        }
    }
    bool overlap() { return use_bits_ ? clash_ : any_overlap(runs_); }

  private:
    int64_t ps_;
    bool use_bits_ = false, clash_ = false;
    std::vector<uint64_t> words_;
    std::vector<Interval> runs_;
};

void fill_info(Problem *p, int64_t tokens_written, int64_t tokens_masked, int64_t pool_need) {
    const int64_t es = p->shape.dtype == PIC_DTYPE_F32 ? 4 : 2;
    int64_t per_token;
    if (p->mode == kInPlace)
        per_token = static_cast<int64_t>(p->shape.num_heads) * p->rope_dim * es;
    else
        per_token = static_cast<int64_t>(p->shape.num_heads) * p->shape.row_dim * es *
                    (1 + p->shape.has_v);
    p->info.n_requests = p->n_requests;
    p->info.n_entries = static_cast<int64_t>(p->entries.size());
    p->info.n_tiles = static_cast<int64_t>(p->tiles.size());
    p->info.tokens_written = tokens_written;
    p->info.tokens_masked = tokens_masked;
    p->info.pool_tokens_required = pool_need;
    p->info.bytes_read_per_layer = tokens_written * per_token;
    p->info.bytes_written_per_layer = tokens_written * per_token;
    p->info.tile_tokens = p->tile_tokens;
}

// Launch order of a copy plan whose pool rows are read more than once (a
// chunk placed into several requests).  In request order, the next read of a
// repeated chunk lies a whole layer of traffic later, far past any cache.
// Instead, the tiles of every placement of one chunk are merged by their
// first token in the chunk, so that tiles reading the same rows are launched
// together, and each chunk's merged run goes to one of eight queues (the
// shortest so far) that are then interleaved: workgroup w of a launch runs on
// XCD w % 8 (the same offset for every layer of a launch), so the placements
// of a chunk share that XCD's L2 and all but the first read of a row hit it.
// Tiles write disjoint rows, so the order changes no result.  ent_tile0[e]
// is entry e's first tile (its tiles run to the next entry's first).
constexpr int kXcds = 8;

void order_tiles_by_source(Problem *p, int n_chunks, const std::vector<int32_t> &ent_chunk,
                           const std::vector<int32_t> &ent_tile0,
                           const std::vector<int32_t> &tile_off) {
    const int32_t n_ent = static_cast<int32_t>(ent_chunk.size());
    const int32_t n_tiles = static_cast<int32_t>(p->tiles.size());
    if (n_ent < 2) return;
    // entries grouped by chunk, chunks in the order of their first placement
    std::vector<int32_t> first(static_cast<size_t>(n_chunks), -1), last(static_cast<size_t>(n_chunks), -1),
        next(static_cast<size_t>(n_ent), -1), chunk_order;
    for (int32_t e = 0; e < n_ent; e++) {
        const int32_t c = ent_chunk[e];
        if (first[c] < 0) {
            first[c] = e;
            chunk_order.push_back(c);
        } else {
            next[last[c]] = e;
        }
        last[c] = e;
    }
    auto tile_end = [&](int32_t e) { return e + 1 < n_ent ? ent_tile0[e + 1] : n_tiles; };
    // each queue a list of tile indices
    std::vector<std::vector<int32_t>> queue(kXcds);
    for (auto &q : queue) q.reserve(static_cast<size_t>(n_tiles / kXcds + 1));
    std::vector<int32_t> cur, end;
    for (int32_t c : chunk_order) {
        size_t j = 0;
        for (size_t m = 1; m < queue.size(); m++)
            if (queue[m].size() < queue[j].size()) j = m;
        std::vector<int32_t> &q = queue[j];
        if (next[first[c]] < 0) {  // placed once
            for (int32_t t = ent_tile0[first[c]]; t < tile_end(first[c]); t++) q.push_back(t);
            continue;
        }
        cur.clear();
        end.clear();
        for (int32_t e = first[c]; e >= 0; e = next[e]) {
            cur.push_back(ent_tile0[e]);
            end.push_back(tile_end(e));
        }
        // k-way merge by first token (k: the chunk's placements, a few)
        for (;;) {
            int best = -1;
            for (size_t k = 0; k < cur.size(); k++)
                if (cur[k] < end[k] && (best < 0 || tile_off[cur[k]] < tile_off[cur[best]]))
                    best = static_cast<int>(k);
            if (best < 0) break;
            q.push_back(cur[best]++);
        }
    }
    // a workgroup takes `group` consecutive tiles, so each queue contributes
    // that many at a time
    const size_t group = static_cast<size_t>((kBlockThreads / 64) / p->launch.wpt);
    std::vector<DevTile> out;
    out.reserve(p->tiles.size());
    for (size_t i = 0; out.size() < p->tiles.size(); i += group)
        for (const auto &q : queue)
            for (size_t k = i; k < i + group && k < q.size(); k++) out.push_back(p->tiles[q[k]]);
    p->tiles.swap(out);
}

// Tiles of tokens [from, to) of one placement: at most tile_tokens tokens,
// and never across a page of a paged destination or a paged pool, so each
// tile has one source and one destination row base with consecutive rows
// after them.
void add_tiles(Problem *p, const HostEntry &e, const int32_t *dst_pages, const int32_t *src_pages,
               int32_t from, int32_t to, std::vector<int32_t> *offs = nullptr) {
    if (from >= to) return;
    const int64_t sps = p->src_page_size, ps = p->page_size;
    // page and slot of the first token, then advanced tile by tile
    int64_t s_pg = 0, d_pg = 0;
    int32_t s_slot = 0, d_slot = 0;
    if (src_pages) {
        s_pg = (e.src_tok + from) / sps;
        s_slot = static_cast<int32_t>((e.src_tok + from) % sps);
    }
    if (p->mode == kPaged) {
        d_pg = (e.dst_pos + from) / ps;
        d_slot = static_cast<int32_t>((e.dst_pos + from) % ps);
    }
    for (int32_t t = from; t < to;) {
        int32_t n = std::min(p->tile_tokens, to - t);
        DevTile tile{e.src_tok + t, 0, 0, 0, e.cs_idx, 0};
        if (src_pages) {
            n = std::min<int32_t>(n, static_cast<int32_t>(sps) - s_slot);
            tile.src_row = src_pages[s_pg];
            tile.src_slot = s_slot;
        }
        if (p->mode == kPaged) {
            n = std::min<int32_t>(n, static_cast<int32_t>(ps) - d_slot);
            tile.dst_a = dst_pages[d_pg];
            tile.dst_b = d_slot;
        } else if (p->mode == kContiguous) {
            tile.dst_a = e.request;
            tile.dst_b = static_cast<int32_t>(e.dst_pos + t);
        }
        tile.ntok = n;
        p->tiles.push_back(tile);
        if (offs) offs->push_back(t);
        t += n;
        if (src_pages && (s_slot += n) == sps) {
            s_slot = 0;
            s_pg++;
        }
        if (p->mode == kPaged && (d_slot += n) == ps) {
            d_slot = 0;
            d_pg++;
        }
    }
}


}  // namespace

pic_status build_stitch(const pic_kv_shape *shape, const pic_rope_config *rope,
                        const pic_chunk *chunks, int32_t n_chunks, const pic_request *requests,
                        int32_t n_requests, const pic_geom *geom, Problem *out) {
    Units u{};
    pic_status st = derive_units(shape, rope, false, &u);
    if (st) return st;
    if (!geom) return fail(PIC_ERR_INVALID_ARG, "geometry must not be NULL");
    if (n_chunks < 0 || n_requests < 0)
        return fail(PIC_ERR_INVALID_ARG, "negative chunk or request count");
    if ((n_chunks > 0 && !chunks) || (n_requests > 0 && !requests))
        return fail(PIC_ERR_INVALID_ARG, "chunk or request array is NULL");
    if (geom->dst_page_size < 0 || geom->src_page_size < 0)
        return fail(PIC_ERR_INVALID_ARG, "negative page size");
    const bool paged = geom->dst_page_size > 0;
    const bool src_paged = geom->src_page_size > 0;
    if (!paged && geom->dst_capacity < 0) return fail(PIC_ERR_INVALID_ARG, "negative capacity");
    if (paged && geom->dst_num_pages < 0)
        return fail(PIC_ERR_INVALID_ARG, "negative destination page count");
    if (src_paged && geom->src_num_pages < 0)
        return fail(PIC_ERR_INVALID_ARG, "negative pool page count");
    for (int r = 0; r < n_requests; r++) {
        const pic_request &rq = requests[r];
        if (rq.n_entries < 0 || (rq.n_entries > 0 && !rq.entries))
            return fail(PIC_ERR_INVALID_ARG, "request %d: bad entry array", r);
        if (paged && (rq.n_pages < 0 || (rq.n_pages > 0 && !rq.page_table)))
            return fail(PIC_ERR_INVALID_ARG, "request %d: bad page table", r);
    }
    if (src_paged)
        for (int c = 0; c < n_chunks; c++)
            if (chunks[c].n_pages < 0 || (chunks[c].n_pages > 0 && !chunks[c].page_table))
                return fail(PIC_ERR_INVALID_ARG, "chunk %d: bad page table", c);

    // ranges
    const int64_t sps = geom->src_page_size;
    int64_t pool_need = src_paged ? geom->src_num_pages * sps : 0;
    for (int c = 0; c < n_chunks; c++) {
        const pic_chunk &ch = chunks[c];
        if (ch.token_start < 0 || ch.length < 1 ||
            (src_paged && ch.token_start + ch.length > static_cast<int64_t>(ch.n_pages) * sps))
            return fail(PIC_ERR_RANGE, "chunk %d: tokens [%lld, %lld)", c,
                        static_cast<long long>(ch.token_start),
                        static_cast<long long>(ch.token_start + ch.length));
        if (ch.base_pos < -kMaxBase || ch.base_pos > kMaxBase)
            return fail(PIC_ERR_RANGE, "chunk %d: base_pos %lld outside [-2^62, 2^62]", c,
                        static_cast<long long>(ch.base_pos));
        if (!src_paged) pool_need = std::max(pool_need, ch.token_start + ch.length);
    }
    for (int r = 0; r < n_requests; r++) {
        const pic_request &rq = requests[r];
        const int64_t span =
            paged ? static_cast<int64_t>(rq.n_pages) * geom->dst_page_size : geom->dst_capacity;
        for (int j = 0; j < rq.n_entries; j++) {
            const pic_entry &e = rq.entries[j];
            if (e.reserved != 0) return fail(PIC_ERR_RANGE, "request %d entry %d: reserved", r, j);
            if (e.chunk_id < 0 || e.chunk_id >= n_chunks)
                return fail(PIC_ERR_RANGE, "request %d entry %d: chunk_id %d", r, j, e.chunk_id);
            const pic_chunk &ch = chunks[e.chunk_id];
            if (e.length < 1 || e.length > ch.length)
                return fail(PIC_ERR_RANGE, "request %d entry %d: length %d of a %d-token chunk", r,
                            j, e.length, ch.length);
            if (e.recompute_k < 0 || e.recompute_k > e.length)
                return fail(PIC_ERR_RANGE, "request %d entry %d: recompute_k %d", r, j,
                            e.recompute_k);
            if (e.dst_offset < 0 || e.dst_offset + e.length > span ||
                e.dst_offset + e.length > kMaxPosition)
                return fail(PIC_ERR_RANGE, "request %d entry %d: positions [%lld, %lld) outside "
                            "[0, %lld)", r, j, static_cast<long long>(e.dst_offset),
                            static_cast<long long>(e.dst_offset + e.length),
                            static_cast<long long>(span));
            if (e.recompute_k == e.length) continue;  // nothing read or written
            if (paged) {
                const int64_t p0 = (e.dst_offset + e.recompute_k) / geom->dst_page_size;
                const int64_t p1 = (e.dst_offset + e.length - 1) / geom->dst_page_size;
                for (int64_t pg = p0; pg <= p1; pg++) {
                    const int32_t phys = rq.page_table[pg];
                    if (phys < 0 || phys >= geom->dst_num_pages)
                        return fail(PIC_ERR_RANGE, "request %d: logical page %lld maps to %d "
                                    "(destination has %lld)", r, static_cast<long long>(pg),
                                    phys, static_cast<long long>(geom->dst_num_pages));
                }
            }
            if (src_paged) {
                const int64_t p0 = (ch.token_start + e.recompute_k) / sps;
                const int64_t p1 = (ch.token_start + e.length - 1) / sps;
                for (int64_t pg = p0; pg <= p1; pg++) {
                    const int32_t phys = ch.page_table[pg];
                    if (phys < 0 || phys >= geom->src_num_pages)
                        return fail(PIC_ERR_RANGE, "chunk %d: page %lld maps to %d (pool has "
                                    "%lld)", e.chunk_id, static_cast<long long>(pg), phys,
                                    static_cast<long long>(geom->src_num_pages));
                }
            }
        }
    }

    for (int r = 0; r < n_requests; r++) {
        const pic_request &rq = requests[r];
        const int64_t span =
            paged ? static_cast<int64_t>(rq.n_pages) * geom->dst_page_size : geom->dst_capacity;
        if (rq.context_len < 0 || rq.context_len > span || rq.context_len > kMaxPosition)
            return fail(PIC_ERR_RANGE, "request %d: context_len %lld outside [0, %lld]", r,
                        static_cast<long long>(rq.context_len), static_cast<long long>(span));
    }

    // overlaps: whole entry intervals inside a request, then written rows
    {
        std::vector<Interval> iv;
        for (int r = 0; r < n_requests; r++)
            for (int j = 0; j < requests[r].n_entries; j++) {
                const pic_entry &e = requests[r].entries[j];
                iv.push_back(Interval{r, e.dst_offset, e.dst_offset + e.length});
            }
        if (any_overlap(iv)) return fail(PIC_ERR_OVERLAP, "entries of a request overlap");
    }
    int64_t to_write = 0;  // tokens every entry writes, summed
    for (int r = 0; r < n_requests; r++)
        for (int j = 0; j < requests[r].n_entries; j++)
            to_write += requests[r].entries[j].length - requests[r].entries[j].recompute_k;
    if (paged) {
        const int64_t ps = geom->dst_page_size;
        SlotClaims claims(geom->dst_num_pages, ps, to_write);
        for (int r = 0; r < n_requests; r++)
            for (int j = 0; j < requests[r].n_entries; j++) {
                const pic_entry &e = requests[r].entries[j];
                int64_t pos = e.dst_offset + e.recompute_k;
                const int64_t end = e.dst_offset + e.length;
                while (pos < end) {
                    const int64_t lp = pos / ps, slot = pos % ps;
                    const int64_t run = std::min(ps - slot, end - pos);
                    claims.claim(requests[r].page_table[lp], slot, slot + run);
                    pos += run;
                }
            }
        if (claims.overlap())
            return fail(PIC_ERR_OVERLAP, "two placements write the same physical row");
    }

    // the plan
    Problem &p = *out;
    p.shape = *shape;
    p.rope_dim = rope->rope_dim;
    p.style = rope->style;
    p.mode = paged ? kPaged : kContiguous;
    p.page_size = geom->dst_page_size;
    p.capacity = geom->dst_capacity;
    p.num_phys_pages = geom->dst_num_pages;
    p.src_page_size = geom->src_page_size;
    p.n_requests = n_requests;
    p.u = u;
    p.launch = launch_shape_of(shape->dtype, u);
    p.tile_tokens = kTileSteps * 4 * p.launch.g;
    {
        int64_t bound = paged ? geom->dst_page_size : 0;
        if (src_paged) bound = bound > 0 ? std::min<int64_t>(bound, sps) : sps;
        set_tile_waves(&p, bound);
    }
    {
        // Pool rows read more than once per layer (a chunk placed twice, or
        // chunks sharing rows) may be served from cache on the second read;
        // only a plan that reads every row once streams its loads.
        std::vector<Interval> iv;  // contiguous pool: one run per entry
        SlotClaims claims(src_paged ? geom->src_num_pages : 0, src_paged ? sps : 1, to_write);
        for (int r = 0; r < n_requests; r++)
            for (int j = 0; j < requests[r].n_entries; j++) {
                const pic_entry &e = requests[r].entries[j];
                const pic_chunk &ch = chunks[e.chunk_id];
                int64_t t = ch.token_start + e.recompute_k;
                const int64_t end = ch.token_start + e.length;
                if (t < end && !src_paged) iv.push_back(Interval{0, t, end});
                while (src_paged && t < end) {
                    const int64_t slot = t % sps;
                    const int64_t run = std::min(sps - slot, end - t);
                    claims.claim(ch.page_table[t / sps], slot, slot + run);
                    t += run;
                }
            }
        p.launch.stream_loads = (src_paged ? claims.overlap() : any_overlap(iv)) ? 0 : 1;
    }
    {
        // tiles end at tile_tokens and at destination and pool page ends
        int64_t bound = 0;
        for (int r = 0; r < n_requests; r++)
            for (int j = 0; j < requests[r].n_entries; j++) {
                const int64_t n = requests[r].entries[j].length - requests[r].entries[j].recompute_k;
                if (n <= 0) continue;
                bound += n / p.tile_tokens + 1;
                if (paged) bound += n / geom->dst_page_size + 1;
                if (src_paged) bound += n / sps + 1;
            }
        p.tiles.reserve(static_cast<size_t>(bound));
    }
    const std::vector<double> freq = plane_frequencies(*rope);
    std::unordered_map<int64_t, int32_t> table_of_delta;
    std::vector<int32_t> cs_of_entry;
    int64_t written = 0, masked = 0;
    // chunk-relative first token of every tile, and every entry's tiles, for
    // the launch order below
    std::vector<int32_t> tile_off;
    std::vector<int32_t> ent_chunk, ent_tile0;
    const bool reorder = p.launch.stream_loads == 0;
    if (reorder) tile_off.reserve(p.tiles.capacity());
    for (int r = 0; r < n_requests; r++) {
        const pic_request &rq = requests[r];
        for (int j = 0; j < rq.n_entries; j++) {
            const pic_entry &e = rq.entries[j];
            const pic_chunk &c = chunks[e.chunk_id];
            const int64_t delta = e.dst_offset - c.base_pos;
            int32_t cs_idx = -1;
            if (delta != 0) {
                auto it = table_of_delta.find(delta);
                if (it == table_of_delta.end()) {
                    cs_idx = static_cast<int32_t>(table_of_delta.size());
                    table_of_delta.emplace(delta, cs_idx);
                    append_shift_table(freq, delta, p.cs);
                } else {
                    cs_idx = it->second;
                }
            }
            const HostEntry he{c.token_start, e.dst_offset, r, 0, cs_idx, 0};
            p.entries.push_back(he);
            cs_of_entry.push_back(cs_idx);
            if (reorder) {
                ent_chunk.push_back(e.chunk_id);
                ent_tile0.push_back(static_cast<int32_t>(p.tiles.size()));
            }
            add_tiles(&p, he, paged ? rq.page_table : nullptr,
                      src_paged ? c.page_table : nullptr, e.recompute_k, e.length,
                      reorder ? &tile_off : nullptr);
            p.bounds.insert(p.bounds.end(), {r, e.dst_offset, e.dst_offset + e.length});
            p.recompute.insert(p.recompute.end(), {r, e.dst_offset, e.dst_offset + e.recompute_k});
            written += e.length - e.recompute_k;
            masked += e.recompute_k;
        }
    }
    if (reorder) order_tiles_by_source(&p, n_chunks, ent_chunk, ent_tile0, tile_off);
    int64_t context_tokens = 0;
    for (int r = 0; r < n_requests; r++) {
        const pic_request &rq = requests[r];
        int64_t L = rq.context_len;
        for (int j = 0; j < rq.n_entries && rq.context_len == 0; j++)
            L = std::max(L, rq.entries[j].dst_offset + rq.entries[j].length);
        context_tokens += L;
    }
    // copies of what the attention map is built from, when a call needs it
    AttnSource &as = p.attn_src;
    as.cs_of_entry = std::move(cs_of_entry);
    as.chunks.assign(chunks, chunks + n_chunks);
    if (src_paged) {
        size_t n = 0;
        for (int c = 0; c < n_chunks; c++) n += static_cast<size_t>(chunks[c].n_pages);
        as.chunk_pages.reserve(n);
        for (int c = 0; c < n_chunks; c++)
            as.chunk_pages.insert(as.chunk_pages.end(), chunks[c].page_table,
                                  chunks[c].page_table + chunks[c].n_pages);
    }
    {
        size_t ne = 0, np = 0;
        for (int r = 0; r < n_requests; r++) {
            ne += static_cast<size_t>(requests[r].n_entries);
            if (paged) np += static_cast<size_t>(requests[r].n_pages);
        }
        as.entries.reserve(ne);
        as.req_pages.reserve(np);
        for (int r = 0; r < n_requests; r++) {
            as.entries.insert(as.entries.end(), requests[r].entries,
                              requests[r].entries + requests[r].n_entries);
            if (paged)
                as.req_pages.insert(as.req_pages.end(), requests[r].page_table,
                                    requests[r].page_table + requests[r].n_pages);
        }
    }
    size_t at = 0;
    for (int c = 0; c < n_chunks; c++) {
        as.chunks[c].page_table = src_paged ? as.chunk_pages.data() + at : nullptr;
        if (src_paged) at += static_cast<size_t>(chunks[c].n_pages);
    }
    as.requests.assign(requests, requests + n_requests);
    size_t e0 = 0, p0 = 0;
    for (int r = 0; r < n_requests; r++) {
        as.requests[r].entries = as.entries.data() + e0;
        as.requests[r].page_table = paged ? as.req_pages.data() + p0 : nullptr;
        e0 += static_cast<size_t>(requests[r].n_entries);
        if (paged) p0 += static_cast<size_t>(requests[r].n_pages);
    }
    fill_info(&p, written, masked, pool_need);
    p.info.context_tokens = context_tokens;
    return PIC_OK;
}

void build_attention(Problem *p) {
    const AttnSource &as = p->attn_src;
    int32_t entry0 = 0;
    for (size_t r = 0; r < as.requests.size(); r++) {
        build_attention_map(p, as.chunks.data(), as.requests[r], static_cast<int32_t>(r),
                            as.cs_of_entry, entry0);
        entry0 += as.requests[r].n_entries;
    }
    build_attention_blocks(p);
    p->info.attend_blocks = static_cast<int64_t>(p->ablocks.size());
    p->info.attend_block_tokens = p->attn_block_tokens;
    p->attn_built = true;
}

pic_status build_inplace(const pic_kv_shape *shape, const pic_rope_config *rope,
                         int64_t buf_tokens, const pic_segment *segments, int32_t n_segments,
                         Problem *out) {
    Units u{};
    pic_status st = derive_units(shape, rope, true, &u);
    if (st) return st;
    if (buf_tokens < 0 || n_segments < 0 || (n_segments > 0 && !segments))
        return fail(PIC_ERR_INVALID_ARG, "bad buffer length or segment array");
    for (int g = 0; g < n_segments; g++) {
        const pic_segment &s = segments[g];
        if (s.token_start < 0 || s.length < 1 || s.token_start + s.length > buf_tokens)
            return fail(PIC_ERR_RANGE, "segment %d: tokens [%lld, %lld) outside [0, %lld)", g,
                        static_cast<long long>(s.token_start),
                        static_cast<long long>(s.token_start + s.length),
                        static_cast<long long>(buf_tokens));
        if (s.recompute_k < 0 || s.recompute_k > s.length)
            return fail(PIC_ERR_RANGE, "segment %d: recompute_k %d", g, s.recompute_k);
    }
    {
        std::vector<Interval> iv;
        for (int g = 0; g < n_segments; g++)
            iv.push_back(Interval{0, segments[g].token_start,
                                  segments[g].token_start + segments[g].length});
        if (any_overlap(iv)) return fail(PIC_ERR_OVERLAP, "segments overlap");
    }
    Problem &p = *out;
    p.shape = *shape;
    p.shape.has_v = 0;
    p.rope_dim = rope->rope_dim;
    p.style = rope->style;
    p.mode = kInPlace;
    p.capacity = buf_tokens;
    p.n_requests = 1;
    p.u = u;
    p.launch = launch_shape_of(shape->dtype, u);
    p.tile_tokens = kTileSteps * 4 * p.launch.g;
    p.launch.stream_loads = 1;  // segments never overlap: every row is read once
    const std::vector<double> freq = plane_frequencies(*rope);
    std::unordered_map<int64_t, int32_t> table_of_delta;
    int64_t written = 0, masked = 0;
    for (int g = 0; g < n_segments; g++) {
        const pic_segment &s = segments[g];
        masked += s.recompute_k;
        p.bounds.insert(p.bounds.end(), {0, s.token_start, s.token_start + s.length});
        p.recompute.insert(p.recompute.end(), {0, s.token_start, s.token_start + s.recompute_k});
        if (s.delta == 0) continue;  // R(0) is the identity: nothing to touch
        int32_t cs_idx;
        auto it = table_of_delta.find(s.delta);
        if (it == table_of_delta.end()) {
            cs_idx = static_cast<int32_t>(table_of_delta.size());
            table_of_delta.emplace(s.delta, cs_idx);
            append_shift_table(freq, s.delta, p.cs);
        } else {
            cs_idx = it->second;
        }
        const HostEntry he{s.token_start, s.token_start, 0, 0, cs_idx, 0};
        p.entries.push_back(he);
        add_tiles(&p, he, nullptr, nullptr, s.recompute_k, s.length);
        written += s.length - s.recompute_k;
    }
    fill_info(&p, written, masked, buf_tokens);
    p.info.n_entries = n_segments;
    return PIC_OK;
}

pic_status build_rotate_paged(const pic_kv_shape *shape, const pic_rope_config *rope,
                              int32_t page_size, int64_t n_phys_pages,
                              const pic_page_segment *segments, int32_t n_segments,
                              Problem *turn, Problem *copy) {
    Units ut{}, uc{};
    pic_status st = derive_units(shape, rope, true, &ut);
    if (st) return st;
    st = derive_units(shape, rope, false, &uc);
    if (st) return st;
    if (page_size < 1 || n_phys_pages < 1 || n_phys_pages > INT32_MAX)
        return fail(PIC_ERR_INVALID_ARG, "page_size %d and n_phys_pages %lld must be >= 1 (pages "
                    "fit int32)", page_size, static_cast<long long>(n_phys_pages));
    if (n_segments < 0 || (n_segments > 0 && !segments))
        return fail(PIC_ERR_INVALID_ARG, "bad segment array");
    // the token run [lo, hi) of segment g that page i holds, as logical
    // positions, and the part of it that is turned
    auto page_run = [&](const pic_page_segment &sg, int32_t i, int64_t from_t, int64_t *lo,
                        int64_t *hi) {
        *lo = std::max<int64_t>(int64_t{sg.first} + from_t, int64_t{i} * page_size);
        *hi = std::min<int64_t>(int64_t{sg.first} + sg.length, int64_t{i + 1} * page_size);
    };
    // writes and reads, collected as intervals and page lists and checked
    // after sorting (no per-slot sets: a call may turn ~10^5 tokens)
    std::vector<Interval> turned_runs;  // key = page, [lo, hi) slots turned in place
    std::vector<int64_t> targets, sources, turned_pages, all_pages;
    for (int g = 0; g < n_segments; g++) {
        const pic_page_segment &sg = segments[g];
        if (!sg.pages) return fail(PIC_ERR_INVALID_ARG, "segment %d: pages is NULL", g);
        if (sg.first < 0 || sg.first >= page_size || sg.length < 1)
            return fail(PIC_ERR_RANGE, "segment %d: first %d, length %d (page_size %d)", g, sg.first,
                        sg.length, page_size);
        const int64_t need = (int64_t{sg.first} + sg.length + page_size - 1) / page_size;
        if (need * page_size > INT32_MAX)  // logical positions of the pages fit int32
            return fail(PIC_ERR_RANGE, "segment %d: first %d + length %d spans %lld pages of %d, "
                        "past 2^31 - 1 positions", g, sg.first, sg.length,
                        static_cast<long long>(need), page_size);
        if (sg.recompute_k < 0 || sg.recompute_k > sg.length)
            return fail(PIC_ERR_RANGE, "segment %d: recompute_k %d", g, sg.recompute_k);
        if (sg.n_pages != need)
            return fail(PIC_ERR_INVALID_ARG, "segment %d: n_pages %d, its tokens span %lld pages", g,
                        sg.n_pages, static_cast<long long>(need));
        for (int32_t i = 0; i < sg.n_pages; i++) {
            if (sg.pages[i] < 0 || sg.pages[i] >= n_phys_pages)
                return fail(PIC_ERR_RANGE, "segment %d: page %d = %d outside [0, %lld)", g, i,
                            sg.pages[i], static_cast<long long>(n_phys_pages));
            if (sg.cow && (sg.cow[i] < -1 || sg.cow[i] >= n_phys_pages))
                return fail(PIC_ERR_RANGE, "segment %d: copy target %d = %d outside [-1, %lld)", g, i,
                            sg.cow[i], static_cast<long long>(n_phys_pages));
            all_pages.push_back(sg.pages[i]);
            if (sg.cow && sg.cow[i] >= 0) {
                targets.push_back(sg.cow[i]);
                sources.push_back(sg.pages[i]);
                continue;
            }
            int64_t lo, hi;
            page_run(sg, i, sg.recompute_k, &lo, &hi);
            if (sg.delta == 0 || lo >= hi) continue;  // nothing written in place
            turned_pages.push_back(sg.pages[i]);
            turned_runs.push_back(Interval{sg.pages[i], lo - int64_t{i} * page_size,
                                           hi - int64_t{i} * page_size});
        }
    }
    if (any_overlap(turned_runs))
        return fail(PIC_ERR_OVERLAP, "two segments turn the same slot of a page in place");
    auto sort_unique = [](std::vector<int64_t> &v) {
        std::sort(v.begin(), v.end());
        v.erase(std::unique(v.begin(), v.end()), v.end());
    };
    std::sort(targets.begin(), targets.end());
    if (std::adjacent_find(targets.begin(), targets.end()) != targets.end())
        return fail(PIC_ERR_OVERLAP, "a copy target is used twice");
    sort_unique(all_pages);
    sort_unique(sources);
    sort_unique(turned_pages);
    for (int64_t t : targets)
        if (std::binary_search(all_pages.begin(), all_pages.end(), t))
            return fail(PIC_ERR_OVERLAP, "copy target %lld is also a page a segment maps",
                        static_cast<long long>(t));
    for (int64_t t : sources)
        if (std::binary_search(turned_pages.begin(), turned_pages.end(), t))
            return fail(PIC_ERR_OVERLAP, "page %lld is copied by one segment and turned in place by "
                        "another", static_cast<long long>(t));

    auto init = [&](Problem &p, const Units &u, int32_t mode) {
        p.shape = *shape;
        p.rope_dim = rope->rope_dim;
        p.style = rope->style;
        p.mode = mode;
        p.page_size = page_size;
        p.src_page_size = page_size;
        p.capacity = n_phys_pages * page_size;
        p.num_phys_pages = n_phys_pages;
        p.n_requests = 1;
        p.u = u;
        p.launch = launch_shape_of(shape->dtype, u);
        p.tile_tokens = kTileSteps * 4 * p.launch.g;
        set_tile_waves(&p, page_size);
    };
    init(*turn, ut, kInPlace);
    turn->shape.has_v = 0;
    turn->launch.stream_loads = 1;  // every turned slot is read once
    init(*copy, uc, kPaged);
    // a shared page may be copied for several segments: then its second read
    // can come from cache; if every copied page is read once, loads stream
    {
        std::vector<uint8_t> seen(static_cast<size_t>(n_phys_pages), 0);
        bool repeat = false;
        for (int g = 0; g < n_segments && !repeat; g++)
            for (int32_t i = 0; i < segments[g].n_pages && !repeat; i++)
                if (segments[g].cow && segments[g].cow[i] >= 0)
                    repeat = seen[static_cast<size_t>(segments[g].pages[i])]++ != 0;
        copy->launch.stream_loads = repeat ? 0 : 1;
    }
    const std::vector<double> freq = plane_frequencies(*rope);
    std::unordered_map<int64_t, int32_t> tab_turn, tab_copy;
    auto table = [&](Problem &p, std::unordered_map<int64_t, int32_t> &m, int64_t delta) {
        auto it = m.find(delta);
        if (it != m.end()) return it->second;
        const int32_t idx = static_cast<int32_t>(m.size());
        m.emplace(delta, idx);
        append_shift_table(freq, delta, p.cs);
        return idx;
    };
    int64_t turned = 0, copied = 0;
    for (int g = 0; g < n_segments; g++) {
        const pic_page_segment &sg = segments[g];
        for (int32_t i = 0; i < sg.n_pages; i++) {
            const int64_t p0 = int64_t{i} * page_size;  // logical position of the page's slot 0
            int64_t lo, hi;
            page_run(sg, i, sg.recompute_k, &lo, &hi);
            const bool turn_run = sg.delta != 0 && lo < hi;
            if (sg.cow && sg.cow[i] >= 0) {
                // the whole page to its copy: slots before and after the
                // turned run bit for bit, the run turned
                const int32_t cs = turn_run ? table(*copy, tab_copy, sg.delta) : -1;
                const HostEntry plain{0, 0, 0, 0, -1, 0}, turned_e{0, 0, 0, 0, cs, 0};
                if (turn_run) {
                    add_tiles(copy, plain, sg.cow, sg.pages, static_cast<int32_t>(p0), static_cast<int32_t>(lo));
                    add_tiles(copy, turned_e, sg.cow, sg.pages, static_cast<int32_t>(lo), static_cast<int32_t>(hi));
                    add_tiles(copy, plain, sg.cow, sg.pages, static_cast<int32_t>(hi),
                              static_cast<int32_t>(p0 + page_size));
                    turned += hi - lo;
                } else {
                    add_tiles(copy, plain, sg.cow, sg.pages, static_cast<int32_t>(p0),
                              static_cast<int32_t>(p0 + page_size));
                }
                copied += page_size;
            } else if (turn_run) {
                const HostEntry e{0, 0, 0, 0, table(*turn, tab_turn, sg.delta), 0};
                add_tiles(turn, e, nullptr, sg.pages, static_cast<int32_t>(lo), static_cast<int32_t>(hi));
                turned += hi - lo;
            }
        }
    }
    fill_info(turn, turned, 0, 0);
    fill_info(copy, copied, 0, 0);
    return PIC_OK;
}

Staged stage(const Problem &p) {
    Staged s;
    auto align = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
    s.off_tiles = 0;
    s.off_cs = align(p.tiles.size() * sizeof(DevTile));
    s.total = std::max<size_t>(align(s.off_cs + p.cs.size() * sizeof(double)), 256);
    return s;
}

void write_staged(const Problem &p, const Staged &s, uint8_t *out) {
    if (!p.tiles.empty()) std::memcpy(out + s.off_tiles, p.tiles.data(), p.tiles.size() * sizeof(DevTile));
    if (!p.cs.empty()) std::memcpy(out + s.off_cs, p.cs.data(), p.cs.size() * sizeof(double));
}

pic_status ensure_attention(struct ::pic_plan *plan) {
    std::lock_guard<std::mutex> lock(plan->mu);
    if (plan->prob.attn_built) return PIC_OK;
    try {
        build_attention(&plan->prob);
    } catch (const std::bad_alloc &) {
        return fail(PIC_ERR_NOMEM, "out of host memory (attention map)");
    }
    return PIC_OK;
}

}  // namespace pic

extern "C" {

pic_status pic_plan(const pic_kv_shape *shape, const pic_rope_config *rope,
                    const pic_chunk *chunks, int32_t n_chunks, const pic_request *requests,
                    int32_t n_requests, const pic_geom *geom, pic_plan_t **out) {
    pic::clear_error();
    if (!out) return pic::fail(PIC_ERR_INVALID_ARG, "out must not be NULL");
    *out = nullptr;
    pic_plan_t *plan = new (std::nothrow) pic_plan_t();
    if (!plan) return pic::fail(PIC_ERR_NOMEM, "out of host memory");
    try {
        pic_status st =
            pic::build_stitch(shape, rope, chunks, n_chunks, requests, n_requests, geom, &plan->prob);
        if (st) {
            delete plan;
            return st;
        }
        plan->staged = pic::stage(plan->prob);
    } catch (const std::bad_alloc &) {
        delete plan;
        return pic::fail(PIC_ERR_NOMEM, "out of host memory");
    }
    *out = plan;
    return PIC_OK;
}

pic_status pic_plan_info(const pic_plan_t *plan, pic_plan_info_t *info) {
    pic::clear_error();
    if (!plan || plan->magic != pic::kPlanMagic)
        return pic::fail(PIC_ERR_STATE, "invalid or destroyed plan");
    if (!info) return pic::fail(PIC_ERR_INVALID_ARG, "info must not be NULL");
    // the attention counts need the map: built here if no call has built it
    pic_status st = pic::ensure_attention(const_cast<pic_plan_t *>(plan));
    if (st) return st;
    *info = plan->prob.info;
    return PIC_OK;
}

pic_status pic_plan_ranges(const pic_plan_t *plan, int64_t *boundaries, int64_t *recompute) {
    pic::clear_error();
    if (!plan || plan->magic != pic::kPlanMagic)
        return pic::fail(PIC_ERR_STATE, "invalid or destroyed plan");
    const auto &p = plan->prob;
    if (boundaries && !p.bounds.empty())
        std::memcpy(boundaries, p.bounds.data(), p.bounds.size() * sizeof(int64_t));
    if (recompute && !p.recompute.empty())
        std::memcpy(recompute, p.recompute.data(), p.recompute.size() * sizeof(int64_t));
    return PIC_OK;
}

const char *pic_last_error(void) { return pic::g_error.c_str(); }

}  // extern "C"
