#!/usr/bin/env python3
"""Throughput of position-independent KV stitching on one MI355X.

One step = the whole batched-RAG stitch: 32 layers, 8 KV heads x 128 dims,
bf16; a pool of 256 cached chunks of 128..4096 tokens; 64 requests, each
placing 4..16 pool chunks (drawn with replacement, in random order) behind
a prefix of 32..512 tokens into a paged cache of 16-token pages.  Every
layer of every request is stitched inside the step.  The pool holds all 32
layers; the destination holds as many layers as fit beside it in HBM, and
each layer group of the step is one pic_stitch launch into it.  Inputs are
synthetic (N(0, 1), seed 0) and resident in HBM before timing.

The value is algorithmic stitched-KV bytes (rows read + rows written) per
second; token-layers/s and the fraction of the 8 TB/s HBM peak are reported
beside it, with the roofline of the stitch kernel (its average launch
duration from HIP events on the launch stream), the library's own 16-byte
streaming copy at the same read/write mix as the practical ceiling, the
planner's time, and the fp64 CPU oracle timed on the host cores over a
stated sample of the same workload.  --workload selects the other paths.

Prints one JSON line on stdout.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "stitched-KV HBM GB/s (read+write) and token-layers/s; % of HBM peak"
PEAK_GBS = 8000.0  # MI355X HBM3E, published
# 32-bit integer vector ALU: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
ALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
CSRC = os.path.join(ROOT, "position_independent_kv_stitch_amd", "csrc")
# The sources that decide what each timed kernel reads and writes: a counter
# summary counts only while their sha256 is the one it was taken with.
STITCH_SOURCES = ("stitch.hip", "rotate.hpp", "plan.cpp", "pic_internal.hpp")
KERNEL_SOURCES = {
    "stitch": STITCH_SOURCES,
    "gqa": ("attend_gqa.hip", "attend_plan.cpp", "attend_map.hpp", "lds_load.hpp", "acc_scale.hpp",
            "attend.hip", "pic_internal.hpp"),
    "mla": ("attend_mla.hip", "attend_plan.cpp", "attend_map.hpp", "lds_load.hpp", "acc_scale.hpp",
            "rotate.hpp", "pic_internal.hpp"),
    "bnd": ("attend_boundary.hip", "attend_plan.cpp", "attend_map.hpp", "lds_load.hpp",
            "rotate.hpp", "pic_internal.hpp"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(kind: str = "stitch") -> str:
    """sha256 over the sources that decide what a kernel reads and writes."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counters_file(workload: str, kernel: str) -> str:
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.md")


def measured_traffic(workload: str, kernel: str, kind: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this workload, or None if there is none or the kernel's sources changed
    since it was taken."""
    path = counters_file(workload, kernel)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
    if not h or not t or h.group(1) != kernel_source_hash(kind):
        return None
    return int(t.group(1))


DEFAULT = "batched-rag"
WORKLOADS = {
    DEFAULT: "batched RAG, all 32 layers: 64 requests of 4..16 chunks drawn with replacement from "
             "a pool of 256 chunks of 128..4096 tokens behind prefixes of 32..512 tokens, "
             "8 kv heads x 128, bf16, 16-token pages, recompute_k 0 (stitch, paged); the pool "
             "holds all 32 layers, the destination the layers of one group, written by each "
             "layer-group launch of the step",
    "batched-rag-tp4": "one GPU's share of the batched-RAG workload under 4-way tensor "
                       "parallelism: the same 64 requests, pool chunks and pages with 2 of the 8 "
                       "kv heads (a 512-byte K row per token), all 32 layers in one launch",
    "llama3-8b-paged": "32 layers, 8 kv heads x 128, bf16, one request of 8 chunks x 2048 tokens "
                       "after a 128-token prefix, 16-token pages, recompute_k 32 (stitch, paged)",
    "llama3-8b-paged-pool": "the default workload with its chunks read from a paged pool of "
                            "16-token blocks in random order (stitch, paged to paged)",
    "mla": "DeepSeek-V3 MLA rows, 61 layers, 576-wide (512 copied + 64 rotated), bf16, 16 chunks "
           "x 4096 tokens (stitch, contiguous)",
    "inplace": "Qwen3-8B, 36 layers, 8 kv heads x 128, bf16, 131072 tokens, 64 segments rotated "
               "in place by shifts in [-65536, 65536], recompute_k 16 (pic_rotate_inplace)",
    "inplace-paged-cow": "the inplace workload on a paged pool of 16-token pages (random physical "
                         "order): 48 chunks turned in place, 16 shared chunks copied page by page "
                         "(K and V) to fresh pages and turned there (pic_rotate_paged)",
    "single-layer": "1 layer, 8 kv heads x 128, fp32, 3 chunks of 512/1024/256 tokens "
                    "(stitch, contiguous; launch-bound)",
    "attend-decode": "decode attention over stitched contexts, chunk keys turned on load: 16 "
                     "requests x 16512 positions (8 own chunks x 2048 behind a 128-token prefix, "
                     "recompute_k 32), 32 query heads over 8 kv heads x 128, bf16, 16-token "
                     "pages; one pic_attend per layer, 32 layers per step",
    "attend-decode-single": "the attend-decode workload with one request (16512 positions): "
                            "a latency-bound decode step",
    "attend-mla-decode": "MLA decode attention over stitched contexts, chunk rotary keys turned "
                         "on load (pic_attend_latent): DeepSeek-V3 rows (576 = 512 latent + "
                         "64 rotary, bf16), 128 query heads, 16 requests x 16512 positions "
                         "(8 own chunks x 2048 behind a 128-token prefix, recompute_k 32), "
                         "64-token pages; one call per layer, 61 layers per step",
    "attend-mla-decode-16h": "the attend-mla-decode workload with 16 query heads (DeepSeek-V2-"
                             "Lite's head count, or one GPU's share of 128 heads over 8)",
    "legolink-boundary": "LegoLink boundary reconnection (pic_attend_boundary): the first 16 "
                         "tokens of every relocated chunk attend causally over the stitched "
                         "context, chunk keys turned on load; Llama-3-8B decode batch (16 "
                         "requests x 8 chunks x 2048 behind a 128-token prefix, recompute_k 32, "
                         "16-token pages), 32 query heads over 8 kv heads x 128, bf16, damping "
                         "4 x -15; one call per layer, 32 layers per step",
    "cdc-rag": "content-defined chunking + xxHash64 fingerprints + registry lookup + 128-token "
               "fallback windows (pic_match) over the batched-RAG prompt stream: 64 requests, "
               "~1.44 M tokens, 10% of placed documents edited, registry of the 256 pool "
               "documents' chunks and windows; mean chunk 256 tokens",
    "cdc-rag-sha256": "the cdc-rag workload with SHA-256 fingerprints (the EPIC registry's key)",
}


def setup_workload(name, torch, pic):
    """Inputs resident on cuda:0 and a step function for one workload."""
    from pic_workloads import (config1, config2, config3, config4, config5, normal_values,
                               pool_values, sentinel_like, with_paged_pool)
    log(f"workload {name}: generating inputs on cuda:0")
    if name == "inplace":
        wl = config5()
        buf = normal_values(wl.buf_shape(), wl.dtype, 0, "cuda:0")
        rot = [s for s in wl.segments if s.delta != 0]
        tokens = sum(s.length - s.recompute_k for s in rot)
        per_tl = wl.n_heads * wl.rope_dim * wl.esize * 2  # rotary slice read + written
        return {"wl": wl, "step": lambda: pic.rotate_workload(wl, buf),
                "bytes": tokens * per_tl * wl.n_layers, "token_layers": tokens * wl.n_layers,
                "kernel": "stitch_kernel<bf16, half> (in place)", "plan": None,
                "cpu": lambda: cpu_baseline_inplace(wl, buf), "counters": "stitch",
                "tensors": [buf],
                "config": {"workload": WORKLOADS[name], "storage": "bf16",
                           "layers": wl.n_layers, "tokens": wl.n_tokens, "segments": 64}}
    if name == "inplace-paged-cow":
        from pic_workloads import config5_paged_cow
        wl, n_phys, segs = config5_paged_cow()
        shape = (wl.n_layers, n_phys, wl.page_size, wl.n_heads, wl.row_dim)
        k = normal_values(shape, wl.dtype, 0, "cuda:0")
        v = normal_values(shape, wl.dtype, 1, "cuda:0")
        row = wl.n_heads * wl.row_dim * wl.esize  # one token's K (or V) row
        rot = wl.n_heads * wl.rope_dim * wl.esize
        turned = sum(s.length - s.recompute_k for s in segs if s.delta != 0)
        copied = sum(len(s.pages) * wl.page_size for s in segs if s.cow is not None)
        in_place = sum(s.length - s.recompute_k for s in segs if s.delta != 0 and s.cow is None)
        # in place: the rotary slice read and written; copies: K and V rows read and written
        nbytes = (in_place * rot * 2 + copied * row * 2 * 2) * wl.n_layers

        def step():
            pic.rotate_paged(k, v, segs, rope_dim=wl.rope_dim, theta=wl.theta, style=wl.style,
                             rope_offset=wl.rope_offset)
        return {"wl": wl, "step": step, "bytes": nbytes, "token_layers": turned * wl.n_layers,
                "kernel": "stitch_kernel<bf16, half> (page copies, then in-place turns)",
                "plan": None, "counters": "stitch", "tensors": [k, v],
                "config": {"workload": WORKLOADS[name], "storage": "bf16", "layers": wl.n_layers,
                           "page_size": wl.page_size, "phys_pages": n_phys, "segments": len(segs),
                           "shared_segments": sum(1 for s in segs if s.cow is not None),
                           "copied_tokens": copied, "turned_in_place_tokens": in_place}}
    if name.startswith("attend-decode"):
        return setup_attend(name, torch, pic)
    if name.startswith("attend-mla-decode"):
        return setup_attend_mla(name, torch, pic)
    if name == "legolink-boundary":
        return setup_boundary(name, torch, pic)
    if name.startswith("cdc-rag"):
        return setup_cdc(name, torch, pic)
    if name in (DEFAULT, "batched-rag-tp4"):
        return setup_rag(name, torch, pic)
    wl = {"llama3-8b-paged": config2, "mla": config4, "single-layer": config1,
          "llama3-8b-paged-pool": lambda: with_paged_pool(config2(), page_size=16, seed=1)}[name]()
    pk, pv = pool_values(wl, seed=0, device="cuda:0")
    dk = sentinel_like(wl.dst_shape(), wl.dtype, "cuda:0")
    dv = sentinel_like(wl.dst_shape(), wl.dtype, "cuda:0") if wl.has_v else None
    plan = pic.Plan.from_workload(wl)
    info = plan.info
    step_bytes = (info["bytes_read_per_layer"] + info["bytes_written_per_layer"]) * wl.n_layers
    cfg = {"workload": WORKLOADS[name], "storage": wl.dtype, "layers": wl.n_layers,
           "kv_heads": wl.n_heads, "row_dim": wl.row_dim, "rope_dim": wl.rope_dim,
           "rope_theta": wl.theta, "page_size": wl.page_size,
           "requests": len(wl.requests), "entries": info["n_entries"],
           "stitched_tokens": info["tokens_written"], "masked_tokens": info["tokens_masked"],
           "parallelism": "single-gpu"}
    kernel = f"stitch_kernel<{wl.dtype}, {wl.style}>"
    return {"wl": wl, "step": lambda: pic.stitch(plan, pk, pv, dk, dv), "bytes": step_bytes,
            "token_layers": info["tokens_written"] * wl.n_layers, "kernel": kernel,
            "plan": plan, "info": info, "pk": pk, "pv": pv, "config": cfg,
            "cpu": lambda: cpu_baseline_stitch(wl, pk, pv, info), "counters": "stitch",
            "tensors": [pk, pv, dk, dv]}


def setup_rag(name, torch, pic):
    """The batched-RAG stitch over all 32 layers: the pool holds every layer,
    the destination as many layers (a divisor of 32) as fit beside it; a
    step is one pic_stitch per layer group, each reading its own pool
    layers and writing the destination's layers."""
    from pic_workloads import config3, layers_per_launch, pool_values, sentinel_like, tp_share
    wl = config3() if name == DEFAULT else tp_share(config3(), 4)
    row = wl.n_heads * wl.row_dim * wl.esize
    pool_bytes = 2 * wl.n_layers * wl.pool_tokens * row
    dst_layer = 2 * wl.n_phys_pages * wl.page_size * row
    free, total = torch.cuda.mem_get_info()
    group = layers_per_launch(wl, free)  # 6 GiB kept for value generation and the runtime
    assert group > 0, "HBM too small for the batched-RAG pool"
    log(f"workload {name}: {free / 2**30:.1f} of {total / 2**30:.1f} GiB free; pool "
        f"{pool_bytes / 2**30:.1f} GiB, destination {group} layers x {dst_layer / 2**30:.2f} GiB")
    pk, pv = pool_values(wl, seed=0, device="cuda:0")
    dk = sentinel_like((group,) + tuple(wl.dst_shape()[1:]), wl.dtype, "cuda:0")
    dv = sentinel_like((group,) + tuple(wl.dst_shape()[1:]), wl.dtype, "cuda:0")
    plan = pic.Plan.from_workload(wl)
    info = plan.info
    groups = [(pk[g:g + group], pv[g:g + group]) for g in range(0, wl.n_layers, group)]

    def step():
        for gk, gv in groups:
            pic.stitch(plan, gk, gv, dk, dv, 0, group)

    step_bytes = (info["bytes_read_per_layer"] + info["bytes_written_per_layer"]) * wl.n_layers
    cfg = {"workload": WORKLOADS[name], "storage": wl.dtype, "layers": wl.n_layers,
           "kv_heads": wl.n_heads, "row_dim": wl.row_dim, "rope_dim": wl.rope_dim,
           "rope_theta": wl.theta, "page_size": wl.page_size, "requests": len(wl.requests),
           "pool_chunks": len(wl.chunks), "pool_tokens": wl.pool_tokens,
           "entries": info["n_entries"], "stitched_tokens": info["tokens_written"],
           "masked_tokens": info["tokens_masked"], "dst_phys_pages": wl.n_phys_pages,
           "layers_per_launch": group, "launches_per_step": wl.n_layers // group,
           "hbm_gib": {"total": round(total / 2**30, 1), "free_before": round(free / 2**30, 1),
                       "pool": round(pool_bytes / 2**30, 1),
                       "destination": round(group * dst_layer / 2**30, 1)},
           "parallelism": "single-gpu" if name == DEFAULT else "one GPU's share of tp4"}
    return {"wl": wl, "step": step, "bytes": step_bytes,
            "token_layers": info["tokens_written"] * wl.n_layers,
            "launches": wl.n_layers // group,
            "kernel": f"stitch_kernel<{wl.dtype}, {wl.style}>", "plan": plan, "info": info,
            "config": cfg, "cpu": lambda: cpu_baseline_rag(wl, pk, pv), "counters": "stitch",
            "tensors": [pk, pv, dk, dv]}


def setup_attend(name, torch, pic):
    """The decode-attention workload: one step is a pic_attend per layer."""
    from pic_workloads import Request, Workload, decode_batch, normal_values, pool_values
    wl = decode_batch(n_requests=1 if name == "attend-decode-single" else 16)
    group = 4
    pk, pv = pool_values(wl, seed=0, device="cuda:0")
    ck = normal_values(wl.dst_shape(), wl.dtype, 2, "cuda:0")
    cv = normal_values(wl.dst_shape(), wl.dtype, 3, "cuda:0")
    R, L = len(wl.requests), wl.n_layers
    q = normal_values((L, R, wl.n_heads * group, wl.row_dim), wl.dtype, 4, "cuda:0")
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda:0")
    plan = pic.Plan.from_workload(wl)
    info = plan.info
    # the same contexts with no placed chunks: every position read from the cache
    plain_wl = Workload(wl.name, wl.dtype, L, wl.n_heads, wl.row_dim, wl.rope_offset,
                        wl.rope_dim, wl.style, wl.theta, True, pool_tokens=wl.pool_tokens,
                        chunks=wl.chunks,
                        requests=[Request([], rq.page_table, rq.context_len)
                                  for rq in wl.requests],
                        page_size=wl.page_size, n_phys_pages=wl.n_phys_pages)
    plain = pic.Plan.from_workload(plain_wl)

    def run(p):
        def step():
            for layer in range(L):
                pic.attend(p, pk, pv, ck, cv, q[layer], layer=layer, out=out[layer],
                           sink_tokens=4, sink_bias=-15.0)
        return step

    row = wl.n_heads * wl.row_dim * 2  # one bf16 K (or V) row of all kv heads
    cfg = {"workload": WORKLOADS[name], "storage": wl.dtype, "layers": L,
           "kv_heads": wl.n_heads, "q_heads": wl.n_heads * group, "row_dim": wl.row_dim,
           "requests": R, "context_tokens": info["context_tokens"],
           "chunk_positions": info["tokens_written"], "page_size": wl.page_size,
           "sink_tokens": 4, "sink_bias": -15.0, "parallelism": "single-gpu"}
    return {"wl": wl, "step": run(plan), "plain_step": run(plain),
            "bytes": info["context_tokens"] * 2 * row * L,
            "token_layers": info["context_tokens"] * L, "launches": L,
            "arithmetic": "f32 softmax and accumulation, bf16 matrix-core products (vector f32 off the matrix-core shapes)", "kernel": "gqa_tile_kernel + gqa_combine_kernel (one pic_attend)", "counters": "gqa",
            "plan": plan, "plans": [plain], "info": info, "config": cfg}


def setup_attend_mla(name, torch, pic):
    """MLA decode attention: one step is a pic_attend_latent per layer."""
    from pic_workloads import mla_decode_batch, normal_values, pool_values
    wl = mla_decode_batch()
    heads = 16 if name.endswith("16h") else 128
    pk, _ = pool_values(wl, seed=0, device="cuda:0")
    ck = normal_values(wl.dst_shape(), wl.dtype, 2, "cuda:0")
    R, L = len(wl.requests), wl.n_layers
    q = normal_values((L, R, heads, wl.row_dim), wl.dtype, 4, "cuda:0")
    out = torch.empty((L, R, heads, 512), dtype=torch.float32, device="cuda:0")
    plan = pic.Plan.from_workload(wl)
    info = plan.info
    scale = 192 ** -0.5

    def step():
        for layer in range(L):
            pic.attend_latent(plan, pk, ck, q[layer], layer=layer, out=out[layer], scale=scale,
                              sink_tokens=4, sink_bias=-15.0)

    row = wl.row_dim * 2
    flops = info["context_tokens"] * heads * 2 * (wl.row_dim + 512) * L  # q.k and w.v per head
    cfg = {"workload": WORKLOADS[name], "storage": wl.dtype, "layers": L, "q_heads": heads,
           "row_dim": wl.row_dim, "requests": R, "context_tokens": info["context_tokens"],
           "chunk_positions": info["tokens_written"], "page_size": wl.page_size,
           "softmax_scale": "1/sqrt(192)", "sink_tokens": 4, "sink_bias": -15.0,
           "parallelism": "single-gpu"}
    return {"wl": wl, "step": step, "bytes": info["context_tokens"] * row * L,
            "token_layers": info["context_tokens"] * L, "launches": L, "flops": flops,
            "arithmetic": "f32 softmax and accumulation, bf16 matrix-core products (vector f32 off the matrix-core shapes)", "kernel": ("mla_wide_kernel" if heads % 128 == 0 else "mla_block_kernel") + "<half> + mla_combine_kernel (one pic_attend_latent)", "counters": "mla",
            "plan": plan, "info": info, "config": cfg}


def setup_boundary(name, torch, pic):
    """Boundary reconnection: one step is a pic_attend_boundary per layer."""
    from pic_workloads import decode_batch, normal_values, pool_values
    wl = decode_batch()
    k, group = 16, 4
    pk, pv = pool_values(wl, seed=0, device="cuda:0")
    ck = normal_values(wl.dst_shape(), wl.dtype, 2, "cuda:0")
    cv = normal_values(wl.dst_shape(), wl.dtype, 3, "cuda:0")
    plan = pic.Plan.from_workload(wl)
    n = pic.boundary_row_count(plan, k)
    L = wl.n_layers
    q = normal_values((L, n, wl.n_heads * group, wl.row_dim), wl.dtype, 4, "cuda:0")
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda:0")

    def step():
        for layer in range(L):
            pic.attend_boundary(plan, pk, pv, ck, cv, q[layer], layer=layer, boundary_k=k,
                                out=out[layer], scale=wl.row_dim ** -0.5, sink_tokens=4,
                                sink_bias=-15.0)

    # the method must read each request's K and V rows of [0, last boundary
    # position] once (all its boundary rows share them), the queries, and
    # write the outputs
    bounds, _ = plan.ranges()
    reloc = [(int(b), int(e - b)) for _, b, e in bounds if b > 0]
    last = {}
    for r, b, e in bounds:
        if b > 0:
            last[int(r)] = max(last.get(int(r), 0), int(b) + min(k, int(e - b)))
    ctx = sum(last.values())
    row_bytes = 2 * wl.n_heads * wl.row_dim * 2
    qo_bytes = n * wl.n_heads * group * wl.row_dim * (2 + 4)
    pairs = sum(sum(d + j + 1 for j in range(min(k, ln))) for d, ln in reloc)  # (row, position)
    flops = pairs * wl.n_heads * group * 2 * 2 * wl.row_dim * L
    cfg = {"workload": WORKLOADS[name], "storage": wl.dtype, "layers": L,
           "kv_heads": wl.n_heads, "q_heads": wl.n_heads * group, "row_dim": wl.row_dim,
           "requests": len(wl.requests), "relocated_entries": len(reloc), "boundary_k": k,
           "boundary_rows": n, "context_positions_read": ctx, "page_size": wl.page_size,
           "sink_tokens": 4, "sink_bias": -15.0, "parallelism": "single-gpu"}
    return {"wl": wl, "step": step, "bytes": (ctx * row_bytes + qo_bytes) * L, "token_layers": n * L,
            "launches": L, "flops": flops,
            "arithmetic": "f32 softmax and accumulation, bf16 matrix-core products (vector f32 off the matrix-core shapes)", "kernel": "bnd_block_kernel<half> + bnd_combine_kernel (one pic_attend_boundary)", "counters": "bnd",
            "plan": plan, "config": cfg}


def setup_cdc(name, torch, pic):
    """The chunking workload: one step is one pic_match over the whole stream.
    The registry is filled the way a serving system would fill it, from the
    library's own chunking of every pool document on its own (its chunks, and
    the 128-token windows of each chunk)."""
    from pic_workloads import CDC_THRESHOLD, rag_token_stream
    kind = "sha256" if name.endswith("sha256") else "xxh64"
    ts = rag_token_stream(0, edit_prob=0.1)
    reg = pic.Registry(kind)
    seen = set()
    for doc in ts.docs:
        d = torch.from_numpy(doc).to("cuda:0")
        for window in (0, 128):  # empty registry: window 0 gives chunks, 128 their windows
            out, n_out = pic.match(d, CDC_THRESHOLD, None, kind=kind, window=window)
            recs, m = pic.match_records(out, n_out)
            for r in recs[:m]:
                key = (bytes(r["fp"]), int(r["length"]))
                if key not in seen:
                    seen.add(key)
                    reg.add(key[0], key[1], len(seen) - 1)
    tokens = torch.from_numpy(ts.tokens).to("cuda:0")
    n = len(ts.tokens)
    out = torch.empty((n, 56), dtype=torch.uint8, device="cuda:0")
    n_out = torch.empty(1, dtype=torch.int64, device="cuda:0")

    def step():
        pic.match(tokens, CDC_THRESHOLD, reg, kind=kind, window=128, out=out, n_out=n_out)

    step()
    recs, m = pic.match_records(out, n_out)
    hits = recs[:m]["chunk_id"] >= 0
    window_tokens = int(recs[:m]["length"][recs[:m]["level"] == 1].sum())
    # Integer work of one call, in 32-bit ALU operations counted from the
    # definitions (a 64-bit add, xor, shift or rotate counts 2, a 64-bit
    # multiply 4): Gear value and rolling step per token, then every chunk
    # token hashed once and every window token once more.
    hash_ops = 6.0 if kind == "xxh64" else 2296.0 / 16  # per token: xxHash64 lane / SHA-256 block
    alu_ops = n * 40 + (n + window_tokens) * hash_ops
    cfg = {"workload": WORKLOADS[name], "tokens": n, "requests": len(ts.request_starts),
           "registry_entries": len(seen), "segments": int(m),
           "registered_segments": int(hits.sum()),
           "registered_tokens": int(recs[:m]["length"][hits].sum()),
           "fingerprint": kind, "window": 128, "threshold": "2^56",
           "parallelism": "single-gpu"}
    return {"wl": None, "step": step, "bytes": 4 * n, "token_layers": n,
            "arithmetic": "64-bit integer hashing", "kernel": "pic_match (8 kernels: Gear flags, scans, ends, chunk hashes, emit)",
            "plan": None, "registry": reg, "config": cfg, "alu_ops": alu_ops}


def time_steps(torch, step, steps):
    """Average ms per step over `steps` back-to-back steps (HIP events on the
    current stream)."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(steps):
        step()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def host_cpu():
    """What the host offers the oracle: logical CPUs, this process's CPU
    share (affinity) and the CPU model."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    share = len(os.sched_getaffinity(0))
    # one GPU's share of the host: at most 16 worker threads whatever nproc shows
    return {"nproc": os.cpu_count(), "affinity": share, "threads": min(16, share),
            "model": model}


def _timed_pool(fn, units, threads):
    """Run fn over units on `threads` host threads (the oracle's C calls
    release the GIL); returns (wall s, process CPU s)."""
    from concurrent.futures import ThreadPoolExecutor
    c0, t0 = time.process_time(), time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(fn, units))
    return time.perf_counter() - t0, time.process_time() - c0


def _baseline(host, unit_bytes, unit_tl, all_units, one_units, fn, what):
    """The oracle over `all_units` on the host's threads and over `one_units`
    on one thread, as GB/s of algorithmic bytes and token-layers/s."""
    wall, cpu_s = _timed_pool(fn, all_units, host["threads"])
    wall1, _ = _timed_pool(fn, one_units, 1)
    nb, nt = sum(unit_bytes(u) for u in all_units), sum(unit_tl(u) for u in all_units)
    nb1, nt1 = sum(unit_bytes(u) for u in one_units), sum(unit_tl(u) for u in one_units)
    return {"value": round(nb / wall / 1e9, 4), "unit": "GB/s", "cores": host["threads"],
            "kind": "oracle",
            "sample": f"{what}: {len(all_units)} units on {host['threads']} threads in "
                      f"{wall:.2f} s wall ({cpu_s:.1f} s CPU); one thread: {len(one_units)} "
                      f"units in {wall1:.2f} s",
            "token_layers_per_s": round(nt / wall, 1),
            "one_core": {"value": round(nb1 / wall1 / 1e9, 4), "unit": "GB/s",
                         "token_layers_per_s": round(nt1 / wall1, 1)},
            "process_cpu_s": round(cpu_s, 1),
            "host": {"nproc": host["nproc"], "affinity_cpus": host["affinity"],
                     "cpu_model": host["model"]}}


def cpu_baseline_stitch(wl, pk, pv, plan_info, passes=4):
    """The oracle, as it is, over `passes` full steps of a stitch workload:
    one oracle call per layer (a unit) on the host threads; one thread runs
    one step."""
    import oracle
    from pic_workloads import sentinel_like, to_host

    host = host_cpu()
    log(f"cpu baseline: copying pool to host, {host['threads']} threads")
    hk = to_host(pk)
    hv = to_host(pv) if pv is not None else None
    sent = to_host(sentinel_like((1,) + tuple(wl.dst_shape()[1:]), wl.dtype, "cpu"))

    def one(layer):
        dk = sent.copy()
        dv = sent.copy() if hv is not None else None
        st = oracle.stitch(wl, hk[layer:layer + 1], hv[layer:layer + 1] if hv is not None else None,
                           dk, dv, layer, layer + 1, layer_base=layer)
        assert st == "ok"

    per_layer = plan_info["bytes_read_per_layer"] + plan_info["bytes_written_per_layer"]
    layers = list(range(wl.n_layers))
    return _baseline(host, lambda u: per_layer, lambda u: plan_info["tokens_written"],
                     layers * passes, layers, one,
                     f"{passes} full steps ({wl.n_layers} layers x "
                     f"{plan_info['tokens_written']} stitched tokens), one oracle call per layer")


def cpu_baseline_rag(wl, pk, pv, layers=(0,), one_requests=8):
    """The oracle on a sample of the batched-RAG step: every request of
    `layers` (each (layer, request) a one-request problem over that layer's
    whole pool, its pages renumbered), on the host threads; one thread runs
    `one_requests` requests of the first layer."""
    import numpy as np

    import oracle
    from pic_workloads import SENTINEL_BITS, Request, Workload, to_host

    host = host_cpu()
    log(f"cpu baseline: copying layers {list(layers)} of the pool to host, "
        f"{host['threads']} threads")
    hk = {layer: to_host(pk[layer:layer + 1]) for layer in layers}
    hv = {layer: to_host(pv[layer:layer + 1]) for layer in layers}
    row = wl.n_heads * wl.row_dim * wl.esize
    subs = []
    for rq in wl.requests:
        n = len(rq.page_table)
        subs.append(Workload(wl.name, wl.dtype, wl.n_layers, wl.n_heads, wl.row_dim,
                             wl.rope_offset, wl.rope_dim, wl.style, wl.theta, wl.has_v,
                             pool_tokens=wl.pool_tokens, chunks=wl.chunks,
                             requests=[Request(rq.entries, np.arange(n, dtype=np.int32))],
                             page_size=wl.page_size, n_phys_pages=n))
    tokens = [sum(e.length - e.recompute_k for e in rq.entries) for rq in wl.requests]

    def one(unit):
        layer, r = unit
        sub = subs[r]
        shape = (1,) + tuple(sub.dst_shape()[1:])
        dk = np.full(shape, SENTINEL_BITS[wl.dtype], dtype=np.uint16 if wl.dtype == "bf16"
                     else np.uint32)
        if wl.dtype == "f32":
            dk = dk.view(np.float32)
        dv = dk.copy()
        assert oracle.stitch(sub, hk[layer], hv[layer], dk, dv, layer, layer + 1,
                             layer_base=layer) == "ok"

    units = [(layer, r) for layer in layers for r in range(len(wl.requests))]
    return _baseline(host, lambda u: tokens[u[1]] * 2 * 2 * row, lambda u: tokens[u[1]],
                     units, units[:one_requests], one,
                     f"layers {list(layers)} of the step, all {len(wl.requests)} requests "
                     f"(one unit = one request at one layer)")


def cpu_baseline_inplace(wl, buf, n_layers=8):
    """The oracle's in-place rotation over the first n_layers layers of the
    in-place workload: one call per layer on the host threads; one thread
    runs 2 layers."""
    import oracle
    from pic_workloads import to_host

    host = host_cpu()
    log(f"cpu baseline: copying the buffer to host, {host['threads']} threads")
    hb = to_host(buf[:n_layers])
    rot = [sg for sg in wl.segments if sg.delta != 0]
    tokens = sum(sg.length - sg.recompute_k for sg in rot)
    per_layer = tokens * wl.n_heads * wl.rope_dim * wl.esize * 2

    def one(layer):
        part = hb[layer:layer + 1].copy()
        assert oracle.rotate_inplace(wl, part, layer, layer + 1, layer_base=layer) == "ok"

    layers = list(range(n_layers))
    return _baseline(host, lambda u: per_layer, lambda u: tokens, layers, layers[:2], one,
                     f"{n_layers} of the step's {wl.n_layers} layers ({tokens} turned tokens "
                     f"each), one oracle call per layer")


def copy_ceiling(torch, pic, nbytes, reps=20):
    """The library's 16-byte streaming copy (pic_stream_copy) moving the same
    read+write bytes: half read, half written, as in the stitch."""
    n = (nbytes // 2) // 16 * 16
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        pic.stream_copy(dst, src)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        pic.stream_copy(dst, src)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    assert torch.equal(dst[:4096], src[:4096])
    del src, dst
    return {"value": round(2 * n / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
            "kind": "pic_stream_copy (16-byte non-temporal loads and stores, 1:1 read/write)",
            "bytes_moved": 2 * n}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy-ceiling", action="store_true")
    ap.add_argument("--no-plain-attention", action="store_true",
                    help="attend-decode: skip timing attention over the cache alone")
    ap.add_argument("--workload", default=DEFAULT, choices=sorted(WORKLOADS),
                    help="the default is the workload the headline metric is quoted on; the "
                         "others time the remaining paths")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures the single-GPU path only (asked for --gpus {args.gpus}): under "
              "tensor, pipeline or data parallelism each GPU stitches its own KV heads, layers or "
              "requests with the same plan and nothing crosses GPUs; --workload batched-rag-tp4 "
              "times one GPU's share under 4-way tensor parallelism", file=sys.stderr)
        sys.exit(2)

    import torch

    import position_independent_kv_stitch_amd as pic

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    W = setup_workload(args.workload, torch, pic)
    step = W["step"]
    step_bytes, step_tl = W["bytes"], W["token_layers"]

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    launches = W.get("launches", 1)
    kernel_ms = sorted(s.elapsed_time(e) / launches for s, e in zip(starts, ends))
    avg_kernel_ms = sum(kernel_ms) / len(kernel_ms)
    ms_per_step = total_ms / args.steps

    value = step_bytes * args.steps / (total_ms * 1e-3) / 1e9
    achieved = step_bytes / launches / (avg_kernel_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": W["config"].get("storage", "int32"),  # cdc workloads: int32 token ids
        "arithmetic": W.get("arithmetic", "f64 rotation, one rounding to the storage type"),
        "data": "synthetic",
        "config": W["config"],
        "token_layers_per_s": round(step_tl * args.steps / (total_ms * 1e-3), 1),
        "hbm_peak_frac": round(value / PEAK_GBS, 4),
        "bytes_per_step": step_bytes,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_GBS, 4),
                     "traffic": measured_traffic(args.workload, W["kernel"].split("<")[0].split()[0],
                                                 W.get("counters", "")) if W.get("counters")
                     else None,
                     "kernel": W["kernel"],
                     "avg_launch_ms": round(avg_kernel_ms, 5),
                     "median_launch_ms": round(kernel_ms[len(kernel_ms) // 2], 5),
                     "algorithmic_bytes_per_launch": step_bytes // launches},
    }
    if "alu_ops" in W:  # integer hashing: priced against the chip's 32-bit vector ALU rate
        tops = W["alu_ops"] / (avg_kernel_ms * 1e-3) / 1e12
        out["roofline"] = {"bound": "alu", "achieved": round(tops, 4), "peak": ALU_PEAK_TOPS,
                           "unit": "TOP/s", "frac": round(tops / ALU_PEAK_TOPS, 5),
                           "traffic": None, "kernel": W["kernel"],
                           "avg_launch_ms": round(avg_kernel_ms, 5),
                           "median_launch_ms": round(kernel_ms[len(kernel_ms) // 2], 5),
                           "algorithmic_int_ops_per_call": int(W["alu_ops"])}
        out["tokens_per_s"] = round(W["token_layers"] * args.steps / (total_ms * 1e-3), 1)
    if launches > 1:
        out["roofline"]["launches_per_step"] = launches
    if out["roofline"].get("traffic"):
        # the HBM bandwidth the launch actually used (counter traffic over the
        # same launch time): below `achieved` where repeated rows come from cache
        out["roofline"]["traffic_gbps"] = round(out["roofline"]["traffic"] / (avg_kernel_ms * 1e-3) / 1e9, 1)
    if "flops" in W:  # matrix-core work beside the bytes: bf16 dense peak 2.5 PFLOP/s
        tf = W["flops"] / launches / (avg_kernel_ms * 1e-3) / 1e12
        out["roofline"]["mfma"] = {"achieved": round(tf, 1), "peak": 2500.0, "unit": "TFLOP/s",
                                   "frac": round(tf / 2500.0, 4),
                                   "algorithmic_flops_per_launch": W["flops"] // launches}
    if "plain_step" in W and not args.no_plain_attention:
        for _ in range(3):
            W["plain_step"]()
        plain_ms = time_steps(torch, W["plain_step"], max(5, args.steps // 4))
        out["attention_over_cache"] = {
            "ms_per_step": round(plain_ms, 5),
            "value": round(step_bytes / (plain_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
            "what": "the same contexts with no placed chunks (every row from the cache, "
                    "no rotation): the cost of attention alone"}
    if W.get("plan") is not None:
        out["planner_ms"] = round(W["plan"].plan_seconds * 1e3, 3)
    out["cpu_baseline"] = None
    if not args.no_cpu_baseline and "cpu" in W:
        out["cpu_baseline"] = W["cpu"]()
    for p in [W.get("plan")] + W.get("plans", []):
        if p is not None:
            p.destroy()
    step = None
    W.clear()  # the workload's tensors go before the copy ceiling allocates its own
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_copy_ceiling:
        out["copy_ceiling"] = copy_ceiling(torch, pic, min(step_bytes // launches, 8 << 30))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
