"""Sparse-MLA decode throughput on one MI355X.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--cpu-seconds 15] [--no-cpu-baseline]

A step is one pass of the decode hot path over one batch of seeded synthetic input:
slot resolution (logical top-k -> physical slots through the page table), stage 1 (split
gather + MFMA scores + online softmax + MFMA P*V) and stage 2 (LSE merge). The headline
step runs the resolution inside stage 1 (smla_sparse_decode_topk); the two-kernel form
(smla_resolve_slots, then decode over the slot table) is timed beside it. The headline
workload is the bf16 batch of 32 requests x 64 heads, latent 512 + rope 64, contexts
U[8K, 32K] in a 2^20-slot pool of 64-slot pages, top-k 2048. The inputs are resident in
HBM when a timed step starts: before every timed step a 1 GiB buffer is read, so that
neither the L2 nor the 256 MB Infinity Cache holds the cache rows (reading rather than
writing it leaves no dirty lines whose write-back would compete with the step).

Prints exactly one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import contextlib
import csv
import gc
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-MLA decode queries/s + achieved HBM GB/s (% of peak) at top-k 2048"
HBM_PEAK_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


@contextlib.contextmanager
def section(torch, name):
    """A named range in the marker trace of a profiler (torch's NVTX ranges are roctx ranges on
    ROCm; rocprofv3 --marker-trace records them), with the device drained on both sides so that
    the range holds exactly the kernels launched inside it. --summarize-profile trace labels
    each dispatch with its innermost "workload:" and "form:" ranges."""
    torch.cuda.synchronize()
    pushed = True
    try:
        torch.cuda.nvtx.range_push(name)
    except Exception:                      # no marker library: the ranges are only labels
        pushed = False
    try:
        yield
    finally:
        torch.cuda.synchronize()
        if pushed:
            torch.cuda.nvtx.range_pop()


KERNEL_SOURCES = ["sparse_mla_attention_resolve_amd/csrc/decode.hip", "sparse_mla_attention_resolve_amd/csrc/stage1_common.h",
                  "sparse_mla_attention_resolve_amd/csrc/smla_device.h", "sparse_mla_attention_resolve_amd/csrc/smla_internal.h"]
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode_kernels_hbm_traffic.md")


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload`, as the committed rocprofv3 counter summary
    records them (FETCH_SIZE + WRITE_SIZE, each scaled by a copy kernel's reading), or None when
    there is no such line or the decode kernel sources changed since the counters were taken."""
    import hashlib
    try:
        text = open(TRAFFIC_PROFILE).read().split()
    except OSError:
        return None
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    try:
        recorded = text[text.index("source_sha256") + 1]
    except (ValueError, IndexError):
        return None
    if recorded != h.hexdigest():
        return None
    for i, tok in enumerate(text):
        if tok == "traffic_bytes_per_launch" and text[i + 1] == kernel and text[i + 2] == workload:
            return int(text[i + 3])
    return None


def algorithmic_bytes(c, kv_dtype: str) -> dict:
    """Bytes the method must move for one decode step of case `c` (every row, q element,
    index and output read or written once). Split partials and repeated reads are not
    counted: they are the implementation's overhead."""
    T, H = c.q.shape[0], c.q.shape[1]
    n_rows = int((c.idx >= 0).sum()) if len(c.dense_tokens) == 0 else None
    row_bytes = 1152 if kv_dtype == "bf16" else 644        # fp8: 512 codes + 128 rope + 4 scale
    kv = n_rows * row_bytes
    q = T * H * 576 * 2
    out = T * H * 512 * 2
    lse = T * H * 4
    idx = int(c.idx.size) * 4                               # logical indices read by resolve
    slots = int(c.idx.size) * 4                             # resolved slots read by stage 1
    pages = 0
    for t in range(T):
        row = c.idx[t][c.idx[t] >= 0]
        pages += len(np.unique(row // c.layout.page_size)) * 4
    return {"kv": kv, "q": q, "out": out, "lse": lse, "idx": idx, "page_table": pages,
            "step": kv + q + out + lse + idx + pages,      # resolved slots stay on chip (fused stage 1)
            "stage1": kv + q + idx + pages,                # stage 1 resolving the indices itself
            "stage1_slots": kv + q + slots}                # stage 1 over resolved slots


def setup_decode(c, smla, torch):
    dev = "cuda"

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    lay = c.layout
    code = {"bf16": smla.SMLA_BF16, "fp8": smla.SMLA_FP8_E4M3}[c.kv_dtype]
    kv = smla.KvCache.empty(code, lay.num_slots, device=dev)
    smap = smla.smla_resolve_slots(t(c.rows.pos[:, None]), None, t(c.rows.req), t(lay.page_table), t(lay.ctx),
                                   lay.page_size)[:, 0].contiguous()
    vals = c.rows.values
    src = t(vals.view(np.int16)).view(torch.bfloat16) if vals.dtype == np.uint16 else t(vals)
    smla.smla_kv_write(src, smap, kv)
    T, H = c.q.shape[0], c.q.shape[1]
    st = {
        "q": t(c.q.view(np.int16)).view(torch.bfloat16), "kv": kv, "idx": t(c.idx), "valid": t(c.valid),
        "req": t(c.tok_req), "pt": t(lay.page_table), "ctx": t(lay.ctx),
        "slots": torch.empty(c.idx.shape, dtype=torch.int32, device=dev),
        "out": torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev),
        "lse": torch.empty((T, H), dtype=torch.float32, device=dev),
    }
    st["call"] = smla.DecodeCall(st["q"], kv, st["slots"], st["valid"], 1, c.scale, st["out"], st["lse"])
    # the fused form: stage 1 resolves the logical indices through the page table itself
    st["fused"] = smla.DecodeCall(st["q"], kv, st["idx"], st["valid"], 1, c.scale, st["out"], st["lse"],
                                  page_map=(st["req"], st["pt"], st["ctx"], lay.page_size))
    torch.cuda.synchronize()
    return st


GRAPH_STEPS = 8


def split_sweep(smla, torch, flush, steps, dtypes=("bf16", "fp8"), batches=(1, 2, 4, 8, 16, 32, 64, 128),
                width=2048):
    """Cold step time of the decode against the split count, per batch size and cache dtype, at
    top-k `width` over a 2^20-slot pool of random rows (64 heads; the values do not change the
    work). Prints one line per (dtype, T) and returns the table."""
    n = 1 << 20
    res = {}
    for dt in dtypes:
        code = {"bf16": smla.SMLA_BF16, "fp8": smla.SMLA_FP8_E4M3}[dt]
        kv = smla.KvCache.empty(code, n, device="cuda", poison=False)
        if dt == "bf16":
            kv.storage.normal_(0.0, 0.5)
        else:
            kv.storage.copy_(torch.randint(0, 0x7E, kv.storage.shape, dtype=torch.uint8, device="cuda"))
            kv.rope16().copy_((torch.randn(n, 64, device="cuda") * 0.5).to(torch.bfloat16).view(torch.int16))
            kv.scale().fill_(0.01)
        for T in batches:
            g = torch.Generator(device="cuda").manual_seed(1000 + T)
            q = (torch.randn(T, 64, 576, device="cuda", generator=g) * 0.5).to(torch.bfloat16)
            table = torch.randint(0, n, (T, width), dtype=torch.int32, device="cuda", generator=g)
            lens = torch.full((T,), width, dtype=torch.int32, device="cuda")
            out = torch.empty((T, 64, 512), dtype=torch.bfloat16, device="cuda")
            lse = torch.empty((T, 64), dtype=torch.float32, device="cuda")
            auto = smla.DecodeCall(q, kv, table, lens, 1, 1 / 16, out, lse).splits
            row = {}
            for S in sorted({1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64, auto}):
                if S < (width + 1023) // 1024 or S > width // 32:
                    continue
                call = smla.DecodeCall(q, kv, table, lens, 1, 1 / 16, out, lse, num_splits=S)
                for _ in range(3):
                    flush.sum()
                    call()
                ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
                for k in range(steps):
                    flush.sum()
                    ev[k][0].record()
                    call()
                    ev[k][1].record()
                torch.cuda.synchronize()
                row[call.splits] = float(np.median([e[0].elapsed_time(e[1]) for e in ev])) * 1e3
            best = min(row, key=row.get)
            res[(dt, T)] = {"auto": auto, "best": best, "us": row}
            log(f"split sweep {dt} T={T}: auto S={auto} {row[auto]:.1f} us, best S={best} {row[best]:.1f} us; " +
                " ".join(f"{k}:{v:.1f}" for k, v in sorted(row.items())))
        del kv
        torch.cuda.empty_cache()
    return res


def overlap_sweep(smla, torch, flush, steps, Q=4096, W=2048, ns=24576,
                  overlaps=(0.0, 0.25, 0.5, 0.7, 0.9, 1.0), groups=(2, 4, 8)):
    """Grouped prefill (union build + grouped attention, G queries of H = 128 / G heads per
    group) against every query attending its own list alone (the decode kernel over the lists,
    page size 1), for lists of W slots of which a fraction `overlap` is shared by the group's
    members (the rest disjoint). bf16 cache of ns random rows. Prints a line per (G, overlap)."""
    kv = smla.KvCache.empty(smla.SMLA_BF16, ns, device="cuda", poison=False)
    kv.storage.normal_(0.0, 0.5)
    res = {}
    for G in groups:
        H = 128 // G
        ng = (Q + G - 1) // G
        g = torch.Generator(device="cuda").manual_seed(77 + G)
        q = (torch.randn(Q, H, 576, device="cuda", generator=g) * 0.5).to(torch.bfloat16)
        out = torch.empty((Q, H, 512), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((Q, H), dtype=torch.float32, device="cuda")
        valid = torch.full((Q,), W, dtype=torch.int32, device="cuda")
        for ov in overlaps:
            n_sh = int(round(ov * W))
            own = W - n_sh
            # per group one permutation of the pool: its first n_sh entries are shared, then each
            # member's own entries follow, disjoint from the shared ones and from each other's
            perm = torch.rand(ng, ns, device="cuda", generator=g).argsort(dim=1).to(torch.int32)
            m = torch.arange(Q, device="cuda") % G
            rows = perm[torch.arange(Q, device="cuda") // G]
            cols = torch.cat([torch.arange(n_sh, device="cuda").expand(Q, n_sh),
                              n_sh + m[:, None] * own + torch.arange(own, device="cuda")[None, :]], dim=1)
            lists = torch.gather(rows, 1, cols)
            lists = torch.gather(lists, 1, torch.rand(Q, W, device="cuda", generator=g).argsort(dim=1)).contiguous()
            del perm, rows
            enc, lens = smla.smla_build_group_union(lists, valid, G, ns)
            dec = smla.DecodeCall(q, kv, lists, valid, 1, 1 / 16, out, lse)

            def grouped():
                smla.smla_build_group_union(lists, valid, G, ns, enc=enc, lens=lens)
                smla.smla_grouped_prefill(q, kv, enc, lens, G, 1 / 16, out=out, lse=lse)

            def timed(fn):
                for _ in range(2):
                    flush.sum()
                    fn()
                ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
                for k in range(steps):
                    flush.sum()
                    ev[k][0].record()
                    fn()
                    ev[k][1].record()
                torch.cuda.synchronize()
                return float(np.median([e[0].elapsed_time(e[1]) for e in ev])) * 1e3

            tg, td = timed(grouped), timed(dec)
            ratio = float(lens.float().mean()) / W
            res[(G, ov)] = {"grouped_us": tg, "alone_us": td, "union_per_list": ratio}
            log(f"overlap sweep G={G} H={H} overlap {ov:.2f}: union {ratio:.2f} x W per group, grouped {tg:.0f} us, "
                f"each query alone {td:.0f} us, speedup {td / tg:.2f}x")
            del lists, enc, lens, dec
    return res


BATCHES = 8


def extra_batches(c, st, smla, torch, n, seed=9):
    """n more batches of the same shape over the same cache: per token a fresh draw of its top-k
    positions over its context, with the rows they name written (random values). Returns
    their index tables (device)."""
    import workloads as wl
    rng = np.random.default_rng(seed)
    lay = c.layout
    T, W = c.idx.shape
    g = torch.Generator(device="cuda").manual_seed(seed)
    out = []
    for _ in range(n):
        idx = np.full((T, W), -1, np.int32)
        for t in range(T):
            v = int(c.valid[t])
            idx[t, :v] = wl.sample_unique(rng, int(lay.ctx[c.tok_req[t]]), v)
        req, pos = wl.referenced_positions(c.tok_req, idx, lay.ctx)
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        slots = smla.smla_resolve_slots(dev(pos[:, None]), None, dev(req), st["pt"], st["ctx"],
                                        lay.page_size)[:, 0].contiguous()
        vals = torch.randn(len(pos), 576, device="cuda", generator=g) * (0.5 if c.kv_dtype == "bf16" else 1.0)
        smla.smla_kv_write(vals.to(torch.bfloat16) if c.kv_dtype == "bf16" else vals, slots, st["kv"])
        out.append(dev(idx))
    torch.cuda.synchronize()
    return out


def time_decode(c, smla, torch, steps, warmup, flush):
    """Cold steps (a 1 GiB read before each) of the fused step, which is one kernel: stage 1
    resolving the logical indices itself and merging the splits at its end. The same for the
    two-kernel form (smla_resolve_slots, then the decode over the resolved slots), and warm /
    graph-replay figures of the fused step."""
    st = setup_decode(c, smla, torch)
    lay = c.layout
    fused, call = st["fused"], st["call"]
    # BATCHES batches of the workload's shape over one cache, stepped through in rotation: a
    # batch's rows come back after BATCHES - 1 other batches (about 600 MB of other rows, more
    # than the 256 MB Infinity Cache), so back-to-back steps read HBM as a decode loop over
    # layers or steps would
    tables = [st["idx"]] + extra_batches(c, st, smla, torch, BATCHES - 1)
    rot = [fused] + [smla.DecodeCall(st["q"], st["kv"], tb, st["valid"], 1, c.scale, st["out"], st["lse"],
                                     workspace=fused.workspace,
                                     page_map=(st["req"], st["pt"], st["ctx"], lay.page_size)) for tb in tables[1:]]

    def resolve():
        smla.smla_resolve_slots(st["idx"], st["valid"], st["req"], st["pt"], st["ctx"], lay.page_size, slots=st["slots"])

    def step():
        fused()

    with section(torch, "form: warm-up"):
        for _ in range(warmup):
            flush.sum()
            step()
            flush.sum()
            resolve()
            call()

    # cold steps: the flush runs between steps, outside the events, on the same stream as the
    # decode kernel, so the event pair brackets exactly its one launch. Python's collector is
    # off meanwhile, so that a collection cannot stall the host between two launches.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    ev2 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    gc.disable()
    with section(torch, "form: fused, cold (isolated launches)"):
        wall0 = time.perf_counter()
        for k in range(steps):
            flush.sum()                       # reads 1 GiB: evicts the caches, leaves nothing dirty
            e = evs[k]
            e[0].record()
            step()
            e[1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
    with section(torch, "form: two kernels, cold (resolve, then decode over slots)"):
        for k in range(steps):
            flush.sum()
            e = ev2[k]
            e[0].record()
            resolve()
            e[1].record()
            call()
            e[2].record()
        torch.cuda.synchronize()
    gc.enable()
    step_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    two = {"step_ms": np.array([e[0].elapsed_time(e[2]) for e in ev2]),
           "resolve_ms": np.array([e[0].elapsed_time(e[1]) for e in ev2]),
           "decode_ms": np.array([e[1].elapsed_time(e[2]) for e in ev2])}

    # the headline form: `steps` steps back to back over the rotating batches, one pair of events
    # around all of them (a barrier and a device synchronise on both sides)
    with section(torch, "form: warm-up"):
        for k in range(warmup):
            rot[k % BATCHES]()
    with section(torch, "form: fused, back to back over rotating batches (the headline)"):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for k in range(steps):
            rot[k % BATCHES]()
        e1.record()
        torch.cuda.synchronize()
    stream_ms = e0.elapsed_time(e1) / steps
    # the same back-to-back loop again with an event after every step, for the spread of the
    # per-step times (the events sit between launches, so this run is reported beside the first)
    with section(torch, "form: fused, back to back, an event after every step"):
        evb = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        evb[0].record()
        for k in range(steps):
            rot[k % BATCHES]()
            evb[k + 1].record()
        torch.cuda.synchronize()
    per_step_ms = np.array([evb[k].elapsed_time(evb[k + 1]) for k in range(steps)])

    # warm steps: back to back, no flush
    with section(torch, "form: fused, warm (one batch, back to back)"):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
    warm_ms = e0.elapsed_time(e1) / steps

    # GRAPH_STEPS steps back to back captured in one HIP graph and replayed (warm): a layer
    # loop's launches without the host in between; the figure is per step
    graph_ms = None
    try:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(GRAPH_STEPS):
                step()
        g.replay()
        torch.cuda.synchronize()
        with section(torch, "form: fused, graph replay (warm)"):
            e0.record()
            for _ in range(steps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / (steps * GRAPH_STEPS)
    except Exception as ex:  # graph capture is a report-only extra
        log(f"graph capture skipped: {ex}")
    return {"step_ms": step_ms, "two_kernel": two, "warm_ms": warm_ms, "graph_ms": graph_ms, "wall_s": wall,
            "splits": fused.splits, "stream_ms": stream_ms, "per_step_ms": per_step_ms}


def time_ragged(c, smla, torch, steps, warmup, flush):
    """Ragged batch with dense requests: the fused top-k decode over the sparse tokens and the
    dense paged decode (page 64, length = context) over the others, on one stream, cold."""
    dev = "cuda"

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    lay = c.layout
    T, H = c.q.shape[0], c.q.shape[1]
    kv = smla.KvCache.empty(smla.SMLA_BF16, lay.num_slots, device=dev)
    smap = smla.smla_resolve_slots(t(c.rows.pos[:, None]), None, t(c.rows.req), t(lay.page_table), t(lay.ctx),
                                   lay.page_size)[:, 0].contiguous()
    smla.smla_kv_write(t(c.rows.values.view(np.int16)).view(torch.bfloat16), smap, kv)
    dense = np.asarray(c.dense_tokens, np.int64)
    sparse = np.setdiff1d(np.arange(T), dense)
    q = c.q.view(np.int16)
    qs, qd = t(q[sparse]).view(torch.bfloat16), t(q[dense]).view(torch.bfloat16)
    out_s = torch.empty((len(sparse), H, 512), dtype=torch.bfloat16, device=dev)
    lse_s = torch.empty((len(sparse), H), dtype=torch.float32, device=dev)
    out_d = torch.empty((len(dense), H, 512), dtype=torch.bfloat16, device=dev)
    lse_d = torch.empty((len(dense), H), dtype=torch.float32, device=dev)
    keep = [t(c.idx[sparse]), t(c.valid[sparse]), t(c.tok_req[sparse]), t(lay.page_table), t(lay.ctx),
            t(lay.page_table[c.tok_req[dense]]), t(lay.ctx[c.tok_req[dense]])]
    fs = smla.DecodeCall(qs, kv, keep[0], keep[1], 1, c.scale, out_s, lse_s,
                         page_map=(keep[2], keep[3], keep[4], lay.page_size))
    fd = smla.DecodeCall(qd, kv, keep[5], keep[6], lay.page_size, c.scale, out_d, lse_d)

    def step():
        fs()
        fd()

    with section(torch, "form: warm-up"):
        for _ in range(warmup):
            flush.sum()
            step()
    with section(torch, "form: cold (isolated steps)"):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for k in range(steps):
            flush.sum()
            ev[k][0].record()
            step()
            ev[k][1].record()
        torch.cuda.synchronize()
    ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    rows = int(c.valid[sparse].sum()) + int(lay.ctx[c.tok_req[dense]].sum())
    alg = rows * 1152 + T * (73728 + 65536 + 256 + 8192)
    m = float(ms.mean())
    return {"workload": f"{c.name}: fused top-k decode over {len(sparse)} tokens + dense paged decode (page "
                        f"{lay.page_size}, length = context) over {len(dense)}, one stream",
            "queries_per_s": T / (m / 1e3), "ms_per_step": m, "step_median_us": float(np.median(ms)) * 1e3,
            "rows": rows, "algorithmic_bytes_step": alg, "hbm_gbs_step": alg / (m / 1e3) / 1e9,
            "hbm_frac_step": alg / (m / 1e3) / 1e9 / HBM_PEAK_GBS,
            "splits": {"sparse": fs.splits, "dense": fd.splits}}


def time_kv_write(smla, torch, steps, warmup, flush, rows=1 << 20):
    """smla_kv_write of `rows` bf16 rows into a bf16 pool and into an fp8 pool (e4m3 codes +
    bf16 rope + fp32 scale per row), slots dealt as whole 64-slot pages in a seeded random
    order (the page layout of the decode workloads), cold."""
    gen = torch.Generator(device="cpu").manual_seed(7)
    src = (torch.randn((rows, 576), generator=gen) * 0.5).to(torch.bfloat16).cuda()
    pages = torch.randperm(rows // 64, generator=gen).to(torch.int64)
    smap = (pages[:, None] * 64 + torch.arange(64)[None, :]).reshape(-1).to(torch.int32).cuda()
    res = {"workload": f"{rows} bf16 rows of 576, slots in 64-slot pages dealt in random order"}
    for name, code, row_out in (("bf16", smla.SMLA_BF16, 1152), ("fp8", smla.SMLA_FP8_E4M3, 644)):
        kv = smla.KvCache.empty(code, rows, device="cuda", poison=False)
        with section(torch, f"form: {name} pool"):
            for _ in range(warmup):
                smla.smla_kv_write(src, smap, kv)
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
            for k in range(steps):
                flush.sum()
                ev[k][0].record()
                smla.smla_kv_write(src, smap, kv)
                ev[k][1].record()
            torch.cuda.synchronize()
        ms = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))   # median: a first touch can stall one step
        alg = rows * (1152 + 4 + row_out)                  # source row + slot index + stored payload
        res[name] = {"us": ms * 1e3, "algorithmic_bytes": alg, "hbm_gbs": alg / (ms / 1e3) / 1e9,
                     "hbm_frac": alg / (ms / 1e3) / 1e9 / HBM_PEAK_GBS}
        del kv
    return res


def gather_ceiling(torch, flush, steps, rows=1 << 16, pool_rows=1 << 20):
    """Context for the decode's HBM figures, measured on this GPU with torch's own kernels (not
    libsmla): torch.index_select of `rows` random 1,152-byte rows out of a pool of `pool_rows`
    (each row read once and written once), and a plain copy of 1 GiB, both cold (a 1 GiB read
    before each), as GB/s of bytes read + written."""
    pool = torch.zeros((pool_rows, 576), dtype=torch.bfloat16, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(5)
    idx = torch.rand(pool_rows, device="cuda", generator=g).argsort()[:rows]
    out = torch.empty((rows, 576), dtype=torch.bfloat16, device="cuda")
    src = torch.ones((1 << 30) // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)

    def cold(fn):
        for _ in range(2):
            flush.sum()
            fn()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for k in range(steps):
            flush.sum()
            ev[k][0].record()
            fn()
            ev[k][1].record()
        torch.cuda.synchronize()
        return float(np.median([e[0].elapsed_time(e[1]) for e in ev]))

    with section(torch, "form: index_select of random rows"):
        tg = cold(lambda: torch.index_select(pool, 0, idx, out=out))
    with section(torch, "form: 1 GiB copy"):
        tc = cold(lambda: dst.copy_(src))
    gb = 2 * rows * 1152
    res = {"what": "torch kernels on this GPU, cold, median: index_select of 65,536 random 1,152-byte rows of a 2^20-row "
                   "pool (read + write), and a 1 GiB device copy (read + write); context for the HBM fractions, "
                   "not the roofline peak",
           "index_select_rows_gbs": gb / (tg / 1e3) / 1e9, "copy_gbs": 2 * (1 << 30) / (tc / 1e3) / 1e9}
    del pool, out, src, dst
    torch.cuda.empty_cache()
    return res


def time_decode_h128(smla, torch, steps, warmup, T=32, W=2048, n=1 << 20):
    """Decode with 128 heads per token (two blocks of 64 head slots), batch T, top-k W, over a
    bf16 pool of n random rows: the index lists are fresh unique draws, back to back over 8
    batches in rotation (a batch's rows return after ~530 MB of other rows)."""
    kv = smla.KvCache.empty(smla.SMLA_BF16, n, device="cuda", poison=False)
    kv.storage.normal_(0.0, 0.5)
    g = torch.Generator(device="cuda").manual_seed(128)
    q = (torch.randn(T, 128, 576, device="cuda", generator=g) * 0.5).to(torch.bfloat16)
    out = torch.empty((T, 128, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, 128), dtype=torch.float32, device="cuda")
    lens = torch.full((T,), W, dtype=torch.int32, device="cuda")
    tables = [torch.rand(T, n, device="cuda", generator=g).argsort(dim=1)[:, :W].to(torch.int32).contiguous()
              for _ in range(BATCHES)]
    calls = [smla.DecodeCall(q, kv, tables[0], lens, 1, 1 / 16, out, lse)]
    calls += [smla.DecodeCall(q, kv, tb, lens, 1, 1 / 16, out, lse, workspace=calls[0].workspace) for tb in tables[1:]]
    with section(torch, "form: warm-up"):
        for k in range(warmup):
            calls[k % BATCHES]()
    with section(torch, "form: back to back over rotating batches"):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for k in range(steps):
            calls[k % BATCHES]()
        e1.record()
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    alg = T * W * 1152 + T * 128 * (576 + 512) * 2 + T * 128 * 4 + T * W * 4
    del kv, tables
    torch.cuda.empty_cache()
    return {"workload": f"sparse MLA decode, bf16, batch {T}, 128 heads (two blocks of 64 head slots), top-k {W}, "
                        f"{n}-slot pool, resolved slot tables, 8 rotating batches back to back",
            "queries_per_s": T / (ms / 1e3), "ms_per_step": ms, "algorithmic_bytes_step": alg,
            "hbm_gbs_step": alg / (ms / 1e3) / 1e9, "hbm_frac_step": alg / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
            "splits": calls[0].splits}


def time_dense_paged(smla, torch, steps, warmup, flush, T=64, lo=32768, hi=65536, page=64):
    """Dense paged decode (the block-table case, page size 64, length = context) of T tokens with
    contexts uniform in [lo, hi], bf16, over a page-permuted pool holding exactly their pages: the
    splits are planned on the device from the lengths. Cold steps (the flush before each)."""
    rng = np.random.default_rng(64)
    ctx = rng.integers(lo, hi + 1, size=T).astype(np.int32)
    npages = -(-ctx // page)
    width = int(npages.max())
    total = int(npages.sum())
    perm = rng.permutation(total).astype(np.int32)
    table = np.full((T, width), -1, np.int32)
    off = 0
    for t in range(T):
        table[t, :npages[t]] = perm[off:off + npages[t]]
        off += npages[t]
    kv = smla.KvCache.empty(smla.SMLA_BF16, total * page, device="cuda", poison=False)
    kv.storage.normal_(0.0, 0.5)
    g = torch.Generator(device="cuda").manual_seed(65)
    q = (torch.randn(T, 64, 576, device="cuda", generator=g) * 0.5).to(torch.bfloat16)
    out = torch.empty((T, 64, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, 64), dtype=torch.float32, device="cuda")
    call = smla.DecodeCall(q, kv, torch.from_numpy(table).cuda(), torch.from_numpy(ctx).cuda(), page, 1 / 16, out, lse)
    with section(torch, "form: warm-up"):
        for _ in range(warmup):
            flush.sum()
            call()
    with section(torch, "form: cold (isolated launches)"):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for k in range(steps):
            flush.sum()
            ev[k][0].record()
            call()
            ev[k][1].record()
        torch.cuda.synchronize()
    ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    rows = int(ctx.sum())
    alg = rows * 1152 + T * (73728 + 65536 + 256) + int(npages.sum()) * 4
    m = float(np.median(ms))
    del kv
    torch.cuda.empty_cache()
    return {"workload": f"dense paged decode, bf16, {T} tokens, contexts U[{lo}, {hi}], page {page}, splits planned on "
                        f"the device from the lengths; cold (1 GiB read before each step)",
            "rows": rows, "step_median_us": m * 1e3, "step_p10_us": float(np.percentile(ms, 10)) * 1e3,
            "step_p90_us": float(np.percentile(ms, 90)) * 1e3, "algorithmic_bytes_step": alg,
            "hbm_gbs_step": alg / (m / 1e3) / 1e9, "hbm_frac_step": alg / (m / 1e3) / 1e9 / HBM_PEAK_GBS}


def prefill_flop_done(enc, lens, G, H):
    """FLOP the grouped-prefill kernel issues: its workgroups each serve 64 / H members of a group
    (64 head slots) and walk the group's union entries that name one of them, 2 * (576 + 512)
    FLOP per (entry, head slot)."""
    enc = enc.cpu().numpy().view(np.uint32)
    lens = lens.cpu().numpy()
    mpw = 64 // H
    total = 0
    for g in range(len(lens)):
        bits = enc[g, :int(lens[g])] >> 24
        for m0 in range(0, G, mpw):
            total += int(np.count_nonzero(bits & (((1 << mpw) - 1) << m0)))
    return float(total) * 64 * 2 * (576 + 512)


MFMA_BF16_PEAK_TFLOPS = 2500.0
PREFILL_KERNEL = {"bf16": "decode_stage1_mfma<bf16, union>", "fp8": "decode_stage1_mfma<fp8, union>"}


def time_prefill(c, smla, torch, steps, warmup, flush, cpu_seconds, kv_dtype="bf16"):
    """Grouped sparse prefill (union build + grouped attention) on case `c`, over a bf16 or an fp8
    cache written from the case's rows: cold steps (the flush before each), each kernel alone and
    the two together, against the bf16 MFMA peak; the oracle on a bounded sample of groups."""
    dev = "cuda"

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    lay = c.layout
    Q, H = c.q.shape[0], c.q.shape[1]
    kv = smla.KvCache.empty(smla.SMLA_BF16 if kv_dtype == "bf16" else smla.SMLA_FP8_E4M3, lay.num_slots, device=dev)
    smap = smla.smla_resolve_slots(t(c.rows.pos[:, None]), None, t(c.rows.req), t(lay.page_table), t(lay.ctx),
                                   lay.page_size)[:, 0].contiguous()
    smla.smla_kv_write(t(c.rows.values.view(np.int16)).view(torch.bfloat16), smap, kv)
    req = t(np.zeros(Q, np.int32))
    slots = smla.smla_resolve_slots(t(c.idx), t(c.valid), req, t(lay.page_table), t(lay.ctx), lay.page_size)
    valid = t(c.valid)
    q = t(c.q.view(np.int16)).view(torch.bfloat16)
    enc, lens = smla.smla_build_group_union(slots, valid, c.G, lay.num_slots)
    out = torch.empty((Q, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((Q, H), dtype=torch.float32, device=dev)

    def union():
        smla.smla_build_group_union(slots, valid, c.G, lay.num_slots, enc=enc, lens=lens)

    def prefill():
        smla.smla_grouped_prefill(q, kv, enc, lens, c.G, c.scale, out=out, lse=lse)

    with section(torch, "form: warm-up"):
        for _ in range(warmup):
            flush.sum()
            union()
            prefill()
    with section(torch, f"form: union over the {lay.num_slots}-slot pool, then attention, cold"):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for k in range(steps):
            flush.sum()
            ev[k][0].record()
            union()
            ev[k][1].record()
            prefill()
            ev[k][2].record()
        torch.cuda.synchronize()
    u_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    p_ms = np.array([e[1].elapsed_time(e[2]) for e in ev])
    both = np.array([e[0].elapsed_time(e[2]) for e in ev])
    # the same lists over a 2^20-slot pool (the slots mapped one to one onto a random subset of
    # it, in order): the union builder's bit map then spans 2^20 rows
    union_big = None
    if kv_dtype == "bf16":
        big = 1 << 20
        gen = torch.Generator(device="cuda").manual_seed(11)
        remap = torch.sort(torch.randperm(big, device="cuda", generator=gen)[:lay.num_slots])[0].to(torch.int32)
        slots_big = torch.where(slots >= 0, remap[slots.clamp(min=0).long()], slots).contiguous()
        ub = []
        with section(torch, "form: union over a 2^20-slot pool, cold"):
            enc_b, lens_b = smla.smla_build_group_union(slots_big, valid, c.G, big)
            for k in range(steps + 2):
                flush.sum()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                smla.smla_build_group_union(slots_big, valid, c.G, big, enc=enc_b, lens=lens_b)
                e1.record()
                torch.cuda.synchronize()
                if k >= 2:
                    ub.append(e0.elapsed_time(e1))
        assert torch.equal(lens_b, lens)                   # the same union sizes as over the small pool
        union_big = float(np.median(ub)) * 1e3
        del slots_big, enc_b, lens_b, remap
    n_union = int(lens.sum().item())
    flop_alg = float(c.valid.astype(np.int64).sum()) * H * 2 * (576 + 512)
    flop_done = prefill_flop_done(enc, lens, c.G, H)
    p_mean = float(p_ms.mean())
    res = {"workload": f"{c.name}: union build + grouped attention; {kv_dtype} KV pool of {lay.num_slots} slots "
                       f"(cache-resident)",
           "queries": Q, "group": c.G, "kv_dtype": kv_dtype, "union_rows": n_union,
           "union_over_topk": n_union / float(c.valid.sum()) * c.G,
           "step_ms": float(both.mean()), "union_us": float(u_ms.mean()) * 1e3,
           "union_us_pool_2e20": union_big, "prefill_ms": p_mean,
           "prefill_p10_ms": float(np.percentile(p_ms, 10)), "prefill_p90_ms": float(np.percentile(p_ms, 90)),
           "tokens_per_s": Q / (float(both.mean()) / 1e3),
           "roofline": {"bound": "mfma", "kernel": PREFILL_KERNEL[kv_dtype], "achieved": flop_alg / (p_mean / 1e3) / 1e12,
                        "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": flop_alg / (p_mean / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                        "algorithmic_flop_per_launch": flop_alg, "issued_flop_per_launch": flop_done,
                        "issued_tflops": flop_done / (p_mean / 1e3) / 1e12, "avg_launch_us": p_mean * 1e3}}
    if cpu_seconds > 0:
        import oracle
        pool = oracle.Pool(lay.num_slots, "bf16")
        osl = oracle.resolve_slots(c.rows.pos[:, None], None, c.rows.req, lay.page_table, lay.ctx, lay.page_size)[:, 0]
        oracle.kv_write(pool, c.rows.values, "bf16", osl)
        n_groups = -(-Q // c.G)
        req_h = np.zeros(Q, np.int32)
        done, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < cpu_seconds:
            g = done % n_groups
            mem = np.arange(g * c.G, min(g * c.G + c.G, Q))
            osl_g = oracle.resolve_slots(c.idx[mem], c.valid[mem], req_h[mem], lay.page_table, lay.ctx, lay.page_size)
            enc_g, lens_g = oracle.group_union(osl_g, c.valid[mem], c.G, lay.num_slots)
            oracle.grouped_prefill(c.q[mem], pool, enc_g, lens_g, c.G, c.scale)
            done += 1
        el = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": done * c.G / el, "unit": "queries/s", "kind": "oracle",
                               "sample": f"{done} groups ({done * c.G} queries) of the same workload: resolve, union "
                                         f"and fp64 grouped attention per group, {el:.1f} s wall on the host"}
    return res


def cpu_model() -> str:
    """The host CPU's model name (as lscpu reports it)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def host_threads() -> int:
    """Cores this process may run on, capped at the 16 host cores one GPU's share of the box has."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _oracle_decode_queries(d: str, tokens, seconds: float, start_at: float):
    """One oracle process: resolve + fp64 attention of the given tokens, one token at a time,
    for `seconds` from the wall-clock time `start_at`, with one BLAS thread. The workload's
    arrays come memory-mapped from directory d. Returns the number of queries done."""
    from threadpoolctl import threadpool_limits
    import oracle
    a = {k[:-4]: np.load(os.path.join(d, k), mmap_mode="r") for k in os.listdir(d) if k.endswith(".npy")}
    meta = json.load(open(os.path.join(d, "meta.json")))
    # the cache the oracle's own kv_write stored (written once, by the parent)
    pool = oracle.Pool(meta["num_slots"], meta["kv_dtype"])
    pool.store(a["pool_slots"], {k[6:]: np.asarray(v) for k, v in a.items() if k.startswith("plane_")})
    done = 0
    with threadpool_limits(1):
        while time.time() < start_at:
            time.sleep(0.005)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            t = int(tokens[done % len(tokens)])
            sl = oracle.resolve_slots(a["idx"][t:t + 1], a["valid"][t:t + 1], a["tok_req"][t:t + 1], a["page_table"],
                                      a["ctx"], meta["page_size"])
            oracle.sparse_decode(np.asarray(a["q"][t:t + 1]), meta["q_dtype"], pool, sl, a["valid"][t:t + 1], 1,
                                 meta["scale"])
            done += 1
    return done


def cpu_baseline(c, seconds: float) -> dict:
    """The oracle (plain numpy fp64, as it stands) on the host: decode queries of the workload
    (resolve + attention per token). Two rates: one core (one process, one BLAS thread) for a
    third of `seconds`, and all cores (one process per core, each one BLAS thread, over its
    share of the tokens) for the rest. Runs before anything touches the GPU, so that the worker
    processes start from a process without GPU state."""
    import concurrent.futures as cf
    import multiprocessing as mp
    import shutil
    import tempfile
    lay = c.layout
    d = tempfile.mkdtemp(prefix="smla_oracle_")
    try:
        import oracle
        pool = oracle.Pool(lay.num_slots, c.kv_dtype)
        osl = oracle.resolve_slots(c.rows.pos[:, None], None, c.rows.req, lay.page_table, lay.ctx, lay.page_size)[:, 0]
        oracle.kv_write(pool, c.rows.values, "bf16" if c.rows.values.dtype == np.uint16 else "f32", osl)
        written = np.unique(osl[osl >= 0])
        arrays = {"pool_slots": written, "page_table": lay.page_table, "ctx": lay.ctx, "idx": c.idx,
                  "valid": c.valid, "tok_req": c.tok_req, "q": c.q}
        arrays.update({"plane_" + k: v for k, v in pool.stored(written).items()})
        del pool
        for k, v in arrays.items():
            np.save(os.path.join(d, k + ".npy"), np.ascontiguousarray(v))
        json.dump({"num_slots": int(lay.num_slots), "kv_dtype": c.kv_dtype, "page_size": int(lay.page_size),
                   "q_dtype": c.q_dtype, "scale": float(c.scale)}, open(os.path.join(d, "meta.json"), "w"))
        T = c.q.shape[0]
        s1 = seconds / 3
        n1 = _oracle_decode_queries(d, np.arange(T), s1, time.time())
        n = host_threads()
        s2 = seconds - s1
        env = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
        for k in env:
            os.environ[k] = "1"
        try:
            with cf.ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn")) as ex:
                start_at = time.time() + 5.0                  # every worker has started and loaded by then
                futs = [ex.submit(_oracle_decode_queries, d, np.arange(i, T, n) if i < T else np.arange(T), s2,
                                  start_at) for i in range(n)]
                counts = [f.result() for f in futs]
        finally:
            for k, v in env.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
    finally:
        shutil.rmtree(d, ignore_errors=True)
    rate_all = sum(counts) / s2
    return {"value": rate_all, "unit": "queries/s", "cores": n, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{sum(counts)} decode queries of the same workload (resolve + fp64 attention per token, "
                      f"tokens dealt over {n} processes of one BLAS thread each), {s2:.1f} s wall on the host",
            "single_core": {"value": n1 / s1, "unit": "queries/s", "cores": 1,
                            "sample": f"{n1} decode queries, one process, one BLAS thread, {s1:.1f} s wall"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-ragged", action="store_true")
    ap.add_argument("--no-kv-write", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the context rows: 128-head decode, fp8 grouped prefill, dense paged decode, gather ceiling")
    ap.add_argument("--flush-mib", type=int, default=1024)
    ap.add_argument("--overlap-sweep", action="store_true",
                    help="only time grouped prefill against per-query decode for G = 2 / 4 / 8 over list "
                         "overlaps 0 .. 1 and print the table (markdown); no JSON line")
    ap.add_argument("--split-sweep", action="store_true",
                    help="only time the decode against its split count for batches 1 .. 128 (bf16 and fp8, "
                         "top-k 2048) and print the table (markdown); no JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="end with three plain 256 MiB fp32 copy kernels (y = x * 1), whose HBM counter "
                         "readings give the scale for the decode kernels' FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--summarize-profile", nargs="+", metavar=("KIND", "DIR"),
                    help="no GPU work: reduce rocprofv3 output directories into a profiles/ table. KIND trace DIR | "
                         "traffic FETCH_DIR WRITE_DIR | sq DIR_A DIR_B")
    args = ap.parse_args()
    if args.summarize_profile:
        summarize_profile(args.summarize_profile)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: libsmla has no multi-GPU path (decode would shard by request, with no "
              "exchange between GPUs). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import workloads as wl
    sweeping = args.split_sweep or args.overlap_sweep
    c2 = None
    cpu = None
    if not sweeping:
        log("generating the bf16 decode workload (batch 32, top-k 2048)")
        c2 = wl.decode_bf16_b32()
        if not args.no_cpu_baseline:
            # before anything touches the GPU: the oracle's worker processes start from this one
            log(f"timing the CPU oracle for about {args.cpu_seconds:.0f} s")
            cpu = cpu_baseline(c2, args.cpu_seconds)
            log(f"oracle: {cpu['single_core']['value']:.0f} queries/s on one core, {cpu['value']:.0f} on "
                f"{cpu['cores']} ({cpu['cpu_model']})")

    import torch
    import sparse_mla_attention_resolve_amd as smla

    if not os.path.exists(smla.LIB_PATH):
        raise SystemExit("libsmla.so is not built: run python -m sparse_mla_attention_resolve_amd.build")
    torch.cuda.set_device(0)
    flush = torch.ones((args.flush_mib << 20) // 4, dtype=torch.float32, device="cuda")
    if args.split_sweep:
        print(split_sweep_markdown(split_sweep(smla, torch, flush, max(5, args.steps // 2))), end="", flush=True)
        return
    if args.overlap_sweep:
        n = max(3, args.steps // 10)
        print(overlap_sweep_markdown(overlap_sweep(smla, torch, flush, n), n), end="", flush=True)
        return

    ab = algorithmic_bytes(c2, "bf16")
    log("timing bf16 decode")
    with section(torch, "workload: bf16 decode, batch 32"):
        r = time_decode(c2, smla, torch, args.steps, args.warmup, flush)
    T = c2.q.shape[0]
    step_ms = r["stream_ms"]
    value = T / (step_ms / 1e3)
    step_gbs = ab["step"] / (step_ms / 1e3) / 1e9
    iso_ms = float(r["step_ms"].mean())
    two = r["two_kernel"]
    ps = r["per_step_ms"]
    log(f"step {step_ms*1e3:.1f} us back to back over {BATCHES} rotating batches (one kernel: {step_gbs:.0f} GB/s "
        f"of algorithmic bytes; per-step p10/p50/p90 {np.percentile(ps, 10)*1e3:.1f}/{np.median(ps)*1e3:.1f}/"
        f"{np.percentile(ps, 90)*1e3:.1f} us); one isolated cold launch {iso_ms*1e3:.1f} us; warm "
        f"{r['warm_ms']*1e3:.1f} us; graph {(r['graph_ms'] or 0)*1e3:.1f} us. Two-kernel form: "
        f"{two['step_ms'].mean()*1e3:.1f} us (resolve {two['resolve_ms'].mean()*1e3:.1f}, decode "
        f"{two['decode_ms'].mean()*1e3:.1f})")

    def us(a):
        return float(np.mean(a)) * 1e3

    line = {
        "metric": METRIC, "value": value, "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": step_ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "sparse MLA decode, bf16 q and KV, batch 32, 64 heads, latent 512 + rope 64, "
                               "contexts U[8K,32K], 2^20-slot pool of 64-slot pages, top-k 2048; step = one "
                               "kernel: slot resolution, split decode and LSE merge of the splits; steps back "
                               "to back over 8 batches of fresh top-k draws in rotation (a batch's rows return "
                               "after ~600 MB of other rows), inputs HBM-resident",
                   "batch": T, "heads": 64, "topk": 2048, "splits": r["splits"], "parallelism": "none (1 GPU)"},
        "hbm_gbs_step": step_gbs, "hbm_frac_step": step_gbs / HBM_PEAK_GBS,
        "algorithmic_bytes_step": ab["step"],
        "timing_us": {"step_back_to_back": step_ms * 1e3,
                      "per_step_events": {"what": "the back-to-back loop rerun with an event recorded after every "
                                                  "step; the events between launches lengthen each step a little",
                                          "p10": float(np.percentile(ps, 10)) * 1e3, "p50": float(np.median(ps)) * 1e3,
                                          "p90": float(np.percentile(ps, 90)) * 1e3, "mean": float(ps.mean()) * 1e3},
                      "isolated_cold_launch_mean": iso_ms * 1e3,
                      "isolated_cold_launch_median": float(np.median(r["step_ms"])) * 1e3,
                      "isolated_cold_launch_p10": float(np.percentile(r["step_ms"], 10)) * 1e3,
                      "isolated_cold_launch_p90": float(np.percentile(r["step_ms"], 90)) * 1e3,
                      "warm_step": r["warm_ms"] * 1e3,
                      "graph_replay_step": None if r["graph_ms"] is None else r["graph_ms"] * 1e3,
                      "graph_steps_per_replay": GRAPH_STEPS,
                      "two_kernel_form": {"step": us(two["step_ms"]), "resolve": us(two["resolve_ms"]),
                                          "decode": us(two["decode_ms"])}},
        "roofline": {"bound": "hbm", "kernel": "decode_stage1_mfma<bf16>", "achieved": step_gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": step_gbs / HBM_PEAK_GBS,
                     "algorithmic_bytes_per_launch": ab["step"], "avg_launch_us": step_ms * 1e3,
                     "traffic": measured_traffic("decode_stage1_mfma<bf16>", "bf16_batch_32")},
    }

    if not args.no_fp8:
        log("generating the fp8-KV decode workload (batch 64)")
        c5 = wl.decode_fp8_b64()
        ab5 = algorithmic_bytes(c5, "fp8")
        log("timing fp8-KV decode")
        with section(torch, "workload: fp8 decode, batch 64"):
            r5 = time_decode(c5, smla, torch, args.steps, args.warmup, flush)
        ms5 = r5["stream_ms"]
        two5 = r5["two_kernel"]
        gbs5 = ab5["step"] / (ms5 / 1e3) / 1e9
        ps5 = r5["per_step_ms"]
        line["fp8_kv_decode"] = {
            "workload": "batch 64, 64 heads, fp8 e4m3 latent + bf16 rope + fp32 scale per row, context 64K, top-k 2048",
            "queries_per_s": c5.q.shape[0] / (ms5 / 1e3), "ms_per_step": ms5,
            "hbm_gbs_step": gbs5, "hbm_frac_step": gbs5 / HBM_PEAK_GBS,
            "algorithmic_bytes_step": ab5["step"],
            "per_step_us_p10_p50_p90": [float(np.percentile(ps5, 10)) * 1e3, float(np.median(ps5)) * 1e3,
                                        float(np.percentile(ps5, 90)) * 1e3],
            "isolated_cold_launch_us": float(np.mean(r5["step_ms"])) * 1e3,
            "warm_step_us": r5["warm_ms"] * 1e3, "splits": r5["splits"],
            "roofline": {"bound": "hbm", "kernel": "decode_stage1_mfma<fp8>", "achieved": gbs5, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": gbs5 / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": ab5["step"],
                         "avg_launch_us": ms5 * 1e3,
                         "traffic": measured_traffic("decode_stage1_mfma<fp8>", "fp8_batch_64")},
            "two_kernel_form_us": {"step": us(two5["step_ms"]), "resolve": us(two5["resolve_ms"]),
                                   "decode": us(two5["decode_ms"])}}
        log(f"fp8: step {ms5*1e3:.1f} us back to back (isolated cold launch {np.mean(r5['step_ms'])*1e3:.1f}; "
            f"{gbs5:.0f} GB/s); two-kernel form {us(two5['step_ms']):.1f} us")
        del c5

    if not args.no_ragged:
        log("generating the ragged decode workload (batch 128, 13 dense requests)")
        c3 = wl.decode_ragged_b128()
        log("timing ragged decode")
        with section(torch, "workload: ragged decode, batch 128"):
            rg = time_ragged(c3, smla, torch, args.steps, args.warmup, flush)
        line["ragged_decode"] = rg
        log(f"ragged: step {rg['ms_per_step']*1e3:.1f} us ({rg['hbm_gbs_step']:.0f} GB/s over {rg['rows']} rows)")

    if not args.no_prefill:
        log("generating the grouped-prefill workload (8192 queries on 16384 cached, G = 2)")
        c4 = wl.prefill_grouped_q8192()
        log("timing grouped prefill")
        with section(torch, "workload: grouped prefill, bf16 cache"):
            pr = time_prefill(c4, smla, torch, max(3, args.steps // 5), 2, flush,
                              0.0 if args.no_cpu_baseline else min(5.0, args.cpu_seconds))
        line["grouped_prefill"] = pr
        log(f"grouped prefill: union {pr['union_us']:.0f} us ({pr['union_us_pool_2e20']:.0f} us over a 2^20-slot pool) "
            f"+ attention {pr['prefill_ms']:.2f} ms "
            f"({pr['roofline']['achieved']:.0f} TFLOP/s algorithmic, {pr['roofline']['issued_tflops']:.0f} issued)")
        if not args.no_extra:
            log("timing grouped prefill over an fp8 cache")
            with section(torch, "workload: grouped prefill, fp8 cache"):
                pf = time_prefill(c4, smla, torch, max(3, args.steps // 5), 2, flush, 0.0, kv_dtype="fp8")
            line["grouped_prefill_fp8"] = pf
            log(f"grouped prefill (fp8 cache): union {pf['union_us']:.0f} us + attention {pf['prefill_ms']:.2f} ms "
                f"({pf['roofline']['achieved']:.0f} TFLOP/s algorithmic)")
        del c4

    if not args.no_extra:
        log("timing dense paged decode (64 tokens, contexts 32K-64K)")
        with section(torch, "workload: dense paged decode, 64 tokens of 32K-64K"):
            dp = time_dense_paged(smla, torch, max(5, args.steps // 2), 3, flush)
        line["dense_paged_decode"] = dp
        log(f"dense paged: {dp['step_median_us']:.1f} us over {dp['rows']} rows ({dp['hbm_gbs_step']:.0f} GB/s)")
        log("timing 128-head decode (batch 32, top-k 2048)")
        with section(torch, "workload: bf16 decode, 128 heads, batch 32"):
            h1 = time_decode_h128(smla, torch, args.steps, args.warmup)
        line["decode_h128"] = h1
        log(f"128 heads: step {h1['ms_per_step']*1e3:.1f} us ({h1['hbm_gbs_step']:.0f} GB/s)")
        log("measuring the gather and copy ceilings (torch kernels)")
        with section(torch, "workload: gather and copy ceilings (torch kernels)"):
            line["context_ceilings"] = gather_ceiling(torch, flush, max(5, args.steps // 5))
        log(f"index_select of random rows {line['context_ceilings']['index_select_rows_gbs']:.0f} GB/s, "
            f"copy {line['context_ceilings']['copy_gbs']:.0f} GB/s")

    if not args.no_kv_write:
        log("timing smla_kv_write (1M rows)")
        with section(torch, "workload: kv_write, 1M rows"):
            kw = time_kv_write(smla, torch, max(5, args.steps // 5), 3, flush)
        line["kv_write"] = kw
        log(f"kv_write: bf16 {kw['bf16']['us']:.0f} us ({kw['bf16']['hbm_gbs']:.0f} GB/s), fp8 {kw['fp8']['us']:.0f} us "
            f"({kw['fp8']['hbm_gbs']:.0f} GB/s)")

    if cpu is not None:
        line["cpu_baseline"] = cpu
    if args.copy_calibration:
        x = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        with section(torch, "workload: copy calibration"):
            for _ in range(3):
                flush.sum()
                torch.mul(x, 1.0, out=y)
        log("copy calibration: 3 x (read 256 MiB, write 256 MiB)")
    print(json.dumps(line), flush=True)


# ---- profile summaries (no GPU work): rocprofv3 CSV output -> the tables under profiles/

PROFILE_DIR = os.path.join(ROOT, "profiles")
CSRC = "sparse_mla_attention_resolve_amd/csrc/"
ALL_KERNEL_SOURCES = [CSRC + f for f in ("decode.hip", "union.hip", "resolve.hip", "kv_write.hip", "prefill.hip",
                                          "abi.hip", "stage1_common.h", "smla_device.h", "smla_internal.h")] + ["include/smla.h"]
# the commands whose output the summaries reduce (run from the repository root); the summary
# documents quote them
BENCH_TRACE = "python3 bench.py --steps 30 --warmup 5 --no-cpu-baseline"
BENCH_PMC = ("python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-ragged --no-prefill --no-extra "
             "--no-kv-write --copy-calibration")
BENCH_SQ = "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-ragged --no-extra --no-kv-write"
SQ_PASSES = {"A": "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_LDS_ADDR_CONFLICT SQ_LDS_DATA_FIFO_FULL SQ_INSTS_LDS "
                  "SQ_BUSY_CU_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_WAVE_CYCLES",
             "B": "SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS SQ_ACTIVE_INST_LDS SQ_INST_LEVEL_LDS SQ_BUSY_CYCLES "
                  "SQ_ACTIVE_INST_VALU SQ_INSTS_VALU_MFMA_MOPS_BF16"}


def profile_commands(kind: str, dirs) -> list:
    """The shell commands that produce and reduce one kind of profile, with `dirs` its output
    directories (relative to the repository root)."""
    if kind == "trace":
        d = dirs[0]
        return [f"mkdir -p {d}",
                f"rocprofv3 --kernel-trace --marker-trace --stats --output-format csv -d {d} -o run -- "
                f"{BENCH_TRACE} > {d}/bench.json 2> {d}/bench.err",
                f"python3 bench.py --summarize-profile trace {d}"]
    if kind == "traffic":
        fd, wd = dirs
        return [f"mkdir -p {fd} {wd}",
                f"rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d {fd} -o run -- {BENCH_PMC} "
                f"> {fd}/bench.json 2> {fd}/bench.err",
                f"rocprofv3 --pmc WRITE_SIZE --kernel-trace --output-format csv -d {wd} -o run -- {BENCH_PMC} "
                f"> {wd}/bench.json 2> {wd}/bench.err",
                f"python3 bench.py --summarize-profile traffic {fd} {wd}"]
    if kind == "sq":
        da, db = dirs
        return [f"mkdir -p {da} {db}"] + [
            f"rocprofv3 --pmc {SQ_PASSES[p]} --kernel-trace --output-format csv -d {d} -o run -- {BENCH_SQ} "
            f"> {d}/bench.json 2> {d}/bench.err" for p, d in (("A", da), ("B", db))] + [
            f"python3 bench.py --summarize-profile sq {da} {db}"]
    raise ValueError(kind)


def sources_sha256(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


_KV_NAMES = {"1": "bf16", "2": "fp8"}
_KERNEL_RULES = [
    (re.compile(r"decode_stage1_mfma<(\d+), (true|false)(?:, (?:true|false))*>"),
     lambda m: f"decode_stage1_mfma<{_KV_NAMES.get(m.group(1), m.group(1))}{', union' if m.group(2) == 'true' else ''}>"),
    (re.compile(r"decode_stage1_f32\b"), lambda m: "decode_stage1_f32"),
    (re.compile(r"decode_stage2_packed\b"), lambda m: "decode_stage2_packed"),
    (re.compile(r"decode_stage2\b"), lambda m: "decode_stage2"),
    (re.compile(r"resolve_kernel\b"), lambda m: "resolve_kernel"),
    (re.compile(r"union_bitmap_kernel<(\d+)>"), lambda m: f"union_bitmap_kernel<{m.group(1)}>"),
    (re.compile(r"union_sort_kernel<(\d+), (\d+)>"), lambda m: f"union_sort_kernel<{m.group(1)}, {m.group(2)}>"),
    (re.compile(r"kv_write_kernel\b"), lambda m: "kv_write_kernel"),
    (re.compile(r"zero_kernel\b"), lambda m: "zero_kernel"),
]


def kernel_label(name: str):
    """Short name of a libsmla kernel from its demangled name; None for any other kernel."""
    for rx, f in _KERNEL_RULES:
        m = rx.search(name)
        if m:
            return f(m)
    return None


def torch_label(name: str) -> str:
    """'torch <kernel>' for another library's kernel: its function name without scope or
    template arguments."""
    base = re.split(r"[<(]", name.replace("(anonymous namespace)::", ""), maxsplit=1)[0].strip()
    return "torch " + (base.split("::")[-1].split() or ["?"])[-1]


def _read_csv(path):
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def _grid(r) -> int:
    if "Grid_Size" in r:
        return int(r["Grid_Size"])
    return int(r.get("Grid_Size_X", 0)) * int(r.get("Grid_Size_Y", 1)) * int(r.get("Grid_Size_Z", 1))


def _bench_line(d):
    """The JSON line that the profiled bench run printed (d/bench.json), or None."""
    try:
        for ln in open(os.path.join(d, "bench.json")):
            if ln.startswith("{"):
                return json.loads(ln)
    except OSError:
        pass
    return None


def _write_profile(name: str, lines) -> None:
    path = os.path.join(PROFILE_DIR, name)
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"wrote {os.path.relpath(path, ROOT)}")


def _fmt_cmds(kind, dirs):
    return ["```"] + profile_commands(kind, dirs) + ["```", ""]


def summarize_trace(d: str) -> None:
    """profiles/decode_prefill_kernels_trace.md from a kernel + marker trace of the full bench:
    every libsmla dispatch (and the torch kernels of the ceiling and calibration sections)
    labelled with the bench section (workload) and form it ran in."""
    kt = sorted(_read_csv(os.path.join(d, "run_kernel_trace.csv")), key=lambda r: int(r["Start_Timestamp"]))
    mpath = os.path.join(d, "run_marker_api_trace.csv")
    ranges = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Function"]) for r in _read_csv(mpath)] \
        if os.path.exists(mpath) else []

    def inner(ts, prefix):
        best = None
        for a, b, n in ranges:
            if n.startswith(prefix) and a <= ts <= b and (best is None or a > best[0]):
                best = (a, n[len(prefix):])
        return best[1] if best else None

    groups = {}
    for r in kt:
        t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        wl = inner(t0, "workload: ")
        lab = kernel_label(r["Kernel_Name"])
        if lab is None:
            if wl is None or not (wl.startswith("gather") or wl.startswith("copy")):
                continue                      # the 1 GiB flush reads and other torch work
            lab = torch_label(r["Kernel_Name"])
        key = (lab, wl or "(outside every section)", inner(t0, "form: ") or "set-up (outside the timed forms)")
        groups.setdefault(key, []).append((t1 - t0) / 1e3)
    sha = sources_sha256(ALL_KERNEL_SOURCES)
    L = ["# libsmla kernels in the bench: rocprofv3 kernel trace", "",
         "Every kernel dispatch of one full bench run, labelled with the bench section it ran in (a marker range per "
         "workload and per timing form; the device is drained at each range's ends). Workloads are the bench's: "
         "sparse MLA decode at top-k 2048 (bf16 batch 32 over a 2^20-slot pool of 64-slot pages; fp8 e4m3 batch 64; "
         "the ragged bf16 batch of 128 with 13 dense requests; 128 heads), grouped sparse prefill (8,192 queries on "
         "16,384 cached tokens, G = 2, bf16 and fp8 caches), dense paged decode and kv_write. Durations in "
         "microseconds. From the repository root:", ""]
    L += _fmt_cmds("trace", [d])
    L += [f"Kernel source sha256 ({', '.join(os.path.basename(f) for f in ALL_KERNEL_SOURCES)}): `{sha}`", ""]
    L += ["| kernel | workload | form | dispatches | mean | median | min | max |", "|---|---|---|---|---|---|---|---|"]
    for (lab, wl, form), v in groups.items():
        L.append(f"| {lab} | {wl} | {form} | {len(v)} | {statistics.mean(v):.2f} | {statistics.median(v):.2f} | "
                 f"{min(v):.2f} | {max(v):.2f} |")
    L.append("")
    bl = _bench_line(d)
    head = groups.get(("decode_stage1_mfma<bf16>", "bf16 decode, batch 32",
                       "fused, back to back over rotating batches (the headline)"))
    if bl and head:
        L.append(f"The profiled run's bench line gives {bl['ms_per_step'] * 1e3:.2f} us per headline step (one pair of "
                 f"events around {bl['steps']} back-to-back steps); the trace's mean duration of those "
                 f"{len(head)} dispatches is {statistics.mean(head):.2f} us. Its roofline figure divides the step's "
                 f"{bl['algorithmic_bytes_step']:,} algorithmic bytes by the step time: "
                 f"{bl['roofline']['achieved']:.0f} GB/s, {bl['roofline']['frac']:.3f} of 8 TB/s.")
        L.append("")
    spath = os.path.join(d, "run_kernel_stats.csv")
    if os.path.exists(spath):
        rows = [r for r in _read_csv(spath) if kernel_label(r["Name"])]
        rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
        L += ["rocprofv3 --stats over the whole run (libsmla kernels):", "",
              "| kernel | calls | total ms | mean us | min us | max us |", "|---|---|---|---|---|---|"]
        for r in rows:
            L.append(f"| {kernel_label(r['Name'])} | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.2f} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
        L.append("")
    _write_profile("decode_prefill_kernels_trace.md", L)


def _pmc(d: str, counters):
    """Per-dispatch sums of `counters` from d/run_counter_collection.csv, averaged per kernel label;
    the calibration copy (torch's x * 1 over 64M floats: an elementwise kernel of a tensor and a
    scalar, not the fill that creates x) is labelled "copy"."""
    per = {}
    dur = {}
    for r in _read_csv(os.path.join(d, "run_counter_collection.csv")):
        if r["Counter_Name"] not in counters:
            continue
        lab = kernel_label(r["Kernel_Name"])
        if lab is None:
            if "AUnaryFunctor" in r["Kernel_Name"] and _grid(r) == (64 << 20) // 4:
                lab = "copy"
            else:
                continue
        key = (lab, r["Dispatch_Id"])
        per.setdefault(key, {}).setdefault(r["Counter_Name"], 0.0)
        per[key][r["Counter_Name"]] += float(r["Counter_Value"])
        if "Start_Timestamp" in r and r.get("End_Timestamp"):
            dur[key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    out, n, du = {}, {}, {}
    for (lab, _), cs in per.items():
        for c, v in cs.items():
            out.setdefault(lab, {}).setdefault(c, []).append(v)
    for lab, cs in out.items():
        n[lab] = max(len(v) for v in cs.values())
        out[lab] = {c: statistics.mean(v) for c, v in cs.items()}
        ds = [v for (l2, _), v in dur.items() if l2 == lab]
        du[lab] = statistics.mean(ds) if ds else float("nan")
    return out, n, du


def summarize_traffic(fd: str, wd: str) -> None:
    """profiles/decode_kernels_hbm_traffic.md: HBM bytes per launch of the decode kernels from
    FETCH_SIZE and WRITE_SIZE, each scaled by the copy kernel's reading of a known size."""
    fe, nf, _ = _pmc(fd, {"FETCH_SIZE"})
    wr, nw, _ = _pmc(wd, {"WRITE_SIZE"})
    copy_kib = (256 << 20) / 1024.0
    sf, sw = copy_kib / fe["copy"]["FETCH_SIZE"], copy_kib / wr["copy"]["WRITE_SIZE"]
    sha = sources_sha256(KERNEL_SOURCES)
    bl = _bench_line(fd) or {}
    alg = {"decode_stage1_mfma<bf16>": bl.get("algorithmic_bytes_step"),
           "decode_stage1_mfma<fp8>": (bl.get("fp8_kv_decode") or {}).get("algorithmic_bytes_step")}
    L = ["# Decode kernels: HBM traffic from rocprofv3 counters", "",
         "Two counter passes over the same bench command (bf16 decode batch 32, fp8 decode batch 64, then a plain "
         "copy y = x * 1 over 256 MiB of fp32: 262,144 KiB read and 262,144 KiB written, which calibrates each "
         "counter). From the repository root:", ""]
    L += _fmt_cmds("traffic", [fd, wd])
    L += [f"Kernel source sha256 (decode.hip + stage1_common.h + smla_device.h + smla_internal.h): `{sha}`", "",
          f"Calibration: FETCH_SIZE reads {fe['copy']['FETCH_SIZE']:.1f} KiB for the copy's 262,144 KiB of reads "
          f"(scale {sf:.4f}); WRITE_SIZE reads {wr['copy']['WRITE_SIZE']:.1f} KiB for its 262,144 KiB of writes "
          f"(scale {sw:.4f}).", "",
          "| kernel | workload | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes (scaled) | written bytes "
          "(scaled) | traffic bytes | algorithmic bytes | traffic / algorithmic |",
          "|---|---|---|---|---|---|---|---|---|---|"]
    mach = []
    for k, wk in (("decode_stage1_mfma<bf16>", "bf16_batch_32"), ("decode_stage1_mfma<fp8>", "fp8_batch_64"),
                  ("resolve_kernel", "both")):
        if k not in fe or k not in wr:
            continue
        rb, wb = fe[k]["FETCH_SIZE"] * sf * 1024, wr[k]["WRITE_SIZE"] * sw * 1024
        a = alg.get(k)
        L.append(f"| {k} | {wk.replace('_', ' ')} | {nf[k]} | {fe[k]['FETCH_SIZE']:.1f} | {wr[k]['WRITE_SIZE']:.1f} | "
                 f"{rb:,.0f} | {wb:,.0f} | {rb + wb:,.0f} | {f'{a:,}' if a else '-'} | "
                 f"{f'{(rb + wb) / a:.3f}' if a else '-'} |")
        if k != "resolve_kernel":
            mach.append(f"traffic_bytes_per_launch {k} {wk} {rb + wb:.0f} read {rb:.0f} write {wb:.0f}")
    L += ["", "Each decode's launches in every timed form (fused resolution, over resolved slots, back to back, graph "
          "replay) are averaged together: they move the same cache rows. The algorithmic bytes are the bench's: cache "
          "rows gathered once, q, the index table, the output and LSE, the split partials written and read back once.",
          "", "Machine-readable lines (bench.py reports `roofline.traffic` from these while the kernel source hash "
          "matches):", "", "```"] + mach + [f"source_sha256 {sha}", "```"]
    _write_profile("decode_kernels_hbm_traffic.md", L)


SQ_CLOCK_HZ = 2.1e9          # shader clock over the decode loop, measured with s_memtime on this GPU


def summarize_sq(da: str, db: str) -> None:
    """profiles/decode_prefill_sq_counters.md from the two SQ counter passes."""
    cols = [("decode bf16", "decode_stage1_mfma<bf16>"), ("decode fp8", "decode_stage1_mfma<fp8>"),
            ("union (prefill)", "decode_stage1_mfma<bf16, union>")]
    pa, na, dura = _pmc(da, set(SQ_PASSES["A"].split()))
    pb, nb, _ = _pmc(db, set(SQ_PASSES["B"].split()))
    mean = {c: {**pa.get(k, {}), **pb.get(k, {})} for c, k in cols}
    dur = {c: dura.get(k, float("nan")) for c, k in cols}
    names = sorted({n for c, _ in cols for n in mean[c]})
    sha = sources_sha256(KERNEL_SOURCES)
    L = ["# Shader-sequencer counters: bf16 and fp8 decode, grouped prefill (MI355X)", "",
         "Two counter passes (eight SQ counters each) over the same short bench run. From the repository root:", ""]
    L += _fmt_cmds("sq", [da, db])
    L += [f"Kernel source sha256 (decode.hip + stage1_common.h + smla_device.h + smla_internal.h): `{sha}`", "",
          "Per-dispatch means: `decode bf16` = `decode_stage1_mfma<bf16>` on bf16 batch 32 (every form the bench runs); "
          "`decode fp8` = `decode_stage1_mfma<fp8>` on fp8 batch 64; `union (prefill)` = "
          "`decode_stage1_mfma<bf16, union>` on grouped prefill Q 8192 (G 2, 64 heads). Counter values are the device "
          "totals rocprofv3 reports; the derived rows divide them by 256 compute units (or 1,024 SIMDs) and by the "
          f"dispatch's cycles at {SQ_CLOCK_HZ / 1e9:.1f} GHz (the shader clock measured over the decode loop with "
          "s_memtime). Durations under counter collection run longer than in the kernel trace.", "",
          "| counter | " + " | ".join(c for c, _ in cols) + " |", "|---" * (len(cols) + 1) + "|"]
    for n in names:
        L.append(f"| {n} | " + " | ".join(f"{mean[c].get(n, float('nan')):.4g}" for c, _ in cols) + " |")
    L.append("| dispatches (pass A / B) | " + " | ".join(f"{na.get(k, 0)} / {nb.get(k, 0)}" for _, k in cols) + " |")
    L.append("| mean duration us (pass A) | " + " | ".join(f"{dur[c]:.1f}" for c, _ in cols) + " |")
    derived = [
        ("LDS bank-conflict stall cycles per CU-cycle", lambda m, cy: m["SQ_LDS_BANK_CONFLICT"] / (256 * cy)),
        ("LDS busy (indexed) cycles per CU-cycle", lambda m, cy: m["SQ_LDS_IDX_ACTIVE"] / (256 * cy)),
        ("MFMA busy cycles per SIMD-cycle", lambda m, cy: m["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * cy)),
        ("wave-cycles waiting (any) / wave-cycles", lambda m, cy: m["SQ_WAIT_ANY"] / m["SQ_WAVE_CYCLES"]),
        ("wave-cycles waiting to issue / wave-cycles", lambda m, cy: m["SQ_WAIT_INST_ANY"] / m["SQ_WAVE_CYCLES"]),
        ("wave-cycles waiting to issue LDS / wave-cycles", lambda m, cy: m["SQ_WAIT_INST_LDS"] / m["SQ_WAVE_CYCLES"]),
        ("MFMA FLOP per dispatch (BF16 MOPS x 512)", lambda m, cy: m["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512),
        ("MFMA TFLOP/s over the dispatch (pass A duration)",
         lambda m, cy: m["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / (cy / SQ_CLOCK_HZ) / 1e12),
    ]
    L += ["", "Derived:", "", "| quantity | " + " | ".join(c for c, _ in cols) + " |", "|---" * (len(cols) + 1) + "|"]
    val = {}
    for label, f in derived:
        cells = []
        for c, _ in cols:
            try:
                v = f(mean[c], dur[c] * 1e-6 * SQ_CLOCK_HZ)
            except (KeyError, ZeroDivisionError):
                v = float("nan")
            val[(label, c)] = v
            cells.append(f"{v:.4g}")
        L.append(f"| {label} | " + " | ".join(cells) + " |")
    mf = [val[("MFMA busy cycles per SIMD-cycle", c)] for c, _ in cols]
    ld = [val[("LDS busy (indexed) cycles per CU-cycle", c)] for c, _ in cols]
    wt = [val[("wave-cycles waiting (any) / wave-cycles", c)] for c, _ in cols]
    L += ["", f"Over the three kernels the matrix unit is busy {min(mf):.2f}-{max(mf):.2f} of the SIMD cycles, the LDS "
              f"{min(ld):.2f}-{max(ld):.2f} of the CU cycles, and the waves wait {min(wt):.2f}-{max(wt):.2f} of "
              "theirs: no unit is saturated, so the loops are bound by latency (operand reads, accumulation chains, "
              "barriers) and, in decode, by the row gathers."]
    _write_profile("decode_prefill_sq_counters.md", L)


def summarize_profile(argv) -> None:
    kind, dirs = argv[0], argv[1:]
    need = {"trace": 1, "traffic": 2, "sq": 2}
    if kind not in need or len(dirs) != need[kind]:
        raise SystemExit("--summarize-profile: trace DIR | traffic FETCH_DIR WRITE_DIR | sq DIR_A DIR_B")
    {"trace": summarize_trace, "traffic": summarize_traffic, "sq": summarize_sq}[kind](*dirs)


def split_sweep_markdown(res) -> str:
    cols = sorted({S for v in res.values() for S in v["us"]})
    sha = sources_sha256([CSRC + f for f in ("decode.hip", "stage1_common.h", "smla_device.h", "smla_internal.h", "abi.hip")])
    L = ["# Decode step against the split count (MI355X, one GPU)", "",
         "Cold steps (1 GiB read before each, median) of `smla_sparse_decode` at top-k 2048, 64 heads, over a "
         "2^20-slot pool of random rows, for each batch size and cache format, at every split count from the fewest "
         "(a split holds at most 1,024 rows) to one 32-row chunk per split. From the repository root:", "",
         "```", "python3 bench.py --split-sweep > profiles/decode_split_sweep.md", "```", "",
         f"Source sha256 (decode.hip + stage1_common.h + smla_device.h + smla_internal.h + abi.hip): `{sha}`", "",
         "`auto` is the split count the library picks when `num_splits` is 0. Step time in microseconds.", "",
         "| cache | T | auto S | auto us | best S | best us | " + " | ".join(f"S={S}" for S in cols) + " |",
         "|---" * (6 + len(cols)) + "|"]
    for (dt, T), v in res.items():
        cells = " | ".join(f"{v['us'][S]:.1f}" if S in v["us"] else "-" for S in cols)
        L.append(f"| {dt} | {T} | {v['auto']} | {v['us'][v['auto']]:.1f} | {v['best']} | {v['us'][v['best']]:.1f} | "
                 f"{cells} |")
    return "\n".join(L) + "\n"


def overlap_sweep_markdown(res, steps) -> str:
    sha = sources_sha256([CSRC + f for f in ("decode.hip", "union.hip", "stage1_common.h", "smla_device.h", "smla_internal.h")])
    L = ["# Grouped prefill against per-query decode, by list overlap (MI355X, one GPU)", "",
         "4,096 queries with lists of 2,048 slots over a 24,576-slot bf16 cache of random rows (the grouped-prefill "
         "configuration's pool). Queries come in groups of G with H = 128 / G heads; a fraction `overlap` of each list "
         "is shared by the group's members and the rest is disjoint (so the union holds exactly "
         f"(overlap + G (1 - overlap)) x 2,048 rows). Cold steps (1 GiB read before each, median of {steps}):", "",
         "- grouped: `smla_build_group_union` + `smla_grouped_prefill`;",
         "- alone: `smla_sparse_decode` over the same lists (page size 1), every query attending its own rows.", "",
         "From the repository root:", "", "```", "python3 bench.py --overlap-sweep > profiles/grouped_prefill_overlap_sweep.md",
         "```", "", f"Source sha256 (decode.hip + union.hip + stage1_common.h + smla_device.h + smla_internal.h): `{sha}`", "",
         "| G | H | overlap | union rows / W | grouped us | alone us | speedup |", "|---|---|---|---|---|---|---|"]
    for (G, ov), v in res.items():
        L.append(f"| {G} | {128 // G} | {ov:.2f} | {v['union_per_list']:.2f} | {v['grouped_us']:.0f} | "
                 f"{v['alone_us']:.0f} | {v['alone_us'] / v['grouped_us']:.2f}x |")
    return "\n".join(L) + "\n"


if __name__ == "__main__":
    main()
