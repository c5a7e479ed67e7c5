"""Decode-step paged attention benchmark on one MI355X.

A step is one pass of the whole hot path over the batch: grow every sequence
by one token in the host allocator (one batched call), export the block tables
and lengths and scatter the new tokens' K/V into their page slots for every
layer (one fused launch reading pinned staging), and run paged decode
attention for every layer (partition kernel + merge).  Inputs are resident in HBM when the
timed region starts.  Sequences keep growing over the steps; bytes are counted
from the actual lengths.

Output: one JSON line per side measurement as it finishes (``{"leg": ...}``:
each other workload and frame order, the contiguous twin, copy-on-write,
swapping, fused scatter + attention, the page-size sweep, the CPU baseline's
details), then, LAST, the headline line, kept under 4 KB.  ``value`` is the
algorithmic KV bandwidth of the whole step (attention's K/V + q + out + table
+ length bytes, plus the scatter's reads and writes) over the step time;
``roofline`` is for the attention partition kernel alone, timed with HIP
events recorded around it on its own stream; ``cpu_baseline`` times the CPU
fp64 oracle on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
HOST_LINK_GBS = 64.0   # PCIe 5.0 x16 host link, per direction, nominal

WORKLOADS = {
    "tiny": "Tiny: 4 seqs, 1 layer, 2 heads, d_head 16, fp32, block 16, pool 64 pages, context U[1,64], {frames} frames",
    "gpt2": "GPT-2-124M shape: 12 layers x 12 heads, d_head 64, fp16, 32 seqs, prompts U[8,64] + 50 decode steps, block 16, pool 1024 pages, {frames} frames",
    "mixed": "Mixed-length: 32 seqs, 50% U[32,128] / 30% U[256,512] / 20% U[1024,2048], 12 heads, d_head 64, fp16, block 16, pool 4096, {frames} frames",
    "mixed_s7": "Mixed-length, seed 7: 32 seqs, 50% U[32,128] / 30% U[256,512] / 20% U[1024,2048], 12 heads, d_head 64, fp16, block 16, pool 4096, {frames} frames",
    "13b": "13B-style: 40 heads, d_head 128, fp16, one layer's decode, 64 seqs, context U[256,2048], block 16, pool 1.1x blocks used, {frames} frames",
    "gqa": "GQA large batch: 14 q heads / 2 kv heads, d_head 64, bf16, 256 seqs, context U[1024,4096], block 16, pool 70k pages after 500x16 alloc/free churn, {frames} frames",
    "13b_32k": "13B-style at 32k-token contexts: 40 heads, d_head 128, fp16, one layer's decode, 2 seqs, context U[30720,32768], block 16, pool 1.1x blocks used, {frames} frames",
    "gqa_32k": "GQA at 32k-token contexts: 14 q heads / 2 kv heads, d_head 64, bf16, 32 seqs, context U[30720,32768], block 16, pool 1.1x blocks used, {frames} frames",
    "gqa_1m": "GQA, one sequence of 2^20 tokens: 14 q heads / 2 kv heads, d_head 64, bf16, block 16, pool 1.1x blocks used, {frames} frames",
}


# Sources that define the attention partition kernels (the roofline kernel).
ATTN_SOURCES = ("pf_attn.hip", "pf_attn_mfma.hip", "pf_sched.h", "pf_common.h", "pf_attn.h")


def kernel_source_hash():
    """Hash of the sources of the attention partition kernels."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "paged_kv_cache_43_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f in ATTN_SOURCES:
            h.update(f.encode())
            h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(config):
    """HBM bytes per partition launch from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, copy-kernel calibrated) and the
    algorithmic bytes of the same launches (the counter runs' lengths), or None
    when the kernels changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    try:
        kv = dict(l.split(":", 1) for l in open(path) if ":" in l and not l.startswith("#"))
    except OSError:
        return None
    if kv.get("source_hash", "").strip() != kernel_source_hash() or config not in kv:
        return None
    f = kv[config].split()
    return int(f[0]), (int(f[1]) if len(f) > 1 else None)


def _flush(buf):
    """Read the whole 1 GiB flush buffer (a max over it as int64: ~0.18 ms on
    MI355X, where a max over bytes takes ~0.93 ms).  Evicts the K/V from the
    L2s and the 256 MB MALL and leaves nothing dirty."""
    import torch
    buf.view(torch.int64).amax()


def alg_bytes_attention(ctx, w, out_bytes):
    """Bytes attention must move: K+V of every context token, q, out, the
    table entries in use, the lengths."""
    ctx = np.asarray(ctx, dtype=np.int64)
    kv = int(ctx.sum()) * w.hkv * w.d * 2 * w.es
    qo = w.n * w.hq * w.d * (w.es + out_bytes)
    tables = int(((ctx + w.block - 1) // w.block).sum()) * 4
    return kv + qo + tables + 4 * w.n


def alg_bytes_scatter(w):
    """One new token per sequence: read k and v, write them into the pool, read
    tok_seq/tok_pos and one table entry each."""
    return w.n * w.hkv * w.d * 2 * w.es * 2 + w.n * 12


class TimingEvent:
    """A timing event on the library's stream markers (hipEvent_t without the
    system-scope fence), used like torch.cuda.Event(enable_timing=True): a
    default event costs ~6 us of stream time on MI355X (a cache writeback and
    invalidation), which would otherwise be counted into the timed kernels."""

    def __init__(self):
        from paged_kv_cache_43_amd import pf
        self.m = pf.Marker(timing=True)
        self.cuda_event = self.m.handle

    def record(self, stream=None):
        self.m.record(stream)

    def elapsed_time(self, stop):
        return self.m.elapsed_ms(stop.m)


def run_gpu(args, name, frames, steps, warmup, flush, share=None):
    import torch
    from paged_kv_cache_43_amd import inputs, pf, runner

    dev = "cuda"
    w = inputs.Workload(name, frames=frames)
    if share is not None:
        w.share_values(share)   # the other frame order's draws (identical values)
    ksteps = min(steps, 20)
    kv = runner.PagedKV(w, device=dev, sentinel=False, extra_tokens=steps + ksteps + warmup + 1)
    q = runner.fill_workload(kv, device=dev)
    stream = torch.cuda.current_stream()
    rng = np.random.default_rng(123)
    newk = runner.bits_to_device(inputs.normal_bits(rng, (w.layers, w.n, w.hkv, w.d), w.dtype), dev)
    newv = runner.bits_to_device(inputs.normal_bits(rng, (w.layers, w.n, w.hkv, w.d), w.dtype), dev)
    out_t = torch.empty((w.layers, w.n, w.hq, w.d), dtype=torch.int32 if w.es == 4 else torch.int16,
                        device=dev)
    ids = np.arange(w.n, dtype=np.uint64)
    base = w.ctx.astype(np.int64)
    # warmup, K timed steps (step events only), min(K, 20) steps with events
    # around every partition kernel; then, at the final lengths, attention calls
    # alone with events around each (partition + merge)
    total_steps = warmup + steps + ksteps
    attn_iters = max(50, steps)
    max_ctx_final = int(base.max()) + total_steps
    kv.ensure_workspace(max_ctx_final)
    flush_buf = torch.zeros(1 << 30, dtype=torch.uint8, device=dev) if flush else None
    ev_a = [[TimingEvent() for _ in range(w.layers)] for _ in range(total_steps)]
    ev_b = [[TimingEvent() for _ in range(w.layers)] for _ in range(total_steps)]
    ev_c = [[TimingEvent() for _ in range(w.layers)] for _ in range(attn_iters + 5)]
    ev_d = [[TimingEvent() for _ in range(w.layers)] for _ in range(attn_iters + 5)]
    ev_step = [(TimingEvent(), TimingEvent())
               for _ in range(total_steps)]
    for row in ev_a + ev_b + ev_c + ev_d:
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    ctx_per_step = []

    def step(t, events, kernel_events=False):
        new_lens = (base + t + 1).astype(np.int32)
        st, _ = pf.pf_alloc_for_seqs(kv.h, ids, new_lens)
        pf.check(st, "pf_alloc_for_seqs")
        if flush:
            _flush(flush_buf)   # read 1 GiB: evicts the K/V from L2 and the 256 MB MALL, leaves nothing dirty
        if events:
            ev_step[t][0].record(stream)
        kv.decode_prepare(newk, newv)          # tables + every layer's new token, one launch
        mc = int(new_lens.max())
        for layer in range(w.layers):
            if kernel_events:
                pf.check(pf.pf_pool_set_timing_events(kv.h, ev_a[t][layer].cuda_event,
                                                      ev_b[t][layer].cuda_event))
            kv.attention(layer, q[layer], out_t[layer], mc)
        if kernel_events:
            pf.check(pf.pf_pool_set_timing_events(kv.h, None, None))
        if events:
            ev_step[t][1].record(stream)
        ctx_per_step.append(new_lens.astype(np.int64))

    for t in range(warmup):
        step(t, False)
    torch.cuda.synchronize()
    # the K timed steps: only the step's own pair of events in the stream
    # (and none at all without --flush, where the wall clock times them)
    t0 = time.perf_counter()
    for t in range(warmup, warmup + steps):
        step(t, flush)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # more steps with HIP events around every partition kernel (roofline)
    for t in range(warmup + steps, total_steps):
        step(t, True, kernel_events=True)
    torch.cuda.synchronize()
    # attention calls alone at the final lengths: 5 untimed, then attn_iters
    # with events around each layer's call (partition + merge), flushed first
    mc = int(ctx_per_step[-1].max())
    for r in range(attn_iters + 5):
        if flush:
            _flush(flush_buf)
        for layer in range(w.layers):
            ev_c[r][layer].record(stream)
            kv.attention(layer, q[layer], out_t[layer], mc)
            ev_d[r][layer].record(stream)
    torch.cuda.synchronize()
    # the scatter alone: one pf_scatter_kv launch writing every sequence's
    # newest token of layer 0 (the bytes it already holds), flushed first
    tok_seq = torch.arange(w.n, dtype=torch.int32, device=dev)
    tok_pos = torch.from_numpy((ctx_per_step[-1] - 1).astype(np.int32)).to(dev)
    ev_s = [(TimingEvent(), TimingEvent()) for _ in range(attn_iters + 5)]
    for r in range(attn_iters + 5):
        if flush:
            _flush(flush_buf)
        ev_s[r][0].record(stream)
        kv.scatter(0, newk[0], newv[0], tok_seq, tok_pos)
        ev_s[r][1].record(stream)
    torch.cuda.synchronize()
    sc_ms = [a.elapsed_time(b) for a, b in ev_s[5:]]

    timed = range(warmup, warmup + steps)
    evsteps = range(warmup + steps, total_steps)
    step_ms = [ev_step[t][0].elapsed_time(ev_step[t][1]) for t in (timed if flush else evsteps)]
    part_ms = [ev_a[t][l].elapsed_time(ev_b[t][l]) for t in evsteps for l in range(w.layers)]
    attn_ms = [ev_c[r][l].elapsed_time(ev_d[r][l]) for r in range(5, attn_iters + 5) for l in range(w.layers)]
    attn_call_bytes = [alg_bytes_attention(ctx_per_step[-1], w, w.es)] * len(attn_ms)
    attn_bytes = [alg_bytes_attention(ctx_per_step[t], w, w.es) for t in timed]
    part_bytes = [alg_bytes_attention(ctx_per_step[t], w, w.es) for t in evsteps]
    step_bytes = [b * w.layers + alg_bytes_scatter(w) * w.layers for b in attn_bytes]
    # free everything: the pool must come back whole
    for s in range(w.n):
        pf.check(pf.pf_free_seq(kv.h, s))
    assert pf.pf_free_pages(kv.h) == w.num_pages
    split = pf.pf_attention_split_tokens(kv.h, w.n, w.hq, max_ctx_final)
    waves = pf.pf_attention_waves(kv.h, w.n, w.hq, max_ctx_final)
    mfma = pf.pf_attention_kernel(kv.h, w.hq) == 1
    kv.close()
    ms_step_events = float(np.mean(step_ms))
    ms_step_wall = wall * 1e3 / steps
    # value uses the step time the timed loop actually took (flushes excluded
    # only when --flush is given, then from per-step events)
    ms_step = ms_step_events if flush else ms_step_wall
    avg_step_bytes = float(np.mean(step_bytes))
    avg_attn_bytes = float(np.mean(part_bytes))
    part_avg_ms = float(np.mean(part_ms))
    achieved = avg_attn_bytes / (part_avg_ms * 1e-3) / 1e9
    attn_med_ms = float(np.median(attn_ms))
    attention = {
        "what": "attention calls alone at the final lengths (partition + merge kernels), events around each "
                "layer's call, cache flushed before each iteration; 5 untimed first",
        "launches": len(attn_ms), "median_us": round(attn_med_ms * 1e3, 2),
        "mean_us": round(float(np.mean(attn_ms)) * 1e3, 2), "sd_us": round(float(np.std(attn_ms)) * 1e3, 2),
        "min_us": round(float(np.min(attn_ms)) * 1e3, 2),
        "kv_GBps": round(float(np.median(attn_call_bytes)) / (attn_med_ms * 1e-3) / 1e9, 1),
        "pct_hbm_peak": round(float(np.median(attn_call_bytes)) / (attn_med_ms * 1e-3) / 1e9 / HBM_PEAK_GBS * 100, 1),
        "seqs_per_ms": round(w.n / (attn_med_ms * w.layers), 2)}
    sc_med = float(np.median(sc_ms))
    scatter = {
        "what": "one pf_scatter_kv launch (every sequence's newest token, one layer), events around it, "
                "cache flushed first; 5 untimed first",
        "launches": len(sc_ms), "median_us": round(sc_med * 1e3, 2), "min_us": round(float(np.min(sc_ms)) * 1e3, 2),
        "alg_bytes": alg_bytes_scatter(w), "GBps": round(alg_bytes_scatter(w) / (sc_med * 1e-3) / 1e9, 1)}
    return dict(
        w=w, name=name, frames=frames, ms_step=ms_step, ms_step_wall=ms_step_wall,
        ms_step_events=ms_step_events, value=avg_step_bytes / (ms_step * 1e-3) / 1e9,
        seqs_per_ms=w.n / ms_step, part_avg_us=part_avg_ms * 1e3,
        part_med_us=float(np.median(part_ms)) * 1e3, part_min_us=float(np.min(part_ms)) * 1e3,
        part_sd_us=float(np.std(part_ms)) * 1e3,
        attn_bytes=avg_attn_bytes, achieved=achieved, split=split, waves=waves, mfma=bool(mfma),
        whole=bool(split) and split >= max_ctx_final,
        kernel_seqs_per_ms=w.n / (part_avg_ms * w.layers), attention=attention, scatter=scatter)


def run_twin(name, frames, reps):
    """Paged attention vs the contiguous-cache twin (the same kernels with no
    table walk) on one layer of the workload at its measured step: partition
    kernel times from HIP events, alternating the two, and the largest output
    difference (the twin must return the same bits)."""
    import torch
    from paged_kv_cache_43_amd import inputs, pf, runner

    w = inputs.Workload(name, frames=frames)
    kv = runner.PagedKV(w, sentinel=False)
    q = runner.fill_workload(kv)
    mc = int(w.ctx.max())
    max_len = -(-mc // 16) * 16
    k, v = kv.gather(0, max_len)
    kh = k.permute(0, 2, 1, 3).contiguous()
    vh = v.permute(0, 2, 1, 3).contiguous()
    layouts = {"head_major": (kh.permute(0, 2, 1, 3), vh.permute(0, 2, 1, 3)), "token_major": (k, v)}
    dt = torch.int32 if w.es == 4 else torch.int16
    outs = {x: torch.empty((w.n, w.hq, w.d), dtype=dt, device="cuda") for x in ["paged"] + list(layouts)}
    kv.ensure_workspace(mc)
    # back to back, alternating, one event pair per launch; synchronized once
    order = [x for _ in range(reps + 3) for x in outs]
    ev = [(TimingEvent(), TimingEvent()) for _ in order]
    for a, b in ev:
        a.record()
        b.record()
    torch.cuda.synchronize()
    for (a, b), x in zip(ev, order):
        pf.check(pf.pf_pool_set_timing_events(kv.h, a.cuda_event, b.cuda_event))
        if x == "paged":
            kv.attention(0, q[0], outs[x], mc)
        else:
            kv.contiguous_attention(layouts[x][0], layouts[x][1], q[0], outs[x], mc)
    pf.check(pf.pf_pool_set_timing_events(kv.h, None, None))
    torch.cuda.synchronize()
    times = {x: [] for x in outs}
    for i, ((a, b), x) in enumerate(zip(ev, order)):
        if i >= 3 * len(outs):
            times[x].append(a.elapsed_time(b) * 1e3)
    as_float = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    ref = outs["paged"]
    res = {"paged_us": round(float(np.median(times["paged"])), 2)}
    diff = 0.0
    for x in layouts:
        t = float(np.median(times[x]))
        res["contiguous_%s_us" % x] = round(t, 2)
        res["paged_slowdown_vs_%s" % x] = round(res["paged_us"] / t, 4)
        got = outs[x]
        d = (got.view(as_float).double() - ref.view(as_float).double()).abs().max().item()
        diff = max(diff, float(d))
        res["bitwise_equal_%s" % x] = bool(torch.equal(got, ref))
    res["max_abs_paged_minus_contiguous"] = diff
    res["alg_kv_bytes"] = int(w.ctx.sum()) * w.hkv * w.d * 2 * w.es
    res["frames"] = frames
    res["median_of"] = reps
    kv.close()
    return res


def run_cow(prompts, beam, reps, seed=43):
    """Copy-on-write prefix sharing (PagedAttention blog, "Copy-on-Write for
    Parallel Sampling") on the 13B-style head shape: ``prompts`` prompts with
    lengths U[256, 2048], each forked into ``beam`` sequences that then decode
    one token each.  Reports pages in use against private copies of every
    prompt, the page-copy kernel of the first decode step against the HBM
    roofline, and the attention partition kernel over the aliased tables
    against the same contents in private pages (cache flushed before each)."""
    import torch
    from paged_kv_cache_43_amd import pf

    L, H, D, B = 1, 40, 128, 16
    rng = np.random.default_rng(seed)
    lens = rng.integers(256, 2049, size=prompts)
    n = prompts * beam
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    bits = lambda shape: torch.randn(shape, generator=gen, device="cuda").half().view(torch.int16)
    fl = torch.zeros(1 << 30, dtype=torch.uint8, device="cuda")
    pages_needed = int(sum(-(-int(x) // B) + 1 for x in lens)) * beam + 64
    kp = [bits((int(x), H, D)) for x in lens]
    vp = [bits((int(x), H, D)) for x in lens]

    def make(shared):
        st, h = pf.pf_pool_create(pages_needed, B, L, H, D, "f16", None)
        pf.check(st)
        nbytes = pf.pf_pool_bytes(h)
        pool = torch.zeros(nbytes // 2, dtype=torch.int16, device="cuda")
        pf.check(pf.pf_pool_bind(h, pool, nbytes))
        for p in range(prompts):
            owners = [p * beam] if shared else [p * beam + b for b in range(beam)]
            for s in owners:
                pf.check(pf.pf_alloc_for_seq(h, s, int(lens[p]))[0])
                st, bt, _ = pf.pf_block_tables(h, [s], 128)
                btd = torch.from_numpy(bt).cuda()
                m = int(lens[p])
                pf.check(pf.pf_scatter_kv(h, 0, kp[p], vp[p], torch.zeros(m, dtype=torch.int32, device="cuda"),
                                          torch.arange(m, dtype=torch.int32, device="cuda"), m, btd, 1, 128))
            if shared:
                for b in range(1, beam):
                    pf.check(pf.pf_fork_seq(h, p * beam, p * beam + b))
        torch.cuda.synchronize()
        return h, pool

    hs, pool_s = make(True)
    hp, pool_p = make(False)
    res = {"workload": "%d prompts x beam %d, prompt lengths U[256,2048], 40 heads, d_head 128, fp16, block 16"
                       % (prompts, beam),
           "pages_in_use_shared": pages_needed - pf.pf_free_pages(hs),
           "pages_in_use_private": pages_needed - pf.pf_free_pages(hp)}
    res["memory_saved_fraction"] = round(1 - res["pages_in_use_shared"] / res["pages_in_use_private"], 4)
    ids = np.arange(n, dtype=np.uint64)
    new = np.repeat(lens, beam).astype(np.int32) + 1
    st, nn, copies = pf.pf_grow_seqs(hs, ids, new)
    pf.check(st)
    pf.check(pf.pf_alloc_for_seqs(hp, ids, new)[0])
    res["first_step_copies"] = int(len(copies))
    page_bytes = pf.pf_page_bytes(hs)
    pairs = torch.from_numpy(np.ascontiguousarray(copies)).cuda()
    ev = [(TimingEvent(), TimingEvent()) for _ in range(reps + 3)]
    torch.cuda.synchronize()
    for a, b in ev:       # the copies are idempotent: re-running them times the kernel
        _flush(fl)
        a.record()
        pf.check(pf.pf_copy_pages(hs, pairs, len(copies)))
        b.record()
    torch.cuda.synchronize()
    t_copy = float(np.median([a.elapsed_time(b) * 1e3 for a, b in ev[3:]]))
    copy_bytes = 2 * page_bytes * len(copies)
    res["copy_kernel_us"] = round(t_copy, 2)
    res["copy_bytes"] = int(copy_bytes)
    res["copy_GBps"] = round(copy_bytes / t_copy / 1e3, 1)
    res["copy_frac_of_hbm_peak"] = round(copy_bytes / t_copy / 1e3 / HBM_PEAK_GBS, 4)
    # attention over aliased vs private tables, same logical K/V
    mc = int(new.max())
    mb = -(-mc // B)
    q = bits((n, H, D))
    out = torch.empty((n, H, D), dtype=torch.int16, device="cuda")
    setup = {}
    for tag, h in (("shared", hs), ("private", hp)):
        st, bt, ln = pf.pf_block_tables(h, ids, mb)
        pf.check(st)
        need = pf.pf_attention_workspace_bytes(h, n, H, mc)
        setup[tag] = (h, torch.from_numpy(bt).cuda(), torch.from_numpy(ln.astype(np.int32)).cuda(),
                      torch.empty(max(need, 1), dtype=torch.uint8, device="cuda"), need)
    order = [t for _ in range(reps + 3) for t in ("shared", "private")]
    ev = [(TimingEvent(), TimingEvent()) for _ in order]
    for a, b in ev:
        a.record()
        b.record()
    torch.cuda.synchronize()
    for (a, b), tag in zip(ev, order):
        h, bt, ctx, ws, need = setup[tag]
        _flush(fl)
        pf.check(pf.pf_pool_set_timing_events(h, a.cuda_event, b.cuda_event))
        pf.check(pf.pf_paged_decode_attention(h, 0, q, H, bt, mb, ctx, n, mc, 0.0, out, "f16", ws, need))
        pf.check(pf.pf_pool_set_timing_events(h, None, None))
    torch.cuda.synchronize()
    alg = alg_bytes_attention(new, type("W", (), dict(n=n, hq=H, hkv=H, d=D, es=2, block=B))(), 2)
    for tag in ("shared", "private"):
        t = float(np.median([a.elapsed_time(b) * 1e3 for i, ((a, b), x) in enumerate(zip(ev, order))
                             if x == tag and i >= 6]))
        res["attn_%s_us" % tag] = round(t, 2)
        res["attn_%s_alg_GBps" % tag] = round(alg / t / 1e3, 1)
    res["attn_private_over_shared"] = round(res["attn_private_us"] / res["attn_shared_us"], 4)
    res["attn_alg_bytes"] = int(alg)
    for h in (hs, hp):
        pf.pf_pool_destroy(h)
    return res


def run_swap(n_seqs, reps, seed=44):
    """Swapping (PagedAttention blog, "Preemption and Swapping") on the
    13B-style head shape: ``n_seqs`` sequences with lengths U[256, 2048] are
    swapped out to a pinned host store and back in, ``reps`` times.  Reports
    the swap kernel's host-link bandwidth each way beside a DMA-engine copy of
    the same number of contiguous bytes (torch ``copy_`` between pinned and
    device memory), the achievable ceiling of the link."""
    import torch
    from paged_kv_cache_43_amd import pf

    L, H, D, B = 1, 40, 128, 16
    rng = np.random.default_rng(seed)
    lens = rng.integers(256, 2049, size=n_seqs)
    pages = int(sum(-(-int(x) // B) for x in lens))
    P = 2 * pages + 64
    st, h = pf.pf_pool_create(P, B, L, H, D, "f16", rng.permutation(P).astype(np.int32))
    pf.check(st)
    nb = pf.pf_pool_bytes(h)
    pool = torch.zeros(nb // 2, dtype=torch.int16, device="cuda")
    pf.check(pf.pf_pool_bind(h, pool, nb))
    pb = pf.pf_page_bytes(h)
    host = torch.zeros(pages * pb // 2, dtype=torch.int16).pin_memory()
    pf.check(pf.pf_swap_bind(h, host, pages * pb, pages))
    ids = np.arange(n_seqs, dtype=np.uint64)
    pf.check(pf.pf_alloc_for_seqs(h, ids, lens.astype(np.int32))[0])
    staging = torch.zeros(2 * pages, dtype=torch.int32).pin_memory()
    nbytes = pages * pb
    # default events here: their system-scope release is part of a copy to host
    # memory being complete
    t_out, t_in = [], []
    for r in range(reps + 2):
        for to_host, acc in ((True, t_out), (False, t_in)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            fn = pf.pf_swap_out if to_host else pf.pf_swap_in
            pf.check(fn(h, ids, staging, 2 * pages))
            b.record()
            torch.cuda.synchronize()
            if r >= 2:
                acc.append(a.elapsed_time(b) * 1e3)
    # block ranges: the second half of every sequence's blocks out and back
    # (the blocks a scheduler would evict first while the prefix stays), one
    # call per sequence
    halves = [(i, nb_i // 2, nb_i - nb_i // 2) for i, nb_i in enumerate(-(-lens // B))]
    half_pages = sum(c for _, _, c in halves)
    b_out, b_in = [], []
    for r in range(reps + 2):
        for to_host, acc in ((True, b_out), (False, b_in)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            fn = pf.pf_swap_out_blocks if to_host else pf.pf_swap_in_blocks
            off = 0
            for i, first, count in halves:
                pf.check(fn(h, int(ids[i]), int(first), int(count), staging[off:], 2 * count))
                off += 2 * count
            b.record()
            torch.cuda.synchronize()
            if r >= 2:
                acc.append(a.elapsed_time(b) * 1e3)
    dev = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda")
    dma_out, dma_in = [], []
    for r in range(reps + 2):
        for d2h, acc in ((True, dma_out), (False, dma_in)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            if d2h:
                host.copy_(dev, non_blocking=True)
            else:
                dev.copy_(host, non_blocking=True)
            b.record()
            torch.cuda.synchronize()
            if r >= 2:
                acc.append(a.elapsed_time(b) * 1e3)
    pf.pf_pool_destroy(h)
    med = lambda x: float(np.median(x))
    res = {"workload": "%d sequences, lengths U[256,2048], 40 heads, d_head 128, fp16, block 16: %d pages of %d KiB"
                       % (n_seqs, pages, pb // 1024),
           "bytes_each_way": int(nbytes),
           "swap_out_us": round(med(t_out), 1), "swap_in_us": round(med(t_in), 1),
           "swap_out_GBps": round(nbytes / med(t_out) / 1e3, 1), "swap_in_GBps": round(nbytes / med(t_in) / 1e3, 1),
           "dma_copy_d2h_GBps": round(nbytes / med(dma_out) / 1e3, 1),
           "dma_copy_h2d_GBps": round(nbytes / med(dma_in) / 1e3, 1),
           "host_link_peak_GBps_each_way": HOST_LINK_GBS, "median_of": reps}
    res["block_ranges"] = {"what": "second half of each sequence's blocks, one call per sequence",
                           "calls": n_seqs, "bytes_each_way": int(half_pages * pb),
                           "out_us": round(med(b_out), 1), "in_us": round(med(b_in), 1),
                           "out_GBps": round(half_pages * pb / med(b_out) / 1e3, 1),
                           "in_GBps": round(half_pages * pb / med(b_in) / 1e3, 1)}
    res["swap_out_frac_of_link_peak"] = round(res["swap_out_GBps"] / HOST_LINK_GBS, 4)
    res["swap_in_frac_of_link_peak"] = round(res["swap_in_GBps"] / HOST_LINK_GBS, 4)
    return res


def run_block_sweep(names, blocks, reps):
    """Page-size sweep (PageFault, "Stage 2: memory", block-size table: smaller
    pages waste less memory but mean longer tables and more indirection per
    token): the same workload, values and lengths at each block size, shuffled
    frames, cache flushed before every launch.  Reports the attention
    partition kernel's time and algorithmic bandwidth, the kernel family, table
    entries per sequence and the unused tail slots of the reserved pages."""
    import torch
    from paged_kv_cache_43_amd import inputs, pf, runner

    fl = torch.zeros(1 << 30, dtype=torch.uint8, device="cuda")
    out = {}
    for name in names:
        rows = {}
        first = None
        for b in blocks:
            w = inputs.Workload(name, frames="shuffled", block=b)
            if first is not None:
                w.share_values(first)   # values do not depend on the page size
            first = first or w
            kv = runner.PagedKV(w, sentinel=False)
            q = runner.fill_workload(kv)
            mc = int(w.ctx.max())
            kv.ensure_workspace(mc)
            o = torch.empty((w.n, w.hq, w.d), dtype=torch.int32 if w.es == 4 else torch.int16, device="cuda")
            ev = [(TimingEvent(), TimingEvent()) for _ in range(reps + 3)]
            for a, e in ev:
                a.record()
                e.record()
            torch.cuda.synchronize()
            for a, e in ev:
                _flush(fl)
                pf.check(pf.pf_pool_set_timing_events(kv.h, a.cuda_event, e.cuda_event))
                kv.attention(0, q[0], o, mc)
            pf.check(pf.pf_pool_set_timing_events(kv.h, None, None))
            torch.cuda.synchronize()
            t = float(np.median([a.elapsed_time(e) * 1e3 for a, e in ev[3:]]))
            pages = (w.ctx + b - 1) // b
            alg = alg_bytes_attention(w.ctx, w, w.es)   # table entries at this page size
            rows[str(b)] = {"partition_us": round(t, 2), "alg_GBps": round(alg / t / 1e3, 1),
                            "pct_hbm_peak": round(100 * alg / t / 1e3 / HBM_PEAK_GBS, 1),
                            "kernel": "mfma" if pf.pf_attention_kernel(kv.h, w.hq) == 1 else "valu",
                            "table_entries_per_seq": round(float(pages.mean()), 1),
                            "tail_slots_per_seq": round(float((pages * b - w.ctx).mean()), 2),
                            "reserved_utilization": round(float(w.ctx.sum() / (pages * b).sum()), 4)}
            kv.close()
            del kv, q
            torch.cuda.empty_cache()
        out[name] = rows
    return out


def run_fused(names, steps):
    """Fused scatter + attention (PageForge, "Five techniques": a decode step's
    per-layer scatter launches are the cost to remove).  One decode step as a
    model runs it, layer by layer with the new token's K/V known only at its
    layer: table upload, then per layer either pf_scatter_kv + attention
    ("separate") or the fused pf_paged_decode_attention_append ("fused").
    Cache flushed before each step (outside the events); mean step time over
    ``steps`` steps, sequences growing one token per step."""
    import torch
    from paged_kv_cache_43_amd import inputs, pf, runner

    fl = torch.zeros(1 << 30, dtype=torch.uint8, device="cuda")
    res = {}
    for name in names:
        row = {}
        for mode in ("separate", "fused"):
            w = inputs.Workload(name, frames="shuffled")
            kv = runner.PagedKV(w, sentinel=False, extra_tokens=steps + 4)
            q = runner.fill_workload(kv)
            rng = np.random.default_rng(5)
            nk = runner.bits_to_device(inputs.normal_bits(rng, (w.layers, w.n, w.hkv, w.d), w.dtype))
            nv = runner.bits_to_device(inputs.normal_bits(rng, (w.layers, w.n, w.hkv, w.d), w.dtype))
            out = torch.empty((w.n, w.hq, w.d), dtype=torch.int32 if w.es == 4 else torch.int16, device="cuda")
            ids = np.arange(w.n, dtype=np.uint64)
            base = w.ctx.astype(np.int64)
            kv.ensure_workspace(int(base.max()) + steps + 2)
            seq = torch.arange(w.n, dtype=torch.int32, device="cuda")
            times = []
            for t in range(steps + 2):
                lens = (base + t + 1).astype(np.int32)
                pf.check(pf.pf_alloc_for_seqs(kv.h, ids, lens)[0])
                mc = int(lens.max())
                _flush(fl)
                a, b = TimingEvent(), TimingEvent()
                a.record()
                kv.export_tables()
                for l in range(w.layers):
                    if mode == "separate":
                        kv.scatter(l, nk[l], nv[l], seq, kv.last_pos)
                        kv.attention(l, q[l], out, mc)
                    else:
                        kv.attention_append(l, q[l], nk[l], nv[l], out, mc)
                b.record()
                torch.cuda.synchronize()
                if t >= 2:
                    times.append(a.elapsed_time(b))
            row[mode + "_ms_per_step"] = round(float(np.mean(times)), 4)
            kv.close()
            del kv, q
            torch.cuda.empty_cache()
        row["layers"] = w.layers
        row["saved_us_per_layer"] = round((row["separate_ms_per_step"] - row["fused_ms_per_step"]) * 1e3 / w.layers, 2)
        row["speedup"] = round(row["separate_ms_per_step"] / row["fused_ms_per_step"], 4)
        res[name] = row
    return res


def _oracle_pass_worker(barrier, results, wid, dtype, hq, hkv, d, qb, ks, vs, budget_s):
    """One worker of the all-cores oracle leg: whole passes of the fp64 oracle
    over its share of the sequences (q bits [m][hq][d], K/V bits per sequence
    [ctx][hkv][d]) until budget_s seconds are spent, one BLAS thread."""
    sys.path.insert(0, ROOT)
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        pass
    import oracle.attention as oa
    qd = oa.decode_bits(qb, dtype)
    g, sc = hq // hkv, oa.default_scale(d)
    barrier.wait()
    t0 = time.perf_counter()
    done = tokens = 0
    while True:
        for s in range(len(ks)):
            K = oa.decode_bits(ks[s], dtype)
            V = oa.decode_bits(vs[s], dtype)
            for h in range(hq):
                oa.attention(qd[s, h], K[:, h // g, :], V[:, h // g, :], sc)
            done += 1
            tokens += len(ks[s])
        if time.perf_counter() - t0 >= budget_s:
            break
    results.put((wid, done, tokens, time.perf_counter() - t0))


def host_description():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity_cpus": aff}


def cpu_baseline(name, budget_s, max_workers=16):
    """The CPU fp64 oracle (contiguous two-pass softmax attention on decoded
    K/V) on the same workload, layer 0, all query heads.  Headline: the
    sequences split across worker processes, one per usable core (at most
    max_workers), each repeating whole passes over its share for a bounded
    time; also one thread alone, whole passes over every sequence until about
    budget_s seconds are spent."""
    import multiprocessing as mp
    from paged_kv_cache_43_amd import inputs
    import oracle.attention as oa
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        limiter = None
    w = inputs.Workload(name, frames="shuffled")
    ks, vs, qb = w.values()
    qd = oa.decode_bits(qb[0], w.dtype)
    g = w.hq // w.hkv
    sc = oa.default_scale(w.d)
    wl = type("W", (), dict(hq=w.hq, hkv=w.hkv, d=w.d, es=w.es, block=w.block))

    # one thread, whole passes over all sequences
    t0 = time.perf_counter()
    done = 0
    while True:
        for s in range(w.n):
            K = oa.decode_bits(ks[s][0], w.dtype)
            V = oa.decode_bits(vs[s][0], w.dtype)
            for h in range(w.hq):
                oa.attention(qd[s, h], K[:, h // g, :], V[:, h // g, :], sc)
            done += 1
            if done >= w.n and time.perf_counter() - t0 >= budget_s:
                break
        else:
            continue
        break
    el = time.perf_counter() - t0
    if limiter is not None and hasattr(limiter, "unregister"):
        limiter.unregister()
    full, part = divmod(done, w.n)
    ctx1 = np.concatenate([np.tile(w.ctx, full), w.ctx[:part]])
    wl.n = done
    one = {"value": round(alg_bytes_attention(ctx1, wl, w.es) / el / 1e9, 4), "cores": 1,
           "seqs_per_ms": round(done / (el * 1e3), 5), "seconds": round(el, 2),
           "sample": "%d sequence-attentions (%d whole passes over all %d sequences, %d context tokens each "
                     "pass), one thread" % (done, full, w.n, int(w.ctx.sum()))}

    # all usable cores: sequences dealt round-robin to worker processes
    # (started fresh, not forked from this process), timed from a common barrier
    host = host_description()
    nw = max(1, min(max_workers, host["affinity_cpus"] or 1, w.n))
    per_worker_s = max(1.0, 24.0 / nw)
    ctx = mp.get_context("spawn")
    barrier, results = ctx.Barrier(nw), ctx.Queue()
    procs = []
    for k in range(nw):
        idx = list(range(k, w.n, nw))
        procs.append(ctx.Process(target=_oracle_pass_worker, args=(
            barrier, results, k, w.dtype, w.hq, w.hkv, w.d, np.ascontiguousarray(qb[0][idx]),
            [ks[s][0] for s in idx], [vs[s][0] for s in idx], per_worker_s)))
    for pr in procs:
        pr.start()
    res = [results.get(timeout=600) for _ in procs]
    for pr in procs:
        pr.join(timeout=60)
    secs = max(r[3] for r in res)
    seqs = sum(r[1] for r in res)
    bytes_all = 0
    for wid, dn, toks, _ in res:
        idx = np.arange(wid, w.n, nw)
        passes = dn // len(idx)
        wl.n = dn
        bytes_all += alg_bytes_attention(np.tile(w.ctx[idx], passes), wl, w.es)
    return {"value": round(bytes_all / secs / 1e9, 4), "unit": "GB/s", "cores": nw, "kind": "oracle",
            "seqs_per_ms": round(seqs / (secs * 1e3), 5), "seconds": round(secs, 2),
            "sample": "%d sequence-attentions in whole passes, the %d sequences dealt round-robin to %d worker "
                      "processes (one BLAS thread each, %.1f s each, timed from a common barrier), layer 0, all %d "
                      "query heads; decode + fp64 two-pass softmax attention" % (seqs, w.n, nw, per_worker_s, w.hq),
            "sample_short": "%s layer 0, %d sequence-attentions over %d processes, %.0f s" % (
                name, seqs, nw, secs),
            "one_core": one, "host": host}


def describe(r):
    w = r["w"]
    return {"workload": WORKLOADS[r["name"]].format(frames=r["frames"]), "n_seqs": w.n,
            "layers": w.layers, "q_heads": w.hq, "kv_heads": w.hkv, "head_dim": w.d,
            "block_size": 16, "pool_pages": w.num_pages, "frames": r["frames"],
            "schedule": "balanced" if r["waves"] else (
                "whole (sequence, head) items, no merge" if r["whole"] else "fixed splits"),
            "waves": r["waves"] or None, "split_tokens": r["split"] or None,
            "kernel": "mfma" if r["mfma"] else "valu"}


LINE_LIMIT = 4000   # bytes per printed JSON line: every line survives a short stdout tail


def side_line(leg, name, payload):
    """One side measurement as its own JSON line, printed at once."""
    line = {"leg": leg, "name": name}
    line.update(payload)
    text = json.dumps(line)
    if len(text) > LINE_LIMIT:
        # keep the line short: drop the prose, then anything nested
        line = {k: v for k, v in line.items() if k != "what" and k != "sample"}
        for k, v in list(line.items()):
            if isinstance(v, dict):
                line[k] = {a: b for a, b in v.items() if a not in ("what", "sample")}
        text = json.dumps(line)
    print(text, flush=True)
    return line


def workload_summary(r):
    """The figures of one workload run that its side line and the headline share."""
    return {"value_GBps": round(r["value"], 1), "pct_hbm_peak": round(100 * r["value"] / HBM_PEAK_GBS, 1),
            "seqs_per_ms": round(r["seqs_per_ms"], 2), "ms_per_step": round(r["ms_step"], 4),
            "attn_partition_avg_us": round(r["part_avg_us"], 2),
            "attn_partition_GBps": round(r["achieved"], 1)}


def headline_line(head, args, traffic, cpu, cost):
    """The compact headline: metric, value, step time, config, roofline and
    the CPU baseline's figures, all scalars or small dicts (under 4 KB)."""
    w = head["w"]
    line = {
        "metric": "paged decode attention KV GB/s (% of MI355X HBM peak) + sequences/ms",
        "value": round(head["value"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": describe(head),
        "pct_hbm_peak": round(100 * head["value"] / HBM_PEAK_GBS, 1),
        "seqs_per_ms": round(head["seqs_per_ms"], 2),
        "ms_per_step_wall": round(head["ms_step_wall"], 4),
        "attention_median_us": head["attention"]["median_us"],
        "attention_pct_hbm_peak": head["attention"]["pct_hbm_peak"],
        "scatter_median_us": head["scatter"]["median_us"],
        "roofline": {"bound": "hbm", "achieved": round(head["achieved"], 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(head["achieved"] / HBM_PEAK_GBS, 4),
                     "traffic": traffic[0] if traffic else None,
                     "traffic_alg_bytes": traffic[1] if traffic else None,
                     "traffic_over_alg": round(traffic[0] / traffic[1], 4) if traffic and traffic[1] else None,
                     "kernel": "attention partition", "avg_launch_us": round(head["part_avg_us"], 2),
                     "median_launch_us": round(head["part_med_us"], 2),
                     "alg_bytes_per_launch": int(head["attn_bytes"])},
        "shuffled_over_ordered": cost,
    }
    if cpu is not None:
        line["cpu_baseline"] = {"value": cpu["value"], "unit": cpu["unit"], "cores": cpu["cores"],
                                "kind": cpu["kind"], "seqs_per_ms": cpu["seqs_per_ms"],
                                "seconds": cpu["seconds"], "sample": cpu["sample_short"],
                                "one_core_GBps": cpu["one_core"]["value"]}
    return line


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="13b", choices=sorted(WORKLOADS))
    ap.add_argument("--frames", default="shuffled", choices=["shuffled", "ordered"])
    ap.add_argument("--also", default="gqa,13b_32k,gqa_32k,gqa_1m,mixed,mixed_s7,gpt2,tiny",
                    help="comma list of extra configs reported beside the headline (both frame orders)")
    ap.add_argument("--flush", choices=["on", "off"], default="on",
                    help="read a 1 GiB buffer before every step, outside the step's events (default on)")
    ap.add_argument("--twin", default="13b,gqa",
                    help="comma list of configs for the paged vs contiguous-cache comparison (shuffled frames)")
    ap.add_argument("--twin-reps", type=int, default=20)
    ap.add_argument("--fused", default="gpt2,mixed,13b,gqa",
                    help="comma list of configs for the fused scatter + attention comparison")
    ap.add_argument("--block-sweep", default="13b,gqa",
                    help="comma list of configs for the page-size sweep (8, 16, 32, 64 tokens per page)")
    ap.add_argument("--swap", choices=["on", "off"], default="on",
                    help="swap out/in leg (16 sequences, 13B-style heads)")
    ap.add_argument("--cow", choices=["on", "off"], default="on",
                    help="copy-on-write prefix sharing leg (16 prompts x beam 4, 13B-style heads)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first copy a 256 MiB buffer 3 times (a plain copy kernel of known size, "
                         "the reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: measures one GPU only (the path has no multi-GPU part); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.synchronize()
    if args.calibrate_copy:
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    flush = args.flush == "on"

    def report(name, r):
        summary = workload_summary(r)
        side_line("workload", "%s_%s" % (name, r["frames"]), dict(
            summary, attention=r["attention"], scatter=r["scatter"], config=describe(r)))
        return summary

    head = run_gpu(args, args.config, args.frames, args.steps, args.warmup, flush)
    report(args.config, head)
    head_ordered = run_gpu(args, args.config, "ordered" if args.frames == "shuffled" else "shuffled",
                           args.steps, args.warmup, flush, share=head["w"])
    report(args.config, head_ordered)
    head["w"].drop_values()
    head_ordered["w"].drop_values()
    attn = {(args.config, head["frames"]): head["attention"],
            (args.config, head_ordered["frames"]): head_ordered["attention"]}
    for extra in [x for x in args.also.split(",") if x and x != args.config]:
        first = None
        for fr in ("shuffled", "ordered"):
            r = run_gpu(args, extra, fr, args.steps, args.warmup, flush,
                        share=first["w"] if first else None)
            report(extra, r)
            attn[(extra, fr)] = r["attention"]
            if first is not None:   # both frame orders done: the drawn values are no longer needed
                first["w"].drop_values()
                r["w"].drop_values()
            first = first or r
    # PageFault's pending "cost of scattering pages": shuffled / ordered median
    # attention time (partition + merge)
    cost = {}
    for name in dict.fromkeys(n for n, _ in attn):
        a_s, a_o = attn.get((name, "shuffled")), attn.get((name, "ordered"))
        if a_s and a_o:
            cost[name] = round(a_s["median_us"] / a_o["median_us"], 3)
    for name in [x for x in args.twin.split(",") if x]:
        side_line("paged_vs_contiguous", name, run_twin(name, "shuffled", args.twin_reps))
    if args.cow == "on":
        side_line("cow_prefix_sharing", "13b_heads_16x4", run_cow(16, 4, 20))
    if args.swap == "on":
        side_line("swap", "13b_heads_16", run_swap(16, 10))
    fused = [x for x in args.fused.split(",") if x]
    if fused:
        for name, row in run_fused(fused, 10).items():
            side_line("fused_scatter_attention", name, row)
    sweep = [x for x in args.block_sweep.split(",") if x]
    if sweep:
        for name, rows in run_block_sweep(sweep, (8, 16, 32, 64), 15).items():
            side_line("block_size_sweep", name, {"rows": rows})
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.config, args.cpu_seconds)
        side_line("cpu_baseline", args.config, cpu)
    traffic = measured_traffic(args.config)
    print(json.dumps(headline_line(head, args, traffic, cpu, cost)), flush=True)


if __name__ == "__main__":
    main()
