"""GPU: paged decode attention against the fp64 oracle (max-abs error <= 2e-3,
plus half an output ulp when the output is 16-bit), ordered vs shuffled frames
bitwise equal, and the edge cases: empty, single-token and ragged contexts,
split invariance, grouped heads, every head dim, invalid table entries."""
import numpy as np
import pytest

import gpu_util as gu
import oracle.attention as oa
import oracle.layout as ol
from paged_kv_cache_43_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _r():
    from paged_kv_cache_43_amd import runner
    return runner


SCHED_GRID, SCHED_BALANCED = 1, 2


def _run(w, layer=0, out_dtype=None, split=None, mfma=None, kv=None, q=None, sched=None, waves=None):
    r = _r()
    from paged_kv_cache_43_amd import pf
    own = kv is None
    if own:
        kv = r.PagedKV(w)
        q = r.fill_workload(kv)
    if split is not None:
        pf.check(pf.pf_pool_set_option(kv.h, pf.PF_OPT_SPLIT_TOKENS, split))
    if mfma is not None:
        pf.check(pf.pf_pool_set_option(kv.h, pf.PF_OPT_GQA_MFMA, mfma))
    if sched is not None:
        pf.check(pf.pf_pool_set_option(kv.h, pf.PF_OPT_SCHEDULE, sched))
    if waves is not None:
        pf.check(pf.pf_pool_set_option(kv.h, pf.PF_OPT_WAVES_PER_CU, waves))
    od = out_dtype or w.dtype
    out = torch.empty((w.n, w.hq, w.d), dtype=torch.float32 if od == "f32" else
                      (torch.int32 if w.dtype == "f32" else torch.int16), device="cuda")
    kv.attention(layer, q[layer], out, int(w.ctx.max()) if w.n else 0, out_dtype=od)
    torch.cuda.synchronize()
    res = gu.out_to_f64(out, od if w.dtype != "f32" else "f32")
    if own:
        return res, kv, q
    return res


@pytest.mark.parametrize("sched", [SCHED_GRID, SCHED_BALANCED])
@pytest.mark.parametrize("name", ["tiny", "gpt2", "mixed", "mixed_s7"])
@pytest.mark.parametrize("out_dtype", ["f32", None])
def test_attention_parity_small_configs(name, out_dtype, sched):
    print("parity", name, out_dtype, sched, flush=True)
    w = inputs.Workload(name, frames="shuffled")
    layers = sorted({0, w.layers // 2, w.layers - 1})
    res, kv, q = _run(w, layers[0], out_dtype, sched=sched)
    for layer in layers:
        got = res if layer == layers[0] else _run(w, layer, out_dtype, kv=kv, q=q)
        ref = gu.oracle_attention_contiguous(w, layer)
        err = gu.assert_close(got, ref, out_dtype or w.dtype, "%s layer %d" % (name, layer))
        print("  layer", layer, "max err", err, flush=True)
    kv.close()


@pytest.mark.parametrize("name", ["tiny", "gpt2", "mixed", "mixed_s7", "13b", "gqa", "13b_32k", "gqa_32k"])
def test_ordered_equals_shuffled_bitwise(name):
    print("ordered vs shuffled", name, flush=True)
    wa = inputs.Workload(name, frames="ordered")
    a, kva, _ = _run(wa)
    kva.close()
    b, kvb, _ = _run(inputs.Workload(name, frames="shuffled").share_values(wa))
    kvb.close()
    assert np.array_equal(a, b)


@pytest.mark.parametrize("name", ["mixed", "gqa", "gqa_32k"])
def test_schedules_agree(name):
    """Fixed splits and the balanced schedule (several wave counts, so the
    slices fall differently) give the same results to fp32 rounding."""
    print("schedules", name, flush=True)
    w = inputs.Workload(name, frames="shuffled")
    base, kv, q = _run(w, out_dtype="f32", sched=SCHED_GRID)
    ref = gu.oracle_attention_contiguous(w, 0)
    gu.assert_close(base, ref, "f32", name + " grid")
    for waves in (1, 3, 16, 40):
        got = _run(w, out_dtype="f32", kv=kv, q=q, sched=SCHED_BALANCED, waves=waves)
        assert np.max(np.abs(got - base)) <= 1e-5, waves
        gu.assert_close(got, ref, "f32", "%s balanced %d" % (name, waves))
    kv.close()


@pytest.mark.parametrize("name", ["13b", "gqa", "13b_32k", "gqa_32k", "gqa_1m"])
def test_attention_parity_full_size(name):
    """The bench's configurations at full size, in the launch configuration it
    times; every output against the oracle on the generated K/V, and sampled
    sequences through the oracle's own read-back of the device pool."""
    print("parity full", name, flush=True)
    w = inputs.Workload(name, frames="shuffled")
    got, kv, q = _run(w)
    ref = gu.oracle_attention_contiguous(w, 0)
    err = gu.assert_close(got, ref, w.dtype, name)
    print("  max err", err, flush=True)
    got32 = _run(w, out_dtype="f32", kv=kv, q=q)
    print("  f32-out max err", gu.assert_close(got32, ref, "f32", name + " f32 out"), flush=True)
    pool = _r().bits_from_device(kv.pool)
    model = gu.oracle_tables(w)
    g = gu.geometry(w)
    rng = np.random.default_rng(1)
    ks, vs, qb = w.values()
    if int(w.ctx.max()) <= 4096:
        sample = sorted(rng.choice(w.n, size=3, replace=False).tolist())
        paged = oa.paged_decode_attention(qb[0][sample], pool, g, 0, [model.table(s) for s in sample],
                                          [int(w.ctx[s]) for s in sample], w.dtype)
        assert np.array_equal(paged, ref[sample])
    else:
        # 32k-token contexts: one sequence read back through its table (bit-exact
        # against the drawn K/V) and a few heads attended from the read-back bits
        s = int(rng.integers(w.n))
        kc, vc = ol.readback(pool, g, 0, model.table(s), int(w.ctx[s]))
        assert np.array_equal(kc, ks[s][0]) and np.array_equal(vc, vs[s][0])
        qd = oa.decode_bits(qb[0][s], w.dtype)
        grp = w.hq // w.hkv
        for h in sorted(rng.choice(w.hq, size=4, replace=False).tolist()):
            K = oa.decode_bits(np.ascontiguousarray(kc[:, h // grp, :]), w.dtype)
            V = oa.decode_bits(np.ascontiguousarray(vc[:, h // grp, :]), w.dtype)
            assert np.array_equal(oa.attention(qd[h], K, V, oa.default_scale(w.d)), ref[s, h])
    kv.close()


def _custom(lens, hq=2, hkv=2, d=16, dtype="f32", seed=0, layers=1):
    """A small workload with given lengths and shape (the tiny config's recipe)."""
    w = inputs.Workload("tiny", seed=seed, frames="shuffled", lens=lens)
    w.hq, w.hkv, w.d, w.dtype, w.es, w.layers = hq, hkv, d, dtype, inputs.DTYPE_BYTES[dtype], layers
    need = sum(-(-int(c) // 16) for c in lens)
    w.num_pages = max(need + 8, 16)
    w.free_order = np.random.default_rng(seed + 99).permutation(w.num_pages)
    return w


@pytest.mark.parametrize("shape", [("f32", 2, 2, 16), ("f16", 12, 12, 64), ("bf16", 14, 2, 64),
                                   ("f16", 8, 1, 128), ("bf16", 6, 3, 128)])
def test_short_contexts_whole_items(shape):
    """The automatic plan on contexts of at most 256 tokens: one wave per whole
    (sequence, head) -- per kv head for the matrix-core kernel -- no workspace
    and no merge, against the oracle, with empty and one-token sequences, a
    page boundary and the 256-token limit."""
    dtype, hq, hkv, d = shape
    print("whole items", shape, flush=True)
    from paged_kv_cache_43_amd import pf
    lens = [0, 1, 15, 16, 17, 100, 255, 256] + np.random.default_rng(d).integers(1, 257, size=24).tolist()
    w = _custom(lens, hq=hq, hkv=hkv, d=d, dtype=dtype, seed=hq)
    for od in (["f32", None] if dtype != "f32" else [None]):
        r = _r()
        kv = r.PagedKV(w)
        q = r.fill_workload(kv)
        assert pf.pf_attention_waves(kv.h, w.n, hq, 256) == 0
        assert pf.pf_attention_split_tokens(kv.h, w.n, hq, 256) == 256
        assert pf.pf_attention_workspace_bytes(kv.h, w.n, hq, 256) == 0
        got = _run(w, out_dtype=od, kv=kv, q=q)
        gu.assert_close(got, gu.oracle_attention_contiguous(w, 0), od or dtype, "whole items %s" % (shape,))
        kv.close()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [16, 32, 64, 128, 256])
def test_head_dims_and_dtypes(dtype, d):
    """Every head dim with every element type, both schedules requested (fp32
    at head dim 256 always runs balanced, in 8-token units)."""
    print("head dim", d, dtype, flush=True)
    w = _custom([1, 15, 16, 17, 33, 200, 513], hq=4, hkv=2, d=d, dtype=dtype, seed=d)
    for od in (["f32", None] if dtype != "f32" else [None]):
        for sched in (SCHED_GRID, SCHED_BALANCED):
            got, kv, q = _run(w, out_dtype=od, mfma=0, sched=sched)
            ref = gu.oracle_attention_contiguous(w, 0)
            gu.assert_close(got, ref, od or dtype, "d=%d %s sched %d" % (d, dtype, sched))
            kv.close()


@pytest.mark.parametrize("sched", [SCHED_GRID, SCHED_BALANCED])
def test_edge_lengths_and_empty(sched):
    print("edge lengths", sched, flush=True)
    lens = [0, 1, 2, 15, 16, 17, 31, 32, 33, 255, 256, 257, 1000, 0]
    w = _custom(lens, hq=3, hkv=3, d=64, dtype="f16", seed=3)
    got, kv, q = _run(w, out_dtype="f32", sched=sched, waves=2 if sched == SCHED_BALANCED else None)
    ref = gu.oracle_attention_contiguous(w, 0)
    gu.assert_close(got, ref, "f32", "edge")
    assert np.all(got[0] == 0) and np.all(got[-1] == 0)
    # a single token returns its value (exactly, up to the output rounding)
    _, vs, _ = w.values()
    one = oa.decode_bits(vs[1][0], "f16")[0]
    assert np.max(np.abs(got[1] - one[None, :])) <= 1e-6
    kv.close()


@pytest.mark.parametrize("mfma", [0, 1])
@pytest.mark.parametrize("sched", [0, SCHED_GRID, SCHED_BALANCED])
def test_lengths_clamped_to_bound(sched, mfma):
    """Device lengths outside [0, max_context_len] are clamped into it: a
    negative length attends to nothing (zeros), one above the bound attends to
    the first max_context_len tokens.  Schedule 0 with a bound of at most 256
    tokens is the whole-item path."""
    from paged_kv_cache_43_amd import pf
    print("clamped lengths", sched, mfma, flush=True)
    w = _custom([100, 300, 50, 600, 37], hq=8, hkv=2, d=64, dtype="bf16", seed=21)
    r = _r()
    kv = r.PagedKV(w)
    q = r.fill_workload(kv)
    pf.check(pf.pf_pool_set_option(kv.h, pf.PF_OPT_GQA_MFMA, mfma))
    pf.check(pf.pf_pool_set_option(kv.h, pf.PF_OPT_SCHEDULE, sched))
    bound = 250
    dev = [100, 900, -7, 600, 37]
    kv.ctx.copy_(torch.tensor(dev, dtype=torch.int32))
    out = torch.full((w.n, w.hq, w.d), float("nan"), dtype=torch.float32, device="cuda")
    kv.attention(0, q[0], out, bound, out_dtype="f32")
    torch.cuda.synchronize()
    got = gu.out_to_f64(out, "f32")
    ks, vs, qb = w.values()
    qd = oa.decode_bits(qb[0], w.dtype)
    g = w.hq // w.hkv
    for s, n in enumerate(dev):
        eff = min(max(n, 0), bound)
        if eff == 0:
            assert np.all(got[s] == 0), s
            continue
        for hk in range(w.hkv):
            K = oa.decode_bits(np.ascontiguousarray(ks[s][0][:eff, hk, :]), w.dtype)
            V = oa.decode_bits(np.ascontiguousarray(vs[s][0][:eff, hk, :]), w.dtype)
            for h in range(hk * g, (hk + 1) * g):
                ref = oa.attention(qd[s, h], K, V, oa.default_scale(w.d))
                assert np.max(np.abs(got[s, h] - ref)) <= gu.ATOL, (s, h)
    kv.close()


@pytest.mark.parametrize("pattern", ["rising", "late_jump", "one_survivor", "flat"])
@pytest.mark.parametrize("dtype,hq,hkv,d", [("f16", 8, 2, 64), ("bf16", 14, 2, 64), ("bf16", 4, 4, 128),
                                            ("f32", 2, 2, 64)])
def test_score_extremes(pattern, dtype, hq, hkv, d):
    """Scores forced along each sequence: every query head gets the same unit
    vector u and token t's key is a_t * sqrt(D) * u, so its score is about
    a_t -- rising to 40 (the running max is raised again and again), one
    score 60 above the rest near the end, all at -60 but one, all equal (the
    mean of V).  Both schedules, vector and matrix-core kernels, against the
    oracle on the stored bits."""
    from paged_kv_cache_43_amd import runner
    print("score extremes", pattern, dtype, hq, hkv, d, flush=True)
    lens = [1, 17, 300, 2000]
    w = _custom(lens, hq, hkv, d, dtype, seed=d + hq)
    kv = runner.PagedKV(w)
    q = runner.fill_workload(kv)
    rng = np.random.default_rng(5)
    sign = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    qbits = inputs.to_bits(np.broadcast_to(sign / np.sqrt(d), (w.n, w.hq, d)), dtype)
    q[0].copy_(runner.bits_to_device(qbits))
    _, vs, _ = w.values()
    kbits = []
    for n in lens:
        if pattern == "rising":
            a = 40.0 * np.arange(1, n + 1) / n
        elif pattern == "late_jump":
            a = np.zeros(n)
            a[max(0, n - 3)] = 60.0
        elif pattern == "one_survivor":
            a = np.full(n, -60.0)
            a[n // 3] = 0.0
        else:
            a = np.zeros(n)
        kbits.append(inputs.to_bits(a[:, None, None] * np.broadcast_to(sign, (1, hkv, d)), dtype))
    tok_seq, tok_pos = runner.token_arrays(w, [range(n) for n in lens])
    kv.scatter(0, runner.bits_to_device(np.concatenate(kbits)),
               runner.bits_to_device(np.concatenate([vs[s][0] for s in range(w.n)])),
               torch.from_numpy(tok_seq).cuda(), torch.from_numpy(tok_pos).cuda())
    qd = oa.decode_bits(qbits, dtype)
    g = hq // hkv
    ref = np.zeros((w.n, hq, d))
    for s in range(w.n):
        K = oa.decode_bits(kbits[s], dtype)
        V = oa.decode_bits(vs[s][0], dtype)
        for h in range(hq):
            ref[s, h] = oa.attention(qd[s, h], K[:, h // g], V[:, h // g], oa.default_scale(d))
    if pattern == "flat":
        for s in range(w.n):
            V = oa.decode_bits(vs[s][0], dtype)
            assert np.allclose(ref[s], V.mean(axis=0)[np.arange(hq) // g], atol=1e-12)
    for mfma in (0, 1):
        for sched in (SCHED_GRID, SCHED_BALANCED):
            got = _run(w, out_dtype="f32", mfma=mfma, sched=sched, kv=kv, q=q)
            gu.assert_close(got, ref, "f32", "%s mfma %d sched %d" % (pattern, mfma, sched))
    kv.close()


@pytest.mark.parametrize("split", [16, 32, 64, 128, 512, 1024])
def test_split_invariance(split):
    print("split", split, flush=True)
    lens = [1, 16, 100, 1024, 3000, 4096]
    w = _custom(lens, hq=4, hkv=4, d=64, dtype="bf16", seed=11)
    base, kv, q = _run(w, out_dtype="f32", split=1024, sched=SCHED_GRID)
    got = _run(w, out_dtype="f32", split=split, kv=kv, q=q)
    assert np.max(np.abs(got - base)) <= 1e-5
    ref = gu.oracle_attention_contiguous(w, 0)
    gu.assert_close(got, ref, "f32", "split %d" % split)
    kv.close()


@pytest.mark.parametrize("group", [1, 2, 3, 4, 7, 8, 16, 32])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_grouped_heads(group, dtype):
    print("group", group, dtype, flush=True)
    hkv = 2
    w = _custom([5, 64, 300, 1500], hq=group * hkv, hkv=hkv, d=64, dtype=dtype, seed=group)
    for mfma in (0, 1):
        for sched in (SCHED_GRID, SCHED_BALANCED):
            got, kv, q = _run(w, out_dtype="f32", mfma=mfma, sched=sched, waves=1 if sched == SCHED_BALANCED else None)
            from paged_kv_cache_43_amd import pf
            # the matrix-core kernel takes groups of 2 to 16 heads; others run on the vector kernel
            assert pf.pf_attention_kernel(kv.h, w.hq) == (1 if mfma and 1 < group <= 16 else 0)
            ref = gu.oracle_attention_contiguous(w, 0)
            gu.assert_close(got, ref, "f32", "group %d mfma %d sched %d" % (group, mfma, sched))
            kv.close()


@pytest.mark.parametrize("sched", [SCHED_GRID, SCHED_BALANCED])
def test_invalid_table_entry_contributes_nothing(sched):
    """A table entry that is not a valid page is skipped without any access
    outside the pool; the result is attention over the remaining tokens."""
    print("invalid entry", sched, flush=True)
    w = _custom([40, 40], hq=2, hkv=2, d=16, dtype="f32", seed=5)
    r = _r()
    kv = r.PagedKV(w)
    q = r.fill_workload(kv)
    bt = kv.bt.clone()
    bt[0, 1] = -1           # tokens 16..31 of sequence 0
    bt[1, 2] = w.num_pages  # tokens 32..39 of sequence 1
    kv.bt.copy_(bt)
    got = _run(w, out_dtype="f32", kv=kv, q=q, sched=sched, waves=1 if sched == SCHED_BALANCED else None)
    ks, vs, qb = w.values()
    qd = oa.decode_bits(qb[0], "f32")
    for s, drop in ((0, range(16, 32)), (1, range(32, 40))):
        keep = [t for t in range(40) if t not in drop]
        K = oa.decode_bits(ks[s][0], "f32")[keep]
        V = oa.decode_bits(vs[s][0], "f32")[keep]
        for h in range(2):
            ref = oa.attention(qd[s, h], K[:, h], V[:, h], oa.default_scale(16))
            assert np.max(np.abs(got[s, h] - ref)) <= gu.ATOL
    kv.close()


def test_scale_argument():
    print("scale", flush=True)
    w = _custom([10, 70], hq=2, hkv=2, d=16, dtype="f32", seed=8)
    r = _r()
    kv = r.PagedKV(w)
    q = r.fill_workload(kv)
    out = torch.empty((w.n, w.hq, w.d), dtype=torch.float32, device="cuda")
    kv.attention(0, q[0], out, int(w.ctx.max()), scale=0.9)
    torch.cuda.synchronize()
    got = gu.out_to_f64(out, "f32")
    ref = gu.oracle_attention_contiguous(w, 0, scale=0.9)
    gu.assert_close(got, ref, "f32", "scale 0.9")
    kv.close()


@pytest.mark.parametrize("block", [8, 32, 64])
@pytest.mark.parametrize("dtype,hq,hkv,d", [("f16", 4, 4, 128), ("bf16", 14, 2, 64), ("f16", 8, 2, 128)])
@pytest.mark.parametrize("out_dtype", ["f32", None])
def test_block_sizes(block, dtype, hq, hkv, d, out_dtype):
    """Pages of 8, 32 and 64 tokens: lengths on both sides of every unit and
    page boundary, vector kernel and (for 32 and 64) the matrix-core kernel;
    ordered and shuffled frames give the same bits."""
    print("block", block, dtype, hq, hkv, d, out_dtype, flush=True)
    from paged_kv_cache_43_amd import pf
    lens = [0, 1, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 200, 513, 1000]
    res = {}
    for frames in ("ordered", "shuffled"):
        w = inputs.Workload("tiny", seed=block + d, frames=frames, lens=lens, block=block)
        w.hq, w.hkv, w.d, w.dtype, w.es = hq, hkv, d, dtype, inputs.DTYPE_BYTES[dtype]
        w.num_pages = sum(-(-int(c) // block) for c in lens) + 8
        w.free_order = (np.arange(w.num_pages) if frames == "ordered"
                        else np.random.default_rng(block).permutation(w.num_pages))
        got, kv, q = _run(w, out_dtype=out_dtype)
        mfma = pf.pf_attention_kernel(kv.h, hq) == 1
        assert mfma == (hq > hkv), (block, mfma)
        od = out_dtype or dtype
        gu.assert_close(got, gu.oracle_attention_contiguous(w, 0), od, "block %d %s" % (block, frames))
        res[frames] = got
        kv.close()
    assert np.array_equal(res["ordered"], res["shuffled"])


@pytest.mark.parametrize("name", ["13b", "gqa"])
def test_block_sizes_full_size(name):
    """The page-size sweep's workloads at full size (the same lengths and
    values at 8, 32 and 64 tokens per page, shuffled frames): every output
    against the oracle, 16-bit and fp32 output."""
    print("block sizes full", name, flush=True)
    ref = None
    for block in (8, 32, 64):
        w = inputs.Workload(name, frames="shuffled", block=block)
        if ref is None:
            ref = gu.oracle_attention_contiguous(w, 0)
        got, kv, q = _run(w)
        err = gu.assert_close(got, ref, w.dtype, "%s block %d" % (name, block))
        got32 = _run(w, out_dtype="f32", kv=kv, q=q)
        err32 = gu.assert_close(got32, ref, "f32", "%s block %d f32 out" % (name, block))
        print("  block", block, "max err", err, "f32 out", err32, flush=True)
        kv.close()


@pytest.mark.parametrize("block,drops", [(8, {0: [1], 1: [2], 2: [4]}), (32, {0: [0], 1: [1]}),
                                         (16, {0: [1], 1: [2], 2: [0]})])
def test_invalid_entries_grouped_heads(block, drops):
    """Matrix-core kernel with invalid table entries at every position a page
    can hold in a tile: with 8-token pages the first or the second page of a
    16-token tile (the other half still counts), with 32-token pages a page of
    two tiles.  The result is attention over the remaining tokens."""
    print("invalid entries mfma block", block, flush=True)
    from paged_kv_cache_43_amd import pf
    lens = [40, 45, 80]
    w = inputs.Workload("tiny", seed=block, frames="shuffled", lens=lens, block=block)
    w.hq, w.hkv, w.d, w.dtype, w.es = 4, 2, 64, "bf16", 2
    w.num_pages = sum(-(-c // block) for c in lens) + 8
    w.free_order = np.random.default_rng(block + 1).permutation(w.num_pages)
    r = _r()
    kv = r.PagedKV(w)
    q = r.fill_workload(kv)
    assert pf.pf_attention_kernel(kv.h, 4) == 1
    bt = kv.bt.clone()
    for s, pages in drops.items():
        for i, page_idx in enumerate(pages):
            bt[s, page_idx] = -1 if i % 2 == 0 else w.num_pages
    kv.bt.copy_(bt)
    got = _run(w, out_dtype="f32", kv=kv, q=q)
    ks, vs, qb = w.values()
    qd = oa.decode_bits(qb[0], "bf16")
    for s, n in enumerate(lens):
        drop = {t for p_ in drops.get(s, []) for t in range(p_ * block, (p_ + 1) * block)}
        keep = [t for t in range(n) if t not in drop]
        K = oa.decode_bits(ks[s][0], "bf16")[keep]
        V = oa.decode_bits(vs[s][0], "bf16")[keep]
        for h in range(4):
            ref = oa.attention(qd[s, h], K[:, h // 2], V[:, h // 2], oa.default_scale(64))
            assert np.max(np.abs(got[s, h] - ref)) <= gu.ATOL, (s, h)
    kv.close()


@pytest.mark.parametrize("n", [2048, 2049, 3000])
@pytest.mark.parametrize("dtype,hq,hkv", [("f16", 2, 2), ("bf16", 8, 2)])
def test_many_sequences(n, dtype, hq, hkv):
    """Up to 2048 sequences the balanced schedule holds every length in LDS;
    beyond that the automatic plan switches to fixed splits (contexts over 256
    tokens; shorter ones are whole items either way).  Both against the
    oracle; the plan is as stated."""
    print("many sequences", n, dtype, hq, hkv, flush=True)
    from paged_kv_cache_43_amd import pf
    lens = np.random.default_rng(n).integers(1, 120, size=n).tolist()
    lens[n // 2] = 300
    w = _custom(lens, hq=hq, hkv=hkv, d=64, dtype=dtype, seed=n % 97)
    got, kv, q = _run(w, out_dtype="f32")
    waves = pf.pf_attention_waves(kv.h, w.n, hq, int(max(lens)))
    assert (waves > 0) == (n <= 2048)
    ref = gu.oracle_attention_contiguous(w, 0)
    gu.assert_close(got, ref, "f32", "n=%d" % n)
    kv.close()
