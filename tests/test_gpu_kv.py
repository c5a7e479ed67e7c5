"""GPU: scatter_kv writes exactly the oracle's pool image, and gather_kv reads
back exactly what was written (bit-exact, NaN-sentinel pool)."""
import numpy as np
import pytest

import gpu_util as gu
import oracle.layout as ol
from paged_kv_cache_43_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _runner():
    from paged_kv_cache_43_amd import runner
    return runner


@pytest.mark.parametrize("name,frames", [("tiny", "shuffled"), ("tiny", "ordered"),
                                         ("gpt2", "shuffled"), ("mixed", "ordered")])
def test_scatter_pool_image_bit_exact(name, frames):
    print("scatter image", name, frames, flush=True)
    r = _runner()
    w = inputs.Workload(name, frames=frames)
    kv = r.PagedKV(w)
    r.fill_workload(kv)
    torch.cuda.synchronize()
    got = r.bits_from_device(kv.pool)
    model = gu.oracle_tables(w)
    tables = [model.table(s) for s in range(w.n)]
    g = gu.geometry(w)
    ks, vs, _ = w.values()
    exp = ol.empty_pool(g, inputs.NAN_BITS[w.dtype])
    tok_seq = [s for s in range(w.n) for _ in range(int(w.ctx[s]))]
    tok_pos = [p for s in range(w.n) for p in range(int(w.ctx[s]))]
    for layer in range(w.layers):
        k = np.concatenate([ks[s][layer] for s in range(w.n)])
        v = np.concatenate([vs[s][layer] for s in range(w.n)])
        exp = ol.scatter(exp, g, layer, k, v, tok_seq, tok_pos, tables)
    assert got.shape == exp.shape
    diff = np.flatnonzero(got != exp)
    assert diff.size == 0, "first differing elements: %s" % diff[:5].tolist()
    kv.close()


@pytest.mark.parametrize("name,frames", [("tiny", "shuffled"), ("gpt2", "ordered"), ("mixed", "shuffled"),
                                         ("13b", "shuffled"), ("gqa", "shuffled")])
def test_gather_readback_bit_exact(name, frames):
    print("gather", name, frames, flush=True)
    r = _runner()
    w = inputs.Workload(name, frames=frames)
    kv = r.PagedKV(w)
    r.fill_workload(kv)
    ks, vs, _ = w.values()
    max_len = int(w.ctx.max())
    layers = sorted({0, w.layers - 1})
    rng = np.random.default_rng(0)
    sample = sorted(rng.choice(w.n, size=min(w.n, 6), replace=False).tolist())
    pool = None
    model = None
    if w.num_pages * w.layers * w.hkv * 2 * 16 * w.d * w.es <= 2 << 30:
        pool = r.bits_from_device(kv.pool)
        model = gu.oracle_tables(w)
    for layer in layers:
        k, v = kv.gather(layer, max_len)
        kb = r.bits_from_device(k)
        vb = r.bits_from_device(v)
        for s in range(w.n):
            c = int(w.ctx[s])
            assert np.array_equal(kb[s, :c], ks[s][layer]), (layer, s)
            assert np.array_equal(vb[s, :c], vs[s][layer]), (layer, s)
        if pool is not None:
            g = gu.geometry(w)
            for s in sample:
                ok, ov = ol.readback(pool, g, layer, model.table(s), int(w.ctx[s]))
                assert np.array_equal(ok, kb[s, :int(w.ctx[s])]) and np.array_equal(ov, vb[s, :int(w.ctx[s])])
    kv.close()


def test_scatter_decode_steps_incremental():
    """A decode loop: each step allocates one more token per sequence, exports
    the tables, and scatters just the new token; the pool ends equal to the
    oracle image of all tokens."""
    print("scatter incremental", flush=True)
    r = _runner()
    w = inputs.Workload("tiny", frames="shuffled")
    kv = r.PagedKV(w, extra_tokens=40)
    ks, vs, _ = w.values()
    steps = 40
    rng = np.random.default_rng(5)
    newk = [inputs.normal_bits(rng, (steps, w.hkv, w.d), w.dtype) for _ in range(w.n)]
    newv = [inputs.normal_bits(rng, (steps, w.hkv, w.d), w.dtype) for _ in range(w.n)]
    kv.apply(w.history_ops + w.step_ops)
    kv.export_tables()
    r_seq, r_pos = r.token_arrays(w, [range(int(c)) for c in w.ctx])
    kv.scatter(0, r.bits_to_device(np.concatenate([ks[s][0] for s in range(w.n)])),
               r.bits_to_device(np.concatenate([vs[s][0] for s in range(w.n)])),
               torch.from_numpy(r_seq).cuda(), torch.from_numpy(r_pos).cuda())
    ops = list(w.history_ops + w.step_ops)
    for t in range(steps):
        step = [("alloc", s, int(w.ctx[s]) + t + 1) for s in range(w.n)]
        kv.apply(step)
        ops += step
        kv.export_tables()
        ts = torch.arange(w.n, dtype=torch.int32).cuda()
        tp = torch.tensor([int(w.ctx[s]) + t for s in range(w.n)], dtype=torch.int32).cuda()
        kv.scatter(0, r.bits_to_device(np.stack([newk[s][t] for s in range(w.n)])),
                   r.bits_to_device(np.stack([newv[s][t] for s in range(w.n)])), ts, tp)
        torch.cuda.synchronize()
    got = r.bits_from_device(kv.pool)
    model = gu.oracle_tables(w, ops)
    g = gu.geometry(w)
    exp = ol.empty_pool(g, inputs.NAN_BITS[w.dtype])
    for s in range(w.n):
        c = int(w.ctx[s])
        k = np.concatenate([ks[s][0], newk[s]])
        v = np.concatenate([vs[s][0], newv[s]])
        exp = ol.scatter(exp, g, 0, k, v, [s] * (c + steps), list(range(c + steps)),
                         [model.table(x) for x in range(w.n)])
    assert np.array_equal(got, exp)
    kv.close()


def test_scatter_skips_out_of_range_tokens():
    """Tokens whose row, position or table entry is out of range write nothing."""
    print("scatter out of range", flush=True)
    r = _runner()
    w = inputs.Workload("tiny", frames="shuffled")
    kv = r.PagedKV(w)
    kv.apply(w.history_ops + w.step_ops)
    kv.export_tables()
    before = r.bits_from_device(kv.pool).copy()
    bt = kv.bt.clone()
    bt[0, 0] = -1
    bt[1, 0] = w.num_pages
    kv.bt.copy_(bt)
    ts = torch.tensor([0, 1, -1, w.n, 2, 3], dtype=torch.int32).cuda()
    tp = torch.tensor([0, 0, 0, 0, -5, kv.max_blocks * 16], dtype=torch.int32).cuda()
    rng = np.random.default_rng(1)
    k = r.bits_to_device(inputs.normal_bits(rng, (6, w.hkv, w.d), w.dtype))
    kv.scatter(0, k, k, ts, tp)
    torch.cuda.synchronize()
    assert np.array_equal(r.bits_from_device(kv.pool), before)
    kv.close()
