"""GPU: incremental table export (PF_OPT_EXPORT_DELTA) through the upload
kernel.  Over a decode history with copy-on-write forks and copies, frees,
re-created ids and whole-sequence swaps out and back in, the device table,
lengths and newest positions written by pf_export_tables / pf_decode_prepare
must equal pf_block_tables bit for bit after every step -- the same as a whole
export would leave."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", [0, 1])
def test_incremental_export_matches_host_tables(seed):
    print("incremental export seed", seed, flush=True)
    from paged_kv_cache_43_amd import pf
    rng = np.random.default_rng(seed)
    n, mb, B, P = 16, 48, 16, 2048
    st, h = pf.pf_pool_create(P, B, 1, 2, 64, "f16", rng.permutation(P).astype(np.int32))
    pf.check(st)
    nbytes = pf.pf_pool_bytes(h)
    pool = torch.zeros(nbytes // 2, dtype=torch.int16, device="cuda")
    pf.check(pf.pf_pool_bind(h, pool, nbytes))
    pb = pf.pf_page_bytes(h)
    slots = 256
    host = torch.zeros(slots * pb // 2, dtype=torch.int16).pin_memory()
    pf.check(pf.pf_swap_bind(h, host, slots * pb, slots))
    swap_stage = torch.zeros(2 * slots, dtype=torch.int32).pin_memory()
    pf.check(pf.pf_pool_set_option(h, pf.PF_OPT_EXPORT_DELTA, 1))
    ids = np.arange(n, dtype=np.uint64)
    lens = rng.integers(1, 300, size=n).astype(np.int32)
    pf.check(pf.pf_alloc_for_seqs(h, ids, lens)[0])
    staging = torch.zeros(n * mb + 3 * n, dtype=torch.int32).pin_memory()
    meta = torch.full((n * mb + 2 * n,), 777, dtype=torch.int32, device="cuda")
    for step in range(50):
        r = rng.random()
        if r < 0.1:
            s = int(rng.integers(n))
            pf.check(pf.pf_free_seq(h, s))
            lens[s] = int(rng.integers(1, 400))
            pf.check(pf.pf_alloc_for_seq(h, s, int(lens[s]))[0])
        elif r < 0.2:
            p, c = (int(x) for x in rng.choice(n, size=2, replace=False))
            pf.check(pf.pf_free_seq(h, c))
            pf.check(pf.pf_fork_seq(h, p, c))
            lens[c] = lens[p]
        elif r < 0.3:
            sel = np.sort(rng.choice(n, size=3, replace=False)).astype(np.uint64)
            pf.check(pf.pf_swap_out(h, sel, swap_stage, 2 * slots))
            torch.cuda.synchronize()     # the swap staging is rewritten by the swap in
            pf.check(pf.pf_swap_in(h, sel, swap_stage, 2 * slots))
            torch.cuda.synchronize()
        lens = lens + 1
        st, _, copies = pf.pf_grow_seqs(h, ids, lens)
        pf.check(st)
        if len(copies):
            cp = torch.from_numpy(np.ascontiguousarray(copies, dtype=np.int32)).cuda()
            pf.check(pf.pf_copy_pages(h, cp, len(copies)))
        if step % 2:
            pf.check(pf.pf_export_tables(h, ids, mb, staging, meta))
        else:
            pf.check(pf.pf_decode_prepare(h, ids, mb, staging, meta, None, None, 0, 0))
        torch.cuda.synchronize()     # the staging is reused next step
        st, bt, hl = pf.pf_block_tables(h, ids, mb)
        pf.check(st)
        got = meta.cpu().numpy()
        assert np.array_equal(got[:n * mb].reshape(n, mb), bt), "step %d" % step
        assert np.array_equal(got[n * mb:n * mb + n], hl)
        assert np.array_equal(got[n * mb + n:], hl - 1)
    pf.pf_pool_destroy(h)
