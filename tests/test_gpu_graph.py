"""GPU: the attention entry point inside a HIP graph.  Every layer's
pf_paged_decode_attention of a decode step is captured once, with a bound on
the context lengths that covers the steps to come; each later step grows the
sequences, uploads the tables and scatters the new tokens eagerly, then
replays the graph.  Every replay must equal an eager call with the same bound,
bit for bit, and follow the changing lengths."""
import numpy as np
import pytest

from paged_kv_cache_43_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,steps", [("gpt2", 6), ("mixed", 6), ("gqa", 4)])
def test_attention_replays_in_a_graph(name, steps):
    from paged_kv_cache_43_amd import pf, runner
    print("graph", name, flush=True)
    w = inputs.Workload(name, frames="shuffled")
    kv = runner.PagedKV(w, extra_tokens=steps)
    q = runner.fill_workload(kv)
    bound = int(w.ctx.max()) + steps
    kv.ensure_workspace(bound)
    outs = [torch.empty((w.n, w.hq, w.d), dtype=torch.float32, device="cuda") for _ in range(w.layers)]
    # eager warm-up on a side stream (device queries cached before capture)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for layer in range(w.layers):
            kv.attention(layer, q[layer], outs[layer], bound, out_dtype="f32")
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for layer in range(w.layers):
            kv.attention(layer, q[layer], outs[layer], bound, out_dtype="f32")
    rng = np.random.default_rng(5)
    ids = np.arange(w.n, dtype=np.uint64)
    prev = None
    for t in range(1, steps + 1):
        st, _ = pf.pf_alloc_for_seqs(kv.h, ids, (w.ctx + t).astype(np.int32))
        pf.check(st, "pf_alloc_for_seqs")
        nk = runner.bits_to_device(inputs.normal_bits(rng, (w.layers, w.n, w.hkv, w.d), w.dtype))
        nv = runner.bits_to_device(inputs.normal_bits(rng, (w.layers, w.n, w.hkv, w.d), w.dtype))
        kv.decode_prepare(nk, nv)
        g.replay()
        eager = [torch.empty_like(o) for o in outs]
        for layer in range(w.layers):
            kv.attention(layer, q[layer], eager[layer], bound, out_dtype="f32")
        torch.cuda.synchronize()
        for layer in range(w.layers):
            assert torch.equal(outs[layer], eager[layer]), (t, layer)
        snap = torch.stack(outs).clone()
        assert prev is None or not torch.equal(snap, prev)      # the replay saw the new step
        prev = snap
    kv.close()
