"""GPU: the contiguous-cache twin.  pf_contiguous_decode_attention runs the
kernels of pf_paged_decode_attention with each 16-token block addressed in a
per-sequence cache instead of through the block table (PageFault, "Four
stages": the paged kernel of stage 3 is checked against the contiguous kernel
of stage 1).  For the same values, lengths and handle options it must return
the paged entry point's output bit for bit, in every cache layout, and match
the oracle within the attention tolerance."""
import numpy as np
import pytest

import gpu_util as gu
from paged_kv_cache_43_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SCHED_GRID, SCHED_BALANCED = 1, 2


def _out(w, od):
    dt = torch.float32 if od == "f32" else (torch.int32 if w.dtype == "f32" else torch.int16)
    return torch.empty((w.n, w.hq, w.d), dtype=dt, device="cuda")


def _layouts(k, v, w, max_len):
    """The gathered [n][max_len][H][D] cache in three layouts, each viewed as
    [n][t][h][d]: token-major as gathered, head-major [n][H][max_len][D], and
    token-major with every (token, head) row padded by 8 elements."""
    yield "token", k, v
    kh = k.permute(0, 2, 1, 3).contiguous()
    vh = v.permute(0, 2, 1, 3).contiguous()
    yield "head", kh.permute(0, 2, 1, 3), vh.permute(0, 2, 1, 3)
    kp = torch.zeros((w.n, max_len, w.hkv, w.d + 8), dtype=k.dtype, device=k.device)
    vp = torch.zeros_like(kp)
    kp[..., :w.d] = k
    vp[..., :w.d] = v
    yield "padded", kp[..., :w.d], vp[..., :w.d]


def _check_twin(w, kv, q, layer, od, max_len):
    """Paged output vs the twin in every layout (bitwise) and vs the oracle."""
    mc = int(w.ctx.max()) if w.n else 0
    k, v = kv.gather(layer, max_len, fill=inputs.NAN_BITS[w.dtype])   # tails hold NaN
    ref_out = _out(w, od)
    kv.attention(layer, q[layer], ref_out, mc, out_dtype=od)
    torch.cuda.synchronize()
    for name, kk, vv in _layouts(k, v, w, max_len):
        got = _out(w, od)
        got.fill_(-1)
        kv.contiguous_attention(kk, vv, q[layer], got, mc, out_dtype=od)
        torch.cuda.synchronize()
        assert torch.equal(got, ref_out), "%s layer %d: contiguous (%s) != paged" % (w.name, layer, name)
    res = gu.out_to_f64(ref_out, od if w.dtype != "f32" else "f32")
    ref = gu.oracle_attention_contiguous(w, layer)
    return gu.assert_close(res, ref, od if w.dtype != "f32" else "f32", "%s layer %d" % (w.name, layer))


@pytest.mark.parametrize("sched", [SCHED_GRID, SCHED_BALANCED])
@pytest.mark.parametrize("name", ["tiny", "mixed", "gpt2"])
def test_twin_small_configs(name, sched):
    print("twin", name, sched, flush=True)
    from paged_kv_cache_43_amd import pf, runner
    w = inputs.Workload(name, frames="shuffled")
    kv = runner.PagedKV(w)
    q = runner.fill_workload(kv)
    pf.check(pf.pf_pool_set_option(kv.h, pf.PF_OPT_SCHEDULE, sched))
    max_len = kv.max_blocks * 16
    for layer in sorted({0, w.layers - 1}):
        for od in ("f32", w.dtype):
            _check_twin(w, kv, q, layer, od, max_len)
    kv.close()


@pytest.mark.parametrize("name", ["13b", "gqa", "13b_32k", "gqa_32k"])
def test_twin_full_size(name):
    """The bench's configurations at full size and default options (the
    launch configuration it times)."""
    print("twin full", name, flush=True)
    from paged_kv_cache_43_amd import runner
    w = inputs.Workload(name, frames="shuffled")
    kv = runner.PagedKV(w)
    q = runner.fill_workload(kv)
    err = _check_twin(w, kv, q, 0, w.dtype, -(-int(w.ctx.max()) // 16) * 16)
    print("  max err", err, flush=True)
    kv.close()


def _custom(lens, hq, hkv, d, dtype, seed):
    w = inputs.Workload("tiny", seed=seed, frames="shuffled", lens=lens)
    w.hq, w.hkv, w.d, w.dtype, w.es = hq, hkv, d, dtype, inputs.DTYPE_BYTES[dtype]
    need = sum(-(-int(c) // 16) for c in lens)
    w.num_pages = max(need + 8, 16)
    w.free_order = np.random.default_rng(seed + 99).permutation(w.num_pages)
    return w


@pytest.mark.parametrize("sched", [SCHED_GRID, SCHED_BALANCED])
@pytest.mark.parametrize("dtype,d,hq,hkv", [("f32", 16, 2, 2), ("f16", 32, 3, 3), ("f16", 128, 4, 2),
                                            ("bf16", 64, 14, 2), ("bf16", 256, 2, 1), ("f32", 256, 4, 2)])
def test_twin_shapes_and_edge_lengths(dtype, d, hq, hkv, sched):
    """Every kernel family (vector and matrix-core), edge lengths including 0,
    1 and block boundaries, and a cache longer than any sequence."""
    print("twin shape", dtype, d, hq, hkv, sched, flush=True)
    from paged_kv_cache_43_amd import pf, runner
    w = _custom([0, 1, 15, 16, 17, 33, 200, 513], hq, hkv, d, dtype, seed=d + hq)
    kv = runner.PagedKV(w)
    q = runner.fill_workload(kv)
    pf.check(pf.pf_pool_set_option(kv.h, pf.PF_OPT_SCHEDULE, sched))
    _check_twin(w, kv, q, 0, "f32", kv.max_blocks * 16 + 32)
    kv.close()
