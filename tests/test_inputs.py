"""The seeded input generators (no arithmetic of the method): chunked normal
draws equal one full-size draw, value sharing between frame orders, and the
32k-token-context workloads' shapes."""
import numpy as np
import pytest

from paged_kv_cache_43_amd import inputs


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", [(0, 3), (5,), (3, 7, 11), (7, 333, 3)])
def test_chunked_draws_equal_one_draw(dtype, shape, monkeypatch):
    # chunk sizes that split the draw unevenly, evenly, and not at all
    for chunk in (1000, 7, 1 << 22):
        monkeypatch.setattr(inputs, "NORMAL_CHUNK", chunk)
        g1, g2 = np.random.default_rng(11), np.random.default_rng(11)
        got = inputs.normal_bits(g1, shape, dtype)
        want = inputs.to_bits(g2.standard_normal(size=shape), dtype)
        assert got.shape == want.shape and got.dtype == want.dtype
        assert np.array_equal(got, want)
        # the generator is left at the same point of its stream
        assert g1.standard_normal() == g2.standard_normal()


def test_share_values_across_frame_orders():
    a = inputs.Workload("mixed", frames="ordered")
    b = inputs.Workload("mixed", frames="shuffled")
    fresh = inputs.Workload("mixed", frames="shuffled").values()
    b.share_values(a)
    for x, y in zip(b.values()[0] + b.values()[1] + [b.values()[2]],
                    fresh[0] + fresh[1] + [fresh[2]]):
        assert np.array_equal(x, y)
    with pytest.raises(ValueError):
        inputs.Workload("gpt2").share_values(a)


@pytest.mark.parametrize("name,n", [("13b_32k", 2), ("gqa_32k", 32)])
def test_32k_context_workloads(name, n):
    w = inputs.Workload(name)
    assert w.n == n and w.ctx.min() >= 30720 and w.ctx.max() <= 32768
    used = int(sum(-(-int(c) // 16) for c in w.ctx))
    assert w.num_pages == int(np.ceil(1.1 * used))
    assert sorted(w.free_order.tolist()) == list(range(w.num_pages))
    assert len(w.step_ops) == n and w.max_blocks() <= 2048


def test_dropped_values_redraw_identically():
    w = inputs.Workload("tiny")
    ks, vs, q = w.values()
    ks, vs, q = [a.copy() for a in ks], [a.copy() for a in vs], q.copy()
    w.drop_values()
    ks2, vs2, q2 = w.values()
    assert all(np.array_equal(a, b) for a, b in zip(ks + vs + [q], ks2 + vs2 + [q2]))
