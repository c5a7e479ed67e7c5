"""Seeded synthetic workloads for decode-step paged attention.

This module only draws inputs: context lengths, the physical frame order of
the pool, allocator churn schedules and N(0,1) query/key/value bit patterns.
It computes nothing of the method itself and imports neither the HIP binding
nor the oracle, so the tests can hand the very same arrays to both.

Shapes follow the workloads on the pages and the ones derived from them:

* ``tiny``   -- 4 sequences, 1 layer, 2 heads, head dim 16, fp32, 64-page pool,
  context uniform 1..64, shuffled frames.
* ``gpt2``   -- GPT-2 124M shape (12 layers x 12 heads, head dim 64, fp16),
  32 sequences, prompts uniform 8..64 then 50 decode steps that grow every
  sequence by one token in turn (PageForge, "Real numbers": decode step 50),
  1024-page pool.
* ``mixed``  -- PageFault's "Stage 2: memory" traffic mix: 50 % U[32,128],
  30 % U[256,512], 20 % U[1024,2048]; 12 heads, head dim 64, fp16,
  4096-page pool.  ``mixed_s7`` is the same mix drawn from seed 7 (PageFault
  reports the mix under seeds 42 and 7; its lengths come from another
  generator, so only the recipe is shared).
* ``13b``    -- a 13B-style layer (PagedAttention blog, opening section:
  40 heads of dimension 128): 64 sequences with context U[256,2048], fp16,
  pool sized to 1.1x the blocks in use.
* ``gqa``    -- grouped-query heads (14 query / 2 kv), head dim 64, bf16,
  256 sequences with context U[1024,4096], 70 000-page pool that went through
  500 alloc/free cycles of 16 sequences first (PageForge, "Allocator stress
  test").
* ``13b_32k`` -- the 13B-style layer at 32k-token contexts: 2 sequences with
  context U[30720,32768], fp16, pool sized to 1.1x the blocks in use.
* ``gqa_32k`` -- the grouped-query shape at 32k-token contexts: 32 sequences
  with context U[30720,32768], bf16, pool sized to 1.1x the blocks in use.
* ``gqa_1m`` -- one sequence of 2^20 tokens in the grouped-query shape: the
  whole grid splits one sequence's context.

Randomness: ``numpy.random.SeedSequence(seed).spawn(4)`` gives independent
PCG64 streams for lengths, frame order, churn and values.  Values are drawn in
float64, rounded to float32 (round to nearest even) and, for the 16-bit types,
rounded once more to nearest even; the stored bit patterns are what both sides
consume.
"""
import math

import numpy as np

BLOCK = 16

DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
# Quiet-NaN patterns used to pre-fill a pool so any read of a never-written
# slot would poison the result.
NAN_BITS = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0}

CONFIGS = {
    "tiny": dict(n=4, layers=1, hq=2, hkv=2, d=16, dtype="f32", pool=64,
                 lens=("uniform", 1, 64), seed=0, churn=None),
    "gpt2": dict(n=32, layers=12, hq=12, hkv=12, d=64, dtype="f16", pool=1024,
                 lens=("prompt_decode", 8, 64, 50), seed=1, churn=None),
    "mixed": dict(n=32, layers=1, hq=12, hkv=12, d=64, dtype="f16", pool=4096,
                  lens=("mix",), seed=42, churn=None),
    "mixed_s7": dict(n=32, layers=1, hq=12, hkv=12, d=64, dtype="f16", pool=4096,
                     lens=("mix",), seed=7, churn=None),
    "13b": dict(n=64, layers=1, hq=40, hkv=40, d=128, dtype="f16", pool="1.1x",
                lens=("uniform", 256, 2048), seed=3, churn=None),
    "gqa": dict(n=256, layers=1, hq=14, hkv=2, d=64, dtype="bf16", pool=70000,
                lens=("uniform", 1024, 4096), seed=4, churn=(500, 16, 4096)),
    "13b_32k": dict(n=2, layers=1, hq=40, hkv=40, d=128, dtype="f16", pool="1.1x",
                    lens=("uniform", 30720, 32768), seed=5, churn=None),
    "gqa_32k": dict(n=32, layers=1, hq=14, hkv=2, d=64, dtype="bf16", pool="1.1x",
                    lens=("uniform", 30720, 32768), seed=6, churn=None),
    "gqa_1m": dict(n=1, layers=1, hq=14, hkv=2, d=64, dtype="bf16", pool="1.1x",
                   lens=("uniform", 1 << 20, 1 << 20), seed=8, churn=None),
}

CHURN_SEQ_BASE = 1 << 40


def streams(seed):
    """Four independent generators: lengths, frames, churn, values."""
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(4)]


def draw_lengths(spec, n, gen):
    """Context lengths at the measured decode step (the new token included)."""
    kind = spec[0]
    if kind == "uniform":
        return gen.integers(spec[1], spec[2] + 1, size=n).astype(np.int64)
    if kind == "prompt_decode":
        prompts = gen.integers(spec[1], spec[2] + 1, size=n).astype(np.int64)
        return prompts + spec[3]
    if kind == "mix":
        cat = gen.choice(3, size=n, p=[0.5, 0.3, 0.2])
        lo = np.array([32, 256, 1024])[cat]
        hi = np.array([128, 512, 2048])[cat]
        return np.array([gen.integers(a, b + 1) for a, b in zip(lo, hi)], dtype=np.int64)
    raise ValueError(kind)


def round_f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def to_bits(x, dtype):
    """Stored bit patterns of float64 values ``x`` in ``dtype``."""
    f = round_f32(x)
    if dtype == "f32":
        return f.view(np.uint32).copy()
    if dtype == "f16":
        return f.astype(np.float16).view(np.uint16).copy()
    if dtype == "bf16":
        u = f.view(np.uint32).astype(np.uint64)
        r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        return r.astype(np.uint16)
    raise ValueError(dtype)


# Values drawn per chunk by normal_bits (float64 scratch of this many).
NORMAL_CHUNK = 1 << 22


def normal_bits(gen, shape, dtype):
    """N(0,1) draws of ``shape`` as ``dtype`` bit patterns.  The draws go in
    chunks through one reused float64 buffer: the generator produces the same
    sequence as a single call of the full size, without a full-size float64
    array (long contexts hold billions of values)."""
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.uint32 if dtype == "f32" else np.uint16)
    buf = np.empty(max(min(n, NORMAL_CHUNK), 0))
    for a in range(0, n, NORMAL_CHUNK):
        x = buf[: min(n - a, NORMAL_CHUNK)]
        gen.standard_normal(out=x)
        out[a:a + len(x)] = to_bits(x, dtype)
    return out.reshape(shape)


def churn_ops(gen, cycles, seqs_per_cycle, max_len):
    """Alloc/free op log: each cycle grows ``seqs_per_cycle`` sequences to a
    length U[1, max_len] in 1-4 increments, interleaved, then frees them in a
    random order."""
    ops = []
    sid = CHURN_SEQ_BASE
    for _ in range(cycles):
        ids = list(range(sid, sid + seqs_per_cycle))
        sid += seqs_per_cycle
        targets = gen.integers(1, max_len + 1, size=seqs_per_cycle)
        steps = gen.integers(1, 5, size=seqs_per_cycle)
        plans = []
        for t, k in zip(targets, steps):
            cuts = np.sort(gen.choice(np.arange(1, t + 1), size=min(int(k), int(t)), replace=False))
            cuts[-1] = t
            plans.append([int(c) for c in cuts])
        rounds = max(len(p) for p in plans)
        for r in range(rounds):
            for s, p in zip(ids, plans):
                if r < len(p):
                    ops.append(("alloc", s, p[r]))
        for j in gen.permutation(seqs_per_cycle):
            ops.append(("free", ids[int(j)]))
    return ops


class Workload:
    """One seeded instance of a configuration.

    Attributes: geometry (``n, layers, hq, hkv, d, dtype, block``), ``ctx``
    (context length of each sequence at the measured step), ``num_pages``,
    ``free_order`` (initial free-list order, pops first at index 0),
    ``history_ops`` (alloc/free ops that bring the pool to the state just
    before the measured step, churn included) and ``step_ops`` (the measured
    step's allocations).  Sequence ids of the workload are 0..n-1.
    """

    def __init__(self, name, seed=None, frames="shuffled", n=None, lens=None, block=BLOCK):
        cfg = dict(CONFIGS[name])
        self.name = name
        self.seed = cfg["seed"] if seed is None else seed
        self.frames = frames
        g_len, g_frame, g_churn, _ = streams(self.seed)
        self.n = cfg["n"] if n is None else n
        self.layers, self.hq, self.hkv, self.d = cfg["layers"], cfg["hq"], cfg["hkv"], cfg["d"]
        self.dtype = cfg["dtype"]
        self.es = DTYPE_BYTES[self.dtype]
        self.block = int(block)
        spec = cfg["lens"]
        if lens is not None:
            self.ctx = np.asarray(lens, dtype=np.int64)
            self.n = len(self.ctx)
        else:
            self.ctx = draw_lengths(spec, self.n, g_len)
        if cfg["pool"] == "1.1x":
            used = int(sum(-(-int(c) // self.block) for c in self.ctx))
            self.num_pages = int(math.ceil(1.1 * used))
        else:
            # the same token capacity in pages of this block size
            self.num_pages = -(-int(cfg["pool"]) * BLOCK // self.block)
        if frames == "ordered":
            self.free_order = np.arange(self.num_pages, dtype=np.int64)
        elif frames == "shuffled":
            self.free_order = g_frame.permutation(self.num_pages).astype(np.int64)
        else:
            raise ValueError(frames)
        ops = []
        if cfg["churn"] is not None:
            cyc, per, mx = cfg["churn"]
            ops += churn_ops(g_churn, cyc, per, mx)
        if spec[0] == "prompt_decode" and lens is None:
            decode = spec[3]
            prompt = self.ctx - decode
            ops += [("alloc", s, int(prompt[s])) for s in range(self.n)]
            for k in range(1, decode):
                ops += [("alloc", s, int(prompt[s]) + k) for s in range(self.n)]
        else:
            ops += [("alloc", s, max(int(self.ctx[s]) - 1, 0)) for s in range(self.n)]
        self.history_ops = ops
        self.step_ops = [("alloc", s, int(self.ctx[s])) for s in range(self.n)]
        self._values = None

    def max_blocks(self, extra_tokens=0):
        return int(-(-(int(self.ctx.max()) + extra_tokens) // self.block)) if self.n else 1

    def share_values(self, other):
        """Take ``other``'s drawn K/V/q instead of drawing them again.  Values
        come from their own generator stream, so two workloads of the same
        configuration and seed that differ only in frame order (or page size)
        draw identical values; this checks that the shapes and lengths agree."""
        same = (self.seed == other.seed and self.n == other.n and self.layers == other.layers and
                self.hq == other.hq and self.hkv == other.hkv and self.d == other.d and
                self.dtype == other.dtype and np.array_equal(self.ctx, other.ctx))
        if not same:
            raise ValueError("share_values: workloads differ in seed, geometry or lengths")
        self._values = other.values()
        return self

    def drop_values(self):
        """Forget the drawn values (they are drawn again on the next use)."""
        self._values = None

    def values(self):
        """K/V bits per sequence ``[L][ctx_s][Hkv][D]`` and q bits ``[L][n][Hq][D]``."""
        if self._values is None:
            g = streams(self.seed)[3]   # a fresh values stream: a redraw gives the same values
            ks, vs = [], []
            for s in range(self.n):
                shape = (self.layers, int(self.ctx[s]), self.hkv, self.d)
                ks.append(normal_bits(g, shape, self.dtype))
                vs.append(normal_bits(g, shape, self.dtype))
            q = normal_bits(g, (self.layers, self.n, self.hq, self.d), self.dtype)
            self._values = (ks, vs, q)
        return self._values
