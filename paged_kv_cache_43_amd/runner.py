"""Drive libpf for a workload: device pool, allocator handle, table export,
scatter and attention.  PyTorch supplies device memory, host staging and the
stream; every step of the method runs in libpf (``pf``).
"""
import numpy as np
import torch

from . import inputs
from . import pf

_BITS_TORCH = {"f32": torch.int32, "f16": torch.int16, "bf16": torch.int16}
_BITS_NP = {"f32": np.int32, "f16": np.int16, "bf16": np.int16}


def bits_to_device(bits, device="cuda"):
    """Upload raw bit patterns (uint16/uint32 numpy) without any conversion."""
    signed = bits.view(np.int32 if bits.dtype == np.uint32 else np.int16)
    return torch.from_numpy(np.ascontiguousarray(signed)).to(device)


def _signed_bits(bits, dtype):
    """A raw bit pattern as the signed integer torch stores for it."""
    return int(np.array(bits, dtype=np.uint32 if inputs.DTYPE_BYTES[dtype] == 4 else np.uint16)
               .view(_BITS_NP[dtype]))


def bits_from_device(t):
    a = t.cpu().numpy()
    return a.view(np.uint32 if a.dtype == np.int32 else np.uint16)


class StagingRing:
    """Pinned staging buffers for the per-step table upload, so the host can
    fill step t+1's tables while the device still runs step t.  A buffer is
    refilled only after the upload that read it has run.  That is learnt from
    stream markers (pf_marker_*), but not one per upload: on MI355X any marker
    between two kernels costs ~4.5 us of stream time, so one marker follows
    every GROUP-th upload, and before slot i is refilled the host waits for the
    first marker recorded after slot i's previous upload (SLOTS > GROUP keeps
    that marker in the past)."""

    SLOTS = 16
    GROUP = 8

    def __init__(self, words, gpu, pin=None):
        import torch
        self.gpu = gpu
        pin = gpu if pin is None else pin
        self.bufs = []
        for _ in range(self.SLOTS):
            t = torch.empty(max(words, 1), dtype=torch.int32)
            self.bufs.append(t.pin_memory() if pin else t)
        # marker j covers uploads up to the last of its group; a marker object
        # is re-recorded only after every wait on its previous group
        self.markers = [pf.Marker() for _ in range(self.SLOTS // self.GROUP + 1)] if gpu else []
        self.count = 0   # uploads enqueued so far

    def acquire(self):
        """The buffer for the next upload, free to overwrite."""
        k = self.count
        if self.gpu and k >= self.SLOTS:
            prev = k - self.SLOTS                   # the upload that last used this slot
            covering = prev | (self.GROUP - 1)      # the marker recorded after it (< k)
            self.markers[(covering // self.GROUP) % len(self.markers)].wait()
        return self.bufs[k % self.SLOTS]

    def enqueued(self, stream=None):
        """Call right after the upload that read acquire()'s buffer was enqueued."""
        k = self.count
        if self.gpu and k % self.GROUP == self.GROUP - 1:
            self.markers[(k // self.GROUP) % len(self.markers)].record(stream)
        self.count = k + 1


class PagedKV:
    """A pool handle bound to a torch-allocated device pool, plus device tables."""

    def __init__(self, w, device="cuda", sentinel=True, extra_tokens=0, max_blocks=None, delta_export=True):
        self.w = w
        self.device = device
        st, self.h = pf.pf_pool_create(w.num_pages, w.block, w.layers, w.hkv, w.d, w.dtype,
                                       w.free_order)
        pf.check(st, "pf_pool_create")
        nbytes = pf.pf_pool_bytes(self.h)
        self.pool = torch.empty(nbytes // inputs.DTYPE_BYTES[w.dtype], dtype=_BITS_TORCH[w.dtype],
                                device=device)
        if sentinel:
            self.pool.fill_(_signed_bits(inputs.NAN_BITS[w.dtype], w.dtype))
        pf.check(pf.pf_pool_bind(self.h, self.pool, nbytes), "pf_pool_bind")
        self.max_blocks = max_blocks or w.max_blocks(extra_tokens)
        self.ids = np.arange(w.n, dtype=np.uint64)
        # Per-step metadata, packed so one copy moves it: block tables
        # [n][max_blocks], lengths [n], and each sequence's newest position [n].
        nb = w.n * self.max_blocks
        self.meta_elems = nb + 2 * w.n
        self.stage_elems = nb + 3 * w.n
        self.meta = torch.empty(max(self.meta_elems, 1), dtype=torch.int32, device=device)
        self.bt = self.meta[:nb].view(w.n, self.max_blocks)
        self.ctx = self.meta[nb:nb + w.n]
        self.last_pos = self.meta[nb + w.n:nb + 2 * w.n]
        self.ring = StagingRing(self.stage_elems, torch.cuda.is_available())
        # self.meta is written only by the exports below: upload only what changed
        pf.check(pf.pf_pool_set_option(self.h, pf.PF_OPT_EXPORT_DELTA, 1 if delta_export else 0))
        self.ws = None
        self.ws_bytes = 0
        # device addresses of the handle's own buffers, passed as ints on the
        # per-layer path (the binding's tensor checks cost ~0.3 us each)
        self._bt_ptr = self.bt.data_ptr()
        self._ctx_ptr = self.ctx.data_ptr()
        self._ws_ptr = None

    def close(self):
        if self.h is not None:
            pf.pf_pool_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -------------------------------------------------------------- host ops
    def apply(self, ops):
        for op in ops:
            if op[0] == "alloc":
                st, _ = pf.pf_alloc_for_seq(self.h, op[1], op[2])
                pf.check(st, "pf_alloc_for_seq")
            else:
                pf.check(pf.pf_free_seq(self.h, op[1]), "pf_free_seq")

    def export_tables(self):
        """Block tables, lengths and newest positions of sequences 0..n-1 to the
        device (pf_export_tables: pinned staging, one upload kernel on the
        current stream), from the next slot of the staging ring."""
        buf = self.ring.acquire()
        st = pf.pf_export_tables(self.h, self.ids, self.max_blocks, buf, self.meta)
        pf.check(st, "pf_export_tables")
        self.ring.enqueued()

    def decode_prepare(self, k_new, v_new, layer0=0, num_layers=None):
        """Export the tables and scatter every sequence's newest token for
        layers layer0.. (k_new, v_new: device [layers][n][H][D]) in one launch."""
        num_layers = self.w.layers - layer0 if num_layers is None else num_layers
        buf = self.ring.acquire()
        st = pf.pf_decode_prepare(self.h, self.ids, self.max_blocks, buf, self.meta, k_new, v_new,
                                  layer0, num_layers)
        pf.check(st, "pf_decode_prepare")
        self.ring.enqueued()

    # --------------------------------------------------------------- kernels
    def scatter(self, layer, k, v, tok_seq, tok_pos, stream=None):
        st = pf.pf_scatter_kv(self.h, layer, k, v, tok_seq, tok_pos, int(tok_seq.numel()), self.bt,
                              self.w.n, self.max_blocks, stream)
        pf.check(st, "pf_scatter_kv")

    def ensure_workspace(self, max_ctx, hq=None):
        need = pf.pf_attention_workspace_bytes(self.h, self.w.n, hq or self.w.hq, max_ctx)
        if need > self.ws_bytes:
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.device)
            self.ws_bytes = need
            self._ws_ptr = self.ws.data_ptr()
        return need

    def attention(self, layer, q, out, max_ctx, out_dtype=None, scale=0.0, stream=None, hq=None):
        """One layer's decode attention.  The call is made with the workspace
        held so far; the library checks its size before launching anything and
        reports PF_ERR_WORKSPACE, on which the workspace is grown and the call
        made again (no size query on every call)."""
        hq = hq or self.w.hq
        od = out_dtype or self.w.dtype
        st = pf.pf_paged_decode_attention(self.h, layer, q, hq, self._bt_ptr, self.max_blocks, self._ctx_ptr,
                                          self.w.n, max_ctx, scale, out, od, self._ws_ptr, self.ws_bytes, stream)
        if st == pf.PF_ERR_WORKSPACE:
            self.ensure_workspace(max_ctx, hq)
            st = pf.pf_paged_decode_attention(self.h, layer, q, hq, self._bt_ptr, self.max_blocks,
                                              self._ctx_ptr, self.w.n, max_ctx, scale, out, od, self._ws_ptr,
                                              self.ws_bytes, stream)
        pf.check(st, "pf_paged_decode_attention")

    def attention_append(self, layer, q, k_new, v_new, out, max_ctx, out_dtype=None, scale=0.0, stream=None,
                         hq=None):
        """Fused form: each sequence's newest token (position ctx-1), K/V
        ``k_new`` / ``v_new`` [n][H][D], written and attended in one launch."""
        hq = hq or self.w.hq
        self.ensure_workspace(max_ctx, hq)
        st = pf.pf_paged_decode_attention_append(self.h, layer, q, hq, k_new, v_new, self.bt, self.max_blocks,
                                                 self.ctx, self.w.n, max_ctx, scale, out,
                                                 out_dtype or self.w.dtype, self.ws, self.ws_bytes, stream)
        pf.check(st, "pf_paged_decode_attention_append")

    def contiguous_attention(self, k, v, q, out, max_ctx, out_dtype=None, scale=0.0, stream=None, hq=None):
        """pf_contiguous_decode_attention over k, v viewed as [n][max_len][H][D]
        (any strides with the last dimension dense: the gather output, or a
        [n][H][max_len][D] buffer permuted to that view), with this pool's
        geometry, options and lengths."""
        hq = hq or self.w.hq
        assert k.shape == v.shape and k.stride() == v.stride() and k.stride(3) == 1
        self.ensure_workspace(max_ctx, hq)
        st = pf.pf_contiguous_decode_attention(self.h, q, hq, k, v, k.stride(0), k.stride(1), k.stride(2),
                                               k.shape[1], self.ctx, self.w.n, max_ctx, scale, out,
                                               out_dtype or self.w.dtype, self.ws, self.ws_bytes, stream)
        pf.check(st, "pf_contiguous_decode_attention")

    def gather(self, layer, max_len, stream=None, fill=None):
        """Read-back into [n][max_len][H][D]; positions past a length keep
        ``fill`` (raw bits) if given, else whatever the buffer held."""
        w = self.w
        if fill is None:
            k = torch.empty((w.n, max_len, w.hkv, w.d), dtype=_BITS_TORCH[w.dtype], device=self.device)
        else:
            k = torch.full((w.n, max_len, w.hkv, w.d), _signed_bits(fill, w.dtype), dtype=_BITS_TORCH[w.dtype],
                           device=self.device)
        v = torch.empty_like(k) if fill is None else k.clone()
        st = pf.pf_gather_kv(self.h, layer, self.bt, self.ctx, w.n, self.max_blocks, max_len, k, v,
                             stream)
        pf.check(st, "pf_gather_kv")
        return k, v


def token_arrays(w, positions):
    """Flattened (tok_seq, tok_pos) for ``positions[s]`` = iterable of positions."""
    seq, pos = [], []
    for s, ps in enumerate(positions):
        for p in ps:
            seq.append(s)
            pos.append(p)
    return np.array(seq, dtype=np.int32), np.array(pos, dtype=np.int32)


def fill_workload(kv, device="cuda"):
    """Replay the workload's history and measured-step allocations, export the
    tables and scatter every context token's K/V of every layer.  Returns the
    device q [L][n][Hq][D] bits."""
    w = kv.w
    kv.apply(w.history_ops + w.step_ops)
    kv.export_tables()
    ks, vs, q = w.values()
    tok_seq, tok_pos = token_arrays(w, [range(int(c)) for c in w.ctx])
    ts = torch.from_numpy(tok_seq).to(device)
    tp = torch.from_numpy(tok_pos).to(device)
    for layer in range(w.layers):
        k = np.concatenate([ks[s][layer] for s in range(w.n)]) if w.n else None
        v = np.concatenate([vs[s][layer] for s in range(w.n)]) if w.n else None
        if len(tok_seq):
            kv.scatter(layer, bits_to_device(k, device), bits_to_device(v, device), ts, tp)
    return bits_to_device(q, device)
