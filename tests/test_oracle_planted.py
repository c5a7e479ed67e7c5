"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch each one: a dropped term, a wrong sign or index, a transposed operand,
the wrong free-list order, a read past the context length."""
import math
import types

import numpy as np
import pytest

import oracle.accounting
import oracle.alloc_model
import oracle.attention
import oracle.layout
import pins


def _ns():
    return types.SimpleNamespace(alloc_model=oracle.alloc_model, layout=oracle.layout,
                                 attention=oracle.attention, accounting=oracle.accounting)


def _no_scale(q, K, V, scale):
    return _orig_attention(q, K, V, 1.0)


def _wrong_sign(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(q.shape[0])
    z = -scale * (K @ q)
    w = np.exp(z - z.max())
    return (w @ V) / w.sum()


def _no_normalise(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(q.shape[0])
    z = scale * (K @ q)
    w = np.exp(z - z.max())
    return w @ V


def _transposed(q, K, V, scale):
    # keys and values swapped
    return _orig_attention(q, V, K, scale)


def _default_scale_1_over_d(d):
    return 1.0 / d


def _floor_blocks(length, block_size):
    return length // block_size


def _slot_off_by_one(table, pos, block_size):
    return table[pos // block_size], (pos + 1) % block_size


def _kind_inner(g, page, layer, head, kind, slot, dim):
    # kind and slot nested the other way round: K and V interleaved per token
    return ((((page * g.L + layer) * g.H + head) * g.B + slot) * 2 + kind) * g.D + dim


def _readback_past_length(pool, g, layer, table, length):
    # reads whole blocks, tail slots included
    full = len(table) * g.B if length else 0
    kc, vc = _orig_readback(pool, g, layer, table, full)
    return kc, vc


def _gqa_interleaved(q_bits, pool, g, layer, tables, lengths, dtype, scale=None):
    q = oracle.attention.decode_bits(q_bits, dtype)
    n, hq, d = q.shape
    if scale is None:
        scale = oracle.attention.default_scale(d)
    out = np.zeros((n, hq, d))
    for s in range(n):
        kc, vc = oracle.layout.readback(pool, g, layer, tables[s], int(lengths[s]))
        K = oracle.attention.decode_bits(kc, dtype)
        V = oracle.attention.decode_bits(vc, dtype)
        for h in range(hq):
            out[s, h] = oracle.attention.attention(q[s, h], K[:, h % g.H, :], V[:, h % g.H, :], scale)
    return out


_orig_attention = oracle.attention.attention
_orig_readback = oracle.layout.readback
_orig_swap_copy = oracle.layout.swap_copy


class _FifoModel(oracle.alloc_model.AllocModel):
    def alloc(self, seq_id, new_len):
        if new_len < 0:
            return oracle.alloc_model.INVALID, 0
        table = self.tables.get(seq_id, [])
        if new_len < self.lengths.get(seq_id, 0):
            return oracle.alloc_model.INVALID, 0
        need = oracle.alloc_model.blocks_for(new_len, self.block_size) - len(table)
        if need > len(self.stack):
            return oracle.alloc_model.OOM, 0
        new_pages = [self.stack.pop(0) for _ in range(need)]   # takes from the bottom
        self.tables[seq_id] = table + new_pages
        self.lengths[seq_id] = new_len
        return oracle.alloc_model.OK, need


class _ForwardPushModel(oracle.alloc_model.AllocModel):
    def free(self, seq_id):
        if seq_id not in self.tables:
            return oracle.alloc_model.UNKNOWN_SEQ
        self.stack.extend(self.tables[seq_id])                # last page ends on top
        del self.tables[seq_id]
        del self.lengths[seq_id]
        return oracle.alloc_model.OK


class _LeakyModel(oracle.alloc_model.AllocModel):
    def free(self, seq_id):
        if seq_id not in self.tables:
            return oracle.alloc_model.UNKNOWN_SEQ
        for page in reversed(self.tables[seq_id][1:]):          # drops the first page
            self.stack.append(page)
        del self.tables[seq_id]
        del self.lengths[seq_id]
        return oracle.alloc_model.OK


class _CowKeepsSourceModel(oracle.alloc_model.AllocModel):
    def grow(self, seq_id, new_len):
        cow = self._writes_shared(seq_id, new_len) if seq_id in self.tables else False
        st, nn, copy = super().grow(seq_id, new_len)
        if cow and copy is not None:
            self.refs[copy[0]] += 1                             # the source keeps the writer's hold
        return st, nn, copy


class _FreeIgnoresRefsModel(oracle.alloc_model.AllocModel):
    def free(self, seq_id):
        if seq_id not in self.tables:
            return oracle.alloc_model.UNKNOWN_SEQ
        for page in reversed(self.tables[seq_id]):
            self.refs[page] = max(self.refs[page] - 1, 0)
            if page not in self.stack:
                self.stack.append(page)                         # shared pages freed too early
        del self.tables[seq_id]
        del self.lengths[seq_id]
        return oracle.alloc_model.OK


class _ForkWithoutRefsModel(oracle.alloc_model.AllocModel):
    def fork(self, parent, child):
        if parent not in self.tables:
            return oracle.alloc_model.UNKNOWN_SEQ
        if child in self.tables:
            return oracle.alloc_model.INVALID
        self.tables[child] = list(self.tables[parent])          # counts not raised
        self.lengths[child] = self.lengths[parent]
        return oracle.alloc_model.OK


class _GrowInPlaceModel(oracle.alloc_model.AllocModel):
    def _writes_shared(self, seq_id, new_len):
        return False                                            # never copies


def _copy_nothing(pool, g, pairs):
    return pool.copy()


class _SwapKeepsPagesModel(oracle.alloc_model.AllocModel):
    def _release(self, table):
        if getattr(self, "_in_swap", False):
            return                                              # device pages never released
        super()._release(table)

    def swap_out(self, seq_ids):
        self._in_swap = True
        try:
            return super().swap_out(seq_ids)
        finally:
            self._in_swap = False


class _SwapInKeepsSlotsModel(oracle.alloc_model.AllocModel):
    def swap_in(self, seq_ids):
        before = list(self.slot_stack)
        st, copies = super().swap_in(seq_ids)
        if st == oracle.alloc_model.OK:
            self.slot_stack = before                            # slots never returned
        return st, copies


def _swap_copy_off_by_one_page(pool, host, g, pairs, to_host):
    return _orig_swap_copy(pool, host, g, [(a, b + 1 if b + 1 < g.P else b) for a, b in pairs], to_host)


class _PeakIsCurrentModel(oracle.alloc_model.AllocModel):
    def _note_peak(self):
        self.peak = self.pages_in_use()                         # the current, not the highest


class _ZeroPaddedTablesModel(oracle.alloc_model.AllocModel):
    def block_tables(self, seq_ids, max_blocks):
        rows, lens = super().block_tables(seq_ids, max_blocks)
        return [[0 if p == -1 else p for p in r] for r in rows], lens   # pads with page 0


class _SortedRowsTablesModel(oracle.alloc_model.AllocModel):
    def block_tables(self, seq_ids, max_blocks):
        return super().block_tables(sorted(seq_ids), max_blocks)          # rows by id, not as asked


class _UncheckedWidthTablesModel(oracle.alloc_model.AllocModel):
    def block_tables(self, seq_ids, max_blocks):
        rows, lens = [], []
        for s in seq_ids:                                                 # truncates instead of refusing
            if s in self.offdev:
                raise ValueError("blocks on the host")
            t = self.tables[s][:max_blocks]
            rows.append(t + [-1] * (max_blocks - len(t)))
            lens.append(self.lengths[s])
        return rows, lens


class _BlockOutForwardPushModel(oracle.alloc_model.AllocModel):
    def _move_out(self, seq_id, blocks):
        before = len(self.stack)
        copies = super()._move_out(seq_id, blocks)
        self.stack[before:] = self.stack[before:][::-1]             # pushed first block first: last on top
        return copies


class _BlockInKeepsSlotsModel(oracle.alloc_model.AllocModel):
    def swap_in_blocks(self, seq_id, first, count):
        before = list(self.slot_stack)
        st, copies = super().swap_in_blocks(seq_id, first, count)
        if st == oracle.alloc_model.OK:
            self.slot_stack = before                                # slots never returned
        return st, copies


class _BlockRangeOffByOneModel(oracle.alloc_model.AllocModel):
    def swap_out_blocks(self, seq_id, first, count):
        nb = len(self.table(seq_id)) if seq_id in self.tables or seq_id in self.offdev else 0
        return super().swap_out_blocks(seq_id, first + 1 if first + count < nb else first, count)


class _WholeSwapInWholeOnlyModel(oracle.alloc_model.AllocModel):
    def swap_in(self, seq_ids):
        for s in seq_ids:
            if s in self.offdev and any(p is not None for p in self.offdev[s][0]):
                return oracle.alloc_model.INVALID, []               # refuses a partly swapped sequence
        return super().swap_in(seq_ids)


class _BlockOutPartialOnOomModel(oracle.alloc_model.AllocModel):
    def swap_out_blocks(self, seq_id, first, count):
        st, copies = super().swap_out_blocks(seq_id, first, count)
        if st == oracle.alloc_model.OOM and self.slot_stack:
            return super().swap_out_blocks(seq_id, first, len(self.slot_stack))   # moves what fits
        return st, copies


class _EmptySwapStaysResidentModel(oracle.alloc_model.AllocModel):
    def swap_out(self, seq_ids):
        st, copies = super().swap_out(seq_ids)
        if st == oracle.alloc_model.OK:
            for s in seq_ids:
                if s in self.offdev and not self.offdev[s][0]:
                    del self.offdev[s]
                    self.tables[s] = []                     # nothing to move: left resident
        return st, copies


MUTANTS = {
    "attention_without_scale": (oracle.attention, "attention", _no_scale),
    "attention_wrong_sign": (oracle.attention, "attention", _wrong_sign),
    "attention_not_normalised": (oracle.attention, "attention", _no_normalise),
    "attention_keys_values_swapped": (oracle.attention, "attention", _transposed),
    "default_scale_1_over_d": (oracle.attention, "default_scale", _default_scale_1_over_d),
    "gqa_interleaved_heads": (oracle.attention, "paged_decode_attention", _gqa_interleaved),
    "blocks_floor_not_ceil": (oracle.alloc_model, "blocks_for", _floor_blocks),
    "slot_off_by_one": (oracle.layout, "token_location", _slot_off_by_one),
    "kv_interleaved_per_token": (oracle.layout, "elem_offset", _kind_inner),
    "readback_past_length": (oracle.layout, "readback", _readback_past_length),
    "fifo_free_list": (oracle.alloc_model, "AllocModel", _FifoModel),
    "free_pushes_forward": (oracle.alloc_model, "AllocModel", _ForwardPushModel),
    "free_leaks_a_page": (oracle.alloc_model, "AllocModel", _LeakyModel),
    "cow_source_keeps_hold": (oracle.alloc_model, "AllocModel", _CowKeepsSourceModel),
    "free_ignores_refcounts": (oracle.alloc_model, "AllocModel", _FreeIgnoresRefsModel),
    "fork_without_refcounts": (oracle.alloc_model, "AllocModel", _ForkWithoutRefsModel),
    "grow_writes_shared_page": (oracle.alloc_model, "AllocModel", _GrowInPlaceModel),
    "copy_pages_copies_nothing": (oracle.layout, "copy_pages", _copy_nothing),
    "swap_out_keeps_device_pages": (oracle.alloc_model, "AllocModel", _SwapKeepsPagesModel),
    "swap_in_keeps_slots": (oracle.alloc_model, "AllocModel", _SwapInKeepsSlotsModel),
    "swap_copy_wrong_page": (oracle.layout, "swap_copy", _swap_copy_off_by_one_page),
    "peak_is_current_use": (oracle.alloc_model, "AllocModel", _PeakIsCurrentModel),
    "tables_pad_with_zero": (oracle.alloc_model, "AllocModel", _ZeroPaddedTablesModel),
    "tables_rows_sorted_by_id": (oracle.alloc_model, "AllocModel", _SortedRowsTablesModel),
    "tables_truncate_long_rows": (oracle.alloc_model, "AllocModel", _UncheckedWidthTablesModel),
    "block_swap_out_pushes_forward": (oracle.alloc_model, "AllocModel", _BlockOutForwardPushModel),
    "block_swap_in_keeps_slots": (oracle.alloc_model, "AllocModel", _BlockInKeepsSlotsModel),
    "block_swap_range_off_by_one": (oracle.alloc_model, "AllocModel", _BlockRangeOffByOneModel),
    "whole_swap_in_refuses_partial": (oracle.alloc_model, "AllocModel", _WholeSwapInWholeOnlyModel),
    "block_swap_out_partial_on_oom": (oracle.alloc_model, "AllocModel", _BlockOutPartialOnOomModel),
    "empty_swap_stays_resident": (oracle.alloc_model, "AllocModel", _EmptySwapStaysResidentModel),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    module, attr, replacement = MUTANTS[name]
    monkeypatch.setattr(module, attr, replacement)
    if module is oracle.alloc_model and attr == "blocks_for":
        monkeypatch.setattr(oracle.accounting, "blocks_for", replacement)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(_ns())
        except (AssertionError, IndexError, ValueError, OverflowError, ZeroDivisionError):
            caught.append(pin.__name__)
    assert caught, "no pin catches the planted mistake " + name
