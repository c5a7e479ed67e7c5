"""Memory accounting closed forms (test infrastructure only).

Follows PageFault, "Calculate" (core formulas): KV bytes per token of a model,
naive reservation (every sequence holds the maximum length), paged reservation
(whole blocks actually mapped), utilization (stored over reserved tokens) and
internal fragmentation (the unused tail of each sequence's last block).  These
pin the allocator model's block counts against the figures the pages print.
"""
from .alloc_model import blocks_for


def bytes_per_token(num_layers, num_kv_heads, head_dim, elem_bytes):
    """K and V of one token across all layers and kv heads."""
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes


def naive_reserved_bytes(num_seqs, max_seq_len, bpt):
    return num_seqs * max_seq_len * bpt


def blocks_used(lengths, block_size):
    return sum(blocks_for(n, block_size) for n in lengths)


def paged_reserved_bytes(lengths, block_size, bpt):
    return blocks_used(lengths, block_size) * block_size * bpt


def internal_fragmentation_tokens(lengths, block_size):
    return sum(blocks_for(n, block_size) * block_size - n for n in lengths)


def utilization(lengths, reserved_tokens):
    return sum(lengths) / reserved_tokens
