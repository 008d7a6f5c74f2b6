"""Placing and reading rows of the paged KV cache (the layout documented in
include/specverify.h) with plain torch indexing. For callers that fill a cache from elsewhere
(a prompt processed by another engine, test fixtures) or inspect one; the verify pass itself
never goes through here."""
from __future__ import annotations

import torch

from . import PAGE_SIZE, PagedKV


def _pages_slots(kv: PagedKV, b: int, positions: torch.Tensor):
    positions = positions.to(kv.block_table.device, torch.long)
    pages = kv.block_table[b].long()[positions // PAGE_SIZE]
    return pages, positions % PAGE_SIZE


def write_rows(kv: PagedKV, layer: int, b: int, positions: torch.Tensor, k: torch.Tensor,
               v: torch.Tensor) -> None:
    """k, v: [n][n_kv][d] rows for the given positions of request b."""
    pages, slots = _pages_slots(kv, b, positions)
    kv.k_pool[layer][pages, :, slots, :] = k.to(kv.k_pool.device, kv.k_pool.dtype)
    kv.v_pool[layer][pages, :, :, slots] = v.to(kv.v_pool.device, kv.v_pool.dtype)


def read_rows(kv: PagedKV, layer: int, b: int, positions: torch.Tensor):
    """Returns (k, v), each [n][n_kv][d], for the given positions of request b."""
    pages, slots = _pages_slots(kv, b, positions)
    return kv.k_pool[layer][pages, :, slots, :], kv.v_pool[layer][pages, :, :, slots]


def write_context(kv: PagedKV, layer: int, b: int, k: torch.Tensor, v: torch.Tensor) -> None:
    """Positions 0..len(k)-1 of request b."""
    write_rows(kv, layer, b, torch.arange(k.shape[0]), k, v)
