"""Paged KV-cache hot path for MI355X (gfx950): paged decode and chunked-prefill attention,
KV append through a slot mapping, and copy-on-write block copies, behind a C-ABI library.

The device entry points live in ``libpagedattn.so`` (hand-written HIP) and are reached through
the ctypes binding in ``paged_kv_cache_341_amd.ops``; importing the package does not load it.
"""
from .block_manager import BlockManager, OutOfBlocks, blocks_for, tail_waste  # noqa: F401

__all__ = ["BlockManager", "OutOfBlocks", "blocks_for", "tail_waste"]
