"""Rolling sink + window K/V cache, simulated chunk by chunk (oracle side).

TEST INFRASTRUCTURE (see the package docstring).

Page "flashdreams.accelerated", section "Generic Multi Head Attention Interface": streaming
self-attention keeps a BlockKVCache whose K/V storage is [B, sink_size + window_size, H, d];
the caller brackets each chunk with before_update(chunk_idx) / after_update(chunk_idx), and the
current chunk writes its K/V into the rolling cache *before* it is queried. The API-summary page
("Accelerated building blocks", section "Cache lifecycle") adds that chunk, window and sink sizes
are fixed.

The pages do not spell out the slot arithmetic. The reading simulated here:
  * sizes are in tokens and are whole multiples of the chunk length Lc;
  * the first sink_size / Lc chunks are sinks: each keeps its own slot for ever;
  * every later chunk enters the window, a FIFO of at most window_size / Lc chunks: while the
    window has room a chunk takes the next free slot, afterwards it overwrites the slot of the
    oldest window chunk (that chunk is evicted);
  * after chunk c has been written, the visible keys are the sinks followed by the window
    chunks, in the order the chunks arrived (chunk c included).

This module simulates that policy with explicit slot bookkeeping (a list of occupants and a FIFO);
it does not use a closed-form slot formula.
"""
from __future__ import annotations

from collections import deque


class RollingCacheModel:
    def __init__(self, chunk_len: int, sink_size: int, window_size: int):
        if chunk_len <= 0 or sink_size < 0 or window_size <= 0:
            raise ValueError("chunk_len and window_size must be positive, sink_size >= 0")
        if sink_size % chunk_len or window_size % chunk_len:
            raise ValueError("sink_size and window_size must be multiples of chunk_len")
        self.chunk_len = chunk_len
        self.n_sink = sink_size // chunk_len
        self.n_win = window_size // chunk_len
        self.occupant = [None] * (self.n_sink + self.n_win)  # chunk id held by each chunk slot
        self.sinks: list[int] = []
        self.window: deque[int] = deque()
        self.next_chunk = 0

    def write(self, chunk_idx: int) -> int:
        """Place chunk ``chunk_idx`` (must be the next one) and return its first token slot."""
        if chunk_idx != self.next_chunk:
            raise ValueError("chunks must arrive in order 0, 1, 2, ...")
        self.next_chunk += 1
        if len(self.sinks) < self.n_sink:
            slot = len(self.sinks)
            self.sinks.append(chunk_idx)
        elif len(self.window) < self.n_win:
            free = [s for s in range(self.n_sink, self.n_sink + self.n_win) if self.occupant[s] is None]
            slot = free[0]
            self.window.append(chunk_idx)
        else:
            oldest = self.window.popleft()
            slot = self.occupant.index(oldest)
            self.window.append(chunk_idx)
        self.occupant[slot] = chunk_idx
        return slot * self.chunk_len

    def visible_chunks(self) -> list[int]:
        """Chunk ids visible to the current query chunk, in arrival order."""
        return list(self.sinks) + list(self.window)

    def visible_len(self) -> int:
        return self.chunk_len * (len(self.sinks) + len(self.window))

    def slot_of(self, chunk_idx: int) -> int:
        return self.occupant.index(chunk_idx) * self.chunk_len
