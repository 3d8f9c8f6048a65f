"""Oracle: frame-sink + sliding local window cache model (exact integer logic).

Test infrastructure only (see ``oracle/__init__``).

Sources:
* LongLive paper review, section 3 "Frame Sink": the KV of the initial
  frames is kept as a global anchor for the whole stream, next to a short
  local attention window (9 local + 3 sink frames, 12 in all; the same
  split appears in the section 6 implementation table).
* LongLive paper review, section 3 "Short-Window Attention": attention
  covers only the window of recent latent frames.

Readings taken:
* Sinks are frames 0 .. n_sink-1, never evicted.
* The local window holds the n_local most recently appended non-sink frames;
  appending frame f >= n_sink evicts frame f - n_local when that frame is a
  non-sink frame that is still resident.
* Slots: sink frame f sits in sink slot f; non-sink frame f in ring slot
  (f - n_sink) mod n_local.  Logical order is sinks, then local frames
  oldest to newest (frame number increasing).
* Append happens before attend: a frame's own KV is in the window when its
  queries attend.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Tuple


@dataclass(frozen=True)
class SlotEntry:
    frame: int
    t: int
    segment: int   # 0 sink, 1 ring
    slot: int      # index inside its segment


def resident_frames(n_appended: int, n_sink: int, n_local: int) -> List[int]:
    """Frames resident after frames 0..n_appended-1 were appended, in logical order."""
    sinks = list(range(min(n_sink, n_appended)))
    local = list(range(max(n_sink, n_appended - n_local), n_appended))
    return sinks + local


def slot_of(frame: int, n_sink: int, n_local: int) -> Tuple[int, int]:
    """(segment, slot) of a frame: sink slot f, else ring slot (f - n_sink) mod n_local."""
    if frame < n_sink:
        return 0, frame
    return 1, (frame - n_sink) % n_local


class CacheModel:
    """Frame-granular cache with pinned sinks and a ring of local frames.

    Holds, for every resident frame, the stored (rotated) K and V arrays
    handed to ``append``; the arithmetic that produced them lives elsewhere.
    """

    def __init__(self, n_sink: int, n_local: int):
        if n_sink < 0 or n_local < 1:
            raise ValueError("need n_sink >= 0 and n_local >= 1")
        self.n_sink = n_sink
        self.n_local = n_local
        self.n_appended = 0
        self.t: Dict[int, int] = {}
        self.k: Dict[int, object] = {}
        self.v: Dict[int, object] = {}
        self.evicted: List[int] = []

    def resident(self) -> List[int]:
        return resident_frames(self.n_appended, self.n_sink, self.n_local)

    def append(self, n_frames: int, t0: int, k_frames=None, v_frames=None) -> List[int]:
        """Append frames n_appended .. n_appended+n_frames-1 with times t0, t0+1, ...

        Returns the frames evicted by this append.  The chunk may not evict
        its own frames: the non-sink part of the chunk must fit the ring.
        """
        first = self.n_appended
        new = list(range(first, first + n_frames))
        non_sink = [f for f in new if f >= self.n_sink]
        if len(non_sink) > self.n_local:
            raise ValueError("chunk larger than the local window")
        if self.t and t0 <= self.t[max(self.t)]:
            raise ValueError("time positions must increase")
        before = set(self.resident())
        for i, f in enumerate(new):
            self.t[f] = t0 + i
            if k_frames is not None:
                self.k[f] = k_frames[i]
            if v_frames is not None:
                self.v[f] = v_frames[i]
        self.n_appended += n_frames
        after = set(self.resident())
        gone = sorted(before - after)
        for f in gone:
            self.t.pop(f, None)
            self.k.pop(f, None)
            self.v.pop(f, None)
        self.evicted.extend(gone)
        return gone

    def slots(self) -> List[SlotEntry]:
        out = []
        for f in self.resident():
            seg, s = slot_of(f, self.n_sink, self.n_local)
            out.append(SlotEntry(f, self.t[f], seg, s))
        return out

    def reset(self) -> None:
        """Drop every frame (the 'no KV cache' switch policy)."""
        self.__init__(self.n_sink, self.n_local)
