"""Oracle of the HBM object store's placement and backpressure order (test
infrastructure only).

Source: the PATHWAYS page ("PATHWAYS: Asynchronous Distributed Dataflow for
ML"), section 4.6 "Data management": each host keeps an object store that
tracks the buffers held in accelerator memory, objects are named by opaque
handles, ownership labels let everything of a failed client or program be
garbage collected, and when an allocation fails because other programs'
buffers occupy the memory, simple backpressure stalls that computation
instead of failing it.

Readings (the pages give no allocator): the store is one extent of device
memory; sizes round up to 256 bytes; placement is first fit by address over
the free extents, and freed extents merge with free neighbours; a request
that does not fit waits, and waiting requests are served in arrival order
(a later request never overtakes a waiting one, so large requests are not
starved); a request larger than the whole store fails at once.
"""
from __future__ import annotations

ALIGN = 256


def round_up(n: int) -> int:
    return (n + ALIGN - 1) // ALIGN * ALIGN


class Store:
    def __init__(self, size: int):
        self.size = size - size % ALIGN
        self.free = [(0, self.size)]      # (offset, length), sorted by offset, no two adjacent
        self.live = {}                    # name -> (offset, length, owner)
        self.waiting = []                 # [(name, length, owner)] in arrival order
        self.grants = []                  # (name, offset) in the order requests were satisfied

    def _fit(self, length):
        for i, (off, ln) in enumerate(self.free):
            if ln >= length:
                if ln == length:
                    del self.free[i]
                else:
                    self.free[i] = (off + length, ln - length)
                return off
        return None

    def _serve(self):
        while self.waiting:
            name, length, owner = self.waiting[0]
            off = self._fit(length)
            if off is None:
                return
            self.waiting.pop(0)
            self.live[name] = (off, length, owner)
            self.grants.append((name, off))

    def alloc(self, name, nbytes: int, owner: int = 0):
        """Returns the offset, or None if the request waits; raises
        MemoryError if it can never fit."""
        length = round_up(max(nbytes, 1))
        if length > self.size:
            raise MemoryError(name)
        self.waiting.append((name, length, owner))
        self._serve()
        return self.live[name][0] if name in self.live else None

    def _release(self, off, length):
        self.free.append((off, length))
        self.free.sort()
        merged = []
        for o, ln in self.free:
            if merged and merged[-1][0] + merged[-1][1] == o:
                merged[-1] = (merged[-1][0], merged[-1][1] + ln)
            else:
                merged.append((o, ln))
        self.free = merged

    def free_obj(self, name):
        off, length, _ = self.live.pop(name)
        self._release(off, length)
        self._serve()

    def release_owner(self, owner: int) -> int:
        names = [n for n, (_, _, o) in self.live.items() if o == owner]
        for n in names:
            off, length, _ = self.live.pop(n)
            self._release(off, length)
        self._serve()
        return len(names)

    def in_use(self) -> int:
        return sum(ln for _, ln, _ in self.live.values())


def run(size: int, ops):
    """Apply ops in order: ("alloc", name, bytes, owner), ("free", name),
    ("release", owner). Returns the store (its .grants list the satisfied
    requests in order with their offsets)."""
    st = Store(size)
    for op in ops:
        if op[0] == "alloc":
            st.alloc(op[1], op[2], op[3] if len(op) > 3 else 0)
        elif op[0] == "free":
            st.free_obj(op[1])
        elif op[0] == "release":
            st.release_owner(op[1])
        else:
            raise ValueError(op)
    return st
