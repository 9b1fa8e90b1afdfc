"""Layer-ahead decode into reused scratch buffers, overlapped with the consumer.

A model's weights stay compressed in HBM; each transformer layer is decoded just
before it is used, one launch per layer (DFloat11 article, 方法介绍: decompression
at transformer-block level into a temporary buffer; its cost does not depend on the
batch, 消融研究).  `LayerPipeline` decodes layer l + 1 on a side stream while the
consumer (the layer's GEMMs) runs layer l on its own stream, into the other of
`depth` scratch buffer sets.  Events order the two streams:

  * the consumer of layer l waits for the decode of layer l (`acquire`);
  * the decode into a buffer set waits until the consumer that last read that set
    has finished (`release` records it).

Both streams have the default priority.  The decode launches take device buffers
prepared once (containers and output pointers are marshalled in the constructor),
so a layer costs one library call on the host.  `max_workgroups` caps the decode's
resident workgroups (zx_decode_block_batch_wg): the decode then leaves CUs, and
their LDS, to the consumer's kernels.
"""
from __future__ import annotations

import ctypes as C
from typing import List, Optional, Sequence

import torch

from . import zx as _zx


class LayerPipeline:
    """Decode `layers[l]` (a list of up to 16 `Compressed` tensors with the same
    shapes and dtype in every layer) into reused scratch buffers, ahead of use."""

    def __init__(self, layers: Sequence[Sequence[_zx.Compressed]], depth: int = 2,
                 err: Optional[torch.Tensor] = None, max_workgroups: int = 0):
        if depth < 2:
            raise ValueError("depth must be at least 2 (decode ahead needs a second buffer set)")
        if not layers:
            raise ValueError("no layers")
        shapes = [(c.shape, c.dtype) for c in layers[0]]
        for l, layer in enumerate(layers):
            if [(c.shape, c.dtype) for c in layer] != shapes:
                raise ValueError(f"layer {l} differs in tensor shapes or dtypes from layer 0")
            if len(layer) > 16:
                raise ValueError("at most 16 tensors per layer (one launch)")
        self.layers = [list(layer) for layer in layers]
        self.depth = depth
        self.err = err
        self.max_workgroups = int(max_workgroups)   # 0: the decode's default (all resident slots)
        self.side = torch.cuda.Stream()   # default priority
        self.bufs: List[List[torch.Tensor]] = [[_zx.empty_output(c) for c in layers[0]] for _ in range(depth)]
        # the containers (and the scratch buffers just allocated) were produced on the
        # current stream: the side stream's first decodes must come after that work
        self.side.wait_stream(torch.cuda.current_stream())
        # the buffers are written on the side stream: their memory is not handed out
        # again before the side stream's work on them is done, whenever they are freed
        for bset in self.bufs:
            for t in bset:
                t.record_stream(self.side)
        self._ready = [torch.cuda.Event() for _ in range(depth)]
        self._free = [torch.cuda.Event() for _ in range(depth)]
        self._freed = [False] * depth     # a release was recorded for this set
        self._started = {}
        # marshalled once: per layer, the container array; per buffer set, the output pointers
        self._arrays = []
        self._keep = []
        for layer in self.layers:
            cons = [c.container() for c in layer]
            self._keep.append(cons)
            self._arrays.append((_zx.zx_container * len(cons))(*cons))
        self._outs = [(C.c_void_p * len(bset))(*[t.data_ptr() for t in bset]) for bset in self.bufs]
        self._lib = _zx.lib()

    def __len__(self) -> int:
        return len(self.layers)

    def start(self, l: int) -> None:
        """Enqueue the decode of layer l on the side stream (after the consumer that
        last read its buffer set)."""
        b = l % self.depth
        if self._freed[b]:
            self.side.wait_event(self._free[b])
        arr = self._arrays[l]
        st = self._lib.zx_decode_block_batch_wg(arr, self._outs[b], len(self.layers[l]), self.max_workgroups,
                                                None if self.err is None else C.c_void_p(self.err.data_ptr()),
                                                C.c_void_p(self.side.cuda_stream))
        if st != 0:
            raise _zx.ZxError("zx_decode_block_batch_wg", st)
        self._ready[b].record(self.side)
        self._started[l] = b

    def acquire(self, l: int, stream: Optional[torch.cuda.Stream] = None) -> List[torch.Tensor]:
        """Make `stream` (default: the current one) wait for layer l's decode and
        return its decoded tensors (valid until `release(l)` and the next use of the
        buffer set)."""
        if l not in self._started:
            raise RuntimeError(f"layer {l} was not started")
        b = self._started[l]
        s = torch.cuda.current_stream() if stream is None else stream
        s.wait_event(self._ready[b])
        return self.bufs[b]

    def release(self, l: int, stream: Optional[torch.cuda.Stream] = None) -> None:
        """Record that the consumer on `stream` is done with layer l's buffers."""
        b = self._started.pop(l)
        s = torch.cuda.current_stream() if stream is None else stream
        self._free[b].record(s)
        self._freed[b] = True

    def run(self, consumer, stream: Optional[torch.cuda.Stream] = None) -> None:
        """Decode every layer one ahead of `consumer(l, tensors)`, which enqueues its
        work on `stream` (default: the current stream)."""
        n = len(self.layers)
        self.start(0)
        for l in range(n):
            if l + 1 < n:
                self.start(l + 1)
            w = self.acquire(l, stream)
            consumer(l, w)
            self.release(l, stream)
