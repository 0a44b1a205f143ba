"""Python binding of the host block manager (pa_bm_* in include/pagedkv.h).

``BlockManager`` wraps the native manager (allocation and step planning run in
C++); ``StepStager`` adds the device side an engine needs: pinned host blobs
and device blobs used in turn, and the single host-to-device copy per step,
overlapped with the previous step's kernels on a copy stream.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np

from ._lib import BmLayout, check, lib


class BlockManager:
    """Paged KV block allocation for ``max_seqs`` sequences (ids 0..max_seqs-1)."""

    def __init__(self, num_blocks: int, block_size: int, max_seqs: int, max_blocks_per_seq: int,
                 max_step_seqs: int, max_step_tokens: int):
        h = ctypes.c_void_p()
        check(lib.pa_bm_create(num_blocks, block_size, max_seqs, max_blocks_per_seq, max_step_seqs,
                               max_step_tokens, ctypes.byref(h)))
        self._h = h
        self.num_blocks, self.block_size = num_blocks, block_size
        self.max_seqs, self.width = max_seqs, max_blocks_per_seq
        self.max_step_seqs, self.max_step_tokens = max_step_seqs, max_step_tokens
        lay = BmLayout()
        check(lib.pa_bm_layout_of(h, ctypes.byref(lay)))
        self.layout = lay
        self._scratch = None

    def close(self) -> None:
        if self._h:
            lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def free_blocks(self) -> int:
        return int(lib.pa_bm_free_blocks(self._h))

    def seq_len(self, seq: int) -> int:
        n = int(lib.pa_bm_seq_len(self._h, seq))
        if n < 0:
            raise ValueError(f"bad sequence id {seq}")
        return n

    def seq_table(self, seq: int) -> np.ndarray:
        out = np.empty(self.width, dtype=np.int32)
        n = int(lib.pa_bm_seq_table(self._h, seq, out.ctypes.data, self.width))
        if n < 0:
            raise ValueError(f"bad sequence id {seq}")
        return out[:n].copy()

    def release(self, seq: int) -> None:
        check(lib.pa_bm_release(self._h, seq))

    def plan_into(self, host_ptr: int, host_bytes: int, seqs, num_new, pad_seqs=None,
                  pad_tokens=None) -> tuple[int, int, int]:
        """Plan a step into the blob at host_ptr; returns (rows, tokens, real tokens)
        where rows/tokens are the (padded) sizes to launch with."""
        s = np.ascontiguousarray(seqs, dtype=np.int32)
        n = np.ascontiguousarray(num_new, dtype=np.int32)
        if s.shape != n.shape or s.ndim != 1:
            raise ValueError("seqs and num_new must be 1-D of equal length")
        total = int(n.sum()) if n.size else 0
        rows = len(s) if pad_seqs is None else int(pad_seqs)
        toks = total if pad_tokens is None else int(pad_tokens)
        got = ctypes.c_int64()
        check(lib.pa_bm_plan_step(self._h, s.ctypes.data, n.ctypes.data, len(s), rows, toks, host_ptr,
                                  host_bytes, ctypes.byref(got)))
        return rows, toks, int(got.value)

    def plan_host(self, seqs, num_new, pad_seqs=None, pad_tokens=None):
        """Plan a step into a host blob and return numpy copies of its arrays:
        (slot_mapping, block_tables, context_lens, cu_seqlens_q)."""
        if self._scratch is None:
            self._scratch = np.zeros(self.layout.bytes + 256, dtype=np.uint8)
        base = self._scratch.ctypes.data
        off = (-base) % 256
        rows, toks, _ = self.plan_into(base + off, self.layout.bytes, seqs, num_new, pad_seqs, pad_tokens)
        return host_views(self._scratch[off:off + self.layout.bytes], self.layout, rows, toks, self.width,
                          copy=True)


def host_views(blob: np.ndarray, lay, rows: int, toks: int, width: int, copy: bool = False):
    def view(off, count, dt):
        a = blob[off:off + count * np.dtype(dt).itemsize].view(dt)
        return a.copy() if copy else a
    sm = view(lay.slot_mapping, toks, np.int64)
    bt = view(lay.block_tables, rows * width, np.int32).reshape(rows, width)
    cl = view(lay.context_lens, rows, np.int32)
    cu = view(lay.cu_seqlens_q, rows + 1, np.int32)
    return sm, bt, cl, cu


@dataclass
class DeviceStep:
    """One step's metadata on the device: views into one of the stager's device
    blobs, valid for the kernels enqueued before the stager's next call (the
    blob is rewritten ``depth`` calls later, after those kernels)."""
    slot_mapping: object   # int64 [num_tokens]
    block_tables: object   # int32 [num_seqs, max_blocks_per_seq]
    context_lens: object   # int32 [num_seqs]
    cu_seqlens_q: object   # int32 [num_seqs + 1]
    num_seqs: int          # rows to launch with (padded)
    num_tokens: int        # tokens to launch with (padded)
    real_tokens: int


class StepStager:
    """Plans steps into pinned host blobs and uploads each with one asynchronous
    copy into a device blob; ``depth`` pairs of blobs are used in turn.

    With ``overlap`` (the default) the copies run on a stream of their own, so
    the upload of step k+1 proceeds while step k's kernels run; the compute
    stream waits for it where step k+1's kernels start. Before a pair of blobs
    is reused, the host waits until the kernels that read its previous step have
    finished (``depth`` steps back, normally long done). The copy stream itself
    never waits on the compute stream: such a wait on a copy queue can stall the
    enqueuing host thread. Without ``overlap`` the copy goes on the compute
    stream."""

    def __init__(self, bm: BlockManager, device="cuda", depth: int = 3, overlap: bool = True):
        import torch
        self.torch = torch
        self.bm = bm
        n = bm.layout.bytes
        self.host = [torch.empty(n, dtype=torch.uint8, pin_memory=True) for _ in range(depth)]
        self.devs = [torch.empty(n, dtype=torch.uint8, device=device) for _ in range(depth)]
        self.dev = self.devs[0]
        self.copy_stream = torch.cuda.Stream(device=device) if overlap else None
        # per pair: an event recorded after the kernels that read it, and one after
        # its upload (created once and re-recorded: a wait or sync binds to the
        # latest record, which is all a step needs)
        self.consumed = [torch.cuda.Event() for _ in range(depth)]
        self.recorded = [False] * depth
        self.uploaded = [torch.cuda.Event() for _ in range(depth)]
        self._views = {}                    # (pair, rows, tokens) -> device views
        self.k = 0

    def step(self, seqs, num_new, pad_seqs=None, pad_tokens=None, stream=None) -> DeviceStep:
        torch = self.torch
        st = stream or torch.cuda.current_stream()
        depth = len(self.host)
        if self.k > 0:                      # everything enqueued so far read the previous pair
            j = (self.k - 1) % depth
            self.consumed[j].record(st)
            self.recorded[j] = True
        i = self.k % depth
        self.k += 1
        if self.recorded[i]:
            self.consumed[i].synchronize()  # its last kernels (and so its upload) are done
        h, d = self.host[i], self.devs[i]
        rows, toks, real = self.bm.plan_into(h.data_ptr(), h.numel(), seqs, num_new, pad_seqs, pad_tokens)
        cs = self.copy_stream or st
        check(lib.pa_bm_upload(self.bm._h, h.data_ptr(), d.data_ptr(), rows, cs.cuda_stream))
        if self.copy_stream is not None:
            up = self.uploaded[i]
            up.record(cs)
            st.wait_event(up)
        self.dev = d
        v = self._views.get((i, rows, toks))
        if v is None:
            lay, W = self.bm.layout, self.bm.width

            def view(off, count, dt, itemsize):
                return d[off:off + count * itemsize].view(dt)
            v = (view(lay.slot_mapping, toks, torch.int64, 8),
                 view(lay.block_tables, rows * W, torch.int32, 4).view(rows, W),
                 view(lay.context_lens, rows, torch.int32, 4),
                 view(lay.cu_seqlens_q, rows + 1, torch.int32, 4))
            self._views[(i, rows, toks)] = v
        return DeviceStep(slot_mapping=v[0], block_tables=v[1], context_lens=v[2], cu_seqlens_q=v[3],
                          num_seqs=rows, num_tokens=toks, real_tokens=real)
