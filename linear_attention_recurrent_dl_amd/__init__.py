"""DeltaLog recurrent-state decode for MI355X (gfx950): Python binding.

The compute path is the HIP library ``libdeltalog.so`` built from ``csrc/``
with the C ABI of ``include/deltalog.h``.  This module only marshals
arguments: the functions below carry the C names and forward to the library;
``DeltaLogPool`` allocates the pool buffers as torch device tensors (PyTorch is
used for device memory and streams only) and passes their addresses and the
current stream.  If the library is missing every call raises.
"""

from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np

from . import _native as N
from ._native import DeltaLogError, DL_DECAY, DL_DTYPE, DL_UPDATE  # noqa: F401

__all__ = ["dl_pool_sizes", "dl_pool_create", "dl_pool_destroy", "dl_slot_assign", "dl_decode_step",
           "dl_decode_step_noalloc", "dl_decode_window", "dl_eager_step", "dl_merge", "dl_flush_all",
           "dl_get_log_len", "dl_schedule", "dl_read_log_len_device", "dl_value_tile", "dl_last_error",
           "dl_launch_slot_limit", "make_desc", "DeltaLogPool", "DeltaLogError"]


def make_desc(num_slots: int, max_batch: int, H_v: int, H_k: int, d: int, L: int,
              decay: str, update: str, state_dtype: str, in_dtype: str,
              value_tile: int = 0, replay_split: int = 0) -> N.dl_pool_desc:
    return N.dl_pool_desc(num_slots, max_batch, H_v, H_k, d, d, L, DL_DECAY[decay],
                          DL_UPDATE[update], DL_DTYPE[state_dtype], DL_DTYPE[in_dtype], value_tile,
                          int(replay_split))


def _ids(slot_ids) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(slot_ids, dtype=np.int32).reshape(-1))
    return a


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


# ------------------------------------------------------------ C-named calls
def dl_pool_sizes(desc: N.dl_pool_desc) -> list:
    out = (ctypes.c_size_t * N.DL_NUM_BUFS)()
    N.check(N.lib().dl_pool_sizes(ctypes.byref(desc), out), "dl_pool_sizes")
    return [int(x) for x in out]


def dl_pool_create(desc: N.dl_pool_desc, buffers: Optional[N.dl_pool_buffers]) -> int:
    h = ctypes.c_void_p()
    N.check(N.lib().dl_pool_create(ctypes.byref(desc), None if buffers is None else ctypes.byref(buffers),
                                   ctypes.byref(h)), "dl_pool_create")
    return h.value


def dl_pool_destroy(pool: int) -> None:
    N.check(N.lib().dl_pool_destroy(pool), "dl_pool_destroy")


def dl_slot_assign(pool: int, slot_ids, init_base, stream) -> None:
    ids = _ids(slot_ids)
    N.check(N.lib().dl_slot_assign(pool, len(ids), _i32p(ids), N.ptr(init_base), stream), "dl_slot_assign")


def dl_decode_step(pool: int, slot_ids, q, a_or_k, b_or_v, lam, beta, out, stream) -> None:
    ids = _ids(slot_ids)
    N.check(N.lib().dl_decode_step(pool, len(ids), _i32p(ids), N.ptr(q), N.ptr(a_or_k), N.ptr(b_or_v),
                                   N.ptr(lam), N.ptr(beta), N.ptr(out), stream), "dl_decode_step")


def dl_decode_step_noalloc(pool: int, slot_ids, q, a_or_k, b_or_v, lam, beta, out, stream) -> None:
    ids = _ids(slot_ids)
    N.check(N.lib().dl_decode_step_noalloc(pool, len(ids), _i32p(ids), N.ptr(q), N.ptr(a_or_k), N.ptr(b_or_v),
                                           N.ptr(lam), N.ptr(beta), N.ptr(out), stream), "dl_decode_step_noalloc")


def dl_decode_window(pool: int, slot_ids, W: int, q, a_or_k, b_or_v, lam, beta, out, stream) -> None:
    ids = _ids(slot_ids)
    N.check(N.lib().dl_decode_window(pool, len(ids), _i32p(ids), int(W), N.ptr(q), N.ptr(a_or_k), N.ptr(b_or_v),
                                     N.ptr(lam), N.ptr(beta), N.ptr(out), stream), "dl_decode_window")


def dl_eager_step(pool: int, slot_ids, q, a_or_k, b_or_v, lam, beta, out, stream) -> None:
    ids = _ids(slot_ids)
    N.check(N.lib().dl_eager_step(pool, len(ids), _i32p(ids), N.ptr(q), N.ptr(a_or_k), N.ptr(b_or_v),
                                  N.ptr(lam), N.ptr(beta), N.ptr(out), stream), "dl_eager_step")


def dl_merge(pool: int, slot_ids, stream) -> None:
    ids = _ids(slot_ids)
    N.check(N.lib().dl_merge(pool, len(ids), _i32p(ids), stream), "dl_merge")


def dl_flush_all(pool: int, stream) -> None:
    N.check(N.lib().dl_flush_all(pool, stream), "dl_flush_all")


def dl_read_base(pool: int, slot_ids, out, stream) -> None:
    ids = _ids(slot_ids)
    N.check(N.lib().dl_read_base(pool, len(ids), _i32p(ids), N.ptr(out), stream), "dl_read_base")


def dl_get_log_len(pool: int, num_slots: int) -> np.ndarray:
    out = np.zeros(num_slots, dtype=np.int32)
    N.check(N.lib().dl_get_log_len(pool, _i32p(out)), "dl_get_log_len")
    return out


def dl_schedule(pool: int, slot_ids):
    ids = _ids(slot_ids)
    merge = np.zeros(len(ids), dtype=np.int32)
    index = np.zeros(len(ids), dtype=np.int32)
    N.check(N.lib().dl_schedule(pool, len(ids), _i32p(ids), _i32p(merge), _i32p(index)), "dl_schedule")
    return merge, index


def dl_value_tile(desc: N.dl_pool_desc) -> int:
    rc = N.lib().dl_value_tile(ctypes.byref(desc))
    if rc < 0:
        N.check(rc, "dl_value_tile")
    return int(rc)


def dl_read_log_len_device(pool: int, num_slots: int, H_v: int, stream, tiles: int = 1) -> np.ndarray:
    """Live length of every value tile, [num_slots, H_v * tiles]."""
    out = np.zeros((num_slots, H_v * tiles), dtype=np.int32)
    N.check(N.lib().dl_read_log_len_device(pool, _i32p(out), stream), "dl_read_log_len_device")
    return out


def dl_last_error() -> str:
    return N.lib().dl_last_error().decode()


def dl_launch_slot_limit() -> int:
    return int(N.lib().dl_launch_slot_limit())


# ------------------------------------------------------------- torch pool
class DeltaLogPool:
    """A pool whose buffers are torch device tensors (or a host-only pool).

    ``device=None`` creates the host-only pool of the C ABI: every call
    validates and advances the live-log bookkeeping, nothing runs on a GPU.
    """

    def __init__(self, num_slots: int, H_v: int, H_k: int, d: int, L: int, decay: str,
                 update: str, state_dtype: str = "f32", in_dtype: str = "f32",
                 max_batch: Optional[int] = None, device="cuda", value_tile: int = 0,
                 replay_split: bool = False, coef_buffer: bool = True):
        self.num_slots, self.H_v, self.H_k, self.d, self.L = num_slots, H_v, H_k, d, L
        self.decay, self.update = decay, update
        self.state_dtype, self.in_dtype = state_dtype, in_dtype
        self.max_batch = max_batch or num_slots
        self.replay_split = bool(replay_split)
        self.desc = make_desc(num_slots, self.max_batch, H_v, H_k, d, L, decay, update,
                              state_dtype, in_dtype, value_tile, int(replay_split))
        self.sizes = dl_pool_sizes(self.desc)
        self.value_tile = dl_value_tile(self.desc)
        self.tiles = d // self.value_tile
        self.device = device
        self.bufs = {}
        if device is None:
            self.handle = dl_pool_create(self.desc, None)
            return
        import torch
        self._torch = torch
        ptrs = []
        for name, nbytes in zip(N.BUF_NAMES, self.sizes):
            if name == "coef" and not coef_buffer:
                nbytes = 0                  # decoded through dl_decode_step_noalloc only
            t = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
            self.bufs[name] = t
            ptrs.append(t.data_ptr() if nbytes else None)
        self.handle = dl_pool_create(self.desc, N.dl_pool_buffers(*ptrs))

    # -- helpers --------------------------------------------------------
    def _stream(self):
        return self._torch.cuda.current_stream().cuda_stream if self.device is not None else None

    def _tdtype(self, name: str):
        return {"f32": self._torch.float32, "bf16": self._torch.bfloat16}[name]

    def _check(self, t, shape, dtype, what):
        if t is None:
            raise ValueError(f"{what} is required")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{what}: shape {tuple(t.shape)} != {tuple(shape)}")
        if t.dtype != dtype:
            raise ValueError(f"{what}: dtype {t.dtype} != {dtype}")
        if not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError(f"{what}: must be a contiguous CUDA tensor")

    @property
    def base_tiles(self):
        """[P, H_v, d / B_V, d, B_V] view of the value-tile-major dense base."""
        t = self.bufs["base"][: self.sizes[0]]
        return t.view(self._tdtype(self.state_dtype)).view(
            self.num_slots, self.H_v, self.tiles, self.d, self.value_tile)

    def read_base(self, slot_ids) -> "torch.Tensor":
        """Bases of the given slots in the natural layout, [n, H_v, d, d] (state
        dtype), in launches of at most max_batch slots.  A base is the logical
        state only for a slot whose log is empty (after merge / flush_all)."""
        ids = _ids(slot_ids)
        out = self._torch.empty((len(ids), self.H_v, self.d, self.d), dtype=self._tdtype(self.state_dtype),
                                device=self.bufs["base"].device)
        for lo in range(0, len(ids), self.max_batch):
            dl_read_base(self.handle, ids[lo: lo + self.max_batch], out[lo: lo + self.max_batch], self._stream())
        return out

    def nlog_tensor(self):
        return self.bufs["nlog"][: self.sizes[4]].view(self._torch.int32).view(
            self.num_slots, self.H_v * self.tiles)

    # -- calls ------------------------------------------------------------
    def assign(self, slot_ids, init=None) -> None:
        ids = _ids(slot_ids)
        if self.device is not None and init is not None:
            self._check(init, (len(ids), self.H_v, self.d, self.d), self._tdtype(self.state_dtype), "init")
        dl_slot_assign(self.handle, ids, init, self._stream())

    def _token_args(self, ids, q, a_or_k, b_or_v, lam, beta, out, W=None):
        lead = (len(ids),) if W is None else (int(W), len(ids))     # [B, ..] or step-major [W, B, ..]
        if self.device is None:
            return q, a_or_k, b_or_v, lam, beta, out
        it = self._tdtype(self.in_dtype)
        f32 = self._torch.float32
        self._check(q, lead + (self.H_k, self.d), it, "q")
        self._check(a_or_k, lead + (self.H_k, self.d), it, "a_or_k")
        self._check(b_or_v, lead + (self.H_v, self.d), it, "b_or_v")
        if self.decay == "scalar":
            self._check(lam, lead + (self.H_v,), f32, "lambda")
        elif self.decay == "per_key":
            self._check(lam, lead + (self.H_v, self.d), f32, "lambda")
        if self.update == "delta":
            self._check(beta, lead + (self.H_v,), f32, "beta")
        if out is None:
            out = self._torch.empty(lead + (self.H_v, self.d), dtype=f32, device=q.device)
        self._check(out, lead + (self.H_v, self.d), f32, "out")
        return q, a_or_k, b_or_v, lam, beta, out

    def decode_step(self, slot_ids, q=None, a_or_k=None, b_or_v=None, lam=None, beta=None, out=None):
        ids = _ids(slot_ids)
        q, a_or_k, b_or_v, lam, beta, out = self._token_args(ids, q, a_or_k, b_or_v, lam, beta, out)
        dl_decode_step(self.handle, ids, q, a_or_k, b_or_v, lam, beta, out, self._stream())
        return out

    def decode_step_noalloc(self, slot_ids, q=None, a_or_k=None, b_or_v=None, lam=None, beta=None, out=None):
        """decode_step through the entry point that allocates nothing (the
        library's static scratch holds the split-replay coefficients)."""
        ids = _ids(slot_ids)
        q, a_or_k, b_or_v, lam, beta, out = self._token_args(ids, q, a_or_k, b_or_v, lam, beta, out)
        dl_decode_step_noalloc(self.handle, ids, q, a_or_k, b_or_v, lam, beta, out, self._stream())
        return out

    def decode_window(self, slot_ids, W: int, q=None, a_or_k=None, b_or_v=None, lam=None, beta=None, out=None):
        """W consecutive steps of the same slots in one launch; token tensors
        are step-major [W, B, ..] and out is [W, B, H_v, d].  Every slot's log
        is empty afterwards."""
        ids = _ids(slot_ids)
        q, a_or_k, b_or_v, lam, beta, out = self._token_args(ids, q, a_or_k, b_or_v, lam, beta, out, W)
        dl_decode_window(self.handle, ids, W, q, a_or_k, b_or_v, lam, beta, out, self._stream())
        return out

    def eager_step(self, slot_ids, q=None, a_or_k=None, b_or_v=None, lam=None, beta=None, out=None):
        ids = _ids(slot_ids)
        q, a_or_k, b_or_v, lam, beta, out = self._token_args(ids, q, a_or_k, b_or_v, lam, beta, out)
        dl_eager_step(self.handle, ids, q, a_or_k, b_or_v, lam, beta, out, self._stream())
        return out

    def merge(self, slot_ids) -> None:
        dl_merge(self.handle, slot_ids, self._stream())

    def flush_all(self) -> None:
        dl_flush_all(self.handle, self._stream())

    def log_len(self) -> np.ndarray:
        return dl_get_log_len(self.handle, self.num_slots)

    def schedule(self, slot_ids):
        return dl_schedule(self.handle, slot_ids)

    def device_log_len(self) -> np.ndarray:
        return dl_read_log_len_device(self.handle, self.num_slots, self.H_v, self._stream(), self.tiles)

    def close(self) -> None:
        if getattr(self, "handle", None):
            dl_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
