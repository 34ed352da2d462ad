"""Host control plane of the paged KV cache (include/pagedkv_host.h): page
allocator, sequences, step-metadata builder and prefix index, all in the C++
of libpagedkv.so.  This module only marshals numpy arrays into that C ABI."""
from __future__ import annotations

import ctypes

import numpy as np

from ._binding import PagedKVError, load

# every function include/pagedkv_host.h declares
HOST_EXPORTS = ("pkv_pool_create", "pkv_pool_destroy", "pkv_pool_free_pages", "pkv_pool_used_pages",
                "pkv_page_alloc", "pkv_page_release", "pkv_page_confirm", "pkv_page_refcount", "pkv_page_dirty",
                "pkv_seq_create", "pkv_seq_append", "pkv_seq_append_batch", "pkv_seq_fork", "pkv_seq_release", "pkv_seq_length",
                "pkv_seq_pages", "pkv_build_step", "pkv_prefix_insert", "pkv_prefix_match", "pkv_prefix_evict",
                "pkv_prefix_pages")
NO_PAGES, BAD_HANDLE, DIRTY = -20, -21, -22

_declared = False


def _lib():
    global _declared
    lib = load()
    if not _declared:
        vp, i64, i32, u64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint64
        sig = {
            "pkv_pool_create": ([i64, i32], vp),
            "pkv_pool_destroy": ([vp], None),
            "pkv_pool_free_pages": ([vp], i64),
            "pkv_pool_used_pages": ([vp], i64),
            "pkv_page_alloc": ([vp, i64, vp], i32),
            "pkv_page_release": ([vp, vp, i64], i32),
            "pkv_page_confirm": ([vp, vp, i64], i32),
            "pkv_page_refcount": ([vp, i64], i32),
            "pkv_page_dirty": ([vp, i64], i32),
            "pkv_seq_create": ([vp, vp], i32),
            "pkv_seq_append": ([vp, i64, i64, vp], i32),
            "pkv_seq_append_batch": ([vp, vp, i64, vp, vp], i32),
            "pkv_seq_fork": ([vp, i64, i64, vp, vp], i32),
            "pkv_seq_release": ([vp, i64], i32),
            "pkv_seq_length": ([vp, i64], i64),
            "pkv_seq_pages": ([vp, i64, vp, i64], i64),
            "pkv_build_step": ([vp, vp, i64, vp, i64, i64, vp, vp, vp], i32),
            "pkv_prefix_insert": ([vp, u64, i64, vp, i64], i32),
            "pkv_prefix_match": ([vp, u64, vp, i64, vp, vp], i32),
            "pkv_prefix_evict": ([vp, i64, vp], i32),
            "pkv_prefix_pages": ([vp], i64),
        }
        for name, (args, res) in sig.items():
            f = getattr(lib, name)
            f.argtypes, f.restype = args, res
        _declared = True
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data if a.size else None


def _check(st: int, what: str) -> int:
    if st < 0:
        raise PagedKVError(st, f"{what}: {load().pkv_status_string(int(st)).decode()}")
    return st


class PagePool:
    """A pool of page ids [0, num_pages) of page_size rows (see pagedkv_host.h)."""

    def __init__(self, num_pages: int, page_size: int = 16):
        self._lib = _lib()
        self._h = self._lib.pkv_pool_create(int(num_pages), int(page_size))
        if not self._h:
            raise PagedKVError(-2, "pkv_pool_create: bad arguments")
        self.num_pages, self.page_size = int(num_pages), int(page_size)

    def close(self):
        if self._h:
            self._lib.pkv_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    # ---- pages
    @property
    def free_pages(self) -> int:
        return self._lib.pkv_pool_free_pages(self._h)

    @property
    def used_pages(self) -> int:
        return self._lib.pkv_pool_used_pages(self._h)

    def alloc(self, n: int) -> np.ndarray:
        out = np.empty(int(n), dtype=np.int64)
        _check(self._lib.pkv_page_alloc(self._h, int(n), _ptr(out)), "pkv_page_alloc")
        return out

    def release(self, handles) -> None:
        h = np.ascontiguousarray(handles, dtype=np.int64)
        _check(self._lib.pkv_page_release(self._h, _ptr(h), h.size), "pkv_page_release")

    def confirm(self, page_ids) -> None:
        p = np.ascontiguousarray(page_ids, dtype=np.int64)
        _check(self._lib.pkv_page_confirm(self._h, _ptr(p), p.size), "pkv_page_confirm")

    def refcount(self, page_id: int) -> int:
        return self._lib.pkv_page_refcount(self._h, int(page_id))

    def dirty(self, page_id: int) -> int:
        return self._lib.pkv_page_dirty(self._h, int(page_id))

    # ---- sequences
    def create(self) -> int:
        out = ctypes.c_int64()
        _check(self._lib.pkv_seq_create(self._h, ctypes.byref(out)), "pkv_seq_create")
        return out.value

    def append(self, seq: int, n: int) -> np.ndarray:
        slots = np.empty(int(n), dtype=np.int64)
        _check(self._lib.pkv_seq_append(self._h, int(seq), int(n), _ptr(slots)), "pkv_seq_append")
        return slots

    def append_batch(self, seqs, n) -> np.ndarray:
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        k = np.ascontiguousarray(n, dtype=np.int64)
        slots = np.empty(int(k.sum()), dtype=np.int64)
        _check(self._lib.pkv_seq_append_batch(self._h, _ptr(s), s.size, _ptr(k), _ptr(slots)),
               "pkv_seq_append_batch")
        return slots

    def fork(self, parent: int, n_tokens: int) -> tuple[int, tuple[int, int, int]]:
        child = ctypes.c_int64()
        copy = np.zeros(3, dtype=np.int64)
        _check(self._lib.pkv_seq_fork(self._h, int(parent), int(n_tokens), ctypes.byref(child), _ptr(copy)),
               "pkv_seq_fork")
        return child.value, (int(copy[0]), int(copy[1]), int(copy[2]))

    def release_seq(self, seq: int) -> None:
        _check(self._lib.pkv_seq_release(self._h, int(seq)), "pkv_seq_release")

    def length(self, seq: int) -> int:
        return _check(self._lib.pkv_seq_length(self._h, int(seq)), "pkv_seq_length")

    def pages(self, seq: int) -> np.ndarray:
        n = _check(self._lib.pkv_seq_pages(self._h, int(seq), None, 0), "pkv_seq_pages")
        out = np.empty(n, dtype=np.int64)
        self._lib.pkv_seq_pages(self._h, int(seq), _ptr(out), n)
        return out

    # ---- one step's metadata
    def build_step(self, seqs, n_new, max_blocks: int, pad_page: int):
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        n = np.ascontiguousarray(n_new, dtype=np.int64)
        B = s.size
        bt = np.empty((B, int(max_blocks)), dtype=np.int64)
        sl = np.empty(B, dtype=np.int64)
        qsl = np.empty(B + 1, dtype=np.int64)
        _check(self._lib.pkv_build_step(self._h, _ptr(s), B, _ptr(n), int(max_blocks), int(pad_page), _ptr(bt),
                                        _ptr(sl), qsl.ctypes.data), "pkv_build_step")
        return bt, sl, qsl

    # ---- prefix index
    def prefix_insert(self, namespace: int, seq: int, tokens) -> None:
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        _check(self._lib.pkv_prefix_insert(self._h, int(namespace), int(seq), _ptr(t), t.size), "pkv_prefix_insert")

    def prefix_match(self, namespace: int, tokens) -> tuple[int, int]:
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        seq, matched = ctypes.c_int64(), ctypes.c_int64()
        _check(self._lib.pkv_prefix_match(self._h, int(namespace), _ptr(t), t.size, ctypes.byref(seq),
                                          ctypes.byref(matched)), "pkv_prefix_match")
        return seq.value, matched.value

    def prefix_evict(self, pages: int) -> int:
        freed = ctypes.c_int64()
        _check(self._lib.pkv_prefix_evict(self._h, int(pages), ctypes.byref(freed)), "pkv_prefix_evict")
        return freed.value

    @property
    def prefix_pages(self) -> int:
        return self._lib.pkv_prefix_pages(self._h)
