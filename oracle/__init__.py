"""CPU oracle for the paged KV write and paged attention step.

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library and
its Python binding never import it, and it imports nothing from them.

The arithmetic lives in ``pagedkv_oracle.c`` (plain C, fp64, OpenMP over
(sequence, KV head)); this module only loads it with ctypes and marshals numpy
arrays.  See that file's header for the passages of the pages each step
follows and for the readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pagedkv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPE_CODES = {"f32": 0, "bf16": 1, "fp8_e4m3fn": 2}
ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8_e4m3fn": 1}

ERRORS = {
    -1: "slot out of range",
    -2: "duplicate slot",
    -3: "page id out of range",
    -4: "inconsistent metadata",
    -5: "unsupported dtype",
    -6: "out of host memory",
}


class OracleError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"oracle status {status}: {ERRORS.get(status, 'unknown')}")
        self.status = status


def compile_source(src: str, out: str) -> str:
    """gcc, plain -O2 (no fast-math), OpenMP."""
    tmp = out + ".tmp"
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", src, "-o", tmp, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle in place (oracle/liboracle.so)."""
    if force or not os.path.exists(_LIB_PATH):
        compile_source(_SRC, _LIB_PATH)
    return _LIB_PATH


_lib = None


def open_library(path: str):
    """Load a compiled oracle from ``path`` and declare its C signatures."""
    lib = ctypes.CDLL(path)
    i64, vp, dbl, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double, ctypes.c_int
    lib.orc_paged_kv_write.argtypes = [vp, vp, vp, i64, vp, vp, i64, i64, i64]
    lib.orc_paged_kv_write.restype = i32
    lib.orc_paged_attention.argtypes = [
        vp, i32, i64, i64,            # q, q_dtype, T, Hq
        vp, vp, i32, i64, i64, i64, i64,  # pools, kv_dtype, num_pages, page_size, Hkv, D
        vp, vp,                       # k_scale, v_scale
        vp, i64, i64,                 # block_table, B, max_blocks
        vp, vp,                       # seq_lens, query_start_loc
        dbl, vp, i64,                 # scale, sel_tokens, n_sel
        vp, i32,                      # out, n_threads
    ]
    lib.orc_paged_attention.restype = i32
    lib.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_to_double.restype = dbl
    lib.orc_e4m3fn_to_double.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3fn_to_double.restype = dbl
    lib.orc_e4m3fn_table.argtypes = [vp]
    lib.orc_e4m3fn_table.restype = None
    lib.orc_e4m3fn_from_float.argtypes = [ctypes.c_float]
    lib.orc_e4m3fn_from_float.restype = ctypes.c_uint8
    lib.orc_e4m3fn_encode_array.argtypes = [vp, i64, vp]
    lib.orc_e4m3fn_encode_array.restype = None
    lib.orc_paged_kv_write_fp8.argtypes = [vp, vp, vp, i64, vp, vp, vp, vp, i64, i64, i64, i64]
    lib.orc_paged_kv_write_fp8.restype = i32
    lib.orc_block_table_from_csr.argtypes = [vp, vp, i64, vp, i64, i64, i64, i64, vp, vp]
    lib.orc_block_table_from_csr.restype = i32
    lib.orc_max_threads.argtypes = []
    lib.orc_max_threads.restype = i32
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        _lib = open_library(_LIB_PATH)
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def e4m3fn_table() -> np.ndarray:
    """fp64 value of each of the 256 E4M3FN codes (NaN for the two NaN codes)."""
    out = np.empty(256, dtype=np.float64)
    _load().orc_e4m3fn_table(_ptr(out))
    return out


def e4m3fn_encode(y: np.ndarray) -> np.ndarray:
    """E4M3FN codes (uint8) of float32 values: nearest finite code, ties to
    even, saturating at +-448, NaN kept (see orc_e4m3fn_from_float)."""
    yc = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(yc.shape, dtype=np.uint8)
    _load().orc_e4m3fn_encode_array(_ptr(yc), yc.size, _ptr(out))
    return out


def bf16_to_f64(bits: int) -> float:
    return _load().orc_bf16_to_double(int(bits) & 0xFFFF)


def max_threads() -> int:
    return _load().orc_max_threads()


def paged_kv_write(k: np.ndarray, v: np.ndarray, slot_mapping: np.ndarray,
                   key_pool: np.ndarray, value_pool: np.ndarray) -> None:
    """Scatter k/v rows into the pools in place.

    k, v: [T_new, Hkv, D] of the pool's element type (any numpy dtype of the
    right width); pools: [num_pages, page_size, Hkv, D] of the same type;
    slot_mapping: [T_new] int64.
    """
    assert k.dtype == key_pool.dtype and v.dtype == value_pool.dtype
    num_pages, page_size = key_pool.shape[0], key_pool.shape[1]
    row_bytes = int(np.prod(key_pool.shape[2:])) * key_pool.itemsize
    assert k.shape[0] == slot_mapping.shape[0] and k.nbytes == k.shape[0] * row_bytes
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    st = _load().orc_paged_kv_write(_ptr(k), _ptr(v), _ptr(sm), sm.shape[0],
                                    _ptr(key_pool), _ptr(value_pool),
                                    num_pages, page_size, row_bytes)
    if st != 0:
        raise OracleError(st)


def paged_kv_write_fp8(k: np.ndarray, v: np.ndarray, slot_mapping: np.ndarray,
                       k_scale: np.ndarray, v_scale: np.ndarray,
                       key_pool: np.ndarray, value_pool: np.ndarray) -> None:
    """Quantising scatter into fp8 pools in place.

    k, v: [T_new, Hkv, D] bf16 bit patterns (uint16); pools: [num_pages,
    page_size, Hkv, D] uint8 E4M3FN codes; k_scale, v_scale: [Hkv] float32
    dequantisation factors (element x is stored as the code of x / scale[h]).
    """
    assert k.dtype == np.uint16 and v.dtype == np.uint16
    assert key_pool.dtype == np.uint8 and value_pool.dtype == np.uint8
    num_pages, page_size, Hkv, D = key_pool.shape
    assert value_pool.shape == key_pool.shape and k.shape == v.shape == (slot_mapping.shape[0], Hkv, D)
    kc, vc = np.ascontiguousarray(k), np.ascontiguousarray(v)
    ks = np.ascontiguousarray(k_scale, dtype=np.float32)
    vs = np.ascontiguousarray(v_scale, dtype=np.float32)
    assert ks.shape == (Hkv,) and vs.shape == (Hkv,)
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    st = _load().orc_paged_kv_write_fp8(_ptr(kc), _ptr(vc), _ptr(sm), sm.shape[0], _ptr(ks), _ptr(vs),
                                        _ptr(key_pool), _ptr(value_pool), num_pages, page_size, Hkv, D)
    if st != 0:
        raise OracleError(st)


def block_table_from_csr(kv_indptr: np.ndarray, kv_indices: np.ndarray, kv_last_page_len: np.ndarray,
                         page_size: int, pad_page: int, max_blocks: int) -> tuple[np.ndarray, np.ndarray]:
    """(block_table [B, max_blocks], seq_lens [B]) from the packed page list."""
    ip = np.ascontiguousarray(kv_indptr, dtype=np.int64)
    ix = np.ascontiguousarray(kv_indices, dtype=np.int64)
    ll = np.ascontiguousarray(kv_last_page_len, dtype=np.int64)
    B = ip.shape[0] - 1
    bt = np.empty((B, int(max_blocks)), dtype=np.int64)
    sl = np.empty(B, dtype=np.int64)
    st = _load().orc_block_table_from_csr(_ptr(ip), _ptr(ix) if ix.size else None, ix.size, _ptr(ll), B,
                                          int(page_size), int(pad_page), int(max_blocks), _ptr(bt), _ptr(sl))
    if st != 0:
        raise OracleError(st)
    return bt, sl


def paged_attention(q: np.ndarray, q_dtype: str, key_pool: np.ndarray, value_pool: np.ndarray,
                    kv_dtype: str, block_table: np.ndarray, seq_lens: np.ndarray,
                    query_start_loc: np.ndarray, scale: float,
                    k_scale: np.ndarray | None = None, v_scale: np.ndarray | None = None,
                    sel_tokens: np.ndarray | None = None, threads: int = 0) -> np.ndarray:
    """fp64 attention output for the selected packed query rows.

    q: [T, Hq, D] raw storage of q_dtype ('f32' as float32, 'bf16' as uint16);
    pools: [num_pages, page_size, Hkv, D] raw storage of kv_dtype ('fp8_e4m3fn'
    as uint8 codes).  Returns [n_sel, Hq, D] float64 (n_sel = T if sel_tokens
    is None).
    """
    T, Hq, D = q.shape
    num_pages, page_size, Hkv, Dk = key_pool.shape
    assert Dk == D and value_pool.shape == key_pool.shape
    assert q.itemsize == ELEM_BYTES[q_dtype] and key_pool.itemsize == ELEM_BYTES[kv_dtype]
    bt = np.ascontiguousarray(block_table, dtype=np.int64)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int64)
    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int64)
    B, max_blocks = bt.shape
    assert sl.shape == (B,) and qsl.shape == (B + 1,)
    ks = None if k_scale is None else np.ascontiguousarray(k_scale, dtype=np.float32)
    vs = None if v_scale is None else np.ascontiguousarray(v_scale, dtype=np.float32)
    sel = None if sel_tokens is None else np.ascontiguousarray(sel_tokens, dtype=np.int64)
    n_sel = T if sel is None else sel.shape[0]
    out = np.zeros((n_sel, Hq, D), dtype=np.float64)
    qc = np.ascontiguousarray(q)
    kp = np.ascontiguousarray(key_pool)
    vp = np.ascontiguousarray(value_pool)
    st = _load().orc_paged_attention(
        _ptr(qc), DTYPE_CODES[q_dtype], T, Hq,
        _ptr(kp), _ptr(vp), DTYPE_CODES[kv_dtype], num_pages, page_size, Hkv, D,
        _ptr(ks), _ptr(vs),
        _ptr(bt), B, max_blocks,
        _ptr(sl), _ptr(qsl),
        float(scale), _ptr(sel), n_sel,
        _ptr(out), int(threads))
    if st != 0:
        raise OracleError(st)
    return out
