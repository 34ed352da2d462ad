"""GPU-side helpers for the parity tests: run one write+attention step through
the C ABI, and compare with the oracle at the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np
import torch

from tests import helpers as H

# max |gpu - oracle| bounds (fp64 oracle on identical dequantised inputs)
TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8_e4m3fn": 6e-2}
# bound on max |gpu - oracle| / rms(oracle output), next to the absolute bars:
# the rounding of P and of the output to bf16 keeps it near 2^-9 times the
# ratio of the largest output element to the rms; the largest value over all
# parity cases is about 0.05, and this bound is twice that
REL_TOL = 0.1


def note(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def gpu_write(pkv, w):
    """Library write into copies of w's pools; returns the written pools."""
    kp, vp = w.key_pool.clone(), w.value_pool.clone()
    pkv.paged_kv_write(w.k_new, w.v_new, w.slot_mapping, kp, vp)
    return kp, vp


def gpu_attend(pkv, w, kp, vp, *, split_tokens=None, max_query_len=None, scale=None, q=None):
    q = w.q if q is None else q
    out = torch.empty_like(q)
    pkv.paged_attention(q, kp, vp, w.block_table, w.seq_lens, w.query_start_loc,
                        w.scale if scale is None else scale, out,
                        k_scale=w.k_scale, v_scale=w.v_scale,
                        max_query_len=w.max_query_len if max_query_len is None else max_query_len,
                        split_tokens=w.split_tokens if split_tokens is None else split_tokens)
    torch.cuda.synchronize()
    return out


def gpu_step(pkv, w, **kw):
    kp, vp = gpu_write(pkv, w)
    return kp, vp, gpu_attend(pkv, w, kp, vp, **kw)


def as_f64(out: torch.Tensor) -> np.ndarray:
    return out.detach().float().cpu().numpy().astype(np.float64)


def assert_close(gpu_out, ref, kv_dtype, what=""):
    g = as_f64(gpu_out) if isinstance(gpu_out, torch.Tensor) else gpu_out
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    err = float(np.max(np.abs(g - ref))) if g.size else 0.0
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 1.0
    note(f"{what}: max|err| = {err:.3e} (tol {TOL[kv_dtype]:.0e}), max|err|/rms = {err / max(rms, 1e-30):.3e}")
    assert err <= TOL[kv_dtype], f"{what}: max|err| {err} > {TOL[kv_dtype]}"
    assert err <= REL_TOL * rms, f"{what}: max|err|/rms {err / rms} > {REL_TOL}"
    return err


def sample_rows(w, per_seq: int, seed: int = 0) -> np.ndarray:
    """Packed query rows to check at full size: first, last and random rows of
    every sequence (all rows of short sequences)."""
    rng = np.random.default_rng(seed)
    qsl = H.S(w.query_start_loc)
    rows = []
    for b in range(len(qsl) - 1):
        lo, hi = int(qsl[b]), int(qsl[b + 1])
        if hi - lo <= per_seq:
            rows.extend(range(lo, hi))
        else:
            pick = set([lo, hi - 1]) | set(rng.choice(np.arange(lo, hi), per_seq - 2, replace=False).tolist())
            rows.extend(sorted(pick))
    return np.array(rows, dtype=np.int64)
