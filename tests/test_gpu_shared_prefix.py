"""GPU parity of the shared-prefix form of decode (shared_prefix_pages): the
prefix's attention as MFMA tiles over all sequences, merged with each
sequence's own split-K decode, must give the plain attention the oracle
computes (which knows nothing of the sharing)."""
import dataclasses

import numpy as np
import pytest
import torch

from paged_kv_cache_243_amd import workloads as W
from tests import helpers as H
from tests.gpu_helpers import assert_close, gpu_write, note

pytestmark = pytest.mark.gpu
DEV = "cuda"


def attend_shared(gpu, w, kp, vp, pages, split_tokens=None):
    out = torch.empty_like(w.q)
    gpu.paged_attention(w.q, kp, vp, w.block_table, w.seq_lens, w.query_start_loc, w.scale, out,
                        k_scale=w.k_scale, v_scale=w.v_scale, max_query_len=1,
                        split_tokens=w.split_tokens if split_tokens is None else split_tokens,
                        shared_prefix_pages=pages)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3fn"])
@pytest.mark.parametrize("split", [0, 64])
def test_shared_prefix_small(gpu, kv, split):
    note(f"shared prefix small kv={kv} split={split}")
    cfg = W.SMALL[4] if kv == "bf16" else dataclasses.replace(W.SMALL[4], kv_dtype=kv, name="shared-prefix-fp8-small")
    w = W.generate(cfg, DEV)
    kp, vp = gpu_write(gpu, w)
    out = attend_shared(gpu, w, kp, vp, cfg.shared_prefix_tokens // 16, split)
    _, _, ref = H.oracle_step(w)
    assert_close(out, ref, kv, f"shared prefix small kv={kv} split={split}")


def test_shared_prefix_full(gpu):
    """256 sequences on 128 shared pages, in the launch configuration the
    benchmark times; every row against the oracle."""
    note("shared prefix full config 4")
    w = W.generate(4, DEV)
    kp, vp = gpu_write(gpu, w)
    out = attend_shared(gpu, w, kp, vp, w.cfg.shared_prefix_tokens // 16)
    okp, ovp = H.oracle_write(w)
    ref = H.oracle_attend(w, okp, ovp)
    assert_close(out, ref, "bf16", "shared prefix full config 4")


def test_shared_prefix_with_sequences_without_query_rows(gpu):
    note("shared prefix with empty query spans")
    w = W.generate(W.SMALL[4], DEV)
    B = w.cfg.batch
    n = np.ones(B, dtype=np.int64)
    n[1::3] = 0
    keep = torch.as_tensor(np.flatnonzero(n), device=DEV)
    qsl = np.concatenate([[0], np.cumsum(n)])
    w2 = dataclasses.replace(w, q=w.q[keep].contiguous(), k_new=w.k_new[keep].contiguous(),
                             v_new=w.v_new[keep].contiguous(), slot_mapping=w.slot_mapping[keep].contiguous(),
                             query_start_loc=torch.as_tensor(qsl, device=DEV),
                             seq_lens=w.seq_lens - 1 + torch.as_tensor(n, device=DEV))
    w2.meta = dict(w.meta, n_new=n)
    kp, vp = gpu_write(gpu, w2)
    out = attend_shared(gpu, w2, kp, vp, w.cfg.shared_prefix_tokens // 16)
    _, _, ref = H.oracle_step(w2)
    assert_close(out, ref, "bf16", "shared prefix with empty spans")


def test_shared_prefix_matches_the_plain_call(gpu):
    """Same inputs through both forms: both within the bar of the oracle, and
    close to each other (different summation orders only)."""
    note("shared prefix vs plain call")
    w = W.generate(W.SMALL[4], DEV, seed=77)
    kp, vp = gpu_write(gpu, w)
    a = attend_shared(gpu, w, kp, vp, w.cfg.shared_prefix_tokens // 16)
    b = attend_shared(gpu, w, kp, vp, 0)
    _, _, ref = H.oracle_step(w)
    assert_close(a, ref, "bf16", "shared prefix form")
    assert_close(b, ref, "bf16", "plain form")
    assert float((a.float() - b.float()).abs().max()) <= 2e-2
