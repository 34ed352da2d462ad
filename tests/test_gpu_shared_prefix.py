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


@pytest.mark.parametrize("split", [0, 64])
def test_shared_prefix_single_kv_head(gpu, split):
    """One KV head (8 query heads): the private decode runs 8 one-wave parts per
    workgroup, their partials merged with the prefix chunks'."""
    note(f"shared prefix, one KV head, split={split}")
    cfg = dataclasses.replace(W.SMALL[4], hq=8, hkv=1, name="shared-prefix-1kv-small")
    w = W.generate(cfg, DEV)
    kp, vp = gpu_write(gpu, w)
    out = attend_shared(gpu, w, kp, vp, cfg.shared_prefix_tokens // 16, split)
    _, _, ref = H.oracle_step(w)
    assert_close(out, ref, "bf16", f"shared prefix one KV head split={split}")


def test_shared_prefix_in_rounds_head_dim_64(gpu):
    """1024 sequences, 32 KV heads, head_dim 64: 8 groups of sequences per KV
    head against at most 6 prefix workgroups per KV head beside the decode, so
    each prefix workgroup runs several items in turn.  Every row against the
    oracle, and the allocation-free form gives the same bits."""
    cfg = dataclasses.replace(W.SMALL[4], name="shared-prefix-rounds-d64", batch=1024, hq=64, hkv=32, head_dim=64,
                              num_pages=3300, old_max=40, shared_prefix_tokens=128)
    note(f"shared prefix in rounds {cfg.name}")
    w = W.generate(cfg, DEV)
    kp, vp = gpu_write(gpu, w)
    pages = cfg.shared_prefix_tokens // 16
    out = attend_shared(gpu, w, kp, vp, pages)
    _, _, ref = H.oracle_step(w)
    assert_close(out, ref, "bf16", cfg.name)
    got = torch.full_like(w.q, float("nan"))
    gpu.paged_attention_noalloc(w.q, kp, vp, w.block_table, w.seq_lens, w.query_start_loc, w.scale, got,
                                max_query_len=1, shared_prefix_pages=pages)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().view(torch.int16).numpy(), out.cpu().view(torch.int16).numpy())


@pytest.mark.parametrize("hq,hkv", [(6, 3), (24, 12)])
def test_shared_prefix_decode_groups_below_eight_waves(gpu, hq, hkv):
    """3 and 12 KV heads: a decode workgroup's groups use 6 of its 8 waves
    (the shared-prefix kernel launches 8 for its prefix items), so 2 waves
    only take part in the length scan.  Against the oracle, and the one-call
    write + attention (whose new rows the decode workgroups store, surplus
    waves included) bit for bit against the two calls."""
    cfg = dataclasses.replace(W.SMALL[4], name=f"shared-prefix-{hkv}kv", hq=hq, hkv=hkv, batch=40, num_pages=1024)
    note(f"shared prefix {cfg.name}")
    w = W.generate(cfg, DEV)
    kp, vp = gpu_write(gpu, w)
    pages = cfg.shared_prefix_tokens // 16
    out = attend_shared(gpu, w, kp, vp, pages)
    _, _, ref = H.oracle_step(w)
    assert_close(out, ref, "bf16", cfg.name)
    fkp, fvp = w.key_pool.clone(), w.value_pool.clone()
    fused = torch.full_like(w.q, float("nan"))
    gpu.paged_kv_write_attention(w.k_new, w.v_new, w.slot_mapping, fkp, fvp, w.q, w.block_table, w.seq_lens,
                                 w.query_start_loc, w.scale, fused, max_query_len=1, shared_prefix_pages=pages)
    torch.cuda.synchronize()
    assert torch.equal(fkp.view(torch.uint8), kp.view(torch.uint8)) and torch.equal(fvp.view(torch.uint8), vp.view(torch.uint8))
    assert torch.equal(fused.view(torch.int16), out.view(torch.int16))


@pytest.mark.parametrize("g,d,kv", [(16, 128, "bf16"), (2, 64, "fp8_e4m3fn"), (4, 64, "bf16")])
def test_shared_prefix_geometries(gpu, g, d, kv):
    """The shared-prefix kernel's other instances and group sizes: the largest
    GQA group (16 query heads per KV head, 16 sequences per prefix item), fp8
    pools at head_dim 64, and bf16 at head_dim 64; against the oracle."""
    cfg = dataclasses.replace(W.SMALL[4], name=f"shared-prefix-g{g}-d{d}-{kv}", hq=2 * g, hkv=2, head_dim=d,
                              kv_dtype=kv, batch=48, num_pages=1024, shared_prefix_tokens=96)
    note(f"shared prefix {cfg.name}")
    w = W.generate(cfg, DEV, seed=23)
    kp, vp = gpu_write(gpu, w)
    out = attend_shared(gpu, w, kp, vp, cfg.shared_prefix_tokens // 16)
    _, _, ref = H.oracle_step(w)
    assert_close(out, ref, kv, cfg.name)


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


def test_control_plane_batch_through_the_kernels(gpu):
    """Metadata from the host control plane driving the GPU path: a 3-page
    prompt prefix written once and published in the prefix index; 8 requests
    match it, append their own prompt tokens (one chunked-prefill call over
    the batch), then one decode token each (a shared-prefix decode call).
    Both calls against the oracle on the same pools."""
    note("control plane batch through the kernels")
    from paged_kv_cache_243_amd import host as Hs
    import oracle
    rng = np.random.default_rng(12)
    ps, num_pages, Hkv, Hq, D = 16, 512, 8, 32, 128
    pool = Hs.PagePool(num_pages, ps)
    kp = torch.zeros((num_pages, ps, Hkv, D), dtype=torch.bfloat16, device=DEV)
    vp = torch.zeros_like(kp)
    gen = torch.Generator(device="cpu").manual_seed(5)

    def write(slots):
        n = len(slots)
        k = torch.randn((n, Hkv, D), generator=gen).to(torch.bfloat16).to(DEV)
        v = torch.randn((n, Hkv, D), generator=gen).to(torch.bfloat16).to(DEV)
        gpu.paged_kv_write(k, v, torch.as_tensor(slots, device=DEV), kp, vp)

    ns = 0xABCD
    prefix = np.arange(3 * ps, dtype=np.int32) + 7
    owner = pool.create()
    write(pool.append(owner, len(prefix)))
    pool.prefix_insert(ns, owner, prefix)
    pool.release_seq(owner)
    seqs, rest = [], []
    for r in range(8):
        prompt = np.concatenate([prefix, rng.integers(0, 999, size=int(rng.integers(1, 70))).astype(np.int32)])
        s, matched = pool.prefix_match(ns, prompt)
        assert matched == len(prefix)
        n = len(prompt) - matched
        write(pool.append(s, n))
        pool.confirm(pool.pages(s))
        seqs.append(s)
        rest.append(n)
    max_blocks = 16

    def run(n_new, shared):
        bt, sl, qsl = pool.build_step(seqs, n_new, max_blocks, num_pages - 1)
        T = int(qsl[-1])
        q = torch.randn((T, Hq, D), generator=gen).to(torch.bfloat16).to(DEV)
        out = torch.empty_like(q)
        gpu.paged_attention(q, kp, vp, torch.as_tensor(bt, device=DEV), torch.as_tensor(sl, device=DEV),
                            torch.as_tensor(qsl, device=DEV), D ** -0.5, out, max_query_len=int(max(n_new)),
                            shared_prefix_pages=shared)
        torch.cuda.synchronize()
        ref = oracle.paged_attention(H.S(q), "bf16", H.S(kp), H.S(vp), "bf16", bt, sl, qsl, D ** -0.5)
        return out, ref

    out, ref = run(rest, 0)
    assert_close(out, ref, "bf16", "control plane: prefill continuation")
    for s in seqs:
        write(pool.append(s, 1))
        pool.confirm(pool.pages(s))
    out, ref = run([1] * len(seqs), len(prefix) // ps - 1)   # an even page count
    assert_close(out, ref, "bf16", "control plane: shared-prefix decode")
