"""Index probes (closed form C4): aim every (query row, query head) at one
key and check that the output row is that key's value row.

The query of (row t, head hq) is set to c times the dequantised K row of its
target key (head hq / G), which gives that key a logit larger than every other
visible key's by a wide margin (about 6c logit units at c = 16; every other
weight is then below e^-60).  The output row is that key's value row, up to
the bf16 rounding of the output, whatever else the sequence holds.  A key the
kernel fetched from a page the sequence does not own, or not at all, or that
the causal mask hid because its page was placed at the wrong position, leaves
the row off by O(1).  (Reordering a sequence's own pages among positions that
every row sees changes no output: attention does not depend on the order of
the keys it sees, so that is not an error.)

Rows are gathered from the pools with torch indexing and widened with torch's
casts; nothing here calls the HIP library or the oracle, which are passed in
as ``attend``.
"""
import numpy as np
import torch

from tests.gpu_helpers import as_f64, note
from tests.helpers import S

C_PROBE = 16.0


def rows_of(w):
    """Sequence of every packed query row and the row's absolute position."""
    qsl, lens = S(w.query_start_loc), S(w.seq_lens)
    seq = np.repeat(np.arange(len(lens)), np.diff(qsl))
    pos = np.empty(qsl[-1], dtype=np.int64)
    for b in range(len(lens)):
        n = qsl[b + 1] - qsl[b]
        pos[qsl[b]:qsl[b + 1]] = lens[b] - n + np.arange(n)
    return seq, pos


def gather_rows(w, pool, scale, slots, heads):
    """fp32 rows pool[slot, head] (dequantised for fp8) on the GPU."""
    cfg = w.cfg
    flat = pool.view(-1, cfg.hkv, cfg.head_dim)
    s = torch.as_tensor(slots.reshape(-1), device=pool.device)
    h = torch.as_tensor(heads.reshape(-1), device=pool.device)
    rows = flat[s, h]
    if cfg.kv_dtype == "fp8_e4m3fn":
        return rows.view(torch.float8_e4m3fn).float() * scale[h].view(-1, 1)
    return rows.float()


def probe_run(w, kp, vp, targets, attend, c=C_PROBE):
    """Aim query (row t, head hq) at key position targets[t, hq] of its
    sequence; run ``attend(q)`` and return (out, expected V rows, probed page
    ids), expected in fp64 on the host."""
    cfg = w.cfg
    G = cfg.hq // cfg.hkv
    seq, pos = rows_of(w)
    assert (targets >= 0).all() and (targets <= pos[:, None]).all(), "a target must be visible to its row"
    bt = S(w.block_table)
    pages = bt[seq[:, None], targets // 16]
    slots = pages * 16 + targets % 16
    heads = np.broadcast_to(np.arange(cfg.hq) // G, targets.shape)
    k = gather_rows(w, kp, w.k_scale, slots, heads)
    q = (c * k).to(w.q.dtype).view(w.q.shape).contiguous()
    want = gather_rows(w, vp, w.v_scale, slots, heads).double().cpu().numpy().reshape(w.q.shape)
    out = attend(q)
    return as_f64(out), want, pages


def assert_probes(got, want, what, quiet=False):
    """Each output row equals its probed value row up to the output's bf16
    rounding (half an ulp, at most 2^-8 relative: bf16 keeps 7 explicit
    mantissa bits; bf16 value rows come back exactly, fp8 rows times their
    scale are rounded once), with a factor 2 of margin, and the e^-gap weight
    of the other keys; a missed key is off by O(1).  Returns the worst
    error / bound."""
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - want)
    bound = np.abs(want) * 2.0 ** -7 + 1e-3
    bad = err > bound
    worst = float((err / bound).max()) if err.size else 0.0
    if not quiet or bad.any():
        note(f"{what}: {want.shape[0] * want.shape[1]} probes, worst error {err.max():.3e}, "
             f"worst error / bound {worst:.3f}")
    if bad.any():
        t, hq, d = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: row {t} head {hq} dim {d}: got {got[t, hq, d]}, want {want[t, hq, d]} "
                             f"({int(bad.any(axis=2).sum())} probes missed)")
    return worst


def decode_runs(w) -> int:
    """Runs of decode_targets that together probe every page of every sequence."""
    pages = -(-S(w.seq_lens).astype(np.int64) // 16)
    return int(-(-pages.max() // w.cfg.hq)) if len(pages) else 0


def decode_targets(w, run, rng):
    """[B, Hq] targets for decode rows: run r aims head k of every sequence at
    its logical page (r * Hq + k) mod (its page count), at a random row of that
    page (on the last page, the sequence's last position: the key this step
    wrote), so runs 0 .. decode_runs(w) - 1 probe every page."""
    lens = S(w.seq_lens)
    B, Hq = len(lens), w.cfg.hq
    out = np.empty((B, Hq), dtype=np.int64)
    for b in range(B):
        L = int(lens[b])
        n = -(-L // 16)
        j = (run * Hq + np.arange(Hq)) % n
        out[b] = np.where(j == n - 1, L - 1, np.minimum(j * 16 + rng.integers(0, 16, Hq), L - 1))
    return out


def prefill_runs(w) -> int:
    """Runs of prefill_targets that together probe every page of every
    sequence: the page-cycling head walks ceil(pages / rows) pages per row."""
    lens, qsl = S(w.seq_lens), S(w.query_start_loc)
    n = np.diff(qsl)
    pages = -(-lens // 16)
    need = [-(-int(pages[b]) // int(n[b])) for b in range(len(n)) if n[b] > 0]
    return max([2] + need)


def prefill_targets(w, rng, run=0):
    """[T, Hq] targets for prefill rows, by head: a page cycled over the
    rows (row i of a sequence takes its page (i + run * n_b) mod (pages it
    sees), so prefill_runs(w) runs reach every page), the old context, the
    new chunk (up to the row itself), a tile edge (32-key boundaries, which
    hold every key-split chunk edge), the diagonal, or key 0 / anywhere."""
    seq, pos = rows_of(w)
    lens, qsl = S(w.seq_lens), S(w.query_start_loc)
    n_b = np.diff(qsl)[seq]
    P = (lens - np.diff(qsl))[seq]                       # old context of each row's sequence
    i = np.arange(len(pos)) - qsl[seq]                   # row index inside its sequence
    T, Hq = len(pos), w.cfg.hq
    out = np.empty((T, Hq), dtype=np.int64)
    for hq in range(Hq):
        kind = hq % 6
        anywhere = (rng.random(T) * (pos + 1)).astype(np.int64)
        if kind == 0:                                     # every page, cycled over the rows
            j = (i + run * n_b) % (pos // 16 + 1)
            t = j * 16 + rng.integers(0, 16, T)
        elif kind == 1:                                   # the new chunk, up to the row
            t = P + (rng.random(T) * (pos - P + 1)).astype(np.int64)
        elif kind == 2:                                   # a tile's first or last key
            edge = (rng.random(T) * (pos // 32 + 1)).astype(np.int64) * 32 + rng.integers(0, 2, T) * 31
            t = np.where(edge <= pos, edge, pos)
        elif kind == 3:
            t = pos.copy()                                # the diagonal
        elif kind == 4:                                   # the old context, else anywhere
            t = np.where(P > 0, (rng.random(T) * np.maximum(P, 1)).astype(np.int64), anywhere)
        else:
            t = np.where(rng.random(T) < 0.25, 0, anywhere)
        out[:, hq] = np.minimum(t, pos)
    return out
