"""The decode kernels' work plan, modelled on the CPU (host logic, no GPU).

Every decode workgroup forms the same plan: the batch's pages laid end to
end on a cost axis, each sequence (or sparse unit) charged `overhead` extra
units for its segment's prologue and epilogue, an equal quota Q of cost
units per worker; worker w serves the pages of [w Q, (w + 1) Q).  A sequence
cut by worker boundaries is split into n segments whose fp16 partials go to
n consecutive slots; the worker whose quota holds the sequence's first page
(for an empty sequence: the worker at its cost position, at most the last
one) records n and the first slot for the combine.  Batches of more than 64
sequences are scanned in chunks of 256 (one per workgroup-wide scan), and a
worker stops scanning once it is past its quota -- the last worker scans
every chunk, since the empty sequences at the very end of the axis are its
to record.

This model restates those rules (the formulas of `plan_worker` and of the
kernels' segment walk) and checks the properties the combine depends on:
every page is served exactly once; a split sequence's segments take
distinct slots below the workspace's 2 (G - 1); every sequence, empty or
not, has exactly one owner, and that owner's scan reaches it.  The last
check is the one an early stop of the last worker breaks (trailing empty
sequences past a 256-sequence chunk boundary, total cost a multiple of G);
`test_the_last_worker_must_scan_every_chunk` shows the model catching it.
The GPU side of the same records is `tests/test_gpu_ranges.py`.
"""

import numpy as np
import pytest
import torch

from mla_inputs.workloads import SPECS, _draw_seq_lens

PAGE = 64
CHUNK = 256            # threads of a decode workgroup: sequences per scan chunk
WAVE_PLAN_MAX = 64     # batches up to this size are planned by one wave, unchunked


def plan(lens, G, overhead, min_quota=1):
    """Cost-axis plan: (pages, C = start of each sequence, Q, n = segments,
    slot = first partial slot, owner of each sequence's record)."""
    lens = np.asarray(lens, dtype=np.int64)
    pages = np.where(lens > 0, (lens + PAGE - 1) // PAGE, 0)
    cost_in = np.where(pages > 0, pages + overhead, 0)
    total = int(cost_in.sum())
    Q = max(-(-total // G), min_quota, 1)
    C = np.concatenate([[0], np.cumsum(cost_in)[:-1]]).astype(np.int64)
    A = C + overhead
    E = A + pages
    n = np.where(pages > 0, (E - 1) // Q - A // Q + 1, 0)
    slot = np.concatenate([[0], np.cumsum(np.where(n > 1, n, 0))[:-1]]).astype(np.int64)
    owner = np.where(pages > 0, A // Q, np.minimum(C // Q, G - 1))
    return pages, C, Q, n, slot, owner


def chunks_scanned(lens, G, overhead, worker, last_worker_scans_all=True):
    """Chunks of the batch the worker's workgroup-wide scan visits."""
    B = len(lens)
    if B <= WAVE_PLAN_MAX:
        return 1
    _, _, Q, _, _, _ = plan(lens, G, overhead)
    w_hi = (worker + 1) * Q
    carry = 0
    visited = 0
    for base in range(0, B, CHUNK):
        visited += 1
        for L in lens[base:base + CHUNK]:
            carry += (-(-L // PAGE) + overhead) if L > 0 else 0
        if carry >= w_hi and (worker < G - 1 or not last_worker_scans_all):
            break
    return visited


def walk(lens, G, overhead):
    """Every worker's segments, as the kernels' segment loop forms them:
    list of (worker, sequence, first page, end page, slot or -1, the
    sequence's segment count as that worker computes it)."""
    pages, C, Q, n, slot_of, _ = plan(lens, G, overhead)
    segs = []
    for w in range(G):
        w_lo, w_hi = w * Q, (w + 1) * Q
        cand = [b for b in range(len(lens)) if pages[b] > 0 and C[b] + overhead + pages[b] > w_lo]
        if not cand:
            continue
        cost, slot_base = int(C[cand[0]]), int(slot_of[cand[0]])
        for b in range(cand[0], len(lens)):
            if pages[b] == 0:
                continue
            A = cost + overhead
            E = A + int(pages[b])
            if A >= w_hi:
                break
            cost = E
            nb = (E - 1) // Q - A // Q + 1
            base = slot_base
            slot_base += nb if nb > 1 else 0
            if E <= w_lo:
                continue
            split = max(w_lo, A) // Q - A // Q
            segs.append((w, b, max(w_lo, A) - A, min(w_hi, E) - A, base + split if nb > 1 else -1, nb))
    return segs


def check_plan(lens, G, overhead):
    pages, C, Q, n, slot_of, owner = plan(lens, G, overhead)
    slots_cap = 2 * (G - 1) if G > 1 else 1
    covered = [np.zeros(int(p), dtype=np.int64) for p in pages]
    per_seq = [[] for _ in lens]
    for w, b, p_lo, p_hi, slot, nb in walk(lens, G, overhead):
        assert 0 <= p_lo < p_hi <= pages[b], (w, b, p_lo, p_hi)
        assert nb == n[b], (w, b, nb, n[b])
        covered[b][p_lo:p_hi] += 1
        per_seq[b].append((w, slot))
    for b in range(len(lens)):
        # every page once, by n[b] workers in order
        assert (covered[b] == 1).all(), (b, covered[b].min(initial=1), covered[b].max(initial=1))
        assert len(per_seq[b]) == n[b], (b, len(per_seq[b]), n[b])
        ws = [w for w, _ in per_seq[b]]
        assert ws == sorted(ws)
        slots = [s for _, s in per_seq[b]]
        if n[b] > 1:
            assert slots == list(range(int(slot_of[b]), int(slot_of[b]) + int(n[b]))), (b, slots)
            assert slot_of[b] + n[b] <= slots_cap, (b, slot_of[b], n[b], slots_cap)
        else:
            assert slots == [-1] * int(n[b])
        # one owner, inside the grid, whose scan reaches the sequence; the
        # owner of a non-empty sequence also serves its first page
        assert 0 <= owner[b] < G, (b, owner[b])
        assert chunks_scanned(lens, G, overhead, int(owner[b])) > b // CHUNK, (b, owner[b])
        if pages[b] > 0:
            assert per_seq[b][0][0] == owner[b]
    # split slots in use fit the workspace
    assert int(np.where(n > 1, n, 0).sum()) <= slots_cap


def _lens_of(name):
    spec = SPECS[name]
    gen = torch.Generator(device="cpu")
    gen.manual_seed(spec.seed)
    lens = [int(x) for x in _draw_seq_lens(spec, gen)]
    if spec.topk:
        lens = [spec.topk] * (spec.batch * spec.s_q)    # sparse units: topk tokens each
    return lens


@pytest.mark.parametrize("name", ["single_1k", "paged_b32", "long_ctx_b4", "fp8_b64", "fp8_b64_d512", "fp4_b64",
                                  "mtp2_b128", "sparse_topk2048_b64", "sparse_fp8_topk2048_b64"])
@pytest.mark.parametrize("G", [1, 3, 16, 128, 256, 300])
def test_plan_of_the_workloads(name, G):
    for overhead in (1, 3, 5):
        check_plan(_lens_of(name), G, overhead)


def test_plan_of_random_batches():
    rng = np.random.default_rng(7)
    for _ in range(150):
        B = int(rng.choice([1, 2, 5, 63, 64, 65, 255, 256, 257, 300, 700]))
        lens = rng.integers(1, 5000, B)
        lens[rng.random(B) < 0.2] = 0                        # empty sequences anywhere
        if rng.random() < 0.3:
            lens[-int(rng.integers(1, B + 1)):] = 0          # a run of empties at the end
        G = int(rng.choice([1, 2, 7, 64, 250, 256, 1000]))
        check_plan([int(x) for x in lens], G, int(rng.integers(1, 6)))


def test_edge_batches():
    for G in (1, 3, 250, 256):
        check_plan([0] * 300, G, 3)                          # nothing visible at all
        check_plan([100] * 250 + [0] * 50, G, 3)             # total cost a multiple of G for G = 1, 250
        check_plan([0] * 257 + [64], G, 3)                   # the only sequence past the first chunk
        check_plan([1] * 1000, G, 3)


def test_the_last_worker_must_scan_every_chunk():
    # the same batch with the last worker stopping like the others: the
    # trailing empty sequences 256 .. 299 (cost position = total = G Q) are
    # owned by worker G - 1, which would stop after the first chunk
    lens = [100] * 250 + [0] * 50
    for G in (1, 250):
        _, _, Q, _, _, owner = plan(lens, G, 3)
        assert 250 * (2 + 3) == G * Q                        # total is a multiple of G
        assert owner[299] == G - 1
        assert chunks_scanned(lens, G, 3, G - 1) == 2
        assert chunks_scanned(lens, G, 3, G - 1, last_worker_scans_all=False) == 1
