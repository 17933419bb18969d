"""Pins of the oracle's router (CPU only): gate logits x . Wg^T, top-k with
ties to the lower expert id, softmax over the k selected logits.

Checked against numpy's fp64 matmul and stable lexicographic sort, PyTorch's
softmax, closed forms (all-zero input, exact ties from duplicated gate rows,
k = E) and invariants; two planted router mistakes (ties to the higher id,
softmax over all E logits) must fail the pins.
"""
import numpy as np
import pytest
import torch

import oracle
import synth


@pytest.fixture(autouse=True)
def _clean(oracle_lib):
    oracle.set_mutation(0)
    yield
    oracle.set_mutation(0)


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)


def _case(T, H, E, seed, dup=None):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    wg = (torch.randn(E, H, generator=g) * 0.02).to(torch.bfloat16)
    if dup:
        for a, b in dup:                       # identical gate rows -> exactly equal logits
            wg[b] = wg[a]
    return x, wg


def _reference(x, wg, k):
    """numpy fp64 matmul for the logits, a stable lexicographic sort on
    (-logit, id) for the selection, torch.softmax over the selected logits."""
    lg = x.float().double().numpy() @ wg.float().double().numpy().T
    E = lg.shape[1]
    order = np.lexsort((np.broadcast_to(np.arange(E), lg.shape), -lg), axis=1)[:, :k]
    sel = np.take_along_axis(lg, order, axis=1)
    w = torch.softmax(torch.from_numpy(sel), dim=1).numpy()
    return order.astype(np.int32), w, lg


def _router_agrees(T, H, E, k, seed, dup=None) -> bool:
    x, wg = _case(T, H, E, seed, dup)
    ids, w, lg = oracle.router(x, wg, k)
    rid, rw, rlg = _reference(x, wg, k)
    if not np.all(np.abs(lg - rlg) <= 1e-12 * np.abs(rlg).max()):
        return False
    # the numpy logits sum in another order: compare ids where no two of the
    # first k + 1 ranked logits lie within that rounding of each other
    srt = -np.sort(-rlg, axis=1)[:, : min(k + 1, E)]
    gap = np.abs(np.diff(srt, axis=1)).min(axis=1) if srt.shape[1] > 1 else np.full(T, np.inf)
    clear = gap > 1e-10
    if dup:
        clear[:] = True                        # duplicated rows tie exactly on both sides
    if not np.array_equal(ids[clear], rid[clear]):
        return False
    return bool(np.all(np.abs(w - rw) <= 1e-6 * np.abs(rw) + 1e-12))


CASES = [(33, 256, 8, 2, 1), (17, 512, 64, 8, 2), (9, 384, 256, 8, 3), (5, 128, 72, 16, 4), (4, 256, 5, 5, 5)]


@pytest.mark.parametrize("T,H,E,k,seed", CASES)
def test_router_matches_library_routines(T, H, E, k, seed):
    assert _router_agrees(T, H, E, k, seed)


def test_router_exact_ties_go_to_the_lower_id():
    """Duplicated gate rows give bit-equal logits: the lower expert id is
    taken first, then the next one."""
    dup = [(3, 40), (7, 11), (11, 12)]
    assert _router_agrees(31, 256, 64, 8, 6, dup=dup)
    x, wg = _case(31, 256, 64, 6, dup)
    ids, _, lg = oracle.router(x, wg, 8)
    for t in range(31):
        row = list(ids[t])
        for a, b in dup:
            if a in row and b in row:
                assert row.index(a) < row.index(b)


def test_router_zero_input_and_k_equals_e():
    """All-zero tokens: every logit is 0, so the ids are 0..k-1 in order and
    each weight is 1/k; with k = E the weights are the full softmax."""
    x = torch.zeros(3, 128, dtype=torch.bfloat16)
    wg = (torch.randn(16, 128, generator=torch.Generator().manual_seed(7)) * 0.02).to(torch.bfloat16)
    ids, w, _ = oracle.router(x, wg, 4)
    assert np.array_equal(ids, np.tile(np.arange(4, dtype=np.int32), (3, 1)))
    assert np.all(w == np.float32(0.25))
    x, wg = _case(6, 256, 12, 8)
    ids, w, lg = oracle.router(x, wg, 12)
    full = torch.softmax(torch.from_numpy(lg), dim=1).numpy()
    assert np.allclose(np.take_along_axis(full, ids.astype(np.int64), axis=1), w, rtol=1e-6, atol=0)
    assert np.all(np.diff(np.take_along_axis(lg, ids.astype(np.int64), axis=1), axis=1) <= 0)


def test_router_weights_are_a_distribution():
    wl = synth.WORKLOADS["decode_fp8"].with_shape(H=512, E=64)
    x = synth.gen_x(20, wl.H, 3, wl.wid)
    ids, w, _ = oracle.router(x, synth.gen_gate(wl, 3), 8)
    assert np.allclose(w.astype(np.float64).sum(axis=1), 1.0, atol=1e-6)
    assert np.all(w > 0) and np.all(np.diff(w, axis=1) <= 0)
    assert all(len(set(r)) == 8 for r in ids.tolist())


@pytest.mark.parametrize("mutation", [7, 8])
def test_planted_router_mistakes_are_caught(mutation):
    ok = lambda: _router_agrees(*CASES[0]) and _router_agrees(31, 256, 64, 8, 6, dup=[(3, 40), (7, 11), (11, 12)])
    assert ok()
    oracle.set_mutation(mutation)
    try:
        assert not ok(), f"mutation {mutation} slipped through"
    finally:
        oracle.set_mutation(0)
