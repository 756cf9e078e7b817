"""Pins for the oracle's paged pools (CPU only).

The paged functions resolve each shadow (per-pool page map) and then call the
flat definitions.  They are pinned to facts that do not come from themselves:
the row resolution is checked against an enumeration from the physical side
(every mapped page slot names the logical row it holds); with identity shadows
over pools holding the flat layout every result equals the flat oracle's
exactly; shuffling the physical pages (and poisoning pages no shadow names)
changes nothing; a freed page removes exactly its rows (window tokens and C4
rows from the attention, indexer rows from the candidates); and streaming
tokens through the paged append gives the ring append's entries.  A wrong
page index, a dropped offset, a window anchored at the wrong token or a read
of a non-resident page fails one of them.
"""
import numpy as np
import pytest


def _pages(flat, P):
    """[B, N, D] -> pool [B * N/P, P, D] and the identity map [B, N/P]."""
    B, N, D = flat.shape
    pool = flat.reshape(B * (N // P), P, D).copy()
    pmap = np.arange(B * (N // P), dtype=np.int32).reshape(B, N // P)
    return pool, pmap


def _shuffle(pool, pmap, rng, extra=3):
    """The same rows on a permuted page order, plus NaN pages no map names."""
    n = pool.shape[0]
    perm = rng.permutation(n + extra)  # logical page i goes to physical page perm[i]
    out = np.full((n + extra,) + pool.shape[1:], np.nan)
    out[perm[:n]] = pool
    new_map = np.where(pmap >= 0, perm[np.maximum(pmap, 0)], pmap).astype(np.int32)
    return out, new_map


def test_rows_against_physical_enumeration(oracle):
    rng = np.random.default_rng(1)
    P, n_pages, D, B, n_rows = 4, 7, 3, 3, 23
    pool = rng.standard_normal((n_pages, P, D))
    pmap = rng.integers(-2, n_pages + 2, size=(B, 5)).astype(np.int32)  # -1, -2, past the pool
    for b in range(B):
        rows, res = oracle.paged_rows(pool, pmap[b], n_rows, P)
        holder = {}  # from the physical side: slot (page, off) of map entry j holds row j*P + off
        for j, pg in enumerate(pmap[b]):
            if 0 <= pg < n_pages:
                for off in range(P):
                    holder[j * P + off] = (int(pg), off)
        for r in range(n_rows):
            at = oracle.physical_row(pmap[b], r, P, n_pages)
            assert at == holder.get(r)
            assert res[r] == (r in holder)
            if r in holder:
                np.testing.assert_array_equal(rows[r], pool[holder[r]])
            else:
                assert np.isnan(rows[r]).all()


def _decode_case(seed, B=3, S=64, P=16, W=8, D=12, H=4, dI=8, HI=3, k=10):
    rng = np.random.default_rng(seed)
    c = dict(B=B, S=S, P=P, W=W, D=D, H=H, k=k)
    c["q"] = rng.standard_normal((B, H, D))
    c["q_idx"] = rng.standard_normal((B, HI, dI))
    c["k_idx"] = rng.standard_normal((B, S, dI))
    c["comp"] = rng.standard_normal((B, S, D))
    c["pos"] = np.array([37, 5, 60], np.int32)[:B]
    c["swa_len"] = np.array([W, W, 3], np.int32)[:B]
    c["n_cand"] = np.array([S, 40, 9], np.int32)[:B]
    c["comp_len"] = np.array([S, 50, S], np.int32)[:B]
    T = 64  # tokens covered by the SWA shadow
    c["tokens"] = rng.standard_normal((B, T, D))  # SWA latents of every token
    # the flat window ring: slot j holds token pos - n + 1 + j
    ring = np.zeros((B, W, D))
    n_win = np.zeros(B, np.int32)
    for b in range(B):
        n = min(int(c["swa_len"][b]), W, int(c["pos"][b]) + 1)
        for j in range(n):
            ring[b, j] = c["tokens"][b, c["pos"][b] - n + 1 + j]
        n_win[b] = n
    c["ring"], c["n_win"] = ring, n_win
    return c


def _flat_chain(oracle, c, scale=0.3):
    s = oracle.index_scores(c["q_idx"], c["k_idx"], c["n_cand"])
    idx = oracle.topk(s.astype(np.float32), c["n_cand"], c["k"])
    o, l = oracle.attn_decode(c["q"], c["ring"], c["n_win"], c["comp"], c["comp_len"], scale, c["D"],
                              comp_idx=idx)
    return s, idx, o, l


def _paged_chain(oracle, c, kI, kmap, cp, cmap, sp, smap, scale=0.3):
    s = oracle.index_scores_paged(c["q_idx"], kI, kmap, c["P"], c["n_cand"], c["S"])
    idx = oracle.topk(s.astype(np.float32), c["n_cand"], c["k"])
    o, l = oracle.attn_decode_paged(c["q"], sp, smap, c["P"], c["swa_len"], c["pos"], c["W"], cp, cmap,
                                    c["P"], c["comp_len"], idx, c["S"], scale, c["D"])
    return s, idx, o, l


def test_identity_and_shuffled_shadows_equal_flat(oracle):
    c = _decode_case(2)
    kI, kmap = _pages(c["k_idx"], c["P"])
    cp, cmap = _pages(c["comp"], c["P"])
    sp, smap = _pages(c["tokens"], c["P"])
    want = _flat_chain(oracle, c)
    got = _paged_chain(oracle, c, kI, kmap, cp, cmap, sp, smap)
    rng = np.random.default_rng(3)
    shuf = _paged_chain(oracle, c, *_shuffle(kI, kmap, rng), *_shuffle(cp, cmap, rng),
                        *_shuffle(sp, smap, rng))
    for w, g, h in zip(want, got, shuf):
        np.testing.assert_array_equal(np.nan_to_num(g, nan=7.0), np.nan_to_num(w, nan=7.0))
        np.testing.assert_array_equal(np.nan_to_num(h, nan=7.0), np.nan_to_num(w, nan=7.0))


def test_freed_pages_remove_exactly_their_rows(oracle):
    c = _decode_case(4, W=8)
    P = c["P"]
    kI, kmap = _pages(c["k_idx"], P)
    cp, cmap = _pages(c["comp"], P)
    sp, smap = _pages(c["tokens"], P)
    # sequence 0: its window (tokens 30..37) straddles SWA pages 1 and 2; free page 1
    smap[0, 1] = -1
    # sequence 0: free C4 / indexer page 2 (rows 32..47); sequence 2: C4 page 0 only
    kmap[0, 2] = -1
    cmap[0, 2] = -1
    cmap[2, 0] = -1
    sp[P * 1:P * 2] = np.nan  # physical page 1 holds sequence 0's freed page: never read
    s, idx, o, l = _paged_chain(oracle, c, kI, kmap, cp, cmap, sp, smap)
    # indexer rows 32..47 of sequence 0 score NaN and are never chosen (k < resident rows)
    assert np.isnan(s[0, 32:48]).all() and not np.isnan(s[0, :32]).any()
    assert not ((idx[0] >= 32) & (idx[0] < 48)).any()
    # the flat oracle over the surviving rows: window tokens 32..37 only; C4 rows
    # of freed pages dropped from the lists
    ring = c["ring"].copy()
    n_win = c["n_win"].copy()
    ring[0, :6] = c["tokens"][0, 32:38]
    n_win[0] = 6
    fidx = idx.copy()
    fidx[0][(fidx[0] >= 32) & (fidx[0] < 48)] = -1
    fidx[2][(fidx[2] >= 0) & (fidx[2] < 16)] = -1
    wo, wl = oracle.attn_decode(c["q"], ring, n_win, c["comp"], c["comp_len"], 0.3, c["D"], comp_idx=fidx)
    np.testing.assert_allclose(o, wo, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, wl, rtol=0, atol=1e-13)
    # and the window really lost rows: the full-window result differs
    fo, _ = oracle.attn_decode(c["q"], c["ring"], c["n_win"], c["comp"], c["comp_len"], 0.3, c["D"],
                               comp_idx=fidx)
    assert np.abs(fo[0] - o[0]).max() > 1e-6


@pytest.mark.parametrize("shuffle", [False, True])
def test_paged_append_matches_ring_append(oracle, shuffle):
    rng = np.random.default_rng(5 + shuffle)
    B, D, m, P, T, S = 3, 5, 4, 16, 40, 12
    x = rng.standard_normal((T, B, D))
    g = rng.standard_normal((T, B, D)) * 2
    bias = rng.standard_normal((m, D))
    # flat: rings and pool
    rx, rg = np.zeros((B, m, D)), np.zeros((B, m, D))
    pool = np.full((B, S, D), np.nan)
    # paged: SWA shadow over T tokens, C4 shadow over S entries
    smap = np.arange(B * (T // P + 1), dtype=np.int32).reshape(B, -1)
    cmap = np.arange(B * (S // P + 1), dtype=np.int32).reshape(B, -1)
    n_sp, n_cp = smap.size, cmap.size
    if shuffle:
        smap = rng.permutation(n_sp).astype(np.int32).reshape(smap.shape)
        cmap = rng.permutation(n_cp).astype(np.int32).reshape(cmap.shape)
    sx, sg = np.full((n_sp, P, D), np.nan), np.full((n_sp, P, D), np.nan)
    entries = {}
    start = [0, 2, 7]
    for step in range(T):
        pos = np.array([step - start[b] if step >= start[b] else -1 for b in range(B)], np.int32)
        flat = oracle.compress_append(x[step], g[step], bias, rx, rg, pos, pool, m)
        paged = oracle.compress_append_paged(x[step], g[step], bias, sx, sg, pos, smap, cmap, P, P,
                                             n_cp, S, m)
        assert [(b, i) for b, i, _, _ in paged] == flat
        for b, i, at, e in paged:
            assert at == oracle.physical_row(cmap[b], i, P, n_cp)
            entries[(b, i)] = e
    for (b, i), e in entries.items():
        np.testing.assert_array_equal(e, pool[b, i])
    # every stored token sits at its SWA row; idle steps stored nothing
    for b in range(B):
        for t in range(T - start[b]):
            at = oracle.physical_row(smap[b], t, P, n_sp)
            np.testing.assert_array_equal(sx[at], x[t + start[b], b])


def test_paged_append_skips_rows_that_are_not_resident(oracle):
    rng = np.random.default_rng(9)
    B, D, m, P = 2, 3, 4, 16
    bias = rng.standard_normal((m, D))
    smap = np.array([[0, -1], [1, 2]], np.int32)  # sequence 0: tokens 16..31 not resident
    cmap = np.array([[0], [-1]], np.int32)        # sequence 1: no C4 page
    sx, sg = np.zeros((3, P, D)), np.zeros((3, P, D))
    x, gt = rng.standard_normal((B, D)), rng.standard_normal((B, D))
    wrote = oracle.compress_append_paged(x, gt, bias, sx, sg, np.array([19, 3], np.int32), smap,
                                         cmap, P, P, 1, 8, m)
    assert wrote == []  # seq 0: token not stored; seq 1: its entry has no C4 row
    np.testing.assert_array_equal(sx[1, 3], x[1])  # seq 1's token itself is stored
    assert not sx[0].any() and not sx[2].any()     # seq 0 wrote nothing
