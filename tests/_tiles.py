"""Which permuted rows land in which output tile of the grouped GEMM's large
tile configuration, so that full-size tests can sample tokens that reach
every m-tile of every expert and every row of a tile split along K.

Host-side bookkeeping of the launch's tile order only (no step of the layer
is computed here): tiles are ordered (expert, group of GM m-tiles, n-tile,
m-tile within the group); a persistent grid of G blocks takes them in rounds
of G, and the tiles after the last full round are the ones split along K."""
import numpy as np

BM = 256   # rows of a large output tile
GM = 8     # m-tiles per group in the tile order


def tile_order(offsets, ntn):
    """List of (expert, m-tile) of every tile, in launch order."""
    out = []
    E = len(offsets) - 1
    for e in range(E):
        rows = int(offsets[e + 1] - offsets[e])
        mt = (rows + BM - 1) // BM
        for g0 in range(0, mt, GM):
            gs = min(GM, mt - g0)
            for _n in range(ntn):
                for m in range(g0, g0 + gs):
                    out.append((e, m))
    return out


def mtile_rows(offsets, e, m):
    lo = int(offsets[e]) + m * BM
    return np.arange(lo, min(lo + BM, int(offsets[e + 1])))


def covering_rows(offsets, ntns, G):
    """Permuted rows to check: the first and last row of every m-tile of
    every expert, and every row of the smallest m-tile among the tiles of the
    last, partly filled round (the K-split tiles) of each GEMM (one n-tile
    count per GEMM in ntns)."""
    rows = set()
    E = len(offsets) - 1
    for e in range(E):
        n = int(offsets[e + 1] - offsets[e])
        for m in range((n + BM - 1) // BM):
            r = mtile_rows(offsets, e, m)
            rows.update((int(r[0]), int(r[-1])))
    for ntn in ntns:
        order = tile_order(offsets, ntn)
        full = len(order) - len(order) % G
        tail = {t for t in order[full:]}
        if tail:
            e, m = min(tail, key=lambda em: len(mtile_rows(offsets, *em)))
            rows.update(int(r) for r in mtile_rows(offsets, e, m))
    return np.array(sorted(rows), np.int64)


def covering_tokens(offsets, src_token, ntns, G, extra=()):
    rows = covering_rows(offsets, ntns, G)
    toks = set(int(t) for t in np.asarray(src_token)[rows])
    toks.update(int(t) for t in extra)
    return np.array(sorted(toks), np.int32)
