"""Host checks of the parity helpers themselves (no GPU)."""
import numpy as np

import oracle
from parity_utils import tile_cover_sample


def test_tile_cover_sample_touches_every_block_and_last_row():
    rng = np.random.default_rng(0)
    for N, E, k, policy, cap in ((2048, 64, 8, oracle.DROPLESS, -1),
                                 (1500, 8, 2, oracle.DROPLESS, -1),
                                 (3000, 16, 1, oracle.DROP, 150)):
        l = (rng.standard_normal((N, E)) - 0.3 * np.log1p(np.arange(E))).astype(np.float32)
        r = oracle.route(l, k, k, True)
        d = oracle.dispatch(r["cand_ids"], r["cand_scores"], r["gates"], E, k, policy, cap)
        sample, cov = tile_cover_sample(d["row_of"], d["offsets"])
        assert cov["blocks"] == cov["blocks_total"]
        rows = set(d["row_of"][sample].ravel().tolist())
        off = d["offsets"]
        for e in range(E):
            for b in range(off[e], off[e + 1], 128):
                assert rows & set(range(b, min(b + 128, off[e + 1]))), (e, b)
            if off[e + 1] > off[e]:
                assert off[e + 1] - 1 in rows
        assert len(sample) == len(np.unique(sample)) <= cov["blocks_total"] + E
