"""Index invariants the forward kernel's band tiles rely on, checked on the host.

The kernel reads a band tile's bias with one per-lane offset plus immediates and
builds the fused producer's values in a per-row LDS slot; both lean on bounds of
its row / key geometry (work-groups of four or eight 32-row waves, i.e. 128 or 256 rows;
64-key tiles, 128 at head-dim class 16, 32-key tiles checked as well; bottom-right causal
mask, the band
0 <= d < E with d = i + (k_len - q_len) - j). This walks that geometry for random
shapes and checks the bounds:

* over the lanes of any band tile, d0 = i + delta - j0 - 4 * hf >= -35 (so offsets
  formed from one bias row before the wave's first row stay positive);
* the lane's offset in its wave's rows, off = i - wi_lo, lies in [0, 31];
* every element's slot u = BN - 1 - c (c its key offset in the tile) lies in
  [0, BN) and holds d = d_b + off + u with d_b = wi_lo + delta - j0 - (BN - 1);
* the producer's writes (32-d blocks of the MFMA output, first and last block
  sharing slots) fill every slot of a row exactly once.
"""
import numpy as np

from workloads import gen


def acc_row(r, hf):
    return 8 * (r >> 2) + 4 * hf + (r & 3)


def walk(q_len, k_len, gp, causal, E, BN, BM=128):
    """Yield (wave rows, j0, lanes) for every band tile of one (batch, head group)."""
    delta = k_len - q_len
    n_rows = q_len * gp
    for tile in range((n_rows + BM - 1) // BM):
        row0 = tile * BM
        r_last = min(row0 + BM, n_rows) - 1
        i_hi = r_last // gp
        kv_end = min(k_len, i_hi + delta + 1) if causal else k_len
        kv_end = max(kv_end, 0)
        for wave in range(BM // 32):
            w_row = row0 + 32 * wave
            wi_lo = min(w_row, r_last) // gp
            wi_hi = min(w_row + 31, r_last) // gp
            qi = [min(w_row + l, r_last) // gp for l in range(32)]
            for kb in range((kv_end + BN - 1) // BN):
                j0 = kb * BN
                band = (wi_hi + delta - j0 >= 0) and (wi_lo + delta - (j0 + BN - 1) < E)
                if band:
                    yield wi_lo, wi_hi, j0, qi, delta


def check_shape(q_len, k_len, gp, causal, E, BN, BM=128):
    nkb = BN // 32
    for wi_lo, wi_hi, j0, qi, delta in walk(q_len, k_len, gp, causal, E, BN, BM):
        assert wi_hi - wi_lo <= 31
        d_b = wi_lo + delta - j0 - (BN - 1)
        for l32 in range(32):
            i = qi[l32]
            off = i - wi_lo
            assert 0 <= off <= 31
            for hf in range(2):
                assert i + delta - j0 - 4 * hf >= -35
                for kb2 in range(nkb):
                    for r in range(16):
                        u = BN - 1 - kb2 * 32 - acc_row(r, hf)
                        assert 0 <= u < BN
                        d = i + delta - (j0 + kb2 * 32 + acc_row(r, hf))
                        assert d == d_b + off + u
        # the producer's slot writes for every possible offset of a row
        nblk = nkb + 1
        for off in range(32):
            hits = np.zeros(BN, dtype=int)
            for hf in range(2):
                for r in range(16):
                    m = acc_row(r, hf)
                    hits[(m - off) % BN] += 1      # first / last block
                    for b in range(1, nblk - 1):
                        u = 32 * b + m - off
                        assert 0 <= u < BN
                        hits[u] += 1
            assert (hits == 1).all()


def test_band_tile_bounds_random_shapes():
    rng = gen.make_rng(4040)
    for _ in range(60):
        q_len = int(rng.integers(1, 700))
        k_len = int(rng.integers(1, 900))
        gp = int(rng.choice([1, 2, 4, 8]))
        causal = bool(rng.random() < 0.6)
        E = int(rng.choice([128, 256, 384]))
        BN = int(rng.choice([64, 32, 128]))
        BM = int(rng.choice([128, 256]))
        check_shape(q_len, k_len, gp, causal, E, BN, BM)


def test_band_tile_bounds_edges():
    # decode rows, q_len > k_len (rows that see nothing), one-key sequences
    for args in [(1, 5000, 8, True, 128, 32), (300, 40, 1, True, 256, 64), (1, 1, 1, False, 128, 64),
                 (129, 129, 1, True, 128, 64), (64, 2000, 8, False, 384, 64),
                 (257, 257, 1, True, 128, 128), (300, 900, 4, False, 256, 128, 256),
                 (513, 513, 1, True, 256, 64, 256), (1, 3000, 8, True, 384, 128)]:
        check_shape(*args)


def test_visibility_limit_and_band_bounds():
    """The kernel tests a key's visibility as one compare of its in-tile offset
    8 (r >> 2) + (r & 3) against a per-lane limit
        lim = (causal ? min(k_len - 1, i + delta) : k_len - 1) - (j0 + 32 kb2) - 4 hf,
    and a band element (0 <= d < E, valid row) as blo <= c <= bhi with
        c = 32 kb2 + 8 (r >> 2) + (r & 3), d0 = i + delta - j0 - 4 hf,
        bhi = valid ? d0 : -1, blo = d0 - E + 1.
    Both must agree with the direct definitions for every element of every tile."""
    rng = gen.make_rng(5151)
    for _ in range(400):
        q_len = int(rng.integers(1, 300))
        k_len = int(rng.integers(0, 400))
        causal = bool(rng.random() < 0.5)
        E = int(rng.choice([128, 256]))
        nkb = int(rng.choice([1, 2, 4]))
        delta = k_len - q_len
        i = int(rng.integers(0, q_len))
        valid = bool(rng.random() < 0.9)
        j0 = 32 * nkb * int(rng.integers(0, max(1, (k_len + 32 * nkb - 1) // (32 * nkb)) + 1))
        for hf in range(2):
            last = min(k_len - 1, i + delta) if causal else k_len - 1
            d0 = i + delta - j0 - 4 * hf
            bhi, blo = (d0 if valid else -1), d0 - E + 1
            for kb2 in range(nkb):
                lim = last - (j0 + 32 * kb2) - 4 * hf
                for r in range(16):
                    j = j0 + 32 * kb2 + acc_row(r, hf)
                    vis = j < k_len and (not causal or j <= i + delta)
                    assert (8 * (r >> 2) + (r & 3) <= lim) == vis
                    c = 32 * kb2 + 8 * (r >> 2) + (r & 3)
                    d = i + delta - j
                    assert (blo <= c <= bhi) == (valid and 0 <= d < E)
