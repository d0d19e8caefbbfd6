"""Score rows for the tests of the select's candidate bound (an input
generator: it holds none of the method's arithmetic)."""
import numpy as np


def bound_rows(rows, n, seed):
    """Score rows aimed at the candidate bound of selects with 32 < k <= 64,
    which compares 128 interleaved group maxima (block i in group
    (i mod 64) + 64 * (floor(i / 64) mod 2)); row r is of kind r mod 4:
    0 all scores within 2^16 codes of each other (the bound's bit search
    must run past its first 16 bits); 1 the top 64 groups' maxima at or just
    above 10.3 (whose low 16 code bits are not zero) and their other keys in
    [10.25, 10.3), the 2^16-code band under it, the other groups' keys
    N(0, 1): a bound cut to 16 bits would admit 500 candidates or more, more
    than the select holds (its exact fallback), against 64 for the exact
    bound; 2 one value everywhere; 3 N(0, 1)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, n)).astype(np.float32)
    idx = np.arange(n)
    grp = (idx & 63) + 64 * ((idx >> 6) & 1)
    for r in range(rows):
        kind = r % 4
        if kind == 0:
            x[r] = (1.0 + rng.uniform(0, 2 ** -9, n)).astype(np.float32)
        elif kind == 1:
            top = rng.permutation(128)[:64]
            for j, gi in enumerate(top):
                cols = idx[grp == gi]
                if len(cols) == 0:
                    continue
                x[r, cols] = rng.uniform(10.25, 10.3, len(cols)).astype(np.float32)
                x[r, rng.choice(cols)] = np.float32(10.3 + 0.001 * j)
        elif kind == 2:
            x[r] = np.float32(0.75)
    return x


def counted_rows(nb, k, extras, seed):
    """Block scores of rows whose candidate count at the 64-group bound of
    selects with k <= 32 (block i in group i mod 64) is k + 1 + extras[r]:
    group l < 63 peaks at 100 + l in block l, group 63 holds 163 and the
    pinned newest block nb - 1 (nb = 64 m, the row's whole width), so the
    k-th largest group maximum is 164 - k; the extras are scores in
    [164 - k, 164 - k + 4) placed, in pairs of equal values, in other blocks
    of groups that peak above them; every other score is N(0, 1).  The
    counts straddle the 64 candidates that one wave's lanes hold."""
    assert nb % 64 == 0 and nb >= 512 and 1 <= k <= 32
    rng = np.random.default_rng(seed)
    t0 = 164.0 - k
    rows = []
    for x_count in extras:
        s = rng.standard_normal(nb).astype(np.float32)
        s[:64] = 100.0 + np.arange(64, dtype=np.float32)
        vals = t0 + 0.0625 * (np.arange(x_count) // 2)
        groups = [g for g in range(63) if 100.0 + g > t0 + 4.0]
        assert len(groups) * (nb // 64 - 1) >= x_count
        for j, v in enumerate(vals):
            g = groups[j % len(groups)]
            s[g + 64 * (1 + j // len(groups))] = v
        rows.append(s)
    return np.stack(rows).astype(np.float32)
