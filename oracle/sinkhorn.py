"""Sinkhorn-style balancing of one tile (oracle; test infrastructure only).

SJ-KVaRN, section 2.2 "Balancing": a 128-token by 256-channel tile is
rescaled by alternating row and column passes until every row and column has
a similar spread; the balancing is done in the log domain, runs 16 passes and
keeps the final scales (the KVarN reference configuration runs 8).  Section 11
names it "Sinkhorn variance balancing" and credits Sinkhorn and Knopp (1967)
for matrix balancing; it lists "scale absorption" among KVarN's parts.  The
KV Cache Precision Tail article calls the same step "iterative variance
normalization".

Readings:
* "spread" is the population standard deviation (mean subtracted), read from
  "variance balancing".  It is computed about the first element of the row
  or column (sigma of y equals sigma of y - y_first), so that a row or column
  whose values are all equal has a spread of exactly zero;
* a "pass" is one sweep over all rows or over all columns, rows first (the
  order of the words "row and column"), so 16 passes = 8 row + 8 column sweeps;
* log-domain state: lr (per row) and lc (per column), with
  y_ij = x_ij * exp(-lr_i - lc_j); a row pass sets lr_i += ln sigma_i where
  sigma_i is the spread of row i of y; a column pass does the same for lc;
* a row or column whose spread is zero cannot be balanced and keeps its scale
  (its log scale is not updated): an all-zero tile keeps unit scales, and so
  do the columns of a tile of repeated tokens.  "Zero" is decided by float64
  arithmetic alone: sigma <= 2^-40 * rms(y).  Values that are equal in exact
  arithmetic can differ after rounding in float64 -- y carries the rounding of
  one exp and one product, ~2^-52 relative, e.g. rows that are power-of-two
  multiples of one another leave columns equal up to an ulp or two after the
  row pass -- so their computed spread is at most a few 2^-52 of their RMS;
  2^-40 sits 2^10 above that, and every spread at or above it is balanced as
  the unguarded passes would balance it;
* scale absorption: the row factors are not stored (each row gets its own
  rounding scale and zero point afterwards, which absorbs them); the column
  factors are kept as C_j = fp16(exp(lc_j)) after centring lc to mean zero
  (the gauge) and clamping it to [-9, 9] (the clamp and the zero-spread rule
  are this implementation's guards; the pages state neither);
* "keep the final scales" (SJ-KVaRN), not "keep the best scales seen".
Arithmetic is float64 throughout.
"""
from __future__ import annotations

import numpy as np

ZERO_SPREAD_REL = 2.0 ** -40  # sigma / rms(y) at or below which a spread counts as zero
LC_CLAMP = 9.0


def spread(y, axis: int):
    """(sigma, rms) of y along `axis`: the population standard deviation,
    taken about the first element, and the root mean square."""
    first = np.take(y, [0], axis=axis)
    sigma = np.std(y - first, axis=axis)
    rms = np.sqrt(np.mean(y * y, axis=axis))
    return sigma, rms


def balance(x, passes: int):
    """Balance a (rows, cols) tile.  Returns a dict with
    lr (rows,), lc_raw (cols,), lc (centred and clamped, cols,), C (fp16, cols,)."""
    x = np.asarray(x, np.float64)
    rows, cols = x.shape
    lr = np.zeros(rows)
    lc = np.zeros(cols)
    for p in range(passes):
        y = x * np.exp(-lr[:, None] - lc[None, :])
        ax = 1 if p % 2 == 0 else 0
        sigma, rms = spread(y, ax)
        upd = sigma > ZERO_SPREAD_REL * rms
        step = np.where(upd, np.log(np.where(upd, sigma, 1.0)), 0.0)
        if ax == 1:
            lr = lr + step
        else:
            lc = lc + step
    lc_c = np.clip(lc - lc.mean(), -LC_CLAMP, LC_CLAMP)
    C = np.exp(lc_c).astype(np.float16)
    return {"lr": lr, "lc_raw": lc, "lc": lc_c, "C": C}
