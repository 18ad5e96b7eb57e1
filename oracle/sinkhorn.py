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
  "variance balancing";
* a "pass" is one sweep over all rows or over all columns, rows first (the
  order of the words "row and column"), so 16 passes = 8 row + 8 column sweeps;
* log-domain state: lr (per row) and lc (per column), with
  y_ij = x_ij * exp(-lr_i - lc_j); a row pass sets lr_i += ln sigma_i where
  sigma_i is the spread of row i of y; a column pass does the same for lc;
* a row or column whose spread is zero cannot be balanced and keeps its scale
  (its log scale is not updated): an all-zero tile keeps unit scales.  Adding
  ln of a floor instead would grow the log scales of such a row or column by
  ~69 per pass until exp overflows.  "Zero" is sigma <= 1e-30 or
  sigma^2 <= 2^-16 mean(y^2) (a spread under 1/256 of the RMS): the fp32
  one-pass form E[y^2] - mean^2 with 22-bit factors errs by up to ~2^-20
  mean(y^2), so below that a spread cannot be told from zero and a row or
  column of identical values (repeated tokens) must read as constant;
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

LOG_FLOOR = 1e-30
ZERO_SPREAD_REL = 2.0 ** -16  # sigma^2 / mean(y^2) at or below which a spread counts as zero
LC_CLAMP = 9.0


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
        sigma = y.std(axis=ax)
        upd = (sigma > LOG_FLOOR) & (sigma * sigma > ZERO_SPREAD_REL * (y * y).mean(axis=ax))
        step = np.where(upd, np.log(np.maximum(sigma, LOG_FLOOR)), 0.0)
        if ax == 1:
            lr = lr + step
        else:
            lc = lc + step
    lc_c = np.clip(lc - lc.mean(), -LC_CLAMP, LC_CLAMP)
    C = np.exp(lc_c).astype(np.float16)
    return {"lr": lr, "lc_raw": lc, "lc": lc_c, "C": C}
