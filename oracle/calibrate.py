"""Energy-threshold block selection of calibrated static masks.

[CalibAtt] section 3.1: for one (layer, head, timestep) and each query block r,
the key blocks c are ranked by their attention energy E(r, c) from high to
low, and the smallest leading set S(r) whose energies add up to at least eps
is kept.

Readings:
* eps is a fraction of the row's total energy (the row need not be
  normalised): keep the shortest prefix of the descending order whose running
  sum reaches eps * total;
* the running sums and the total are accumulated in that descending order, in
  float64, one term after another (total = the last running sum), so a GPU
  implementation can take the same decision in the same arithmetic;
* equal energies are ranked by smaller key-block index first.
"""
import numpy as np


def calibrate_row(E_row: np.ndarray, eps: float) -> np.ndarray:
    """uint8 [nKB] keep-flags of one query block's key blocks."""
    E_row = np.asarray(E_row, dtype=np.float64)
    n = E_row.shape[0]
    order = np.lexsort((np.arange(n), -E_row))      # energy descending, then index
    running = np.zeros(n)
    acc = 0.0
    for t, c in enumerate(order):                   # sequential float64 sum
        acc = acc + E_row[c]
        running[t] = acc
    threshold = eps * running[-1]
    count = int(np.argmax(running >= threshold)) + 1
    keep = np.zeros(n, dtype=np.uint8)
    keep[order[:count]] = 1
    return keep


def calibrate_mask(E: np.ndarray, eps: float) -> np.ndarray:
    """uint8 [nQB, nKB] static mask of one head from its energy matrix."""
    return np.stack([calibrate_row(E[r], eps) for r in range(E.shape[0])])
