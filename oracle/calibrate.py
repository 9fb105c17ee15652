"""Offline calibration of static block masks ([CalibAtt] section 3.1).

* Block energy: E(r, c) of one head is the attention weight that the queries
  of query block r give to the keys of key block c.
* Energy threshold: for one (layer, head, timestep) and each query block r,
  the key blocks c are ranked by their attention energy E(r, c) from high to
  low, and the smallest leading set S(r) whose energies add up to at least
  eps is kept.
* The threshold eps(t) follows an exponential decay over the denoising steps,
  from about 0.99 at the first step to about 0.84 at the last.
* Candidate masks of several prompts are merged by the frequency with which
  each block is kept, against a threshold rho = 0.5.

Readings:
* the energy of a block pair is the sum of the dense softmax weights
  p_ij = exp(s_ij - lse_i) over its queries i and keys j (the "share of the
  attention energy" the pages count blocks by), so a row of E sums to the
  number of queries in block r;
* the decay of eps(t) is geometric between its two end values:
  eps(t) = eps_first * (eps_last / eps_first) ** (t / (T - 1)) for steps
  t = 0 .. T-1 (a single step takes eps_first);
* a block survives the merge when the fraction of candidate masks that keep it
  reaches rho (count / n >= rho, in float64);
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


def block_energy(q: np.ndarray, k: np.ndarray, scale: float, B: int) -> np.ndarray:
    """float64 [nQB, nKB] block energies of one head: E[r, c] = sum of the dense
    softmax weights of the queries of block r over the keys of block c."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    N = q.shape[0]
    nB = -(-N // B)
    s = (q @ k.T) * scale
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    E = np.zeros((nB, nB))
    for r in range(nB):
        for c in range(nB):
            E[r, c] = p[r * B:(r + 1) * B, c * B:(c + 1) * B].sum()
    return E


def eps_schedule(t: int, T: int, eps_first: float = 0.99, eps_last: float = 0.84) -> float:
    """Energy threshold of denoising step t of T (exponential decay)."""
    if T <= 1:
        return float(eps_first)
    return float(eps_first * (eps_last / eps_first) ** (t / (T - 1)))


def aggregate_masks(masks: np.ndarray, rho: float = 0.5) -> np.ndarray:
    """uint8 mask keeping the blocks kept by at least a fraction rho of the
    candidate masks (axis 0)."""
    masks = np.asarray(masks) != 0
    n = masks.shape[0]
    freq = masks.sum(axis=0).astype(np.float64) / float(n)
    return (freq >= rho).astype(np.uint8)
