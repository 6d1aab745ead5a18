"""Parity rule between the HIP path and the fp64 oracle.

Two bars are applied to every hidden row:

1. The stated bar: |logit_gpu - logit_oracle| <= 2e-2, and the returned id
   equals the oracle's id wherever the oracle's top-2 gap exceeds 1e-2.
   Where the gap is at most 1e-2 and the ids differ, the oracle logit of the
   GPU's row must be within 2e-2 of the maximum (the GPU's answer is one of
   the near-tied correct answers).

2. A bound derived from the arithmetic, independent of summation order.
   bf16 x bf16 products are exact in fp32 and the kernels add K of them in
   fp32 with round-to-nearest, so any order of additions is within
   (K + 1) * 2**-24 * sum_k |h_k w_k| of the exact sum.  With B(r) that
   bound for row r: the GPU logit of its row r_g is within B(r_g) of the
   oracle's, the GPU's row can trail the true maximum by at most
   B(r_g) + B(r_best), and if the gap exceeds that sum the ids must match.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

import oracle

LOGIT_TOL = 2e-2
GAP_EXEMPT = 1e-2
U32 = 2.0 ** -24


@dataclass
class ParityStats:
    rows: int = 0
    exempt: int = 0          # near-tie rows where the GPU chose another valid id
    max_err: float = 0.0     # max |gpu logit - oracle logit of the GPU's row|
    max_err_over_bound: float = 0.0

    def add(self, other: "ParityStats") -> None:
        self.rows += other.rows
        self.exempt += other.exempt
        self.max_err = max(self.max_err, other.max_err)
        self.max_err_over_bound = max(self.max_err_over_bound, other.max_err_over_bound)


def _row_bound(h_row: np.ndarray, w_row: np.ndarray, k: int) -> float:
    return (k + 1) * U32 * float(np.abs(h_row * w_row).sum()) + 1e-30


def check(h_bits, w_bits, d2t, gpu_id, gpu_logit, res=None) -> ParityStats:
    """Assert the parity rule for one call; returns statistics."""
    h_bits = np.asarray(h_bits)
    w_bits = np.asarray(w_bits)
    gpu_id = np.asarray(gpu_id).astype(np.int64)
    gpu_logit = np.asarray(gpu_logit).astype(np.float64)
    m, k = h_bits.shape
    r = w_bits.shape[0]
    if res is None or res.logits is None:
        res = oracle.oracle_project_argmax(h_bits, w_bits, d2t, keep_logits=True)
    if d2t is None:
        rows = gpu_id.copy()
    else:
        d2t = np.asarray(d2t).astype(np.int64)
        pos = np.full(int(d2t.max()) + 1, -1, dtype=np.int64)
        pos[d2t] = np.arange(r)
        assert np.unique(d2t).size == r, "parity check needs a d2t without duplicates"
        rows = np.where((gpu_id >= 0) & (gpu_id < pos.size), pos[np.clip(gpu_id, 0, pos.size - 1)], -1)
    h = oracle.bf16_bits_to_f64(h_bits)
    st = ParityStats(rows=m)
    for i in range(m):
        assert 0 <= rows[i] < r, f"row {i}: GPU id {gpu_id[i]} is not a projected row"
        lg = res.logits[i, rows[i]]
        wg = oracle.bf16_bits_to_f64(w_bits[rows[i]])
        wb = oracle.bf16_bits_to_f64(w_bits[res.idx[i]])
        b_g = _row_bound(h[i], wg, k)
        b_best = _row_bound(h[i], wb, k)
        err = abs(gpu_logit[i] - lg)
        st.max_err = max(st.max_err, err)
        st.max_err_over_bound = max(st.max_err_over_bound, err / b_g)
        # derived bar
        assert err <= b_g, f"row {i}: logit error {err:.3e} exceeds fp32 bound {b_g:.3e}"
        assert res.logit[i] - lg <= b_g + b_best, (
            f"row {i}: GPU row trails the maximum by {res.logit[i] - lg:.3e}")
        if res.gap[i] > b_g + b_best:
            assert gpu_id[i] == res.id[i], f"row {i}: id {gpu_id[i]} != oracle {res.id[i]}"
        # stated bar
        assert abs(gpu_logit[i] - res.logit[i]) <= LOGIT_TOL
        if res.gap[i] > GAP_EXEMPT:
            assert gpu_id[i] == res.id[i], f"row {i}: id {gpu_id[i]} != oracle {res.id[i]}"
        elif gpu_id[i] != res.id[i]:
            assert res.logit[i] - lg <= LOGIT_TOL
            st.exempt += 1
    return st
