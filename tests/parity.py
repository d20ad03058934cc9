"""Parity criteria between the GPU path (float32) and the float64 oracle.

GEMV outputs (ternary and int8 logits) pass when
  * the relative L2 error over the vector is at most 1e-5, and
  * every element is within 1e-4 of its oracle value relative to that value,
    or within 1e-6 of the row's term magnitude s_r * sum_k |W_rk x_k| (where
    the row sum cancels, a relative bound on a near-zero result is not
    meaningful, so the bound is taken on the size of what was summed).
Greedy tokens must equal the oracle's argmax when the oracle's top-2 gap
exceeds 1e-4; otherwise any id whose oracle logit is within 1e-4 of the
maximum is accepted.  Gathers are compared bit for bit.
"""
from __future__ import annotations

import numpy as np

from oracle import reference as ref

REL_L2 = 1e-5
REL_ELEM = 1e-4
MAG_FLOOR = 1e-6
GAP_TOL = 1e-4


def gemv_report(y_gpu, y_ref, mag):
    y = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    mag = np.asarray(mag, dtype=np.float64)
    d = np.abs(y - y_ref)
    nref = np.linalg.norm(y_ref)
    rel_l2 = float(np.linalg.norm(d) / nref) if nref > 0 else (0.0 if d.max(initial=0) == 0 else float("inf"))
    elem_ok = (d <= REL_ELEM * np.abs(y_ref)) | (d <= MAG_FLOOR * mag)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(np.abs(y_ref) > 0, d / np.abs(y_ref), np.where(d > 0, np.inf, 0.0))
        rel_mag = np.where(mag > 0, d / mag, np.where(d > 0, np.inf, 0.0))
    return {
        "ok": bool(rel_l2 <= REL_L2 and elem_ok.all()),
        "rel_l2": rel_l2,
        "n_bad": int((~elem_ok).sum()),
        "max_rel_elem": float(rel.max(initial=0)),
        "max_rel_to_magnitude": float(rel_mag.max(initial=0)),
        "finite": bool(np.isfinite(y).all()),
    }


def assert_gemv(y_gpu, y_ref, mag, what=""):
    r = gemv_report(y_gpu, y_ref, mag)
    assert r["finite"] and r["ok"], f"{what}: {r}"
    return r


def token_ok(token: int, logits_ref) -> bool:
    ref_tok, gap = ref.greedy_token(logits_ref)
    if gap > GAP_TOL:
        return int(token) == ref_tok
    return int(token) in set(ref.accepted_tokens(logits_ref, GAP_TOL).tolist())
