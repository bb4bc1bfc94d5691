"""Accuracy metrics of a quantized output O' against the full-precision O.

The SageAttention2++ summary ("A.2 Datasets and Metrics") names cosine
similarity, relative L1 distance and RMSE; their formulas are not printed, so
the standard forms over the flattened tensors are used:
    cos   = <O, O'> / (|O| |O'|)
    relL1 = sum |O - O'| / sum |O|
    rmse  = sqrt(mean((O - O')^2))
"""
import numpy as np


def cosine(ref, out) -> float:
    a = np.asarray(ref, np.float64).ravel()
    b = np.asarray(out, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def rel_l1(ref, out) -> float:
    a = np.asarray(ref, np.float64).ravel()
    b = np.asarray(out, np.float64).ravel()
    return float(np.abs(a - b).sum() / np.abs(a).sum())


def rmse(ref, out) -> float:
    a = np.asarray(ref, np.float64).ravel()
    b = np.asarray(out, np.float64).ravel()
    return float(np.sqrt(np.mean((a - b) ** 2)))


def compare(ref, out) -> dict:
    """All three metrics, ignoring NaN rows of ref (rows not computed)."""
    a = np.asarray(ref, np.float64)
    b = np.asarray(out, np.float64)
    keep = ~np.isnan(a)
    return {"cos": cosine(a[keep], b[keep]), "rel_l1": rel_l1(a[keep], b[keep]), "rmse": rmse(a[keep], b[keep])}
