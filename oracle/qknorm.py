"""RMSNorm of queries and keys per head, plainly in float64 (test infrastructure).

Vidu S2 paper read, section 2.4 (the kernel-level cut of the inference stack)
names RMSNorm among the adjacent operators fused with elementwise work.  The
pages give no formula; this is the textbook definition, applied per token and
head over the head dimension d with per-channel weights g:

    y = x / sqrt(mean_d(x^2) + eps) * g

Reading: the norm runs over one head's d channels (QK-norm per head), and the
same weights serve every head.
"""
from __future__ import annotations

import numpy as np


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """x [..., d] -> float64 RMSNorm over the last axis, times gamma [d]."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * np.asarray(gamma, dtype=np.float64)
