"""Global gradient-norm clip coefficient.

Not on the pages; the workloads ask for "global-norm clip at 1.0". Reading
taken (PyTorch's clip-by-total-norm convention, the pages' only code being
PyTorch): total = sum of the ranks' squared-norm partials in rank order
(float64), norm = sqrt(total), coefficient = min(1, max_norm / (norm + 1e-6)),
rounded once to float32 and applied in fp32 inside the AdamW step. max_norm
<= 0 means no clipping (coefficient 1). A non-finite norm yields NaN, which
the step reads as "skip this update".
"""
import math
from typing import Sequence

import numpy as np


def clip_scale(partials: Sequence[float], max_norm: float) -> np.float32:
    total = 0.0
    for p in partials:
        total += float(p)
    if not math.isfinite(total):
        return np.float32(np.nan)
    if max_norm <= 0.0:
        return np.float32(1.0)
    norm = math.sqrt(total)
    return np.float32(min(1.0, max_norm / (norm + 1e-6)))
