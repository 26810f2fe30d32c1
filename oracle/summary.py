"""Span summaries for the mixed-resolution attention term, written out in plain numpy (test infrastructure: only
the tests, the smoke check and the benchmark's CPU baseline use this module).

Source: SEKV page ("Resumo Técnico: SEKV"), "Metodologia" sections 2 and 3: every span keeps a light summary key,
and at decode time the attention runs over a mixed-resolution memory in which spans that are not expanded
contribute their coarse summary vectors with a size correction.

Readings (the page's spans, summary weights and expansion gates are learned; none of that is built):
  * a span is one QEvict window (32 tokens); a window gets its summary when it is evicted, from the contents of
    its full-precision slot at that moment (the original data, or the dequantised copy of a promoted window);
  * the summary key and value are the plain means of the window's 32 keys and values: the sum is taken exactly
    (fp64; 32 storage values never exceed its precision), divided by 32, rounded to fp32 and then to the storage
    dtype (round to nearest even at both steps);
  * size correction: the summary's logit is q . k_sum / sqrt(D) + ln 32, so that a window of 32 identical keys
    keeps exactly the attention mass its tokens had;
  * summaries are attended after the tail, in the order the windows were evicted (events in order, windows
    ascending within an event); they belong to no window, so they add nothing to any cumulative score.
"""
from __future__ import annotations

import math

import numpy as np

from .fp import f32_to_storage_rne, storage_to_f64

SIZE_CORRECTION = math.log(32.0)


def summarize(rows_bits: np.ndarray, dtype: str) -> np.ndarray:
    """rows_bits [32][D] storage patterns of one window's keys (or values) -> [D] storage patterns of the mean."""
    x = storage_to_f64(rows_bits, dtype)
    total = np.zeros(x.shape[1], np.float64)
    for j in range(x.shape[0]):   # exact: every partial sum fits the fp64 significand
        total += x[j]
    mean32 = (total / x.shape[0]).astype(np.float32)
    return f32_to_storage_rne(mean32, dtype)
