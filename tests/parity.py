"""Parity criteria shared by the GPU tests (and checked for sensitivity on the CPU).

Attention output [B, H, D] (bf16 storage) against the oracle's fp64 result.  Error
sources of the library's bf16 path, each a rounding to bf16 (relative error at most
2^-9, uniform, so about 2^-9 / sqrt(3) = 1.1e-3 in the root-mean-square sense):
  * the probabilities are rounded to bf16 before the P V product; with value rows
    that are zero-mean the weighted sum's error scales like the sum itself, so the
    relative error of a (query, head) row is about 1.1e-3 whatever the prefix length;
  * each key split's normalised output is stored in bf16 before the split combine
    (one more 1.1e-3 when more than one split runs);
  * the combined output is rounded to bf16 (1.1e-3).
Summed in quadrature that is about 2e-3 per row; the row bound 1e-2 leaves a factor 5.
A row missing one of S equal key splits is off by about sqrt(1/S) (0.18 for S = 32), and
an all-zero row by 1, so both fail.  The element bound, 4e-2 of the row's RMS plus 1e-2
of the element, is about ten standard deviations of the per-element error above.
"""
import numpy as np

ATTN_ROW_REL_L2 = 1e-2
ATTN_ELEM_RMS = 4e-2
ATTN_ELEM_REL = 1e-2


def attention_errors(got: np.ndarray, ref: np.ndarray):
    """(worst per-row relative L2 error, worst element error over the row's RMS bound)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = got - ref
    num = np.sqrt((d * d).sum(axis=-1))
    den = np.sqrt((ref * ref).sum(axis=-1))
    rel = num / np.maximum(den, 1e-30)
    rms = den / np.sqrt(ref.shape[-1])
    bound = ATTN_ELEM_RMS * rms[..., None] + ATTN_ELEM_REL * np.abs(ref)
    elem = np.abs(d) / np.maximum(bound, 1e-30)
    return float(rel.max()), float(elem.max())


def attention_ok(got, ref) -> bool:
    rel, elem = attention_errors(got, ref)
    return rel <= ATTN_ROW_REL_L2 and elem <= 1.0


def assert_attention_close(got, ref, what=""):
    rel, elem = attention_errors(got, ref)
    assert rel <= ATTN_ROW_REL_L2 and elem <= 1.0, \
        f"{what}: worst row relative L2 {rel:.3e} (bound {ATTN_ROW_REL_L2}), worst element {elem:.3f} of its bound"
