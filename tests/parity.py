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

kernel_attention_model() writes those roundings out in numpy, in the order the library's
kernels take them: it is an error model (what a correct bf16 kernel deviates by), used to
size tolerances and to check that the criteria accept such a kernel, never as the
expected value of a test.
"""
import numpy as np

from oracle import bf16_round as _bf16

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


def split_bounds(n_keys: int, nsplit_max: int = 32, unit: int = 64):
    """Key splits of the long-prefix plan, as lists of the (start, end) of their passes: the
    fewest whole 64-key passes per split that cover the keys within nsplit_max splits, the
    passes dealt to the splits in turn (pass j to split j % nsplit)."""
    chunk = -(-n_keys // (nsplit_max * unit)) * unit
    nsplit = -(-n_keys // chunk)
    passes = [(c, min(n_keys, c + unit)) for c in range(0, n_keys, unit)]
    return [passes[s::nsplit] for s in range(nsplit)]


def kernel_attention_model(q, k, v, scale, drop=None, pass_keys=64):
    """Attention as the library's bf16 kernel rounds it.  q [B, Hq, D], k and v [Hkv, N, D]
    (every key visible), grouped query heads.  Per key split: an online softmax over passes
    of pass_keys keys with a running maximum, each pass's probabilities exp(s - m) rounded
    to bf16 for the P V product (the running sum takes them unrounded), the split's
    normalised output stored in bf16; splits merged by (max, sum) weights.  drop: index of
    a split left out of the merge (a failure the criteria must catch)."""
    B, Hq, D = q.shape
    Hkv, N, _ = k.shape
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for h in range(Hq):
        g = h // G
        s_all = (q[:, h, :] @ k[g].T) * scale
        parts = []
        for si, split in enumerate(split_bounds(N, unit=pass_keys)):
            if si == drop:
                continue
            m = np.full(B, -np.inf)
            l = np.zeros(B)
            acc = np.zeros((B, D))
            for p0, p1 in split:
                s = s_all[:, p0:p1]
                m_new = np.maximum(m, s.max(axis=1))
                alpha = np.exp(m - m_new)
                e = np.exp(s - m_new[:, None])
                l = l * alpha + e.sum(axis=1)
                acc = acc * alpha[:, None] + _bf16(e) @ v[g, p0:p0 + e.shape[1]]
                m = m_new
            parts.append((_bf16(acc / l[:, None]), m, l))
        M = np.max([p[1] for p in parts], axis=0)
        w = [p[2] * np.exp(p[1] - M) for p in parts]
        out[:, h, :] = sum(wi[:, None] * p[0] for wi, p in zip(w, parts)) / sum(w)[:, None]
    return out
