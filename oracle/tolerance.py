"""Acceptance check of a GPU fp8 GEMM result against the oracle -- TEST
INFRASTRUCTURE ONLY.

Primary rule, for every element: |gpu - ref| <= 2e-2 |ref| + 1e-3, and over
all checked elements relL2 < 3e-3 (the relL2 gate of mori PR 785, section
Test, and PR 809, section Results).

The fp8 matrix-core instructions of gfx950 sum the 128 (or 32) products of one
instruction with about 12 significant bits relative to the largest of them
(measured: worst |error| / max|product| = 2^-11.7 over 16k outputs, the same
for the K=128 and K=32 fp8 instructions and whether or not the accumulator is
added inside the instruction).  An output whose exact value nearly cancels can
therefore miss the 1e-3 absolute floor by a hardware rounding that no
instruction choice avoids.  Such an element is accepted only if

    |gpu - ref| <= 2e-2 |ref| + 1e-3 + ulp_bf16(ref)
                   + 2^-9 * sum over 128-wide K blocks of max_k |a'(m,k) b'(n,k)|

(a margin of 2^2.7 over the measured worst case), and at most 1e-3 of the
checked elements may need it (a sanity limit: at the full-size workloads
3-4e-5 of the sampled elements need it at K = 1792-2048 and 1.5e-4 at
K = 7168, since near-cancelling outputs fall under the fixed 1e-3 floor more
often as the sums grow; they use at most 2.2 % of their bound).  A wrong K tile, a stale
LDS read or a missing scale gives errors of the order of |C| itself, far
outside the per-element bound whatever their number.
"""
import numpy as np

PRIMARY_REL, PRIMARY_ABS, REL_L2 = 2e-2, 1e-3, 3e-3
MFMA_REL = 2.0**-9
MAX_SECONDARY_FRACTION = 1e-3


def bits_to_f64(h):
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def block_max_bound(mode, qa, qb, sa, sb, m_idx, n_idx):
    """sum over 128-K blocks of max |a'(m,k) b'(n,k)| for element pairs."""
    from oracle import dec_e4m3

    k = qa.shape[1]
    out = np.empty(len(m_idx))
    for t, (m, n) in enumerate(zip(m_idx, n_idx)):
        a = dec_e4m3(qa[m]).astype(np.float64)
        b = dec_e4m3(qb[n]).astype(np.float64)
        if mode == "ptpc":
            a = a * float(sa[m])
            b = b * float(sb[n])
        elif mode == "blockscale":
            a = a * np.repeat(sa[:, m].astype(np.float64), 128)
            b = b * np.repeat(sb[n // 128].astype(np.float64), 128)
        elif mode == "mxfp8":
            from oracle import dec_e8m0

            a = a * np.repeat(dec_e8m0(sa[:, m]).astype(np.float64), 32)
            b = b * np.repeat(dec_e8m0(sb[:, n]).astype(np.float64), 32)
        out[t] = np.abs(a * b).reshape(k // 128, 128).max(axis=1).sum()
    return out


def check(got_bits, ref_bits, what, mode=None, operands=None, rows=None):
    """Assert the acceptance rule; returns a dict of statistics.

    got_bits / ref_bits: bf16 bit patterns of the same elements; ``rows``
    maps their row index to the GEMM's row (for sampled checks); operands =
    (qa, qb, sa, sb) enables the secondary bound (fp8 modes)."""
    g, r = bits_to_f64(got_bits), bits_to_f64(ref_bits)
    assert np.isfinite(g).all(), f"{what}: non-finite output ({np.count_nonzero(~np.isfinite(g))} elements)"
    err = np.abs(g - r)
    rl2 = float(np.sqrt((err**2).sum() / max((r**2).sum(), 1e-300)))
    assert rl2 < REL_L2, f"{what}: relL2 {rl2:.3g} >= {REL_L2}"
    bad = np.argwhere(err > PRIMARY_REL * np.abs(r) + PRIMARY_ABS)
    stats = {"rel_l2": rl2, "elements": int(err.size), "primary_fail": int(len(bad)), "max_err": float(err.max())}
    if len(bad) == 0:
        return stats
    assert operands is not None and mode is not None, \
        f"{what}: {len(bad)} elements out of tolerance (max err {err.max():.3g}) and no secondary bound applies"
    assert len(bad) <= MAX_SECONDARY_FRACTION * err.size + 1, \
        f"{what}: {len(bad)} of {err.size} elements out of the primary tolerance (max err {err.max():.3g})"
    qa, qb, sa, sb = operands
    mi = bad[:, 0] if rows is None else np.asarray(rows)[bad[:, 0]]
    ni = bad[:, 1]
    bound = block_max_bound(mode, qa, qb, sa, sb, mi, ni)
    rr = r[bad[:, 0], bad[:, 1]]
    ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(rr), 1e-38))[1] - 8)
    lim = PRIMARY_REL * np.abs(rr) + PRIMARY_ABS + ulp + MFMA_REL * bound
    e = err[bad[:, 0], bad[:, 1]]
    worst = int(np.argmax(e / lim))
    assert np.all(e <= lim), (f"{what}: element ({mi[worst]}, {ni[worst]}) err {e[worst]:.3g} exceeds the "
                              f"matrix-core bound {lim[worst]:.3g} (ref {rr[worst]:.3g})")
    stats["secondary_max_ratio"] = float((e / lim).max())
    return stats
