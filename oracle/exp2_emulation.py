"""Software 2^x by Cody-Waite range reduction and a minimax polynomial.

Test infrastructure only.  Method followed: the FA4 paper summary ("FlashAttention-4:
Algorithm and Kernel Pipelining Co-Design for Asymmetric Hardware Scaling",
Key claims and Method, paper §3.1.3 and Table 2): split x into its integer
part n = floor(x) and fraction f = x - n in [0, 1); evaluate a polynomial in f
by Horner's rule on fused multiply-adds; put n into the IEEE-754 exponent
field by integer addition.  The pages say degree 3 suffices (after rounding
to bf16 it matches the hardware exp2 to within 1 bf16 ULP on 99% of inputs)
and degree 5 comes within 2x of the hardware's max relative error.

The pages do not print the coefficients (an open question in "How
FlashAttention 4 Works" as well), so this module fits its own: a minimax fit
of the relative error by the Remez exchange algorithm, in float64.  Reading
(listed in the design doc): the polynomial is constrained to p(0) = 1, so every
integer x gives exactly 2^x -- in particular the row maximum's probability is
exactly 1.

Also here: float32 -> bf16 round-to-nearest-even and the bf16 ULP distance
used by the 1-ULP acceptance test.
"""
import numpy as np


# ----------------------------------------------------------------- Remez fit
def _basis(f, degree, fix_one):
    """Columns f^i for the free coefficients."""
    lo = 1 if fix_one else 0
    return np.stack([f ** i for i in range(lo, degree + 1)], axis=1)


def _poly(coeffs, f):
    """Evaluate sum_i coeffs[i] f^i in float64 (coeffs[0] is the constant)."""
    out = np.zeros_like(f, dtype=np.float64)
    for c in coeffs[::-1]:
        out = out * f + c
    return out


def relative_error_curve(coeffs, f):
    """p(f) / 2^f - 1 in float64."""
    f = np.asarray(f, dtype=np.float64)
    return _poly(np.asarray(coeffs, dtype=np.float64), f) / np.exp2(f) - 1.0


def _alternating_extrema(err, grid, count):
    """Pick ``count`` points of alternating sign and locally maximal |err|.

    The grid is cut into runs of constant sign; the largest |err| of each run
    is a candidate; a window of ``count`` consecutive candidates containing
    the global maximum is returned.
    """
    sign = np.sign(err)
    sign[sign == 0] = 1
    cuts = np.flatnonzero(np.diff(sign)) + 1
    runs = np.split(np.arange(len(grid)), cuts)
    cand = [r[np.argmax(np.abs(err[r]))] for r in runs if len(r)]
    cand = np.array(cand)
    if len(cand) < count:
        return None
    best = int(np.argmax(np.abs(err[cand])))
    # windows of `count` consecutive candidates that contain the global max;
    # keep the one whose smallest extremum is largest
    starts = range(max(0, best - count + 1), min(best, len(cand) - count) + 1)
    s = max(starts, key=lambda s: np.min(np.abs(err[cand[s:s + count]])))
    return grid[cand[s:s + count]]


def fit_exp2_minimax(degree, fix_one=True, iters=60, grid_points=200001):
    """Minimax (relative error) polynomial p(f) ~ 2^f on [0, 1].

    Returns (coeffs, max_rel_err) with coeffs[0] the constant term (exactly 1
    when ``fix_one``).  Remez exchange: solve for equal-magnitude,
    alternating error at degree+1 (fix_one) or degree+2 reference points,
    move the references to the extrema of the new error curve, repeat.
    """
    n_free = degree if fix_one else degree + 1
    n_ref = n_free + 1
    lo = 1e-6 if fix_one else 0.0          # error is identically 0 at f = 0
    grid = np.linspace(lo, 1.0, grid_points)
    # Chebyshev-like initial references
    t = (1 - np.cos(np.pi * (np.arange(n_ref) + 0.5) / n_ref)) / 2
    ref = lo + (1.0 - lo) * t
    coeffs = None
    E = 0.0
    for _ in range(iters):
        A = _basis(ref, degree, fix_one)
        w = np.exp2(ref)
        alt = (-1.0) ** np.arange(n_ref)
        M = np.concatenate([A, (-alt * w)[:, None]], axis=1)
        rhs = w - (1.0 if fix_one else 0.0)
        sol = np.linalg.solve(M, rhs)
        free, E = sol[:-1], sol[-1]
        coeffs = np.concatenate([[1.0], free]) if fix_one else free
        err = relative_error_curve(coeffs, grid)
        new_ref = _alternating_extrema(err, grid, n_ref)
        if new_ref is None:
            break
        if np.max(np.abs(new_ref - ref)) < 1e-12:
            break
        ref = new_ref
    err = relative_error_curve(coeffs, grid)
    return np.asarray(coeffs, dtype=np.float64), float(np.max(np.abs(err)))


# ------------------------------------------------------- float32 evaluation
def _fma32(a, b, c):
    """Fused multiply-add of float32 arrays with a single rounding to float32.

    The product of two float32 values is exact in the x87 extended format
    (64-bit significand); for the operand ranges used here the sum is exact
    there as well, so the one rounding is the final cast.
    """
    ld = np.longdouble
    return (a.astype(ld) * b.astype(ld) + c.astype(ld)).astype(np.float32)


def exp2_emulated_f32(x, coeffs):
    """2^x on float32 inputs, in float32 arithmetic, by range reduction.

    Steps: inputs below -126 (and -inf) give 0; n = floor(x); f = x - n
    (exact); p = Horner(f) with float32 FMAs; result bits = bits(p) + n<<23.
    ``coeffs`` are cast to float32 first.
    """
    x = np.asarray(x, dtype=np.float32)
    c = np.asarray(coeffs, dtype=np.float64).astype(np.float32)
    under = ~(x >= np.float32(-126.0))        # also catches -inf and NaN
    xs = np.where(under, np.float32(0.0), x).astype(np.float32)
    n = np.floor(xs).astype(np.float32)
    f = (xs - n).astype(np.float32)
    p = np.full_like(f, c[-1])
    for ci in c[-2::-1]:
        p = _fma32(p, f, np.full_like(f, ci))
    bits = p.view(np.uint32).astype(np.int64) + (n.astype(np.int64) << 23)
    out = bits.astype(np.uint32).view(np.float32)
    return np.where(under, np.float32(0.0), out).astype(np.float32)


# ----------------------------------------------------------------- bf16 ops
def bf16_round(x):
    """float32 -> bf16 with round-to-nearest-even, returned as float32 values.

    Finite inputs only (the callers pass finite or zero values).
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (r << 16).astype(np.uint32).view(np.float32)


def bf16_ulp_distance(a, b):
    """Distance in bf16 ULPs between two arrays of bf16 values (as float32).

    Uses the monotone integer ordering of IEEE bit patterns, so it is valid
    across binade boundaries and signs.
    """
    def key(x):
        u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.int64) >> 16
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(key(a) - key(b))
