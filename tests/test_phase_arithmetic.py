"""Error bounds of the float32 phase arithmetic the kernels use for RoPE angles (CPU only).

The kernels never rotate by a phase formed from a float32 angle at a large offset:
- key rows: R(a) is reduced to a fraction of a turn in double, then each lane steps
  through its 8 consecutive rows with R(a + 1) = R(a) R(1) and, from there,
  R(a + k + 1) = 2 cos(f) R(a + k) - R(a + k - 1) (one fused multiply-add per
  component);
- query rows inside a tile (offsets below 256): the angle in turns is formed in float.

These tests replay both in float32 (fused multiply-adds rounded once) over every
frequency of the RoPE bases the workloads use (1e4 and 5e5, head dim 128) and
compare with float64 truth.  The recurrence's error grows about as k^2 over the
8 rows (the rounding of 2 cos(f) shifts the frequency it follows) and peaks near
2.2e-6 on unit-magnitude components; the bar, 4e-6, sits almost three orders of
magnitude under the bf16 rounding (2^-9) that the rotated rows then take.  The
hardware sine/cosine are modelled as correctly rounded.
"""
import numpy as np
import pytest

F32 = np.float32


def _rev(theta, d=128):
    """Frequencies of the channel pairs in turns per position: theta^(-2i/d) / (2 pi)."""
    return theta ** (-2.0 * np.arange(d // 2) / d) / (2.0 * np.pi)


def _unit(turns):
    """(cos, sin) of an angle in turns, correctly rounded to float32."""
    return np.cos(2 * np.pi * turns).astype(F32), np.sin(2 * np.pi * turns).astype(F32)


def _fma(a, b, c):
    """a * b + c rounded once to float32 (the product of two floats is exact in double)."""
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(F32)


def _key_row_phases(a, rev):
    """The 8 row phases of a lane, as the staging forms them."""
    x = np.mod(a * rev, 1.0)                                  # reduced in double
    c, s = _unit(x)
    r1c, r1s = _unit(rev)                                      # R(1)
    two_c = F32(2.0) * r1c
    out = [(c, s)]
    # R(a + 1) = R(a) R(1): (c r1c - s r1s, c r1s + s r1c), each a product then a fused step
    nc = _fma(c, r1c, -(s * r1s).astype(F32))
    ns = _fma(c, r1s, (s * r1c).astype(F32))
    prev, cur = (c, s), (nc, ns)
    out.append(cur)
    for _ in range(6):
        nxt = (_fma(two_c, cur[0], -prev[0]), _fma(two_c, cur[1], -prev[1]))
        prev, cur = cur, nxt
        out.append(cur)
    return out


@pytest.mark.parametrize("theta", [1e4, 5e5])
def test_key_row_phase_recurrence_bound(theta):
    rev = _rev(theta)
    rng = np.random.default_rng(7)
    worst = 0.0
    # offsets t - p0 of the first row: both signs, up to the 32k-context workload's reach
    for a in np.concatenate([rng.integers(-35000, 35000, 200), [0, 1, -1, -34943, 34943]]):
        ph = _key_row_phases(float(a), rev)
        for k, (c, s) in enumerate(ph):
            tc, ts = np.cos(2 * np.pi * (a + k) * rev), np.sin(2 * np.pi * (a + k) * rev)
            worst = max(worst, float(np.max(np.abs(c - tc))), float(np.max(np.abs(s - ts))))
    assert worst < 4e-6, worst


def test_recurrence_catches_a_wrong_step():
    # the same replay with the sign of the previous phase flipped must miss the bar
    rev = _rev(5e5)
    a = 1234.0
    x = np.mod(a * rev, 1.0)
    c0, s0 = _unit(x)
    r1c, r1s = _unit(rev)
    c1 = _fma(c0, r1c, -(s0 * r1s).astype(F32))
    c2_wrong = _fma(F32(2.0) * r1c, c1, c0)                    # + instead of -
    tc = np.cos(2 * np.pi * (a + 2) * rev)
    assert np.max(np.abs(c2_wrong - tc)) > 1e-2


@pytest.mark.parametrize("theta", [1e4, 5e5])
def test_query_row_float_angle_bound(theta):
    rev = _rev(theta)
    worst = 0.0
    for m in range(256):
        x = (F32(m) * rev.astype(F32)).astype(F32)
        x = (x - np.floor(x)).astype(F32)
        c, s = _unit(x.astype(np.float64))
        worst = max(worst, float(np.max(np.abs(c - np.cos(2 * np.pi * m * rev)))),
                    float(np.max(np.abs(s - np.sin(2 * np.pi * m * rev)))))
    # 41 turns * 2^-23 turns = 3e-5 rad at most
    assert worst < 3.5e-5, worst
