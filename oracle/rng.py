"""Counter-based random numbers for the oracle (test infrastructure only).

The method draws two random objects: the Gaussian matrix whose QR factor is the
feature rotation ("A JoLT for the KV Cache", Sec. 3, "Rotated low-bit residual")
and the Gaussian test matrix of the randomized range finder (Sec. 3.1, FlashJoLT;
Halko, Martinsson & Tropp 2011).  The pages name no generator, so both sides of
this project implement the same published counter-based one independently:

* SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): the n-th output (0-based) of a stream whose state
  starts at ``key`` is ``mix(key + (n + 1) * GAMMA)`` modulo 2**64.
* Uniform in (0, 1): ``((w >> 11) + 0.5) * 2**-53``.
* Box-Muller (1958): Gaussian element e uses the pair k = e // 2 with
  u1 = U(word 2k), u2 = U(word 2k+1); r = sqrt(-2 ln u1), theta = 2 pi u2;
  even e takes r cos(theta), odd e takes r sin(theta).
* The key of stream s under seed S is the s-th SplitMix64 output of seed S.

Streams: 1 = rotation, 2 = sketch, 3 = eps^2 calibration rows.
"""
import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

STREAM_ROTATION = 1
STREAM_SKETCH = 2
STREAM_CALIBRATION = 3


def mix64(z):
    """SplitMix64 finaliser on a uint64 array (wrap-around arithmetic)."""
    z = np.asarray(z, dtype=np.uint64).copy()
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= _M1
        z ^= z >> np.uint64(27)
        z *= _M2
        z ^= z >> np.uint64(31)
    return z


def splitmix_words(key, n):
    """Outputs number n (uint64 array of indices) of the SplitMix64 stream with state ``key``."""
    n = np.asarray(n, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key) + (n + np.uint64(1)) * GAMMA
    return mix64(z)


def stream_key(seed, stream):
    return int(splitmix_words(np.uint64(seed), np.uint64(stream)))


def uniforms(words):
    return ((words >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def gaussians(seed, stream, count, start=0):
    """Gaussian elements start .. start+count-1 of stream ``stream`` under ``seed`` (float64)."""
    key = stream_key(seed, stream)
    e = np.arange(start, start + count, dtype=np.uint64)
    k = e >> np.uint64(1)
    u1 = uniforms(splitmix_words(key, np.uint64(2) * k))
    u2 = uniforms(splitmix_words(key, np.uint64(2) * k + np.uint64(1)))
    r = np.sqrt(-2.0 * np.log(u1))
    th = 2.0 * np.pi * u2
    odd = (e & np.uint64(1)).astype(bool)
    return np.where(odd, r * np.sin(th), r * np.cos(th))
