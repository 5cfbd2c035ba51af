"""YaRN / NTK-by-parts rotary embedding in fp64 -- oracle, test infrastructure.

Follows the "MoE-Xtend" README, section "ROPE + SCALING":
  * base schedule: theta_i = b**(-2i/d), wavelength lambda_i = 2*pi/theta_i;
  * NTK-by-parts ratio r(i) = L * theta_i / (2*pi): how many full turns pair i
    makes over the original training context L;
  * YaRN blend, in the pages' order: freqs_i = base**(i/(d/2)),
    extrapolation = 1/freqs, interpolation = 1/(s*freqs), cutpoints
    i_beta < i_alpha in index space, ramp = (i - i_beta)/(i_alpha - i_beta),
    mask = 1 - clamp(ramp, 0, 1) (1 on fast pairs, 0 on slow pairs),
    inv_freq = interpolation*(1-mask) + extrapolation*mask;
  * concentration c = 0.1*ln(s) + 1, multiplying both cos and sin.

and the position rule of its "DESIGN CONTRACTS" section: the angle uses the
global index p = cache offset + local index, never reset.  The table in the
pages is indexed modulo max_content_length; this oracle takes the contract's
reading instead and uses the true position (no wrap).

Pairing of the two rotated coordinates is not spelled out on the pages.  This
oracle pairs coordinate i with i + d/2 (half split) and rotates
  y_i       = c * (x_i * cos a - x_{i+d/2} * sin a)
  y_{i+d/2} = c * (x_{i+d/2} * cos a + x_i * sin a),   a = p * inv_freq_i,
which is multiplication of (x_i + 1j*x_{i+d/2}) by c*exp(1j*a).
Rotary embeddings touch Q and K only, never V ("GQA Attention" study note,
"How it works").
"""
import numpy as np


def base_theta(d: int, base: float) -> np.ndarray:
    """theta_i = base**(-2i/d) for i in [0, d/2)."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / d)


def wavelength(d: int, base: float) -> np.ndarray:
    return 2.0 * np.pi / base_theta(d, base)


def ntk_rotations(d: int, base: float, orig_ctx: float) -> np.ndarray:
    """r(i) = L * theta_i / (2*pi)."""
    return float(orig_ctx) * base_theta(d, base) / (2.0 * np.pi)


def yarn_cutpoints(d: int, base: float, orig_ctx: float, alpha: float,
                   beta: float):
    """(i_beta, i_alpha), the index-space cutpoints of the ramp."""
    half = d / 2.0
    i_beta = half * np.log(orig_ctx / (beta * 2.0 * np.pi)) / np.log(base)
    i_alpha = half * np.log(orig_ctx / (alpha * 2.0 * np.pi)) / np.log(base)
    return float(i_beta), float(i_alpha)


def yarn_concentration(factor: float) -> float:
    """c = 0.1 * ln(s) + 1.0 (natural log)."""
    return 0.1 * float(np.log(factor)) + 1.0


def yarn_inv_freq(d: int, base: float, factor: float, orig_ctx: float,
                  alpha: float, beta: float) -> np.ndarray:
    """Per-pair angular rate after the NTK-by-parts blend, fp64 [d/2]."""
    if d % 2 or d <= 0:
        raise ValueError("d must be even and positive")
    if not (factor >= 1.0 and 0.0 < alpha < beta and orig_ctx > 0 and base > 1):
        raise ValueError("need s >= 1, 0 < alpha < beta, L > 0, base > 1")
    half = d // 2
    idx = np.arange(half, dtype=np.float64)
    freqs = np.power(float(base), idx / (d / 2.0))
    extrapolation = 1.0 / freqs
    interpolation = 1.0 / (factor * freqs)
    i_beta, i_alpha = yarn_cutpoints(d, base, orig_ctx, alpha, beta)
    ramp = (idx - i_beta) / (i_alpha - i_beta)
    mask = 1.0 - np.clip(ramp, 0.0, 1.0)
    return interpolation * (1.0 - mask) + extrapolation * mask


def rope_rotate(x: np.ndarray, positions: np.ndarray, inv_freq: np.ndarray,
                concentration: float) -> np.ndarray:
    """Rotate head rows x[..., T, H, d] (fp64) at global positions [T].

    Returns the exact fp64 result; rounding to the storage dtype is the
    caller's (``oracle.rounding``)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    pos = np.asarray(positions, dtype=np.float64)
    a = pos[:, None] * inv_freq[None, :]                  # [T, d/2]
    cos = np.cos(a) * concentration
    sin = np.sin(a) * concentration
    cos = cos[:, None, :]                                 # broadcast over heads
    sin = sin[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    y = np.empty_like(x)
    y[..., :half] = x1 * cos - x2 * sin
    y[..., half:] = x2 * cos + x1 * sin
    return y


def rope_apply(x: np.ndarray, offset: int, inv_freq: np.ndarray,
               concentration: float) -> np.ndarray:
    """x[B, T, H, d] at positions offset + arange(T)."""
    T = x.shape[1]
    return rope_rotate(x, offset + np.arange(T, dtype=np.int64), inv_freq,
                       concentration)
