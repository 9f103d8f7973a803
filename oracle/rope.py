"""Rotary position encoding in float64 (test infrastructure only).

The LazyAttention summary names RoPE as the positional encoding that is
deferred into the attention kernel ("Core Concept: Deferred Positional
Encoding") and relies on RoPE attention depending only on the relative offset
n - m ("Mathematical Equivalence"). The pages do not fix the RoPE variant; this
oracle takes the rotate-half form used by Llama-family models (the models the
summary's "Experimental Results" evaluate): dimension k is paired with k + D/2,
the pair is rotated by the angle n * theta_k, theta_k = base ** (-2k / D).
Equivalently, z_k = x_k + i x_{k+D/2} is multiplied by exp(i n theta_k).
"""
import numpy as np


def inv_freq(D: int, base) -> np.ndarray:
    """theta_k = base^(-2k/D) for k = 0 .. D/2-1, float64. `base` may instead be the table
    theta_k itself (D/2 values): a frequency-scaled RoPE variant given explicitly."""
    if D % 2:
        raise ValueError("head dim must be even")
    if np.ndim(base) == 1:
        t = np.asarray(base, dtype=np.float64)
        if t.shape != (D // 2,):
            raise ValueError("frequency table must hold D/2 values")
        return t
    k = np.arange(D // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * k / D)


def llama31_scale(theta, factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0,
                  original_context=8192):
    """Frequency scaling of the Llama 3.1 models, applied to each theta separately.

    With wavelength w = 2 pi / theta: w below original_context / high_freq_factor keeps
    theta; w above original_context / low_freq_factor gives theta / factor; in between,
    with r = original_context / w, the weight s = (r - low) / (high - low) mixes the two:
    (1 - s) theta / factor + s theta.
    """
    out = []
    for t in np.asarray(theta, dtype=np.float64):
        w = 2.0 * np.pi / t
        if w < original_context / high_freq_factor:
            out.append(t)
        elif w > original_context / low_freq_factor:
            out.append(t / factor)
        else:
            s = (original_context / w - low_freq_factor) / (high_freq_factor - low_freq_factor)
            out.append((1.0 - s) * t / factor + s * t)
    return np.array(out)


def rotate(x: np.ndarray, pos, base, rotary_dim=None) -> np.ndarray:
    """Apply R(pos) to the last axis of x (float64); base: a RoPE base or the theta table.

    x: [..., D]; pos: integer array broadcastable to x.shape[:-1].
    y_k        = x_k cos(pos theta_k) - x_{k+D/2} sin(pos theta_k)
    y_{k+D/2}  = x_k sin(pos theta_k) + x_{k+D/2} cos(pos theta_k)

    Partial rotary (rotary_dim = r < D; the form GPT-NeoX-style models use when only a
    fraction of each head is rotated): the formulas above act on the first r dims alone,
    with r in place of D (pairs k, k + r/2; theta_k = base^(-2k/r), k < r/2), and dims
    r .. D-1 are returned unchanged. A theta table then holds r/2 values.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    r = D if rotary_dim is None else int(rotary_dim)
    if r % 2 or not 0 < r <= D:
        raise ValueError("rotary_dim must be even and in (0, D]")
    h = r // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq(r, base)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h], x[..., h:r]
    return np.concatenate([a * c - b * s, a * s + b * c, x[..., r:]], axis=-1)
