"""Float64 layer prep in front of the oracle recurrence (test infrastructure).

The aixai.ru blog, section on how the method is implemented in practice
(its third paragraph), describes the layer around the recurrence: q, k, v
come from convolutional projections, the erase gate b and the write gate w
from independent projections, the log of the decay is computed outside the
kernel in float32, and q and k are L2-normalised before the recurrent
update.  The gates lie in [0, 1] (aiexpert.news/pt, method paragraph); the
map from a projection output to [0, 1] is not stated, and the plainest
reading, the logistic sigmoid, is taken.  The decay input is read as the
natural logarithm g = ln(alpha) of the per-step decay.

``layer_prep`` turns the raw inputs (stored tensors, upcast to float64
exactly) into the recurrence inputs that ``oracle.fwd`` consumes.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def l2_normalise(x) -> np.ndarray:
    """Each vector along the last axis divided by its Euclidean norm (zero
    vectors stay zero)."""
    x = _f64(x)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return np.where(n > 0, x / np.where(n > 0, n, 1.0), 0.0)


def sigmoid(x) -> np.ndarray:
    """Logistic function 1 / (1 + e^-x), elementwise."""
    x = _f64(x)
    return 1.0 / (1.0 + np.exp(-x))


def decay_from_log(g) -> np.ndarray:
    """alpha = e^g for a natural-log decay g <= 0."""
    return np.exp(_f64(g))


def layer_prep(q, k, log_alpha, b_logit, w_logit) -> dict:
    """Recurrence inputs from the raw layer inputs: L2-normalised q and k,
    sigmoid gates, alpha = exp(log_alpha).  Per-(token, head) tensors
    ([B, T, H]) stay per-(token, head)."""
    return {"q": l2_normalise(q), "k": l2_normalise(k), "alpha": decay_from_log(log_alpha),
            "b": sigmoid(b_logit), "w": sigmoid(w_logit)}


def layer_prep_bwd(q, k, log_alpha, b_logit, w_logit, grads) -> dict:
    """Gradients with respect to the raw layer inputs, from the gradients
    with respect to the recurrence inputs (``grads`` as ``oracle.bwd``
    returns them: dq, dk, dalpha, db, dw per channel).  The chain rule
    through each map of ``layer_prep``, written out:

      q = x / |x|        dx = (dq - q (q . dq)) / |x|   (a zero row gets zero)
      b = sigmoid(y)     dy = db b (1 - b), and the same for w
      alpha = e^g        dg = dalpha alpha

    An input given per (token, head) ([B, T, H]) was broadcast over its
    channels, so its gradient is the sum over them.  dv is unchanged."""
    out = {}
    for name, x, gname in (("q", q, "dq"), ("k", k, "dk")):
        x = _f64(x)
        n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
        u = np.where(n > 0, x / np.where(n > 0, n, 1.0), 0.0)
        d = grads[gname]
        out[gname] = np.where(n > 0, (d - u * np.sum(u * d, axis=-1, keepdims=True)) / np.where(n > 0, n, 1.0), 0.0)
    for x, gname, fwd in ((b_logit, "db", sigmoid), (w_logit, "dw", sigmoid), (log_alpha, "dalpha", decay_from_log)):
        x = _f64(x)
        y = fwd(x)
        deriv = y * (1.0 - y) if gname != "dalpha" else y
        d = grads[gname]
        out[gname] = (d.sum(axis=-1) if x.ndim == d.ndim - 1 else d) * deriv
    out["dv"] = grads["dv"]
    return out


def sum_to_layout(grad, like) -> np.ndarray:
    """A per-channel gradient [B, T, H, d] summed over its channels when the
    input it belongs to was given per (token, head) ([B, T, H]) and
    broadcast."""
    return grad.sum(axis=-1) if np.ndim(like) == grad.ndim - 1 else grad
