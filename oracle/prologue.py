"""fp64 oracle of the layer prologue the fused entry points apply.  TEST
INFRASTRUCTURE ONLY (same import rule as the rest of ``oracle``).

Before the recurrence, the layer L2-normalises q and k per (token, head) and maps
the gate logits to their ranges (Q-Delta reading notes §2.1 and §3.1, and the
layer figure of §1: q and k are unit vectors, beta and lambda come from sigmoids,
alpha = exp(-softplus(.)) keeps the decay in (0, 1)):

  q_hat = q / sqrt(|q|^2 + eps),  k_hat likewise          (eps = 1e-6, a reading)
  beta  = 1 / (1 + exp(-b)),  lambda = 1 / (1 + exp(-l))
  alpha = exp(-softplus(a)),  softplus(a) = log(1 + exp(a))

The pages name the operations but not the epsilon of the normalisation; eps only
matters for (near-)zero vectors, where it keeps the result finite (a zero vector
stays zero).  Plain formulas, evaluated in fp64.
"""
import numpy as np

EPS = 1e-6


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def l2_normalise(x):
    """x / sqrt(sum(x^2) + EPS) over the last axis."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + EPS)


def sigmoid(z):
    z = _f64(z)
    return 1.0 / (1.0 + np.exp(-z))


def softplus(z):
    """log(1 + exp(z)), in the overflow-free form max(z, 0) + log1p(exp(-|z|))."""
    z = _f64(z)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def decay(a_logit):
    """alpha = exp(-softplus(a))."""
    return np.exp(-softplus(a_logit))


def prologue(q, k, a_logit, b_logit, l_logit):
    """(q_hat, k_hat, alpha, beta, lambda) from raw q, k and gate logits; a None
    alpha logit means alpha = 1 and a None lambda logit means lambda = 0, returned
    as None like the library's null gates."""
    return (l2_normalise(q), l2_normalise(k),
            None if a_logit is None else decay(a_logit),
            sigmoid(b_logit),
            None if l_logit is None else sigmoid(l_logit))
