"""AdamW update for the training loop that follows the step (fp64 oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The release-news page ("Karpathy再放大招：8000行代碼復現ChatGPT全棧…", section
技術細節與問答) names Muon + AdamW as the optimizers; it defines neither and
gives no hyperparameters.  Muon is left out (it needs a definition the pages
do not give).  AdamW here is the published method: Adam moment estimates with
bias correction and weight decay decoupled from the gradient step
(Loshchilov and Hutter, "Decoupled Weight Decay Regularization").  Every
hyperparameter is an argument.  Readings:
  * the decay multiplies the parameter before the Adam step, p <- p (1 - lr wd);
  * eps is added to sqrt(v_hat) (outside the square root);
  * the gradient may be scaled first by grad_scale (e.g. 1 / accumulation
    count);
  * after the fp32 master update a bf16 copy of the weights is refreshed
    (round to nearest, ties to even) for the next forward pass.
"""
from __future__ import annotations

import numpy as np


def adamw_step(p, g, m, v, t, lr, beta1, beta2, eps, weight_decay, grad_scale=1.0):
    """One AdamW step at step count t >= 1.  Returns (p, m, v) as new fp64 arrays."""
    p = np.asarray(p, np.float64)
    g = np.asarray(g, np.float64) * grad_scale
    m = beta1 * np.asarray(m, np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, np.float64) + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    p = p * (1.0 - lr * weight_decay)
    p = p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p, m, v
