"""fp64 CPU oracle for the dense-decoder training step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything here.  The HIP
path (``dense_decoder_only_amd``) never imports this package and this package
never imports it; the two share only the seeded input generators in
``synthetic``.

The oracle is the plain definition of the model, written in numpy float64,
one sequence at a time, with full T x T attention matrices and full [T, V]
logits.  Its sources are the architecture list in the release-news page
("Karpathy再放大招：8000行代碼復現ChatGPT全棧…", section 技術細節與問答) and the
loss report in bits per byte (nano-series page "Karpathy 的 nano 諧系", section
nanochat).  Where those pages are silent the oracle takes the readings listed
in the module docstring of ``oracle.model``.

Pins: every function is checked in ``tests/test_oracle_*.py`` against closed
forms, invariants, special cases that reduce to textbook routines, brute force
on tiny inputs and central finite differences.  The composed loss value at the
d12/d20/d26 shapes is "parity unpinned" beyond the composition of pinned
parts: the pages print no loss for any given input.
"""
from .model import (  # noqa: F401
    rms_norm,
    rms_norm_bwd,
    rope_angles,
    rope,
    rope_bwd,
    attention,
    attention_bwd,
    softcap,
    cross_entropy,
    embed_bwd,
    relu2,
    relu2_bwd,
    softcap_xent_bwd,
    sequence_forward,
    sequence_backward,
    step,
    to_f64_params,
)
from .optim import adamw_step  # noqa: F401
from .decode import decode_attention, prefix_logits  # noqa: F401
