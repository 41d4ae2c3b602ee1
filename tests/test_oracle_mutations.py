"""Sensitivity of the oracle pins: plant a plausible mistake in the oracle
(on the CPU only), run the pins, and require at least one of them to fail.

Each mutation edits the source of one oracle function (a dropped term, a wrong
sign or index, a transposed operand, a wrong constant) and execs the edited
function in the oracle module's namespace for the duration of the check.
"""
import inspect
import textwrap

import pytest

from oracle import model as om
import test_oracle_pins as pins  # noqa: E402  (tests/ is on sys.path under pytest)

MUTATIONS = [
    # (function, original text, mutated text)
    ("rms_norm", "1.0 / np.sqrt(ms + eps)", "1.0 / (np.sqrt(ms) + eps)"),
    ("rms_norm", "np.mean(x * x, axis=-1", "np.sum(x * x, axis=-1"),
    ("rms_norm_bwd", "r * (g - y * np.mean(g * y, axis=-1, keepdims=True))", "r * g"),
    ("rope_angles", "-2.0 * i / hd", "-1.0 * i / hd"),
    ("rope", "x1 * c - x2 * s, x1 * s + x2 * c", "x1 * c + x2 * s, -x1 * s + x2 * c"),
    ("rope", "x1 * c - x2 * s, x1 * s + x2 * c", "x1 * c - x2 * s, x1 * s - x2 * c"),
    ("rope_bwd", "rope(g, -theta)", "rope(g, theta)"),
    ("attention", "(q[:, h, :] @ k[:, g, :].T) * scale", "(q[:, h, :] @ k[:, g, :].T)"),
    ("attention", "np.where(mask, s, -np.inf)", "s"),
    ("attention", "mask = np.tril(np.ones((T, T), dtype=bool))", "mask = np.tril(np.ones((T, T), dtype=bool), -1) | np.eye(T, k=1, dtype=bool)"),
    ("attention_bwd", "p * (dp - np.sum(dp * p, axis=1, keepdims=True))", "p * dp"),
    ("attention_bwd", "dk[:, g, :] += scale", "dk[:, g, :] = scale"),
    ("attention_bwd", "dv[:, g, :] += p.T @ do[:, h, :]", "dv[:, g, :] += p @ do[:, h, :]"),
    ("relu2", "np.maximum(u, 0.0) ** 2", "np.maximum(u, 0.0)"),
    ("softcap", "c * np.tanh(z / c)", "np.tanh(z / c)"),
    ("cross_entropy", "return lse - zc[np.arange(zc.shape[0]), y], lse", "return lse - zc[np.arange(zc.shape[0]), y - 1], lse"),
    ("embed_bwd", "np.add.at(dE, ids.reshape(-1), de.reshape(-1, de.shape[-1]))",
     "dE[ids.reshape(-1)] = de.reshape(-1, de.shape[-1])"),
    ("sequence_forward", "x0, r0 = rms_norm(e, eps)", "x0, r0 = e, 1.0"),
    ("sequence_forward", "x = x + of @ p[\"w_o\"][l].T", "x = x + of @ p[\"w_o\"][l]"),
    ("sequence_forward", "v = qkv[:, (H + Hkv) * hd:]", "v = qkv[:, H * hd: (H + Hkv) * hd]"),
    ("sequence_forward", "x = x + a2 @ p[\"w_proj\"][l].T", "x = a2 @ p[\"w_proj\"][l].T"),
    ("sequence_forward", "h, rf = rms_norm(x, eps)", "h, rf = x, 1.0"),
    ("sequence_forward", "a2 = relu2(u)", "a2 = relu2(-u)"),
    ("softcap_xent_bwd", "return dzc * (1.0 - (zc / c) ** 2)", "return dzc"),
    ("softcap_xent_bwd", "dzc[np.arange(T), y] -= 1.0", "dzc[np.arange(T), y] -= 0.0"),
    ("relu2_bwd", "g * 2.0 * np.maximum(u, 0.0)", "g * np.maximum(u, 0.0)"),
    ("relu2_bwd", "g * 2.0 * np.maximum(u, 0.0)", "g * 2.0 * np.abs(u)"),
    ("sequence_backward", "dx = dx + rms_norm_bwd(dm, C[\"m\"], C[\"rm\"])", "dx = rms_norm_bwd(dm, C[\"m\"], C[\"rm\"])"),
    ("sequence_backward", "grads[\"w_o\"][l] += dx.T @ C[\"of\"]", "grads[\"w_o\"][l] += C[\"of\"].T @ dx"),
    ("sequence_backward", "dq = rope_bwd(rms_norm_bwd(dqn, C[\"qn\"], C[\"rq\"]), theta)",
     "dq = rope_bwd(dqn, theta)"),
    ("step", "bpb=total / (math.log(2.0) * nbytes)", "bpb=total / nbytes"),
    ("step", "sequence_backward(cfg, p, cache, 1.0 / M, grads)", "sequence_backward(cfg, p, cache, 1.0, grads)"),
]

PIN_TESTS = [getattr(pins, n) for n in dir(pins) if n.startswith("test_")]


def _mutated(fn_name, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(om, fn_name)))
    assert src.count(old) == 1, (fn_name, old)
    ns = {}
    exec(compile(src.replace(old, new), f"<mutant {fn_name}>", "exec"), om.__dict__, ns)
    return ns[fn_name]


@pytest.mark.slow
@pytest.mark.parametrize("fn_name,old,new", MUTATIONS, ids=[f"{m[0]}-{i}" for i, m in enumerate(MUTATIONS)])
def test_some_pin_catches_mutation(monkeypatch, fn_name, old, new):
    mutant = _mutated(fn_name, old, new)
    monkeypatch.setattr(om, fn_name, mutant)
    # the package re-exports some names: patch those too
    import oracle
    if hasattr(oracle, fn_name):
        monkeypatch.setattr(oracle, fn_name, mutant)
    caught = []
    for t in PIN_TESTS:
        try:
            t()
        except Exception as e:  # an assertion or a shape error both count
            caught.append((t.__name__, type(e).__name__))
            break
    assert caught, f"no pin detects mutation {fn_name}: {old!r} -> {new!r}"
