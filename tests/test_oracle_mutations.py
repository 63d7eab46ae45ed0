"""The oracle's pins catch plausible mistakes in it (no GPU).

Each mutant below is a copy of the oracle's source (oracle/muonclip_ref.py and
oracle/rounding.py) with one planted slip of the kind the pins are meant to
catch: a dropped term, a wrong exponent, sign, scale, index or operand order,
a mask off by one, a rounding that is too early or of the wrong kind.  The
copy is loaded as a module of its own and stands in for the oracle while every
pin of tests/test_oracle_*.py runs; each mutant must make at least one of them
fail.  An unmodified copy must pass them all (so a failure is the mutant's,
not the harness's).  Only copies are changed: the oracle's files are never
modified, and nothing here touches the GPU path.
"""

import importlib
import inspect
import itertools
import os
import types

import numpy as np
import pytest

import oracle

ORACLE_DIR = os.path.dirname(os.path.abspath(oracle.__file__))
PIN_MODULES = ["test_oracle_rounding_momentum", "test_oracle_newton_schulz", "test_oracle_maxlogit_clip",
               "test_oracle_attention"]

# (what the slip is, file, text in the oracle, text of the mutant)
MUTANTS = [
    ("momentum fused into one rounding", "muonclip_ref.py",
     'scaled = round_to(mu32 * M_prev.astype(np.float64), "f32")', "scaled = mu32 * M_prev.astype(np.float64)"),
    ("mu not rounded to float32", "muonclip_ref.py",
     "mu32 = np.float64(np.float32(mu))", "mu32 = np.float64(mu)"),
    ("pre-scale by the largest entry, not the Frobenius norm", "muonclip_ref.py",
     "return M / (np.linalg.norm(M) + eps)", "return M / (np.abs(M).max() + eps)"),
    ("Gram matrix X^T X instead of X X^T", "muonclip_ref.py",
     "        A = X @ X.T\n", "        A = X.T @ X\n"),
    ("quintic term dropped", "muonclip_ref.py",
     "B = b * A + c * (A @ A)", "B = b * A"),
    ("B X subtracted", "muonclip_ref.py",
     "X = a * X + B @ X", "X = a * X - B @ X"),
    ("coefficients a and b swapped", "muonclip_ref.py",
     "    for a, b, c in coeffs:\n        A = X @ X.T", "    for b, a, c in coeffs:\n        A = X @ X.T"),
    ("result not transposed back", "muonclip_ref.py",
     "return X.T.copy() if transposed else X", "return X"),
    ("RMS factor from the smaller dimension", "muonclip_ref.py",
     "math.sqrt(max(rows, cols)) * RMS_MATCH", "math.sqrt(min(rows, cols)) * RMS_MATCH"),
    ("weight decay not scaled by the learning rate", "muonclip_ref.py",
     "W - lr * (O + weight_decay * W)", "W - lr * O - weight_decay * W"),
    ("update added instead of subtracted", "muonclip_ref.py",
     "W - lr * (O + weight_decay * W)", "W + lr * (O + weight_decay * W)"),
    ("max logit scaled by 1/d", "muonclip_ref.py",
     "    scale = 1.0 / math.sqrt(d)\n    out = np.full(H, -np.inf)", "    scale = 1.0 / d\n    out = np.full(H, -np.inf)"),
    ("max of |logit|", "muonclip_ref.py",
     "logits = q @ k[j0:j0 + block].T", "logits = np.abs(q @ k[j0:j0 + block].T)"),
    ("shared rotary key left out", "muonclip_ref.py",
     "return np.concatenate([k, np.asarray(Kr[b], dtype=np.float64)], axis=1)",
     "return np.concatenate([k, 0.0 * np.asarray(Kr[b], dtype=np.float64)], axis=1)"),
    ("max logit over the first batch element only", "muonclip_ref.py",
     "        for b in range(B):\n            q = np.asarray(Q[b, h], dtype=np.float64)\n            k = _head_keys",
     "        for b in range(1):\n            q = np.asarray(Q[b, h], dtype=np.float64)\n            k = _head_keys"),
    ("causal mask off by one", "muonclip_ref.py",
     "return j <= i + (Sk - Sq)", "return j < i + (Sk - Sq)"),
    ("softmax not normalised", "muonclip_ref.py",
     "O[b, h] = (p / l[:, None]) @ np.asarray(V[b, h], dtype=np.float64)",
     "O[b, h] = p @ np.asarray(V[b, h], dtype=np.float64)"),
    ("log-sum-exp without the row max", "muonclip_ref.py",
     "lse[b, h] = m + np.log(l)", "lse[b, h] = np.log(l)"),
    ("clip at S >= tau", "muonclip_ref.py",
     "elif s > tau:", "elif s >= tau:"),
    ("gamma inverted", "muonclip_ref.py",
     "gamma[h] = tau / s", "gamma[h] = s / tau"),
    ("q^C scaled by gamma instead of gamma^alpha", "muonclip_ref.py",
     "Wq[q0:q0 + q_c_rows] * g**alpha", "Wq[q0:q0 + q_c_rows] * g"),
    ("rotary query rows not scaled", "muonclip_ref.py",
     "Wq[q0 + q_c_rows:q0 + q_rows_per_head] * g, w_dtype)", "Wq[q0 + q_c_rows:q0 + q_rows_per_head], w_dtype)"),
    ("key rows scaled by gamma^alpha", "muonclip_ref.py",
     "g**(1.0 - alpha)", "g**alpha"),
    ("head offset taken from the wrong row count", "muonclip_ref.py",
     "q0 = h * q_rows_per_head", "q0 = h * q_c_rows"),
    ("total clip from the smallest head", "muonclip_ref.py",
     'numeric.max() if numeric.size else float("nan")', 'numeric.min() if numeric.size else float("nan")'),
    ("clip applied to the weights before the update", "muonclip_ref.py",
     "qk_clip(s_l, new_w[qn], new_w[kn],", "qk_clip(s_l, weights[qn], weights[kn],"),
    ("every layer clipped with the first layer's S_max", "muonclip_ref.py",
     "for a, s_l in zip(layers, smax2):", "for a, s_l in zip(layers, [smax2[0]] * len(layers)):"),
    ("bf16 by truncation", "rounding.py",
     "r = np.rint(xf / q) * q", "r = np.trunc(xf / q) * q"),
    ("bf16 ties away from zero", "rounding.py",
     "r = np.rint(xf / q) * q", "r = np.sign(xf) * np.floor(np.abs(xf / q) + 0.5) * q"),
    ("bf16 rounded through float32 (twice)", "rounding.py",
     "    x = np.asarray(x, dtype=np.float64)\n    out = np.empty_like(x)",
     "    x = np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)\n    out = np.empty_like(x)"),
]


def _load_copy(edit=None):
    """The oracle's two modules from their source text, with `edit` = (file, old,
    new) applied, as fresh module objects (the real modules are untouched)."""
    srcs = {name: open(os.path.join(ORACLE_DIR, name)).read() for name in ("rounding.py", "muonclip_ref.py")}
    if edit is not None:
        fname, old, new = edit
        assert srcs[fname].count(old) == 1, (fname, old)
        srcs[fname] = srcs[fname].replace(old, new)
    rounding = types.ModuleType("oracle_copy_rounding")
    exec(compile(srcs["rounding.py"], "oracle_copy/rounding.py", "exec"), rounding.__dict__)
    ref_src = srcs["muonclip_ref.py"]
    assert ref_src.count("from .rounding import round_to") == 1
    ref = types.ModuleType("oracle_copy_ref")
    ref.__dict__["_rounding_copy"] = rounding
    exec(compile(ref_src.replace("from .rounding import round_to", "round_to = _rounding_copy.round_to"),
                 "oracle_copy/muonclip_ref.py", "exec"), ref.__dict__)
    return rounding, ref


def _pins():
    """Every pin of the oracle test modules as (name, callable, kwargs), one
    entry per parameter combination; the only fixture is `rng`."""
    out = []
    for mod_name in PIN_MODULES:
        mod = importlib.import_module(mod_name)
        for name, fn in inspect.getmembers(mod, inspect.isfunction):
            if not name.startswith("test_") or fn.__module__ != mod.__name__:
                continue
            grids = []
            for mark in getattr(fn, "pytestmark", []):
                if mark.name != "parametrize":
                    continue
                names = [n.strip() for n in mark.args[0].split(",")] if isinstance(mark.args[0], str) else list(mark.args[0])
                vals = [v if len(names) > 1 else (v,) for v in mark.args[1]]
                grids.append([dict(zip(names, v)) for v in vals])
            for combo in itertools.product(*grids) if grids else [()]:
                kwargs = {}
                for d in combo:
                    kwargs.update(d)
                out.append((f"{mod_name}.{name}{kwargs or ''}", fn, kwargs))
    return out


def _failing_pins(monkeypatch, rounding, ref):
    """Run every pin with the copy standing in for the oracle; the pins that fail."""
    for mod in (rounding, ref):
        for name, val in vars(mod).items():
            if not name.startswith("_") and hasattr(oracle, name):
                monkeypatch.setattr(oracle, name, val)
    failed = []
    with np.errstate(all="ignore"):
        for label, fn, kwargs in _pins():
            args = dict(kwargs)
            if "rng" in inspect.signature(fn).parameters:
                args["rng"] = np.random.default_rng(20250711)
            try:
                fn(**args)
            except Exception:  # noqa: BLE001  (an assertion or an error: either way the pin rejects the copy)
                failed.append(label)
    monkeypatch.undo()
    return failed


def test_unmodified_copy_passes_every_pin(monkeypatch):
    rounding, ref = _load_copy()
    assert _failing_pins(monkeypatch, rounding, ref) == []


@pytest.mark.parametrize("what,fname,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_every_planted_mistake_fails_a_pin(monkeypatch, what, fname, old, new):
    rounding, ref = _load_copy((fname, old, new))
    failed = _failing_pins(monkeypatch, rounding, ref)
    assert failed, f"no pin catches: {what}"
