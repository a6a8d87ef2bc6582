"""The backward oracle's pins catch plausible mistakes in it (CPU only, mutation check).

As for the forward oracle: each case plants one mistake in a copy of the source text of
oracle/muse_bwd_ref.py (a dropped term, a wrong sign, a missing normalisation), loads
the copy as a fresh module, and runs the committed pins of test_oracle_bwd.py with the
backward functions rebound to the mutant. Every mutant must fail at least one pin; the
unmutated copy must pass them all. The installed oracle package is never modified.
"""

import importlib.util
import os
import sys
import types
import warnings

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC_PATH = os.path.join(os.path.dirname(HERE), "oracle", "muse_bwd_ref.py")
with open(SRC_PATH) as _f:
    SRC = _f.read()

MUTATIONS = [
    ("attend_softmax_no_centring", "da = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "da = p * dp"),
    ("attend_dk_not_scaled", "return scale * (da @ keys), scale * (da.T @ qrows), dv",
     "return scale * (da @ keys), (da.T @ qrows), dv"),
    ("merge_drops_mean_output", "dLs = al * ((dO * (op - o)).sum(axis=1)", "dLs = al * ((dO * op).sum(axis=1)"),
    ("refine_drops_lse_gradient", "dl += p * np.asarray(dL)[idx][:, None]", "dl += 0.0 * p"),
    ("refine_residual_sign", "dqbar[i] -= dqt.sum(axis=0)", "dqbar[i] += dqt.sum(axis=0)"),
    ("refine_drops_dipole_query_term", "dqt += scale * (g @ S.Dip[i])", "dqt += 0.0 * (g @ S.Dip[i])"),
    ("refine_first_cumulant_grad_unscaled", "G.K[i] += scale * (dl.T @ qt)", "G.K[i] += (dl.T @ qt)"),
    ("s1_drops_VK_term", 'dV -= np.einsum("ivd,id->iv", dC, S.K[:, j])', "dV -= 0.0"),
    ("s1_second_moment_key_term_transposed", 'dk[idx] += np.einsum("im,ivd,mv->md", w, dC, vj)',
     'dk[idx] += np.einsum("im,ivd,mv->md", w, dC, vj) * 0.0'),
    ("s1_P_softmax_not_centred", "dlogZ += np.where(finite, P * (dP - (P * dP).sum(axis=1, keepdims=True)), 0.0)",
     "dlogZ += np.where(finite, P * dP, 0.0)"),
    ("s1_tilt_drops_logZ_gradient", "da = w * (dw - (w * dw).sum(axis=1, keepdims=True)) + w * dlogZ[:, j][:, None]",
     "da = w * (dw - (w * dw).sum(axis=1, keepdims=True))"),
    ("untilted_uncentred", "dv[idx] += ((kj - kj.mean(axis=0)) @ dCov.T) / n", "dv[idx] += (kj @ dCov.T) / n"),
    ("centroid_mean_not_divided", "dq[m] += dqbar[i] / m.sum()", "dq[m] += dqbar[i]"),
]


def _load(src: str, tag: str) -> types.ModuleType:
    src = src.replace("from .muse_ref import", "from oracle.muse_ref import")
    mod = types.ModuleType(f"muse_bwd_variant_{tag}")
    exec(compile(src, f"<muse_bwd_ref {tag}>", "exec"), mod.__dict__)
    return mod


def _pins():
    spec = importlib.util.spec_from_file_location("pins_bwd", os.path.join(HERE, "test_oracle_bwd.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


_PINS = _pins()


def _battery(variant):
    g = dict(_PINS.__dict__)
    for n in ("exact_attention_bwd", "muse_acausal_bwd", "muse_causal_bwd"):
        g[n] = getattr(variant, n)
    out = []
    for n, obj in list(g.items()):
        if isinstance(obj, types.FunctionType) and obj.__module__ == _PINS.__name__:
            g[n] = types.FunctionType(obj.__code__, g, obj.__name__, obj.__defaults__, obj.__closure__)
    for n in sorted(g):
        if not (n.startswith("test_") and isinstance(g[n], types.FunctionType)):
            continue
        marks = [m for m in getattr(_PINS.__dict__[n], "pytestmark", []) if m.name == "parametrize"]
        cases = [{}]
        for m in marks:
            names = [s.strip() for s in m.args[0].split(",")]
            cases = [dict(c, **dict(zip(names, vals if len(names) > 1 else (vals,)))) for c in cases for vals in m.args[1]]
        out.extend((n, g[n], kw) for kw in cases)
    return out


def _fails(variant, stop_at_first: bool):
    failed = []
    for pid, fn, kw in _battery(variant):
        try:
            with warnings.catch_warnings(), np.errstate(all="ignore"):
                warnings.simplefilter("ignore")
                fn(**kw)
        except Exception as e:
            failed.append((pid, type(e).__name__))
            if stop_at_first:
                break
    return failed


def test_unmutated_copy_passes_every_pin():
    v = _load(SRC, "clean")
    assert len(_battery(v)) >= 15
    assert _fails(v, stop_at_first=False) == []


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(name, old, new):
    assert SRC.count(old) == 1, f"mutation target of {name} is not unique"
    assert _fails(_load(SRC.replace(old, new), name), stop_at_first=True), f"no pin catches {name}"
