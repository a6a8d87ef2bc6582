"""The oracle's pins catch plausible mistakes in it (CPU only, mutation check).

Each case below plants one mistake in a copy of the oracle's source text: a dropped
term, a wrong sign or index, a transposed operand, a reading error such as an
untilted mean where the tilted one belongs, or an off-by-one in a mask. The copy
is loaded as a fresh module, and the committed pin tests of ``test_oracle_muse.py``
and ``test_oracle_exact_kmeans.py`` are run against it with their oracle names
rebound to the mutant. Every mutant must fail at least one pin, and the unmutated
copy must pass them all (so a catch is never an artifact of the loading). The
installed oracle package itself is never modified.
"""

import importlib.util
import itertools
import os
import sys
import types
import warnings

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_SRC_PATH = os.path.join(os.path.dirname(HERE), "oracle", "muse_ref.py")
PIN_MODULES = ("test_oracle_exact_kmeans.py", "test_oracle_muse.py", "test_oracle_cap.py", "test_oracle_buckets.py")

with open(ORACLE_SRC_PATH) as _f:
    ORACLE_SRC = _f.read()


# (name, text in the oracle, replacement). Each text must occur exactly once, so an
# edit of the oracle that removes it fails here instead of silently testing nothing.
MUTATIONS = [
    # capped key clusters and the bucket order
    ("cap_keeps_last_members", "labels[members[U:]] = -1", "labels[members[:max(len(members) - U, 0)]] = -1"),
    ("cap_rounds_down", "U = int(np.ceil(cap_ratio * n / Ck))", "U = int(np.floor(cap_ratio * n / Ck))"),
    ("cap_ignored_when_causal", "S = tilted_summaries(qbar, k[pre], v[pre], lk_s[pre], Ck, s, dipole)",
     "S = tilted_summaries(qbar, k[pre], v[pre], lk[pre], Ck, s, dipole)"),
    ("buckets_unstable", 'perm = np.argsort(key, kind="stable")', 'perm = np.argsort(-key, kind="stable")[::-1]'),
    # softmax temperature and exact attention
    ("scale_1_over_D", "return 1.0 / np.sqrt(D)", "return 1.0 / D"),
    ("exact_drops_scale", "a = scale * (qrows @ keys.T)", "a = (qrows @ keys.T)"),
    ("exact_unnormalised", "o[ok] = (e[ok] @ vals) / z[ok, None]", "o[ok] = (e[ok] @ vals)"),
    ("exact_lse_drops_max", "L[ok] = mx_safe[ok, 0] + np.log(z[ok])", "L[ok] = np.log(z[ok])"),
    ("exact_causal_strict", "allowed = (cols[None, :] <= np.arange(r0, r1)[:, None]) if causal",
     "allowed = (cols[None, :] < np.arange(r0, r1)[:, None]) if causal"),
    ("merge_max_not_logaddexp", "L = np.logaddexp(L1, L2)", "L = np.maximum(L1, L2)"),
    ("merge_weight_swapped", "w1 = np.where(np.isfinite(L1), np.exp(L1 - L), 0.0)",
     "w1 = np.where(np.isfinite(L1), np.exp(L2 - L), 0.0)"),
    # K-means
    ("distance_not_squared", 'out[r0:r0 + chunk] = np.einsum("ncd,ncd->nc", diff, diff)',
     'out[r0:r0 + chunk] = np.sqrt(np.einsum("ncd,ncd->nc", diff, diff)) + diff[..., 0]'),
    ("kmeans_init_first_points", "c = x[(np.arange(C) * n) // C].copy()", "c = x[np.arange(C)].copy()"),
    ("kmeans_ties_to_highest", "labels = np.argmin(d, axis=1)  # first minimum",
     "labels = d.shape[1] - 1 - np.argmin(d[:, ::-1], axis=1)  # last minimum"),
    ("kmeans_update_sum", "c[j] = x[members].mean(axis=0)", "c[j] = x[members].sum(axis=0)"),
    ("kmeans_empty_cluster_zeroed", "            if members.any():\n                c[j] = x[members].mean(axis=0)",
     "            c[j] = x[members].mean(axis=0) if members.any() else 0.0"),
    ("kmeans_one_iteration_short", "    for t in range(iters):\n        d = squared_distances(x, c)",
     "    for t in range(max(iters - 1, 1)):\n        d = squared_distances(x, c)"),
    # stage 1: tilted summaries
    ("s1_drops_scale", "a = scale * (qbar @ k[idx].T)            # [Cq, n_j]",
     "a = (qbar @ k[idx].T)            # [Cq, n_j]"),
    ("s1_logZ_drops_max", "logZ[:, j] = mx[:, 0] + np.log(z)", "logZ[:, j] = np.log(z)"),
    ("s1_untilted_key_mean", "Kt[:, j] = w @ k[idx]", "Kt[:, j] = k[idx].mean(axis=0)"),
    ("s1_untilted_value_mean", "Vt[:, j] = w @ v[idx]", "Vt[:, j] = v[idx].mean(axis=0)"),
    ("s1_uniform_cluster_weights", "P = np.where(np.isfinite(logZ), np.exp(logZ - mx), 0.0)",
     "P = np.where(np.isfinite(logZ), 1.0, 0.0)"),
    # centring only one side of C_ij is no mistake (the weighted residuals sum to zero),
    # an uncentred second moment is
    ("s1_dipole_second_moment", "vc = v[idx][None, :, :] - Vt[:, j][:, None, :]        # [Cq, n_j, Dv]\n"
     "            kc = k[idx][None, :, :] - Kt[:, j][:, None, :]",
     "vc = v[idx][None, :, :] + 0.0 * Vt[:, j][:, None, :]        # [Cq, n_j, Dv]\n"
     "            kc = k[idx][None, :, :] + 0.0 * Kt[:, j][:, None, :]"),
    ("s1_dipole_unweighted", "Cij = np.matmul((vc * weights[j][:, :, None]).transpose(0, 2, 1), kc)",
     "Cij = np.matmul(vc.transpose(0, 2, 1), kc) / idx.size"),
    ("s1_dipole_not_aggregated_by_P", "Dip += P[:, j, None, None] * Cij", "Dip += Cij / Ck"),
    ("s1_untilted_sample_covariance", "Cij = np.broadcast_to((vc.T @ kc) / idx.size, (Cq, Dv, D))",
     "Cij = np.broadcast_to((vc.T @ kc) / max(idx.size - 1, 1), (Cq, Dv, D))"),
    # stage 2: refinement
    ("s2_residual_is_query", "qt = q[idx] - qbar[i]  ", "qt = q[idx] + 0.0 * qbar[i]  "),
    ("s2_drops_logZ", "l = S.logZ[i][None, :] + scale * (qt @ S.K[i].T)", "l = 0.0 * S.logZ[i][None, :] + scale * (qt @ S.K[i].T)"),
    ("s2_drops_first_cumulant", "l = S.logZ[i][None, :] + scale * (qt @ S.K[i].T)", "l = S.logZ[i][None, :] + 0.0 * (qt @ S.K[i].T)"),
    ("s2_first_cumulant_sign", "l = S.logZ[i][None, :] + scale * (qt @ S.K[i].T)", "l = S.logZ[i][None, :] - scale * (qt @ S.K[i].T)"),
    ("s2_lse_drops_max", "Li[finite] = mx_safe[finite, 0] + np.log(z[finite])", "Li[finite] = np.log(z[finite])"),
    ("s2_dipole_sign", "oi[finite] += scale * (qt[finite] @ S.Dip[i].T)", "oi[finite] -= scale * (qt[finite] @ S.Dip[i].T)"),
    ("s2_dipole_drops_scale", "oi[finite] += scale * (qt[finite] @ S.Dip[i].T)", "oi[finite] += (qt[finite] @ S.Dip[i].T)"),
    ("s2_dipole_transposed", "oi[finite] += scale * (qt[finite] @ S.Dip[i].T)",
     "oi[finite] += scale * (qt[finite] @ S.Dip[i])"),
    # whole passes
    ("acausal_key_clusters_use_Cq", "km_k, lk, _ = _cluster(k, Ck, iters, labels_k, follow_k, tie_rel)\n"
     "    S = tilted_summaries(qbar, k, v, cap_key_labels(lk, Ck, cap_ratio), Ck, s, dipole)",
     "km_k, lk, _ = _cluster(k, Cq, iters, labels_k, follow_k, tie_rel)\n"
     "    S = tilted_summaries(qbar, k, v, cap_key_labels(lk, Ck, cap_ratio), Ck, s, dipole)"),
    ("fixed_labels_sum_centroid", "            if m.any():\n                c[j] = x[m].mean(axis=0)",
     "            if m.any():\n                c[j] = x[m].sum(axis=0)"),
    ("causal_local_strict", "loc_allowed = (np.arange(r0, r1)[None, :] <= rows[:, None])",
     "loc_allowed = (np.arange(r0, r1)[None, :] < rows[:, None]) | (rows[:, None] == r0)"),
    ("causal_far_includes_own_block", "pre = slice(0, r0)", "pre = slice(0, r1)"),
    ("causal_far_skips_previous_block", "pre = slice(0, r0)", "pre = slice(0, max(r0 - block, 1))"),
    # hierarchical causal decomposition
    ("hier_square_reaches_diagonal", "out.append((q0, q1, lo, lo + h))", "out.append((q0, q1, lo, min(lo + w, nb)))"),
    ("hier_upper_half_not_split", "        split(lo, h)\n        split(lo + h, h)", "        split(lo, h)"),
    ("hier_squares_overwrite", "far[b] = lse_merge(far[b][0], far[b][1], o_s, L_s)", "far[b] = (o_s, L_s)"),
    # retrieval
    ("retrieval_smallest_first", 'order = np.argsort(-values, kind="stable")', 'order = np.argsort(values, kind="stable")'),
    ("retrieval_cluster_score_max", "sj = _lse_rows(sig)", "sj = np.max(sig, axis=1)"),
    ("retrieval_local_unmasked", "allowed[:, R.size:] = np.arange(r0, r1)[None, :] <= qi[:, None]",
     "allowed[:, R.size:] = True"),
    ("retrieval_far_double_counts", "S = tilted_summaries(qbar[i:i + 1], k[F], v[F], lk[F], Ck, s, dipole)",
     "S = tilted_summaries(qbar[i:i + 1], k[:r0], v[:r0], lk[:r0], Ck, s, dipole)"),
    ("retrieval_one_block_short", "sel = [(j, _top(sig[j], k2)) for j in J]", "sel = [(j, _top(sig[j], max(k2 - 1, 1))) for j in J]"),
]


def _load_variant(src: str, tag: str) -> types.ModuleType:
    name = f"_oracle_variant_{tag}"
    mod = types.ModuleType(name)
    mod.__file__ = ORACLE_SRC_PATH
    sys.modules[name] = mod  # dataclasses resolve string annotations through sys.modules
    try:
        exec(compile(src, f"<oracle variant {tag}>", "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    return mod


def _load_pins():
    mods = []
    for fname in PIN_MODULES:
        spec = importlib.util.spec_from_file_location("_pins_" + fname[:-3], os.path.join(HERE, fname))
        m = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(m)
        mods.append(m)
    return mods


_PINS = _load_pins()


def _cases(fn):
    """Argument sets of a (possibly parametrized) pin test."""
    params = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
    if not params:
        return [{}]
    names, values = [], []
    for m in params:
        argnames = m.args[0]
        if isinstance(argnames, str):
            argnames = [a.strip() for a in argnames.split(",")]
        names.append(argnames)
        values.append([v if len(argnames) > 1 else (v,) for v in m.args[1]])
    out = []
    for combo in itertools.product(*values):
        kw = {}
        for ns, vs in zip(names, combo):
            kw.update(zip(ns, vs))
        out.append(kw)
    return out


def _battery(variant: types.ModuleType):
    """(pin id, callable) for every committed pin test, bound to `variant`."""
    exported = [n for n in dir(variant) if not n.startswith("__")]
    out = []
    for pm in _PINS:
        g = dict(pm.__dict__)
        for n in exported:
            if n in g and n != "np":
                g[n] = getattr(variant, n)
        # rebind every function of the pin module so helpers see the variant too
        for n, obj in list(g.items()):
            if isinstance(obj, types.FunctionType) and obj.__module__ == pm.__name__:
                f = types.FunctionType(obj.__code__, g, obj.__name__, obj.__defaults__, obj.__closure__)
                f.__kwdefaults__ = obj.__kwdefaults__
                f.pytestmark = getattr(obj, "pytestmark", [])
                g[n] = f
        for n in sorted(g):
            if n.startswith("test_") and isinstance(g[n], types.FunctionType):
                for kw in _cases(g[n]):
                    out.append((f"{n}{kw if kw else ''}", g[n], kw))
    return out


def _failing_pins(variant, stop_at_first: bool):
    failed = []
    for pid, fn, kw in _battery(variant):
        try:
            with warnings.catch_warnings(), np.errstate(all="ignore"):
                warnings.simplefilter("ignore")
                fn(**kw)
        except Exception as e:  # AssertionError, or a shape error the mistake causes
            failed.append((pid, type(e).__name__))
            if stop_at_first:
                break
    return failed


def test_unmutated_copy_passes_every_pin():
    variant = _load_variant(ORACLE_SRC, "clean")
    battery = _battery(variant)
    assert len(battery) >= 38  # every pin test case of the two modules is in the battery
    assert _failing_pins(variant, stop_at_first=False) == []


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(name, old, new):
    assert ORACLE_SRC.count(old) == 1, f"mutation target of {name} is not unique in the oracle"
    variant = _load_variant(ORACLE_SRC.replace(old, new), name)
    failed = _failing_pins(variant, stop_at_first=True)
    assert failed, f"no pin catches the planted mistake {name}"
