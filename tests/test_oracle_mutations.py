"""Plant plausible mistakes in a copy of the CPU oracle and check that the pins
catch every one of them. Runs on the CPU only; the real oracle is untouched."""
import os
import sys
import types

import pytest

from tests import oracle_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "hga_oracle.py")

MUTATIONS = {
    "summary-sum-not-mean": ("K[:, :, g * group:min((g + 1) * group, T)].mean(axis=2)",
                             "K[:, :, g * group:min((g + 1) * group, T)].sum(axis=2)"),
    "chunk-summary-off-by-one": ("K[:, :, c * chunk:min((c + 1) * chunk, T)].mean(axis=2)",
                                 "K[:, :, c * chunk + 1:min((c + 1) * chunk, T)].mean(axis=2)"),
    "score-scale-1/D": ("scale = 1.0 / math.sqrt(q.shape[0]) if scale is None else scale\n    return (np.asarray(summary_rows",
                        "scale = 1.0 / q.shape[0] if scale is None else scale\n    return (np.asarray(summary_rows"),
    "topk-ascending": ("key=lambda t: (-scores[t], ids[t])", "key=lambda t: (scores[t], ids[t])"),
    "ties-to-higher-index": ("key=lambda t: (-scores[t], ids[t])", "key=lambda t: (-scores[t], -ids[t])"),
    "forced-wrong-last": ("chunks = sorted({0, L, *best})", "chunks = sorted({0, L - 1, *best})"),
    "no-forced-first": ("chunks = sorted({0, L, *best})", "chunks = sorted({L, *best})"),
    "chunk-0-competes": ("middle = list(range(1, L))", "middle = list(range(0, L))"),
    "own-chunk-competes": ("middle = list(range(1, L))", "middle = list(range(1, L + 1))"),
    "group-candidate-strict": ("if g < n_g and g * group <= p]", "if g < n_g and g * group < p]"),
    "group-topk-per-chunk-gap": ("gap = scores[order[k - 1]] - scores[order[k]] if k > 0 else math.inf",
                                 "gap = scores[order[k]] - scores[order[k - 1]] if k > 0 else math.inf"),
    "causal-strict": ("if j <= p)", "if j < p)"),
    "lse-drops-max": ("return (w @ v) / s, m + math.log(s)", "return (w @ v) / s, math.log(s)"),
    "softmax-unnormalised": ("return (w @ v) / s, m + math.log(s)", "return (w @ v), m + math.log(s)"),
    "gqa-modulo": ("toks = routed_tokens(group_idx[b, h, i], group, p, T)\n"
                   "                O[b, h, i], lse[b, h, i] = attend_tokens(Q[b, h, i], K[b, h // r], V[b, h // r],",
                   "toks = routed_tokens(group_idx[b, h, i], group, p, T)\n"
                   "                O[b, h, i], lse[b, h, i] = attend_tokens(Q[b, h, i], K[b, h % r], V[b, h % r],"),
    "query-position-shift": ("p = T - Nq + i\n                toks", "p = T - Nq + i - 1\n                toks"),
    "attention-scale-dropped": ("logits = (k @ q) * scale", "logits = (k @ q)"),
    "route-kv-head-modulo": ("kv = h // r", "kv = h % r"),
}


def _mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor must match exactly once: {old!r}"
    name = "hga_oracle_mutant"
    mod = types.ModuleType(name)
    sys.modules[name] = mod          # dataclasses look their module up here
    try:
        exec(compile(src.replace(old, new), name, "exec"), mod.__dict__)
    finally:
        sys.modules.pop(name, None)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name):
    mod = _mutant(*MUTATIONS[name])
    failed = []
    for pin in oracle_pins.PINS:
        try:
            pin(mod)
        except Exception:           # an assertion or a crash both count as caught
            failed.append(pin.__name__)
    assert failed, f"mutation {name} survived every pin"
