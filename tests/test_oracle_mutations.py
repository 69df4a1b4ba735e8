"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake into a copy of the oracle's source
(a dropped term, a wrong sign or index, an off-by-one, a transposed map),
loads the copy as a separate module, points the pin tests at it
(tests/test_oracle.py and tests/test_oracle_general.py for the NSA oracle,
tests/test_oracle_dsa.py for the token-level sparse attention oracle) and
runs them: at least one pin must fail. A
mutant that every pin passes marks a part of the oracle that nothing
independent checks. The mistakes are planted in the oracle's source text only,
on the CPU; the oracle module itself is never modified.
"""

import inspect
import itertools
import os
import types

import pytest

from tests import test_oracle, test_oracle_dsa, test_oracle_general

PIN_MODULES = (test_oracle, test_oracle_general)

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
ORACLE_SRC = os.path.join(ORACLE_DIR, "nsa_ref.py")
DSA_SRC = os.path.join(ORACLE_DIR, "dsa_ref.py")

# (name, original text, planted text): the original must occur exactly once.
MUTANTS = [
    ("compressed visibility off by one", "nvis = (t - block + 1) // d + 1 if t >= block - 1 else 0",
     "nvis = (t - block + 2) // d + 1 if t >= block - 2 else 0"),
    ("compressed visibility without the own token", "nvis = (t - block + 1) // d + 1 if t >= block - 1 else 0",
     "nvis = (t - block) // d + 1 if t >= block else 0"),
    ("window one key short", "lo = max(0, t - window + 1)", "lo = max(0, t - window + 2)"),
    ("window one key long", "lo = max(0, t - window + 1)", "lo = max(0, t - window)"),
    ("ties go to the higher index", "np.lexsort((np.arange(own), -cand))", "np.lexsort((-np.arange(own), -cand))"),
    ("lowest scores selected", "np.lexsort((np.arange(own), -cand))", "np.lexsort((np.arange(own), cand))"),
    ("compressed branch dropped", "out = g_t[:, 0:1] * o_cmp + g_t[:, 1:2] * o_slc",
     "out = 0.0 * o_cmp + g_t[:, 1:2] * o_slc"),
    ("gates of two branches swapped", "g_t[:, 1:2] * o_slc + g_t[:, 2:3] * o_win",
     "g_t[:, 2:3] * o_slc + g_t[:, 1:2] * o_win"),
    ("scores are raw logits", "scores = probs.sum(axis=0)        # R3",
     "scores = (scale * (qg @ kc.T)).sum(axis=0)        # R3"),
    ("scores from one head", "scores = probs.sum(axis=0)        # R3", "scores = probs[0]        # R3"),
    ("heads grouped by stride", "hs = slice(g * Hg, (g + 1) * Hg)      # R7", "hs = slice(g, Hq, G)      # R7"),
    ("selected tokens past the query",
     "np.arange(j * ls, min(j * ls + ls, t + 1))", "np.arange(j * ls, j * ls + ls)"),
    ("own block not forced", "chosen = sorted(int(j) for j in order[: top_k - 1]) + [own]",
     "chosen = sorted(int(j) for j in order[: top_k])"),
    ("softmax scale missing", "s = scale * (qh @ keys.T)", "s = qh @ keys.T"),
    ("log-sum-exp without the max shift", "return (e / z) @ vals, (m + np.log(z))[:, 0]",
     "return (e / z) @ vals, np.log(z)[:, 0]"),
    ("block mean over one token too many", ".reshape(B, nc, block, G, D).mean(axis=2)",
     ".reshape(B, nc, block, G, D).sum(axis=2) / (block + 1)"),
    ("gap one rank late", "gap = float(ranked[top_k - 2] - ranked[top_k - 1]) if top_k >= 2 else np.inf",
     "gap = float(ranked[top_k - 1] - ranked[min(top_k, own - 1)]) if top_k >= 2 else np.inf"),
    ("gap one rank early", "gap = float(ranked[top_k - 2] - ranked[top_k - 1]) if top_k >= 2 else np.inf",
     "gap = float(ranked[max(top_k - 3, 0)] - ranked[top_k - 2]) if top_k >= 2 else np.inf"),
    ("gap wraps around at top_k 1", "gap = float(ranked[top_k - 2] - ranked[top_k - 1]) if top_k >= 2 else np.inf",
     "gap = float(ranked[top_k - 2] - ranked[top_k - 1])"),
    ("injected repeats counted twice",
     "blocks = sorted({int(j) for j in idx[g] if 0 <= j and j * ls <= t})",
     "blocks = sorted(int(j) for j in idx[g] if 0 <= j and j * ls <= t)"),
    ("injected blocks after the query kept",
     "blocks = sorted({int(j) for j in idx[g] if 0 <= j and j * ls <= t})",
     "blocks = sorted({int(j) for j in idx[g] if 0 <= j})"),
    ("decode one position late", "t = int(seqlens[b]) - 1\n        nvis", "t = int(seqlens[b]) - 2\n        nvis"),
    # general geometry
    ("overlap share over the selection block size", "out[j] += si * overlap / block",
     "out[j] += si * overlap / select_block"),
    ("overlap one token long", "overlap = min(hi, (j + 1) * select_block) - max(lo, j * select_block)",
     "overlap = min(hi, (j + 1) * select_block) - max(lo, j * select_block) + 1"),
    ("compressed blocks placed without the stride", "blk = x[:, i * stride: i * stride + block]",
     "blk = x[:, i * block: i * block + block]"),
    ("one compressed block too few", "return (L - block) // stride + 1 if L >= block else 0",
     "return (L - block) // stride if L >= block else 0"),
    ("compressor weight transposed", 'np.einsum("opc,bpgc->bgo", w, blk)', 'np.einsum("cpo,bpgc->bgo", w, blk)'),
    ("compressor bias dropped", 'out[:, i] = np.einsum("opc,bpgc->bgo", w, blk) + np.asarray(bias, dtype=np.float64)',
     'out[:, i] = np.einsum("opc,bpgc->bgo", w, blk)'),
    ("own selection block by the compressed size", "own = t // ls ", "own = t // block "),
    ("gate sigmoid of the negated logit", "return 1.0 / (1.0 + np.exp(-z))", "return 1.0 / (1.0 + np.exp(z))"),
    ("gate weights of the wrong head",
     'np.einsum("blhd,hdc->blhc", q, np.asarray(weight, dtype=np.float64))',
     'np.einsum("blhd,hdc->blhc", q, np.asarray(weight, dtype=np.float64)[::-1])'),
]


def _pin_calls():
    """Every pin of the pin modules with each of its parameter sets."""
    calls = []
    for mod in PIN_MODULES:
        calls += _module_pins(mod)
    return calls


def _module_pins(module):
    calls = []
    for name, fn in inspect.getmembers(module, inspect.isfunction):
        if not name.startswith("test_") or fn.__module__ != module.__name__:
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not marks:
            calls.append((name, fn, {}))
            continue
        axes = []
        for m in marks:
            names = [s.strip() for s in m.args[0].split(",")]
            axes.append([dict(zip(names, v if len(names) > 1 else (v,))) for v in m.args[1]])
        for combo in itertools.product(*axes):
            kw = {}
            for part in combo:
                kw.update(part)
            calls.append((name, fn, kw))
    return calls


# mistakes planted in the token-level sparse attention oracle
DSA_MUTANTS = [
    ("indexer without its ReLU", "np.maximum(qi_t @ ki.T, 0.0)", "(qi_t @ ki.T)"),
    ("indexer head weights ignored", "(w_t[:, None] * np.maximum(qi_t @ ki.T, 0.0)).sum(axis=0)",
     "np.maximum(qi_t @ ki.T, 0.0).sum(axis=0)"),
    ("ties to the higher token", "np.lexsort((np.arange(n), -cand))", "np.lexsort((-np.arange(n), -cand))"),
    ("one candidate past the query", "n = t + 1\n    if n <= top_k:", "n = t + 2\n    if n <= top_k:"),
    ("gap one rank late", "gap = float(ranked[top_k - 1] - ranked[top_k])",
     "gap = float(ranked[top_k] - ranked[min(top_k + 1, n - 1)])"),
    ("attention scale missing", "s = scale * (qh @ keys.T)", "s = qh @ keys.T"),
    ("heads grouped by stride", "hs = slice(g * Hg, (g + 1) * Hg)", "hs = slice(g, Hq, G)"),
    ("injected tokens after the query kept", "toks = sorted({int(j) for j in idx if 0 <= j <= t})",
     "toks = sorted({int(j) for j in idx if 0 <= j})"),
    ("injected repeats counted twice", "toks = sorted({int(j) for j in idx if 0 <= j <= t})",
     "toks = sorted(int(j) for j in idx if 0 <= j <= t)"),
    ("scores of the next query", "sc = indexer_scores(qi[b, t], KI[: t + 1], w[b, t])",
     "sc = indexer_scores(qi[b, min(t + 1, L - 1)], KI[: t + 1], w[b, t])"),
]


def _mutant_module(original: str, planted: str, path: str = ORACLE_SRC) -> types.ModuleType:
    src = open(path).read()
    assert src.count(original) == 1, f"the original text must occur once in the oracle: {original!r}"
    mod = types.ModuleType("nsa_ref_mutant")
    mod.__file__ = path + " (mutant)"
    exec(compile(src.replace(original, planted), mod.__file__, "exec"), mod.__dict__)
    return mod


def _install(monkeypatch, mod):
    for pins in PIN_MODULES:
        monkeypatch.setattr(pins, "nsa_ref", mod)


def test_pins_pass_on_the_unmodified_oracle_text(monkeypatch):
    # the harness itself: the oracle's own text, loaded the same way, passes every pin
    _install(monkeypatch, _mutant_module("import numpy as np", "import numpy as np"))
    for name, fn, kw in _pin_calls():
        fn(**kw)


@pytest.mark.parametrize("name,original,planted", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_some_pin_kills_the_mutant(name, original, planted, monkeypatch):
    _install(monkeypatch, _mutant_module(original, planted))
    for pin, fn, kw in _pin_calls():
        try:
            fn(**kw)
        except Exception:  # an assertion, or a crash the mistake causes
            return
    pytest.fail(f"no pin detects the planted mistake '{name}'")


def test_dsa_pins_pass_on_the_unmodified_oracle_text(monkeypatch):
    monkeypatch.setattr(test_oracle_dsa, "dsa_ref", _mutant_module("import numpy as np", "import numpy as np", DSA_SRC))
    for name, fn, kw in _module_pins(test_oracle_dsa):
        fn(**kw)


@pytest.mark.parametrize("name,original,planted", DSA_MUTANTS, ids=[m[0] for m in DSA_MUTANTS])
def test_some_dsa_pin_kills_the_mutant(name, original, planted, monkeypatch):
    monkeypatch.setattr(test_oracle_dsa, "dsa_ref", _mutant_module(original, planted, DSA_SRC))
    for pin, fn, kw in _module_pins(test_oracle_dsa):
        try:
            fn(**kw)
        except Exception:
            return
    pytest.fail(f"no pin detects the planted mistake '{name}'")
