"""The oracle's pins catch plausible mistakes.

Each case below plants one mistake (a dropped term, a wrong sign, bias or
index, a transposed operand, a misread rule) in a copy of the oracle's source
held in memory -- the file under oracle/ is never written -- loads the copy as
a module, points the pins of tests/test_oracle.py at it and runs them: at least
one pin must fail. A mistake no pin catches would be a part of the oracle that
nothing outside itself fixes.
"""
import inspect
import itertools
import os
import sys
import types

import pytest

import oracle
from oracle import li_oracle as O_REAL
from tests import test_oracle as PINS

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "li_oracle.py")

# (name, text in the oracle, replacement)
MUTANTS = [
    ("relu dropped", "return w @ np.maximum(x, 0.0)", "return w @ x"),
    ("weights summed outside the relu",
     "return w @ np.maximum(x, 0.0)", "return np.maximum(w @ x, 0.0)"),
    ("tie order reversed", "order = np.lexsort((np.arange(n), -s))",
     "order = np.lexsort((-np.arange(n), -s))"),
    ("ascending scores", "order = np.lexsort((np.arange(n), -s))",
     "order = np.lexsort((np.arange(n), s))"),
    ("causal off by one", "return max(0, min(sk, (i + 1 + orig - sq) // cmp_ratio))",
     "return max(0, min(sk, (i + orig - sq) // cmp_ratio))"),
    ("causal anchored top-left", "orig = sk * cmp_ratio + residual", "orig = sq"),
    ("mode 3 read as mode 0", "    if mode == 0:\n        return sk", "    if mode in (0, 3):\n        return sk"),
    ("transposed query operand", "x = q @ k.T", "x = q.T @ k.T"),
    ("dequant scales dropped",
     "x = (q_scale[:, None] * k_scale[None, :]) * x", "x = x"),
    ("key scale per head", "x = (q_scale[:, None] * k_scale[None, :]) * x",
     "x = (q_scale[:, None] * k_scale[:q_scale.shape[0], None]) * x"),
    ("block table ignored", "blk = wl.block_table[b, j // bs]", "blk = j // bs"),
    ("fp16 exponent bias", "normal = np.ldexp(1.0 + f / 1024.0, (e - 15).astype(np.int32))",
     "normal = np.ldexp(1.0 + f / 1024.0, (e - 16).astype(np.int32))"),
    ("bf16 exponent bias", "normal = np.ldexp(1.0 + f / 128.0, (e - 127).astype(np.int32))",
     "normal = np.ldexp(1.0 + f / 128.0, (e - 126).astype(np.int32))"),
    ("e4m3 subnormal scale", "sub = np.ldexp(f / 8.0, -6)", "sub = np.ldexp(f / 8.0, -7)"),
    ("compressed residual dropped",
     "return r, (int(res[b]) if res is not None else 0)", "return r, 0"),
    ("compressed rule rounds up", "(i + 1 + orig - sq) // cmp_ratio",
     "-(-(i + 1 + orig - sq) // cmp_ratio)"),
    ("index offset on padding slots", "idx[r, h, :m] = order + off",
     "idx[r, h, :m] = order\n                    idx[r, h] += off"),
    ("tail values zero", "val = np.full((R, N2, kk), -np.inf, np.float32)",
     "val = np.full((R, N2, kk), 0.0, np.float32)"),
    ("block sum for block max", "s[c * block_len:min((c + 1) * block_len, n)].max()",
     "s[c * block_len:min((c + 1) * block_len, n)].sum()"),
    ("diagonal block unmasked", "s = block_scores(s, L)",
     "n2 = min(-(-n // L) * L, sk)\n"
     "                        s = block_scores(row_scores(q[t, g], w[t, g], keys[:n2, h], "
     "None if qs is None else qs[t, g], None if kscale is None else kscale[:n2, h]), L)"),
    ("local blocks from the front", "last = set(range(max(nb - local_num, 0), nb))",
     "last = set(range(min(init_num, nb), min(init_num + local_num, nb)))"),
    ("kept blocks last", "return np.concatenate([kept, chosen]), int(kept.shape[0])",
     "return np.concatenate([chosen, kept]), int(kept.shape[0])"),
    ("k not reduced by kept blocks", "topk_order(sb[rest], k - kept.shape[0])",
     "topk_order(sb[rest], k)"),
    ("TND padding ignored", "        if wl.seqused_q is not None:\n            sq = int(wl.seqused_q[b])",
     "        if wl.seqused_q is not None and wl.layout_q != \"TND\":\n"
     "            sq = int(wl.seqused_q[b])"),
    ("TND seqused_k ignored",
     "        if wl.seqused_k is not None:\n            sk = int(wl.seqused_k[b])",
     "        if wl.seqused_k is not None and wl.layout_k != \"TND\":\n"
     "            sk = int(wl.seqused_k[b])"),
    ("TND keys at the query offsets", "r = int(wl.cu_seqlens_k[b]) + j",
     "r = int(wl.cu_seqlens_q[b]) + j"),
    ("TND queries from the first sequence", "r = int(wl.cu_seqlens_q[b]) + rows", "r = rows"),
    ("magnitudes keep the weight signs", "return np.abs(w) @ x", "return w @ x"),
    ("magnitudes of the dot, not of its terms", "x = np.abs(q) @ np.abs(k).T",
     "x = np.abs(q @ k.T)"),
]


def _pins():
    """Every (test function, kwargs) of tests/test_oracle.py, hand examples
    first (they are the quickest)."""
    out = []
    for name, fn in inspect.getmembers(PINS, inspect.isfunction):
        if not name.startswith("test_") or fn.__module__ != PINS.__name__:
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        grids = []
        for m in marks:
            names = [a.strip() for a in m.args[0].split(",")] if isinstance(m.args[0], str) \
                else list(m.args[0])
            vals = [v if len(names) > 1 else (v,) for v in m.args[1]]
            grids.append([dict(zip(names, v)) for v in vals])
        for combo in itertools.product(*grids) if grids else [()]:
            kw = {}
            for d in combo:
                kw.update(d)
            out.append((name, fn, kw))
    out.sort(key=lambda t: (not t[0].startswith("test_hand"), t[0]))
    return out


def _caught(mutant, monkeypatch):
    """Name of the first pin that fails with the mutant in place, or None."""
    monkeypatch.setattr(PINS, "O", mutant)
    monkeypatch.setattr(oracle, "li_oracle", mutant)
    monkeypatch.setitem(sys.modules, "oracle.li_oracle", mutant)
    for name, fn, kw in _pins():
        try:
            fn(**kw)
        except Exception as e:   # a failed assertion or an error both expose the mistake
            tag = ",".join(f"{k}={v['name'] if isinstance(v, dict) else v}" for k, v in kw.items())
            return f"{name}[{tag}]: {type(e).__name__}"
    return None


def _load(src):
    mod = types.ModuleType("li_oracle_mutant")
    exec(compile(src, "<li_oracle mutant>", "exec"), mod.__dict__)
    return mod


def test_unmutated_copy_passes_every_pin(monkeypatch):
    """The harness itself: the unchanged source, loaded the same way, passes."""
    with open(SRC_PATH) as f:
        src = f.read()
    assert _caught(_load(src), monkeypatch) is None


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new, monkeypatch):
    with open(SRC_PATH) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site of '{name}' not found exactly once"
    caught = _caught(_load(src.replace(old, new)), monkeypatch)
    assert caught is not None, f"no pin catches: {name}"
    print(f"{name}: caught by {caught}")
    # the real module is untouched
    assert O_REAL.row_scores.__module__ == "oracle.li_oracle"
