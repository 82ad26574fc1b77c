"""The oracle's pins must catch plausible mistakes planted in the oracle.

Each case edits one expression of the oracle's source (on the CPU, in a fresh
module object), swaps the mutant into the ``oracle`` package and runs the pin
tests of ``test_oracle``; at least one of them must fail.
"""

import inspect
import os
import types

import pytest

import oracle
import oracle.dcp_oracle as real

from . import test_oracle as pins
from . import test_oracle_kvwrite as kv_pins
from . import test_oracle_prefix as prefix_pins
from . import test_oracle_topk as topk_pins

MUTATIONS = [
    ("value slice", "keys[:, :D_V]) / l", "keys[:, -D_V:]) / l"),
    ("softmax scale dropped", "z = sigma * (q @ keys.T)", "z = (q @ keys.T)"),
    ("max dropped from LSE", "lse = m[:, 0] + np.log(l[:, 0])", "lse = np.log(l[:, 0])"),
    ("owner by div", "own = valid[valid % n == r] // n", "own = valid[valid // n == r] // n"),
    ("local id by mod", "own = valid[valid % n == r] // n", "own = valid[valid % n == r] % n"),
    ("merge weight sign", "lse_parts - m_safe, 0.0)", "m_safe - lse_parts, 0.0)"),
    ("E4M3 bias", "np.exp2(e.astype(np.float64) - 7.0)", "np.exp2(e.astype(np.float64) - 8.0)"),
    ("E4M3 subnormal step", "m.astype(np.float64) * 2.0 ** -9", "m.astype(np.float64) * 2.0 ** -10"),
    ("E4M3 subnormal test", "np.where(e == 0, subnormal, normal)", "np.where(e == 1, subnormal, normal)"),
    ("page walk", "return pages * page_size + j % page_size",
     "return pages * page_size + j // page_size"),
    ("unsharded row", "dequant_rows(pools[r], g[on_r] // n", "dequant_rows(pools[r], g[on_r] % n"),
    ("scale divides", "return _E4M3_TABLE[codes] * s[:, None]", "return _E4M3_TABLE[codes] / s[:, None]"),
    ("empty LSE not -inf", "lse = np.where(any_valid, m_safe + np.log(denom), -np.inf)",
     "lse = np.where(any_valid, m_safe + np.log(denom), 0.0)"),
    ("unsafe denominator", "o = np.where(any_valid[..., None], contrib.sum(axis=0) / denom[..., None], 0.0)",
     "o = contrib.sum(axis=0) / w_sum[..., None]"),
    ("empty shard weighted", "contrib = np.where(valid[..., None], o_parts, 0.0) * w[..., None]",
     "contrib = o_parts * w[..., None]"),
    ("E4M3 encode bias", "codes[nrm] = ((e + 7) << 3) | m8", "codes[nrm] = ((e + 8) << 3) | m8"),
    ("E4M3 encode truncates", "m8 = np.rint((2.0 * mant - 1.0) * 8.0)", "m8 = np.floor((2.0 * mant - 1.0) * 8.0)"),
    ("E4M3 encode no carry", "carry = m8 == 8", "carry = m8 == 9"),
    ("E4M3 encode subnormal step", "np.rint(a[sub] * 2.0 ** 9)", "np.rint(a[sub] * 2.0 ** 8)"),
    ("quant scale inverted", "scale = np.float32(amax / e4m3_max)", "scale = np.float32(e4m3_max / amax)"),
    ("quant divides by the inverse", "q = (x * inv).astype(np.float32)", "q = (x / inv).astype(np.float32)"),
    ("kv write shard by div", "r, row = int(g % num_shards), int(g // num_shards)",
     "r, row = int(g // num_shards) % num_shards, int(g % num_shards)"),
    ("quant divides by the scale", "q = (x * inv).astype(np.float32)", "q = (x / scale).astype(np.float32)"),
    ("kv write placement blocked", "r, row = int(g % num_shards), int(g // num_shards)",
     "r, row = int(g // pools[0].shape[0]), int(g % pools[0].shape[0])"),
    ("prefix span without shards", "span = int(page_size) * int(num_shards)", "span = int(page_size)"),
    ("prefix gather row by mod", "        r, row = g % n, g // n\n        rows[j]",
     "        r, row = g // n % n, g % n\n        rows[j]"),
    ("bf16 rounding truncates", "np.ldexp(np.rint(m * 256.0), e - 8)", "np.ldexp(np.trunc(m * 256.0), e - 8)"),
    ("bf16 keeps 8 fraction bits", "np.ldexp(np.rint(m * 256.0), e - 8)", "np.ldexp(np.rint(m * 512.0), e - 9)"),
    ("running merge drops the new chunk", "lse_merge(np.stack([o_acc, o_new]), np.stack([lse_acc, lse_new]))",
     "lse_merge(np.stack([o_acc, o_acc]), np.stack([lse_acc, lse_new]))"),
    ("index ReLU dropped", "(np.maximum(dots, 0.0) * w[None, :])", "(dots * w[None, :])"),
    ("index scale dropped", "return s * (np.maximum(dots, 0.0)", "return 1.0 * (np.maximum(dots, 0.0)"),
    ("ties to the later position", "order = np.lexsort((positions, -scores))",
     "order = np.lexsort((-positions, -scores))"),
    ("local position by shard block", "pos = np.arange(int(n_local), dtype=np.int64) * int(num_shards) + int(shard)",
     "pos = np.arange(int(n_local), dtype=np.int64) + int(shard) * int(n_local)"),
    ("merge keeps the first shard only", "sc = np.concatenate([np.asarray(c, dtype=np.float64) for c in cand_scores])",
     "sc = np.concatenate([np.asarray(c, dtype=np.float64) for c in cand_scores[:1]] + [np.full(len(c), -np.inf) for c in cand_scores[1:]])"),
    ("kv write keeps skipped", "        if g < 0:\n            continue\n        r, row",
     "        if g < -1:\n            continue\n        r, row"),
]


def _pin_calls():
    calls = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction) + \
            inspect.getmembers(kv_pins, inspect.isfunction) + \
            inspect.getmembers(prefix_pins, inspect.isfunction) + \
            inspect.getmembers(topk_pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if not params:
            calls.append((name, fn, {}))
            continue
        # first value of every parametrize axis keeps this fast
        kwargs = {}
        for m in params:
            argnames = [a.strip() for a in m.args[0].split(",")] if isinstance(m.args[0], str) else m.args[0]
            first = m.args[1][0]
            first = first if isinstance(first, tuple) and len(argnames) > 1 else (first,)
            kwargs.update(dict(zip(argnames, first)))
        calls.append((name, fn, kwargs))
    return calls


@pytest.mark.parametrize("label,before,after", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(label, before, after, monkeypatch):
    src = inspect.getsource(real)
    assert before in src, label
    mutant = types.ModuleType("oracle_mutant")
    mutant.__file__ = os.path.join(os.path.dirname(real.__file__), "mutant.py")
    exec(compile(src.replace(before, after), mutant.__file__, "exec"), mutant.__dict__)
    for name in oracle.__dict__:
        if name in mutant.__dict__ and not name.startswith("__"):
            monkeypatch.setattr(oracle, name, mutant.__dict__[name])
    failed = []
    for name, fn, kwargs in _pin_calls():
        try:
            fn(**kwargs)
        except Exception:
            failed.append(name)
    assert failed, f"mutation '{label}' was not caught by any pin"


def test_unmutated_oracle_passes_every_pin_call():
    failed = []
    for name, fn, kwargs in _pin_calls():
        try:
            fn(**kwargs)
        except Exception as exc:  # pragma: no cover - reported below
            failed.append((name, repr(exc)))
    assert not failed, failed
