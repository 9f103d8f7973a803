"""The oracle's pins catch planted mistakes (CPU only).

Each case below plants one plausible mistake in the float64 oracle: a flipped sign, a
dropped term, an index or convention error. The case recompiles one oracle function from
its own source with a single textual change and binds the result wherever the oracle
package or a pin refers to that function. Then every pin runs (tests/test_oracle_pins.py and
the hand-worked pool traces of tests/test_pool.py), and at least one must fail. The
unmutated oracle must pass all of them (control).

Mistakes are planted only in the oracle, on the CPU; nothing here touches the library.
"""
import functools
import inspect
import textwrap

import numpy as np
import pytest

import oracle
from oracle import alibi, attention, docrot, meta, overhead, pool, rope

_MODULES = (oracle, rope, meta, attention, overhead, pool, alibi, docrot)


POOL_PINS = ("test_ingest_reference_hand_example", "test_model_textbook_lru_trace")


def _pin_modules():
    import tests.test_oracle_pins as pins
    import tests.test_pool as pool_pins
    return pins, pool_pins


def _pins():
    """(name, zero-argument callable) for every pin, one entry per parameter set."""
    pins, pool_pins = _pin_modules()
    out = [(name, getattr(pool_pins, name)) for name in POOL_PINS]
    for name in sorted(dir(pins)):
        fn = getattr(pins, name)
        if not name.startswith("test_") or not callable(fn):
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not marks:
            out.append((name, fn))
            continue
        argnames = [a.strip() for a in marks[0].args[0].split(",")]
        for vals in marks[0].args[1]:
            vals = vals if isinstance(vals, tuple) else (vals,)
            out.append((f"{name}{list(vals)}",
                        functools.partial(fn, **dict(zip(argnames, vals)))))
    return out


def _failing_pins():
    failed = []
    for name, fn in _pins():
        try:
            with np.errstate(all="ignore"):
                fn()
        except (Exception, pytest.fail.Exception):   # an assertion, pytest.raises or a crash
            failed.append(name)
    return failed


def _plant(monkeypatch, owner, fname, old, new):
    """Recompile owner.fname (a module's function or a class's method) with `old` replaced
    by `new` (exactly one occurrence) and bind it in place of the original wherever the
    oracle or a pin module holds it."""
    orig = getattr(owner, fname)
    src = textwrap.dedent(inspect.getsource(orig))
    assert src.count(old) == 1, f"{fname}: the planted text must occur once"
    home = inspect.getmodule(orig)
    ns = dict(vars(home))
    exec(compile(src.replace(old, new), f"<{home.__name__}.{fname}, mutated>", "exec"), ns)
    if inspect.isclass(owner):
        monkeypatch.setattr(owner, fname, ns[fname])
        return
    for m in _MODULES + _pin_modules():
        if getattr(m, fname, None) is orig:
            monkeypatch.setattr(m, fname, ns[fname])


# (module, function, original text, planted text): one mistake each
MUTANTS = {
    "rope: sine sign flipped": (
        rope, "rotate", "[a * c - b * s, a * s + b * c,", "[a * c + b * s, -a * s + b * c,"),
    "rope: cosine and sine swapped": (
        rope, "rotate", "c, s = np.cos(ang), np.sin(ang)", "s, c = np.cos(ang), np.sin(ang)"),
    "rope: interleaved pairs (2k, 2k + 1)": (
        rope, "rotate", "a, b = x[..., :h], x[..., h:r]", "a, b = x[..., 0:r:2], x[..., 1:r:2]"),
    "rope: frequency exponent -k/D": (
        rope, "inv_freq", "-2.0 * k / D", "-1.0 * k / D"),
    "llama 3.1: high-frequency band test reversed": (
        rope, "llama31_scale", "if w < original_context / high_freq_factor:",
        "if w > original_context / high_freq_factor:"),
    "attend: 1/sqrt(D) scale dropped": (
        attention, "attend", "scale = 1.0 / np.sqrt(D)", "scale = 1.0"),
    "attend: strict causal mask": (
        attention, "attend", "visible = key_pos[None, :] <= np.asarray",
        "visible = key_pos[None, :] < np.asarray"),
    "attend: mask on table order, not logical position": (
        attention, "attend", "visible = key_pos[None, :] <= np.asarray",
        "visible = np.arange(key_pos.shape[0])[None, :] + key_pos[0] <= np.asarray"),
    "attend: GQA head map h % Hkv": (
        attention, "attend", "g = h // G", "g = h % Hkv"),
    "attend: keys in place of values": (
        attention, "attend", "o = (p @ V_hat[g])", "o = (p @ K_hat[g])"),
    "attend: softmax not normalised": (
        attention, "attend", "o = (p @ V_hat[g]) / np.where(l > 0, l, 1.0)",
        "o = (p @ V_hat[g])"),
    "materialise: slot index dropped from key positions": (
        attention, "materialise", "pos = int(offsets[t]) + np.arange(n_t, dtype=np.int64)",
        "pos = int(offsets[t]) + np.zeros(n_t, dtype=np.int64)"),
    "materialise: last key of the partial block dropped": (
        attention, "materialise", "else kv_len - (T - 1) * B", "else kv_len - (T - 1) * B - 1"),
    "materialise: values rotated too": (
        attention, "materialise", "vs.append(np.asarray(vb, dtype=np.float64))",
        "vs.append(rotate(vb, pos[None, :], base, rotary_dim))"),
    "materialise: keys rotated from the first entry's offset": (
        attention, "materialise", "ks.append(rotate(kb, pos[None, :], base, rotary_dim)",
        "ks.append(rotate(kb, pos[None, :] - int(offsets[0]), base, rotary_dim)"),
    "queries: rotated one position late": (
        attention, "_rot_queries", "[:, None], base, rotary_dim)", "[:, None] + 1, base, rotary_dim)"),
    "queries: not rotated": (
        attention, "_rot_queries", "return rotate(qf,", "return qf + 0 * rotate(qf,"),
    "rotated pool: rotation one position late": (
        attention, "rotated_pool", "pos = int(seq_offsets[s][t]) + np.arange",
        "pos = int(seq_offsets[s][t]) + 1 + np.arange"),
    "word encode: delta sign flipped": (
        meta, "encode_meta", "delta = off - t * B", "delta = t * B - off"),
    "word encode: delta field one bit low": (
        meta, "encode_meta", "d15 * (1 << ID_BITS)", "d15 * (1 << (ID_BITS - 1))"),
    "word decode: sign extension off by one": (
        meta, "decode_meta", "d15 >= (1 << (DELTA_BITS - 1))", "d15 > (1 << (DELTA_BITS - 1))"),
    "word decode: entry term subtracted": (
        meta, "decode_meta", "return ids, delta + t * B", "return ids, delta - t * B"),
    "word entry index: boundary entries given to the previous sequence": (
        meta, "_entry_index", 'side="right"', 'side="left"'),
    "overhead: P V term dropped": (
        overhead, "attention_flops", "return 2 * M * N * D + 2 * M * N * D",
        "return 2 * M * N * D"),
    "alibi: bias sign flipped": (
        alibi, "attend_alibi", "- float(slopes[h]) * dist", "+ float(slopes[h]) * dist"),
    "alibi: slopes start at exponent 0": (
        alibi, "alibi_slopes", "for i in range(1, n + 1)", "for i in range(0, n)"),
    "document-rotated pool: stored rotation applied instead of undone": (
        docrot, "materialise_doc_rotated", "raw = rotate(kb, -(int(stored_offsets[t]) + j)",
        "raw = rotate(kb, (int(stored_offsets[t]) + j)"),
    "ingest: block and slot indices swapped": (
        pool, "ingest", "k_out[s // B, :, s % B, :] = k_new[i]",
        "k_out[s % B, :, s // B, :] = k_new[i]"),
    "pool index: most recently released document evicted first": (
        pool.PoolIndexModel, "_make_room", "self.lru.popitem(last=False)",
        "self.lru.popitem(last=True)"),
    "pool index: evicted blocks pushed back in reverse": (
        pool.PoolIndexModel, "_make_room", "self.free.extend(blocks)",
        "self.free.extend(blocks[::-1])"),
}


def test_pins_pass_on_the_oracle_as_written():
    assert _failing_pins() == []


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_planted_mistake(mutant, monkeypatch):
    _plant(monkeypatch, *MUTANTS[mutant])
    failed = _failing_pins()
    assert failed, f"no pin fails with the planted mistake: {mutant}"
