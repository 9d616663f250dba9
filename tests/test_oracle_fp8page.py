"""Pins for the oracle's per-page fp8 indexer-K cache append ("Inference Optimization for Kimi K3.1
Pro", §3: the indexer prolog writes each step's new keys into the cache; the fp8 indexer keys carry
one float32 scale per 64-token page).

Reading pinned here: a page's scale only grows and equals the largest |key| the page has received
divided by 448 (1 while it has received only zeros); when new keys raise it, the keys the page
already holds are decoded with the old scale and encoded again with the new one.

Each pin is written once as a check that takes an implementation, so that the planted mistakes at
the end (copies of the oracle with one plausible error) are shown to fail at least one of them:
  * a hand-derived worked example (tests/golden/fp8_page_append_worked_example.json), replayed
    call by call: scales and codes after every call, nothing else changed;
  * exactness: keys whose page scales are powers of two and whose elements have three significand
    bits re-encode without loss, so any order of appends must equal the one-shot quantisation of
    each page (scale amax / 448, codes through torch's float8_e4m3fn cast);
  * closed form of the scale: after any sequence of appends, a page's scale is float32(amax of
    every key it received / 448), whatever the order (float32 division is monotone);
  * error bound: every decoded key is within one E4M3 half-step per encoding it went through;
  * slots, pages and sequences outside the appended range are unchanged.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle.codecs import e4m3_table
from oracle.quant import _e4m3_rne, indexer_cache_append_fp8_ref

GOLD = os.path.join(os.path.dirname(__file__), "golden", "fp8_page_append_worked_example.json")
PAGE = 64


def _torch_e4m3(x):
    t = torch.from_numpy(np.clip(np.asarray(x, np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _bf16(x):
    """Round float32 to bf16 (nearest even), returned as float32."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return (b.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- pins, each taking an implementation
def golden_pin(fn):
    g = json.load(open(GOLD))
    D, P = g["dim"], g["num_pages"]
    bt = np.array([g["block_table"]], np.int32)
    kc = np.full((P, PAGE, D), g["initial_code"], np.uint8)
    ks = np.full(P, g["initial_scale"], np.float32)
    for call in g["calls"]:
        L, T = call["seq_len"], call["T"]
        new = np.zeros((1, T, D), np.float32)
        for pos, v in call["keys"].items():
            new[0, int(pos) - (L - T)] = v
        prev_c, prev_s = kc.copy(), ks.copy()
        kc, ks = fn(new, kc, ks, bt, np.array([L], np.int32), T)
        want_c, want_s = prev_c.copy(), prev_s.copy()
        for page, bits in call["expect_scale_bits"].items():
            want_s[int(page)] = np.array([int(bits, 16)], np.uint32).view(np.float32)[0]
        for page, rows in call["expect_codes"].items():
            for slot, hexrow in enumerate(rows):
                want_c[int(page), slot] = np.frombuffer(bytes.fromhex(hexrow), np.uint8)
        # slots of a touched page that received zero keys and are not listed: code 0
        first = L - T
        for pos in range(first, L):
            page, slot = int(bt[0, pos // PAGE]), pos % PAGE
            if slot >= len(call["expect_codes"].get(str(page), [])):
                want_c[page, slot] = 0
        if not (np.array_equal(kc, want_c) and np.array_equal(ks.view(np.uint32), want_s.view(np.uint32))):
            return False
    return True


def _lens_and_calls(rng, B, steps):
    """Random ragged appends: a first call per sequence writes a prefix of its own length (a batch
    of one), then each call grows every sequence by the batch's T."""
    lens = rng.integers(1, 200, B)
    calls = [(int(L), np.array([L]), b) for b, L in enumerate(lens)]
    for _ in range(steps):
        T = int(rng.choice([1, 1, 3, 17, 64, 130]))
        lens = lens + T
        calls.append((T, lens.copy(), None))
    return calls


def _run(fn, keys, call, kc, ks, bt):
    """One append; a call with a sequence index runs on that sequence alone."""
    T, lens, only = call
    sel = range(len(lens)) if only is None else [only]
    new = np.stack([keys[b, int(L) - T:int(L)] for b, L in zip(sel, lens)])
    return fn(new, kc, ks, bt[list(sel)], lens.astype(np.int32), T)


def _pool(B, max_pages, rng):
    P = B * max_pages + 3
    perm = rng.permutation(P).astype(np.int32)
    return perm[:B * max_pages].reshape(B, max_pages), P


def _final_lens(calls):
    return calls[-1][1]


def exact_pin(fn):
    """Three-significand-bit elements, token maxima 448 * 2^e: every re-encode is exact, so the
    final cache equals the one-shot quantisation of each page, by torch's cast."""
    rng = np.random.default_rng(61)
    B, D = 3, 8
    calls = _lens_and_calls(rng, B, 6)
    max_len = int(_final_lens(calls).max())
    mp = (max_len + PAGE - 1) // PAGE
    bt, P = _pool(B, mp, rng)
    keys = np.zeros((B, max_len, D), np.float32)
    mant = rng.integers(8, 16, (B, max_len, D)) / 8.0                  # 1, 1.125, ..., 1.875
    expo = rng.integers(-3, 8, (B, max_len, D))                        # elements in [2^-3, 240]
    keys[:] = mant * np.ldexp(1.0, expo) * rng.choice([-1.0, 1.0], (B, max_len, D))
    # token max = 448 * 2^e, e growing at slots 20 and 40 of every page: appends that cross those
    # slots raise the scale of a page that already holds keys
    e = np.minimum((np.arange(max_len) % PAGE) // 20, 2)[None, :].repeat(B, 0)
    keys[np.arange(B)[:, None], np.arange(max_len)[None, :], rng.integers(0, D, (B, max_len))] = 448.0 * np.ldexp(1.0, e)
    keys[:, :, 0] = np.where(rng.random((B, max_len)) < 0.2, 0.0, keys[:, :, 0])
    assert np.array_equal(_bf16(keys), keys)
    kc = np.full((P, PAGE, D), 0x7F, np.uint8)
    ks = np.full(P, np.float32(3.0), np.float32)
    for call in calls:
        kc, ks = _run(fn, keys, call, kc, ks, bt)
    final = _final_lens(calls)
    for b in range(B):
        for j in range((int(final[b]) + PAGE - 1) // PAGE):
            page = int(bt[b, j])
            n = min(PAGE, int(final[b]) - PAGE * j)
            x = keys[b, PAGE * j:PAGE * j + n]
            s = np.float32(np.abs(x).max()) / np.float32(448.0)
            if ks[page] != s or not np.array_equal(kc[page, :n], _torch_e4m3(x / s)):
                return False
    return True


def _gauss_keys(rng, B, max_len, D):
    """Gaussian keys whose magnitude drifts upwards along the sequence (scales keep growing)."""
    x = rng.standard_normal((B, max_len, D)) * np.exp(rng.standard_normal((B, max_len, 1)) * 0.7)
    return _bf16(x.astype(np.float32))


def closed_form_and_bound_pin(fn):
    """Scale = float32(amax of the page's keys / 448); each decoded key within one half-step per
    encoding; untouched slots and pages keep their contents."""
    rng = np.random.default_rng(62)
    B, D = 4, 16
    calls = _lens_and_calls(rng, B, 7)
    max_len = int(_final_lens(calls).max())
    mp = (max_len + PAGE - 1) // PAGE + 1
    bt, P = _pool(B, mp, rng)
    keys = _gauss_keys(rng, B, max_len, D)
    kc = np.full((P, PAGE, D), 0x7F, np.uint8)
    ks = np.full(P, np.float32(3.0), np.float32)
    encodings = np.zeros((B, max_len), np.int64)        # times each key was (re-)encoded
    for call in calls:
        T, lens, only = call
        seqs = range(B) if only is None else [only]
        before_c, before_s = kc.copy(), ks.copy()
        kc, ks = _run(fn, keys, call, kc, ks, bt)
        touched = np.zeros(P, bool)
        for b, L in zip(seqs, lens):
            L = int(L)
            encodings[b, L - T:L] += 1
            for j in range((L - T) // PAGE, (L - 1) // PAGE + 1):
                page = int(bt[b, j])
                touched[page] = True
                if ks[page] != before_s[page] and L - T > PAGE * j:   # held keys re-encoded
                    encodings[b, PAGE * j:L - T] += 1
        if not np.array_equal(kc[~touched], before_c[~touched]) or not np.array_equal(
                ks[~touched].view(np.uint32), before_s[~touched].view(np.uint32)):
            return False
        # within a touched page, slots past the sequence's end keep their contents
        for b, L in zip(seqs, lens):
            L = int(L)
            j = (L - 1) // PAGE
            if not np.array_equal(kc[int(bt[b, j]), L - PAGE * j:], before_c[int(bt[b, j]), L - PAGE * j:]):
                return False
    final = _final_lens(calls)
    tab = e4m3_table()
    for b in range(B):
        for j in range((int(final[b]) + PAGE - 1) // PAGE):
            page = int(bt[b, j])
            a, z = PAGE * j, min(int(final[b]), PAGE * j + PAGE)
            x = keys[b, a:z].astype(np.float64)
            s = np.float32(np.float32(np.abs(x).max()) / np.float32(448.0))
            if s == 0:
                s = np.float32(1.0)
            if ks[page] != s:
                return False
            dec = tab[kc[page, a - PAGE * j:z - PAGE * j]] * np.float64(s)
            # one E4M3 half-step (2^-4 relative, 2^-10 * s absolute below the normals) per encoding,
            # plus the float32 roundings of the products and quotients
            per = 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * float(s)
            bound = encodings[b, a:z, None] * per * 1.0001 + 1e-30
            if not (np.abs(dec - x) <= bound).all():
                return False
    return True


PINS = [golden_pin, exact_pin, closed_form_and_bound_pin]


def test_pins_pass_on_the_oracle():
    for pin in PINS:
        assert pin(indexer_cache_append_fp8_ref), pin.__name__


def test_one_call_over_fresh_pages_is_the_one_shot_rule():
    """A whole context appended in one call: each page's scale and codes are those of quantising
    the page at once (the rule of the fp8 workloads), by torch's cast."""
    rng = np.random.default_rng(63)
    B, D, L = 2, 128, 1000
    bt, P = _pool(B, 16, rng)
    keys = _gauss_keys(rng, B, L, D)
    kc = np.full((P, PAGE, D), 0x7F, np.uint8)
    ks = np.zeros(P, np.float32)
    kc, ks = indexer_cache_append_fp8_ref(keys, kc, ks, bt, np.array([L, L], np.int32), L)
    for b in range(B):
        for j in range((L + PAGE - 1) // PAGE):
            n = min(PAGE, L - PAGE * j)
            x = keys[b, PAGE * j:PAGE * j + n]
            s = np.float32(np.abs(x).max()) / np.float32(448.0)
            assert ks[bt[b, j]] == s
            np.testing.assert_array_equal(kc[bt[b, j], :n], _torch_e4m3(x / s))


# ---------------------------------------------------------------- planted mistakes
def _mutant(rescale=True, grow_only=True, held_shift=0, decode_with_new=False, zero_scale=1.0):
    f32 = np.float32

    def fn(k_new, k_cache, k_scale, block_table, seq_lens, T):
        kc, ks = k_cache.copy(), np.asarray(k_scale, f32).copy()
        x = np.asarray(k_new, f32)
        for b in range(x.shape[0]):
            L = int(seq_lens[b])
            first = L - T
            for j in range(first // 64, (L - 1) // 64 + 1):
                page = int(block_table[b, j])
                lo, hi = max(first, 64 * j), min(L, 64 * j + 64)
                held = max(lo - 64 * j + held_shift, 0)
                new = x[b, lo - first:hi - first]
                cand = f32(f32(np.abs(new).max()) / f32(448.0))
                s_old = ks[page] if held > 0 else f32(0.0)
                s = max(s_old, cand) if grow_only else cand
                if s == 0:
                    s = f32(zero_scale)
                if rescale and held > 0 and s != s_old:
                    sd = s if decode_with_new else s_old
                    dec = (e4m3_table()[kc[page, :held]].astype(f32) * sd).astype(f32)
                    kc[page, :held] = _e4m3_rne((dec / s).astype(f32).astype(np.float64))
                slot0 = lo - 64 * j
                kc[page, slot0:slot0 + hi - lo] = _e4m3_rne((new / s).astype(f32).astype(np.float64))
                ks[page] = s
        return kc, ks
    return fn


MUTANTS = {
    "held keys not re-encoded": _mutant(rescale=False),
    "scale follows the newest keys only": _mutant(grow_only=False),
    "one held slot too many": _mutant(held_shift=1),
    "held keys decoded with the new scale": _mutant(decode_with_new=True),
    "zero page takes scale 0": _mutant(zero_scale=0.0),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch(name):
    caught = False
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                if not pin(MUTANTS[name]):
                    caught = True
        except (AssertionError, IndexError, ValueError, FloatingPointError):
            caught = True
    assert caught, name
