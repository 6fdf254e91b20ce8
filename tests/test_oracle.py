"""CPU tests of the fp64 oracle against its pins (no GPU)."""

import importlib.util
import json
import os

import numpy as np
import pytest

import oracle
from tests import oracle_pins

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


# ---------------------------------------------------------------------------
# Mutation check: plant plausible mistakes in a private copy of the oracle and
# make sure at least one pin rejects each of them.
# ---------------------------------------------------------------------------

def _fresh_oracle():
    path = os.path.join(os.path.dirname(HERE), "oracle", "ref.py")
    spec = importlib.util.spec_from_file_location("oracle_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _m_no_scale(np_):
    def head(q, k, v, scale):
        s = q @ k.T
        m = s.max(axis=1, keepdims=True)
        e = np_.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        return (e @ v) / l, (m + np_.log(l))[:, 0]
    return ("_attn_head", head)


def _m_lse_drops_max(np_):
    def head(q, k, v, scale):
        s = scale * (q @ k.T)
        m = s.max(axis=1, keepdims=True)
        e = np_.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        return (e @ v) / l, np_.log(l)[:, 0]
    return ("_attn_head", head)


def _m_normalise_by_max(np_):
    def head(q, k, v, scale):
        s = scale * (q @ k.T)
        m = s.max(axis=1, keepdims=True)
        e = np_.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        return (e @ v) / e.max(axis=1, keepdims=True), (m + np_.log(l))[:, 0]
    return ("_attn_head", head)


def _m_softmax_wrong_axis(np_):
    def head(q, k, v, scale):
        s = scale * (q @ k.T)
        m = s.max(axis=1, keepdims=True)
        l = np_.exp(s - m).sum(axis=1, keepdims=True)
        p = np_.exp(s - s.max(axis=0, keepdims=True))
        p = p / p.sum(axis=0, keepdims=True)
        return p @ v, (m + np_.log(l))[:, 0]
    return ("_attn_head", head)


def _m_k_for_v(np_):
    def head(q, k, v, scale):
        s = scale * (q @ k.T)
        m = s.max(axis=1, keepdims=True)
        e = np_.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        return (e @ k) / l, (m + np_.log(l))[:, 0]
    return ("_attn_head", head)


def _m_merge_sign(np_, mod):
    orig = mod.ref_lse_merge

    def merge(O_a, L_a, O_b, L_b):
        O, L = orig(O_a, L_a, O_b, L_b)
        La, Lb = mod.decode(L_a), mod.decode(L_b)
        m = np_.maximum(La, Lb)
        wa, wb = np_.exp(m - La), np_.exp(m - Lb)
        ok = np_.isfinite(La) & np_.isfinite(Lb)
        O2 = (wa[..., None] * mod.decode(O_a) + wb[..., None] * mod.decode(O_b)) / (wa + wb)[..., None]
        O = np_.where(ok[..., None], O2, O)
        return O, L
    return ("ref_lse_merge", merge)


def _m_merge_lse_no_max(np_, mod):
    orig = mod.ref_lse_merge

    def merge(O_a, L_a, O_b, L_b):
        O, L = orig(O_a, L_a, O_b, L_b)
        La, Lb = mod.decode(L_a), mod.decode(L_b)
        m = np_.maximum(La, Lb)
        ok = np_.isfinite(La) & np_.isfinite(Lb)
        return O, np_.where(ok, L - m, L)
    return ("ref_lse_merge", merge)


def _m_merge_empty_nan(np_, mod):
    def merge(O_a, L_a, O_b, L_b):
        Oa, Ob = mod.decode(O_a), mod.decode(O_b)
        La, Lb = mod.decode(L_a), mod.decode(L_b)
        m = np_.maximum(La, Lb)
        wa, wb = np_.exp(La - m), np_.exp(Lb - m)
        return (wa[..., None] * Oa + wb[..., None] * Ob) / (wa + wb)[..., None], m + np_.log(wa + wb)
    return ("ref_lse_merge", merge)


def _m_cfg_wrong_base(np_, mod):
    def cfg(u, c, s):
        u, c = mod.decode(u), mod.decode(c)
        return c + float(s) * (c - u)
    return ("ref_cfg", cfg)


def _m_splice_off_by_one(np_, mod):
    def patch(Q_p, K_p, V_p, K_buf, V_buf, p0, scale, rows=None):
        Np = Q_p.shape[2]
        K_new, V_new = np_.array(K_buf, copy=True), np_.array(V_buf, copy=True)
        K_new[:, :, p0 + 1:p0 + 1 + Np] = K_p[:, :, : K_new.shape[2] - p0 - 1]
        V_new[:, :, p0 + 1:p0 + 1 + Np] = V_p[:, :, : V_new.shape[2] - p0 - 1]
        O, L = mod.ref_attn(Q_p, K_new, V_new, scale, rows=rows)
        return O, L, K_new, V_new
    return ("ref_patch", patch)


def _m_strided_runs_packed(np_, mod):
    """Runs placed back to back in the buffer (the stride ignored)."""
    def patch(Q_p, K_p, V_p, K_buf, V_buf, p0, run_len, run_stride, scale, rows=None):
        return mod.ref_patch(Q_p, K_p, V_p, K_buf, V_buf, p0, scale, rows=rows)
    return ("ref_patch_strided", patch)


def _m_strided_run_offset(np_, mod):
    """Run r starts one row late for r >= 1."""
    def patch(Q_p, K_p, V_p, K_buf, V_buf, p0, run_len, run_stride, scale, rows=None):
        K_new, V_new = np_.array(K_buf, copy=True), np_.array(V_buf, copy=True)
        for r in range(Q_p.shape[2] // run_len):
            st = p0 + r * run_stride + (1 if r else 0)
            K_new[:, :, st:st + run_len] = K_p[:, :, r * run_len:(r + 1) * run_len]
            V_new[:, :, st:st + run_len] = V_p[:, :, r * run_len:(r + 1) * run_len]
        O, L = mod.ref_attn(Q_p, K_new, V_new, scale, rows=rows)
        return O, L, K_new, V_new
    return ("ref_patch_strided", patch)


def _m_decode_shift(np_, mod):
    def decode(x):
        x = np_.asarray(x)
        if x.dtype == np_.uint16:
            return (x.astype(np_.uint32) << 15).view(np_.float32).astype(np_.float64)
        return x.astype(np_.float64)
    return ("decode", decode)


def _m_relmae_denominator(np_, mod):
    def relmae(u, c):
        u, c = mod.decode(u), mod.decode(c)
        return float(np_.abs(c - u).sum() / np_.abs(c).sum())
    return ("ref_cfg_relmae", relmae)


HEAD_MUTANTS = [_m_no_scale, _m_lse_drops_max, _m_normalise_by_max, _m_softmax_wrong_axis, _m_k_for_v]
MOD_MUTANTS = [_m_merge_sign, _m_merge_lse_no_max, _m_merge_empty_nan, _m_cfg_wrong_base,
               _m_splice_off_by_one, _m_strided_runs_packed, _m_strided_run_offset,
               _m_decode_shift, _m_relmae_denominator]


@pytest.mark.parametrize("mutant", HEAD_MUTANTS + MOD_MUTANTS, ids=lambda f: f.__name__)
def test_pins_catch_planted_mistake(mutant):
    mod = _fresh_oracle()
    if mutant in HEAD_MUTANTS:
        name, fn = mutant(np)
    else:
        name, fn = mutant(np, mod)
    setattr(mod, name, fn)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except Exception:  # an assertion, or a crash on the broken shapes
            caught.append(pin.__name__)
    assert caught, f"no pin rejects mutant {mutant.__name__}"


# ---------------------------------------------------------------------------
# Regression fixture written by tests/golden/make_golden.py (oracle only).
# ---------------------------------------------------------------------------

def test_golden_regression():
    from tests.golden.make_golden import compute_cases

    with open(os.path.join(HERE, "golden", "oracle_small.json")) as f:
        stored = json.load(f)
    fresh = compute_cases()
    assert stored.keys() == fresh.keys()
    for name in stored:
        for key in stored[name]:
            a = np.array(stored[name][key], dtype=np.float64)
            b = np.array(fresh[name][key], dtype=np.float64)
            assert np.allclose(a, b, rtol=1e-12, atol=1e-12, equal_nan=True), (name, key)


def test_oracle_is_independent_of_product():
    """The oracle imports nothing from the HIP package and vice versa."""
    root = os.path.dirname(HERE)
    for fn in os.listdir(os.path.join(root, "oracle")):
        if fn.endswith(".py"):
            src = open(os.path.join(root, "oracle", fn)).read()
            assert "attention_attn_block_amd" not in src, fn
    pkg = os.path.join(root, "attention_attn_block_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, fn)).read()
                assert "import oracle" not in src and "from oracle" not in src, fn
