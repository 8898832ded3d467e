"""Planted mistakes in the oracle must be caught by the pins.

Each case below copies one oracle function (or the C source), plants a
plausible mistake (a dropped term, a flipped sign, a wrong index, a transposed
operand), and checks that at least one of the pin checks fails for the
mutant while the unmodified oracle passes it.  Everything runs on the CPU.
"""
import ctypes
import inspect
import os
import subprocess
import tempfile
import textwrap

import numpy as np
import pytest

import oracle

from test_oracle_pins import (orthonormal_keys, rand_problem, rel_err)


def _pins_pass(mod_fns) -> bool:
    """Run the key chunked-form pins with the given replacement functions
    patched into the oracle module.  Returns True when all pins hold."""
    saved = {name: getattr(oracle, name) for name in mod_fns}
    try:
        for name, fn in mod_fns.items():
            setattr(oracle, name, fn)
        rng = np.random.default_rng(123)
        # recurrent == chunked, square state so transposes are not shape errors
        q, k, v, g, beta, cu, s0 = rand_problem(rng, [29, 1, 40], 2, 6, 6)
        for init in (s0, None):
            o1, s1, _ = oracle.recurrent(q, k, v, g, beta, cu, init)
            r = oracle.chunked(q, k, v, g, beta, cu, 8, init)
            if not (rel_err(r["o"], o1) < 1e-10 and rel_err(r["state_out"], s1) < 1e-10):
                return False
        # L, M against the brute-force products
        _, k2, v2, g2, b2, _, _ = rand_problem(rng, [7], 1, 6, 6, state0=False)
        loc = oracle.chunk_local(k2[:, 0], v2[:, 0], g2[:, 0], b2[:, 0])
        if rel_err(loc["M"], oracle.transfer_bruteforce(k2[:, 0], g2[:, 0], b2[:, 0])) > 1e-10:
            return False
        return True
    except Exception:
        return False
    finally:
        for name, fn in saved.items():
            setattr(oracle, name, fn)


def _mutant(fn, old, new):
    src = textwrap.dedent(inspect.getsource(fn))
    assert old in src, f"mutation anchor {old!r} not found in {fn.__name__}"
    src = src.replace(old, new, 1)
    ns = dict(vars(oracle))
    exec(compile(src, f"<mutant {fn.__name__}>", "exec"), ns)
    return ns[fn.__name__]


PY_MUTATIONS = [
    ("chunk_local", "k=-1)", "k=-2)"),                                  # first subdiagonal dropped
    ("chunk_local", "bc[:, None] * Gamma", "bc[None, :] * Gamma"),      # wrong beta index
    ("chunk_local", "(bc * gamma)[:, None]", "bc[:, None]"),           # gamma dropped in W
    ("chunk_local", "gamma[-1] * np.eye(dk) - W.T", "gamma[-1] * np.eye(dk) + W.T"),  # sign
    ("chunk_local", "L = Ut.T @ DK", "L = Ut.T @ Kc"),                  # decay D dropped
    ("chunk_local", "Gamma * KK", "Gamma.T * KK"),                      # transposed decay
    ("chunk_out", 'loc["W"] @ S0.T', 'loc["W"] @ S0'),                   # transposed state
    ("chunk_out", '* loc["Gamma"]', '* loc["Gamma"].T'),                # transposed mask
    ("chunk_out", 'loc["gamma"][:, None] *', ''),                       # gamma dropped
    ("fixup", "S @ M_list[c]", "M_list[c] @ S"),                        # wrong orientation
    ("fixup", "start = 1", "start = 0"),                                # L_0 applied twice
    ("chunk_gates", "np.exp(G[-1] - G)", "np.exp(G - G[0])"),            # wrong decay anchor
]


def test_unmodified_oracle_passes_the_mutation_pins():
    assert _pins_pass({})


@pytest.mark.parametrize("fname,old,new", PY_MUTATIONS)
def test_python_mutant_is_caught(fname, old, new):
    fn = getattr(oracle, fname)
    assert not _pins_pass({fname: _mutant(fn, old, new)})


C_MUTATIONS = [
    ("s[j] - b * sk * kk[j]", "s[j] + b * sk * kk[j]"),          # erase sign
    ("alpha * (s[j] - b * sk * kk[j])", "alpha * s[j] - b * sk * kk[j]"),  # decay not on erase
    ("+ b * vi * kk[j]", "+ vi * kk[j]"),                          # beta dropped on write
    ("oi += s[j] * qq[j]", "oi += s[j] * kk[j]"),                  # wrong query
    ("exp(g[th])", "exp(0.5 * g[th])"),                           # wrong gate
]


def _c_pins_pass(lib_path) -> bool:
    lib = ctypes.CDLL(lib_path)
    ref = oracle._lib()
    lib.oracle_recurrent.argtypes = ref.oracle_recurrent.argtypes
    lib.oracle_recurrent.restype = ctypes.c_int
    lib.oracle_max_threads.restype = ctypes.c_int
    saved = oracle._lib_handle
    oracle._lib_handle = lib
    try:
        rng = np.random.default_rng(7)
        q, k, v, g, beta, cu, s0 = rand_problem(rng, [6], 1, 4, 3)
        o, sT, _ = oracle.recurrent(q, k, v, g, beta, cu, s0)
        ref_s = oracle.state_bruteforce(s0[0, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0])
        if rel_err(sT[0, 0], ref_s) > 1e-12:
            return False
        St = oracle.state_bruteforce(s0[0, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0])
        if rel_err(o[-1, 0], St @ q[-1, 0]) > 1e-12:
            return False
        return True
    finally:
        oracle._lib_handle = saved


def _build_c(src_text, out_dir):
    src = os.path.join(out_dir, "m.c")
    so = os.path.join(out_dir, "m.so")
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fopenmp", "-shared", "-fPIC", src,
                           "-o", so, "-lm"])
    return so


def test_unmodified_c_oracle_passes():
    with open(os.path.join(os.path.dirname(oracle.__file__), "gdr_oracle.c")) as f:
        text = f.read()
    with tempfile.TemporaryDirectory() as d:
        assert _c_pins_pass(_build_c(text, d))


@pytest.mark.parametrize("old,new", C_MUTATIONS)
def test_c_mutant_is_caught(old, new):
    with open(os.path.join(os.path.dirname(oracle.__file__), "gdr_oracle.c")) as f:
        text = f.read()
    assert old in text
    with tempfile.TemporaryDirectory() as d:
        assert not _c_pins_pass(_build_c(text.replace(old, new, 1), d))
