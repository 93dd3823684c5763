"""The pins must catch plausible mistakes. Each case plants one mistake in a
copy of the oracle's C source (a flipped sign, a transposed operand, a wrong
index or GQA map, a dropped term), builds it on the CPU, points the oracle
module at it, and runs the pin suite: at least one pin must fail. Nothing
here touches the HIP library or a GPU."""
import ctypes
import inspect
import os

import pytest

import oracle as O
from oracle import build as ob
from tests import test_oracle_pins as pins

MUTANTS = [
    ("delta sign", "delta[r] = beta * (v[r] - u[r]);", "delta[r] = beta * (v[r] + u[r]);"),
    ("decay on rows", "S[(size_t)r * K + c] *= decay[c];", "S[(size_t)r * K + c] *= decay[r % K];"),
    ("rank-1 transposed", "S[(size_t)r * K + c] += delta[r] * k[c];",
     "S[(size_t)r * K + c] += delta[c % V] * k[r % K];"),
    ("output with k", "acc += S[(size_t)r * K + c] * q[c];", "acc += S[(size_t)r * K + c] * k[c];"),
    ("residual with q", "acc += S[(size_t)r * K + c] * k[c];\n        u[r] = acc;",
     "acc += S[(size_t)r * K + c] * q[c];\n        u[r] = acc;"),
    ("dt_bias sign", "orc_softplus(a + dt_bias)", "orc_softplus(a - dt_bias)"),
    ("A_log not exponentiated", "*g = -exp(A_log) *", "*g = -A_log *"),
    ("beta sign", "*beta = orc_sigmoid(b);", "*beta = orc_sigmoid(-b);"),
    ("GQA interleaved", "const int h = hv / G;\n            const double *row = qkv + (size_t)bi * qkv_stride;\n            double *q = malloc",
     "const int h = hv % H;\n            const double *row = qkv + (size_t)bi * qkv_stride;\n            double *q = malloc"),
    ("q not scaled", "q[c] = qin[c] * qn * scale;", "q[c] = qin[c] * qn;"),
    ("k not normalised", "k[c] = kin[c] * kn;", "k[c] = kin[c];"),
    ("norm sum not mean", "sqrt(ss / V + eps)", "sqrt(ss + eps)"),
    ("norm act swapped", "act == ORC_ACT_SIGMOID ? orc_sigmoid(gate[r]) : orc_silu(gate[r])",
     "act == ORC_ACT_SIGMOID ? orc_silu(gate[r]) : orc_sigmoid(gate[r])"),
    ("conv no roll", "cs[j] = win[j + 1];", "cs[j] = win[j];"),
    ("conv taps reversed", "acc += w[(size_t)c * W + j] * win[j];", "acc += w[(size_t)c * W + j] * win[W - 1 - j];"),
    ("kda gate sign", "return lb * orc_sigmoid(raw_g);", "return lb * orc_sigmoid(-raw_g);"),
    ("kda keeps slot 0", "if (s <= 0 || s >= num_slots)\n                continue;\n            const size_t C",
     "if (s < 0 || s >= num_slots)\n                continue;\n            const size_t C"),
    ("replay without decay", "S[(size_t)r * K + c] = dj * S[(size_t)r * K + c] +",
     "S[(size_t)r * K + c] = S[(size_t)r * K + c] +"),
    ("no flush", "if (p == L - 1)\n                memcpy(ck, S", "if (p == L)\n                memcpy(ck, S"),
    ("ring stores unrounded delta", "dring[(size_t)p * V + r] = orc_round_fmt(delta[r], ring_fmt);",
     "dring[(size_t)p * V + r] = delta[r];"),
    ("16-bit state not rounded", "S[e] = orc_round_fmt(S[e], state_fmt);", "S[e] = S[e];"),
    ("mamba drops input", "Bm[(size_t)bi * N + n];\n                h[n] = dA * h[n] + dB * xv;",
     "Bm[(size_t)bi * N + n];\n                h[n] = dA * h[n] + dB;"),
    ("mamba no D skip", "acc += Dv[d] * xv;\n            if (z)", "acc += Dv[d];\n            if (z)"),
    ("scan drops input", "Bm[bt * N + n];\n                    h[n] = dA * h[n] + dB * xv;",
     "Bm[bt * N + n];\n                    h[n] = dA * h[n] + dB;"),
    ("scan ignores stored state", "if (zero_init)\n                for (int n = 0; n < N; ++n)",
     "if (1)\n                for (int n = 0; n < N; ++n)"),
    ("scan drops last token", "for (int t = 0; t < len; ++t) {", "for (int t = 0; t < len - 1; ++t) {"),
    ("scan reads token-major B", "const double dB = dtv * Bm[bt * N + n];",
     "const double dB = dtv * Bm[((size_t)t * B + bi) * N + n];"),
    ("multi reads token-major gates", "memcpy(a_t + (size_t)bi * HV, a + bt * HV, sizeof(double) * HV);",
     "memcpy(a_t + (size_t)bi * HV, a + ((size_t)t * B + bi) * HV, sizeof(double) * HV);"),
    ("multi ignores lengths", "idx_t[bi] = t < len ? idx[bi] : -1;", "idx_t[bi] = idx[bi];"),
    ("bf16 rounding truncates", "double r = nearbyint(x / ulp) * ulp;", "double r = trunc(x / ulp) * ulp;"),
]


def _pin_functions():
    fns = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        params = inspect.signature(fn).parameters
        if "L" in params:
            fns += [(f"{name}[L={L}]", lambda fn=fn, L=L: fn(L)) for L in (1, 3, 8)]
        elif "fmt" in params:
            fns += [(f"{name}[fmt={f}]", lambda fn=fn, f=f: fn(f)) for f in (O.FMT_BF16, O.FMT_F16)]
        elif not params:
            fns.append((name, fn))
    return fns


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(mutant, tmp_path, monkeypatch):
    name, old, new = mutant
    with open(ob.SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site for '{name}' not unique in the oracle source"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = ob.build(src=str(mpath), lib=str(tmp_path / "libmutant.so"))
    monkeypatch.setattr(O, "_LIB", O.configure(ctypes.CDLL(lib)))
    caught = []
    for pname, fn in _pin_functions():
        try:
            fn()
        except Exception:  # an assertion, or a shape/NaN error the mistake provokes
            caught.append(pname)
    assert caught, f"no pin caught the planted mistake '{name}'"


def test_unmutated_copy_passes_every_pin(tmp_path, monkeypatch):
    lib = ob.build(src=ob.SRC, lib=str(tmp_path / "libcopy.so"))
    monkeypatch.setattr(O, "_LIB", O.configure(ctypes.CDLL(lib)))
    for pname, fn in _pin_functions():
        fn()
    assert os.path.exists(lib)
