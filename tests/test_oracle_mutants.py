"""Plant plausible mistakes in a copy of the oracle's C source (on the CPU),
build each copy, and check that at least one pin rejects it.  This shows the
pins are strong enough to catch a dropped term, a wrong sign or index, a
transposed operand, a flipped kernel or a missing bounds check."""
import os
import tempfile

import pytest

from oracle import oracle as O
from tests import pins

SRC = os.path.join(os.path.dirname(O.__file__), "oracle.c")

# (name, text to replace, replacement, which occurrence (0-based))
MUTANTS = [
    ("flat-index wrap: no column bounds check",
     "if (yy >= 0 && yy < H && xx >= 0 && xx < W) v = map[yy * W + xx];",
     "{ int32_t q = yy * W + xx; if (q >= 0 && q < H * W) v = map[q]; }", 0),
    ("tap order transposed (dx-major)",
     "int32_t yy = y + (j / K - r), xx = x + (j % K - r);",
     "int32_t yy = y + (j % K - r), xx = x + (j / K - r);", 0),
    ("map not reset between frames",
     "for (int64_t c = 0; c < cells; ++c) map[c] = -1;",
     "if (t == 0) for (int64_t c = 0; c < cells; ++c) map[c] = -1;", 0),
    ("duplicate coordinate not detected",
     "if (map[p] != -1) { status = ORC_DUPLICATE; break; }", "", 0),
    ("forward drops the centre tap",
     "int32_t m = N[k * taps + j];\n            if (m < 0) continue;\n            const double *x",
     "int32_t m = N[k * taps + j];\n            if (m < 0 || j == taps / 2) continue;\n            const double *x", 0),
    ("forward flips the kernel (true convolution)",
     "const double *w = Wt + (int64_t)j * Ci * Co;",
     "const double *w = Wt + (int64_t)(taps - 1 - j) * Ci * Co;", 0),
    ("forward reads the own row instead of the neighbour",
     "const double *x = X + (int64_t)m * Ci;", "const double *x = X + k * Ci;", 0),
    ("forward drops the bias",
     "if (b)\n            for (int32_t o = 0; o < Co; ++o) acc[o] += b[o];", "", 0),
    ("dX gather without the mirrored tap",
     "int32_t m = N[k * taps + (taps - 1 - j)];", "int32_t m = N[k * taps + j];", 0),
    ("dX scatter with the wrong sign",
     "dX[(int64_t)m * Ci + i] += s;", "dX[(int64_t)m * Ci + i] -= s;", 0),
    ("dW with operands swapped between gathered and own row",
     "double xv = X[(int64_t)m * Ci + i];\n            const double *g = dY + k * Co;",
     "double xv = X[k * Ci + i];\n            const double *g = dY + (int64_t)m * Co;", 0),
    ("K x K offsets not centred (radius taken as K - 1 over 2 rounded up)",
     "const int taps = K * K, r = K / 2;", "const int taps = K * K, r = (K + 1) / 2;", 0),
    ("db drops the last token",
     "for (int64_t k = 0; k < n; ++k)\n        for (int32_t o = 0; o < Co; ++o) db[o]",
     "for (int64_t k = 0; k + 1 < n; ++k)\n        for (int32_t o = 0; o < Co; ++o) db[o]", 0),
    ("cross-attention scores not scaled",
     "srow[j] = scale * s;", "srow[j] = s;", 0),
    ("cross-attention softmax without the max shift",
     "for (int64_t j = 0; j < n; ++j) sum += exp(srow[j] - mx);\n        for (int64_t j = 0; j < n; ++j) {\n            double pj = exp(srow[j] - mx) / sum;",
     "for (int64_t j = 0; j < n; ++j) sum += exp(srow[j]);\n        for (int64_t j = 0; j < n; ++j) {\n            double pj = exp(srow[j]) / sum;", 0),
    ("adapter forward without the residual",
     "for (int64_t e = 0; e < n * C; ++e) Y[e] += X[e];", "", 0),
    ("adapter backward without the residual's gradient",
     "for (int64_t e = 0; e < n * C; ++e) dX[e] += dY[e];", "", 0),
    ("adapter dWu from the down-projected features",
     "orc_bwd_dw(H2, I, dY, dWu, n, r, C, 1);", "orc_bwd_dw(H1, I, dY, dWu, n, r, C, 1);", 0),
    ("adapter dbd from the upstream gradient",
     "orc_bwd_db(dH1, dbd, n, r);", "orc_bwd_db(dH2, dbd, n, r);", 0),
    ("adapter conv on the input instead of the down-projection",
     "orc_fwd(H1, N, Wc, bc, H2, n, r, r, taps);\n    orc_fwd(H2, I, Wu, bu, Y, n, r, C, 1);",
     "orc_fwd(X, N, Wc, bc, H2, n, r, r, taps);\n    orc_fwd(H2, I, Wu, bu, Y, n, r, C, 1);", 0),
    ("cross-attention lse without the shift added back",
     "lse[q] = mx + log(sum);", "lse[q] = log(sum);", 0),
    ("cross-attention dX drops the value term",
     "dX[j * d + c] = scale * key + val;", "dX[j * d + c] = scale * key;", 0),
    ("cross-attention dX drops the key term",
     "dX[j * d + c] = scale * key + val;", "dX[j * d + c] = val;", 0),
    ("cross-attention softmax backward without the row correction",
     "dS[q * n + j] = P[q * n + j] * (dS[q * n + j] - D);", "dS[q * n + j] = P[q * n + j] * dS[q * n + j];", 0),
    ("cross-attention dQ not scaled",
     "dQ[q * d + c] = scale * acc;", "dQ[q * d + c] = acc;", 0),
    ("cross-attention dQ contracts with the queries instead of the keys",
     "for (int64_t j = 0; j < n; ++j) acc += dS[q * n + j] * X[j * d + c];",
     "for (int64_t j = 0; j < n; ++j) acc += dS[q * n + j] * Q[q * d + c];", 0),
]


def _mutate(src, old, new, occ):
    pos = -1
    for _ in range(occ + 1):
        pos = src.index(old, pos + 1)
    return src[:pos] + new + src[pos + len(old):]


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_rejected(name, old, new, occ, tmp_path):
    src = open(SRC).read()
    assert old in src, f"mutation anchor not found: {name}"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(_mutate(src, old, new, occ))
    lib = O.compile_source(str(mpath), str(tmp_path / "libmutant.so"))
    orc = O.Oracle(lib)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin rejects the mutant '{name}'"
