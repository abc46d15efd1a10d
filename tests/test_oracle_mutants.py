"""Planted mistakes in the oracle must each fail at least one pin.

Each mutant is a copy of ``oracle/sgmv_oracle.c`` with one plausible mistake
(a dropped term or factor, a wrong sign, index or stride, a transposed
operand, an off-by-one segment bound, a wrong rounding), built with gcc into
a temporary directory and run through every pin. The real oracle is never
modified."""
import tempfile
from pathlib import Path

import numpy as np
import pytest

import oracle as oracle_pkg

from . import oracle_pins as pins

# (name, text to replace, replacement, which occurrence: 0 = every one, n = the n-th)
MUTANTS = [
    ("scale_missing_div_r", "double scale = alpha / (double)r;", "double scale = alpha;", 0),
    ("scale_dropped", "Y[m * d_out + n] += scale * acc;", "Y[m * d_out + n] += acc;", 0),
    ("assign_not_accumulate", "Y[m * d_out + n] += scale * acc;", "Y[m * d_out + n] = scale * acc;", 0),
    ("wrong_sign_shrink", "acc += x * a;", "acc -= x * a;", 0),
    ("wrong_sign_expand", "Y[m * d_out + n] += scale * acc;", "Y[m * d_out + n] -= scale * acc;", 0),
    ("A_transposed", "a_base + j * d_in + i", "a_base + i * r + j", 0),
    ("B_transposed", "b_base + j * d_out + n", "b_base + n * r + j", 0),
    # wrong adapter, kept inside the pool so the mutant reads no memory it does not own
    ("wrong_adapter_shrink", "int64_t k = seg_adapter[s];",
     "int64_t k = (seg_adapter[s] + 1) % num_adapters;", 1),
    ("wrong_adapter_expand", "int64_t k = seg_adapter[s];",
     "int64_t k = (seg_adapter[s] + 1) % num_adapters;", 2),
    ("segment_end_off_by_one", "clamp_row(seg_start[s + 1], M)", "clamp_row(seg_start[s + 1] - 1, M)", 1),
    ("segment_start_off_by_one", "clamp_row(seg_start[s], M)", "clamp_row(seg_start[s] + 1, M)", 2),
    ("dropped_last_k", "i < d_in; ++i", "i < d_in - 1; ++i", 0),
    ("dropped_last_rank", "for (int64_t j = 0; j < r; ++j)\n                    acc +=",
     "for (int64_t j = 0; j + 1 < r; ++j)\n                    acc +=", 0),
    ("bf16_widen_shift", "<< 16;", "<< 15;", 0),
    ("bf16_round_truncates", "nearbyint(ldexp(f, 8))", "trunc(ldexp(f, 8))", 0),
    ("bf16_round_7_bits", "nearbyint(ldexp(f, 8)), e - 8", "nearbyint(ldexp(f, 7)), e - 7", 0),
    ("adapter_stride", "k * (int64_t)r * d_in", "k * (int64_t)d_in", 0),
    ("V_transposed_store", "V[m * r + j] = acc;", "V[j * M + m] = acc;", 0),
    # binary32 output rounding: truncation toward zero, and rounding to bf16 width
    ("f32_round_truncates", "out[i] = (float)in[i];",
     "{ float f = (float)in[i]; if (fabs((double)f) > fabs(in[i])) f = nextafterf(f, 0.0f); out[i] = f; }", 0),
    ("f32_round_bf16_width", "out[i] = (float)in[i];",
     "{ int e; double f = frexp(in[i], &e); out[i] = (float)ldexp(nearbyint(ldexp(f, 8)), e - 8); }", 0),
]


def _mutate(src: str, old: str, new: str, which: int) -> str:
    assert old in src, old
    if which == 0:
        return src.replace(old, new)
    pos = -1
    for _ in range(which):
        pos = src.index(old, pos + 1)
    return src[:pos] + new + src[pos + len(old):]


@pytest.mark.parametrize("name,old,new,which", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, which):
    src = oracle_pkg.SOURCE.read_text()
    with tempfile.TemporaryDirectory() as tmp:
        c = Path(tmp) / "mutant.c"
        c.write_text(_mutate(src, old, new, which))
        lib = oracle_pkg.build(source=c, output=Path(tmp) / "libmutant.so")
        orc = oracle_pkg.Oracle(lib)
        failed = []
        for pin in pins.ALL_PINS:
            try:
                pin(orc)
            except (AssertionError, ValueError):
                failed.append(pin.__name__)
        assert failed, f"mutant {name} passed every pin"


# Planted mistakes in the oracle's gather/scatter layer (Python): each must
# fail the per-token pin.
def _inverse(rows):
    return np.argsort(np.asarray(rows, np.int64))


class _GatherInverse(oracle_pkg.Oracle):
    def shrink_gather(self, X, A_pool, seg_start, seg_adapter, rows):
        return super().shrink_gather(X, A_pool, seg_start, seg_adapter, _inverse(rows))


class _NoGather(oracle_pkg.Oracle):
    def shrink_gather(self, X, A_pool, seg_start, seg_adapter, rows):
        return self.shrink(X, A_pool, seg_start, seg_adapter)


class _ScatterInverse(oracle_pkg.Oracle):
    def expand_scatter(self, Y_in, V, B_pool, seg_start, seg_adapter, rows, alpha):
        return super().expand_scatter(Y_in, V, B_pool, seg_start, seg_adapter, _inverse(rows), alpha)


class _NoScatter(oracle_pkg.Oracle):
    def expand_scatter(self, Y_in, V, B_pool, seg_start, seg_adapter, rows, alpha):
        return self.expand(Y_in, V, B_pool, seg_start, seg_adapter, alpha)


@pytest.mark.parametrize("cls", [_GatherInverse, _NoGather, _ScatterInverse, _NoScatter],
                         ids=lambda c: c.__name__.strip("_"))
def test_gather_mutant_is_caught(cls):
    orc = cls()
    with pytest.raises(AssertionError):
        pins.pin_gather_per_token(orc)
