"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that the pins in
test_oracle_pins.py catch every one of them.  A mutant that passes every pin would mean the
pins leave that part of the oracle unchecked."""
import importlib.util
import inspect
import os
import shutil
import subprocess

import pytest

import tests.test_oracle_pins as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mla_oracle.c")

# (name, code text to find, replacement, which occurrence in code to replace (1-based))
MUTATIONS = [
    ("rope sign", "yo[rope_off + j] = a * c - b * s;", "yo[rope_off + j] = a * c + b * s;", 1),
    ("rope pairing", "double b = xi[rope_off + 2 * j + 1];", "double b = xi[rope_off + half + j];", 1),
    ("rope frequency", "-2.0 * (double)j / (double)rope_dim", "-1.0 * (double)j / (double)rope_dim", 1),
    ("rope output slot", "yo[rope_off + half + j] = b * c + a * s;", "yo[rope_off + 2 * j + 1] = b * c + a * s;", 1),
    ("indexer relu dropped", "float r = (a > 0.0f) ? a : 0.0f;", "float r = a;", 1),
    ("indexer dim order", "for (int32_t d = 0; d < hd; ++d) a = fmaf(", "for (int32_t d = hd - 1; d >= 0; --d) a = fmaf(", 1),
    ("indexer unfused product", "a = fmaf(q[h * hd + d], k[d], a);", "a = q[h * hd + d] * k[d] + a;", 1),
    ("indexer weight index", "s = fmaf(w[h], r, s);", "s = fmaf(w[n_ih - 1 - h], r, s);", 1),
    ("topk tie rule", "return (a->t > b->t) - (a->t < b->t);", "return (a->t < b->t) - (a->t > b->t);", 1),
    ("topk output order", "qsort(sel, (size_t)nsel, sizeof(int32_t), orc_cmp_i32);", "", 1),
    ("topk n_valid ignored", "nsel[b] = orc_topk(scores + (int64_t)b * t_max, n_valid[b], k,", "nsel[b] = orc_topk(scores + (int64_t)b * t_max, t_max, k,", 1),
    ("absorbed W_UV offset", "const float *wuv = wuk + (int64_t)nope * L;", "const float *wuv = wuk + (int64_t)(nope - 1) * L;", 1),
    ("absorbed rope term dropped", "s[j] = sm_scale * (dl + dr);", "s[j] = sm_scale * dl;", 1),
    ("absorbed head index", "const float *wuk = kv_b + (int64_t)h * rows_per_head * L;", "const float *wuk = kv_b + (int64_t)(H - 1 - h) * rows_per_head * L;", 1),
    ("nonabsorbed scale dropped", "s[j] = sm_scale * (dn + dr);", "s[j] = (dn + dr);", 1),
    ("nonabsorbed value rows", "a += (double)wuv[(int64_t)jv * L + c] * (double)l[c];", "a += (double)wuk[(int64_t)jv * L + c] * (double)l[c];", 1),
    ("prefill excludes own key", "const int64_t nk = (int64_t)pos_base + i + 1;", "const int64_t nk = (int64_t)pos_base + i + (i > 0 ? 0 : 1);", 1),
    ("prefill ignores pos_base", "const int64_t nk = (int64_t)pos_base + i + 1;", "const int64_t nk = (int64_t)i + 1;", 1),
    ("prefill rope term dropped", "s[t] = sm_scale * (dn + dr);", "s[t] = sm_scale * dn;", 1),
    ("rmsnorm eps dropped", "double inv = 1.0 / sqrt(ms + eps);", "double inv = 1.0 / sqrt(ms);", 1),
    ("tiny layer rotates at position 0", "int32_t pos = t;", "int32_t pos = 0;", 1),
    ("tiny layer positions off by one", "int32_t pos = t;", "int32_t pos = t + 1;", 1),
    ("tiny layer query one position late", "orc_rope_interleave(qf, q, 1, H, qh, nope, rope, &pos, theta);",
     "{ int32_t qp = pos + 1; orc_rope_interleave(qf, q, 1, H, qh, nope, rope, &qp, theta); }", 1),
    ("cache write rmsnorm over the rope tail too", "for (int32_t c = 0; c < L; ++c) ms += (double)cj[c] * (double)cj[c];",
     "for (int32_t c = 0; c < L + rope; ++c) ms += (double)cj[c] * (double)cj[c];", 1),
    ("cache write gain reversed", "(kv_gain ? (double)kv_gain[c] : 1.0)", "(kv_gain ? (double)kv_gain[L - 1 - c] : 1.0)", 1),
    ("cache write rope key at the sequence index", "orc_rope_interleave(u, rc + row * rope, 1, 1, rope, 0, rope, pos + j, theta);",
     "orc_rope_interleave(u, rc + row * rope, 1, 1, rope, 0, rope, seq + j, theta);", 1),
    ("cache write paged offset dropped", "row = blk < 0 ? -1 : (int64_t)blk * bs + pos[j] % bs;",
     "row = blk < 0 ? -1 : (int64_t)blk * bs;", 1),
    ("cache write layernorm without the mean", "y[c] = ((double)kj[c] - mean) * is", "y[c] = ((double)kj[c]) * is", 1),
    ("cache write variance of raw values", "var += ((double)kj[c] - mean) * ((double)kj[c] - mean);",
     "var += (double)kj[c] * (double)kj[c];", 1),
    ("cache write indexer rope slice at 0", "orc_rope_interleave(y, ic + row * hd, 1, 1, hd, ix_off, ix_rdim, pos + j, theta);",
     "orc_rope_interleave(y, ic + row * hd, 1, 1, hd, 0, ix_rdim, pos + j, theta);", 1),
    ("cache write beta dropped", "+ (beta ? (double)beta[c] : 0.0);", ";", 1),
    ("e4m3 subnormal exponent", "ldexp((double)m, -9)", "ldexp((double)m, -10)", 1),
    ("e4m3 exponent bias", "ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)", 1),
    ("e4m3 mantissa weight", "ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 16.0, e - 7)", 1),
    ("e2m1 subnormal value", "double v = e == 0 ? 0.5 * (double)m", "double v = e == 0 ? (double)m", 1),
    ("mxfp4 nibble order", "unsigned nib = (j & 1) ? (c[j / 2] >> 4) : (c[j / 2] & 15);",
     "unsigned nib = (j & 1) ? (c[j / 2] & 15) : (c[j / 2] >> 4);", 1),
    ("e8m0 bias", "ldexp(1.0, (int)x[j / 32] - 127)", "ldexp(1.0, (int)x[j / 32] - 128)", 1),
    ("mxfp4 block size", "const uint8_t *x = (const uint8_t *)scales + r * (cols / 32);",
     "const uint8_t *x = (const uint8_t *)scales + r * (cols / 16);", 1),
    ("int8 read unsigned", "(double)(int8_t)c[j]", "(double)c[j]", 1),
    ("row scale of the wrong row", "double sc = (double)((const float *)scales)[r];",
     "double sc = (double)((const float *)scales)[0];", 1),
]


def _pin_functions():
    out = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if name.startswith("test_") and "oracle" in inspect.signature(fn).parameters:
            out.append(fn)
    return out


def _call(fn, mod):
    params = inspect.signature(fn).parameters
    kw = {"oracle": mod}
    if "dims" in params:
        kw["dims"] = (4, 16, 8, 16, 32, 50)
    fn(**kw)


def _mutant(tmp_path, find, repl, occ):
    src = open(SRC).read()
    def in_comment(i):
        return src.rfind("/*", 0, i) > src.rfind("*/", 0, i)

    idx, seen = -1, 0
    while seen < occ:
        idx = src.find(find, idx + 1)
        assert idx >= 0, f"mutation target not found in code: {find!r}"
        if not in_comment(idx):
            seen += 1
    src = src[:idx] + repl + src[idx + len(find):]
    d = tmp_path / "oracle_mut"
    d.mkdir()
    (d / "mla_oracle.c").write_text(src)
    shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), d / "__init__.py")
    lib = d / "libmla_oracle.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fopenmp",
                    "-o", str(lib), str(d / "mla_oracle.c"), "-lm"], check=True)
    spec = importlib.util.spec_from_file_location(f"oracle_mut_{abs(hash(find + repl))}", d / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod._LIB = str(lib)
    mod._load()
    return mod


@pytest.mark.parametrize("name,find,repl,occ", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, name, find, repl, occ):
    mod = _mutant(tmp_path, find, repl, occ)
    caught = []
    for fn in _pin_functions():
        try:
            _call(fn, mod)
        except (AssertionError, FloatingPointError, ValueError):
            caught.append(fn.__name__)
    assert caught, f"no pin detects the planted mistake '{name}'"
