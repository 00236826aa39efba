"""Each plausible mistake planted in a copy of the oracle source is caught by some pin.

The mutants are compiled from text edits of oracle/attn_oracle.c into a
temporary directory and run, each in its own process, through tests/pins.py.
Nothing here touches the GPU.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from oracle import oracle as oracle_mod

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, text in attn_oracle.c, replacement)
MUTANTS = [
    ("causal_off_by_one", "c->causal && j > i + delta", "c->causal && j >= i + delta"),
    ("causal_top_left", "const long long delta = k_len - q_len;", "const long long delta = 0;"),
    ("delta_sign", "const long long delta = k_len - q_len;",
     "const long long delta = q_len - k_len;"),
    ("gqa_interleaved", "const int hk = h / G;", "const int hk = h % c->Hkv;"),
    ("band_skips_d0", "if (dd >= 0 && dd < c->E)", "if (dd > 0 && dd < c->E)"),
    ("band_one_too_far", "if (dd >= 0 && dd < c->E)", "if (dd >= 0 && dd <= c->E)"),
    ("band_index_flipped", "long long dd = i + delta - j;", "long long dd = j - i - delta;"),
    ("bias_dropped", "sj += widen(c->bias[", "sj += 0.0 * widen(c->bias["),
    ("bias_wrong_head", "c->bias[((q_off + i) * c->Hq + h)", "c->bias[((q_off + i) * c->Hq + hk)"),
    ("bias_scaled", "double sj = c->scale * dot;\n        if (c->bias) {",
     "double sj = dot;\n        if (c->bias) {"),
    ("lse_drops_max", "*lse = m + log(l);", "*lse = log(l);"),
    ("scale_dropped", "double sj = c->scale * dot;", "double sj = dot;"),
    ("fp16_exponent", "expo - 25);", "expo - 24);"),
    ("fp16_subnormal", "ldexp((double)mant, -24);", "ldexp((double)mant, -25);"),
    ("q_uses_k_offset", "c->q + ((q_off + i) * c->Hq + h)", "c->q + ((k_off + i) * c->Hq + h)"),
    ("k_uses_q_offset", "c->k + ((k_off + j) * c->Hkv + hk)", "c->k + ((q_off + j) * c->Hkv + hk)"),
    ("seqused_ignored", "if (c->seqused_k) *k_len = c->seqused_k[b];", ""),
    ("no_normalise", "for (int d = 0; d < c->Dv; d++) o[d] /= l;", ""),
    ("v_stride_D", "c->v + ((k_off + j) * c->Hkv + hk) * (long long)c->Dv",
     "c->v + ((k_off + j) * c->Hkv + hk) * (long long)c->D"),
    ("empty_row_lse_zero", "*lse = -INFINITY;\n        return;", "*lse = 0.0;\n        return;"),
    ("combine_weight_uses_max", "double w = exp(lse_parts[(long long)s * n_rows + r] - L);",
     "double w = exp(lse_parts[(long long)s * n_rows + r] - M);"),
    ("combine_lse_drops_max", "double L = M + log(sum);", "double L = log(sum);"),
    ("bf16_widen_shift", "((uint32_t)b) << 16;", "((uint32_t)b) << 15;"),
]


def _run_mutant(src_text, name, old, new, tmpdir):
    assert src_text.count(old) == 1, f"mutation {name}: pattern must occur exactly once"
    path_c = os.path.join(tmpdir, f"{name}.c")
    path_so = os.path.join(tmpdir, f"lib{name}.so")
    with open(path_c, "w") as f:
        f.write(src_text.replace(old, new))
    oracle_mod.build(force=True, src=path_c, out=path_so)
    code = ("import sys; sys.path.insert(0, %r); from oracle.oracle import OracleLib; "
            "from tests import pins; f = pins.run_all(OracleLib(%r)); "
            "print('FAILED_PINS', f); sys.exit(0 if f else 3)" % (REPO, path_so))
    env = dict(os.environ, OMP_NUM_THREADS="2", PYTHONWARNINGS="ignore")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       timeout=300)
    return name, r.returncode, r.stdout[-400:], r.stderr[-400:]


def test_every_mutant_is_caught(tmp_path):
    with open(os.path.join(REPO, "oracle", "attn_oracle.c")) as f:
        src = f.read()
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(lambda m: _run_mutant(src, *m, str(tmp_path)), MUTANTS))
    survivors = [(n, out, err) for n, rc, out, err in results if rc == 3]
    assert not survivors, f"mutants not caught by any pin: {survivors}"
    for n, rc, out, err in results:
        # exit 0: the run finished and at least one pin failed
        assert rc == 0, (n, rc, out, err)


def test_unmutated_source_passes_all_pins(tmp_path):
    with open(os.path.join(REPO, "oracle", "attn_oracle.c")) as f:
        src = f.read()
    name, rc, out, err = _run_mutant(src, "identity", "int oracle_combine(",
                                     "int oracle_combine(", str(tmp_path))
    assert rc == 3, (rc, out, err)  # exit 3 = no pin failed
