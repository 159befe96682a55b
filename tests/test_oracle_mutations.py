"""The oracle's pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of oracle/oracle.c (on the CPU only),
builds it, and runs the oracle pin suites against that build in a child
process: at least one pin must fail.  This is what makes the pins a check on
the oracle rather than a restatement of it.
"""

import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PIN_FILES = ["tests/test_oracle_basics.py", "tests/test_oracle_attention.py",
             "tests/test_oracle_quant.py"]

# (name, text to find, replacement, which occurrence (0-based) to replace)
MUTATIONS = [
    ("drop_scale", "*logit = p->scale * dot + m;", "*logit = dot + m;", 0),
    ("drop_mask_term", "*logit = p->scale * dot + m;", "*logit = p->scale * dot;", 0),
    ("strict_exclusion", "if (m <= ORC_MASKED)\n        return 0;\n    uint32_t D",
     "if (m < ORC_MASKED)\n        return 0;\n    uint32_t D", 0),
    ("gqa_modulo", "uint32_t hk = h / (p->n_heads / p->n_kv_heads); /* GQA",
     "uint32_t hk = h % p->n_kv_heads; /* GQA", 0),
    ("causal_off_by_one", "(int64_t)j <= last) ? 0.0 : ORC_MASKED;",
     "(int64_t)j < last) ? 0.0 : ORC_MASKED;", 0),
    ("head_major_output", "i = r / p->n_heads; /* out row",
     "i = r % p->q_l; h = r / p->q_l; if (0) /* out row", 0),
    ("no_normalisation", "o[d] = (s > 0.0) ? o[d] / s : 0.0; /* R2 */",
     "o[d] = o[d];", 0),
    ("mask_prefix_short", "for (uint32_t j = 0; j < base; ++j)\n            row[j] = 0.0f;",
     "for (uint32_t j = 1; j < base; ++j)\n            row[j] = 0.0f;", 0),
    ("f16_exponent_bias", "v = ldexp((double)(1024 + m), e - 25);",
     "v = ldexp((double)(1024 + m), e - 24);", 0),
    ("code_order_reversed", "uint32_t code = (word >> ((d % pf) * p->bits))",
     "uint32_t code = (word >> ((pf - 1 - d % pf) * p->bits))", 0),
    ("group_index_modulo", "double sc = q_elem(p, scales, tok * ngroups + d / p->group);",
     "double sc = q_elem(p, scales, tok * ngroups + (d / p->group + 1) % ngroups);", 0),
    ("bf16_exponent_bias", "v = ldexp((double)(128 + m), e - 134);",
     "v = ldexp((double)(128 + m), e - 133);", 0),
    ("bf16_mantissa_width", "int m = b & 0x7f;", "int m = b & 0x3f;", 0),
    ("f32_read_as_f16", "        return (double)((const float *)base)[idx];",
     "        return orc_f16_to_f64(((const uint16_t *)base)[idx]);", 0),
    ("bias_dropped", "return sc * (double)code + bi;", "return sc * (double)code;", 0),
    ("sink_scaled", "sink = (double)p->sinks[q_idx % p->nq]; /* R12 */",
     "sink = p->scale * (double)p->sinks[q_idx % p->nq]; /* R12 */", 0),
    ("quant_kv_modulo", "uint32_t kv = q_idx / (p->nq / p->nkv); /* [FQS]",
     "uint32_t kv = q_idx % p->nkv; /* [FQS]", 0),
    ("lse_sign", "double f = exp(m[pr] - mstar);", "double f = exp(mstar - m[pr]);", 0),
    ("mask_row_stride", "return (double)p->mask[(size_t)i * p->mask_stride + j];",
     "return (double)p->mask[(size_t)i * p->kv_seq_len + j];", 0),
    ("key_transposed", "size_t krow = ((size_t)hk * p->kv_capacity + j) * D;",
     "size_t krow = ((size_t)j * p->n_kv_heads + hk) * D;", 0),
    ("window_off_by_one", "(uint64_t)t + p->window <= (uint64_t)p->kv_seq_len - 1u",
     "(uint64_t)t + p->window < (uint64_t)p->kv_seq_len - 1u", 0),
    ("window_from_start", "(uint64_t)t + p->window <= (uint64_t)p->kv_seq_len - 1u",
     "(uint64_t)t >= p->window", 0),
    ("window_start_exclusive", "return (j >= p->window_start && (int64_t)j <= last)",
     "return (j > p->window_start && (int64_t)j <= last)", 0),
    ("window_start_ignored", "return (j >= p->window_start && (int64_t)j <= last)",
     "return ((int64_t)j <= last)", 0),
    ("bool_inverted", "return p->mask_bool[cell] != 0u ? 0.0 : ORC_MASKED;",
     "return p->mask_bool[cell] == 0u ? 0.0 : ORC_MASKED;", 0),
    ("bool_low_bit_only", "return p->mask_bool[cell] != 0u ? 0.0 : ORC_MASKED;",
     "return (p->mask_bool[cell] & 1u) ? 0.0 : ORC_MASKED;", 0),
]


def _apply(src, find, repl, occ):
    idx = -1
    for _ in range(occ + 1):
        idx = src.index(find, idx + 1)
    return src[:idx] + repl + src[idx + len(find):]


def _run_mutant(name, find, repl, occ, tmpdir):
    src = open(SRC).read()
    assert find in src, "mutation %s no longer matches oracle.c" % name
    mutated = _apply(src, find, repl, occ)
    c_path = os.path.join(tmpdir, name + ".c")
    so_path = os.path.join(tmpdir, name + ".so")
    open(c_path, "w").write(mutated)
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
                    "-std=c11", "-w", "-o", so_path, c_path, "-lm", "-lpthread"],
                   check=True)
    env = dict(os.environ, TREEATTN_ORACLE_LIB=so_path)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PIN_FILES], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    return name, r.returncode


def test_every_planted_mistake_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            futs = [ex.submit(_run_mutant, *m, tmp) for m in MUTATIONS]
            results = dict(f.result() for f in futs)
    survivors = [n for n, rc in results.items() if rc == 0]
    assert not survivors, "mistakes not caught by any pin: %s" % survivors
