"""The oracle's pins have teeth: plausible mistakes planted in copies of
oracle.c (on the CPU only) must each make the pin suite fail.

Each mutant is one small textual change -- a dropped term, an off-by-one, a
wrong sign, a wrong index, a transposed layout -- compiled to a temporary
library that the pin suite then loads in a subprocess.
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "positions drop computed tokens": ("const int32_t pos = nct[r] + t;", "const int32_t pos = t;"),
    "slot drops block size factor": ("(int64_t)phys * block_size + pos % block_size",
                                     "(int64_t)phys + pos % block_size"),
    "slot uses logical block": ("const int32_t phys = block_table[(int64_t)r * bt_stride + logical];",
                                "const int32_t phys = logical;"),
    "logits index off by one": ("logits_indices[r] = qsl[r + 1] - 1;", "logits_indices[r] = qsl[r + 1];"),
    "qsl tail not padded": ("qsl[k] = total;", "qsl[k] = 0;"),
    "seq_lens drop scheduled": ("seq_lens[r] = nct[r] + nst[r];", "seq_lens[r] = nct[r];"),
    "causal top-left alignment": ("const int32_t p = L - q_len + (row - qsl[r]);",
                                  "const int32_t p = (row - qsl[r]);"),
    "causal excludes diagonal": ("for (int32_t j = 0; j <= p; ++j) {\n            double acc",
                                 "for (int32_t j = 0; j < p; ++j) {\n            double acc"),
    "scale dropped": ("s[j] = scale * acc;", "s[j] = acc;"),
    "softmax sign flipped": ("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    "gqa interleaved heads": ("for (int32_t h = g * group; h < (g + 1) * group; ++h) {",
                              "for (int32_t h = g; h < num_q_heads; h += num_kv_heads) {"),
    "value tiles in token-major order": (
        "const int64_t tile = (int64_t)(dim / dw) * (block_size / tg) + tok / tg;",
        "const int64_t tile = (int64_t)(tok / tg) * (head_dim / dw) + dim / dw;"),
    "value tile transposed inside": (
        "return run + tile * dw * tg + (int64_t)(dim % dw) * tg + tok % tg;",
        "return run + tile * dw * tg + (int64_t)(tok % tg) * dw + dim % dw;"),
    "gather offset uses block index": ("const int32_t off = j % block_size;\n        for (int32_t c = 0; c < head_dim; ++c) {\n          if (kv_dtype",
                                       "const int32_t off = (j / block_size) % block_size;\n        for (int32_t c = 0; c < head_dim; ++c) {\n          if (kv_dtype"),
    "kv write uses key layout for values": (
        "const int64_t dv = orc_v_elem(block, h, off, c, num_kv_heads, block_size, head_dim);",
        "const int64_t dv = orc_k_elem(block, h, off, c, num_kv_heads, block_size, head_dim);"),
    "bf16 widening wrong half": ("uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;",
                                 "uint32_t bits = (uint32_t)((const uint16_t*)base)[idx];"),
    "normaliser dropped": ("const double wj = s[j] / denom;", "const double wj = s[j];"),
    "fp8 exponent bias off by one": ("ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    "fp8 subnormals scaled as normals": ("ldexp(m / 8.0, -6)", "ldexp(m / 8.0, -7)"),
    "fp8 rounds half away from zero": ("const double v = rint(a / q) * q;",
                                       "const double v = floor(a / q + 0.5) * q;"),
    "fp8 no saturation": ("if (a >= 448.0) return sign | 0x7E;", "if (a >= 448.0) return sign | 0x7F;"),
    "fp8 write multiplies by the scale": ("(float)orc_load(key, src_k, dtype) / k_scale;",
                                          "(float)orc_load(key, src_k, dtype) * k_scale;"),
    "fp8 read ignores the value scale": ("phys, g, off, c, num_kv_heads, block_size, head_dim)]) * v_scale;",
                                         "phys, g, off, c, num_kv_heads, block_size, head_dim)]);"),
    "token index uses position as the row": ("token_indices[i] = (int64_t)p + (int64_t)r * row_width;",
                                             "token_indices[i] = (int64_t)r + (int64_t)p * row_width;"),
    "discard mask keeps finished requests": ("discard[r] = seq_lens[r] < num_tokens_total[r] ? 1 : 0;",
                                            "discard[r] = seq_lens[r] <= num_tokens_total[r] ? 1 : 0;"),
    "block copy reversed": ("memmove(key_cache + dst * block_bytes, key_cache + src * block_bytes, (size_t)block_bytes);",
                            "memmove(key_cache + src * block_bytes, key_cache + dst * block_bytes, (size_t)block_bytes);"),
    "zeroing skips the value pool": ("memset(value_cache + (int64_t)block_ids[k] * block_bytes, 0, (size_t)block_bytes);",
                                     "(void)0;"),
    "fp8 value layout collides": ("* 4 + (dim / 16) % 4) * 4 + tok % 4;", "* 4 + (dim / 32) % 4) * 4 + tok % 4;"),
    "fp8 value dim and token fields swapped": ("* 4 + (dim / 16) % 4) * 4 + tok % 4;",
                                               "* 4 + tok % 4) * 4 + (dim / 16) % 4;"),
    "fp8 key stored dim-major": (
        "return run + ((int64_t)(dim / 64) * block_size + tok) * 64 + dim % 64;",
        "return run + (int64_t)dim * block_size + tok;"),
    "fp8 key stored token-major": (
        "return run + ((int64_t)(dim / 64) * block_size + tok) * 64 + dim % 64;",
        "return run + (int64_t)tok * head_dim + dim;"),
    "key stored token-major": (
        "return run + ((int64_t)(dim / kw) * block_size + tok) * kw + dim % kw;",
        "return run + (int64_t)tok * head_dim + dim;"),
    "key slab transposed inside": (
        "return run + ((int64_t)(dim / kw) * block_size + tok) * kw + dim % kw;",
        "return run + ((int64_t)(dim / kw) * kw + dim % kw) * block_size + tok;"),
    "key slab width 16": ("const int32_t kw = head_dim % 32 == 0 ? 32 : head_dim;",
                          "const int32_t kw = head_dim % 16 == 0 ? 16 : head_dim;"),
}


def _run_mutant(name, find, repl, tmp):
    src = open(SRC).read()
    assert src.count(find) == 1, f"mutation site for {name!r} not unique/found"
    path_c = os.path.join(tmp, f"m{abs(hash(name))}.c")
    path_so = path_c[:-2] + ".so"
    with open(path_c, "w") as f:
        f.write(src.replace(find, repl))
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", path_c, "-o",
                    path_so, "-lm"], check=True, capture_output=True)
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=path_so, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return name, r.returncode


def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(max_workers=4) as ex:
            futs = [ex.submit(_run_mutant, n, f, r, tmp) for n, (f, r) in MUTANTS.items()]
            results = dict(f.result() for f in futs)
    survivors = [n for n, rc in results.items() if rc == 0]
    assert not survivors, f"mutants not caught by any pin: {survivors}"
