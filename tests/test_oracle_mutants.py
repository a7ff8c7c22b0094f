"""Each plausible mistake planted in a copy of the oracle fails at least one pin.

The mistake is planted in a temporary copy of oracle/decode_ref.c on the CPU;
the copy is built with gcc and the pins of oracle_pins.py run against it.  This
shows the pins have teeth: a dropped term, a wrong sign or index or a
transposed layout in the oracle would not go unnoticed.
"""
import json
import os
import subprocess
import sys

import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "decode_ref.c")

# (name, text in decode_ref.c, replacement)
MUTANTS = [
    ("drop_scale", "x[j] = scale * dot + slope", "x[j] = dot + slope"),
    ("head_map_modulo", "int g = h / group;", "int g = h % num_kv_heads;"),
    ("max_shift_sign", "double w = exp(x[j] - M);", "double w = exp(M - x[j]);"),
    ("lse_drops_max", "*lse = M + log(l);", "*lse = log(l);"),
    ("no_normalise", "o[d] /= l;", "o[d] /= 1.0;"),
    ("kv_len_ignores_last_page_len",
     "(n - 1) * page_size + last_page_len[b]", "n * page_size"),
    ("token_major_layout",
     "((page * num_kv_heads + g) * page_size + r) * head_dim",
     "((page * page_size + r) * num_kv_heads + g) * head_dim"),
    ("page_order_reversed", "indices[indptr[b] + j / page_size]",
     "indices[indptr[b + 1] - 1 - j / page_size]"),
    ("f16_exponent_bias", "e - 25", "e - 24"),
    ("f16_subnormal_scale", "ldexp((double)m, -24)", "ldexp((double)m, -25)"),
    ("bf16_shift", "(uint32_t)b << 16", "(uint32_t)b << 15"),
    ("merge_weight_unshifted", "double w = exp(lse_parts[s] - out_lse);",
     "double w = exp(lse_parts[s] - M);"),
    ("merge_lse_no_log", "double out_lse = M + log(sum);", "double out_lse = M + sum - 1.0;"),
    ("empty_seq_lse_zero", "*lse = -INFINITY;\n    return;\n  }\n  /* scores */",
     "*lse = 0.0;\n    return;\n  }\n  /* scores */"),
    ("contig_row_stride", "contig_row_offset(layout, num_kv_heads, max_kv_len, head_dim, g, j)",
     "contig_row_offset(layout, num_kv_heads, valid_kv_len, head_dim, g, j)"),
    ("nhd_paged_as_heads_major",
     "if (layout == OR_NHD) return ((page * page_size + r) * num_kv_heads + g) * head_dim;",
     "if (layout == OR_NHD) return ((page * num_kv_heads + g) * page_size + r) * head_dim;"),
    ("nhd_paged_drops_head",
     "if (layout == OR_NHD) return ((page * page_size + r) * num_kv_heads + g) * head_dim;",
     "if (layout == OR_NHD) return ((page * page_size + r) * num_kv_heads) * head_dim;"),
    ("nhd_contig_as_heads_major",
     "if (layout == OR_NHD) return (j * num_kv_heads + g) * head_dim;",
     "if (layout == OR_NHD) return ((int64_t)g * max_kv_len + j) * head_dim;"),
    ("append_past_last_row",
     "indptr,\n                                     b, g, L - 1);",
     "indptr,\n                                     b, g, L);"),
    ("append_to_empty_request", "    if (L == 0) continue;\n    for (int g = 0; g < num_kv_heads",
     "    if (L == 0) L = 1;\n    for (int g = 0; g < num_kv_heads"),
    ("window_one_row_short", "(window > 0 && L > window) ? L - window : 0",
     "(window > 0 && L > window) ? L - window + 1 : 0"),
    ("softcap_scale_outside",
     "if (softcap > 0.0) x[j] = softcap * tanh(x[j] / softcap);",
     "if (softcap > 0.0) x[j] = scale * softcap * tanh(dot / softcap);"),
    ("softcap_drops_outer_factor",
     "if (softcap > 0.0) x[j] = softcap * tanh(x[j] / softcap);",
     "if (softcap > 0.0) x[j] = tanh(x[j] / softcap);"),
    ("alibi_sign", "x[j] = scale * dot + slope * (double)dist[j];",
     "x[j] = scale * dot - slope * (double)dist[j];"),
    ("alibi_absolute_position", "dist[kept++] = j - (L - 1);", "dist[kept++] = j;"),
    ("alibi_after_cap",
     "x[j] = scale * dot + slope * (double)dist[j];\n    if (softcap > 0.0) x[j] = softcap * tanh(x[j] / softcap);",
     "x[j] = scale * dot;\n    if (softcap > 0.0) x[j] = softcap * tanh(x[j] / softcap);\n    x[j] += slope * (double)dist[j];"),
    ("mask_ignored", "return mask == NULL || ((mask[bit >> 3] >> (bit & 7)) & 1);", "return 1;"),
    ("mask_inverted", "return mask == NULL || ((mask[bit >> 3] >> (bit & 7)) & 1);",
     "return mask == NULL || !((mask[bit >> 3] >> (bit & 7)) & 1);"),
    ("mask_bit_order_msb_first", "((mask[bit >> 3] >> (bit & 7)) & 1)",
     "((mask[bit >> 3] >> (7 - (bit & 7))) & 1)"),
    ("mask_ignores_request_offset", "mask_keeps(mask, rows_before[b] + j)", "mask_keeps(mask, j)"),
    ("mask_renumbers_positions", "dist[kept++] = j - (L - 1);",
     "dist[kept] = kept - (L - 1);\n        kept++;"),
    ("validate_skips_upper_bound", "indices[i] >= num_total_pages", "indices[i] > num_total_pages"),
    # the attention over explicit rows (a split's partial)
    ("attend_drops_scale", "    x[j] = scale * dot;\n", "    x[j] = dot;\n"),
    ("attend_k_transposed", "dot += q[d] * k[j * head_dim + d];", "dot += q[d] * k[d * L + j];"),
    ("attend_v_first_row", "o[d] += w * v[j * head_dim + d];", "o[d] += w * v[d];"),
]


def _build_variant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert old in src, f"mutation anchor not found: {name}"
    mutated = src.replace(old, new)
    path = tmp_path / f"{name}.c"
    path.write_text(mutated)
    lib = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", str(lib),
                    str(path), "-lm"], check=True)
    return str(lib)


_RUNNER = """
import json, sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, oracle_pins
oracle.use_library({lib!r})
caught = []
for pin in oracle_pins.ALL_PINS:
    try:
        pin()
    except Exception as e:
        caught.append(pin.__name__)
print(json.dumps(caught))
"""


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    lib = _build_variant(tmp_path, name, old, new)
    tests = os.path.dirname(os.path.abspath(__file__))
    code = _RUNNER.format(root=os.path.dirname(tests), tests=tests, lib=lib)
    # a separate process, so that a mutant that reads out of bounds cannot take
    # the test session down with it
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       timeout=600, env=dict(os.environ, OMP_NUM_THREADS="4"))
    assert r.returncode == 0, f"mutant {name} crashed the pin run: {r.stderr[-2000:]}"
    caught = json.loads(r.stdout.strip().splitlines()[-1])
    assert caught, f"no pin caught the planted mistake {name}"
