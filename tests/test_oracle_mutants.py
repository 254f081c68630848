"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies moe_q4_oracle.c, applies one plausible mistake (a dropped
term, a wrong index, a transposed operand, another rounding or summation
order), builds it with the oracle's own flags and runs the oracle pin tests
against that build.  The pins pass on the real oracle (the other test files)
and must fail on every mutant.  Nothing here touches the GPU path.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PINS = ["test_oracle_formats.py", "test_oracle_routing.py", "test_oracle_layer.py",
        "test_oracle_prefill_bf16.py"]

# (name, exact text in moe_q4_oracle.c, replacement)
MUTANTS = [
    ("nibble_interleaved", "blk[2 + j] = (uint8_t)(q[j] | (q[j + 16] << 4));",
     "blk[2 + j] = (uint8_t)(q[2 * j] | (q[2 * j + 1] << 4));"),
    ("q4_scale_over_8", "float d32 = amax / 7.0f;", "float d32 = amax / 8.0f;"),
    ("q4_round_even", "float t = roundf(v[j] / df);", "float t = rintf(v[j] / df);"),
    ("q4_no_clamp_low", "if (t < -8.0f) t = -8.0f;", ";"),
    ("q4_offset_7", "(float)(q4_code(blk, j) - 8) * d;", "(float)(q4_code(blk, j) - 7) * d;"),
    ("q8_round_even", "(dd == 0.0f) ? (int8_t)0 : (int8_t)roundf(v[j] / dd);",
     "(dd == 0.0f) ? (int8_t)0 : (int8_t)rintf(v[j] / dd);"),
    ("q8_scale_128", "float dd = amax / 127.0f;", "float dd = amax / 128.0f;"),
    ("f16_round_up_ties", "if (rem > 0x1000u || (rem == 0x1000u && (v & 1u)))",
     "if (rem >= 0x1000u)"),
    ("router_transposed", "acc = fmaf(xt[h], Wr[h * E + e], acc);",
     "acc = fmaf(xt[h], Wr[e * H + h], acc);"),
    ("router_unfused", "acc = fmaf(xt[h], Wr[h * E + e], acc);",
     "acc = acc + xt[h] * Wr[h * E + e];"),
    ("router_bias_dropped", "if (bias) l = l + bias[e];", ";"),
    ("tree_left_to_right", "for (size_t i = 0; i < m / 2; i++) buf[i] = buf[2 * i] + buf[2 * i + 1];",
     "for (size_t i = 1; i < m; i++) buf[0] = buf[0] + buf[i]; m = 1;"),
    ("topk_ties_higher_index", "if (best < 0 || l[e] > l[best]) best = e;",
     "if (best < 0 || l[e] >= l[best]) best = e;"),
    ("exp_no_lo_term", "r = fmaf(-n, EXPP_LN2_LO, r);", ";"),
    ("silu_wrong_sign", "return g / (1.0f + orc_exp_p(-g));", "return g / (1.0f + orc_exp_p(g));"),
    ("perm_unstable", "for (int64_t f = 0; f < n; f++) {\n        int32_t e = ids[f];",
     "for (int64_t f = n - 1; f >= 0; f--) {\n        int32_t e = ids[f];"),
    ("w4a8_offset_7", "dot += (int32_t)(q4_code(blk, j) - 8) * (int32_t)qa[b * ORC_BLK + j];",
     "dot += (int32_t)(q4_code(blk, j) - 7) * (int32_t)qa[b * ORC_BLK + j];"),
    ("w4a8_act_scale_dropped", "float s = q4_scale(blk) * da[b];", "float s = q4_scale(blk);"),
    ("ffn_no_activation", "hbuf[i] = gi / (1.0 + exp(-gi)) * ui;", "hbuf[i] = gi * ui;"),
    ("prefill_weight_dropped", "for (int64_t h = 0; h < H; h++) yt[h] += w64[t * L->k + s] * o[h];",
     "for (int64_t h = 0; h < H; h++) yt[h] += o[h];"),
    ("decode_shared_dropped", "if (S) acc = acc + o[k * H + r];", ";"),
    ("decode_up_for_gate", "g[i] = layer_row(L, G + i * layer_row_bytes(L, H), H, qx, dx, buf);",
     "g[i] = layer_row(L, U + i * layer_row_bytes(L, H), H, qx, dx, buf);"),
    ("q8w_scale_128", "float d32 = amax / 127.0f;", "float d32 = amax / 128.0f;"),
    ("q8w_round_even", "float t = (df == 0.0f) ? 0.0f : roundf(v[j] / df);",
     "float t = (df == 0.0f) ? 0.0f : rintf(v[j] / df);"),
    ("q8w_no_clamp_high", "if (t > 127.0f) t = 127.0f;", ";"),
    ("w8a8_offset_8", "dot += (int32_t)q8w_code(blk, j) * (int32_t)qa[b * ORC_BLK + j];",
     "dot += (int32_t)(q8w_code(blk, j) - 8) * (int32_t)qa[b * ORC_BLK + j];"),
    ("w8a8_act_scale_dropped", "float s = q8w_scale(blk) * da[b];", "float s = q8w_scale(blk);"),
    ("decode_q8_read_as_q4", "return L->wfmt ? w8a8_row(row, K, qa, da, NULL, buf) : w4a8_row(row, K, qa, da, NULL, buf);",
     "return w4a8_row(row, K, qa, da, NULL, buf);"),
    ("rmsnorm_mean_h_minus_1", "float r = sqrtf(ss / (float)H + eps);",
     "float r = sqrtf(ss / (float)(H - 1) + eps);"),
    ("bf16_ties_away", "if (rem > 0x8000u || (rem == 0x8000u && (base & 0x00010000u)))",
     "if (rem >= 0x8000u)"),
    ("prefill_bf16_w_unrounded", "float w = orc_bf16_round((float)(q4_code(blk, j) - 8) * d);",
     "float w = (float)(q4_code(blk, j) - 8) * d;"),
    ("prefill_bf16_h_unrounded", "hbuf[i] = (double)orc_bf16_round((float)(gi / (1.0 + exp(-gi)) * ui));",
     "hbuf[i] = gi / (1.0 + exp(-gi)) * ui;"),
    ("prefill_bf16_o_unrounded", "o[r] = round_o ? orc_bf16_round(v) : v;", "o[r] = v;"),
    ("prefill_bf16_shared_rounded", "expert_ffn_bf16(L->s_gate, L->s_up, L->s_down, H, I, xd, hb, o, 0);",
     "expert_ffn_bf16(L->s_gate, L->s_up, L->s_down, H, I, xd, hb, o, 1);"),
    ("prefill_bf16_combine_in_double", "float p = ws * o[h];\n                yt[h] = yt[h] + p;",
     "yt[h] = (float)((double)yt[h] + (double)ws * (double)o[h]);"),
]


def _run_mutant(tmpdir, name, old, new):
    src = open(os.path.join(ROOT, "oracle", "moe_q4_oracle.c")).read()
    assert src.count(old) >= 1, "mutation anchor not found: " + name
    msrc = os.path.join(tmpdir, name + ".c")
    with open(msrc, "w") as f:
        f.write(src.replace(old, new, 1))
    lib = os.path.join(tmpdir, "lib_" + name + ".so")
    oracle.build(out=lib, src=msrc)
    env = dict(os.environ, MOE_Q4_ORACLE_LIB=lib)
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
           *[os.path.join(HERE, p) for p in PINS]]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode, r.stdout[-400:]


def test_every_planted_mistake_is_caught(tmp_path):
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda m: _run_mutant(str(tmp_path), *m), MUTANTS))
    survived = [(n, out) for n, rc, out in results if rc == 0]
    assert not survived, survived
    # pytest exit code 1 = tests failed (not a crash or a collection error)
    assert all(rc == 1 for _, rc, _ in results), [(n, rc) for n, rc, _ in results]
