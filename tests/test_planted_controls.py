"""Planted controls on the CPU oracle: copies of moe_oracle.c with one plausible misreading
planted in each must turn a named pin red.

Each control rewrites one passage of the oracle source (the passage must occur exactly once,
so a control cannot silently stop applying when the oracle changes), builds the copy with
the oracle's own flags, and runs the pin meant to catch it in a child process that loads the
copy through MOE_ORACLE_LIB. The child must report failed tests (exit status 1): a control
whose pin stays green marks a part of the oracle that nothing outside it fixes. Nothing here
touches a GPU.
"""
import concurrent.futures
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")
PINS = "tests/test_oracle_pins.py"

# (name, [(passage, replacement), ...], pin selected with -k)
CONTROLS = [
    ("shared_up_and_down_swapped",
     [("oracle_dense(W->sh_up, in, SI, H, tmp);", "oracle_dense(W->sh_dn, in, SI, H, tmp);"),
      ("oracle_dense(W->sh_dn, in, H, SI, tmp);", "oracle_dense(W->sh_up, in, H, SI, tmp);")],
     "test_shared_expert_is_textbook_relu2_mlp"),
    ("shared_relu2_dropped",
     [("oracle_dense(W->sh_up, in, SI, H, tmp);\n        for (int i = 0; i < n; ++i) out[i] = relu_sq(cfg, rnd(cfg, tmp[i]));",
       "oracle_dense(W->sh_up, in, SI, H, tmp);\n        for (int i = 0; i < n; ++i) out[i] = rnd(cfg, tmp[i]);")],
     "test_shared_expert_is_textbook_relu2_mlp"),
    ("shared_fed_the_latent",
     [("oracle_stage(cfg, W, ORC_ST_SHARED_ACT, 0, x, NULL, NULL, gsh, NULL);",
       "oracle_stage(cfg, W, ORC_ST_SHARED_ACT, 0, u, NULL, NULL, gsh, NULL);")],
     "test_shared_expert_is_textbook_relu2_mlp"),
    ("experts_fed_the_input_not_the_latent",
     [("oracle_stage(cfg, W, ORC_ST_EXPERT_ACT, idx[j], u, NULL, NULL, a + (size_t)j * I, NULL);",
       "oracle_stage(cfg, W, ORC_ST_EXPERT_ACT, idx[j], x, NULL, NULL, a + (size_t)j * I, NULL);")],
     "test_latent_projections_and_expert_input_are_textbook"),
    ("fc2_reads_fc1_weights",
     [("oracle_dense(W->fc2_w, in, H, L, tmp);", "oracle_dense(W->fc1_w, in, H, L, tmp);")],
     "test_latent_projections_and_expert_input_are_textbook"),
    ("routed_relu2_dropped",
     [("W->up_b + (size_t)e * I * (D / gs), in, I, D, gs, nb, tmp);\n        for (int i = 0; i < n; ++i) out[i] = relu_sq(cfg, rnd(cfg, tmp[i]));",
       "W->up_b + (size_t)e * I * (D / gs), in, I, D, gs, nb, tmp);\n        for (int i = 0; i < n; ++i) out[i] = rnd(cfg, tmp[i]);")],
     "test_single_expert_identity_latent_is_textbook_mlp"),
    ("residual_added_before_the_shared_output",
     [("tmp[i] = in[i] + rnd(cfg, in2[i] + (in3 ? in3[i] : 0.0f));",
       "tmp[i] = rnd(cfg, in[i] + in2[i]) + (in3 ? in3[i] : 0.0f);")],
     "test_final_add_order_constructed_cases"),
    ("weights_from_biased_scores",
     [("float v = cfg->norm_topk ? s[idx[j]] / S : s[idx[j]];",
       "float v = cfg->norm_topk ? b[idx[j]] / S : b[idx[j]];"),
      ("float S = s[idx[0]];", "float S = b[idx[0]];"),
      ("for (int j = 1; j < K; ++j) S = S + s[idx[j]];", "for (int j = 1; j < K; ++j) S = S + b[idx[j]];")],
     "test_zero_input"),
    ("routed_scaling_dropped",
     [("w[j] = v * cfg->routed_scaling;", "w[j] = v;")],
     "test_route_weights_sum_to_scale"),
    ("ties_to_the_higher_id",
     [("    return ia < ib;\n}", "    return ia > ib;\n}")],
     "test_route_matches_brute_force"),
    ("group_score_is_the_best_member_only",
     [("gam[g] = (i2 >= 0) ? b[i1] + b[i2] : b[i1];", "gam[g] = b[i1];")],
     "test_route_matches_brute_force"),
    ("nan_ranks_highest",
     [("if (na != nb) return nb;", "if (na != nb) return na;")],
     "test_route_nan_ranks_lowest"),
    ("sigmoid_in_single_precision",
     [("return (float)(1.0 / (1.0 + exp(-(double)z)));", "return 1.0f / (1.0f + expf(-z));")],
     "test_sigmoid_every_bf16_against_library"),
    ("gate_lanes_strided",
     [("int k = 512 * j + 8 * t + i;", "int k = 512 * j + t + 64 * i;")],
     "test_gate_c64_constructed_cases"),
    ("combine_lanes_joined_in_sequence",
     [("out[d] = ((T[0] + T[4]) + (T[2] + T[6])) + ((T[1] + T[5]) + (T[3] + T[7]));",
       "out[d] = ((((((T[0] + T[1]) + T[2]) + T[3]) + T[4]) + T[5]) + T[6]) + T[7];")],
     "test_combine_constructed_cases"),
    ("dequant_offset_by_one_code",
     [("return (float)q * sc + bi;", "return (float)(q + 1u) * sc + bi;")],
     "test_dequant_closed_form_every_code_and_scale"),
    ("code_bits_high_first",
     [("q |= ((qrow[j / 32] >> (j % 32)) & 1u) << i;", "q |= ((qrow[j / 32] >> (j % 32)) & 1u) << (bits - 1 - i);")],
     "test_nibble_layout_low_nibble_first"),
    ("codes_on_a_four_bit_stride",
     [("long j = (long)k * bits + i;", "long j = (long)k * 4 + i;")],
     "test_code_layout_every_width"),
]


def _build(name, edits, tmpdir):
    with open(SRC) as f:
        text = f.read()
    for old, new in edits:
        assert text.count(old) == 1, (name, old)
        text = text.replace(old, new)
    src = os.path.join(tmpdir, f"{name}.c")
    lib = os.path.join(tmpdir, f"lib{name}.so")
    with open(src, "w") as f:
        f.write(text)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fno-unsafe-math-optimizations",
                    "-shared", "-fPIC", src, "-o", lib, "-lm"], check=True)
    return lib


def _run_pin(pin, lib):
    env = dict(os.environ, MOE_ORACLE_LIB=lib or "", OMP_NUM_THREADS="1")
    if not lib:
        env.pop("MOE_ORACLE_LIB")
    p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        PINS, "-k", pin], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return p.returncode, p.stdout[-2000:]


def test_every_planted_control_turns_its_pin_red(tmp_path):
    libs = {name: _build(name, edits, str(tmp_path)) for name, edits, _ in CONTROLS}
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        futs = {name: ex.submit(_run_pin, pin, libs[name]) for name, _, pin in CONTROLS}
        # the same pins against the oracle as it stands: all green
        clean = {pin: ex.submit(_run_pin, pin, None) for pin in sorted({c[2] for c in CONTROLS})}
        res = {k: f.result() for k, f in futs.items()}
        base = {k: f.result() for k, f in clean.items()}
    for pin, (rc, out) in base.items():
        assert rc == 0, (pin, out)
    missed = {name: out for name, (rc, out) in res.items() if rc != 1}
    assert not missed, missed
