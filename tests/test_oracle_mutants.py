"""Plant plausible mistakes in a copy of the oracle source and check that the
pins catch every one of them (mutation testing, CPU only).  The committed
oracle itself is never modified."""
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "strata_oracle.c")

# (label, exact text in strata_oracle.c, replacement)
MUTANTS = [
    ("code offset dropped", "(double)(orc_q2_code(block, i) - 1) * d", "(double)(orc_q2_code(block, i)) * d"),
    ("code bit order reversed", ">> (2 * (i % 4))) & 3", ">> (2 * (3 - i % 4))) & 3"),
    ("scale bytes swapped", "block[0] | ((uint16_t)block[1] << 8)", "block[1] | ((uint16_t)block[0] << 8)"),
    ("codes read from byte 1", "block[2 + i / 4]", "block[1 + i / 4]"),
    ("half exponent off by one", "ex - 25); /* 1.man", "ex - 24); /* 1.man"),
    ("bf16 mantissa width", "(128 + man), ex - 134", "(256 + man), ex - 135"),
    ("gate and up swapped in SwiGLU", "h[j] = orc_silu(g) * u;", "h[j] = orc_silu(u) * g;"),
    ("up read from the down matrix", "*up = blob + mat_bytes;", "*up = blob + 2 * mat_bytes;"),
    ("down rows indexed by input width", "o[r] = q2_row_dot(down, r, FF, h);",
     "o[r] = q2_row_dot(down, r % FF, FF, h);"),
    ("unstable tie order", "(float)p[order[j - 1]] < key", "(float)p[order[j - 1]] <= key"),
    ("ascending sort", "(float)p[order[j - 1]] < key", "(float)p[order[j - 1]] > key"),
    ("renormalisation dropped", "w[k] = p[ids[k]] / den;", "w[k] = p[ids[k]];"),
    ("softmax sign flipped", "p[e] = exp(logits[e] - m);", "p[e] = exp(m - logits[e]);"),
    ("router bias subtracted", "acc += (double)bias[e];", "acc -= (double)bias[e];"),
    ("rmsnorm mean dropped", "1.0 / sqrt(ss / n + eps)", "1.0 / sqrt(ss + eps)"),
    ("combine ignores weights", "acc += w[(size_t)t * K + k] *", "acc += 0.1 *"),
    ("expert input from the wrong token", "xhat + (size_t)(s / K) * H", "xhat + (size_t)(s % K % T) * H"),
    ("silu sign", "return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
]

CHECKS = [
    pins.test_blob_and_store_sizes,
    pins.test_half_decoder_all_patterns,
    pins.test_bf16_decoder_all_patterns,
    pins.test_code_bit_order_matches_quoted_unpack,
    pins.test_hand_built_blocks,
    pins.test_router_one_hot_gives_a_column,
    pins.test_softmax_topk_invariants,
    pins.test_stable_ties,
    pins.test_rmsnorm_closed_forms,
    pins.test_expert_closed_form,
    pins.test_one_hot_gate_up_columns,
    lambda o: pins.test_bruteforce_tiny_instance(o, 2),
    pins.test_bruteforce_tiny_with_ties_bias_and_norm,
    pins.test_identical_experts_give_one_output,
    pins.test_combine_is_weighted_sum_in_routing_order,
    pins.test_bruteforce_tall_down_matrix,
]


@pytest.mark.parametrize("label,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, label, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique for {label!r}"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC",
                    "-shared", "-I", os.path.dirname(SRC), "-o", str(so), str(mpath), "-lm"],
                   check=True)
    caught = []
    with oracle.using(str(so)):
        for chk in CHECKS:
            try:
                chk(oracle)
            except (AssertionError, RuntimeError, ValueError, FloatingPointError):
                caught.append(getattr(chk, "__name__", "check"))
    assert caught, f"no pin caught the planted mistake: {label}"
