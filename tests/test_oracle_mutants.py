"""The pins must catch plausible mistakes in the oracle.

Each case below plants one mistake in a temporary copy of the C oracle (the
committed source is never touched), builds it, and runs the pin suite
against it with PKV_ORACLE_LIB pointing at the mutant.  The suite must fail
for every mutant: a mistake that no pin notices would mean the oracle is
only checked against itself.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "pagedkv_oracle.c")

MUTANTS = {
    "slot_ignores_offset": (
        "int64_t p = (int64_t)offsets[seq] + (int64_t)token_pos[i];",
        "int64_t p = (int64_t)token_pos[i];"),
    "slot_wrong_block_scale": (
        "slot_mapping[i] = phys * block_size + in_block;",
        "slot_mapping[i] = phys * (block_size - 1) + in_block;"),
    "scatter_swaps_block_and_slot": (
        "int64_t b = slot / block_size;\n        int64_t s = slot % block_size;",
        "int64_t s = slot / block_size;\n        int64_t b = slot % block_size;\n"
        "        if (s >= block_size || b >= num_blocks) return -1;"),
    "row_ignores_layer": (
        "return (b * num_layers + layer) * block_size + s;",
        "return (b * num_layers) * block_size + s;"),
    "gather_ignores_offset": (
        "int64_t start = offsets[s];",
        "int64_t start = 0 * offsets[s];"),
    "gather_keeps_offset_on_later_blocks": (
        "            start = 0;\n        }",
        "        }"),
    "gather_full_first_block": (
        "int64_t take = block_size - start;",
        "int64_t take = block_size;"),
    "bf16_wrong_shift": (
        "uint32_t bits = ((uint32_t)h) << 16;",
        "uint32_t bits = ((uint32_t)h) << 15;"),
    "gqa_interleaved_heads": (
        "        for (int64_t h = g * G; h < (g + 1) * G; h++) {\n            const uint8_t *qh",
        "        for (int64_t h = g; h < J->num_q_heads; h += J->num_kv_heads) {\n"
        "            const uint8_t *qh"),
    "decode_drops_scale": (
        "score[t] = J->scale * dot;",
        "score[t] = dot;"),
    "decode_wrong_normaliser": (
        "den += w;",
        "den += 1.0;"),
    "decode_reads_k_for_v": (
        "const uint8_t *vt = vrows + t * row_bytes + g * D * e;",
        "const uint8_t *vt = krows + t * row_bytes + g * D * e;"),
    "decode_off_by_one_token": (
        "for (int64_t t = 0; t <= P; t++) {\n                double w",
        "for (int64_t t = 0; t < P; t++) {\n                double w"),
    "prefill_ignores_prefix": (
        "const int64_t P = L - n + i;",
        "const int64_t P = i;"),
    "prefill_without_causal_mask": (
        "const int64_t P = L - n + i;",
        "const int64_t P = L - 1;"),
}


def _run_mutant(name, tmp):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"{name}: anchor not found exactly once"
    path_c = os.path.join(tmp, f"{name}.c")
    path_so = os.path.join(tmp, f"{name}.so")
    with open(path_c, "w") as f:
        f.write(src.replace(old, new))
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    path_c, "-o", path_so, "-lm", "-lpthread"], check=True,
                   capture_output=True)
    env = dict(os.environ, PKV_ORACLE_LIB=path_so, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode, r.stdout[-400:]


def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda n: _run_mutant(n, tmp), MUTANTS))
    survivors = [(n, out) for n, rc, out in results if rc == 0]
    assert not survivors, f"mutants not caught by any pin: {survivors}"
    # rc 1 = tests failed (what we want); anything else is a harness problem
    bad = [(n, rc, out) for n, rc, out in results if rc not in (1,)]
    assert not bad, bad


def test_unmutated_copy_passes():
    """Control: the same harness with the source unchanged passes."""
    with tempfile.TemporaryDirectory() as tmp:
        MUTANTS["_control"] = ("#define ORC_F32 0", "#define ORC_F32 0")
        try:
            name, rc, out = _run_mutant("_control", tmp)
        finally:
            del MUTANTS["_control"]
    assert rc == 0, out
