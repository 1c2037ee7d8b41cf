"""Mutation pins of the C oracle (CPU only).

Each entry of MUTANTS plants one plausible mistake in a copy of
oracle/a2av_oracle.c: a dropped term, an index transposed, an off-by-one
bound, a wrong stride, a missing check, a rounding or overflow rule bent.
The pins of tests/test_oracle_pins.py and tests/test_signal_model.py are
then run against the mutated library, in a process of its own (a mutant may
write out of bounds); at least one pin must fail.  A mutant no pin notices is
a hole in the pins.

    python -m tests.oracle_mutants <liba2av_oracle.so built from a copy>

runs every pin against that library and exits 0 when all pass (the mutant
survived) or 1 naming the first pin that failed.
"""
from __future__ import annotations

import inspect
import itertools
import os
import subprocess
import sys
import traceback

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "a2av_oracle.c")

# (name, text in a2av_oracle.c, replacement); each text occurs exactly once.
MUTANTS = [
    # CalAllToAllVBlocks
    ("fold_search_starts_below_L",
     "for (int64_t m = L; m >= P; --m)", "for (int64_t m = L - 1; m >= P; --m)"),
    ("fold_L_below_P_gives_P",
     "if (L < P)\n        return L;", "if (L < P)\n        return P;"),
    # recv_counts
    ("recv_counts_not_transposed",
     "recv_counts[d * P + s] = send_counts[s * P + d];",
     "recv_counts[s * P + d] = send_counts[s * P + d];"),
    # displacements
    ("send_displacement_inclusive",
     "sdispl[s * P + d] = off;\n            off += (int64_t)C[s * P + d] * e;",
     "off += (int64_t)C[s * P + d] * e;\n            sdispl[s * P + d] = off;"),
    ("send_displacement_without_type_size",
     "sdispl[s * P + d] = off;\n            off += (int64_t)C[s * P + d] * e;",
     "sdispl[s * P + d] = off;\n            off += (int64_t)C[s * P + d];"),
    ("receive_displacement_reads_the_transpose",
     "rdispl[d * P + s] = off;\n            off += (int64_t)C[s * P + d] * e;",
     "rdispl[d * P + s] = off;\n            off += (int64_t)C[d * P + s] * e;"),
    # the payload move
    ("target_slab_stride_is_the_input_slab",
     "memcpy(target + (int64_t)d * tgt_slab + rdispl[d * P + s],",
     "memcpy(target + (int64_t)d * in_slab + rdispl[d * P + s],"),
    ("receive_displacement_index_transposed",
     "memcpy(target + (int64_t)d * tgt_slab + rdispl[d * P + s],",
     "memcpy(target + (int64_t)d * tgt_slab + rdispl[s * P + d],"),
    ("source_read_at_the_receive_displacement",
     "input + (int64_t)s * in_slab + sdispl[s * P + d], (size_t)nbytes);",
     "input + (int64_t)s * in_slab + rdispl[d * P + s], (size_t)nbytes);"),
    ("last_destination_skipped",
     "for (int32_t d = 0; d < P; ++d) {\n            int64_t nbytes",
     "for (int32_t d = 0; d < P - 1; ++d) {\n            int64_t nbytes"),
    # the signal
    ("signal_last_block_skipped",
     "for (int64_t b = 0; b < B; ++b) {\n            uint32_t v",
     "for (int64_t b = 0; b < B - 1; ++b) {\n            uint32_t v"),
    ("signal_adds_two",
     "signal[(int64_t)r * S + b] = (int32_t)(v + 1u);",
     "signal[(int64_t)r * S + b] = (int32_t)(v + 2u);"),
    ("signal_saturates",
     "signal[(int64_t)r * S + b] = (int32_t)(v + 1u);",
     "signal[(int64_t)r * S + b] = v == 0x7FFFFFFFu ? (int32_t)v : (int32_t)(v + 1u);"),
    ("signal_row_stride_is_B",
     "uint32_t v = (uint32_t)signal[(int64_t)r * S + b];\n"
     "            signal[(int64_t)r * S + b] = (int32_t)(v + 1u);",
     "uint32_t v = (uint32_t)signal[(int64_t)r * B + b];\n"
     "            signal[(int64_t)r * B + b] = (int32_t)(v + 1u);"),
    ("signal_every_column",
     "for (int64_t b = 0; b < B; ++b) {\n            uint32_t v",
     "for (int64_t b = 0; b < S; ++b) {\n            uint32_t v"),
    # the checks
    ("negative_count_accepted",
     "if (send_counts[s * P + d] < 0)\n                return OR_ERR_INVALID_ARGS;",
     "if (send_counts[s * P + d] < -1)\n                return OR_ERR_INVALID_ARGS;"),
    ("exact_row_capacity_refused",
     "if (row * e > in_slab)", "if (row * e >= in_slab)"),
    ("column_capacity_unchecked",
     "if (col * e > tgt_slab)\n            return OR_ERR_OVER_CAPACITY;\n    }\n\n"
     "    int32_t first = signal[0];",
     "if (0 && col * e > tgt_slab)\n            return OR_ERR_OVER_CAPACITY;\n    }\n\n"
     "    int32_t first = signal[0];"),
    ("signal_check_row_0_only",
     "for (int32_t r = 0; r < P; ++r)\n        for (int64_t b = 0; b < B; ++b)\n"
     "            if (signal[(int64_t)r * S + b] != first)\n"
     "                return OR_ERR_INVALID_ARGS;\n    return OR_OK;\n}\n\n/* Argument checks",
     "for (int32_t r = 0; r < 1; ++r)\n        for (int64_t b = 0; b < B; ++b)\n"
     "            if (signal[(int64_t)r * S + b] != first)\n"
     "                return OR_ERR_INVALID_ARGS;\n    return OR_OK;\n}\n\n/* Argument checks"),
    ("signal_stride_one_short_accepted",
     "if ((int64_t)S < B)\n        return OR_ERR_INVALID_ARGS;\n"
     "    if (B > 1 && capacity > 0 && B > capacity)\n        return OR_ERR_LAUNCH_CAPACITY;\n\n"
     "    int64_t bias_e",
     "if ((int64_t)S < B - 1)\n        return OR_ERR_INVALID_ARGS;\n"
     "    if (B > 1 && capacity > 0 && B > capacity)\n        return OR_ERR_LAUNCH_CAPACITY;\n\n"
     "    int64_t bias_e"),
    ("adjacent_operands_overlap",
     "return a < b + nb && b < a + na;", "return a <= b + nb && b <= a + na;"),
    ("unsupported_dtype_accepted",
     ": (dtype != OR_DTYPE_FP32 && dtype != OR_DTYPE_INT8))",
     ": (dtype != OR_DTYPE_FP32 && dtype != OR_DTYPE_INT8 && dtype != OR_DTYPE_FP16))"),
    ("launch_capacity_unchecked",
     "if (B > 1 && capacity > 0 && B > capacity)\n        return OR_ERR_LAUNCH_CAPACITY;\n\n"
     "    int64_t bias_e",
     "if (B > 1 && capacity > 0 && B > 2 * capacity)\n        return OR_ERR_LAUNCH_CAPACITY;\n\n"
     "    int64_t bias_e"),
    # the blocked exchange
    ("blocked_send_offset_not_scaled",
     "a * (row / nblk) +\n                           sdispl[s * P + d] / nblk,",
     "a * (row / nblk) +\n                           sdispl[s * P + d],"),
    ("blocked_sub_blocks_reversed",
     "rdispl[d * P + s] + a * sub,", "rdispl[d * P + s] + (nblk - 1 - a) * sub,"),
    ("blocked_indivisible_count_accepted",
     "if (send_counts[s * P + d] % unit != 0)", "if (send_counts[s * P + d] % unit > unit)"),
    # the 16-bit conversions and the bias Add
    ("bias_of_the_destination",
     "int64_t bi = ((int64_t)s * nblk + a) * hidden + h;",
     "int64_t bi = ((int64_t)d * nblk + a) * hidden + h;"),
    ("bias_column_from_the_sub_block_start",
     "int64_t h = k % hidden;", "int64_t h = k % (hidden + 1);"),
    ("ties_round_down",
     "if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) == 1.0))", "if (frac > 0.5)"),
    ("ties_round_up",
     "if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) == 1.0))", "if (frac >= 0.5)"),
    ("f16_overflow_one_binade_late",
     "if (biased >= 31)                                  /* overflow */",
     "if (biased > 31)                                  /* overflow */"),
    ("bf16_overflow_saturates",
     "if (biased >= 255)                                 /* overflow */\n"
     "        return (uint16_t)(sign | 0x7F80u);",
     "if (biased >= 255)                                 /* overflow */\n"
     "        return (uint16_t)(sign | 0x7F7Fu);"),
    ("f16_nan_becomes_infinity",
     "return (uint16_t)(sign | 0x7E00u | (uint16_t)(frac >> 13)); /* quiet NaN */",
     "return (uint16_t)(sign | 0x7C00u); /* quiet NaN */"),
    ("bf16_nan_without_the_quiet_bit",
     "return (uint16_t)(sign | 0x7FC0u | (uint16_t)(frac >> 16)); /* quiet NaN */",
     "return (uint16_t)(sign | 0x7F80u | (uint16_t)(frac >> 16)); /* quiet NaN */"),
    ("bf16_nan_loses_its_sign",
     "return (uint16_t)(sign | 0x7FC0u | (uint16_t)(frac >> 16)); /* quiet NaN */",
     "return (uint16_t)(0x7FC0u | (uint16_t)(frac >> 16)); /* quiet NaN */"),
    ("f16_subnormal_widening_scale",
     "mag = (float)man * (1.0f / 16777216.0f);", "mag = (float)man * (1.0f / 8388608.0f);"),
    ("f16_subnormal_narrowing_grid",
     "round_to_grid(a, (int)efield - 127, -14, 11, &binade);",
     "round_to_grid(a, (int)efield - 127, -15, 11, &binade);"),
    ("bf16_subnormal_result_as_normal",
     "if (m < 128)                                       /* subnormal (or zero) result */",
     "if (m < 0)                                       /* subnormal (or zero) result */"),
    ("bias_sum_rounded_through_the_wrong_format",
     "y[dst + k] = a2av_oracle_f32_to_f16(bits_from_f32(sum));",
     "y[dst + k] = (uint16_t)(a2av_oracle_f32_to_bf16(bits_from_f32(sum)));"),
    # the indexed exchange
    ("gather_list_restarts_per_destination",
     "memcpy(seg + j * row_bytes, table + (int64_t)list[k] * row_bytes,",
     "memcpy(seg + j * row_bytes, table + (int64_t)list[j] * row_bytes,"),
    ("gather_entry_one_past_the_table_accepted",
     "if (v < 0 || (int64_t)v >= table_rows)", "if (v < 0 || (int64_t)v > table_rows)"),
    ("gather_list_exactly_full_refused",
     "if (rows > index_stride)", "if (rows >= index_stride)"),
    ("gather_entries_past_the_rows_in_use_checked",
     "for (int64_t k = 0; k < rows; ++k) {\n            int32_t v",
     "for (int64_t k = 0; k < index_stride; ++k) {\n            int32_t v"),
]


def mutated_source(old: str, new: str) -> str:
    text = open(SRC).read()
    n = text.count(old)
    if n != 1:
        raise ValueError(f"mutation text found {n} times, expected once: {old!r}")
    return text.replace(old, new)


def build(name: str, out_dir: str) -> str:
    """Compile the named mutant into out_dir; returns the library's path."""
    old, new = next((o, n) for m, o, n in MUTANTS if m == name)
    src = os.path.join(out_dir, f"{name}.c")
    lib = os.path.join(out_dir, f"lib{name}.so")
    with open(src, "w") as f:
        f.write(mutated_source(old, new))
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-w", "-shared", "-fPIC", "-o", lib, src])
    return lib


def _cases(fn):
    """The parameter sets pytest would give fn (its parametrize marks)."""
    marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
    axes = []
    for m in marks:
        names = m.args[0]
        names = [x.strip() for x in names.split(",")] if isinstance(names, str) else list(names)
        values = [v if len(names) > 1 else (v,) for v in m.args[1]]
        axes.append([dict(zip(names, v)) for v in values])
    for combo in itertools.product(*axes):
        kw = {}
        for part in combo:
            kw.update(part)
        yield kw


def pins():
    """Every pin of the two modules as (label, callable, kwargs), those that
    need torch last (a killed mutant then rarely pays torch's import)."""
    from tests import test_oracle_pins, test_signal_model
    found = []
    for mod in (test_oracle_pins, test_signal_model):
        for name, fn in inspect.getmembers(mod, inspect.isfunction):
            if name.startswith("test_") and fn.__module__ == mod.__name__:
                found.append(("torch" in inspect.getsource(fn), mod, name, fn))
    found.sort(key=lambda x: x[0])
    for _, mod, name, fn in found:
        for kw in _cases(fn):
            yield f"{mod.__name__.split('.')[-1]}::{name}{kw or ''}", fn, kw


def main(lib_path: str) -> int:
    import pytest
    import oracle
    oracle.use_library(lib_path)
    for label, fn, kw in pins():
        try:
            fn(**kw)
        except pytest.skip.Exception:
            continue
        except Exception:  # a failed assertion, or an error the mistake causes
            print(f"killed by {label}", flush=True)
            traceback.print_exc(limit=2)
            return 1
    print("survived", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
