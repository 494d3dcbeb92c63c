"""Pin strength: plant plausible mistakes in copies of the oracle (a dropped
term, a wrong index or sign, a swapped operand, a missing clamp or guard) and
require that every mutant fails at least one pin.  All on the CPU; the real
oracle source is never modified.  Each mutant runs the pins in a child process,
since a mutant that drops a guard may read out of bounds; a crash of the child
counts as caught."""
import os
import subprocess
import sys

import pytest

import oracle

# (description, text in oracle.c, replacement, occurrence index).
# Not listed because they are equivalent mutants (they cannot change any
# output): dropping the clamp of a request's first output row (a begin past
# num_tokens already gives an empty extent through the clamped end), and
# rounding the decoded code to bf16 before scaling (an e4m3fn value has at most
# 4 significant bits, so that rounding is exact); and opening a task at slot 0
# instead of on a change of logical page (a request's tokens are consecutive,
# so after its first token the two coincide).
MUTANTS = [
    ("slot off by one", "int64_t slot = t % block_size;", "int64_t slot = (t + 1) % block_size;", 0),
    ("logical block off by one", "int64_t logical = t / block_size;",
     "int64_t logical = (t + 1) / block_size;", 0),
    ("seq_starts ignored by the gather", "int64_t s = seq_starts ? seq_starts[r] : 0;",
     "int64_t s = 0;", 0),
    ("end not clamped to num_tokens",
     "int64_t e = min64(request_end(cu_seq_lens, r, num_reqs, num_tokens, terminal), num_tokens);",
     "int64_t e = request_end(cu_seq_lens, r, num_reqs, num_tokens, terminal);", 0),
    ("open-ended last request reads a terminal entry", "if (terminal || r + 1 < num_reqs)",
     "if (1)", 0),
    ("open-ended last request ends at its start", "    return num_tokens;\n}",
     "    return cu_seq_lens[r];\n}", 0),
    ("table width guard dropped", "if (logical >= block_table_width)\n                continue;",
     "", 0),
    ("physical id upper guard off by one", "phys >= num_blocks", "phys > num_blocks", 0),
    ("negative physical id guard dropped", "phys < 0 || ", "", 0),
    ("cache strides swapped", "phys * src_block_stride + slot * src_token_stride",
     "phys * src_token_stride + slot * src_block_stride", 0),
    ("output row ignores the request offset", "(b + i) * dst_row_stride", "i * dst_row_stride", 0),
    ("block table row pitch uses the width", "(int64_t)r * block_table_ld",
     "(int64_t)r * block_table_width", 0),
    ("decode exponent bias off by one", "e - 10", "e - 9", 0),
    ("decode subnormal scale wrong", "ldexp((double)m, -9)", "ldexp((double)m, -10)", 0),
    ("decode sign dropped", "return (float)(sign ? -v : v);", "return (float)v;", 0),
    ("decode NaN test too wide", "if (e == 15 && m == 7)", "if (e == 15)", 0),
    ("bf16 ties away from zero", "(lower == 0x8000u && (upper & 1u))", "(lower == 0x8000u)", 0),
    ("bf16 truncates", "upper += 1u;", ";", 0),
    ("bf16 NaN not quietened", " | 0x0040u", "", 0),
    ("dequant scale dropped", "oracle_e4m3fn_to_f32(code) * scale", "oracle_e4m3fn_to_f32(code)", 0),
    ("dequant rounds the exact product to bf16 once",
     "volatile float product = oracle_e4m3fn_to_f32(code) * scale;",
     "double p = (double)oracle_e4m3fn_to_f32(code) * (double)scale; int ex;\n"
     "    double q = ldexp(nearbyint(frexp(p, &ex) * 256.0) / 256.0, ex);\n"
     "    volatile float product = (float)q;", 0),
    ("task page from the output row", "int64_t page = t / block_size;",
     "int64_t page = (b + i) / block_size;", 0),
    ("task end never extended", "out[5 * (count - 1) + 3] = (int32_t)(slot + 1);", ";", 0),
    ("task output row relative to the page", "task[4] = (int32_t)(b + i);",
     "task[4] = (int32_t)(b + slot);", 0),
    ("task begin slot off by one", "task[2] = (int32_t)slot;", "task[2] = (int32_t)(slot + 1);", 0),
    ("task map ignores seq_starts", "int64_t s = seq_starts ? seq_starts[r] : 0;",
     "int64_t s = 0;", 1),
    ("indexer position ignores the batch start", "int64_t pos = tid - batch_start;",
     "int64_t pos = tid;", 0),
    ("indexer row range check dropped",
     "if (tid < batch_start || tid >= batch_end)\n            continue;", "", 0),
    ("indexer batch upper bound dropped", "if (batch < 0 || batch >= num_batches)",
     "if (batch < 0)", 0),
    ("indexer table width guard dropped", "block_table_id >= block_table_width ||", "", 0),
    ("indexer block id upper guard off by one", "block_id >= num_blocks", "block_id > num_blocks", 0),
    ("indexer negative block id guard dropped", "block_id < 0 || ", "", 0),
    ("indexer table pitch uses the width", "batch * block_table_ld", "batch * block_table_width", 0),
    ("indexer tiles ordered column-major",
     "(block_offset / block_tile) * (head_dim / head_tile) + d / head_tile",
     "(d / head_tile) * (block_size / block_tile) + block_offset / block_tile", 0),
    ("indexer tile interior byte-major",
     "(block_offset % block_tile) * head_tile +\n                     d % head_tile",
     "(d % head_tile) * block_tile +\n                     block_offset % block_tile", 0),
    ("indexer flat values ignore the slot", "at = block_offset * head_dim + d;", "at = d;", 0),
    ("indexer scales at the record start",
     "record + (int64_t)block_size * head_dim + block_offset * 4", "record + block_offset * 4", 0),
    ("indexer slot from the row, not the position", "int64_t block_offset = pos % block_size;",
     "int64_t block_offset = tid % block_size;", 0),
    ("task end not clamped to num_tokens",
     "int64_t e = min64(request_end(cu_seq_lens, r, num_reqs, num_tokens, terminal), num_tokens);",
     "int64_t e = request_end(cu_seq_lens, r, num_reqs, num_tokens, terminal);", 1),
]


def _mutate(src: str, old: str, new: str, occ: int) -> str:
    pos = -1
    for _ in range(occ + 1):
        pos = src.find(old, pos + 1)
        assert pos >= 0, f"mutation target not found: {old!r}"
    return src[:pos] + new + src[pos + len(old):]


@pytest.mark.parametrize("desc,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, desc, old, new, occ):
    with open(oracle.SOURCE) as f:
        src = f.read()
    mutated = _mutate(src, old, new, occ)
    assert mutated != src
    csrc = os.path.join(tmp_path, "mutant.c")
    with open(csrc, "w") as f:
        f.write(mutated)
    lib = oracle.compile_source(csrc, os.path.join(tmp_path, "libmutant.so"))
    proc = subprocess.run([sys.executable, "-c", _CHILD, lib], cwd=_TESTS,
                          capture_output=True, text=True, timeout=300)
    caught = proc.returncode != 0 or "FAILED" in proc.stdout
    assert caught, f"no pin catches the mutant: {desc}\n{proc.stdout}\n{proc.stderr}"


_TESTS = os.path.dirname(os.path.abspath(__file__))
_CHILD = """
import sys
sys.path.insert(0, '..'); sys.path.insert(0, '.')
import oracle, oracle_pins
o = oracle.Oracle(sys.argv[1])
for check in oracle_pins.ALL_CHECKS:
    try:
        check(o)
        print('passed', check.__name__, flush=True)
    except AssertionError:
        print('FAILED', check.__name__, flush=True)
"""
