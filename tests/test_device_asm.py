"""Checks of the gfx950 instruction stream the library's sources compile to.

- Packed fp32 arithmetic: every source is built with the packed-fp32 target feature
  switched off, so no packed fp32 add, multiply or fma may appear in any kernel.
- m0 in the prefill kernels: the direct-to-LDS copies are issued from inline asm that
  loads m0 (the copy's LDS base) right before each copy.  The compiler reserves m0 and
  does not honour that clobber, so those kernels stay correct only while nothing else in
  them reads or writes m0: every m0 write must be one of these copy pairs.
"""
import concurrent.futures as cf
import os
import re

import pytest

from head_wise_sparse_amd import build as B


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    try:
        B.hipcc()
    except RuntimeError as e:
        pytest.skip(str(e))
    out = tmp_path_factory.mktemp("asm")
    srcs = B.sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        paths = list(ex.map(lambda s: B.device_asm(s, str(out / (os.path.basename(s)[:-4] + ".s"))), srcs))
    return {os.path.basename(p)[:-2]: open(p).read() for p in paths}


def _instructions(text):
    """(line, mnemonic, operands) of every instruction, comments and directives dropped."""
    out = []
    for line in text.splitlines():
        line = line.split(";")[0].strip()
        if not line or line.startswith(".") or line.endswith(":"):
            continue
        parts = line.split(None, 1)
        out.append((line, parts[0], parts[1] if len(parts) > 1 else ""))
    return out


def test_no_packed_fp32_arithmetic(asm):
    pat = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")
    bad = {name: pat.findall(text) for name, text in asm.items() if pat.search(text)}
    assert not bad, f"packed fp32 instructions in {sorted(bad)}"


def test_prefill_m0_only_feeds_the_lds_copies(asm):
    ins = _instructions(asm["rtp_prefill"])
    m0 = re.compile(r"\bm0\b")
    copies = 0
    for i, (line, op, args) in enumerate(ins):
        if op.startswith("global_load_lds_"):
            copies += 1
            prev = ins[i - 1]
            assert prev[1] == "s_mov_b32" and re.match(r"m0\s*,\s*s\d+$", prev[2]), \
                f"copy not preceded by its m0 load: {prev[0]!r} / {line!r}"
        elif m0.search(args):
            assert op == "s_mov_b32" and args.startswith("m0") and i + 1 < len(ins) \
                and ins[i + 1][1].startswith("global_load_lds_"), f"other use of m0: {line!r}"
    assert copies > 0, "no direct-to-LDS copies found in the prefill kernels"
