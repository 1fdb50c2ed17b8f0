"""The attention tiles' buffer loads to LDS are waited for before the LDS is touched (no GPU needed).

attn_tile sends K rows straight to LDS with buffer loads to LDS; the compiler does not order LDS
reads after such loads by itself, so the tile waits explicitly (vmcnt <= the loads issued after
them).  This test builds attn.hip to gfx950 assembly (default and timeline variants) and checks, in
every kernel, that each such load is followed in straight-line code by an s_waitcnt whose vmcnt
covers it before any LDS instruction, barrier or branch.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_kv_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

VMEM = re.compile(r"^(global_|buffer_|flat_|scratch_)")
STOP = re.compile(r"^(ds_|s_barrier|s_endpgm|s_branch|s_cbranch|s_setpc|s_swappc)")
WAIT = re.compile(r"^s_waitcnt\b.*\bvmcnt\((\d+)\)")


def uncovered_lds_loads(asm: str):
    """(kernel, line) of every buffer load to LDS not waited for before the next LDS access, and the
    number of such loads seen."""
    bad, seen = [], 0
    for m in re.finditer(r"^(_Z\w+):.*?^\.Lfunc_end", asm, re.S | re.M):
        name = m.group(1)
        body = [l.strip() for l in m.group(0).splitlines()]
        body = [l for l in body if l and not l.startswith((";", "."))]
        for k, line in enumerate(body):
            words = line.split(";")[0].split()
            if not (words[0].startswith("global_load_lds") or
                    (words[0].startswith("buffer_load") and words[-1] == "lds")):
                continue
            seen += 1
            after, ok = 0, False
            for nxt in body[k + 1:]:
                w = WAIT.match(nxt)
                if w:
                    ok = int(w.group(1)) <= after
                    break
                if STOP.match(nxt):
                    break
                if VMEM.match(nxt):
                    after += 1
            if not ok:
                bad.append((name, line))
    return bad, seen


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="hipcc not found")
@pytest.mark.parametrize("timeline", [False, True])
def test_lds_loads_waited(tmp_path, timeline):
    out = tmp_path / "attn.s"
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           os.path.join(CSRC, "attn.hip"), "-o", str(out)]
    if timeline:
        cmd.insert(1, "-DKVS_TIMELINE")
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    bad, seen = uncovered_lds_loads(out.read_text())
    # fp16 tiles: 8 loads each; Q8_0 and INT8 tiles: 4 each; 4 IL/PHYS variants x 5 group sizes
    assert seen == 20 * 8 + 2 * 20 * 4, seen
    assert not bad, bad[:5]


def test_checker_catches_a_missing_wait():
    """The scan itself: a load to LDS read back before its wait, or waited with too large a count, is
    reported; one covered by the wait is not."""
    good = """_Zk:
\tbuffer_load_dwordx4 v1, s[4:7], 0 offen nt lds
\tglobal_load_dwordx4 v[2:5], v[6:7], off nt
\ts_waitcnt vmcnt(1)
\tds_read_b128 v[8:11], v12
.Lfunc_end0:
"""
    early = good.replace("\ts_waitcnt vmcnt(1)\n\tds_read_b128 v[8:11], v12\n",
                         "\tds_read_b128 v[8:11], v12\n\ts_waitcnt vmcnt(1)\n")
    loose = good.replace("vmcnt(1)", "vmcnt(2)")
    assert uncovered_lds_loads(good) == ([], 1)
    assert len(uncovered_lds_loads(early)[0]) == 1
    assert len(uncovered_lds_loads(loose)[0]) == 1
