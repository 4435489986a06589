"""The C ABI from C: tests/c_consumer.c is compiled with gcc (C11, -Wall
-Werror) against include/pgqa.h and include/pgqa_sched.h, linked to libpgqa.so
and run on the host; what it prints must match the Python binding and the
host-producer oracle.  No GPU."""
import os
import shutil
import subprocess

import pytest

import oracle.sched as S
import paged_gqa_decode_head_amd as pg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def output(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not available")
    exe = str(tmp_path_factory.mktemp("cabi") / "c_consumer")
    libdir = os.path.dirname(pg.LIB_PATH)
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_consumer.c"), "-L", libdir, "-lpgqa", f"-Wl,-rpath,{libdir}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    return r.stdout.splitlines()


def _line(lines, key):
    return [l for l in lines if l.startswith(key + " ")]


def test_version_pool_bytes_and_plans(output):
    assert _line(output, "version") == [f"version {pg.version()}"]
    assert _line(output, "pool_bytes") == [f"pool_bytes {pg.pool_bytes(32, 16, 8)}"]
    plans = _line(output, "decode_plan")
    for line, args in zip(plans, [(64, 2049), (1, 32769)]):
        p = pg.plan_decode(256, 16, args[0], 8, 16, args[1])
        assert line == f"decode_plan {p.split_tokens} {p.max_splits} {p.waves_per_split} {p.load_hint} {p.kernel}"
    want = []
    for args in [(9, 552, 512, 6656), (8, 40, 5, 4096)]:  # a prefill slice with verify rows; verify rows only
        c = pg.plan_chunk(256, 16, args[0], args[1], 8, 16, args[2], args[3])
        want.append(f"chunk_plan {c.split_tokens} {c.max_splits} {c.short_split_tokens} {c.kernel}")
    assert _line(output, "chunk_plan") == want
    assert want[0].endswith(" 1") and want[1].endswith(" 2")


def test_mixed_plan_matches_the_binding(output):
    import numpy as np

    qsl = np.array([0, 1, 2, 7, 47], dtype=np.int32)
    ctx = np.array([300, 1200, 900, 2040], dtype=np.int32)
    p, items = pg.plan_mixed(256, 16, 8, 16, qsl, ctx)
    flat = items.reshape(-1).astype(np.int64)
    checksum = int(((np.arange(flat.size, dtype=np.int64) + 1) * flat).sum())
    assert _line(output, "mixed_plan") == [
        f"mixed_plan {p.split_wide} {p.split_columns} {p.max_splits} {p.num_items} {p.num_combine} {checksum}"]
    assert p.num_items > 0 and p.num_combine > 0


def test_error_reporting(output):
    (line,) = _line(output, "error")
    assert line.startswith("error ") and "|" in line and len(line.split("|")[1].strip()) > 0


def test_producers_match_the_oracle(output):
    toks = [5, 1, 2, 3, 7, 1, 2, 3]
    draft = S.prompt_lookup(toks, 1, 3, 4)
    assert _line(output, "draft") == ["draft " + " ".join(str(x) for x in [len(draft)] + draft)]
    acc = S.accept_greedy([7, 1, 9], [7, 1, 2, 4])
    assert _line(output, "accept") == ["accept " + " ".join(str(x) for x in [len(acc)] + acc)]


def test_plan_step_matches_the_oracle(output):
    cfg = {"token_budget": 16, "max_segments": 4, "chunked_prefill": 1, "block_size": 16, "max_blocks_per_seq": 4}
    seqs = [{"cached": 20, "prompt_left": 0, "num_draft": 2, "num_blocks": 2},
            {"cached": 0, "prompt_left": 40, "num_draft": 0, "num_blocks": 0}]
    tables = [[3, 8, -1, -1], [-1, -1, -1, -1]]
    free = [0, 1, 2, 4, 5, 6]
    r = S.plan_step(cfg, seqs, tables, free)
    segs = r["segs"]
    assert _line(output, "plan") == [f"plan {len(segs)} segments {r['query_start_loc'][-1]} tokens"]
    assert _line(output, "seg") == [f"seg {a} {b} {c} {d}" for a, b, c, d in segs]
    t = " ".join(str(x) for x in tables[0]) + " | " + " ".join(str(x) for x in tables[1])
    assert _line(output, "tables") == [f"tables {t} | free {len(free)}"]
