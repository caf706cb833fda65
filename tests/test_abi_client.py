"""The C ABI used from plain C: tests/abi_client.c is compiled with gcc as C11 against
include/forkkv.h and linked to libforkkv.so; its block tables and copy-on-write reports must
equal the pool model's, and its decode plan the Python binding's, bit for bit."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import PoolModel

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INCLUDE = "/opt/rocm/include"

# the script abi_client.c replays (same order)
OPS = [("create", "root", 0), ("append", "root", 45), ("fork", "root", 45, "a0"),
       ("append", "a0", 10), ("fork", "root", 32, "a1"), ("append", "a1", 20),
       ("fork", "a1", 40, "a2"), ("append", "a2", 3)]
AGENTS = ["a0", "a1", "a2"]
MAX_PAGES = 8


@pytest.fixture(scope="module")
def client_output(tmp_path_factory):
    from lora_shared_prefix_amd import forkkv
    if shutil.which("gcc") is None or not os.path.isdir(os.path.join(ROCM_INCLUDE, "hip")):
        pytest.skip("gcc or the HIP headers are not available")
    lib_dir = os.path.dirname(forkkv.LIB_PATH)
    exe = str(tmp_path_factory.mktemp("abi") / "abi_client")
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I" + ROCM_INCLUDE,
           os.path.join(ROOT, "tests", "abi_client.c"), "-o", exe, "-L" + lib_dir, "-lforkkv",
           "-Wl,-rpath," + lib_dir]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=120)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    lines = run.stdout.strip().splitlines()
    assert lines[-1] == "ok", run.stdout
    return lines


def _model():
    pm = PoolModel(64, 64, 16)
    names, cows = {}, []
    for op in OPS:
        if op[0] == "create":
            names[op[1]] = pm.create(bool(op[2]))
        elif op[0] == "append":
            c = pm.append(names[op[1]], op[2])[2]
            cows += [c] if c else []
        else:
            names[op[3]], c = pm.fork(names[op[1]], op[2])
            cows += [c] if c else []
    return pm, names, cows


def test_c_client_tables_match_the_model(client_output):
    pm, names, cows = _model()
    bt, rt, lens = pm.tables([names[a] for a in AGENTS], MAX_PAGES)
    got_cows = [tuple(int(v) for v in l.split()[1:]) for l in client_output if l.startswith("cow ")]
    assert got_cows == [tuple(c) for c in cows]
    assert len(got_cows) == 2  # a0's packed tail and a2's
    seqs = [l.split() for l in client_output if l.startswith("seq ")]
    assert [s[1] for s in seqs] == AGENTS
    for i, s in enumerate(seqs):
        vals = [int(v) for v in s[2:]]
        assert vals[0] == lens[i]
        assert vals[1:1 + MAX_PAGES] == list(bt[i])
        assert vals[1 + MAX_PAGES:] == list(rt[i])


def test_c_client_plan_matches_the_binding(client_output):
    from lora_shared_prefix_amd import forkkv as fk
    pool = fk.Pool(64, 64, 2, 64, 8, "f32")
    names, _ = pool.replay(OPS)
    plan = fk.Plan(pool, [names[a] for a in AGENTS], 4)
    want = np.asarray(plan.blob(), dtype=np.int64)
    head = [l.split() for l in client_output if l.startswith("plan ")][0]
    blob = [l.split() for l in client_output if l.startswith("blob")][0][1:]
    got = np.array([int(v) for v in blob], dtype=np.int64)
    assert int(head[1]) == plan.info["n_items"] and int(head[2]) == plan.info["n_slots"]
    assert int(head[3]) == got.size == want.size
    assert np.array_equal(got, want)


def test_c_client_error_paths(client_output):
    """Calls that the header says fail before any device work return the documented codes."""
    from lora_shared_prefix_amd import forkkv as fk
    got = {l.split()[1]: int(l.split()[2]) for l in client_output if l.startswith("err ")}
    assert got == {"decode_null": fk.EINVAL, "decode_no_storage": fk.ESTATE,
                   "prefill_null": fk.EINVAL, "prefill_no_storage": fk.ESTATE,
                   "upload_null": fk.EINVAL, "plan_heads": fk.EINVAL,
                   "fork_past_end": fk.EINVAL, "page_size": fk.EINVAL,
                   "append_freed": fk.EINVAL}
