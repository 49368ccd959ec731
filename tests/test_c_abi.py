"""The ABI from plain C: tests/c/plan_from_c.c, built with gcc against include/pkv.h
and libpkv.so, runs the host-only entry points; its plan must equal the oracle's bit
for bit (automatic and fixed tiles), and its status codes and strings those of the
header."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import paged_kv_gqa_amd as pkv
from oracle import plan as ref_plan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.dirname(pkv.LIB_PATH)


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    out = str(tmp_path_factory.mktemp("c_abi") / "plan_from_c")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "plan_from_c.c"), "-L", LIB_DIR, "-lpkv",
                    "-Wl,-rpath," + LIB_DIR, "-o", out], check=True)
    return out


def run(exe, W, Hkv, tile, lens):
    r = subprocess.run([exe, str(W), str(Hkv), str(tile)] + [str(x) for x in lens],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return r.stdout.splitlines()


@pytest.mark.parametrize("W,Hkv,tile,lens", [
    (7, 2, 0, [1, 15, 16, 17, 33, 100, 257, 700]),
    (3, 2, 48, [31, 32, 47, 48, 49, 95, 96, 97]),
    (64, 8, 0, [4096, 128, 30000, 777, 1, 65536]),
    (512, 8, 2048, [int(x) for x in np.random.default_rng(7).integers(1, 40000, 100)]),
])
def test_plan_from_c_equals_the_oracle(exe, W, Hkv, tile, lens):
    out = run(exe, W, Hkv, tile, lens)
    kv = {}
    items = []
    for line in out:
        key, _, rest = line.partition(" ")
        if key == "item":
            items.append([int(x) for x in rest.split()])
        else:
            kv.setdefault(key, []).append(rest)
    assert int(kv["abi"][0]) == pkv.pkv_abi_version()
    for s in kv["status"]:
        code, _, text = s.partition(" ")
        assert text == pkv.pkv_status_string(int(code))
    T, N, NP = (int(x) for x in kv["plan"][0].split())
    want_T = tile or ref_plan.auto_tile_tokens(lens, 1, 4 * Hkv, Hkv, 128, 16, "bf16", W)
    ref = ref_plan.lpt_plan(lens, Hkv, want_T, W)
    assert T == want_T and N == NP == len(ref["items"])
    assert np.array_equal(np.array(items, np.int32).reshape(-1, 4), ref["items"])
    assert [int(x) for x in kv["offsets"][0].split()] == ref["worker_offsets"].tolist()
    assert [int(x) for x in kv["rtb"][0].split()] == ref["req_tile_base"].tolist()
    assert int(kv["workspace"][0]) == pkv.pkv_workspace_bytes(NP, 4, 128)
    code, _, msg = kv["seq_error"][0].partition(" ")
    assert int(code) == pkv.PKV_ERR_SEQ and "seq_lens[0] = 0" in msg
