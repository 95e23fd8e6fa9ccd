"""libpa used from C alone (tests/native/c_abi_demo.c: HIP runtime, block manager,
executor, pa_decode; no Python, no PyTorch), checked against the CPU oracle.

The demo writes every input it drew and everything the device computed; the oracle
replays the prompts' append, the copy-on-write pairs and the step's append on its
own zeroed pools, which must then equal the device pools bit for bit, and decodes
(fp32 KV: max-abs 1e-5).  pa_decode on the executor's tables must reproduce the
executor's output bit for bit, and so must pa_decode_append given the step's rows
again (it rewrites them into the slots the executor put them in)."""

from __future__ import annotations

import pathlib
import shutil
import subprocess

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

ROOT = pathlib.Path(__file__).resolve().parents[1]


@pytest.fixture(scope="module")
def demo(tmp_path_factory):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_414_amd import ops
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = tmp_path_factory.mktemp("c_abi") / "c_abi_demo"
    lib_dir = ops.LIB_PATH.parent
    subprocess.run([cc, "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    f"-I{ROOT / 'include'}", str(ROOT / "tests" / "native" / "c_abi_demo.c"),
                    f"-L{lib_dir}", "-lpa", "-L/opt/rocm/lib", "-lamdhip64",
                    f"-Wl,-rpath,{lib_dir}", "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)],
                   check=True, timeout=120)
    return exe


def _read(path):
    raw = path.read_bytes()
    pos = 0

    def take(dtype, shape):
        nonlocal pos
        n = int(np.prod(shape)) * np.dtype(dtype).itemsize
        a = np.frombuffer(raw, dtype=dtype, count=int(np.prod(shape)), offset=pos).reshape(shape)
        pos += n
        return a.copy()

    h, d, bs, nb, s, mb, t, c = take(np.int32, (8,)).tolist()
    rec = {"H": h, "D": d, "BS": bs, "NB": nb, "S": s, "MB": mb}
    rec["prompt_slots"] = take(np.int32, (t,))
    rec["prompt_k"] = take(np.float32, (t, h, d))
    rec["prompt_v"] = take(np.float32, (t, h, d))
    rec["q"] = take(np.float32, (s, h, d))
    rec["new_k"] = take(np.float32, (s, h, d))
    rec["new_v"] = take(np.float32, (s, h, d))
    rec["slots"] = take(np.int32, (s,))
    rec["pairs"] = take(np.int32, (c, 2))
    rec["tables"] = take(np.int32, (s, mb))
    rec["ctx"] = take(np.int32, (s,))
    rec["out"] = take(np.float32, (s, h, d))
    rec["out2"] = take(np.float32, (s, h, d))
    rec["out3"] = take(np.float32, (s, h, d))
    rec["k_pool"] = take(np.float32, (nb, h, bs, d))
    rec["v_pool"] = take(np.float32, (nb, h, bs, d))
    assert pos == len(raw)
    return rec


def test_c_program_matches_oracle(demo, tmp_path):
    out_file = tmp_path / "demo.bin"
    res = subprocess.run([str(demo), str(out_file)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    r = _read(out_file)
    # sequence 3 was forked from sequence 0 (20 tokens: a partly filled shared block)
    assert r["pairs"].shape == (1, 2)
    assert r["ctx"].tolist() == [21, 34, 17, 21]
    shape = (r["NB"], r["H"], r["BS"], r["D"])
    k = np.zeros(shape, np.float32)
    v = np.zeros(shape, np.float32)
    oracle.cache_append(k, v, r["prompt_k"], r["prompt_v"], r["prompt_slots"], inplace=True)
    oracle.block_copy(k, v, r["pairs"], inplace=True)
    want_slots = oracle.slots_for_positions(r["tables"], range(r["S"]), r["ctx"] - 1, r["BS"])
    assert np.array_equal(r["slots"].astype(np.int64), want_slots)
    oracle.cache_append(k, v, r["new_k"], r["new_v"], r["slots"], inplace=True)
    assert np.array_equal(r["k_pool"].view(np.uint32), k.view(np.uint32))
    assert np.array_equal(r["v_pool"].view(np.uint32), v.view(np.uint32))
    want = oracle.decode(r["q"], k, v, r["tables"], r["ctx"], 0.125)
    assert float(np.max(np.abs(r["out"].astype(np.float64) - want))) <= 1e-5
    assert np.array_equal(r["out"].view(np.uint32), r["out2"].view(np.uint32))
    assert np.array_equal(r["out"].view(np.uint32), r["out3"].view(np.uint32))
