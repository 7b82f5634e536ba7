"""Host-side helpers of bench.py (no GPU): the input rotation of the isolated phase, and the
counter-summary lookup that gives a bench line its `traffic` only while the kernels are unchanged."""
import importlib.util
import os
import shutil
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    argv = sys.argv
    try:
        sys.argv = ["bench.py"]
        spec.loader.exec_module(mod)
    finally:
        sys.argv = argv
    return mod


def test_rotation_cycles_enough_copies():
    b = _bench()
    t = torch.arange(256, dtype=torch.float32)                 # 1 KiB
    nxt = b.rotation(t, min_bytes=4096)                        # four copies of 1 KiB
    seen = [nxt()[0] for _ in range(9)]
    ptrs = [x.data_ptr() for x in seen]
    assert seen[0] is t and len(set(ptrs[:4])) == 4            # the original and three distinct copies
    assert ptrs[4:8] == ptrs[:4] and ptrs[8] == ptrs[0]        # then the same four again, in order
    assert all(torch.equal(x, t) for x in seen)                # every copy holds the same values
    pair = b.rotation(t, t + 1, min_bytes=1)()                  # at least two copies; tuples for several inputs
    assert len(pair) == 2 and torch.equal(pair[1], t + 1)


def test_resident_hands_out_the_same_tensors():
    b = _bench()
    t = torch.zeros(8)
    nxt = b.resident(t)
    assert all(nxt()[0] is t for _ in range(3))


def test_traffic_applies_only_to_unchanged_sources(tmp_path):
    b = _bench()
    got = b.measured_traffic("b1_32k", 2)
    assert got and all(v is None or v > 0 for v in got.values())
    assert b.measured_traffic("b1_32k", 3) == {}              # another chunking: another launch
    assert b.measured_traffic("no_such_workload", 1) == {}
    # a copy of the tree with one kernel source changed: the calls built from it lose their figure
    root = tmp_path / "repo"
    shutil.copytree(os.path.join(ROOT, "profiles"), root / "profiles")
    shutil.copytree(os.path.join(ROOT, "speculative_kv_sparsity_amd", "csrc"),
                    root / "speculative_kv_sparsity_amd" / "csrc")
    with open(root / "speculative_kv_sparsity_amd" / "csrc" / "spc_attn.hip", "a") as f:
        f.write("\n// edited\n")
    b.ROOT = str(root)
    edited = b.measured_traffic("b1_32k", 2)
    assert edited["attn_partial"] is None and edited["attn"] is None
    assert edited["scores"] == got["scores"]                   # the scoring sources are untouched
