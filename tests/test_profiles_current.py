"""The committed rocprofv3 summaries describe the kernels as they are: each
summary records the sha256 of the source file its kernels were built from,
and that must be the current file's.  (bench.py applies the same rule to the
traffic counters of the GEMM and of search+compress, and reports no traffic
when they are stale.)"""
import hashlib
import json
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
LINE = re.compile(r"Kernel source sha256\[:16\] = `([0-9a-f]{16})` \(([^)]+)\)")


def sha16(rel):
    with open(os.path.join(ROOT, rel), "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def test_every_kernel_summary_matches_its_source():
    seen = 0
    for name in sorted(os.listdir(PROFILES)):
        if not name.endswith(".md"):
            continue
        for want, rel in LINE.findall(open(os.path.join(PROFILES, name)).read()):
            assert sha16(rel) == want, f"{name} was profiled from another version of {rel}"
            seen += 1
    assert seen >= 5


def test_counter_summaries_match_their_sources():
    for name, src in (("spmm_group_gpt2-1.5b_counters.json", "sp24_spmm.hip"),
                      ("search_compress_gpt2-1.5b_counters.json", "sp24_search.hip")):
        c = json.load(open(os.path.join(PROFILES, name)))
        assert c["source_sha256_16"] == sha16("structured_sparse_transformer_amd/csrc/" + src), name
        assert c["hbm_bytes_per_launch"] > 0 and c["algorithmic_bytes_per_launch"] > 0
