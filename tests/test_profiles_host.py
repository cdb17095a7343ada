"""The committed rocprofv3 summaries under profiles/ belong to the current
kernels: the HBM traffic record (the source of bench.py's roofline.traffic)
carries the SHA-256 of the kernel sources it was measured on, and every
summary names the command that produced it."""

import hashlib
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROF = os.path.join(ROOT, "profiles")


def test_traffic_record_matches_kernel_sources():
    with open(os.path.join(PROF, "hbm_traffic.json")) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    assert h.hexdigest() == rec["source_sha256"], (
        "kernel sources changed since profiles/hbm_traffic.json was measured: "
        "take the FETCH_SIZE / WRITE_SIZE runs again")
    # every HIP source of the library that the timed kernels come from is hashed
    csrc = os.path.join("sliding_window_attention_amd", "csrc")
    for name in ("fwd_bf16.hip", "split_kv.hip", "swa_internal.h", "swa_api.hip", "rope.hip"):
        assert os.path.join(csrc, name) in rec["sources"]
    for k in rec["kernels"].values():
        assert k["read_bytes"] > 0 and k["write_bytes"] > 0


def test_summaries_name_their_commands():
    names = sorted(n for n in os.listdir(PROF) if n.endswith((".txt", ".md")))
    assert names, "no profile summaries"
    for n in names:
        with open(os.path.join(PROF, n)) as f:
            text = f.read()
        assert "rocprofv3" in text, f"{n} does not give the command that made it"
        assert len(text) < 64 * 1024, f"{n} is not a short summary"
