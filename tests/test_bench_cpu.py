"""Host logic of bench.py: the traffic-record lookup (a record counts only
while the sources it was measured on are unchanged and present) and the
algorithmic byte model of the MX expert GEMMs (OCP MX v1.0: 4- or 6-bit
element codes plus one E8M0 byte per 32 weights)."""
import hashlib
import importlib.util
import json
import os

import synth

_spec = importlib.util.spec_from_file_location("bench", os.path.join(os.path.dirname(__file__), "..", "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)


def _write_record(root, sources, digest):
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    rec = {"kernel": "expert_gate_up", "workload": "moe", "sources": sources, "sources_sha256": digest}
    with open(os.path.join(root, "profiles", "x_traffic.md"), "w") as fh:
        fh.write("# a record\n\ntraffic-record: " + json.dumps(rec) + "\n")


def _digest(root, sources):
    h = hashlib.sha256()
    for f in sources:
        h.update(f.encode())
        with open(os.path.join(root, "masked_block_diffusion_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def test_traffic_record_current_stale_and_missing(tmp_path):
    root = str(tmp_path)
    csrc = os.path.join(root, "masked_block_diffusion_amd", "csrc")
    os.makedirs(csrc)
    for f, text in (("a.hip", "one"), ("b.h", "two")):
        with open(os.path.join(csrc, f), "w") as fh:
            fh.write(text)
    _write_record(root, ["a.hip", "b.h"], _digest(root, ["a.hip", "b.h"]))
    rec = bench.traffic_record("expert_gate_up", "moe", root)
    assert rec is not None and rec["file"] == os.path.join("profiles", "x_traffic.md")
    assert bench.traffic_record("expert_gate_up", "moe-fp8", root) is None      # other workload
    with open(os.path.join(csrc, "b.h"), "w") as fh:                             # a source changed
        fh.write("three")
    assert bench.traffic_record("expert_gate_up", "moe", root) is None
    _write_record(root, ["a.hip", "gone.hip"], "0" * 64)                        # a source removed
    assert bench.traffic_record("expert_gate_up", "moe", root) is None


def test_mx_expert_bytes_per_weight():
    """Expert gate/up bytes at one assignment routed to one expert: the codes
    and scales of its two [De, d] matrices, the bf16 row, the bf16 output."""
    for name, bits in (("moe-mxfp4", 4), ("moe-mxfp6", 6)):
        cfg = synth.get_run(name).model
        d, De = cfg.d_model, cfg.d_expert
        nbytes, flops = bench.kernel_model("expert_gate_up", cfg, 1, [1], experts_used=1)
        A = cfg.top_k
        assert nbytes == 2 * De * d * (bits / 8 + 1 / 32) + A * d * 2 + A * De * 2
        assert flops == 2.0 * A * 2 * De * d
