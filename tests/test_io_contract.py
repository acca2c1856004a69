"""The probe branch streams no extra K/V and issues no extra matrix
instructions in decode (the news.chathome.org article on Parallax, "Hardware
argument": the two scoring branches share the K/V tiles, so no extra I/O per
iteration; the gist.science summary, "Hardware-aware algorithm": QK and RK
inside the matrix instructions attention already issues).

Checked on the committed counter summary of the decode workload, taken with
and without the probe on the same inputs: fetched bytes may differ by at most
the probe rows plus 1% of the K/V (counter noise), and the MFMA and VALU
instruction counts must be equal.  The summary must have been taken on the
decode kernel sources as they are now.
"""
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

PROFILE = os.path.join(ROOT, "profiles", "decode_io_contract_b64_l4096.md")


def _values():
    text = open(PROFILE).read()
    return dict(re.findall(r"^(\w+):\s*([0-9a-f.eE+]+)\s*$", text, flags=re.M))


def test_profile_taken_on_current_decode_sources():
    assert _values()["kernel_source_digest"] == bench.source_digest(bench.DECODE_SOURCES)


def test_probe_adds_no_kv_traffic():
    v = _values()
    kv, rho = float(v["kv_bytes_per_call"]), float(v["rho_bytes_per_call"])
    with_rho, without = float(v["fetch_bytes_mean_rho"]), float(v["fetch_bytes_mean_null"])
    assert without >= kv  # both read the whole cache
    assert with_rho - without <= rho + 0.01 * kv


def test_probe_adds_no_matrix_or_vector_instructions():
    v = _values()
    assert int(v["mfma_instructions_rho"]) == int(v["mfma_instructions_null"]) > 0
    assert int(v["valu_instructions_rho"]) == int(v["valu_instructions_null"]) > 0
