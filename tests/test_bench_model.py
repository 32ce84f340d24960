"""CPU checks of the benchmark's byte model and of its committed counter record.

The roofline entry divides algorithmic bytes by measured time, so the byte
model is pinned here against figures worked out by hand from the shapes:
at 4 sequences x 262,144 keys, bf16 rows of 256 B, the step moves K once
(256 MiB), writes the fp32 scores (4 MiB), reads the pool's scores back
(262,016 x 4 B per sequence), gathers 1,152 K and V rows per sequence
(2.25 MiB) and reads q twice and writes o (0.125 MiB).
"""

import json
import os

import pytest

import bench
from workloads import WORKLOADS

MIB = 1 << 20


def test_headline_step_bytes():
    ab = bench.algorithmic_bytes(WORKLOADS["decode_bf16_256k_b4"])
    assert ab["k_stream"] == 256 * MIB
    assert ab["scores_write"] == 4 * MIB
    assert ab["scores_read"] == 4 * 262016 * 4
    assert ab["gather"] == 4 * 1152 * 2 * 256
    assert ab["q_out"] == 4 * 32 * 128 * 8
    assert ab["scoring_call"] == 256 * MIB + 4 * MIB
    assert ab["step"] / MIB == pytest.approx(266.37, abs=0.01)


def test_e4m3_rows_halve_the_stream():
    bf, f8 = (bench.algorithmic_bytes(WORKLOADS[n])
              for n in ("decode_bf16_256k_b4", "decode_fp8_256k_b4"))
    assert f8["k_stream"] * 2 == bf["k_stream"]
    assert f8["gather"] * 2 == bf["gather"]
    assert f8["scores_write"] == bf["scores_write"]


def test_counter_record_is_well_formed():
    path = os.path.join(bench.ROOT, "profiles", f"{bench.WORKLOAD}_traffic.json")
    rec = json.load(open(path))
    assert rec["workload"] == bench.WORKLOAD
    per = rec["bytes_per_dispatch"]
    # the one-pass scoring kernel reads the 256 MiB of K once and, after its
    # grid barrier, the blocks it could not keep on chip again (3 of each
    # wave's 32 blocks at 4,096 keys per workgroup: 9.4 %), give or take a
    # few percent of other traffic
    for k in ("score_onepass<false, false, 20>", "score_onepass<false, true, 20>"):
        assert 256 * MIB * (1 + 3 / 32) <= per[k] <= 1.15 * 256 * MIB
    assert 1.9 <= rec["fetch_scale"] <= 2.1
