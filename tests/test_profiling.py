"""Host logic of the rocprofv3 summaries: the code digest that ties a traffic
record to the kernels it was measured on, and the record lookup."""

from __future__ import annotations

import json

from mixture_experts_gemv_amd import profiling


def test_code_only_ignores_comments_and_layout():
    a = "int x = 1; // one\n/* block\n comment */ int  y =\n 2;\n"
    b = "int x = 1;\nint y = 2; /* other words */\n"
    assert profiling._code_only(a) == profiling._code_only(b) == "int x = 1; int y = 2;"
    assert profiling._code_only("int x = 1;") != profiling._code_only("int x = 2;")


def test_digest_is_stable_and_hex():
    d = profiling.source_digest()
    assert d == profiling.source_digest()
    assert len(d) == 64 and int(d, 16) >= 0


def test_load_traffic_matches_kernel_workload_and_digest(tmp_path):
    rec = dict(kernel="k_gemm_lds<0, false, 4, false>", workload="w_M8",
               source_sha256=profiling.source_digest(), traffic_bytes=123.0)
    (tmp_path / "a.traffic.json").write_text(json.dumps(rec))
    got = profiling.load_traffic(str(tmp_path), "k_gemm_lds<0", "w_M8")
    assert got is not None and got["traffic_bytes"] == 123.0
    assert profiling.load_traffic(str(tmp_path), "k_gemm_lds<0", "w_M16") is None
    assert profiling.load_traffic(str(tmp_path), "k_gateup_m1", "w_M8") is None
    rec["source_sha256"] = "0" * 64
    (tmp_path / "a.traffic.json").write_text(json.dumps(rec))
    assert profiling.load_traffic(str(tmp_path), "k_gemm_lds<0", "w_M8") is None
