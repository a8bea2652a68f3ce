"""Host checks of the rocprofv3 summariser and of how bench.py picks up measured traffic."""
import json
import sqlite3

import bench
from dynamic_sparse_attention_dsv_amd import profile_summary as ps
from workloads import get_config

KNAME = "void dsv::attn_fwd_bf16_kernel<128, 128>(unsigned short const*, int)"


def _db(path, kernels=None, counter=None, values=None):
    con = sqlite3.connect(path)
    con.execute("create table top_kernels (name text, total_calls int, total_duration real, average real, "
                "percentage real)")
    con.execute("create table counters_collection (kernel_name text, counter_name text, value real)")
    for row in kernels or []:
        con.execute("insert into top_kernels values (?,?,?,?,?)", row)
    for name, v in values or []:
        con.execute("insert into counters_collection values (?,?,?)", (name, counter, v))
    con.commit()
    con.close()
    return str(path)


def test_summary_scales_counters_by_the_calibration_copy(tmp_path):
    kt = _db(tmp_path / "kt.db", kernels=[(KNAME, 2, 84000.0, 42000.0, 90.0),
                                          ("__amd_rocclr_copyBuffer", 1, 400.0, 400.0, 1.0)])
    fe = _db(tmp_path / "fe.db", counter="FETCH_SIZE",
             values=[("__amd_rocclr_copyBuffer", 524288.0), (KNAME, 1000.0), (KNAME, 3000.0)])
    wr = _db(tmp_path / "wr.db", counter="WRITE_SIZE", values=[("__amd_rocclr_copyBuffer", 1048576.0), (KNAME, 10.0)])
    cal, table = ps.summarise(kt, fe, wr)
    assert cal["fetch_scale"] == 2.0 and cal["write_scale"] == 1.0
    row = [r for r in table if r["kernel"].startswith("attn_fwd_bf16_kernel")][0]
    assert row["avg_ms"] == 42.0                      # microseconds -> milliseconds
    assert row["read_bytes"] == 2000.0 * 2 * 1024     # mean over dispatches, x2, KiB -> bytes
    assert row["write_bytes"] == 10.0 * 1024
    rec = ps.to_record(cal, table, "cmd", "w")
    assert rec["kernels"]["attn_fwd_kernel"]["source_sha256"] == ps.source_hash("attn_fwd_kernel")
    assert "| attn_fwd_bf16_kernel<128, 128> | 2 | 42.000 |" in ps.to_markdown(cal, table, "cmd", "t")


def test_bench_reports_traffic_only_for_an_unchanged_kernel(tmp_path, monkeypatch):
    cfg = get_config("C5")
    (tmp_path / "profiles").mkdir()
    rec = {"workload": f"C5: ..., {cfg.generator} inputs",
           "kernels": {"attn_fwd_kernel": {"read_bytes": 5.0, "write_bytes": 1.0,
                                           "source_sha256": ps.source_hash("attn_fwd_kernel")},
                       "attn_bwd_dq_kernel": {"read_bytes": 5.0, "write_bytes": 1.0, "source_sha256": "0" * 64}}}
    (tmp_path / "profiles" / "c5_kernel_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic(cfg, "attn_fwd_kernel")[0] == 6.0
    assert bench.measured_traffic(cfg, "attn_bwd_dq_kernel") == (None, None)   # sources changed since
    assert bench.measured_traffic(cfg, "scores_kernel") == (None, None)        # never measured
    other = "g2" if cfg.generator == "g1" else "g1"
    rec["workload"] = f"C5: ..., {other} inputs"
    (tmp_path / "profiles" / "c5_kernel_traffic.json").write_text(json.dumps(rec))
    assert bench.measured_traffic(cfg, "attn_fwd_kernel") == (None, None)      # counters of other inputs


def test_counter_summary_ratios(tmp_path):
    from dynamic_sparse_attention_dsv_amd import profile_counters as pc

    def pmc(path, rows):
        con = sqlite3.connect(path)
        con.execute("create table counters_collection (kernel_name text, counter_name text, value real)")
        con.executemany("insert into counters_collection values (?,?,?)", rows)
        con.commit()
        con.close()
        return str(path)

    # two passes; GRBM_GUI_ACTIVE in both (the first is kept); two dispatches averaged in pass 1
    p1 = pmc(tmp_path / "p1.db", [(KNAME, "GRBM_GUI_ACTIVE", 1000.0), (KNAME, "SQ_BUSY_CU_CYCLES", 256000.0),
                                  (KNAME, "SQ_VALU_MFMA_BUSY_CYCLES", 512000.0),
                                  (KNAME, "SQ_VALU_MFMA_BUSY_CYCLES", 512000.0), (KNAME, "SQ_INSTS_MFMA", 100.0),
                                  (KNAME, "SQ_INSTS_VALU", 250.0)])
    p2 = pmc(tmp_path / "p2.db", [(KNAME, "GRBM_GUI_ACTIVE", 999.0), (KNAME, "SQ_VALU_MFMA_COEXEC_CYCLES", 128000.0),
                                  (KNAME, "TCC_HIT_sum", 30.0), (KNAME, "TCC_MISS_sum", 10.0),
                                  (KNAME, "SQ_WAVE_CYCLES", 400.0), (KNAME, "SQ_WAIT_INST_ANY", 100.0)])
    data = pc.merge([p1, p2])
    r = pc.ratios(data["attn_fwd_bf16_kernel<128, 128>"], cus=256)
    assert r["MFMA busy"] == 512000.0 / (4 * 256000.0)   # 0.5
    assert r["co-exec"] == 0.25 and r["VALU / MFMA"] == 2.5
    assert r["L2 hit"] == 0.75 and r["wait"] == 0.25 and r["LDS conflicts"] is None
    md = pc.to_markdown(data, ["attn_fwd"], 256, "cmd", "t")
    assert "| attn_fwd_bf16_kernel<128, 128> | 50.0 % | 25.0 % | 2.50 | 25.0 % | - | - | 75.0 % |" in md


def test_effective_clocks(tmp_path):
    from dynamic_sparse_attention_dsv_amd import profile_counters as pc

    db = _db(tmp_path / "clk.db", kernels=[(KNAME, 2, 20000.0, 10000.0, 90.0)])  # 10 ms per dispatch
    con = sqlite3.connect(db)
    con.executemany("insert into counters_collection values (?,?,?)",
                    [(KNAME, "GRBM_GUI_ACTIVE", 8 * 1.5e7), (KNAME, "SQ_BUSY_CU_CYCLES", 256 * 1.4e7)])
    con.commit()
    con.close()
    (k, ms, g1, g2), = pc.clocks(db, ["attn_fwd"], xcds=8, cus=256)
    assert ms == 10.0 and abs(g1 - 1.5) < 1e-12 and abs(g2 - 1.4) < 1e-12
    assert "| 1.500 | 1.400 |" in pc.clocks_markdown([(k, ms, g1, g2)], "cmd", "t")
