"""Host-only checks of the rocprofv3 summariser that feeds bench.py's traffic field."""
import csv
import os

import profsum


def test_digest_ignores_comments_only():
    base = {r: f"int x{i} = {i};\n" for i, r in enumerate(profsum.ATTN_SOURCES)}
    d0 = profsum.attention_source_digest(lambda r: base[r])
    commented = {r: "// note\n/* block\n comment */" + t + "  // tail\n" for r, t in base.items()}
    assert profsum.attention_source_digest(lambda r: commented[r]) == d0
    changed = dict(base)
    changed[profsum.ATTN_SOURCES[0]] = "int x0 = 7;\n"
    assert profsum.attention_source_digest(lambda r: changed[r]) != d0


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writerows(rows)


def test_traffic_scaling_and_readback(tmp_path):
    attn = "void cosa::(anonymous namespace)::attn_fwd_kernel<128, 4, 1>(cosa::AttnParams)"
    _counter_csv(tmp_path / "f.csv", [(attn, "FETCH_SIZE", 100.0), (attn, "FETCH_SIZE", 300.0)])
    _counter_csv(tmp_path / "w.csv", [(attn, "WRITE_SIZE", 50.0)])
    _counter_csv(tmp_path / "cf.csv", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 512.0)])
    _counter_csv(tmp_path / "cw.csv", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024.0)])
    md = profsum.traffic_md(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                            str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"), 1024 * 1024,
                            "wl", 0.1, 8.0, "cmd")
    prof = tmp_path / "p.md"
    prof.write_text(md)
    r = profsum.read_traffic(str(prof), "wl", 0.1, 8.0)
    # fetch: mean 200 KiB x (1 MiB / 512 KiB) = 400 KiB; write: 50 KiB x 1
    assert r["read_bytes"] == 400 * 1024 and r["write_bytes"] == 50 * 1024
    assert profsum.read_traffic(str(prof), "wl", 0.2, 8.0) is None
    assert profsum.read_traffic(str(prof), "other", 0.1, 8.0) is None
    stale = md.replace(profsum.attention_source_digest(), "0" * 16)
    prof.write_text(stale)
    assert profsum.read_traffic(str(prof), "wl", 0.1, 8.0) is None


def test_committed_profile_parses():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    path = os.path.join(root, "profiles", "attn_kap_llama128k_hbm_traffic.md")
    assert os.path.exists(path)
    with open(path) as f:
        assert any(line.startswith("bench-traffic: ") for line in f)


def test_entry_points_from_kernel_names():
    k = "void cosa::(anonymous namespace)::attn_fwd_kernel<128, 4, {}>(cosa::AttnParams)"
    assert profsum.entry_of(k.format(1)) == "cosa_osk_prefill"
    assert profsum.entry_of(k.format(0)) == "cosa_dense_prefill"
    assert profsum.entry_of(k.format(2)) == "cosa_block_mask_prefill"
    assert profsum.entry_of(k.format("1, 2")) == "cosa_osk_prefill"
    assert profsum.entry_of(k.format("0, 1")) == "cosa_dense_prefill"
    assert profsum.entry_of(k.format("1, 1, 1, 2")) == "cosa_osk_prefill"
    assert profsum.entry_of(k.format("0, 1, 2, 4")) == "cosa_dense_prefill"
    assert profsum.entry_of("void cosa::(anonymous namespace)::kap_select<128, 8, false>(x)") is None


def test_trace_groups_launches_by_grid(tmp_path):
    hdr = ('"Kind","Kernel_Name","Start_Timestamp","End_Timestamp","Workgroup_Size_X",'
           '"Workgroup_Size_Y","Workgroup_Size_Z","Grid_Size_X","Grid_Size_Y","Grid_Size_Z"\n')
    k = "void cosa::(anonymous namespace)::attn_fwd_kernel<128, 4, 1, 1, 1, 2>(cosa::AttnParams)"
    rows = [(k, 0, 2_000_000, 256, 8192), (k, 0, 4_000_000, 256, 8192),
            (k, 0, 500_000, 256, 1024)]
    p = tmp_path / "trace.csv"
    p.write_text(hdr + "".join(f'"KERNEL_DISPATCH","{n}",{a},{b},{w},1,1,{g},1,1\n'
                               for n, a, b, w, g in rows))
    md = profsum.trace_md(str(p), "cmd")
    lines = [l for l in md.splitlines() if l.startswith("| `attn")]
    assert len(lines) == 2
    assert "| 32 | 2 | 3.0000 | 3.0000 | 2.0000 | 4.0000 | 6.000 |" in lines[0]
    assert "| 4 | 1 | 0.5000 |" in lines[1]


def test_traffic_keeps_launch_sizes_apart(tmp_path):
    attn = "void cosa::(anonymous namespace)::attn_fwd_kernel<128, 4, 1, 1, 1, 2>(cosa::AttnParams)"

    def rows(path, counter, vals):
        with open(path, "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(["Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name",
                        "Counter_Value"])
            for name, grid, v in vals:
                w.writerow([name, grid, 256, counter, v])

    # two whole-layer launches (8 workgroups) and two chunk launches (1 workgroup)
    rows(tmp_path / "f.csv", "FETCH_SIZE", [(attn, 2048, 800.0), (attn, 2048, 800.0),
                                            (attn, 256, 100.0), (attn, 256, 100.0)])
    rows(tmp_path / "w.csv", "WRITE_SIZE", [(attn, 2048, 80.0), (attn, 256, 10.0)])
    rows(tmp_path / "cf.csv", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 512, 512.0)])
    rows(tmp_path / "cw.csv", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 512, 1024.0)])
    md = profsum.traffic_md(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                            str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"), 1024 * 1024,
                            "wl", 0.1, 8.0, "cmd")
    prof = tmp_path / "p.md"
    prof.write_text(md)
    r = profsum.read_traffic(str(prof), "wl", 0.1, 8.0)
    assert r["workgroups"] == 8
    assert r["read_bytes"] == 1600 * 1024 and r["write_bytes"] == 80 * 1024


def test_mfma_util_lines_and_readback(tmp_path):
    osk = "void cosa::(anonymous namespace)::attn_fwd_kernel<128, 4, 1, 1, 1, 2>(cosa::AttnParams)"
    dense = "void cosa::(anonymous namespace)::attn_dense_pp_kernel<128>(cosa::AttnParams)"
    kap = "void cosa::(anonymous namespace)::kap_select<128, 8, false, 1>(cosa::KapParams)"
    p = tmp_path / "c.csv"
    with open(p, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name", "Counter_Value"])
        # whole-layer OSK launch (8 workgroups) and a chunk launch (1 workgroup)
        for name, grid, busy, active in [(osk, 2048, 4096.0, 64.0), (osk, 256, 1024.0, 64.0),
                                         (dense, 4096, 6144.0, 64.0), (kap, 256, 512.0, 64.0)]:
            w.writerow([name, grid, 256, "SQ_VALU_MFMA_BUSY_CYCLES", busy])
            w.writerow([name, grid, 256, "GRBM_GUI_ACTIVE", active])
    md = profsum.counters_md(str(p), "cmd", xcds=8, simds=64, workload="wl", budget=0.1, tau=8.0)
    prof = tmp_path / "p.md"
    prof.write_text(md)
    # util = busy / (active / 8 XCDs x 64 SIMDs) = busy / 512
    r = profsum.read_mfma_util(str(prof), "wl", 0.1, 8.0, "cosa_osk_prefill")
    assert r["workgroups"] == 8 and r["mfma_util"] == 8.0
    assert profsum.read_mfma_util(str(prof), "wl", 0.1, 8.0, "cosa_dense_prefill")["mfma_util"] == 12.0
    assert profsum.read_mfma_util(str(prof), "wl", 0.2, 8.0, "cosa_osk_prefill") is None
    assert not any("kap_select" in l for l in md.splitlines() if l.startswith("bench-mfma"))
    prof.write_text(md.replace(profsum.attention_source_digest(), "0" * 16))
    assert profsum.read_mfma_util(str(prof), "wl", 0.1, 8.0, "cosa_osk_prefill") is None
    # without a workload no readback lines are written
    assert "bench-mfma" not in profsum.counters_md(str(p), "cmd")
