"""CPU checks of the benchmark's own arithmetic and parsers, and of the
seeded input generators: the byte and flop counts the roofline divides by,
the counter-summary and trace-summary parsers, and input determinism."""
import csv
import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads as wl  # noqa: E402


def test_decode_bytes_by_hand():
    # 2 sequences of 3 and 17 tokens, 4 q / 2 kv heads, D 8, BS 16, bf16 K/V and q
    lens = [3, 17]
    kv = (3 + 17) * 2 * 8 * 2 * 2  # tokens * Hkv * D * (K and V) * 2 bytes
    q = 2 * 4 * 8 * 2
    out = 2 * 4 * 8 * 4
    tables = (1 + 2) * 4  # ceil(3/16) + ceil(17/16) entries
    assert bench.decode_bytes(lens, 4, 2, 8, 16) == kv + q + out + tables + 2 * 4


def test_prefill_flops_brute_force():
    ctx, ql, hq, d = [10, 7, 33], [4, 7, 1], 3, 5
    brute = 0
    for c, q in zip(ctx, ql):
        for i in range(q):
            keys = c - q + i + 1  # row i sees keys 0 .. its position
            brute += 4 * hq * d * keys
    assert bench.prefill_flops(ctx, ql, hq, d) == brute


def _write_counters(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (kern, val) in enumerate(rows):
            w.writerow([i, kern, counter, val])


def test_pmc_summary_scales_by_the_calibration_copy(tmp_path):
    dec = "void pa::(anonymous namespace)::decode_mfma_kernel<128, 16, true>(pa::DecodeParams)"
    cop = "pa::(anonymous namespace)::copy_blocks_kernel(char*, char*, int const*, int, long, int)"
    block_bytes = 32 * 16 * 128 * 2
    expect = bench.CALIB_PAIRS * 2 * block_bytes  # bytes the copy reads (and writes)
    f, w = tmp_path / "f", tmp_path / "w"
    f.mkdir()
    w.mkdir()
    # a counter that reports half of the true bytes, and one that is exact
    _write_counters(f / "x_counter_collection.csv", "FETCH_SIZE",
                    [(dec, 1000.0), (dec, 1200.0), (cop, expect / 2048)])
    _write_counters(w / "x_counter_collection.csv", "WRITE_SIZE",
                    [(dec, 10.0), (dec, 30.0), (cop, expect / 1024)])
    s = bench.pmc_summary(str(f), str(w), block_bytes)
    assert s["FETCH_SIZE"]["scale"] == pytest.approx(2.0)
    assert s["WRITE_SIZE"]["scale"] == pytest.approx(1.0)
    assert s["hbm_bytes_per_launch"] == pytest.approx(1100 * 1024 * 2 + 20 * 1024)


def test_trace_summary_groups_by_marked_workload(tmp_path):
    rows = [("spin_kernel", 0, 1), ("void pa::(anonymous namespace)::decode_mfma_kernel<128, 16, "
                                    "true>(pa::DecodeParams)", 10, 30),
            ("pa::(anonymous namespace)::decode_reduce_kernel(pa::DecodeParams)", 31, 35),
            ("spin_kernel", 40, 41),
            ("void pa::(anonymous namespace)::decode_mfma_kernel<128, 16, true>(pa::DecodeParams)",
             50, 90)]
    with open(tmp_path / "t_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X",
                    "Workgroup_Size_X"])
        for name, a, b in rows:
            w.writerow([name, a * 1000, b * 1000, 6400, 64])
    text = bench.trace_summary(str(tmp_path))
    lines = [ln for ln in text.splitlines() if "decode_mfma" in ln]
    assert len(lines) == 2  # one per marked workload
    assert bench.PHASES[0] in lines[0] and "| 20.0 |" in lines[0]
    assert bench.PHASES[1] in lines[1] and "| 40.0 |" in lines[1]


def test_inputs_are_deterministic_and_poisoned():
    sh = wl.DecodeShape("t", 3, 4, 2, 64, 16, 0, "bf16", 123)
    a = wl.make_decode_case(sh, "cpu", lengths=[5, 16, 40], num_blocks=12)
    b = wl.make_decode_case(sh, "cpu", lengths=[5, 16, 40], num_blocks=12)
    assert (a.tables == b.tables).all() and (a.perm == b.perm).all()
    assert torch.equal(a.q, b.q)
    assert torch.equal(a.k_pool.view(torch.int16), b.k_pool.view(torch.int16))
    # rows past a sequence's length in its last block, and unused blocks, are NaN
    blk = int(a.tables[0][0])
    assert torch.isnan(a.k_pool[blk, :, 5:, :].float()).all()
    assert torch.isfinite(a.k_pool[blk, :, :5, :].float()).all()
    used = set(int(a.tables[s][j]) for s, L in enumerate([5, 16, 40])
               for j in range(wl.blocks_needed(L, 16)))
    unused = [x for x in range(12) if x not in used]
    assert unused and torch.isnan(a.k_pool[unused].float()).all()


def test_length_recipes():
    rng = np.random.default_rng(wl.MHA_7B.seed)
    lens = wl.draw_lengths(wl.MHA_7B, rng)
    assert lens.min() >= 128 and lens.max() <= 4096 and len(lens) == 64
    rng = np.random.default_rng(wl.GQA.seed)
    g = wl.draw_lengths(wl.GQA, rng)
    assert g.min() >= 16 and g.max() <= 8192 and len(g) == 128
    plan = wl.prefix_plan()
    assert all(2049 <= x <= 2063 for x in plan.shared_lens)
    assert plan.tail_lens.min() >= 1 and plan.tail_lens.max() <= 512


def test_kernel_names_and_spread():
    # demangled libpa names, the tracer's mangled bf16 instantiation, others skipped
    assert bench.kernel_short_name(
        "void pa::(anonymous namespace)::decode_reduce_kernel(pa::DecodeParams)") == \
        "decode_reduce_kernel"
    assert bench.kernel_short_name(
        "_ZN2pa12_GLOBAL__N_122cache_write_fp8_kernelIDF16bEEvPKT_S4_PhS5_PKliiiiiff") == \
        "cache_write_fp8_kernel<__bf16>"
    assert bench.kernel_short_name("at::native::vectorized_elementwise_kernel<4>") is None
    s = bench.spread([0.001 * i for i in range(1, 21)])  # 1 .. 20 us
    assert s["p10_us"] == pytest.approx(3.0) and s["p90_us"] == pytest.approx(19.0)


def test_host_threads_is_bounded():
    assert 1 <= bench.host_threads() <= 16


def test_prefill_counter_summary_per_run_and_xcc(tmp_path):
    """Counters of two runs with overlapping dispatch ids stay apart; the
    clock counter (summed over the 8 XCCs in the csv) is divided back; the
    shares follow rocprof's MfmaUtil and VALUBusy definitions."""
    bf16 = "void pa::(anonymous namespace)::prefill_kernel<128, 128, false>(pa::PrefillParams)"
    fp8 = "_ZN2pa12_GLOBAL__N_114prefill_kernelILi128ELi128ELb1EEEvNS_13PrefillParamsE"
    cyc = 400_000.0  # per XCC
    runs = {
        "a": [(1, bf16, "GRBM_GUI_ACTIVE", 8 * cyc),
              (1, bf16, "SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * cyc * bench.NUM_SIMDS),
              (2, fp8, "GRBM_GUI_ACTIVE", 8 * cyc),
              (2, fp8, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * cyc * bench.NUM_SIMDS),
              (3, "other_kernel", "GRBM_GUI_ACTIVE", 1.0)],
        "b": [(1, bf16, "GRBM_GUI_ACTIVE", 8 * cyc),
              (1, bf16, "SQ_ACTIVE_INST_VALU", 0.75 * cyc * bench.NUM_CUS)],
    }
    for name, rows in runs.items():
        os.makedirs(tmp_path / name)
        with open(tmp_path / name / f"{name}_counter_collection.csv", "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writerows(rows)
    text = bench.prefill_counter_summary([str(tmp_path / "a"), str(tmp_path / "b")])
    assert "bf16: 4e+05 GPU cycles" in text
    assert "bf16: matrix core busy 25.0%" in text
    assert "bf16: vector ALU busy 75.0%" in text
    assert "fp8: matrix core busy 50.0%" in text
    assert "other_kernel" not in text


def test_decode_counter_summary_splits_workloads_and_scales(tmp_path):
    """Counter rows of a --decode-only run: dispatches are attributed to the
    workload of the last spin-kernel marker before them; FETCH_SIZE and
    WRITE_SIZE are scaled by the calibration copy's reading."""
    import json
    dec = "void pa::(anonymous namespace)::decode_mfma_kernel<128, 16, true>(pa::DecodeParams)"
    red = "pa::(anonymous namespace)::decode_reduce_kernel(pa::DecodeParams)"
    cop = "pa::(anonymous namespace)::copy_blocks_kernel(char*, char*, int const*, int, long, int)"
    expect = 1 << 30
    meta = [{"phase": p, "algorithmic_bytes": 1000 * 1024, "calls": 2}
            for p in bench.DECODE_PHASES if p != bench.CAL_PHASE]
    meta.append({"phase": bench.CAL_PHASE, "bytes_read": expect, "calls": 1})
    jf = tmp_path / "d.json"
    jf.write_text(json.dumps({"decode_only": meta}))
    seq = [("spin_kernel", {}), (dec, {"FETCH_SIZE": 400.0, "WRITE_SIZE": 3.0}),
           (red, {"FETCH_SIZE": 10.0, "WRITE_SIZE": 2.0}),
           (dec, {"FETCH_SIZE": 600.0, "WRITE_SIZE": 5.0}),
           (red, {"FETCH_SIZE": 10.0, "WRITE_SIZE": 2.0})]
    cal_at = bench.DECODE_PHASES.index(bench.CAL_PHASE)
    for _ in range(cal_at - 1):  # the workloads before the calibration: no dispatches
        seq.append(("spin_kernel", {}))
    seq += [("spin_kernel", {}), (cop, {"FETCH_SIZE": expect / 2048, "WRITE_SIZE": expect / 1024})]
    d = tmp_path / "run"
    d.mkdir()
    with open(d / "x_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (k, cs) in enumerate(seq):
            for c, v in (cs or {"SQ_WAVES": 1.0}).items():
                w.writerow([i + 1, k, c, v])
    text, summary = bench.decode_counter_summary(str(jf), [str(d)])
    head = summary[bench.DECODE_PHASES[0]]
    # reads: (mean 500 + 10) KiB x scale 2; writes: (4 + 2) KiB x scale 1
    assert head["read"] == pytest.approx(510 * 1024 * 2)
    assert head["write"] == pytest.approx(6 * 1024)
    assert head["algorithmic"] == 1000 * 1024
    assert bench.DECODE_PHASES[1] not in summary
    assert "scale 2.0000" in text
