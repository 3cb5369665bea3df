"""bench.py's host-side helpers (no GPU): the stage-kernel keys it gives
rocprofv3 names, and the HBM-traffic record it writes from two counter
files, scaled by a copy kernel of known size."""
import csv
import io
import json
import os
import sys
from contextlib import redirect_stdout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_kernel_keys():
    k = bench.kernel_key
    assert k("_ZN3hla19hla2_forward_kernelIDF16bLi64ELi64ELi64ELb0EEEvNS_9FwdParamsE") == \
        "hla2_forward_kernel"
    # the pipelined forward is stage 3's kernel
    assert k("_ZN3hla24hla2_forward_pipe_kernelIDF16bLi64ELi64ELi64EEEvNS_9FwdParamsE") == \
        "hla2_forward_kernel"
    assert bench.is_stage_kernel("_ZN3hla24hla2_forward_pipe_kernelIDF16bLi64ELi64ELi64EEEvNS_9FwdParamsE")
    assert not bench.is_stage_kernel("__amd_rocclr_copyBuffer")
    assert k("void hla::up_sweep_kernel<true, 64, 64, 256>(hla::FwdParams, int)") == "up_sweep_kernel"
    assert k("_ZN3hla17la_forward_kernelIDF16bLi64ELi64ELb0ELb1EEEvNS_8LaParamsE") == \
        "la_forward_kernel_dual"
    assert k("_ZN3hla17la_summary_kernelIDF16bLi64ELi64ELb1ELb0EEEvNS_8LaParamsE") == \
        "la_summary_kernel_sym"
    assert k("void hla::la_forward_kernel<float, 64, 32, true, false>(hla::LaParams)") == \
        "la_forward_kernel_sym_f32"
    assert k("void hla::la_forward_kernel<float, 64, 32, false, false>(hla::LaParams)") == \
        "la_forward_kernel_f32"
    # stage-3 forms that also write their first pass's rows (last template flag)
    assert k("_ZN3hla24hla2_forward_pipe_kernelIDF16bLi64ELi64ELi64ELb1EEEvNS_9FwdParamsE") == \
        "hla2_forward_z_kernel"
    assert k("_ZN3hla24hla2_forward_pipe_kernelIDF16bLi64ELi64ELi64ELb0EEEvNS_9FwdParamsE") == \
        "hla2_forward_kernel"
    assert k("_ZN3hla19hla2_forward_kernelIDF16bLi128ELi128ELi64ELb1ELb0EEEvNS_9FwdParamsE") == \
        "hla2_forward_kernel"
    assert k("_ZN3hla19hla2_forward_kernelIDF16bLi128ELi128ELi64ELb1ELb1EEEvNS_9FwdParamsE") == \
        "hla2_forward_z_kernel"
    assert k("void hla::ahla_forward_kernel<__bf16, 64, 64, 64, false, true>(hla::FwdParams)") == \
        "ahla_forward_z_kernel"


def test_la_kernel_filter():
    assert bench.is_la_kernel("_ZN3hla17la_forward_kernelIDF16bLi64ELi64ELb0ELb0EEEvNS_8LaParamsE")
    assert bench.is_la_kernel("void hla::la_summary_kernel<float, 64, 32, true, false>(hla::LaParams)")
    assert not bench.is_la_kernel("_ZN3hla23ahla_step_sliced_kernelIDF16bLi64ELi64ELi256EEEvNS_10StepParamsE")
    assert not bench.is_la_kernel("_ZN3hla19ahla_forward_kernelIDF16bLi64ELi64ELi64EEEvNS_9FwdParamsE")
    assert not bench.is_la_kernel("_ZN3hla19hla2_forward_kernelIDF16bLi64ELi64ELi64ELb0EEEvNS_9FwdParamsE")


def _csv(path, counter, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=cols)
        w.writeheader()
        for disp, name, val in rows:
            # two partial rows per dispatch (as per-XCD values are): summed
            for part in (0.25, 0.75):
                w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter,
                            "Counter_Value": val * part})


def test_counters_summary(tmp_path):
    neg = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>"
    fwd = "_ZN3hla19hla2_forward_kernelIDF16bLi64ELi64ELi64ELb0EEEvNS_9FwdParamsE"
    f, w = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # the copy moves 256 MiB each way; its fetch counter reads half of that
    _csv(f, "FETCH_SIZE", [(1, neg, 131072.0), (2, fwd, 1000.0), (3, fwd, 3000.0)])
    _csv(w, "WRITE_SIZE", [(1, neg, 262144.0), (2, fwd, 500.0), (3, fwd, 500.0)])
    out = io.StringIO()
    with redirect_stdout(out):
        bench.counters_summary(str(f), str(w))
    rec = json.loads(out.getvalue())
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["source_hash"] == bench.kernel_source_hash()
    ent = rec["hla2_forward_kernel"]
    assert ent["FETCH_SIZE_KiB"] == 2000.0 and ent["WRITE_SIZE_KiB"] == 500.0
    assert ent["fetch_bytes"] == 2000 * 1024 * 2 and ent["write_bytes"] == 500 * 1024
    assert ent["hbm_bytes_per_launch"] == 2000 * 1024 * 2 + 500 * 1024


def test_stored_traffic_follows_the_source_hash():
    """The committed record is used only while it matches the kernel sources."""
    path = os.path.join(ROOT, "profiles", "hla2_forward_counters.json")
    rec = json.load(open(path))
    got = bench.stored_traffic("hla2_forward_kernel")
    if rec["source_hash"] == bench.kernel_source_hash():
        assert got == rec["hla2_forward_kernel"]["hbm_bytes_per_launch"]
    else:
        assert got is None
