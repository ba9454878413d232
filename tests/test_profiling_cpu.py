"""The profiler summaries' arithmetic on synthetic counter files: request
counts to bytes, the known-size kernels' factors, and the digest rule that
voids a traffic summary once the kernel sources change."""
import csv
import os

import pytest

from online_structured_ffn_amd import profiling as prof

PROBE = prof.PROBE_BYTES


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "pmc_counter_collection.csv"), "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name",
                                            "Counter_Value"])
        wr.writeheader()
        for disp, kern, grid, counters in rows:
            for name, val in counters.items():
                # two L2 instances per counter, as the per-instance rows of a real run
                wr.writerow({"Dispatch_Id": disp, "Kernel_Name": kern, "Grid_Size": grid, "Counter_Name": name,
                             "Counter_Value": val / 2})
                wr.writerow({"Dispatch_Id": disp, "Kernel_Name": kern, "Grid_Size": grid, "Counter_Name": name,
                             "Counter_Value": val / 2})


def test_request_bytes():
    c = {"TCC_EA0_RDREQ_32B_sum": 3, "TCC_EA0_RDREQ_64B_sum": 5, "TCC_EA0_RDREQ_128B_sum": 7}
    assert prof._read_bytes(c) == 32 * 3 + 64 * 5 + 128 * 7
    w = {"TCC_EA0_WRREQ_sum": 10, "TCC_EA0_WRREQ_64B_sum": 4}
    assert prof._write_bytes(w) == 64 * 4 + 32 * 6


@pytest.mark.parametrize("probe_scale,fill_scale", [(1.0, 1.0), (0.5, 2.0)])
def test_traffic_summary_calibration_and_digest(tmp_path, monkeypatch, probe_scale, fill_scale):
    rd, wr = str(tmp_path / "rd"), str(tmp_path / "wr")
    probe = "pop::k_read_probe(unsigned char const*, int*)"
    fill = "void at::native::vectorized_elementwise_kernel<16, at::native::FillFunctor<unsigned char>>(int)"
    kern = "void pop::k_pop_linked<pop::bf16s, 1, false>(args)"
    n128 = PROBE * probe_scale / 128
    _write_counters(rd, [
        (1, probe, 262144, {"TCC_EA0_RDREQ_sum": n128, "TCC_EA0_RDREQ_128B_sum": n128}),
        (2, probe, 262144, {"TCC_EA0_RDREQ_sum": n128, "TCC_EA0_RDREQ_128B_sum": n128}),
        # two dispatches of the kernel: 1000 and 3000 128-byte requests plus 10 of 32 bytes
        (3, kern, 131072, {"TCC_EA0_RDREQ_128B_sum": 1000, "TCC_EA0_RDREQ_32B_sum": 10}),
        (4, kern, 131072, {"TCC_EA0_RDREQ_128B_sum": 3000, "TCC_EA0_RDREQ_32B_sum": 10}),
    ])
    n64 = PROBE * fill_scale / 64
    _write_counters(wr, [
        (1, fill, PROBE // 16, {"TCC_EA0_WRREQ_sum": n64, "TCC_EA0_WRREQ_64B_sum": n64}),
        (3, kern, 131072, {"TCC_EA0_WRREQ_sum": 50, "TCC_EA0_WRREQ_64B_sum": 20}),
        (4, kern, 131072, {"TCC_EA0_WRREQ_sum": 50, "TCC_EA0_WRREQ_64B_sum": 20}),
    ])
    out = str(tmp_path / "traffic.md")
    monkeypatch.setattr(prof, "_algorithmic_reads", lambda *a, **k: {})
    prof.traffic(rd, wr, None, out)
    rb, wb = prof.traffic_bytes("pop::k_pop_linked<pop::bf16s, 1, false>", out)
    assert rb == round((2000 * 128 + 320) / probe_scale)
    assert wb == round((20 * 64 + 30 * 32) / fill_scale)
    # a summary taken on other kernel sources is void
    text = open(out).read().replace(f"digest={prof.source_digest()}", "digest=0000000000000000")
    open(out, "w").write(text)
    assert prof.traffic_bytes("pop::k_pop_linked<pop::bf16s, 1, false>", out) is None


def test_committed_traffic_summary_parses():
    """Every machine-readable line of the committed summaries parses."""
    for name in ("ffn_kernels_llama2_7b_b1_hbm_traffic.md", "layer_kernels_llama2_7b_layer_b1_hbm_traffic.md"):
        path = os.path.join(prof.ROOT, "profiles", name)
        if not os.path.exists(path):
            continue
        lines = [l.strip() for l in open(path) if l.startswith("kernel=")]
        assert all(prof._LINE.match(l) for l in lines), name
