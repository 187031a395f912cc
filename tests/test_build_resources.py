"""The hot kernels keep their register budget.

The build keeps the compiler's per-kernel resource report beside the objects
(transformer_attention_02_amd/_build/<source>.resources.txt). A kernel whose
registers spill still computes the same values, so the parity tests cannot see
it, but it runs much slower (a 4-wave prefill instance that spilled 200 vector
registers ran 1.3-2.1 times slower). These checks read the report of the last
build: no vector-register spills in the matrix-core prefill and decode kernels,
and the occupancy each is laid out for. Skipped where no build report exists.
"""
import pytest

from transformer_attention_02_amd.build import resource_report

# source: (kernel name, waves per SIMD the kernel is laid out for)
HOT = {
    "prefill_mfma.hip": ("prefill_mfma_kernel", 2),
    "decode.hip": ("decode_split_mfma_kernel", 2),
    "decode_latent.hip": ("latent_split_kernel", 1),
}


def expected_occupancy(src, kernel):
    # the wave-split prefill instances (last template argument true) hold all
    # 160 KiB of LDS for one 4-wave workgroup: one wave per SIMD
    if src == "prefill_mfma.hip" and "Lb1EEEv" in kernel:
        return 1
    return HOT[src][1]


@pytest.mark.parametrize("src", sorted(HOT))
def test_hot_kernels_keep_their_registers(src):
    rep = resource_report(src)
    if not rep:
        pytest.skip("no resource report: the library was not built in this tree")
    name = HOT[src][0]
    kernels = {k: v for k, v in rep.items() if name in k}
    assert kernels, f"no {name} instance in the report of {src}"
    for k, v in kernels.items():
        assert int(v["VGPRs Spill"]) == 0, f"{k}: {v['VGPRs Spill']} vector registers spilled"
        assert int(v["SGPRs Spill"]) <= 4, f"{k}: {v['SGPRs Spill']} scalar registers spilled"
        want = expected_occupancy(src, k)
        assert int(v["Occupancy [waves/SIMD]"]) >= want, f"{k}: occupancy {v['Occupancy [waves/SIMD]']} < {want}"


def test_report_parser_reads_the_compiler_remarks(tmp_path, monkeypatch):
    """The parser turns the remark lines into per-kernel fields."""
    import transformer_attention_02_amd.build as b

    (tmp_path / "_build").mkdir()
    (tmp_path / "_build" / "x.resources.txt").write_text(
        "x.hip:1:1: remark: Function Name: k1 [-Rpass-analysis=kernel-resource-usage]\n"
        "x.hip:1:1: remark:     VGPRs: 120 [-Rpass-analysis=kernel-resource-usage]\n"
        "x.hip:1:1: remark:     VGPRs Spill: 3 [-Rpass-analysis=kernel-resource-usage]\n"
        "x.hip:9:1: remark: Function Name: k2 [-Rpass-analysis=kernel-resource-usage]\n"
        "x.hip:9:1: remark:     Occupancy [waves/SIMD]: 2 [-Rpass-analysis=kernel-resource-usage]\n")
    monkeypatch.setattr(b, "PKG", str(tmp_path))
    rep = b.resource_report("x.hip")
    assert rep == {"k1": {"VGPRs": "120", "VGPRs Spill": "3"}, "k2": {"Occupancy [waves/SIMD]": "2"}}
