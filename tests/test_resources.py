"""Register budget of the shipped kernels, from the compiler's kernel-resource-usage
remarks on the gfx950 device code (causal_attention_flash_amd/resources.py; no GPU).

Occupancy has been the lever that mattered most in these kernels, and it changes
silently when an edit adds a few live registers; these pins catch that.  Spills:
none, except measured cases kept on purpose:
* bwd_dkdv_mfma_kernel<E, 96, 64, 8, *, false>: up to 5 VGPRs, a few scratch
  accesses per query tile; the spill-free alternatives measured slower (32-query
  tiles with 8 waves 154 us, 32-query tiles with 4 waves at one wave per SIMD
  173 us, against 133 us at B=4 H=16 S=2048 D=96, when this kernel spilled 17).
* bwd_dkdv_mfma_kernel<E, 128, 64, 8, *, false, 2> (the dK-only pass at D = 128):
  up to 6 VGPRs, one 4-byte reload per query tile inside the loop; the two
  one-accumulator passes with it measured 2.6-3.5% faster than the one-pass
  kernel at one wave per SIMD.
* fwd_mfma_kernel<E, 128, 1, 4, false, 64, true> (the split-key forward of small
  grids at D = 128): 1 VGPR, stored once before the key loop and reloaded once after
  it; the split form measured 25-30% faster than the unsplit kernel on such grids.
"""
import re

import pytest

from causal_attention_flash_amd import resources

# kernel (short demangled name, regex) -> (max VGPRs spilled, max scratch bytes per lane)
ALLOWED_SPILLS = {
    r"bwd_dkdv_mfma_kernel<(Bf16|F16), 96, 64, 8, (true|false), false, 0>": (5, 24),
    r"bwd_dkdv_mfma_kernel<(Bf16|F16), 128, 64, 8, (true|false), false, 2>": (6, 28),
    r"fwd_mfma_kernel<(Bf16|F16), 128, 1, 4, false, 64, true>": (1, 8),
}

# waves per SIMD the hot kernels must keep
OCCUPANCY = {
    "fwd_mfma_kernel<Bf16, 64, 1, 4, false, 32, false>": 3,
    "fwd_mfma_kernel<Bf16, 64, 1, 4, false, 64, true>": 3,
    "fwd_mfma_kernel<Bf16, 80, 1, 4, false, 64, true>": 2,
    "fwd_mfma_kernel<Bf16, 96, 1, 4, false, 64, true>": 2,
    "fwd_mfma_kernel<Bf16, 128, 1, 4, false, 64, true>": 2,
    "fwd_mfma_kernel<Bf16, 80, 1, 4, false, 32, false>": 2,
    "fwd_mfma_kernel<Bf16, 96, 1, 4, false, 32, false>": 2,
    "fwd_mfma_kernel<Bf16, 128, 1, 4, false, 32, false>": 2,
    "fwd_mfma_kernel<Bf16, 64, 1, 4, true, 64, false>": 2,
    "fwd_mfma_kernel<Bf16, 128, 1, 4, true, 32, false>": 2,
    "bwd_dq_mfma_kernel<Bf16, 64, 64, 4, true>": 3,
    "bwd_dq_mfma_kernel<Bf16, 128, 32, 4, true>": 2,
    "bwd_dkdv_mfma_kernel<Bf16, 64, 64, 8, false, false, 0>": 2,
    "bwd_dkdv_mfma_kernel<Bf16, 128, 64, 8, false, false, 1>": 2,
    "bwd_dkdv_mfma_kernel<Bf16, 128, 64, 8, false, false, 2>": 2,
}


@pytest.fixture(scope="module")
def kernels():
    ks = resources.kernel_resources()
    assert ks, "no kernel-resource-usage remarks parsed"
    return {k["kernel"]: k for k in ks}


def test_every_source_reports(kernels):
    sources = {k["source"] for k in kernels.values()}
    assert {"attn_fwd_mfma.hip", "attn_bwd_mfma.hip", "attn_decode.hip"} <= sources


def test_no_unexpected_spills(kernels):
    bad = []
    for name, k in kernels.items():
        if k["sgpr_spill"]:
            bad.append(f"{name}: {k['sgpr_spill']} SGPRs spilled")
        if not k["vgpr_spill"] and not k["scratch"]:
            continue
        limit = next((v for pat, v in ALLOWED_SPILLS.items() if re.fullmatch(pat, name)), None)
        if limit is None or k["vgpr_spill"] > limit[0] or k["scratch"] > limit[1]:
            bad.append(f"{name}: {k['vgpr_spill']} VGPRs spilled, {k['scratch']} B/lane scratch")
    assert not bad, "\n".join(bad)


@pytest.mark.parametrize("name", sorted(OCCUPANCY))
def test_hot_kernel_occupancy(kernels, name):
    assert name in kernels, f"{name} not found; kernels: {sorted(kernels)[:8]}..."
    assert kernels[name]["occupancy"] == OCCUPANCY[name], kernels[name]


def test_parse_remarks():
    text = "\n".join([
        "a.hip:1:1: remark: Function Name: _Z1kv [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     TotalSGPRs: 12 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     VGPRs: 40 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     Occupancy [waves/SIMD]: 8 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:1:1: remark:     LDS Size [bytes/block]: 1024 [-Rpass-analysis=kernel-resource-usage]",
    ])
    (k,) = resources.parse(text)
    assert (k["name"], k["vgpr"], k["sgpr"], k["occupancy"], k["lds"]) == ("_Z1kv", 40, 12, 8, 1024)
    assert resources.short("void attn::fwd_mfma_kernel<attn::Bf16, 64, 1>(int, float)") == "fwd_mfma_kernel<Bf16, 64, 1>"
