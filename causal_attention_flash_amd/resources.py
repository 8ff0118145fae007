"""Registers, scratch, LDS and occupancy of every kernel in the library, from the
compiler's kernel-resource-usage remarks on the gfx950 device code (no GPU needed).

    python -m causal_attention_flash_amd.resources      # markdown table on stdout

Occupancy (waves per SIMD) is what sets how much of one wave's latency the others
hide; in these kernels it has been the main lever (a variant that fit one more wave
per SIMD ran 10-25% faster).  tests/test_resources.py pins the occupancy of the hot
kernels and that nothing spills beyond two documented, measured exceptions.
"""
from __future__ import annotations

import concurrent.futures
import os
import re
import shutil
import subprocess

from causal_attention_flash_amd import build

_FIELDS = {
    "TotalSGPRs": "sgpr",
    "VGPRs": "vgpr",
    "AGPRs": "agpr",
    "ScratchSize [bytes/lane]": "scratch",
    "Occupancy [waves/SIMD]": "occupancy",
    "SGPRs Spill": "sgpr_spill",
    "VGPRs Spill": "vgpr_spill",
    "LDS Size [bytes/block]": "lds",
}
_LINE = re.compile(r"remark:\s+(.*?):\s+(\S+)\s+\[-Rpass-analysis=kernel-resource-usage\]")
_NAME = re.compile(r"remark: Function Name: (\S+)")


def remarks(src: str) -> str:
    """The kernel-resource-usage remarks of one source's device code."""
    cmd = [build.hipcc(), *build.CFLAGS, "--cuda-device-only", "-S", "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage", src]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return r.stderr


def parse(text: str) -> list:
    """One dict per kernel: name (mangled) and the integer fields of _FIELDS."""
    out, cur = [], None
    for line in text.splitlines():
        m = _NAME.search(line)
        if m:
            cur = {"name": m.group(1)}
            out.append(cur)
            continue
        m = _LINE.search(line)
        if m and cur is not None and m.group(1) in _FIELDS:
            v = m.group(2)
            cur[_FIELDS[m.group(1)]] = int(v) if v.isdigit() else v
    return [k for k in out if "vgpr" in k]


def demangle(names: list) -> list:
    tool = shutil.which("c++filt") or shutil.which("llvm-cxxfilt", path="/opt/rocm/llvm/bin")
    if not tool:
        return list(names)
    r = subprocess.run([tool], input="\n".join(names), capture_output=True, text=True)
    out = r.stdout.splitlines()
    return out if len(out) == len(names) else list(names)


def short(demangled: str) -> str:
    """'void attn::fwd_mfma_kernel<attn::Bf16, 64, ...>(args)' -> 'fwd_mfma_kernel<Bf16, 64, ...>'."""
    m = re.match(r"(?:void )?attn::(\w+)(<.*?>)?\(", demangled)
    if not m:
        return demangled
    return m.group(1) + (m.group(2) or "").replace("attn::", "")


def kernel_resources() -> list:
    """Every kernel of every source under csrc/, with its source file and short name."""
    srcs = build.sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        texts = list(ex.map(remarks, srcs))
    ks = []
    for src, text in zip(srcs, texts):
        for k in parse(text):
            k["source"] = os.path.basename(src)
            ks.append(k)
    for k, d in zip(ks, demangle([k["name"] for k in ks])):
        k["kernel"] = short(d)
    return ks


def table(ks: list) -> str:
    rows = ["| source | kernel | VGPR | AGPR | SGPR | scratch (B/lane) | VGPR / SGPR spills | LDS (B) | waves/SIMD |",
            "|---|---|---|---|---|---|---|---|---|"]
    for k in ks:
        rows.append(f"| {k['source']} | `{k['kernel']}` | {k['vgpr']} | {k['agpr']} | {k['sgpr']} | {k['scratch']} | "
                    f"{k['vgpr_spill']} / {k['sgpr_spill']} | {k['lds']} | {k['occupancy']} |")
    return "\n".join(rows)


if __name__ == "__main__":
    print(table(kernel_resources()))
