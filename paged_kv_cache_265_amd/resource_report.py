"""Per-kernel resource report of libpkv's gfx950 code, from the compiler's own output.

Compiles every HIP source of the library the way build.py does, keeping the gfx950
assembly (--save-temps, in a scratch directory), and reads, for each kernel, the
resource lines the compiler writes there: vector and accumulation registers (VGPR,
AGPR), scalar registers, LDS bytes, scratch (spill) bytes and the occupancy (waves
per SIMD) the register and LDS use allow.  It also scans the assembly for a vector
instruction that reads the result of a matrix-core product before 8 wait states have
passed, on the fall-through path and across up to two taken branches (the padding a
4-pass product's result needs on gfx950 before a VALU read), and reports how many it
finds.  Writes a Markdown table to stdout, or to the file given as the argument.

    python paged_kv_cache_265_amd/resource_report.py profiles/kernel_resources.md
"""

import os
import re
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
from paged_kv_cache_265_amd import build as _b  # noqa: E402

KEYS = {"NumVgprs": "vgpr", "NumAgprs": "agpr", "TotalNumSgprs": "sgpr", "ScratchSize": "scratch",
        "Occupancy": "occupancy", "LDSByteSize": "lds"}
kWaitStates = 8


def _assembly(src: str, tmp: str) -> str:
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [_b.HIPCC] + _b.COMMON + lang + ["--save-temps", "-c", os.path.join(_b.CSRC, src), "-o",
                                           os.path.join(tmp, src + ".o")]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=tmp)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stderr[-2000:]}")
    stem = os.path.splitext(src)[0] if src.endswith(".hip") else src
    path = os.path.join(tmp, f"{stem}-hip-amdgcn-amd-amdhsa-{_b.ARCH}.s")
    return open(path).read() if os.path.exists(path) else ""


def _demangle(names):
    r = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True)
    return r.stdout.split("\n") if r.returncode == 0 else list(names)


def _regs(s):
    out = {("v", int(x)) for x in re.findall(r"\bv(\d+)\b", s)}
    out |= {("a", int(x)) for x in re.findall(r"\ba(\d+)\b", s)}
    for k, a, b in re.findall(r"([va])\[(\d+):(\d+)\]", s):
        out |= {(k, r) for r in range(int(a), int(b) + 1)}
    return out


def _dst(s):
    m = re.match(r"\s*\S+\s+([va]\[\d+:\d+\]|[va]\d+)", s)
    return _regs(m.group(1)) if m else set()


def _short_reads(lines, start, end):
    """Vector reads of a matrix-core result after fewer than kWaitStates wait states."""
    labels = {l.split(":")[0]: i for i, l in enumerate(lines[start:end], start) if re.match(r"^\.LBB\w+:", l)}
    found = []

    def walk(j, written, ws, depth, origin):
        while j < end and ws < kWaitStates:
            s = lines[j].strip()
            j += 1
            if not s or s.startswith(";") or s.startswith("."):
                continue
            if s.startswith("s_endpgm"):
                return
            if s.startswith("v_") and not s.startswith("v_mfma") and (_regs(s) & written):
                found.append((origin, s.split()[0], ws))
                return
            if s.startswith("v_mfma") and (_dst(s) & written):
                return
            ws += int(s.split()[1], 0) + 1 if s.startswith("s_nop") else 1
            if s.startswith("s_cbranch") and depth < 2 and s.split()[1] in labels:
                walk(labels[s.split()[1]] + 1, written, ws, depth + 1, origin)
            if s.startswith("s_branch") and s.split()[1] in labels:
                j = labels[s.split()[1]] + 1

    for i in range(start, end):
        if re.match(r"\s+v_mfma\w* [va]", lines[i]):
            walk(i + 1, _dst(lines[i]), 0, 0, i)
    return found


def kernels(asm: str):
    lines = asm.split("\n")
    starts = [(i, l.split(":")[0]) for i, l in enumerate(lines) if re.match(r"^_Z\w+:", l)]
    out = []
    for k, (i, name) in enumerate(starts):
        end = starts[k + 1][0] if k + 1 < len(starts) else len(lines)
        info = {"name": name}
        for l in lines[i:end]:
            m = re.match(r"\s*; (NumVgprs|NumAgprs|TotalNumSgprs|ScratchSize|Occupancy|LDSByteSize): (\d+)", l)
            if m:
                info[KEYS[m.group(1)]] = int(m.group(2))
        info["short_reads"] = len(_short_reads(lines, i, end))
        out.append(info)
    return out


def _hot(name: str) -> bool:
    """Kernels the bf16, head_dim 128, block_size 16 workloads launch, and the untyped ones."""
    if "<" not in name:
        return True
    first = re.search(r"<(?:pkv::\w+<)?(\d+)", name)
    if first and first.group(1) != "2":
        return False
    if "Loop<" in name:
        return bool(re.search(r"Loop<2, 128, (\d+, )?16>", name))
    if name.startswith(("chunked_fa", "mixed_kernel")):
        return "<2, 128, 16>" in name or "128, 16>, 2, 128, 16>" in name
    return True


def report() -> str:
    srcs = [s for s in _b.SOURCES if s.endswith(".hip")]
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=6) as ex:
            asms = list(ex.map(lambda s: _assembly(s, tmp), srcs))
    rows = []
    for src, asm in zip(srcs, asms):
        for k in kernels(asm):
            if "vgpr" in k:  # kernels carry a resource block; device functions do not
                rows.append((src, k))
    names = _demangle([k["name"] for _, k in rows])
    for (src, k), name in zip(rows, names):
        name = re.sub(r"^void ", "", name).replace("pkv::(anonymous namespace)::", "").replace("pkv::", "")
        k["pretty"] = re.sub(r"\((\w+Params(, )?)+(int)?\)$|\(.*\)$", "", name)
    out = ["# Kernel resources (gfx950, from the compiler's assembly)", "",
           "Command (repo root): `python paged_kv_cache_265_amd/resource_report.py profiles/kernel_resources.md`", "",
           "Registers are per lane (AGPRs hold what does not fit in 256 VGPRs, or matrix-core accumulators);",
           "LDS is the static LDS per workgroup; scratch is private (spill or dynamically indexed array) bytes",
           "per lane; occupancy is waves per SIMD as the compiler computes it from registers and LDS.",
           "`short reads`: vector reads of a matrix-core result with fewer than 8 wait states on some path",
           "(fall-through or up to two taken branches) -- 0 means every such read is padded.", "",
           "## Kernels of the bf16 / head_dim 128 / block_size 16 workloads", "",
           "(A template compiled into several sources is listed once, under the first.)", "",
           "| source | kernel | VGPR | AGPR | SGPR | LDS bytes | scratch | occupancy | short reads |",
           "|---|---|---|---|---|---|---|---|---|"]
    seen = set()
    for src, k in rows:
        if _hot(k["pretty"]) and k["pretty"] not in seen:  # the same template in several sources: first one
            seen.add(k["pretty"])
            out.append(f"| {src} | `{k['pretty']}` | {k['vgpr']} | {k.get('agpr', 0)} | {k.get('sgpr', '')} | "
                       f"{k.get('lds', 0)} | {k.get('scratch', 0)} | {k.get('occupancy', '')} | {k['short_reads']} |")
    out += ["", "## Every kernel, by source and template", "",
            "| source | template | instances | VGPR | max AGPR | max LDS | max scratch | occupancy | short reads |",
            "|---|---|---|---|---|---|---|---|---|"]
    groups = {}
    for src, k in rows:
        groups.setdefault((src, k["pretty"].split("<")[0]), []).append(k)
    for (src, fam), ks in groups.items():
        v = [k["vgpr"] for k in ks]
        occ = [k.get("occupancy", 0) for k in ks]
        out.append(f"| {src} | `{fam}` | {len(ks)} | {min(v)}-{max(v)} | {max(k.get('agpr', 0) for k in ks)} | "
                   f"{max(k.get('lds', 0) for k in ks)} | {max(k.get('scratch', 0) for k in ks)} | "
                   f"{min(occ)}-{max(occ)} | {sum(k['short_reads'] for k in ks)} |")
    total_short = sum(k["short_reads"] for _, k in rows)
    out += ["", f"Kernels: {len(rows)}; short matrix-core result reads in total: {total_short}."]
    return "\n".join(out) + "\n"


if __name__ == "__main__":
    text = report()
    if len(sys.argv) > 1:
        with open(sys.argv[1], "w") as f:
            f.write(text)
    else:
        sys.stdout.write(text)
