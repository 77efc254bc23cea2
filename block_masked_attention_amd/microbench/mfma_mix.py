"""How fast a gfx950 SIMD issues 32x32x16 bf16 matrix products (MFMA) when
vector (VALU) instructions or LDS reads are mixed in.

Each generated kernel repeats one inline-assembly block: four independent
`v_mfma_f32_32x32x16_bf16` (rotating accumulators), each followed by V vector
instructions (`v_fma_f32`, or the transcendental `v_exp_f32`) on 16
independent registers and L `ds_read_b128` (1 KiB per wave, the 16 bytes of
each lane side by side, conflict-free), the reads waited for at the end of
the same block. One workgroup per CU (it holds 100 KiB of LDS), with 4 waves
(one per SIMD) or 8 (two per SIMD, issuing the same mix). The wave's shader
cycle counter (`s_memtime`) around the loop gives cycles per MFMA per SIMD
(the median over waves); a 32x32x16 bf16 MFMA alone takes 32.

The bdattn kernels issue 3-6 vector instructions per MFMA (with 1 exponential
for every 1-2 of them) and 1.3-2 LDS instructions (rocprof SQ counters), so
these rates bound how busy their matrix cores can be. Usage (on the GPU
machine, from the repository root):

    python -m block_masked_attention_amd.microbench.mfma_mix [--out DIR]

prints one line per (mix, waves per SIMD) and a markdown table.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
import tempfile

VALU_COUNTS = (0, 1, 2, 3, 4, 6, 8, 12, 16)
LDS_COUNTS = (1, 2, 3, 4)
ITERS = 2000
CLOBBER = ",".join(f'"v{i}"' for i in range(128))


def mixes():
    """(vector op, vector instructions per MFMA, LDS reads per MFMA)."""
    out = [(op, v, 0) for op in ("fma", "exp") for v in VALU_COUNTS]
    out += [("fma", v, l) for l in LDS_COUNTS for v in (0, 2)]
    return out


def block(op, v, l):
    """The assembly of one loop iteration: 4 MFMAs, each followed by the mix."""
    lines, vi, li = [], 0, 0
    for m in range(4):
        acc = f"v[{16 * m}:{16 * m + 15}]"
        lines.append(f"v_mfma_f32_32x32x16_bf16 {acc}, v[64:67], v[68:71], {acc}")
        for _ in range(v):
            r = 80 + vi % 16
            lines.append(f"v_fma_f32 v{r}, v{r}, v96, v97" if op == "fma" else f"v_exp_f32 v{r}, v{r}")
            vi += 1
        for _ in range(l):
            d = 100 + 4 * (li % 4)
            lines.append(f"ds_read_b128 v[{d}:{d + 3}], v98")
            li += 1
    if l:
        lines.append("s_waitcnt lgkmcnt(0)")  # the reads complete inside the block
    return "\\n\\t".join(lines)


def source():
    ks, calls = [], []
    for op, v, l in mixes():
        name = f"mix_{op}_{v}_{l}"
        ks.append(f'''
__global__ __launch_bounds__(512) void {name}(unsigned long long* cyc, int iters) {{
  // v96, v97: fma operands; v98: this lane's LDS byte offset (16 * lane, < 1 KiB)
  asm volatile("v_mov_b32 v96, 0x3f7ff000\\n\\tv_mov_b32 v97, 0x3a000000\\n\\t"
               "v_mbcnt_lo_u32_b32 v99, -1, 0\\n\\tv_mbcnt_hi_u32_b32 v99, -1, v99\\n\\t"
               "v_lshlrev_b32 v98, 4, v99\\n\\tv_and_b32 v98, 0x3f0, v98" ::: {CLOBBER});
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int i = 0; i < iters; ++i) asm volatile("{block(op, v, l)}" ::: {CLOBBER}, "memory");
  asm volatile("s_nop 7\\n\\ts_nop 7" ::: "memory");  // the last products drain
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  if ((threadIdx.x & 63) == 0) cyc[blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64] = t1 - t0;
}}''')
        for wps in (1, 2):
            calls.append(f'  run({name}, "{op}", {v}, {l}, {wps});')
    main = f'''
#define CHECK(x) do {{ if ((x) != hipSuccess) {{ printf("HIP error at line %d\\n", __LINE__); exit(1); }} }} while (0)
static unsigned long long* d_cyc;
static std::vector<unsigned long long> h_cyc(256 * 8);
template <class K>
static void run(K k, const char* op, int v, int l, int wps) {{
  const int nblk = 256, thr = 256 * wps, waves = nblk * thr / 64;
  for (int rep = 0; rep < 2; ++rep) {{  // the first launch warms up
    hipLaunchKernelGGL(k, dim3(nblk), dim3(thr), 100 * 1024, 0, d_cyc, {ITERS});
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
  }}
  CHECK(hipMemcpy(h_cyc.data(), d_cyc, sizeof(unsigned long long) * waves, hipMemcpyDeviceToHost));
  std::vector<unsigned long long> c(h_cyc.begin(), h_cyc.begin() + waves);
  std::sort(c.begin(), c.end());
  // each wave issues 4 * iters MFMAs; wps waves share a SIMD
  printf("%s %d %d %d %.2f\\n", op, wps, v, l, double(c[c.size() / 2]) / (4.0 * {ITERS} * wps));
  fflush(stdout);
}}
int main() {{
  CHECK(hipMalloc(&d_cyc, sizeof(unsigned long long) * 256 * 8));
  printf("op waves_per_simd valu_per_mfma lds_per_mfma cycles_per_mfma\\n");
{chr(10).join(calls)}
  CHECK(hipFree(d_cyc));
  return 0;
}}
'''
    head = "#include <hip/hip_runtime.h>\n#include <stdio.h>\n#include <stdlib.h>\n#include <algorithm>\n#include <vector>\n"
    return head + "\n".join(ks) + main


def build(out_dir):
    src = os.path.join(out_dir, "mfma_mix.hip")
    exe = os.path.join(out_dir, "mfma_mix")
    with open(src, "w") as fh:
        fh.write(source())
    hipcc = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    cmd = [hipcc, "-O3", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", src, "-o", exe]
    subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    return exe


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--out", default=None, help="directory for the source and binary (default: a temporary one)")
    ap.add_argument("--build-only", action="store_true")
    args = ap.parse_args()
    out = args.out or tempfile.mkdtemp(prefix="mfma_mix_")
    os.makedirs(out, exist_ok=True)
    exe = build(out)
    if args.build_only:
        print(exe)
        return
    res = subprocess.run([exe], check=True, stdout=subprocess.PIPE, text=True, timeout=300)
    print(res.stdout, end="", flush=True)
    rows = [l.split() for l in res.stdout.splitlines()[1:] if l.strip()]
    print("\n| mix per MFMA | 1 wave per SIMD | 2 waves per SIMD |\n|---|---|---|")
    table = {}
    for op, wps, v, l, c in rows:
        table.setdefault((op, int(v), int(l)), {})[int(wps)] = float(c)
    for (op, v, l), c in table.items():
        what = f"{v} {op}" + (f" + {l} ds_read_b128" if l else "")
        print(f"| {what} | {c.get(1, float('nan')):.1f} | {c.get(2, float('nan')):.1f} |")


if __name__ == "__main__":
    sys.exit(main())
