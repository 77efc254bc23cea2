"""How many bf16 matrix products per second the whole chip sustains, and at
what shader clock, when every SIMD of every CU issues them back to back: the
power-limited rate that bounds any kernel built from these products.

One workgroup of 8 waves per CU (two per SIMD; it holds 100 KiB of LDS, so no
second one fits). Each wave repeats one inline-assembly block of four
independent `v_mfma_f32_32x32x16_bf16`, which alternate between two A and two
B operand sets (A0 B0, A1 B1, A0 B1, A1 B0), each product followed by V
`v_fma_f32` on independent registers and L `ds_read_b128` (1 KiB per wave). The operands come from a buffer filled
on the host, either with zeros or with bf16 values drawn from N(0, 0.25) (the
attention inputs' distribution), distinct per wave and lane; the accumulators
start at zero. One launch runs for about half a second; the wall time of the
second launch (HIP events) gives the sustained rate, and every wave reads the
shader cycle counter (`s_memtime`) and the 100 MHz real-time counter
(`s_memrealtime`) around its loop, which give the clock the CUs ran at and the
loops' span (first start to last end).

Usage (on the GPU machine, from the repository root):

    python -m block_masked_attention_amd.microbench.mfma_power [--out DIR]

prints one line per (data, vector instructions and LDS reads per product)
and a markdown table.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
import tempfile

# (vector instructions, LDS reads) after each product
MIXES = ((0, 0), (4, 0), (0, 1), (4, 1))
DATA = ("zeros", "normal")
ITERS = 3_000_000
FLOP_PER_MFMA = 2 * 32 * 32 * 16
CLOBBER = ",".join(f'"v{i}"' for i in range(128))
# operand registers: A0 v[64:67], B0 v[68:71], A1 v[72:75], B1 v[76:79]
PAIRS = (("v[64:67]", "v[68:71]"), ("v[72:75]", "v[76:79]"), ("v[64:67]", "v[76:79]"), ("v[72:75]", "v[68:71]"))


def block(v, l=0):
    """The assembly of one loop iteration: 4 MFMAs over alternating operand
    sets, each followed by v vector instructions and l `ds_read_b128` (1 KiB
    per wave, the lanes' 16 bytes side by side), the reads waited for at the
    end of the block."""
    lines, vi, li = [], 0, 0
    for m, (a, b) in enumerate(PAIRS):
        acc = f"v[{16 * m}:{16 * m + 15}]"
        lines.append(f"v_mfma_f32_32x32x16_bf16 {acc}, {a}, {b}, {acc}")
        for _ in range(v):
            r = 80 + vi % 16
            lines.append(f"v_fma_f32 v{r}, v{r}, v96, v97")
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
    moves = "\\n\\t".join(f"v_mov_b32 v{64 + i}, %{i}" for i in range(16))
    ins = ", ".join(f'"v"(r[{i}])' for i in range(16))
    zero_acc = "\\n\\t".join(f"v_mov_b32 v{i}, 0" for i in range(64))
    for v, l in MIXES:
        name = f"power_{v}_{l}"
        ks.append(f'''
__global__ __launch_bounds__(512) void {name}(const unsigned* ops, unsigned long long* clk, int iters) {{
  // this lane's 16 operand dwords (8 waves per workgroup, 64 lanes per wave)
  const unsigned* o = ops + ((size_t)(blockIdx.x * 8 + threadIdx.x / 64) * 64 + (threadIdx.x & 63)) * 16;
  unsigned r[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = o[i];
  asm volatile("{moves}" :: {ins} : {CLOBBER});
  // v96, v97: fma operands; v98: this lane's LDS byte offset (16 * lane, < 1 KiB)
  asm volatile("{zero_acc}\\n\\tv_mov_b32 v96, 0x3f7ff000\\n\\tv_mov_b32 v97, 0x3a000000\\n\\t"
               "v_mbcnt_lo_u32_b32 v99, -1, 0\\n\\tv_mbcnt_hi_u32_b32 v99, -1, v99\\n\\t"
               "v_lshlrev_b32 v98, 4, v99\\n\\tv_and_b32 v98, 0x3f0, v98" ::: {CLOBBER});
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) asm volatile("{block(v, l)}" ::: {CLOBBER}, "memory");
  asm volatile("s_nop 7\\n\\ts_nop 7" ::: "memory");  // the last products drain
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  const unsigned long long t1 = __builtin_amdgcn_s_memrealtime();
  if ((threadIdx.x & 63) == 0) {{
    unsigned long long* w = clk + 4 * (blockIdx.x * 8 + threadIdx.x / 64);
    w[0] = c0;
    w[1] = c1;
    w[2] = t0;
    w[3] = t1;
  }}
}}''')
        for d in DATA:
            calls.append(f'  run({name}, "{d}", {v}, {l}, cus);')
    main = f'''
#define CHECK(x) do {{ if ((x) != hipSuccess) {{ printf("HIP error at line %d\\n", __LINE__); exit(1); }} }} while (0)
static unsigned* d_ops;
static unsigned long long* d_clk;
static size_t n_ops;

static unsigned short bf16_bits(float x) {{  // round to nearest even
  unsigned u;
  memcpy(&u, &x, 4);
  return (unsigned short)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}}

static void fill(const char* data) {{
  std::vector<unsigned> h(n_ops, 0u);
  if (strcmp(data, "normal") == 0) {{
    std::mt19937 rng(1234);
    std::normal_distribution<float> nd(0.f, 0.5f);
    for (auto& w : h) w = bf16_bits(nd(rng)) | ((unsigned)bf16_bits(nd(rng)) << 16);
  }}
  CHECK(hipMemcpy(d_ops, h.data(), n_ops * 4, hipMemcpyHostToDevice));
}}

template <class K>
static void run(K k, const char* data, int v, int l, int cus) {{
  fill(data);
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  float ms = 0.f;
  for (int rep = 0; rep < 2; ++rep) {{  // the first launch warms up
    CHECK(hipEventRecord(e0, 0));
    hipLaunchKernelGGL(k, dim3(cus), dim3(512), 100 * 1024, 0, d_ops, d_clk, {ITERS});
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1, 0));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipEventElapsedTime(&ms, e0, e1));
  }}
  const int waves = cus * 8;
  std::vector<unsigned long long> c(4 * waves);
  CHECK(hipMemcpy(c.data(), d_clk, sizeof(unsigned long long) * 4 * waves, hipMemcpyDeviceToHost));
  // every wave's loop: shader cycles and real-time ticks (100 MHz); the two
  // waves of a SIMD do not run evenly (the older one issues first and ends
  // its loop early), so the loops' span is taken over all waves
  double cyc = 0.0, ticks = 0.0;
  unsigned long long s0 = ~0ull, s1 = 0, f0 = ~0ull, f1 = 0;
  for (int w = 0; w < waves; ++w) {{
    cyc += double(c[4 * w + 1] - c[4 * w]);
    ticks += double(c[4 * w + 3] - c[4 * w + 2]);
    s0 = std::min(s0, c[4 * w + 2]);
    s1 = std::max(s1, c[4 * w + 2]);
    f0 = std::min(f0, c[4 * w + 3]);
    f1 = std::max(f1, c[4 * w + 3]);
  }}
  const double ghz = cyc / ticks / 10.0, span_ms = (f1 - s0) * 1e-5;
  const double mfma = double(cus) * 8.0 * 4.0 * {ITERS};
  // cycles per product per SIMD: the loops' span at that clock over the
  // 2 waves x 4 x iters products of a SIMD
  printf("%s %d %d %.1f %.3f %.2f %.1f %.1f %.2f %.2f %d\\n", data, v, l, mfma * {FLOP_PER_MFMA} / (ms * 1e-3) / 1e12, ghz,
         ghz * 1e9 * span_ms * 1e-3 / (2.0 * 4.0 * {ITERS}), ms, span_ms, (s1 - s0) * 1e-5, (f1 - f0) * 1e-5, cus);
  fflush(stdout);
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
}}

int main() {{
  int dev = 0, cus = 0;
  CHECK(hipGetDevice(&dev));
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  n_ops = (size_t)cus * 8 * 64 * 16;
  CHECK(hipMalloc(&d_ops, n_ops * 4));
  CHECK(hipMalloc(&d_clk, sizeof(unsigned long long) * 4 * 8 * cus));
  printf("data valu_per_mfma lds_per_mfma tflops shader_ghz cycles_per_mfma ms loop_span_ms start_spread_ms end_spread_ms cus\\n");
{chr(10).join(calls)}
  CHECK(hipFree(d_ops));
  CHECK(hipFree(d_clk));
  return 0;
}}
'''
    head = ("#include <hip/hip_runtime.h>\n#include <stdio.h>\n#include <stdlib.h>\n#include <string.h>\n"
            "#include <algorithm>\n#include <random>\n#include <vector>\n")
    return head + "\n".join(ks) + main


def build(out_dir):
    src = os.path.join(out_dir, "mfma_power.hip")
    exe = os.path.join(out_dir, "mfma_power")
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
    out = args.out or tempfile.mkdtemp(prefix="mfma_power_")
    os.makedirs(out, exist_ok=True)
    exe = build(out)
    if args.build_only:
        print(exe)
        return
    res = subprocess.run([exe], check=True, stdout=subprocess.PIPE, text=True, timeout=120)
    print(res.stdout, end="", flush=True)
    rows = [l.split() for l in res.stdout.splitlines()[1:] if l.strip()]
    print("\n| operands | vector instructions per product | LDS reads (1 KiB) per product | TFLOP/s (wall) "
          "| shader clock (GHz) | cycles per product per SIMD |\n|---|---|---|---|---|---|")
    for data, v, l, tf, ghz, cyc, *_ in rows:
        print(f"| {data} | {v} | {l} | {float(tf):.0f} | {float(ghz):.2f} | {float(cyc):.1f} |")


if __name__ == "__main__":
    sys.exit(main())
