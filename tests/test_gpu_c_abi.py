"""The C ABI end to end from C: a plain C program (no Python, no torch) allocates device memory
with the HIP runtime, binds a cache, runs a small bf16 workload's schedule through
dita_set_block_policy / dita_attn_step and writes out, lse and the per-step block counts to a
file; the outputs are then held to the fp64 oracle like the binding's runs."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import gpu_helpers as gh
from gpu_helpers import compare, log
from workloads import Policy, custom_config
from workloads import configs as wcfg

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_SOURCE = r'''
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>
#include "dita.h"
#define CK(x) do { int s_ = (x); if (s_) { fprintf(stderr, "%s -> %d: %s\n", #x, s_, dita_last_error()); return 1; } } while (0)
#define HK(x) do { if ((x) != hipSuccess) { fprintf(stderr, "%s failed\n", #x); return 2; } } while (0)
/* argv: in out B H T gh gw P D S ; input file: S x 3 x [B,H,N,D] bf16 bits */
int main(int argc, char** argv) {
  if (argc != 11) return 3;
  dita_geometry g; memset(&g, 0, sizeof g);
  g.batch = atoi(argv[3]); g.heads = atoi(argv[4]); g.frames = atoi(argv[5]);
  g.grid_h = atoi(argv[6]); g.grid_w = atoi(argv[7]); g.num_partitions = atoi(argv[8]);
  g.head_dim = atoi(argv[9]); g.tokens = g.frames * g.grid_h * g.grid_w;
  g.qkv_dtype = DITA_BF16; g.cache_o_dtype = DITA_BF16;
  const int S = atoi(argv[10]);
  const size_t n = (size_t)g.batch * g.heads * g.tokens * g.head_dim;
  const size_t nl = (size_t)g.batch * g.heads * g.tokens;
  FILE* fi = fopen(argv[1], "rb"); FILE* fo = fopen(argv[2], "wb");
  if (!fi || !fo) return 4;
  uint16_t* h = malloc(n * 2); float* ho = malloc(n * 4); float* hl = malloc(nl * 4);
  size_t bytes = 0;
  CK(dita_cache_required_bytes(&g, NULL, &bytes));
  void *buf, *q, *k, *v; float *out, *lse;
  HK(hipMalloc(&buf, bytes)); HK(hipMalloc(&q, n * 2)); HK(hipMalloc(&k, n * 2)); HK(hipMalloc(&v, n * 2));
  HK(hipMalloc((void**)&out, n * 4)); HK(hipMalloc((void**)&lse, nl * 4));
  dita_cache* c = NULL;
  CK(dita_cache_alloc(&g, NULL, buf, bytes, &c));
  for (int s = 0; s < S; ++s) {
    void* dst[3] = {q, k, v};
    for (int t = 0; t < 3; ++t) {
      if (fread(h, 2, n, fi) != n) return 5;
      HK(hipMemcpy(dst[t], h, n * 2, hipMemcpyHostToDevice));
    }
    dita_block_policy p; memset(&p, 0, sizeof p);
    p.kind = DITA_POLICY_FRAME_THRESHOLD; p.max_fresh_frame_dist = 1; p.anchor = (s == 0);
    CK(dita_set_block_policy(c, &p));
    int32_t counts[3];
    CK(dita_get_block_plan(c, NULL, NULL, NULL, NULL, NULL, counts));
    CK(dita_attn_step(c, q, k, v, out, lse, NULL));
    HK(hipDeviceSynchronize());
    HK(hipMemcpy(ho, out, n * 4, hipMemcpyDeviceToHost));
    HK(hipMemcpy(hl, lse, nl * 4, hipMemcpyDeviceToHost));
    fwrite(counts, 4, 3, fo); fwrite(ho, 4, n, fo); fwrite(hl, 4, nl, fo);
  }
  dita_step_stats st;
  CK(dita_get_stats(c, &st));
  CK(dita_cache_free(c));
  fclose(fi); fclose(fo);
  printf("steps %lld fresh %llu %llu reused %llu %llu\n", (long long)st.steps_done,
         (unsigned long long)st.device_fresh_blocks, (unsigned long long)st.host_fresh_blocks,
         (unsigned long long)st.device_reuse_blocks, (unsigned long long)st.host_reuse_blocks);
  return 0;
}
'''


def test_c_program_runs_the_schedule(tmp_path):
    import oracle
    import partial_state_reuse_amd as dita
    from oracle.policy import active_mask, partition_offsets
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    B, H, T, GH, GW, P, D, S = 1, 2, 3, 8, 10, 5, 64, 3
    sched = wcfg.AnchorThen(Policy(kind=wcfg.FRAME_THRESHOLD, max_fresh_frame_dist=1))
    cfg = custom_config(name="c-abi", idx=88, batch=B, heads=H, head_dim=D, frames=T, grid_h=GH,
                        grid_w=GW, num_partitions=P, steps=S, qkv_dtype="bf16",
                        cache_dtype="bf16", schedule=sched)
    N = cfg.tokens
    heads = [(b, h) for b in range(B) for h in range(H)]
    bits = np.zeros((S, 3, B, H, N, D), np.uint16)
    kept = {}
    for b, h, st in gh._iter_heads(cfg, S, heads):
        for s in range(S):
            for t in range(3):
                bits[s, t, b, h] = st[s][t]
        kept[(b, h)] = [tuple(gh._as_f32(cfg, x) for x in s_) for s_ in st]
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    bits.tofile(fin)
    src, exe = tmp_path / "run.c", tmp_path / "run"
    src.write_text(C_SOURCE)
    libdir = os.path.dirname(dita.LIB_PATH)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"),
                    str(src), "-o", str(exe), "-L", libdir, "-ldita", "-Wl,-rpath," + libdir,
                    "-L", os.path.join(rocm, "lib"), "-lamdhip64",
                    "-Wl,-rpath," + os.path.join(rocm, "lib")], check=True)
    log(f"C program: B={B} H={H} N={N} P={P} D={D} steps={S}")
    res = subprocess.run([str(exe), str(fin), str(fout), *map(str, (B, H, T, GH, GW, P, D, S))],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    log(res.stdout.strip())
    f = res.stdout.split()
    assert f[1] == str(S) and f[3] == f[4] and f[6] == f[7], res.stdout
    raw = np.fromfile(fout, np.uint8)
    per = 12 + B * H * N * D * 4 + B * H * N * 4
    assert raw.size == S * per
    offs = partition_offsets(N, P)
    act = active_mask(offs, cfg.frame_tokens, False)
    ok = True
    for (b, h) in heads:
        ref = oracle.run_head(cfg, b, h, cache_mode="fp64", active=act, inputs=kept[(b, h)])
        for s in range(S):
            blob = raw[s * per:(s + 1) * per]
            counts = blob[:12].view(np.int32)
            out = blob[12:12 + B * H * N * D * 4].view(np.float32).reshape(B, H, N, D)
            lse = blob[12 + B * H * N * D * 4:].view(np.float32).reshape(B, H, N)
            assert np.array_equal(counts, ref[s].counts), f"step {s + 1} counts"
            good, *_ = compare(out[b, h], ref[s].out, True, f"C step {s + 1} head ({b},{h}) out")
            ok &= good and float(np.abs(lse[b, h] - ref[s].lse).max()) < 2e-3
    assert ok
