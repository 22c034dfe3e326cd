"""Host logic of libdita on the CPU: exported symbols, partition map, block policy, work
lists, slot validity and every error code.  Masks, lists and counts must equal the oracle's
independent builder bit for bit.  No device work is issued (the cache is bound to a dummy
address, which the library never dereferences before the first step)."""
import os
import re
import subprocess

import numpy as np
import pytest

import partial_state_reuse_amd as dita
from oracle.policy import (FRESH, PolicyError, partition_offsets, policy_mask, work_lists,
                           active_mask)
from workloads import CONFIGS, Policy, custom_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7f0000000000          # never dereferenced: no step is run in these tests


def header_functions():
    text = open(os.path.join(ROOT, "include", "dita.h")).read()
    return sorted(set(re.findall(r"\b(dita_[a-z_]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = header_functions()
    assert len(names) >= 12
    out = subprocess.run(["nm", "-D", "--defined-only", dita.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert sorted(dita.EXPORTED) == names


def fake_cache(cfg, active=None):
    g = dita.geometry_from(cfg)
    n = dita.dita_cache_required_bytes(g, active)
    return dita.Cache(g, active_mask=active, buffer_ptr=FAKE, buffer_bytes=n), g


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_offsets_match_oracle(idx):
    cfg = CONFIGS[idx]
    g = dita.geometry_from(cfg)
    assert list(dita.dita_partition_offsets(g)) == partition_offsets(cfg.tokens,
                                                                     cfg.num_partitions)


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_workload_masks_match_oracle(idx):
    """Every step of every workload (validity as the steps would leave it): mask bit-exact
    from the standalone evaluator; the first step's CSR lists and counts from a handle."""
    cfg = CONFIGS[idx]
    offs = partition_offsets(cfg.tokens, cfg.num_partitions)
    P = cfg.num_partitions
    g = dita.geometry_from(cfg)
    valid = np.zeros((P, P), bool)
    for s in range(1, cfg.steps + 1):
        want = policy_mask(offs, cfg.frame_tokens, cfg.policy(s), valid)
        got = dita.dita_policy_mask(g, dita.policy_from(cfg.policy(s)), valid.astype(np.uint8))
        assert np.array_equal(got, want), s
        valid |= want == FRESH
    act = active_mask(offs, cfg.frame_tokens, cfg.policy(1).tile_sparse).astype(np.uint8)
    c, _ = fake_cache(cfg, act)
    c.set_policy(dita.policy_from(cfg.policy(1)))
    got = c.plan()
    fp, fc, rp, rc, counts = work_lists(policy_mask(offs, cfg.frame_tokens, cfg.policy(1)))
    assert np.array_equal(got["fresh_ptr"], fp) and np.array_equal(got["fresh_cols"], fc)
    assert np.array_equal(got["reuse_ptr"], rp) and np.array_equal(got["reuse_cols"], rc)
    assert np.array_equal(got["counts"], counts)
    c.free()


def random_geometry(rng):
    frames = int(rng.integers(1, 6))
    gh, gw = int(rng.integers(1, 5)), int(rng.integers(1, 6))
    N = frames * gh * gw
    P = int(rng.integers(1, min(N, 9) + 1))
    cfg = custom_config(frames=frames, grid_h=gh, grid_w=gw, num_partitions=P,
                        head_dim=64, qkv_dtype="bf16", cache_dtype="bf16")
    if rng.random() < 0.5:
        cuts = np.sort(rng.choice(np.arange(1, N), size=P - 1, replace=False)) if P > 1 else []
        offs = [0] + [int(x) for x in cuts] + [N]
    else:
        offs = None
    return cfg, offs


@pytest.mark.parametrize("seed", range(40))
def test_random_policies_match_oracle(seed):
    rng = np.random.default_rng(seed)
    cfg, offs = random_geometry(rng)
    P = cfg.num_partitions
    o_offs = offs if offs is not None else partition_offsets(cfg.tokens, P)
    g = dita.geometry_from(cfg, offsets=offs)
    valid = rng.random((P, P)) < 0.6
    for trial in range(6):
        kind = int(rng.integers(0, 4))
        pol = Policy(kind=kind, max_fresh_frame_dist=int(rng.integers(-1, 3)),
                     reuse_percent=int(rng.integers(0, 101)),
                     max_fresh_centroid2=int(rng.integers(-1, 2 * cfg.tokens)),
                     tile_sparse=bool(rng.random() < 0.4), anchor=bool(rng.random() < 0.2),
                     explicit_mask=tuple(int(x) for x in rng.integers(0, 3, P * P))
                     if kind == 0 else None)
        if kind == 0 and rng.random() < 0.5:
            m = np.array(pol.explicit_mask).reshape(P, P)
            np.fill_diagonal(m, 1)
            pol = Policy(kind=0, explicit_mask=tuple(int(x) for x in m.ravel()),
                         tile_sparse=False, anchor=pol.anchor)
        try:
            want = policy_mask(o_offs, cfg.frame_tokens, pol, valid)
            want_err = None
        except PolicyError as e:
            want, want_err = None, str(e)
        try:
            got = dita.dita_policy_mask(g, dita.policy_from(pol), valid.astype(np.uint8))
            got_err = None
        except dita.DitaError as e:
            got, got_err = None, e
        if want_err is None:
            assert got_err is None, (pol, got_err)
            assert np.array_equal(got, want)
        else:
            assert got_err is not None and got_err.name in ("POLICY", "CACHE_MISS"), (pol, want_err)


def test_handle_bookkeeping_and_errors():
    cfg = CONFIGS[1]
    c, g = fake_cache(cfg)
    # no policy yet
    with pytest.raises(dita.DitaError) as e:
        c.plan()
    assert e.value.name == "NO_POLICY"
    with pytest.raises(dita.DitaError) as e:
        c.step_raw(FAKE, FAKE, FAKE, FAKE)
    assert e.value.name == "NO_POLICY"
    # reuse before anything was written
    with pytest.raises(dita.DitaError) as e:
        c.set_policy(dita.policy_from(cfg.policy(2)))
    assert e.value.name == "CACHE_MISS"
    # a failed set keeps the previous pending policy
    c.set_policy(dita.policy_from(cfg.policy(1)))
    with pytest.raises(dita.DitaError):
        c.set_policy(dita.policy_from(cfg.policy(2)))
    assert c.plan()["counts"].tolist() == [0, 16, 0]
    # non-fresh diagonal
    m = np.ones((4, 4), np.uint8)
    m[2, 2] = 2
    with pytest.raises(dita.DitaError) as e:
        c.set_policy(kind=dita.POLICY_EXPLICIT, explicit_mask=m)
    assert e.value.name == "POLICY"
    m[2, 2] = 3
    with pytest.raises(dita.DitaError) as e:
        c.set_policy(kind=dita.POLICY_EXPLICIT, explicit_mask=m)
    assert e.value.name == "POLICY"
    # reset drops the pending policy
    c.reset()
    with pytest.raises(dita.DitaError) as e:
        c.plan()
    assert e.value.name == "NO_POLICY"
    # misaligned pointers are rejected before anything is enqueued
    c.set_policy(dita.policy_from(cfg.policy(1)))
    with pytest.raises(dita.DitaError) as e:
        c.step_raw(FAKE + 2, FAKE, FAKE, FAKE)
    assert e.value.name == "INVALID_ARGUMENT"
    assert c.stats()["steps_done"] == 0
    c.free()


def test_active_mask_slots():
    cfg = CONFIGS[4]
    offs = partition_offsets(cfg.tokens, cfg.num_partitions)
    act = active_mask(offs, cfg.frame_tokens, True).astype(np.uint8)
    g = dita.geometry_from(cfg)
    small = dita.dita_cache_required_bytes(g, act)
    full = dita.dita_cache_required_bytes(g, None)
    assert small < full / 4
    c = dita.Cache(g, active_mask=act, buffer_ptr=FAKE, buffer_bytes=small)
    # a block outside the active mask has no slot
    m = np.eye(24, dtype=np.uint8)
    m[23, 0] = 1
    m[23, 5] = 1                       # frame distance 18: not in the tile-sparse set
    with pytest.raises(dita.DitaError) as e:
        c.set_policy(kind=dita.POLICY_EXPLICIT, explicit_mask=m)
    assert e.value.name == "POLICY"
    c.free()
    with pytest.raises(dita.DitaError) as e:
        dita.Cache(g, active_mask=act, buffer_ptr=FAKE, buffer_bytes=small - 256)
    assert e.value.name == "BUFFER_TOO_SMALL"
    bad = act.copy()
    bad[3, 3] = 0
    with pytest.raises(dita.DitaError) as e:
        dita.dita_cache_required_bytes(g, bad)
    assert e.value.name == "POLICY"


def test_geometry_errors():
    def err(**kw):
        base = dict(batch=1, heads=1, tokens=64, head_dim=64, frames=4, grid_h=4, grid_w=4,
                    num_partitions=4, dtype="bf16")
        base.update(kw)
        offsets = base.pop("offsets", None)
        g = dita.make_geometry(**base, offsets=offsets)
        with pytest.raises(dita.DitaError) as e:
            dita.dita_cache_required_bytes(g)
        return e.value.name
    assert err(tokens=63) == "SHAPE"
    assert err(num_partitions=0) == "SHAPE"
    assert err(num_partitions=65) == "SHAPE"
    assert err(head_dim=60) == "UNSUPPORTED"
    assert err(head_dim=136) == "UNSUPPORTED"
    assert err(dtype="f32", head_dim=128) == "UNSUPPORTED"
    assert err(offsets=[0, 10, 10, 40, 64]) == "SHAPE"
    assert err(offsets=[0, 10, 20, 40, 63]) == "SHAPE"
    assert err(batch=0) == "SHAPE"
    # limits: at most 1024 partitions, partitions under 2^21 rows, tensors under 2^40 elements
    assert err(tokens=2048, frames=8, grid_h=16, grid_w=16, num_partitions=1025) == "SHAPE"
    assert err(tokens=1 << 21, frames=32, grid_h=256, grid_w=256, num_partitions=1) == "SHAPE"
    assert err(batch=1 << 10, heads=1 << 10, tokens=1 << 14, frames=1, grid_h=128, grid_w=128,
               head_dim=64) == "SHAPE"
    assert err(dtype="f32", cache_dtype="fp8") == "UNSUPPORTED"
    big = dita.make_geometry(1, 1, 1024, 64, 4, 16, 16, 1024, "bf16")   # P = N = 1024: accepted
    assert dita.dita_cache_required_bytes(big) > 0
    g = dita.make_geometry(1, 1, 64, 64, 4, 4, 4, 4, "bf16")
    with pytest.raises(dita.DitaError) as e:
        dita.Cache(g, buffer_ptr=FAKE, buffer_bytes=dita.dita_cache_required_bytes(g) - 256)
    assert e.value.name == "BUFFER_TOO_SMALL"
    with pytest.raises(dita.DitaError) as e:
        dita.Cache(g, buffer_ptr=FAKE + 16, buffer_bytes=1 << 30)
    assert e.value.name == "INVALID_ARGUMENT"


@pytest.mark.parametrize("idx,cache", [(2, "bf16"), (3, "bf16"), (3, "fp8"), (1, "f32")])
def test_offload_size_and_argument_errors(idx, cache):
    """Host offload (no device work): the offloaded state holds at least every slot's cached
    O and lse (n_i rows of D elements of the cache precision plus one f32 each, per (b, h) and
    active block) and at most the whole device buffer; calls that cannot proceed fail before
    any copy is enqueued."""
    import ctypes
    import dataclasses
    cfg = dataclasses.replace(CONFIGS[idx], cache_dtype=cache)
    offs = partition_offsets(cfg.tokens, cfg.num_partitions)
    act = active_mask(offs, cfg.frame_tokens, cfg.policy(1).tile_sparse)
    c, g = fake_cache(cfg, act.astype(np.uint8))
    n = c.offload_bytes()
    esz = {"f32": 4, "bf16": 2, "fp8": 1}[cache]
    rows = np.diff(np.asarray(offs, np.int64))
    state = int(sum(rows[i] * (cfg.head_dim * esz + 4)
                    for i in range(cfg.num_partitions) for j in range(cfg.num_partitions)
                    if act[i, j])) * cfg.batch * cfg.heads
    assert state < n <= c.required_bytes
    lib = dita._lib
    small = (ctypes.c_uint8 * 64)()
    assert lib.dita_cache_offload(c._h, None, n, None) == 1                  # host_dst NULL
    assert lib.dita_cache_offload(c._h, ctypes.cast(small, ctypes.c_void_p), 64, None) == 1
    assert lib.dita_cache_restore(c._h, dita._P(FAKE), c.required_bytes,
                                  ctypes.cast(small, ctypes.c_void_p), n, None) == 1
    assert "not offloaded" in dita._lib.dita_last_error().decode()
    size = ctypes.c_size_t(0)
    assert lib.dita_cache_offload_bytes(None, ctypes.byref(size)) == 1
    assert lib.dita_cache_offload_bytes(c._h, None) == 1
    c.free()


def test_layout_field():
    """The layout of Q, K, V and out changes neither the buffer size nor the plan; an unknown
    layout is rejected before anything else."""
    cfg = CONFIGS[3]
    g1 = dita.geometry_from(cfg)
    g2 = dita.geometry_from(cfg)
    g2.layout = dita.LAYOUT_BNHD
    assert dita.dita_cache_required_bytes(g1) == dita.dita_cache_required_bytes(g2)
    plans = []
    for g in (g1, g2):
        n = dita.dita_cache_required_bytes(g)
        c = dita.Cache(g, buffer_ptr=FAKE, buffer_bytes=n)
        c.set_policy(dita.policy_from(cfg.policy(1)))
        plans.append(c.plan())
        c.free()
    assert all(np.array_equal(plans[0][k], plans[1][k]) for k in plans[0])
    g3 = dita.geometry_from(cfg)
    g3.layout = 2
    with pytest.raises(dita.DitaError) as e:
        dita.dita_cache_required_bytes(g3)
    assert e.value.name == "INVALID_ARGUMENT"


def test_step_rejects_bad_output_tensors_before_launch():
    """Caller-supplied out / lse of the wrong dtype, shape, layout or device, and inputs that
    are not on a HIP device, raise ValueError in the binding before the library is called
    (host tensors only here; the cache is bound to an address never dereferenced)."""
    torch = pytest.importorskip("torch")
    cfg = CONFIGS[1]
    c, g = fake_cache(cfg)
    c.set_policy(dita.policy_from(cfg.policy(1)))
    B, H, N, D = cfg.batch, cfg.heads, cfg.tokens, cfg.head_dim
    q = k = v = torch.zeros((B, H, N, D), dtype=torch.float32)
    good_out = torch.zeros((B, H, N, D), dtype=torch.float32)
    good_lse = torch.zeros((B, H, N), dtype=torch.float32)
    bad = [
        ("out", dict(out=good_out.to(torch.bfloat16)), "float32"),
        ("out", dict(out=good_out[:, :, : N - 1]), "shape"),
        ("out", dict(out=torch.zeros((B, N, H, D), dtype=torch.float32)), "shape"),
        ("out", dict(out=torch.zeros((B, H, D, N), dtype=torch.float32).transpose(2, 3)),
         "contiguous"),
        ("lse", dict(lse=good_lse.to(torch.float64)), "float32"),
        ("lse", dict(lse=torch.zeros((B, H, N + 1), dtype=torch.float32)), "shape"),
    ]
    for name, kw, word in bad:
        with pytest.raises(ValueError, match=word):
            c.step(q, k, v, **kw)
    with pytest.raises(ValueError, match="HIP device"):     # right tensors, but host memory
        c.step(q, k, v, out=good_out, lse=good_lse)
    assert c.stats()["steps_done"] == 0
    c.free()


def test_static_step_rejects_before_any_device_work():
    """dita_attn_step_static refuses, before touching the device, a step whose scratch
    exceeds its 128 MiB static array (the CFG workload's transposed V alone is 545 MB) and a
    PLANNER step (its measurements need a read-back buffer); the 29-frame workload fits."""
    lib = dita._lib
    P = dita._P
    for idx, want in ((5, "UNSUPPORTED"), (3, None)):
        cfg = CONFIGS[idx]
        c, g = fake_cache(cfg)
        c.set_policy(dita.policy_from(cfg.policy(1)))
        if want is None:
            B, H, N = cfg.batch, cfg.heads, cfg.tokens
            vt = B * H * 64 * sum(-(-int(n) // 64) * 64
                                  for n in np.diff(dita.dita_partition_offsets(g)))
            assert vt * 2 < (128 << 20)
            c.free()
            continue
        rc = lib.dita_attn_step_static(c._h, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, None)
        assert dita.STATUS_NAMES[rc] == want
        assert b"128" in lib.dita_last_error() or b"static maximum" in lib.dita_last_error()
        assert c.stats()["steps_done"] == 0
        c.free()
    cfg = custom_config(name="planner-static", idx=80, heads=1, head_dim=64, frames=2,
                        grid_h=4, grid_w=8, num_partitions=4, steps=2, qkv_dtype="bf16",
                        cache_dtype="bf16")
    c, g = fake_cache(cfg)
    c.set_policy(dita.make_policy(kind=dita.POLICY_PLANNER, reuse_percent=50))
    rc = lib.dita_attn_step_static(c._h, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, None)
    assert dita.STATUS_NAMES[rc] == "UNSUPPORTED"
    assert b"PLANNER" in lib.dita_last_error()
    assert c.stats()["steps_done"] == 0
    c.free()


def test_out_dtype_field():
    """The output dtype: f32 (the zero default) or bf16 with bf16 Q/K/V; it changes neither
    the buffer size nor the plan; bf16 with f32 inputs and unknown values are rejected."""
    cfg = CONFIGS[3]
    sizes = {dt: dita.dita_cache_required_bytes(dita.geometry_from(cfg, out_dtype=dt))
             for dt in ("f32", "bf16")}
    assert sizes["f32"] == sizes["bf16"]
    assert dita.geometry_from(cfg).out_dtype == dita.F32
    with pytest.raises(dita.DitaError) as e:
        dita.dita_cache_required_bytes(dita.geometry_from(CONFIGS[1], out_dtype="bf16"))
    assert e.value.name == "UNSUPPORTED"
    g = dita.geometry_from(cfg)
    g.out_dtype = 2
    with pytest.raises(dita.DitaError) as e:
        dita.dita_cache_required_bytes(g)
    assert e.value.name == "INVALID_ARGUMENT"


def test_header_is_c_and_matches_the_binding(tmp_path):
    """include/dita.h compiles as plain C99, and its structs have the sizes and field offsets
    the ctypes binding declares (a mismatch would pass wrong arguments silently)."""
    import ctypes
    import shutil
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    structs = {"dita_geometry": dita.Geometry, "dita_block_policy": dita.BlockPolicy,
               "dita_step_stats": dita.StepStats}
    lines = ['#include <stddef.h>', '#include <stdio.h>', '#include "dita.h"',
             'int main(void) {']
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'  printf("{cname}.{fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ['  return 0;', '}']
    src = tmp_path / "abi.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "abi"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", "-I",
                    os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(line.rsplit(" ", 1) for line in
               subprocess.run([str(exe)], capture_output=True, text=True, check=True)
               .stdout.splitlines())
    for cname, py in structs.items():
        assert int(got[cname]) == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert int(got[f"{cname}.{fname}"]) == getattr(py, fname).offset, (cname, fname)


def test_c_program_uses_the_library(tmp_path):
    """A plain C program linked against libdita.so drives the host-side calls (geometry, buffer
    size, handle over a dummy address, budget policy, plan, error message): the boundary is
    usable without Python.  The 29-frame workload's steady policy keeps 13 of 32 blocks per
    row fresh."""
    import shutil
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    src = tmp_path / "use.c"
    src.write_text(r'''
#include <stdio.h>
#include <string.h>
#include "dita.h"
int main(void) {
  dita_geometry g;
  memset(&g, 0, sizeof g);
  g.batch = 1; g.heads = 24; g.tokens = 28800; g.head_dim = 64;
  g.frames = 8; g.grid_h = 45; g.grid_w = 80; g.num_partitions = 32;
  g.qkv_dtype = DITA_BF16; g.cache_o_dtype = DITA_BF16;
  size_t bytes = 0;
  if (dita_cache_required_bytes(&g, NULL, &bytes) != DITA_OK) return 1;
  dita_cache* c = NULL;
  if (dita_cache_alloc(&g, NULL, (void*)(size_t)0x7f0000000000ull, bytes, &c) != DITA_OK) return 2;
  dita_block_policy p;
  memset(&p, 0, sizeof p);
  p.kind = DITA_POLICY_FRESH_BUDGET; p.reuse_percent = 60; p.anchor = 1;
  if (dita_set_block_policy(c, &p) != DITA_OK) return 3;
  int32_t counts[3];
  if (dita_get_block_plan(c, NULL, NULL, NULL, NULL, NULL, counts) != DITA_OK) return 4;
  printf("anchor %d %d %d\n", counts[0], counts[1], counts[2]);
  uint8_t valid[32 * 32], mask[32 * 32];
  memset(valid, 1, sizeof valid);
  p.anchor = 0;
  if (dita_policy_mask(&g, &p, valid, mask) != DITA_OK) return 5;
  int fresh = 0;
  for (int j = 0; j < 32; ++j) fresh += mask[j] == DITA_FRESH;
  printf("row0 fresh %d\n", fresh);
  p.reuse_percent = 101;
  const dita_status st = dita_set_block_policy(c, &p);
  printf("bad %d %s\n", (int)st, dita_last_error()[0] ? "msg" : "none");
  dita_cache_free(c);
  printf("%s\n", dita_version());
  return 0;
}
''')
    libdir = os.path.dirname(dita.LIB_PATH)
    exe = tmp_path / "use"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe), "-L", libdir, "-ldita",
                    "-Wl,-rpath," + libdir], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    assert out[0] == "anchor 0 1024 0"
    assert out[1] == "row0 fresh 13"
    assert out[2] == "bad 1 msg"             # INVALID_ARGUMENT, with a message
    assert out[3].startswith("dita ")
