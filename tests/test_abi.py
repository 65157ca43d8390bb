"""CPU checks of the C ABI: the library loads, exports every function that
include/asm_memory.h declares, and rejects bad arguments on the host before
touching the GPU (no compute calls here)."""
import ctypes
import os
import re
import subprocess

import pytest

from attention_state_memory_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "asm_memory.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(asm_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["asm_build_states", "asm_kmeans_assign", "asm_aggregate", "asm_decode_step",
              "asm_centroid_inv_norms", "asm_abi_version", "asm_status_str", "asm_last_error"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    L = api.lib()
    names = declared_functions()
    for n in names:
        assert hasattr(L, n), f"{n} not exported"
    assert set(names) == set(api.SIGNATURES), "binding signatures differ from the header"
    out = subprocess.run(["nm", "-D", "--defined-only", api.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (asm_\w+)$", out, flags=re.M))
    assert set(names) <= exported


def test_abi_version_and_status_text():
    L = api.lib()
    assert L.asm_abi_version() == 9
    text = open(HEADER).read()
    assert int(re.search(r"#define ASM_ABI_VERSION (\d+)", text).group(1)) == 9
    assert L.asm_status_str(0) == b"ok"
    assert L.asm_status_str(-5).startswith(b"workspace")


NULL = None


def _decode(**over):
    args = dict(dtype=0, B=1, Hq=4, Hkv=2, d=128, K=16, scale=0.1, q=1 << 20, C=1 << 20,
                cinv=1 << 20, Abar=1 << 20, LSEbar=1 << 20, Kl=1 << 20, Vl=1 << 20, hs=128 * 64,
                ts=128, cap=64, ks=1 << 20, kn=1 << 20, m=64, out=1 << 20, lse=NULL, idx=NULL,
                ws=NULL, wsb=0)
    args.update(over)
    a = args
    L = api.lib()
    return L.asm_decode_step(a["dtype"], a["B"], a["Hq"], a["Hkv"], a["d"], a["K"], a["scale"],
                             a["q"], a["C"], a["cinv"], a["Abar"], a["LSEbar"], a["Kl"], a["Vl"],
                             a["hs"], a["ts"], a["cap"], a["ks"], a["kn"], a["m"], a["out"],
                             a["lse"], a["idx"], a["ws"], a["wsb"], None)


def test_decode_validation_errors_before_any_launch():
    L = api.lib()
    assert _decode(dtype=5) == -3
    assert _decode(Hq=6, Hkv=4) == -2
    assert _decode(d=300) == -2
    assert _decode(d=12) == -2          # bf16 rows must be multiples of 8
    assert _decode(K=0) == -2
    assert _decode(m=-1) == -2
    assert _decode(q=NULL) == -1
    assert _decode(Kl=NULL) == -1
    assert _decode(ts=12) == -4         # bf16 stride not a multiple of 8
    assert _decode(q=(1 << 20) + 2) == -4
    assert _decode(scale=float("nan")) == -2
    assert _decode() == -5              # a workspace is needed
    assert b"workspace" in L.asm_last_error()
    need = L.asm_decode_step_ws(0, 1, 4, 2, 128, 16, 64)
    assert need > 0
    assert _decode(ws=1 << 20, wsb=need - 1) == -5


def _decode_phase(name, **over):
    args = dict(dtype=0, B=1, Hq=4, Hkv=2, d=128, K=16, scale=0.1, q=1 << 20, C=1 << 20,
                cinv=1 << 20, Abar=1 << 20, LSEbar=1 << 20, Kl=1 << 20, Vl=1 << 20, hs=128 * 64,
                ts=128, cap=64, ks=1 << 20, kn=1 << 20, m=64, out=1 << 20, lse=NULL, idx=NULL,
                ws=NULL, wsb=0)
    args.update(over)
    a = args
    return getattr(api.lib(), name)(a["dtype"], a["B"], a["Hq"], a["Hkv"], a["d"], a["K"],
                                     a["scale"], a["q"], a["C"], a["cinv"], a["Abar"],
                                     a["LSEbar"], a["Kl"], a["Vl"], a["hs"], a["ts"], a["cap"],
                                     a["ks"], a["kn"], a["m"], a["out"], a["lse"], a["idx"],
                                     a["ws"], a["wsb"], None)


def test_decode_two_launches_validate_like_the_step_and_need_the_mfma_path():
    """asm_decode_step_begin / _finish check the step's arguments, then refuse
    what the MFMA path in one launch cannot take (float32, d=96, more than
    2048 sequences), all before any launch."""
    L = api.lib()
    for name in ("asm_decode_step_begin", "asm_decode_step_finish"):
        assert _decode_phase(name, dtype=5) == -3
        assert _decode_phase(name, q=NULL) == -1
        assert _decode_phase(name, ts=12) == -4
        assert _decode_phase(name) == -5            # a workspace is needed
        ws = L.asm_decode_step_ws(1, 1, 4, 2, 128, 16, 64)
        assert _decode_phase(name, dtype=1, ws=1 << 20, wsb=ws) == -2
        assert b"two launches" in L.asm_last_error()
        ws = L.asm_decode_step_ws(0, 1, 4, 2, 96, 16, 64)
        assert _decode_phase(name, d=96, hs=96 * 64, ts=96, ws=1 << 20, wsb=ws) == -2
        ws = L.asm_decode_step_ws(0, 2049, 4, 2, 128, 16, 64)
        assert _decode_phase(name, B=2049, ws=1 << 20, wsb=ws) == -2


def _decode_noalloc(**over):
    args = dict(dtype=0, B=1, Hq=4, Hkv=2, d=128, K=16, scale=0.1, q=1 << 20, C=1 << 20,
                cinv=1 << 20, Abar=1 << 20, LSEbar=1 << 20, Kl=1 << 20, Vl=1 << 20, hs=128 * 64,
                ts=128, cap=64, ks=1 << 20, kn=1 << 20, m=64, out=1 << 20, lse=NULL, idx=NULL)
    args.update(over)
    a = args
    L = api.lib()
    return L.asm_decode_step_noalloc(a["dtype"], a["B"], a["Hq"], a["Hkv"], a["d"], a["K"],
                                     a["scale"], a["q"], a["C"], a["cinv"], a["Abar"], a["LSEbar"],
                                     a["Kl"], a["Vl"], a["hs"], a["ts"], a["cap"], a["ks"], a["kn"],
                                     a["m"], a["out"], a["lse"], a["idx"], None)


def test_decode_noalloc_validation_and_scratch_limit_before_any_device_call():
    """The no-allocation decode checks its arguments, then the scratch its
    shape needs against the fixed per-GPU array, before it touches a device."""
    L = api.lib()
    limit = 16 << 20
    assert re.search(r"#define ASM_NOALLOC_SCRATCH_BYTES \(16u << 20\)", open(HEADER).read())
    assert _decode_noalloc(dtype=5) == -3
    assert _decode_noalloc(q=NULL) == -1
    assert _decode_noalloc(ts=12) == -4
    # the headline shape fits; 2048 sequences at K=65536 do not
    assert L.asm_decode_step_ws(0, 32, 32, 8, 128, 8192, 4096) <= limit
    big = dict(B=2048, Hq=32, Hkv=8, K=65536, m=4096, cap=2048 * 4096, hs=128 * 2048 * 4096)
    assert L.asm_decode_step_ws(0, 2048, 32, 8, 128, 65536, 4096) > limit
    assert _decode_noalloc(**big) == -5
    msg = L.asm_last_error().decode()
    assert "asm_decode_step_noalloc holds 16777216" in msg and "scratch" in msg


def test_workspace_sizes_follow_the_plan():
    L = api.lib()
    # keys (Hq * tiles * B * 8) + partial states (B * Hq * S * d * 4) + lse
    assert L.asm_decode_step_ws(0, 32, 32, 8, 128, 8192, 4096) >= 32 * 32 * 32 * 8
    assert L.asm_decode_step_ws(9, 32, 32, 8, 128, 8192, 4096) == 0  # invalid -> 0
    assert L.asm_aggregate_ws(0, 32, 65536, 8192, 128) >= 4 * 32 * (65536 + 2 * 8192)


def test_decode_table_too_large_for_32_bit_offsets_takes_the_generic_path():
    """The MFMA decode path addresses one head's centroid rows with 32-bit
    buffer offsets, so it needs (K + 64) * d * 2 < 2^31; a larger table must
    be planned on the generic path (workspace: keys [Hq, ceil(K/256), B]
    u64, partial states [B, Hq, splits, d] and their lse, each padded to
    256 bytes; one 128-token split for a 64-token local context)."""
    L = api.lib()
    d = 128
    k_big = (1 << 23) - 64  # (K + 64) * 256 == 2^31
    assert L.asm_decode_step_ws(0, 1, 1, 1, d, k_big, 64) == \
        ((k_big + 255) // 256) * 8 + 512 + 256
    # one entry fewer fits the MFMA path, whose workspace differs
    assert L.asm_decode_step_ws(0, 1, 1, 1, d, k_big - 1, 64) != \
        ((k_big - 1 + 255) // 256) * 8 + 512 + 256


def test_step_over_2_30_work_units_leaves_the_mfma_path():
    """The MFMA path counts pool claims and scoring halves in 32 bits, so its
    planner takes at most 2^30 work units (32-token tiles plus 64-entry
    scoring units) per launch: attention without memory has no other path
    (workspace 0, ASM_ERR_SHAPE), the decode falls back to the generic path."""
    L = api.lib()
    d, Hkv = 128, 8
    fits = (1 << 21) - 32  # 2048 * 8 * ceil(fits / 32) < 2^30
    assert L.asm_attend_step_ws(0, 2048, 8, Hkv, d, fits) > 0
    assert L.asm_attend_step_ws(0, 2048, 8, Hkv, d, 1 << 21) == 0


def test_build_assign_aggregate_validation():
    L = api.lib()
    st = L.asm_build_states(0, 4, 3, 8, 16, 128, 4, 0.1, 1 << 20, 1 << 20, 1 << 20, None, None,
                            1 << 20, 1 << 20, 0, None, 0, None)
    assert st == -2  # Hq % Hkv
    st = L.asm_build_states(0, 4, 2, 8, 16, 128, 4, 0.1, 1 << 20, 1 << 20, 1 << 20, 1 << 20, None,
                            1 << 20, 1 << 20, 0, None, 0, None)
    assert st == -1  # A_chunks without LSE_chunks
    st = L.asm_build_states(0, 4, 2, 8, 16, 128, 0, 0.1, 1 << 20, 1 << 20, 1 << 20, None, None,
                            1 << 20, 1 << 20, 0, None, 0, None)
    assert st == -2  # chunk 0
    assert L.asm_kmeans_assign(0, 2, 8, 0, 128, 1 << 20, 1 << 20, 1 << 20, 1 << 20, None, None, 0,
                               None) == -2
    assert L.asm_kmeans_assign(1, 2, 8, 4, 64, None, 1 << 20, 1 << 20, 1 << 20, None, None, 0,
                               None) == -1
    assert L.asm_aggregate(0, 2, 8, 4, 128, 1 << 20, 1 << 20, None, None, 1 << 20, 1 << 20,
                           1 << 20, 1 << 20, None, None, 0, None) == -1  # Abar without LSEbar
    assert L.asm_aggregate(0, 2, 8, 4, 128, 1 << 20, 1 << 20, None, None, 1 << 20, 1 << 20,
                           1 << 20, None, None, None, 0, None) == -5  # no workspace
    assert L.asm_centroid_inv_norms(3, 1, 1, 8, 1 << 20, 1 << 20, None) == -3
    # empty problems are no-ops that succeed without touching the GPU
    assert L.asm_centroid_inv_norms(0, 0, 5, 8, None, None, None) == 0
    assert L.asm_kmeans_assign(0, 2, 0, 4, 128, None, None, None, None, None, None, 0, None) == 0


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(TypeError):
        api.centroid_inv_norms(torch.zeros(1, 2, 8))


C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "asm_memory.h"

int main(void) {
  /* every entry point has a C prototype; taking its address makes the
     linker resolve it against the shared library */
  const void* fns[] = {%s};
  size_t n = sizeof fns / sizeof fns[0];
  for (size_t i = 0; i < n; ++i)
    if (fns[i] == NULL) return 2;
  if (asm_abi_version() != ASM_ABI_VERSION) return 3;
  if (strcmp(asm_status_str(ASM_OK), "ok") != 0) return 4;
  printf("%%d entry points\n", (int)n);
  return 0;
}
"""


def test_header_compiles_and_links_as_c(tmp_path):
    """include/asm_memory.h is plain C: a C11 program that names every entry
    point compiles without warnings, links against the library and calls
    its host-only functions."""
    gcc = subprocess.run(["which", "gcc"], capture_output=True, text=True).stdout.strip()
    if not gcc:
        pytest.skip("no C compiler")
    names = declared_functions()
    src = tmp_path / "abi_c.c"
    src.write_text(C_PROGRAM % ", ".join(f"(const void*)&{n}" for n in names))
    exe = tmp_path / "abi_c"
    libdir = os.path.dirname(api.LIB_PATH)
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-Wno-pedantic", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I/opt/rocm/include", str(src), "-o", str(exe),
           "-L" + libdir, "-l:" + os.path.basename(api.LIB_PATH), "-Wl,-rpath," + libdir]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert r.stdout.strip() == f"{len(names)} entry points"


def test_index_group_rows_validation_before_any_launch():
    """asm_index_group_rows refuses a bad dtype, head dim, count, null
    pointer, misalignment or an output overlapping the table, before any
    device call."""
    L = api.lib()

    def call(dtype=0, H=2, K=8, d=128, C=1 << 20, cinv=1 << 22, mem=1 << 23, Cg=1 << 24, cg=1 << 25):
        return L.asm_index_group_rows(dtype, H, K, d, C, cinv, mem, Cg, cg, None)
    assert call(dtype=7) == -3
    assert call(d=96) == -2
    assert call(K=0) == -2 and call(H=0) == -2
    assert call(C=NULL) == -1 and call(mem=NULL) == -1 and call(cg=NULL) == -1
    assert call(C=(1 << 20) + 8) == -4 and call(Cg=(1 << 24) + 8) == -4
    assert call(Cg=(1 << 20) + 2 * 8 * 128) == -2       # bf16 [2, 8, 128] = 4 KiB from C: overlaps
    assert b"overlap" in L.asm_last_error()
