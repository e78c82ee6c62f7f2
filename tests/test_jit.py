"""The hipRTC build on the CPU: every kernel the measured tables select compiles for
gfx950 with no scratch (spill) access in its K loop, a compile error comes back as
DG_ERR_JIT, and a damaged cache entry is rebuilt.  Each check runs in a fresh
process with its own cache directory (the library also caches code in memory)."""
import glob
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
READELF = "/opt/rocm/llvm/bin/llvm-readelf"
OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"

# (kind | format flag, rows, N, K, groups, has_c): the benchmark workloads in every format
SF_UE8M0, SF_FP8_FP4, SF_BF16, SF_FP4_FP4 = 4, 8, 16, 32
PLANS = [
    (0, 64, 2112, 7168, 1, 0), (0, 128, 24576, 1536, 1, 0), (0, 128, 24576, 1536, 1, 1),
    (0, 4096, 7168, 16384, 1, 0), (1, 32768, 4096, 7168, 4, 0), (2, 256, 7168, 2048, 4, 0),
    (3, 4096, 7168, 32768, 4, 0),
    (0 | SF_UE8M0, 64, 2112, 7168, 1, 0), (0 | SF_UE8M0, 4096, 7168, 16384, 1, 0),
    (1 | SF_UE8M0, 32768, 4096, 7168, 4, 0), (2 | SF_UE8M0, 256, 7168, 2048, 4, 0),
    (0 | SF_FP8_FP4, 128, 24576, 1536, 1, 0), (0 | SF_FP8_FP4, 4096, 7168, 16384, 1, 0),
    (1 | SF_FP8_FP4, 32768, 4096, 7168, 4, 0), (2 | SF_FP8_FP4, 256, 7168, 2048, 4, 0),
    (0 | SF_FP4_FP4, 128, 24576, 1536, 1, 0), (0 | SF_FP4_FP4, 4096, 7168, 16384, 1, 0),
    (0 | SF_BF16, 4096, 7168, 16384, 1, 0),
    # model-chosen small shapes (ragged, with C)
    (0, 300, 520, 1024, 1, 1), (2, 200, 333, 640, 3, 1), (0 | SF_FP8_FP4, 5, 129, 640, 1, 1),
]


def _run(code, cache_dir, extra_env=None):
    env = dict(os.environ, DG_CACHE_DIR=str(cache_dir), **(extra_env or {}))
    return subprocess.run([sys.executable, "-c", textwrap.dedent(code)], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=600)


PRECOMPILE = """
    import ctypes, sys
    import torch  # the hipRTC library a torch process resolves, as in build()
    lib = ctypes.CDLL("moe_grouped_gemm_scales_amd/libdg.so")
    lib.dg_last_error.restype = ctypes.c_char_p
    for plan in {plans}:
        rc = lib.dg_precompile(*plan, 256)
        print(plan, rc, lib.dg_last_error().decode()[:300], flush=True)
"""


def _notes(path):
    out = subprocess.run([READELF, "--notes", path], capture_output=True, text=True).stdout
    vals = {}
    for line in out.splitlines():
        line = line.strip()
        for key in (".vgpr_spill_count:", ".sgpr_spill_count:", ".private_segment_fixed_size:"):
            if line.startswith(key):
                vals.setdefault(key.strip(":."), []).append(int(line.split()[-1]))
    return vals


def _k_loop_scratch_ops(path):
    """Scratch (spill) instructions between the first and the last MFMA of the GEMM kernel,
    i.e. inside its K loop, in the AMD disassembly of this code object."""
    out = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", path], capture_output=True, text=True).stdout
    body = out.split("<dg_fp8_gemm_nt_kernel>:", 1)[1].split("\n\n", 1)[0].splitlines()
    mfma = [i for i, line in enumerate(body) if "v_mfma" in line]
    assert mfma, "no MFMA in the GEMM kernel"
    return [line.strip() for line in body[mfma[0]:mfma[-1] + 1] if "scratch_" in line]


@pytest.mark.skipif(not (os.path.exists(READELF) and os.path.exists(OBJDUMP)), reason="LLVM tools not installed")
def test_selected_kernels_keep_their_k_loop_out_of_scratch(tmp_path):
    """No kernel a measured table selects touches scratch memory, in its K loop or
    anywhere else.  (A spilled epilogue store address costs a scratch reload, and with
    it a wait for every store issued before, per store.)"""
    r = _run(PRECOMPILE.format(plans=repr(PLANS)), tmp_path)
    assert r.returncode == 0, r.stderr[-2000:]
    assert all(line.split(")")[1].split()[0] == "0" for line in r.stdout.strip().splitlines()), r.stdout
    objs = glob.glob(str(tmp_path / "*.hsaco"))
    assert len(objs) >= len(PLANS) - 2      # a few plans may share a code object
    spilling = []
    for path in objs:
        v = _notes(path)
        name = os.path.basename(path)
        assert v, name
        assert not _k_loop_scratch_ops(path), f"{name}: scratch access in the K loop"
        if max(v.get("vgpr_spill_count", [0])) or max(v.get("private_segment_fixed_size", [0])):
            spilling.append(name.rsplit("-", 1)[0])
    assert not spilling, spilling


def _epilogue_stores(path):
    """Global store instructions of the GEMM kernel, by width, in the AMD disassembly."""
    out = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", path], capture_output=True, text=True).stdout
    body = out.split("<dg_fp8_gemm_nt_kernel>:", 1)[1].split("\n\n", 1)[0]
    return {w: body.count(f"global_store_{w} ") for w in ("dwordx4", "dwordx2", "short", "dword")}


@pytest.mark.skipif(not (os.path.exists(READELF) and os.path.exists(OBJDUMP)), reason="LLVM tools not installed")
def test_wide_tile_epilogues_store_sixteen_bytes(tmp_path):
    """The selected 256-column tiles of eight waves (an even number of n sub-tiles per
    wave) store D in 16-byte pieces only: lanes 16 apart swap values so that a lane holds 8
    consecutive columns.  (With 8-byte stores the contiguous workload wrote D to the fabric
    twice.)"""
    plans = [pl for pl in PLANS if pl[2] in (4096, 7168)]
    r = _run(PRECOMPILE.format(plans=repr(plans)), tmp_path)
    assert r.returncode == 0, r.stderr[-2000:]
    checked = 0
    for path in glob.glob(str(tmp_path / "*.hsaco")):
        name = os.path.basename(path)
        if "n256_w4x2" not in name:
            continue
        st = _epilogue_stores(path)
        assert st["dwordx4"] >= 8 and st["dwordx2"] == 0 and st["short"] == 0, (name, st)
        checked += 1
    assert checked >= 5, checked


def test_compile_error_is_dg_err_jit(tmp_path):
    r = _run(PRECOMPILE.format(plans=repr([(0, 64, 64, 128, 1, 0)])), tmp_path,
             {"DG_JIT_EXTRA_OPTION": "-DDG_BM=not_a_number"})
    assert r.returncode == 0, r.stderr[-2000:]
    assert " -4 " in r.stdout and "hipRTC compile" in r.stdout, r.stdout


def test_damaged_cache_entry_is_rebuilt(tmp_path):
    plan = [(0, 96, 200, 256, 1, 0)]
    r = _run(PRECOMPILE.format(plans=repr(plan)), tmp_path)
    assert r.returncode == 0 and " 0 " in r.stdout, r.stdout + r.stderr[-2000:]
    (obj,) = glob.glob(str(tmp_path / "*.hsaco"))
    with open(obj, "wb") as f:
        f.write(b"not a code object")
    r = _run(PRECOMPILE.format(plans=repr(plan)), tmp_path)
    assert r.returncode == 0 and " 0 " in r.stdout, r.stdout + r.stderr[-2000:]
    with open(obj, "rb") as f:
        assert f.read(4) == b"\x7fELF"


def test_extra_option_is_part_of_the_cache_key(tmp_path):
    """A build with DG_JIT_EXTRA_OPTION gets a cache entry of its own, on disk and in
    memory: it is never served to a caller without the option (or with another)."""
    plan = [(0, 96, 200, 256, 1, 0)]
    count = lambda: len(glob.glob(str(tmp_path / "*.hsaco")))
    r = _run(PRECOMPILE.format(plans=repr(plan)), tmp_path)
    assert r.returncode == 0 and " 0 " in r.stdout, r.stdout + r.stderr[-2000:]
    assert count() == 1
    # another process with the option: a second code object, not the first one
    r = _run(PRECOMPILE.format(plans=repr(plan)), tmp_path, {"DG_JIT_EXTRA_OPTION": "-DDG_FA_AHEAD=2"})
    assert r.returncode == 0 and " 0 " in r.stdout, r.stdout + r.stderr[-2000:]
    assert count() == 2
    # one process that sets the option between two calls builds (and caches) a third
    in_process = textwrap.dedent(PRECOMPILE.format(plans=repr(plan))) + textwrap.dedent("""
        import os
        os.environ["DG_JIT_EXTRA_OPTION"] = "-DDG_FA_AHEAD=3"
        print("second", lib.dg_precompile(*{plan}, 256), flush=True)
    """).format(plan=repr(plan[0]))
    r = _run(in_process, tmp_path)
    assert r.returncode == 0 and "second 0" in r.stdout, r.stdout + r.stderr[-2000:]
    assert count() == 3


def test_register_load_variant_that_spills_is_refused(tmp_path):
    """The kernels that load B straight into registers issue those loads in inline
    assembly, so the compiler must not spill a register such a load may still be
    writing: a forced tile whose code object spills comes back as DG_ERR_JIT instead
    of running.  (128 x 128 with four waves and six stages spills; three stages
    do not.)"""
    plan = [(0, 300, 520, 1024, 1, 1)]
    r = _run(PRECOMPILE.format(plans=repr(plan)), tmp_path, {"DG_FORCE_CONFIG": "128,128,1,4,6,1,1,1"})
    assert r.returncode == 0, r.stderr[-2000:]
    assert " -4 " in r.stdout and "must not spill registers" in r.stdout, r.stdout
    r = _run(PRECOMPILE.format(plans=repr(plan)), tmp_path, {"DG_FORCE_CONFIG": "128,128,1,4,3,1,1,1"})
    assert r.returncode == 0 and " 0 " in r.stdout, r.stdout + r.stderr[-2000:]


@pytest.mark.skipif(not os.path.exists(READELF), reason="LLVM tools not installed")
def test_kernel_takes_one_by_value_argument_of_the_host_layout(tmp_path):
    """The GEMM kernel's only explicit argument is the 96-byte struct the host fills
    (api.cpp's LaunchParams: nine pointers, three ints, the status pointer); its code
    object metadata must say so, for every variant a table selects."""
    plans = [(0, 64, 2112, 7168, 1, 0), (0, 128, 24576, 1536, 1, 0), (0, 4096, 7168, 16384, 1, 0),
             (2, 256, 7168, 2048, 4, 0), (1, 32768, 4096, 7168, 4, 0)]
    r = _run(PRECOMPILE.format(plans=repr(plans)), tmp_path)
    assert r.returncode == 0, r.stderr[-2000:]
    objs = glob.glob(str(tmp_path / "*.hsaco"))
    assert len(objs) >= len(plans)
    for path in objs:
        out = subprocess.run([READELF, "--notes", path], capture_output=True, text=True).stdout
        lines = out.split(".name:           dg_fp8_gemm_nt_kernel")[0].splitlines()
        start = max(i for i, line in enumerate(lines) if line.strip() == ".args:")
        items, cur = [], None
        for line in lines[start + 1:]:
            if line.startswith("      - "):
                cur = {}
                items.append(cur)
                line = line.replace("- ", "  ", 1)
            elif not line.startswith("        "):
                break                                   # the next key of the kernel's entry
            k, _, v = line.strip().partition(":")
            cur[k] = v.strip()
        explicit = [it for it in items if not it[".value_kind"].startswith("hidden_")]
        assert explicit == [{".offset": "0", ".size": "96", ".value_kind": "by_value"}], (os.path.basename(path),
                                                                                          explicit)


def test_split_k_counter_stride_agrees_between_kernel_and_host():
    """The kernel indexes a wave's arrival counter CTR_STRIDE words apart and the
    host sizes the counter buffer kCounterStrideBytes per counter: the two are
    compiled separately (hipRTC and the host compiler), so they are compared here."""
    import re
    kern = open(os.path.join(ROOT, "moe_grouped_gemm_scales_amd", "csrc", "kernels", "fp8_gemm.hip")).read()
    host = open(os.path.join(ROOT, "moe_grouped_gemm_scales_amd", "csrc", "dg_internal.h")).read()
    words = int(re.search(r"constexpr int CTR_STRIDE = (\d+);", kern).group(1))
    stride = int(re.search(r"constexpr size_t kCounterStrideBytes = (\d+);", host).group(1))
    assert words * 4 == stride
    assert stride >= 128, "one counter per 128-byte line: atomics on a shared line are serialised"
