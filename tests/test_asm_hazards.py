"""The SGPR-base LDS-DMA copies of the GEMM (inline asm, so outside the
compiler's hazard recogniser) keep the wait states the gfx9-family rules ask
for: five after a VALU write of an SGPR the copy reads (its base or M0).
The GEMM is compiled to gfx950 assembly here (no GPU needed) and every such
copy is checked along every control-flow path into it."""
import os
import subprocess

import pytest

import asm_scan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_scanner_finds_planted_hazards():
    bad = "\n".join(["k:", "v_readfirstlane_b32 s1, v3", "v_readfirstlane_b32 s0, v2",
                     ";;#ASMSTART", "s_nop 0", "global_load_lds_dwordx4 v0, s[0:1]", ";;#ASMEND", "s_endpgm"])
    n, v = asm_scan.scan(bad)
    assert n == 1 and len(v) == 2
    good = bad.replace("s_nop 0", "s_nop 4")
    assert asm_scan.scan(good) == (1, [])
    # a VALU write of M0, and a write reached through a branch into the block
    m0 = "\n".join(["k:", "v_readfirstlane_b32 m0, v4", "s_nop 2", "global_load_lds_dwordx4 v0, s[4:5]", "s_endpgm"])
    assert len(asm_scan.scan(m0)[1]) == 1
    loop = "\n".join(["k:", "s_branch .LBB0_2", ".LBB0_1:", "v_cmp_gt_u32_e64 s[6:7], v1, v2", "s_branch .LBB0_3",
                      ".LBB0_2:", "s_nop 7", "s_nop 7", ".LBB0_3:", "s_nop 1",
                      "global_load_lds_dwordx4 v0, s[6:7]", "s_cbranch_scc1 .LBB0_1", "s_endpgm"])
    n, v = asm_scan.scan(loop)
    assert n == 1 and len(v) == 1
    # the carry output of a 64-bit multiply-add is an SGPR write
    mad = "\n".join(["k:", "v_mad_u64_u32 v[2:3], s[0:1], v4, v5, v[6:7]", "s_nop 0",
                      "global_load_lds_dwordx4 v0, s[0:1]", "s_endpgm"])
    assert len(asm_scan.scan(mad)[1]) == 1
    # unrelated SGPRs and SALU writes are not hazards
    ok = "\n".join(["k:", "v_readfirstlane_b32 s9, v3", "s_mov_b32 s0, s9", "s_nop 0",
                    "global_load_lds_dwordx4 v0, s[0:1]", "s_endpgm"])
    assert asm_scan.scan(ok) == (1, [])


def test_gemm_sgpr_base_dma_wait_states(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not installed")
    out = tmp_path / "kernel_gemm.s"
    subprocess.check_call([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17",
                           "-I" + os.path.join(ROOT, "include"),
                           "-I" + os.path.join(ROOT, "async_tensor_tile_amd", "csrc"),
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics",
                           "-Wno-unused-command-line-argument", "--cuda-device-only", "-S",
                           os.path.join(ROOT, "async_tensor_tile_amd", "csrc", "kernel_gemm.hip"), "-o", str(out)],
                          stderr=subprocess.DEVNULL)
    asm = out.read_text()
    n, v = asm_scan.scan(asm)
    assert n > 0, "no SGPR-base LDS-DMA copies found"
    assert v == [], v[:5]
    # the operand ring's copies rely on scalar-only bases: no SGPR spills
    # (a spill restore is a VALU write of an SGPR)
    spills = asm_scan.sgpr_spills(asm)
    ring = {k: c for k, c in spills.items() if "k_gemm_bf16_ring5" in k}
    assert len(ring) == 4 and all(c == 0 for c in ring.values()), ring


def _kernel_bodies(asm: str) -> dict:
    """Kernel name -> its assembly text, for every kernel of a listing."""
    import re
    out = {}
    for m in re.finditer(r"^(_ZN3att\w+):", asm, re.M):
        end = asm.find(".Lfunc_end", m.start())
        out[m.group(1)] = asm[m.start():end]
    return out


def _argument_vector_loads(body: str) -> list:
    """Vector-memory loads whose base is the kernel-argument pointer s[0:1]
    (the kernels here have no scratch, so it is their first user SGPR pair)."""
    import re
    return re.findall(r"global_load_\w+\s+v\[?[\d:]+\]?,\s*v\d+,\s*s\[0:1\]", body)


@pytest.mark.parametrize("src", ["kernel_copy.hip", "kernels_tile.hip"])
def test_kernel_arguments_come_through_scalar_loads(tmp_path, src):
    """The copy and the tile load / store / reduce kernels read their maps as
    whole words (scalar loads); a byte field read in place would be a
    vector-memory load of the argument, a memory round trip at the start of
    every workgroup.  The scanner itself is checked on a planted line."""
    assert len(_argument_vector_loads("k:\n\tglobal_load_ubyte v3, v1, s[0:1] offset:94\n")) == 1
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not installed")
    out = tmp_path / (src + ".s")
    subprocess.check_call([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17",
                           "-I" + os.path.join(ROOT, "include"),
                           "-I" + os.path.join(ROOT, "async_tensor_tile_amd", "csrc"),
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics",
                           "-Wno-unused-command-line-argument", "--cuda-device-only", "-S",
                           os.path.join(ROOT, "async_tensor_tile_amd", "csrc", src), "-o", str(out)],
                          stderr=subprocess.DEVNULL)
    bodies = _kernel_bodies(out.read_text())
    assert len(bodies) > 3
    bad = {k: len(_argument_vector_loads(b)) for k, b in bodies.items() if _argument_vector_loads(b)}
    assert bad == {}, list(bad.items())[:5]


def _loops(body: str) -> dict:
    """Innermost-loop header -> the assembly lines of that loop's blocks,
    from the compiler's loop annotations on block labels."""
    import re
    loops, header, lines = {}, None, []
    for line in body.splitlines():
        m = re.match(r"^\.L(BB\w+):\s*(?:;\s*(.*))?$", line)
        if m:
            if header is not None:
                loops.setdefault(header, []).extend(lines)
            ann = m.group(2) or ""
            h = re.search(r"Header=(BB\w+)", ann)
            header = m.group(1) if "Loop Header" in ann else (h.group(1) if h else None)
            lines = []
        else:
            lines.append(line)
    if header is not None:
        loops.setdefault(header, []).extend(lines)
    return loops


def _atomic_loops_without_waits(body: str) -> tuple:
    """(loops holding a non-returning integer atomic, those of them with no
    vmcnt wait in any of their blocks)."""
    import re
    atom = re.compile(r"^\s*global_atomic_(add|smin|smax|umin|umax)(_x2)?\s")
    with_atomic = [ls for ls in _loops(body).values() if any(atom.match(x) and " sc0" not in x for x in ls)]
    free = [ls for ls in with_atomic if not any("s_waitcnt" in x and "vmcnt" in x for x in ls)]
    return len(with_atomic), len(free)


def test_reduce_element_loops_do_not_wait_on_atomics(tmp_path):
    """No loop of the reduce kernels that issues non-returning integer
    atomics (add, min, max) waits on vmcnt, so no iteration waits for the
    previous one's atomics to complete (a loop that also held the other
    types' compare-and-swap paths got such a wait, and a one-box int32 pass
    took twice as long).  Checked on the gfx950 assembly, per reduce kernel,
    after the loop scanner is checked on planted loops."""
    waits = "\n".join(["k:", ".LBB0_1:  ; =>This Inner Loop Header: Depth=1", "\ts_waitcnt vmcnt(0)",
                       "\tglobal_atomic_add v[2:3], v4, off", "\ts_cbranch_scc1 .LBB0_1", "\ts_endpgm"])
    assert _atomic_loops_without_waits(waits) == (1, 0)
    clean = waits.replace("\ts_waitcnt vmcnt(0)\n", "")
    assert _atomic_loops_without_waits(clean) == (1, 1)
    split = "\n".join(["k:", ".LBB0_1:  ; =>This Inner Loop Header: Depth=1", "\tv_add_u32 v1, v1, v2",
                       ".LBB0_2:  ;   in Loop: Header=BB0_1 Depth=1", "\ts_waitcnt vmcnt(0)",
                       "\tglobal_atomic_smax v[2:3], v4, off", "\ts_cbranch_scc1 .LBB0_1", "\ts_endpgm"])
    assert _atomic_loops_without_waits(split) == (1, 0)
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not installed")
    out = tmp_path / "kernels_tile.s"
    subprocess.check_call([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17",
                           "-I" + os.path.join(ROOT, "include"),
                           "-I" + os.path.join(ROOT, "async_tensor_tile_amd", "csrc"),
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics",
                           "-Wno-unused-command-line-argument", "--cuda-device-only", "-S",
                           os.path.join(ROOT, "async_tensor_tile_amd", "csrc", "kernels_tile.hip"), "-o", str(out)],
                          stderr=subprocess.DEVNULL)
    bodies = _kernel_bodies(out.read_text())
    for op in (1, 2, 3):   # add, min, max
        name = f"_ZN3att12k_tile_storeILi{op}EEEv6tmap_tPKiPKh"
        assert name in bodies, sorted(bodies)[:8]
        n, free = _atomic_loops_without_waits(bodies[name])
        assert n > 0 and free == n, (op, n, free)
