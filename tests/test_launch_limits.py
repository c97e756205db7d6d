"""Launch-limit registry (TensorFold PR #949, "Kernel contract": every launch
registered against the chip's limits): each kernel's registers, scratch and
LDS, read from the compiler's resource-usage report for gfx950, checked
against the hardware's limits and against what the kernels' designs assume.
Also checks the assembly for the one register the kernels write by hand (M0,
in the global-to-LDS loads).  CPU only: hipcc cross-compiles for gfx950."""
import glob
import os
import re
import subprocess

import numpy as np
import pytest

from audio_diffusion_transformer_amd import build as BUILD
from audio_diffusion_transformer_amd import synth as S

CSRC = BUILD.CSRC
LDS_PER_CU = 160 * 1024      # gfx950
VGPRS_PER_LANE = 512         # unified VGPR + AGPR file per SIMD lane
MAX_SGPRS = 102


def _compile(src, extra):
    cmd = [BUILD.HIPCC, f"--offload-arch={BUILD.ARCH}", "-O3", "-std=c++17", "-Xclang",
           "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", BUILD.INCLUDE, "-I", CSRC,
           "--cuda-device-only"] + extra + [src]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return r


@pytest.fixture(scope="module")
def usage():
    """{kernel symbol: {field: value}} for every kernel of the library."""
    out = {}
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        r = _compile(src, ["-c", "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"])
        name = None
        for line in r.stderr.splitlines():
            m = re.search(r"remark: Function Name: (\S+)", line)
            if m:
                name = m.group(1)
                out[name] = {}
                continue
            m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\S+) \[-Rpass", line)
            if m and name:
                out[name][m.group(1).strip()] = m.group(2)
    assert out, "no resource-usage remarks"
    return out


def _regs(u):
    return int(u["VGPRs"]) + int(u.get("AGPRs", 0))


def test_every_kernel_within_gfx950_limits(usage):
    for name, u in usage.items():
        assert int(u["ScratchSize"]) == 0, (name, "uses scratch")
        # (SGPR spills land in VGPR lanes, not in memory: allowed, but not on
        # the kernels of the default workload, checked below)
        assert int(u["VGPRs Spill"]) == 0, (name, "spills VGPRs")
        assert u["Dynamic Stack"] == "False", name
        assert _regs(u) <= VGPRS_PER_LANE, name
        assert int(u["TotalSGPRs"]) <= MAX_SGPRS + 6, name   # + VCC, FLAT_SCRATCH, XNACK
        assert int(u["LDS Size"]) <= LDS_PER_CU, name


def test_default_workload_kernels_spill_nothing(usage):
    """The kernels the default forward launches (hidden 5120, 40 x 128 heads,
    242 tiles: the routing variant for up to 256 tiles) keep every value in
    registers."""
    hot = [k for k in usage if re.search(
        r"k_gemm_bf16|k_attnILi128|k_headsILi128|k_modnorm|k_routeILi128ELi4E|k_out_head|k_poke",
        k)]
    assert len(hot) >= 8, hot
    for k in hot:
        assert int(usage[k]["SGPRs Spill"]) == 0 and int(usage[k]["VGPRs Spill"]) == 0, k


def _kernels(usage, pattern):
    ks = [k for k in usage if re.search(pattern, k)]
    assert ks, pattern
    return ks


def test_products_one_512_thread_workgroup_per_cu(usage):
    """The GEMM's ping-pong schedule needs its 8 waves resident together: two
    waves per SIMD (at most 256 registers a lane) and its LDS ring in one CU."""
    for k in _kernels(usage, "k_gemm_bf16|k_gemm_i8g"):
        u = usage[k]
        assert _regs(u) <= VGPRS_PER_LANE // 2, (k, _regs(u))
        assert int(u["Occupancy"]) >= 2, k
        assert int(u["LDS Size"]) <= LDS_PER_CU, k


def _attn_dynamic_lds(sh):
    """Dynamic LDS of one attention workgroup for this workload: the selected
    tiles' scores, chunk starts and offsets, the longest video key list (uint16
    chunk ids) and a byte per 32-row chunk."""
    ts, npt = S.tile_map(sh)
    lens = np.diff(ts)
    chunks = (lens + 31) // 32
    nQ = len(lens) - npt
    nsel = min(sh.top_k, nQ)
    max_list = int(chunks[:npt].sum() + np.sort(chunks[npt:])[::-1][:nsel].sum())
    return 4 * (3 * nsel + 1) + 2 * max_list + int(chunks.sum())


def test_attention_four_workgroups_per_cu(usage):
    """Attention relies on four workgroups (four waves per SIMD) sharing a CU,
    so that one wave's softmax runs beside another's products: at most 128
    registers a lane, and four workgroups' static + dynamic LDS in 160 KB at
    the benchmark's workloads."""
    for k in _kernels(usage, "k_attnILi"):
        u = usage[k]
        assert _regs(u) <= VGPRS_PER_LANE // 4, (k, _regs(u))
        assert int(u["Occupancy"]) >= 4, k
        d = 128 if "ILi128" in k else 64
        for sh in (S.FULL, S.FASTH3, S.MID):
            if sh.head_dim != d:
                continue
            total = int(u["LDS Size"]) + _attn_dynamic_lds(sh)
            assert 4 * total <= LDS_PER_CU, (k, sh, total)


def test_m0_written_only_by_the_lds_loads():
    """M0 is a reserved register the compiler allocates no value to; the
    kernels set it by hand right before each global-to-LDS load (with the one
    wait state the ISA asks for).  No compiler-generated instruction may read
    or write it, so the hand-written writes cannot disturb a value of its."""
    for src in ("k_gemm.hip", "k_attn.hip"):
        r = _compile(os.path.join(CSRC, src), ["-S", "-o", "-"])
        lines = [l.strip() for l in r.stdout.splitlines()]
        code = [l for l in lines if l and not l.startswith((";", ".", "//")) and
                not l.endswith(":")]
        n = 0
        for i, l in enumerate(code):
            if re.search(r"\bm0\b", l):
                assert re.fullmatch(r"s_mov_b32 m0, s\d+", l), (src, l)
                assert code[i + 1] == "s_nop 0", (src, code[i + 1])
                assert code[i + 2].startswith("global_load_lds_dwordx4"), (src, code[i + 2])
                n += 1
        assert n > 0, src
