"""Checks on the gfx950 assembly of the HIP sources (host only: hipcc
cross-compiles, no GPU needed).

- every global -> LDS DMA (inline asm, which the compiler's hazard pass does
  not look into) is immediately preceded by the five wait states it carries
  itself: a base register written by a vector instruction just before needs
  five, an M0 write just before needs one;
- no packed fp32 VALU instructions anywhere (the compile flags disable the feature);
- the grouped-GEMM kernels keep their contraction loops in registers: no
  kernel touches scratch in a basic block that issues MFMAs, the kernels
  without the routed-X row map use no scratch at all, and the routed ones
  (a few more registers for the token rows) at most 16 bytes outside the
  loop (tile set-up and epilogue).
"""
import concurrent.futures as cf
import glob
import importlib.util
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_fake_quant_amd", "csrc")


def _build_mod():
    spec = importlib.util.spec_from_file_location(
        "_fq_build", os.path.join(ROOT, "moe_fake_quant_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    b = _build_mod()
    try:
        cc = b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa")
    flags = [f for f in b.flags() if f not in ("-fPIC", "-shared")]

    def one(src):
        dst = os.path.join(out, os.path.basename(src) + ".s")
        r = subprocess.run([cc, *flags, "--cuda-device-only", "-S", "-o", dst, src],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        with open(dst) as f:
            return os.path.basename(src), f.read()

    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        return dict(ex.map(one, srcs))


def _instructions(text):
    """(line, mnemonic) of the real instructions, comments and labels dropped."""
    out = []
    for line in text.split("\n"):
        t = line.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        out.append((t, t.split()[0]))
    return out


def test_lds_dma_carries_its_wait_states(asm):
    n = 0
    for name, text in asm.items():
        ins = _instructions(text)
        for i, (line, op) in enumerate(ins):
            if op.startswith("global_load_lds") or op.startswith("buffer_load_lds"):
                n += 1
                prev = ins[i - 1][0] if i else ""
                m = re.match(r"s_nop\s+(\d+)$", prev)
                assert m and int(m.group(1)) >= 4, f"{name}: '{line}' after '{prev}'"
    assert n > 0, "no global -> LDS DMA found in the GEMM"


def test_no_packed_fp32_valu(asm):
    bad = re.compile(r"^v_pk_(add|mul|fma|mov)_f32$")
    for name, text in asm.items():
        hits = [line for line, op in _instructions(text) if bad.match(op)]
        assert not hits, f"{name}: {hits[:3]}"


def _kernel_blocks(text, name):
    """The basic blocks of one kernel's body: (has an MFMA, touches scratch)."""
    a = text.index(name + ":")
    b = text.index(".Lfunc_end", a)
    blocks = [[False, False]]
    for line in text[a:b].splitlines()[1:]:
        t = line.strip()
        if re.match(r"^\.LBB\d+_\d+:", t):
            blocks.append([False, False])
        elif t.startswith("v_mfma"):
            blocks[-1][0] = True
        elif t.startswith("scratch_") or t.startswith("buffer_") and "scratch" in t:
            blocks[-1][1] = True
    return blocks


def test_gemm_kernels_do_not_spill(asm):
    text = asm["gemm.hip"]
    kernels = re.findall(r"\.name:\s+(\S*k_grouped_gemm\S*)\s*\n(?:.*\n)*?\s+\.private_segment_fixed_size:\s+(\d+)", text)
    assert kernels, "no grouped-GEMM kernel metadata found"
    for k, scratch in kernels:
        routed = "ELb1E" in k
        assert int(scratch) <= (16 if routed else 0), f"{k} uses {scratch} bytes of scratch"
        blocks = _kernel_blocks(text, k)
        assert any(m for m, _ in blocks), f"{k}: no MFMA found"
        assert not any(m and sc for m, sc in blocks), f"{k} touches scratch in an MFMA block"
