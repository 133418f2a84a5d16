"""Every read of a matrix-product result in the built kernels leaves the
product enough wait states (see isa_hazards.py).  Compiles the device code to
assembly on the host; needs hipcc, not a GPU."""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

from isa_hazards import check_text

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_05_amd", "csrc")
SOURCES = ["fa_fwd.hip", "fa_fwd_merge.hip", "fa_bwd.hip", "fa_decode.hip"]


def _device_asm(src: str, out_dir: str) -> str:
    from exact_attention_05_amd import build

    out = os.path.join(out_dir, src + ".s")
    flags = [f for f in build.compile_flags() if f != "-fPIC"]
    cmd = [build.hipcc(), *flags, *build.FILE_FLAGS.get(src, []), "-S", "--cuda-device-only",
           os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return f.read()


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    d = str(tmp_path_factory.mktemp("asm"))
    with cf.ThreadPoolExecutor(len(SOURCES)) as ex:
        texts = list(ex.map(lambda s: _device_asm(s, d), SOURCES))
    return dict(zip(SOURCES, texts))


@pytest.mark.parametrize("src", SOURCES)
def test_matrix_results_read_after_enough_wait_states(assembly, src):
    text = assembly[src]
    assert text.count("v_mfma") > 40, "no matrix products found: assembly not parsed?"
    bad = check_text(text)
    lines = [f"{k}: {v[:3]}" for k, v in bad.items()]
    assert not bad, "reads too close to a matrix product:\n" + "\n".join(lines)


# The checker itself, on hand-made fragments.
_FRAG = """_Zk:
	v_mfma_f32_32x32x2_f32 a[0:15], v0, v1, a[0:15]
{pad}
	v_accvgpr_read_b32 v2, a15
	s_endpgm
.Lfunc_end0:
"""


def test_checker_flags_an_early_read():
    assert check_text(_FRAG.format(pad="\ts_nop 3"))  # 4 wait states < 18
    assert not check_text(_FRAG.format(pad="\ts_nop 15\n\ts_nop 1"))  # 18
    # a read of a register the product does not write is fine
    assert not check_text(_FRAG.format(pad="").replace("a15", "a16"))


def test_checker_follows_branches_and_takes_the_shortest_path():
    frag = """_Zk:
	v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]
	s_cbranch_scc1 .LBB0_2
	s_nop 15
.LBB0_2:
	v_add_f32_e32 v30, v3, v31
	s_endpgm
.Lfunc_end0:
"""
    bad = check_text(frag)
    assert bad and list(bad.values())[0][0][3] == 1  # the taken branch skips the pad
    assert not check_text(frag.replace("s_cbranch_scc1 .LBB0_2", "s_nop 15"))


def test_checker_ignores_accumulation_chains():
    frag = """_Zk:
	v_mfma_f32_32x32x2_f32 a[0:15], v0, v1, a[0:15]
	v_mfma_f32_32x32x2_f32 a[0:15], v2, v3, a[0:15]
	s_endpgm
.Lfunc_end0:
"""
    assert not check_text(frag)


def test_checker_flags_a_vector_write_just_before_a_product():
    frag = """_Zk:
	v_xor_b32_e32 v20, s0, v20
{pad}
	v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0
	s_nop 15
	v_add_f32_e32 v30, v3, v31
	s_endpgm
.Lfunc_end0:
"""
    assert check_text(frag.format(pad=""))                 # 0 wait states < 2
    assert check_text(frag.format(pad="\ts_nop 0"))        # 1
    assert not check_text(frag.format(pad="\ts_nop 1"))    # 2
    # a load writing the operand is not a vector write (s_waitcnt covers it)
    assert not check_text(frag.format(pad="").replace("v_xor_b32_e32 v20, s0, v20", "ds_read_b128 v[20:23], v1"))
