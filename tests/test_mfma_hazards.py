"""The compiled kernels read no matrix-core result before the hardware has
written it.

tests/mfma_hazards.py walks every control-flow path of each compiled kernel
from every MFMA and flags a VALU instruction or store that reads one of its
result registers after fewer wait states than measured on the MI355X (fp8
scaled product 20, bf16 product 12; tests/test_mfma_wait_states_gpu.py
measures them again).  The compiler allows 19 after the fp8 product on some
paths, so this is checked on the code as compiled, for every kernel of the
library.

The same compiled code is also checked for waits that hold the matrix cores
until the next tile's LDS-DMA loads have landed (mfma_hazards.prefetch_waits):
in a double-buffered tile loop such a wait turns the prefetch into a stall.
"""
import os
import subprocess
import tempfile

import pytest

import mfma_hazards as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "io_aware_softmax_fwd_amd", "csrc")
F8 = "v_mfma_scale_f32_32x32x64_f8f6f4 v[0:15], v[16:23], v[24:31], v[0:15], v32, v32"


def _kernel(body):
    return H.parse_kernels("_Zk:\n" + body + "\n.Lfunc_end0:\n")["_Zk"]


def test_checker_flags_a_read_one_wait_state_short():
    ins, labels = _kernel(F8 + "\ns_nop 15\ns_nop 2\nv_mov_b32 v40, v15\ns_endpgm")
    assert [(i, j, st) for i, j, st in H.check(ins, labels)] == [(0, 3, 19)]
    ins, labels = _kernel(F8 + "\ns_nop 15\ns_nop 3\nv_mov_b32 v40, v15\ns_endpgm")
    assert H.check(ins, labels) == []


def test_checker_follows_branches_and_register_writes():
    # the fall-through path has enough wait states, the branch target not
    body = "\n".join([F8, "s_cbranch_scc1 .LBB0_2", "s_nop 15", "s_nop 15", ".LBB0_2:",
                      "v_max3_f32 v40, v15, v14, v13", "s_endpgm"])
    ins, labels = _kernel(body)
    assert len(H.check(ins, labels)) == 1
    # a write to the register ends its tracking: the read sees the new value
    ins, labels = _kernel(F8 + "\nv_mov_b32 v15, 0\nv_mov_b32 v40, v15\ns_endpgm")
    assert H.check(ins, labels) == []
    # stores read their data operands
    ins, labels = _kernel(F8 + "\nglobal_store_dwordx4 v[40:41], v[12:15], off\ns_endpgm")
    assert len(H.check(ins, labels)) == 1
    # an accumulation into the same registers is forwarded, not a read
    ins, labels = _kernel(F8 + "\n" + F8 + "\ns_endpgm")
    assert H.check(ins, labels) == []


def test_checker_refuses_an_unmeasured_product():
    ins, labels = _kernel("v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]\ns_endpgm")
    with pytest.raises(KeyError):
        H.check(ins, labels)


def _assembly(src, out):
    from io_aware_softmax_fwd_amd import build as B
    cmd = [B.HIPCC, *[f for f in B.device_flags(src) if f not in ("-fPIC",)], "-I", B.INCLUDE, "-I", CSRC,
           "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


@pytest.fixture(scope="module")
def compiled():
    """{(source, kernel symbol): (instructions, labels)} of the library's
    three kernel sources, compiled to gfx950 assembly once."""
    from io_aware_softmax_fwd_amd import build as B
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    sources = ["fa_fwd_bf16.hip", "fa_bwd_bf16.hip", "fa_fp8.hip"]
    kernels = {}
    with tempfile.TemporaryDirectory() as tmp:
        running = [(s, os.path.join(tmp, s + ".s")) for s in sources]
        running = [(s, out, _assembly(s, out)) for s, out in running]
        for s, out, p in running:
            _, err = p.communicate()
            assert p.returncode == 0, "hipcc -S %s failed:\n%s" % (s, err)
            for name, parsed in H.parse_kernels(open(out).read()).items():
                kernels[(s, name)] = parsed
    return kernels


def test_compiled_kernels_have_no_early_result_reads(compiled):
    problems = []
    for (s, name), (ins, labels) in compiled.items():
        for i, j, st in H.check(ins, labels):
            problems.append("%s %s: '%s' read after %d wait states by '%s'"
                            % (s, name[:60], ins[i][:60], st, ins[j][:60]))
    assert len(compiled) >= 20
    assert not problems, "\n".join(problems)


DMA = "buffer_load_dwordx4 v1, s[4:7], 0 offen lds"
BF16 = "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]"


def test_prefetch_wait_checker():
    eight = "\n".join([BF16] * 8)
    # a full wait right after queuing the next tile, before the products
    ins, _ = _kernel("\n".join([DMA, "s_waitcnt vmcnt(0)", eight, "s_barrier", "s_endpgm"]))
    assert H.prefetch_waits(ins) == [(1, 8)]
    # the same wait after the products costs nothing
    ins, _ = _kernel("\n".join([DMA, eight, "s_waitcnt vmcnt(0)", "s_barrier", "s_endpgm"]))
    assert H.prefetch_waits(ins) == []
    # a wait that completes only an older load (loads complete in order)
    ins, _ = _kernel("\n".join(["buffer_load_dword v2, v3, s[4:7], 0 offen", DMA,
                                 "s_waitcnt vmcnt(1)", eight, "s_endpgm"]))
    assert H.prefetch_waits(ins) == []
    # ... but not a newer one queued after the DMA
    ins, _ = _kernel("\n".join([DMA, "buffer_load_dword v2, v3, s[4:7], 0 offen",
                                 "s_waitcnt vmcnt(0)", eight, "s_endpgm"]))
    assert H.prefetch_waits(ins) == [(2, 8)]
    # fewer products than the threshold before the barrier
    ins, _ = _kernel("\n".join([DMA, "s_waitcnt vmcnt(0)", BF16, "s_barrier", eight, "s_endpgm"]))
    assert H.prefetch_waits(ins) == []


# Double-buffered tile loops, which queue the next tile's K/V (or Q/dO) and
# then compute on the current one.  Left out: the forward for small grids
# (one K and one V slot per wave, refilled as soon as each is read, so its
# waits are the pipeline) and the causal d = 128 dK/dV kernel, whose two
# masked steps reload a few spilled registers from scratch (once per
# workgroup) and wait for them, loads queued before included.
_DOUBLE_BUFFERED = ("fwd_bf16_kernel", "fwd_fp8_kernel", "bwd_dq_kernel",
                    "bwd_dkdv_kernelILi64E", "bwd_dkdv_kernelILi128ELb0", "bwd_fused_kernel")


def test_tile_loops_do_not_wait_for_their_prefetch(compiled):
    checked, problems = 0, []
    for (s, name), (ins, _) in compiled.items():
        if not any(k in name for k in _DOUBLE_BUFFERED):
            continue
        checked += 1
        for i, n in H.prefetch_waits(ins):
            problems.append("%s %s: '%s' before %d products" % (s, name[:60], ins[i], n))
    assert checked >= 21
    assert not problems, "\n".join(problems)
