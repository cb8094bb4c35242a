"""The build-time checks of the decode kernel's generated code, on small
hand-written instruction sequences: the inline-assembly QK accumulator chains
(nothing may touch an open chain's registers between its links), the
VALU -> assembly-MFMA operand hazard (the compiler inserts no wait states for
inline assembly), M0 used only by the direct-to-LDS load sequences, no
spill reload inside a per-tile step loop, and no compiler-inserted
vector-memory wait while tile loads are in flight."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "paged_mla_decode_02_amd"))
from asm_check import (check_m0, check_qk_chains, check_scratch_in_step_loops, check_valu_to_mfma,  # noqa: E402
                       check_waits_behind_tile_loads)

BF = "v_mfma_f32_32x32x16_bf16"
F8 = "v_mfma_f32_32x32x64_f8f6f4"


def chain(mnem, acc, out, a, b, links):
    """A chain of `links` products through v[acc], the last writing v[out]."""
    lines = [f"\t{mnem} v[{acc}:{acc + 15}], {a}, {b}, 0"]
    for _ in range(links - 2):
        lines.append(f"\t{mnem} v[{acc}:{acc + 15}], {a}, {b}, v[{acc}:{acc + 15}]")
    lines.append(f"\t{mnem} v[{out}:{out + 15}], {a}, {b}, v[{acc}:{acc + 15}]")
    lines += ["\ts_nop 7", "\ts_nop 5"]
    return lines


def test_clean_chains_of_both_kinds():
    asm = chain(BF, 100, 120, "v[0:3]", "v[4:7]", 36) + chain(F8, 140, 160, "v[0:7]", "v[8:15]", 9)
    chains, bad = check_qk_chains("\n".join(asm))
    assert chains == 2 and bad == []


def test_touching_an_open_accumulator_is_flagged():
    asm = chain(BF, 100, 120, "v[0:3]", "v[4:7]", 4)
    asm.insert(2, "\tv_mov_b32 v105, 0")          # between two links
    _, bad = check_qk_chains("\n".join(asm))
    assert len(bad) == 1 and "v_mov_b32 v105" in bad[0]


def test_moving_the_accumulator_mid_chain_is_flagged():
    asm = chain(F8, 100, 120, "v[0:7]", "v[8:15]", 4)
    asm[2] = f"\t{F8} v[100:115], v[0:7], v[8:15], v[40:55]"   # a link that reads another accumulator
    asm.insert(2, "\tv_mov_b32 v40, v100")
    _, bad = check_qk_chains("\n".join(asm))
    assert bad


def test_interleaved_chains():
    a = chain(BF, 100, 120, "v[0:3]", "v[4:7]", 3)
    b = chain(BF, 140, 160, "v[0:3]", "v[4:7]", 3)
    asm = [a[0], b[0], a[1], b[1], a[2], b[2]] + a[3:]
    chains, bad = check_qk_chains("\n".join(asm))
    assert chains == 2 and bad == []


@pytest.mark.parametrize("mnem,ops", [(BF, "v[0:3], v[4:7]"), (F8, "v[0:7], v[8:15]")])
def test_valu_write_right_before_an_operand_read(mnem, ops):
    asm = ["\tv_cvt_pk_bf16_f32 v5, v30, v31", f"\t{mnem} v[100:115], {ops}, 0"]
    assert len(check_valu_to_mfma("\n".join(asm))) == 1
    asm.insert(1, "\ts_nop 1")                    # two wait states
    assert check_valu_to_mfma("\n".join(asm)) == []
    asm = ["\tv_cvt_pk_bf16_f32 v5, v30, v31", "\tv_add_u32 v40, v41, v42", f"\t{mnem} v[100:115], {ops}, 0"]
    assert len(check_valu_to_mfma("\n".join(asm))) == 1   # one wait state is not enough
    asm = ["\tv_cvt_pk_bf16_f32 v50, v30, v31", f"\t{mnem} v[100:115], {ops}, 0"]
    assert check_valu_to_mfma("\n".join(asm)) == []       # an unrelated register


def test_m0_only_in_lds_load_sequences():
    ok = ["\ts_mov_b32 m0, s88", "\ts_nop 0", "\tglobal_load_lds_dwordx4 v[2:3], off"]
    assert check_m0("\n".join(ok)) == []
    for extra in ("\ts_mov_b32 m0, -1", "\tv_readlane_b32 s4, v1, m0", "\ts_sendmsg sendmsg(MSG_GS), m0"):
        assert len(check_m0("\n".join(ok + [extra]))) == 1
    # an M0 write whose load does not follow right away
    assert check_m0("\n".join(["\ts_mov_b32 m0, s3", "\tv_add_u32 v1, v2, v3", ok[2]]))


def kernel(body):
    return ["_Zkern:", *body, "\ts_endpgm"]


def test_scratch_in_step_loop_is_flagged():
    # the compiler's loop comments: an item loop BB0_0 around a step loop BB0_1
    step = [".LBB0_1:                ;   Parent Loop BB0_0 Depth=1",
            "                        ; =>  This Inner Loop Header: Depth=2",
            f"\t{BF} v[0:15], v[16:19], v[20:23], v[0:15]", "\tds_read_b128 v[16:19], v30",
            "\ts_cbranch_scc1 .LBB0_1"]
    head = [".LBB0_0:                ; =>This Loop Header: Depth=1"]
    tail = ["; %bb.2:                ;   in Loop: Header=BB0_0 Depth=1", "\ts_cbranch_scc0 .LBB0_0"]
    assert check_scratch_in_step_loops("\n".join(kernel(head + step + tail))) == []
    bad = step[:3] + ["\tscratch_load_dword v40, off, off offset:16"] + step[3:]
    assert len(check_scratch_in_step_loops("\n".join(kernel(head + bad + tail)))) == 1
    # a reload in the enclosing item loop, outside the step loop, is allowed
    outer = head + ["\tscratch_load_dword v40, off, off offset:16"] + step + tail
    assert check_scratch_in_step_loops("\n".join(kernel(outer))) == []
    # so is one in item-loop code that the layout places before the step loop
    # and reaches from its exit by a backward branch (no loop of its own)
    late = head + ["\ts_branch .LBB0_1",
                   ".LBB0_3:                ;   in Loop: Header=BB0_0 Depth=1",
                   f"\t{BF} v[0:15], v[16:19], v[20:23], v[0:15]",
                   "\tscratch_load_dword v40, off, off offset:16", "\ts_cbranch_scc0 .LBB0_0"] + \
        step[:4] + ["\ts_cbranch_scc1 .LBB0_1", "; %bb.4:                ;   in Loop: Header=BB0_0 Depth=1",
                    "\ts_branch .LBB0_3"]
    assert check_scratch_in_step_loops("\n".join(kernel(late))) == []
    # without loop comments the placement cannot be checked
    plain = [".LBB0_1:", f"\t{BF} v[0:15], v[16:19], v[20:23], v[0:15]", "\ts_cbranch_scc1 .LBB0_1"]
    assert len(check_scratch_in_step_loops("\n".join(kernel(plain)))) == 1


def test_compiler_wait_behind_tile_loads_is_flagged():
    def decode(flags, body):
        name = f"_ZN3mla12_GLOBAL__N_113decode_kernelI{flags}EEvNS_10DecodeArgsE"
        return "\n".join([f"{name}:"] + body + ["\ts_endpgm"])
    dma = [";;#ASMSTART", "\ts_mov_b32 m0, s4", "\ts_nop 0", "\tglobal_load_lds_dwordx4 v[2:3], off", ";;#ASMEND"]
    own_wait = [";;#ASMSTART", "\ts_waitcnt vmcnt(0)", ";;#ASMEND"]
    reload = ["\tscratch_load_dword v9, off, off offset:12", "\ts_waitcnt vmcnt(0)", "\tv_add_u32_e32 v1, v9, v1"]
    default = "Lb0ELb1ELb0ELb0E"
    # a reload after the kernel's own full wait is harmless
    assert check_waits_behind_tile_loads(decode(default, dma + own_wait + reload)) == []
    # between a tile load and the kernel's own wait it also waits for the tile
    assert len(check_waits_behind_tile_loads(decode(default, dma + reload + own_wait))) == 1
    # a partial wait of the kernel's own leaves loads in flight
    partial = [";;#ASMSTART", "\ts_waitcnt vmcnt(6)", ";;#ASMEND"]
    assert len(check_waits_behind_tile_loads(decode(default, dma + partial + reload))) == 1
    # the in-kernel merge is checked too; the fp8 PV products are not
    assert len(check_waits_behind_tile_loads(decode("Lb0ELb1ELb1ELb0E", dma + reload))) == 1
    assert check_waits_behind_tile_loads(decode("Lb0ELb1ELb0ELb1E", dma + reload)) == []


def test_built_kernel_passes_the_checks():
    path = os.path.join(ROOT, "paged_mla_decode_02_amd", "_build", "decode.gfx950.s")
    if not os.path.exists(path):
        pytest.skip("the library has not been built here")
    text = open(path).read()
    chains, bad = check_qk_chains(text)
    assert chains > 0 and bad == []
    assert check_valu_to_mfma(text) == []
    assert check_m0(text) == []
    assert check_scratch_in_step_loops(text) == []
    assert check_waits_behind_tile_loads(text) == []
