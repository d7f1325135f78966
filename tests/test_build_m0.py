"""The inline-asm LDS copies set m0 themselves (dsa_internal.h); the build
checks the gfx950 device assembly of every source for any compiler use of
m0 outside those asm blocks.  CPU only (hipcc cross-compiles)."""

from long_context_lightning_amd import build


def test_scanner_flags_compiler_m0_and_accepts_asm_blocks():
    asm = "\n".join([
        "\ts_mov_b32 s4, 0",
        "\t;;#ASMSTART",
        "\ts_mov_b32 m0, s6",
        "\ts_nop 0",
        "\tglobal_load_lds_dwordx4 v1, s[2:3]",
        "\t;;#ASMEND",
        "\tv_movrels_b32 v0, v1",
        "\ts_mov_b32 m0, -1",
        "\tds_read_b32 v2, v3 ; m0 in a comment",
        "\tglobal_load_lds_dword v1, s[2:3]",
    ])
    bad = build.m0_violations(asm)
    assert [n for n, _ in bad] == [7, 8, 10]   # implicit m0 reader, explicit write, LDS copy outside asm


def test_no_compiler_m0_in_the_kernels():
    build.check_m0()
