"""CPU checks of the build's assembly guards (no GPU needed)."""
from long_sequence_attention_amd import build


def test_dma_form_check_accepts_the_kernels_form_and_rejects_others():
    good = "\ts_nop 0\n\tglobal_load_lds_dwordx4 v[10:11], off\n"
    assert build._dma_hazards(good) == []
    # no wait state after the M0 write
    assert build._dma_hazards("\ts_mov_b32 m0, s4\n\tglobal_load_lds_dwordx4 v[10:11], off\n")
    # an SGPR base address (a VALU-written SGPR would need wait states the compiler cannot see)
    assert build._dma_hazards("\ts_nop 0\n\tglobal_load_lds_dwordx4 v10, s[4:5]\n")


def test_scratch_check_reads_the_metadata():
    meta = "amdhsa.kernels:\n  - .name: k1\n    .private_segment_fixed_size: 0\n  - .name: k2\n    .private_segment_fixed_size: 16\n"
    assert build._scratch_users(meta) == ["k2 (16 bytes per lane)"]
