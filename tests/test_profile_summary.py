"""Host logic of the profile summaries: splitting a dispatch list into steps and stages."""
from gated_mlp_gemms_amd import profile_summary as ps


def _g(bm, bn, ak, bk, epi, waves=8):
    return f"_ZN4gmlp15gemm_dma_kernelIDF16bDF16bLi{bm}ELi{bn}ELb{ak}ELb{bk}ELi{epi}ELi{waves}EEEvNS_8GemmArgsE"


UP = _g(256, 256, 1, 1, 2)
DOWN = "void gmlp::gemm_dma_kernel<bool _Accum, 256, 256, true, true, 1, 8>(gmlp::GemmArgs)"
RED = "_ZN4gmlp12_GLOBAL__N_120splitk_reduce_kernelIDF16bEEvPKfiiiPvS4_lifS3_S3_i"
DACT_A, DACT_B = _g(256, 256, 1, 0, 4), _g(256, 128, 1, 0, 4)
DW = _g(256, 256, 0, 0, 0)
DX = "void gmlp::gemm_dma_kernel<bool _Accum, 256, 256, true, false, 1, 8>(gmlp::GemmArgs)"
FILL = "void at::native::vectorized_elementwise_kernel<16, at::native::FillFunctor<unsigned char>>"


def _step(split_dact):
    seq = [UP, DOWN, RED, DACT_A] + ([DACT_B] if split_dact else []) + [DW, DX, RED, DW]
    return seq


def test_stages_with_and_without_the_column_split():
    names = [FILL] + _step(False) + [FILL] + _step(True) + _step(True)[:4]   # last step is cut short
    disp = [(i, n, float(i)) for i, n in enumerate(names)]
    steps = ps._per_step(disp, ps.STAGE_ORDER_GATED)
    assert len(steps) == 2
    for s, n_dact in zip(steps, (1, 2)):
        assert [len(s[st]) for st in ps.STAGE_ORDER_GATED] == [1, 2, n_dact, 1, 2, 1]
        assert all(ps.short_name(n).startswith("gemm") for n, _ in s["dact"])
    # the reduce joins the GEMM before it; the fill of another library is skipped
    assert ps.short_name(steps[0]["down"][1][0]) == "splitk_reduce"
    assert ps.short_name(DACT_B) == "gemm<bf16,NN,256x128,8w,DGATED>"
    assert ps.short_name(DW) == "gemm<bf16,TN,256x256,8w,STORE>"
