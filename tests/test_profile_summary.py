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


ACT = _g(128, 128, 1, 1, 6, 4).replace("DF16bDF16b", "N4gmlp4e4m3EDF16b")     # e4m3 up projection
DOWN8 = _g(256, 256, 1, 1, 0, 4).replace("DF16bDF16b", "N4gmlp4e4m3EDF16b")
QUANT = "_ZN4gmlp12_GLOBAL__N_116quantize8_kernelEPKvlPhPKfi"
ABSMAX = "_ZN4gmlp12_GLOBAL__N_119absmax8_part_kernelEPKvlPf"
DACT8 = _g(128, 128, 1, 1, 7, 4).replace("DF16bDF16b", "N4gmlp3f8gEDF16b")
T2D = "_ZN4gmlp12_GLOBAL__N_114quant2d_kernelEPKvlllPhlPKfiiPhl"
DW8 = _g(256, 256, 0, 0, 0, 4).replace("DF16bDF16b", "N4gmlp3f8gEDF16b")   # MN-major operands
DX8 = _g(256, 256, 1, 1, 1, 4).replace("DF16bDF16b", "N4gmlp3f8gEf")


def test_operand_preparation_joins_the_next_gemm():
    # fp8 step: per-tensor quantize before the up projection, the 2-D dout quantize before the
    # d-activation; the weight-gradient products read the row-major codes directly
    step = [ABSMAX, QUANT, ACT, DOWN8, T2D, DACT8, DW8, DX8, RED, DW8]
    names = step + step + [ABSMAX]
    steps = ps._per_step([(i, n, 1.0) for i, n in enumerate(names)], ps.STAGE_ORDER_GATED)
    assert len(steps) == 2
    for s in steps:
        assert [len(s[st]) for st in ps.STAGE_ORDER_GATED] == [3, 1, 2, 1, 2, 1]
        assert [ps.short_name(n) for n, _ in s["up"]] == ["absmax8_part", "quantize8", "gemm<e4m3,NT,128x128,4w,F8ACT>"]
        assert ps.short_name(s["dx"][-1][0]) == "splitk_reduce"
    assert ps.short_name(DACT8) == "gemm<e5m2xe4m3,NT,128x128,4w,F8DACT>"
    assert ps.short_name(DW8) == "gemm<e5m2xe4m3,TN,256x256,4w,STORE>"


def test_recompute_gemm_is_a_stage_not_a_new_step():
    step = [UP, DOWN, RED, UP, DACT_A, DW, DX, RED, DW]
    names = step + step
    disp = [(i, n, 1.0) for i, n in enumerate(names)]
    steps = ps._per_step(disp, ps.STAGE_ORDER_RECOMPUTE)
    assert len(steps) == 2
    assert [len(steps[0][st]) for st in ps.STAGE_ORDER_RECOMPUTE] == [1, 2, 1, 1, 1, 2, 1]
    # without the recompute stage the same launches read as one up projection per forward and
    # per backward, and no step is whole
    assert ps._per_step(disp, ps.STAGE_ORDER_GATED) == []


GROUP = "_ZN4gmlp21gemm_dma_group_kernelIDF16bLi256ELi256ELi8EDF16bLb1ELb0ELi0EfLb0ELb0ELi0EEEvNS_9GemmGroupE"
GROUP_DEM = ("void gmlp::gemm_dma_group_kernel<__bf16, 256, 256, 8, __bf16, true, false, 0, __bf16, false, false, 0>"
             "(gmlp::GemmGroup)")
GROUP_DACT = "_ZN4gmlp21gemm_dma_group_kernelIDF16bLi256ELi256ELi8EDF16bLb1ELb0ELi4EDF16bLb0ELb0ELi0EEEvNS_9GemmGroupE"


def test_grouped_backward_launch_is_one_stage():
    # dx and the weight gradients as one launch: the stage order loses dw_down/dx/dw_up for one
    # bwd_gemms stage, with and without the recompute stage
    step = [UP, DOWN, RED, DACT_A, DACT_B, GROUP]
    names = [FILL] + step + step + step[:3]
    disp = [(i, n, 1.0) for i, n in enumerate(names)]
    order = ps.grouped_order(ps.STAGE_ORDER_GATED, names)
    assert order == ["up", "down", "dact", "bwd_gemms"]
    steps = ps._per_step(disp, order)
    assert len(steps) == 2
    assert [len(steps[0][st]) for st in order] == [1, 2, 2, 1]
    assert ps.grouped_order(ps.STAGE_ORDER_RECOMPUTE, names) == ["up", "down", "recompute", "dact", "bwd_gemms"]
    assert ps.grouped_order(ps.STAGE_ORDER_GATED, [UP, DOWN]) == ps.STAGE_ORDER_GATED
    assert ps.short_name(GROUP) == "gemm_group<bf16,NN:STORE+TN:STORE,256x256,8w,f32 dW out>"
    assert ps.short_name(GROUP_DEM) == "gemm_group<bf16,NN:STORE+TN:STORE,256x256,8w>"
    assert ps.short_name(GROUP_DACT) == "gemm_group<bf16,NN:DGATED+TN:STORE,256x256,8w>"


def test_dact_group_holds_dw_down():
    # with the activation kept by the forward: the d-activation GEMM with dW_down, then dx with
    # dW_gate/dW_up; and the d-activation group alone (dx and dW_gate/dW_up separate)
    step = [UP, DOWN, RED, GROUP_DACT, GROUP]
    names = step + step
    order = ps.grouped_order(ps.STAGE_ORDER_GATED, names)
    assert order == ["up", "down", "dact", "bwd_gemms"]
    steps = ps._per_step([(i, n, 1.0) for i, n in enumerate(names)], order)
    assert len(steps) == 2 and [len(steps[0][st]) for st in order] == [1, 2, 1, 1]
    step = [UP, DOWN, RED, GROUP_DACT, DX, RED, DW]
    names = step + step
    order = ps.grouped_order(ps.STAGE_ORDER_GATED, names)
    assert order == ["up", "down", "dact", "dx", "dw_up"]
    steps = ps._per_step([(i, n, 1.0) for i, n in enumerate(names)], order)
    assert len(steps) == 2 and [len(steps[0][st]) for st in order] == [1, 2, 1, 2, 1]


STORE_NT, PART_NT = _g(256, 256, 1, 1, 0), _g(256, 256, 1, 1, 1).replace("DF16bDF16b", "DF16bf")
STORE_NN, PART_NN = _g(256, 256, 1, 0, 0), _g(256, 256, 1, 0, 1).replace("DF16bDF16b", "DF16bf")
ACT16, DACT16 = _g(256, 256, 1, 1, 3), _g(256, 256, 1, 0, 5)
DW_TN = _g(256, 256, 0, 0, 1).replace("DF16bDF16b", "DF16bf")


def test_rows_split_store_gemm_is_one_stage():
    # the GPT-shape ReLU^2 step: the down projection and dx each cut along M (a store launch,
    # then a split-K launch and its reduce); the weight gradients split-K in another layout
    step = [ACT16, STORE_NT, PART_NT, RED, DACT16, DW_TN, RED, STORE_NN, PART_NN, RED, DW_TN, RED]
    names = step + step
    steps = ps._per_step([(i, n, 1.0) for i, n in enumerate(names)], ps.STAGE_ORDER_GATED)
    assert len(steps) == 2
    assert [len(steps[0][st]) for st in ps.STAGE_ORDER_GATED] == [1, 3, 1, 2, 3, 2]


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    """The kernel-source hash that marks a profile current covers the code, not its comments or
    blank lines: a comment edit keeps it, a code edit changes it."""
    d = tmp_path / "csrc"
    d.mkdir()
    src = "// header\nint f(int x) {  /* note */\n  return x + 1;  // inc\n}\n"
    (d / "k.hip").write_text(src)
    monkeypatch.setattr(ps, "_HERE", str(tmp_path))
    h0 = ps.kernel_sources_sha256()
    (d / "k.hip").write_text("// header, reworded\n\nint f(int x) {  /* another\n note */\n  return x + 1;\n}\n")
    assert ps.kernel_sources_sha256() == h0
    (d / "k.hip").write_text(src.replace("x + 1", "x + 2"))
    assert ps.kernel_sources_sha256() != h0
    assert ps.code_text("a; // c\n/* b\n c */ d;\n\n") == "a;\n d;"
