"""Host-side checks of the benchmark's cost model and counter summaries."""
from fine_grained_mixture_amd import profiling
from fine_grained_mixture_amd.inputs import SHAPES


def _summary(tmp_path, digest):
    p = tmp_path / "t.md"
    p.write_text(f"kernel-sources-sha256: {digest}\n\n"
                 "| kernel | launches | read MB | write MB | HBM MB | algorithmic MB | r |\n"
                 "|---|---|---|---|---|---|---|\n"
                 "| dxt | 3 | 400.0 | 400.0 | 800.5 | 738.2 | 1.08 |\n")
    return p


def test_traffic_only_for_current_sources(tmp_path):
    cur = profiling.kernel_sources_sha256()
    assert profiling.read_traffic(str(_summary(tmp_path, cur)), "dxt") == 800_500_000
    assert profiling.read_traffic(str(_summary(tmp_path, cur)), "dw1") is None
    stale = ("0" if cur[0] != "0" else "1") + cur[1:]
    assert profiling.read_traffic(str(_summary(tmp_path, stale)), "dxt") is None
    assert profiling.read_traffic(str(tmp_path / "missing.md"), "dxt") is None


def test_kernel_model_flops_sum_to_layer_flops():
    # the six GEMMs carry 18 S n d FLOPs; the aggregations add 3 S d
    sh = SHAPES["7b"]
    S = sh.T * sh.K
    gemm = sum(profiling.kernel_model(k, sh, S)[0]
               for k in ("up_swiglu", "down", "dh", "dxt", "dw1", "dw2"))
    assert gemm == 18 * S * sh.n * sh.d == sh.flops
    assert profiling.kernel_model("route_topk", sh, S) is None


def test_intensity_and_saved_bytes_agree_with_the_oracle():
    # the benchmark's helpers and the oracle's are written independently
    from oracle import moe_oracle as orc
    for T, d, n, K, E in [(16384, 1536, 256, 8, 128), (16384, 1024, 512, 2, 32),
                          (8192, 2048, 384, 8, 512)]:
        assert abs(profiling.arithmetic_intensity(T, d, n, K, E)
                   - orc.arithmetic_intensity(T, d, n, K, E)) < 1e-9
        assert profiling.activation_bytes(T, d, n, K, T * K)["minimal"] == \
            orc.cached_activation_bytes(T, d, K, n)


def test_weight_bytes_follow_the_experts_with_slots():
    # the GEMMs read the weights of the E_act experts with slots only; the
    # weight-gradient kernels write the gradients of all E experts (zero
    # tiles for the rest), whatever E_act is
    sh = SHAPES["high_sparsity"]
    S, es = 64384, 2
    w1, w2 = sh.d * 2 * sh.n * es, sh.n * sh.d * es
    for k in ("dw1", "dw2"):
        assert profiling.kernel_model(k, sh, S, E_act=50) == profiling.kernel_model(k, sh, S)
    for k, w in (("up_swiglu", w1), ("dxt", w1), ("down", w2), ("dh", w2)):
        full = profiling.kernel_model(k, sh, S)[1]
        assert full - profiling.kernel_model(k, sh, S, E_act=50)[1] == (sh.E - 50) * w


def test_mfma_table_from_counters(tmp_path):
    # two dispatches of the up-projection: 2 s of 1e9 busy cycles over
    # 8 x 1e9 GRBM cycles (1e9 per XCD): 1 GHz, and 1e9 / (1e9 x 1024) busy
    hdr = ("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,"
           "End_Timestamp\n")
    lines = []
    for i in (1, 2):
        for c, v in (("SQ_VALU_MFMA_BUSY_CYCLES", 512e9), ("GRBM_GUI_ACTIVE", 8e9)):
            lines.append(f'{i},"void moe::k_up_swiglu<cfg>(...)",{c},{v},0,1000000000\n')
    p = tmp_path / "c.csv"
    p.write_text(hdr + "".join(lines))
    (n, dur, busy, grbm), = profiling.mfma_table(str(p)).values()
    assert n == 2 and dur == 1.0 and busy == 512e9 and grbm == 8e9
    assert busy / (grbm / profiling.NUM_XCD * profiling.NUM_SIMD) == 0.5


def test_pipeline_summary_from_counters(tmp_path):
    # one dispatch of the persistent dX-tilde over 1e6 cycles per XCD, its
    # counters split over two runs: 2.56e7 L2 reads of 500 cycles each is
    # 0.1 reads per CU per cycle and 50 in flight; 3 hits per miss
    hdr = ("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,"
           "End_Timestamp\n")
    cu_cyc = 1e6 * 256
    runs = [(("TCP_TCC_READ_REQ_LATENCY_sum", 500 * 2.56e7), ("TCP_TCC_READ_REQ_sum", 2.56e7),
             ("TCP_PENDING_STALL_CYCLES_sum", 0.25 * cu_cyc), ("TA_BUSY_avr", 0.5e6),
             ("GRBM_GUI_ACTIVE", 8e6)),
            (("TD_TD_BUSY_sum", 0.75 * cu_cyc), ("TD_TC_STALL_sum", 0.4 * cu_cyc),
             ("TCC_HIT_sum", 3e6), ("TCC_MISS_sum", 1e6), ("TCC_EA0_RDREQ_LEVEL_sum", 9e8),
             ("TCC_EA0_RDREQ_sum", 1e6), ("GRBM_GUI_ACTIVE", 8e6))]
    paths = []
    for i, counters in enumerate(runs):
        p = tmp_path / f"p{i}.csv"
        p.write_text(hdr + "".join(
            f'1,"void moe::k_dxt_p<cfg>(...)",{c},{v},0,500000\n' for c, v in counters))
        paths.append(str(p))
    (label, (n, dur, v)), = profiling.pipeline_table(paths).items()
    assert label == "dxt" and n == 1 and dur == 5e-4

    class Args:
        csv = paths
        cmd = ["run 1", "run 2"]
    row = [l for l in profiling._pipeline_md(Args).splitlines() if l.startswith("| dxt |")]
    assert row == ["| dxt | 500.0 | 500 | 0.100 | 50 | 0.75 | 900 | 0.50 | 0.75 | 0.40 | 0.25 |"]


def test_twice_launched_kernels_split_by_launch_order(tmp_path):
    # with truncated names the two launches of the persistent weight-gradient
    # kernel (dW1, then dW2) and of the aggregation (O, then dX) are told
    # apart by their order in each step
    p = tmp_path / "run_kernel_trace.csv"
    rows = ["Dispatch_Id,Kernel_Name,Start_Timestamp,End_Timestamp"]
    seq = [("k_aggregate", 80), ("k_dw_p", 200), ("k_aggregate", 81), ("k_dw_p", 110)] * 2
    t = 0
    for i, (k, us) in enumerate(seq):
        rows.append(f"{i + 1},{k},{t},{t + us * 1000}")
        t += us * 1000 + 5000
    p.write_text("\n".join(rows) + "\n")
    split = profiling._split_twice(str(p))
    assert {k: (v[0], v[1]) for k, v in split.items()} == {
        "aggregate_O": ("k_aggregate", [80.0, 80.0]), "dw1": ("k_dw_p", [200.0, 200.0]),
        "aggregate_dX": ("k_aggregate", [81.0, 81.0]), "dw2": ("k_dw_p", [110.0, 110.0])}
    # full names carry the gathered operand in the template arguments
    assert profiling._base_name("k_dw_p<moe::TileCfg<unsigned short, 256>, true, false>(x)") == "k_dw1"
    assert profiling._base_name("k_dw_p<moe::TileCfg<unsigned short, 256>, false, true>(x)") == "k_dw2"
    assert profiling._base_name("k_dw_p") == "k_dw_p"
