"""bench.py helpers that run without a GPU."""

import bench

SMI = """GPU: 0
    POWER:
        SOCKET_POWER: 1332 W
        GFX_VOLTAGE: N/A
    CLOCK:
        GFX_0:
            CLK: 1910 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        GFX_1:
            CLK: 1841 MHz
            MIN_CLK: 500 MHz
        MEM_0:
            CLK: 2000 MHz
"""


def test_parse_amd_smi_power_and_gfx_clocks():
    power, clocks = bench.parse_smi(SMI)
    assert power == 1332.0
    assert clocks == [1910.0, 1841.0]            # memory clocks are not GFX clocks
    assert bench.parse_smi("") == (None, [])


def test_call_kernels_follow_the_workload():
    big = bench.call_kernels("rule-14b+meank-1m")
    small = bench.call_kernels("rule-8b+meank-256k")
    assert "topk_mw_pass*4" in big["kvs_topk_select_redirect[rule]"]
    assert small["kvs_topk_select_redirect[rule]"] == ["topk_wg_kernel<8>", "slotmap_kernel"]
    # the fold's workgroups per CU follow G: 3 at rule-8b (G = 4), 2 at rule-14b (G = 5)
    assert small["kvs_rule_score"][1].endswith("1024, 3>") and big["kvs_rule_score"][1].endswith("1024, 2>")
    assert big["kvs_meank_score"] == small["kvs_meank_score"]


def test_every_listed_kernel_has_profiled_traffic():
    """Each kernel bench.py attributes to a call appears, under that exact short name, in the
    committed HBM-traffic profile of the workload, so no call's traffic silently reads as null."""
    import json
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for wl in bench.WORKLOADS:
        with open(os.path.join(root, "profiles", f"hbm_traffic_all-kernels_{wl}.json")) as f:
            profiled = json.load(f)["kernels"]
        for call, kernels in bench.call_kernels(wl).items():
            for k in kernels:
                alts = [a.split("*")[0] for a in (k if isinstance(k, tuple) else (k,))]
                assert any(a in profiled for a in alts), (wl, call, alts)
