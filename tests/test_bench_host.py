"""Host-side logic of bench.py: the byte model, the counter-summary lookup and
the one-GPU guard.  No GPU is touched."""
import os

import numpy as np
import pytest

import bench
from linear_attention_recurrent_gated_amd import workloads as W


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_byte_model_gdn_bf16_by_hand():
    # GDN, d = 128, bf16 inputs: q, k, v (3 * 128 * 2 B), scalar decay and beta (4 B each)
    wl = W.WORKLOADS[2]
    assert (wl.variant, wl.d_k, wl.d_v, wl.dtype) == (W.GDN, 128, 128, "bf16")
    m = bench.byte_model(wl)
    assert m["St"] == 65536
    assert m["In"] == 3 * 256 + 8
    assert m["E"] == 2 * 256 + 8
    assert m["E_af"] == 256 + 512 + 4
    assert bench.eager_bytes(m) == 2 * 65536 + 776 + 512 + 4
    # empty log: read S0 and the inputs, append one entry, write o, fill counter in and out
    assert bench.log_step_bytes(m, 0) == 65536 + 776 + 520 + 512 + 8
    # three logged entries: their payload plus the R columns (3 packed + 3 new, fp32)
    assert bench.log_step_bytes(m, 3) == 65536 + 3 * 520 + 776 + 520 + 512 + 8 + 4 * 6
    # a step that merges in place writes the base and appends nothing
    assert bench.log_step_bytes(m, 3, merges=True) == 2 * 65536 + 3 * 520 + 776 + 512 + 8 + 4 * 3


def test_byte_model_kda_and_gated_widths():
    kda, gated = bench.byte_model(W.WORKLOADS[3]), bench.byte_model(W.WORKLOADS[6])
    # channel-wise decay: a d_k vector of fp32 log-decays per step
    assert kda["In"] == 3 * 256 + 4 * 128 + 4
    # gated form: erase gate (d_k) and write gate (d_v) instead of one beta
    assert gated["In"] == 3 * 256 + 4 * 128 + 4 * 256
    assert bench.form_model(gated, "af")["R"] == 0


def _write_summary(root, kernel, workload, src, traffic, log_len=None):
    d = os.path.join(root, "profiles")
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, f"{kernel}.{workload}.counters.md"), "w") as f:
        f.write(f"# {kernel}\n\n- traffic_bytes_per_launch: {traffic}\n")
        if log_len is not None:
            f.write(f"- log_len: {log_len}\n")
        f.write(f"- source_sha256_16: `{src}`\n")


def test_counter_traffic_matches_sources_and_log_len(tmp_path, monkeypatch):
    csrc = tmp_path / "linear_attention_recurrent_gated_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in ("dl_step_af.hip", "dl_step.hip", "dl_merge.hip", "dl_common.hpp", "dl_abi.hip"):
        (csrc / name).write_text(f"{name} v1\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    _write_summary(str(tmp_path), "af_step_kernel", "wl", bench.source_hash("af_step_kernel"), 1234, log_len=16)
    _write_summary(str(tmp_path), "eager_step_kernel", "wl", bench.source_hash("eager_step_kernel"), 99)
    _write_summary(str(tmp_path), "merge_wy_kernel", "wl", bench.source_hash("merge_wy_kernel"), 7)
    assert bench.counter_traffic("af_step_kernel", "wl", 16) == 1234.0
    assert bench.counter_traffic("af_step_kernel", "wl", 8) is None      # taken at another L
    assert bench.counter_traffic("eager_step_kernel", "wl", 8) == 99.0   # no log, any L
    assert bench.counter_traffic("missing_kernel", "wl", 16) is None
    # a change to one kernel's file voids that kernel's counters only
    (csrc / "dl_merge.hip").write_text("dl_merge.hip v2\n")
    assert bench.counter_traffic("merge_wy_kernel", "wl") is None
    assert bench.counter_traffic("af_step_kernel", "wl", 16) == 1234.0
    assert bench.counter_traffic("eager_step_kernel", "wl") == 99.0
    # the step kernels' own file
    (csrc / "dl_step_af.hip").write_text("dl_step_af.hip v2\n")
    assert bench.counter_traffic("af_step_kernel", "wl", 16) is None
    assert bench.counter_traffic("eager_step_kernel", "wl") == 99.0
    # shared sources void every summary
    (csrc / "dl_common.hpp").write_text("dl_common.hpp v2\n")
    assert bench.counter_traffic("eager_step_kernel", "wl") is None


def test_committed_summaries_name_their_kernels_sources():
    """Every committed summary carries the hash of the sources behind its
    kernel (so bench.py reports its traffic), as long as those are unchanged."""
    import glob
    for f in sorted(glob.glob(os.path.join(os.path.dirname(bench.__file__), "profiles", "*.md"))):
        kernel = os.path.basename(f).split(".")[0]
        assert kernel in bench.KERNEL_SOURCES, f
        with open(f) as fh:
            hashes = {ln.split("`")[1] for ln in fh if ln.startswith("- source_sha256_16:")}
        assert len(hashes) == 1, f


@pytest.mark.parametrize("cfg", sorted(W.WORKLOADS))
def test_log_step_bytes_grow_with_fill(cfg):
    m = bench.byte_model(W.WORKLOADS[cfg])
    for path in ("log", "af"):
        fm = bench.form_model(m, path)
        b = [bench.log_step_bytes(fm, c) for c in range(8)]
        assert all(x < y for x, y in zip(b, b[1:]))


@pytest.mark.parametrize("spread", [False, True])
@pytest.mark.parametrize("n", [1, 3, 8, 17, 255])
def test_merging_order_is_a_permutation(n, spread):
    rng = np.random.default_rng(n)
    merging = np.sort(rng.choice(256, n, replace=False))
    order = bench.merging_order(256, merging, spread)
    assert sorted(order.tolist()) == list(range(256))
    pos = np.array([int(np.nonzero(order == u)[0][0]) for u in merging])
    rest = order[~np.isin(order, merging)]
    assert np.all(np.diff(rest) > 0)                        # the others keep their order
    if not spread:
        assert np.array_equal(np.sort(pos), np.arange(n))   # merging units first
    else:
        gap = (256 - n) // n
        assert np.array_equal(pos, np.arange(n) * (gap + 1))  # evenly spaced


def test_suggested_log_lens_of_the_workloads():
    """The log lengths the traffic model picks for the bench shapes."""
    from linear_attention_recurrent_gated_amd import binding as B
    cases = [((B.DL_GDN, 128, B.DL_LOG_FACTORS, 1), 13), ((B.DL_KDA, 128, B.DL_LOG_FACTORS, 1), 10),
             ((B.DL_RWKV6, 64, B.DL_LOG_WY, 1), 8), ((B.DL_RWKV6, 64, B.DL_LOG_WY, 0), 11)]
    for (variant, d, form, fuse), L in cases:
        got, _ = B.dl_suggest_log_len(B.DlDesc(variant, 1, 1, d, d, 0, B.DL_BF16, fuse, form))
        assert got == L, (variant, form, fuse, got)


# The measurement plan's table of algorithmic bytes per state update (eager,
# and DeltaLog averaged over a log period with the merge amortised).
SURVEY_BYTES = [
    (1, 8, 33_800, 24_372), (2, 16, 132_360, 79_956),
    (3, 1, 132_868, 200_460), (3, 4, 132_868, 103_698), (3, 8, 132_868, 89_370),
    (3, 16, 132_868, 85_290), (3, 32, 132_868, 89_418), (3, 64, 132_868, 103_818),
    (4, 32, 132_360, 80_020), (5, 32, 33_664, 27_264),
]


@pytest.mark.parametrize("cfg,L,eager,period", SURVEY_BYTES)
def test_update_bytes_match_the_plan_table(cfg, L, eager, period):
    m = bench.byte_model(W.WORKLOADS[cfg])
    assert bench.update_bytes(m, L, "eager") == eager
    assert bench.update_bytes(m, L, "period") == pytest.approx(period, abs=0.5)
    # the step share leaves out exactly the amortised merge
    merge = (2 * m["St"] + L * m["E"]) / L
    assert bench.update_bytes(m, L, "step") == pytest.approx(period - merge)


@pytest.mark.parametrize("cfg,L,reduction", [(1, 8, 5.9), (2, 16, 12.9), (4, 32, 21.4), (5, 32, 13.0)])
def test_write_reduction_model(cfg, L, reduction):
    m = bench.byte_model(W.WORKLOADS[cfg])
    r = bench.write_bytes(m, L, "eager") / bench.write_bytes(m, L, "log")
    assert r == pytest.approx(reduction, abs=0.05)


def test_warmup_rounds_to_whole_periods_only_when_logs_fill_together():
    assert bench.warmup_steps(W.WORKLOADS[2], 16, 5) == 16
    assert bench.warmup_steps(W.WORKLOADS[2], 16, 32) == 32
    assert bench.warmup_steps(W.WORKLOADS[2], 16, None) == 32
    assert bench.warmup_steps(W.WORKLOADS[4], 32, 5) == 5          # ragged: any window
    assert bench.warmup_steps(W.WORKLOADS[2], 16, 0) == 0


def test_default_workload_is_the_largest():
    args = bench.parse_args([])
    wl = W.WORKLOADS[args.config]
    assert wl.name == "gdn-b256-l8-h32-d128-ragged"
    states = wl.units_total * wl.heads * wl.d_k * wl.d_v * 4
    assert states == 4 * 2**30 and all(
        w.units_total * w.heads * w.d_k * w.d_v <= wl.units_total * wl.heads * wl.d_k * wl.d_v
        for w in W.WORKLOADS.values())


@pytest.mark.parametrize("policy", bench.ORDERS)
def test_row_order_policies(policy):
    rng = np.random.default_rng(5)
    L = 32
    fills = rng.integers(0, L, size=256)
    order = bench.row_order(policy, fills, L)
    if policy == "natural":
        assert order is None
        return
    assert sorted(order.tolist()) == list(range(256))
    merging = np.nonzero(fills == L - 1)[0]
    pos = np.argsort(order)[merging]                       # where the merging rows go
    if policy in ("first", "lpt"):
        assert np.array_equal(np.sort(pos), np.arange(len(merging)))
    if policy == "lpt":
        assert np.all(np.diff(fills[order]) <= 0)
    # nothing to order when every row has the same work
    assert bench.row_order(policy, np.zeros(8, dtype=np.int64), L) is None
    assert bench.row_order(policy, np.full(8, L - 1), L) is None
    # with no row merging, the orders built around merging rows keep the
    # batch order and longest work first still sorts by log length
    few = np.array([3, 0, 7, 7, 1, 5, 0, 2])
    if policy in ("lpt", "auto"):
        assert np.array_equal(bench.row_order(policy, few, L), [2, 3, 5, 0, 7, 4, 1, 6])
    else:
        assert bench.row_order(policy, few, L) is None


def test_row_order_auto():
    """The default order: longest work first, for both log forms."""
    rng = np.random.default_rng(7)
    L = 32
    fills = rng.integers(0, L, size=256)
    assert np.array_equal(bench.row_order("auto", fills, L),
                          bench.row_order("lpt", fills, L))
