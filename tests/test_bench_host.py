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
    (csrc / "k.hip").write_text("kernel v1\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    src = bench.source_hash()
    _write_summary(str(tmp_path), "af_step_kernel", "wl", src, 1234, log_len=16)
    _write_summary(str(tmp_path), "eager_step_kernel", "wl", src, 99)
    assert bench.counter_traffic("af_step_kernel", "wl", 16) == 1234.0
    assert bench.counter_traffic("af_step_kernel", "wl", 8) is None      # taken at another L
    assert bench.counter_traffic("eager_step_kernel", "wl", 8) == 99.0   # no log, any L
    assert bench.counter_traffic("missing_kernel", "wl", 16) is None
    (csrc / "k.hip").write_text("kernel v2\n")                            # sources changed
    assert bench.counter_traffic("af_step_kernel", "wl", 16) is None


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
