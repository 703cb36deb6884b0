"""Host logic of bench.py, on the CPU: the pair counts behind every credited FLOP figure,
the parity bookkeeping, the bf16 half-ulp bound, the one-GPU guard and the HBM-traffic
summary (write, then read back only while the forward sources are unchanged)."""

import os
import subprocess
import sys

import numpy as np
import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def brute_pairs(nq, nk, causal):
    return sum(1 for i in range(nq) for j in range(nk) if not causal or j <= i + (nk - nq))


@pytest.mark.parametrize("nq,nk", [(1, 1), (5, 5), (7, 3), (3, 7), (64, 100), (100, 64), (33, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_pairs_equal_brute_force(nq, nk, causal):
    assert bench.pairs(nq, nk, causal) == brute_pairs(nq, nk, causal)


def test_credited_flops_of_the_step_workloads():
    # causal N x N: N (N + 1) / 2 pairs per head
    assert bench.pairs(16384, 16384, True) == 16384 * 16385 // 2 == 134_225_920
    fwd = 4 * 128 * bench.pairs(16384, 16384, True) * 32
    bwd = 10 * 128 * bench.pairs(4096, 4096, True) * 2 * 16
    assert fwd == 2_199_157_473_280  # 2.1992 TFLOP
    assert abs(bwd / 1e9 - 343.69) < 0.01


def test_half_ulp_bf16_is_half_the_spacing():
    x = np.array([1.0, 1.5, 2.0, 3.99, -0.75, 1e-3, 300.0])
    e = np.floor(np.log2(np.abs(x)))
    spacing = 2.0 ** (e - 7)  # bf16 has 8 significant bits
    np.testing.assert_array_equal(bench._half_ulp_bf16(x), spacing / 2)
    assert bench._half_ulp_bf16(np.array([0.0]))[0] > 0


def test_parity_forward_bookkeeping():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((4, 8))
    lse_ref = rng.standard_normal(4)
    ok = bench._Parity("fwd")
    ok.fwd(ref + 5e-3, lse_ref + 5e-4, ref, lse_ref, False)
    assert ok.ok and ok.worst["o_max_abs"] == pytest.approx(5e-3)
    bad_o = bench._Parity("fwd")
    bad_o.fwd(ref + 2e-2, lse_ref, ref, lse_ref, False)
    assert not bad_o.ok
    bad_lse = bench._Parity("fwd")
    bad_lse.fwd(ref, lse_ref + 2e-3, ref, lse_ref, False)
    assert not bad_lse.ok
    nan = bench._Parity("fwd")
    o = ref.copy()
    o[1, 2] = np.nan
    nan.fwd(o, lse_ref, ref, lse_ref, False)
    assert not nan.ok
    # rows with no visible key: LSE -inf on both sides passes, on one side fails
    inf_ok = bench._Parity("fwd")
    l1, l2 = lse_ref.copy(), lse_ref.copy()
    l1[0] = l2[0] = -np.inf
    inf_ok.fwd(ref, l1, ref, l2, False)
    assert inf_ok.ok
    inf_bad = bench._Parity("fwd")
    inf_bad.fwd(ref, l1, ref, lse_ref, False)
    assert not inf_bad.ok


def test_parity_gradient_bookkeeping():
    rng = np.random.default_rng(1)
    ref = [rng.standard_normal((3, 5)) for _ in range(3)]
    good = bench._Parity("bwd")
    good.grads([r * (1 + 1e-3) for r in ref], ref)
    assert good.ok
    bad = bench._Parity("bwd")
    bad.grads([ref[0], ref[1] * 1.05, ref[2]], ref)
    assert not bad.ok and bad.worst["dk_rel_l2"] == pytest.approx(0.05)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _counter_csv(path, counter, fwd_kib, copy_kib):
    rows = ["Kernel_Name,Grid_Size,Counter_Name,Counter_Value"]
    for _ in range(3):
        rows.append(f'"void fa::(anonymous namespace)::fwd_bf16_kernel<128, false, false, false>(fa::FwdParams)",'
                    f"{bench.FWD_GRID_THREADS},{counter},{fwd_kib}")
        rows.append(f'"void fa::(anonymous namespace)::fwd_bf16_kernel<128, false, false, false>(fa::FwdParams)",'
                    f"262144,{counter},1.0")  # another grid: not the timed launch
    rows.append(f'"__amd_rocclr_copyBuffer",8388608,{counter},{copy_kib}')
    open(path, "w").write("\n".join(rows) + "\n")


def test_traffic_summary_round_trip(tmp_path):
    f, w, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "traffic.md"
    # FETCH_SIZE reads half the copy's bytes (scale 2), WRITE_SIZE all of them (scale 1)
    _counter_csv(f, "FETCH_SIZE", 200000.0, bench.COPY_BYTES / 1024 / 2)
    _counter_csv(w, "WRITE_SIZE", 100000.0, bench.COPY_BYTES / 1024)
    bench.write_traffic_summary(str(f), str(w), str(out))
    expect = int(round((200000.0 * 2 + 100000.0) * 1024))
    assert bench.traffic_for(bench.FWD_KERNEL_SRCS, str(out)) == expect
    # the summary is ignored once the forward's sources no longer hash to its line
    text = out.read_text()
    stale = tmp_path / "stale.md"
    stale.write_text(text.replace(bench.sources_sha256(bench.FWD_KERNEL_SRCS), "0" * 64))
    assert bench.traffic_for(bench.FWD_KERNEL_SRCS, str(stale)) is None
    assert bench.traffic_for(bench.FWD_KERNEL_SRCS, str(tmp_path / "missing.md")) is None



def test_source_hash_ignores_comments_only(tmp_path):
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // one more\n}\n")
    b.write_text("// header\nint f(int x) {\n\n  return x + 1;  /* changed comment */\n}\n")
    c.write_text("int f(int x) {\n  return x + 2;  // one more\n}\n")
    assert bench.sources_sha256([str(a)]) == bench.sources_sha256([str(b)])
    assert bench.sources_sha256([str(a)]) != bench.sources_sha256([str(c)])
