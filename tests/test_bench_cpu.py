"""Command-line checks of bench.py that need no GPU: more than one GPU is
refused with a message before anything touches a device, and the options
parse."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_help_lists_the_timing_switches():
    r = _run("--help")
    assert r.returncode == 0
    for opt in ("--steps", "--warmup", "--no-graph", "--no-overlap", "--no-cpu-baseline",
                "--no-other-configs", "--copy-calibration-mib"):
        assert opt in r.stdout


def test_dist_and_host_info():
    sys.path.insert(0, ROOT)
    import bench
    d = bench.dist([1.0, 2.0, 3.0, 4.0, 5.0])
    assert d["median"] == 3.0 and d["n"] == 5 and d["p10"] == 1.4 and d["p90"] == 4.6
    h = bench.host_info()
    assert h["nproc"] == os.cpu_count() and h["affinity_cpus"] >= 1


def test_oracle_check_scores_a_sample_made_by_the_oracle():
    """The bench's untimed check, fed the oracle's own mask (as bits) and its
    output rounded to bf16: no differing rows, errors within bf16 rounding; a
    flipped mask bit and a perturbed row are reported."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    from block_sparse_attention_softmax_amd.workloads import WORKLOADS, f64_to_bf16_bits, generate
    from oracle import sparge_oracle as O
    wl = WORKLOADS["tiny"]
    Q, K, V = generate(wl)
    m = O.predict_mask(Q, K, wl.block_q, wl.block_k, wl.k_frac, wl.p_mass, wl.scale)
    bits = O.kept_to_bits(m.kept)
    rows = []
    for h in range(wl.H):
        blocks = [0, 5, wl.n_q - 1]
        ref = O.masked_attention_head(*(O.bf16_to_f64(X[0, h]) for X in (Q, K, V)), m.kept[0, h],
                                      wl.block_q, wl.block_k, wl.scale, q_blocks=blocks)
        rows.append((h, blocks, f64_to_bf16_bits(ref[~np.isnan(ref[:, 0])])))
    smp = dict(name="tiny", wl=wl, inputs="tiny", k=wl.k_frac, p=wl.p_mass, alpha=None,
               bits=bits, rows=rows)
    r = bench.oracle_check([smp], {"tiny": (Q, K, V)})["tiny"]
    assert r["rows_differing_from_oracle"] == 0 and r["max_abs_err"] <= 2.0 ** -8 * 4
    bad_bits = bits.copy()
    bad_bits[0, 1, 3, 0] ^= 1
    bad_rows = [(h, b, x.copy()) for h, b, x in rows]
    bad_rows[0][2][0, 0] ^= 0x4000   # a large change of one element
    smp2 = dict(smp, bits=bad_bits, rows=bad_rows)
    r2 = bench.oracle_check([smp2], {"tiny": (Q, K, V)})["tiny"]
    assert r2["rows_differing_from_oracle"] == 1 and r2["max_abs_err"] > 0.1
