"""bench.py's command-line contract that needs no GPU: more than one GPU is
refused with a message and a non-zero exit, before any device work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2",
                        "--steps", "1", "--warmup", "0"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_code_digest_ignores_comments_not_code(tmp_path):
    """The traffic figure is keyed to the attention code: a comment or layout
    edit keeps the digest, a change to the code or to a string literal does not."""
    import bench
    a = tmp_path / "a.hip"
    a.write_text('int f(int x) {  // one\n  return x + 1; /* two\n lines */ }\nconst char* s = "a//b";\n')
    b = tmp_path / "b.hip"
    b.write_text('int f(int x) {\n\n  return x + 1;   }  // other words\nconst char* s = "a//b";\n')
    c = tmp_path / "c.hip"
    c.write_text('int f(int x) { return x + 2; }\nconst char* s = "a//b";\n')
    d = tmp_path / "d.hip"
    d.write_text('int f(int x) { return x + 1; }\nconst char* s = "a/*b";\n')
    assert bench.code_digest(a) == bench.code_digest(b)
    assert bench.code_digest(a) != bench.code_digest(c)
    assert bench.code_digest(a) != bench.code_digest(d)


def _oracle_step(cfg, inp, tp):
    """The oracle's lists and its natural-order output (bf16 bits, round to
    nearest even) for every query block: what a correct GPU step returns."""
    from math import sqrt

    import numpy as np

    from oracle import svsa_oracle as orc
    N, Bk, nb, D = cfg.N, cfg.Bk, cfg.nb, cfg.head_dim
    slots, n = orc.block_layout(cfg.grid, cfg.tile, cfg.pad3d)
    qp, kp, vp = (orc.permute_fwd(x, cfg.grid, cfg.tile, cfg.pad3d) for x in (inp.q, inp.k, inp.v))
    S = orc.block_scores(orc.pool(qp, N, Bk, n), orc.pool(kp, N, Bk, n), 1 / sqrt(D))
    rp, ci = orc.block_mask(S, cfg.band, top_p=tp)
    out = np.zeros((cfg.batch, cfg.heads, N, D), np.uint16)
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            for i in range(nb):
                r = (b * cfg.heads + h) * nb + i
                o = orc.attention_rows(qp, kp, vp, b, h, i, ci[rp[r]: rp[r + 1]], N, Bk,
                                       1 / sqrt(D), n).astype(np.float32)
                u = o.view(np.uint32).astype(np.uint64)
                bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
                out[b, h, slots[i * Bk: i * Bk + int(n[i])]] = bits
    return rp, ci, out


def test_oracle_leg_reports_parity_of_a_correct_step_and_flags_a_wrong_list():
    """bench.py's oracle leg on the small config: given the oracle's own lists
    and bf16-rounded output it reports every row identical and errors within
    bf16 rounding; a list with one block swapped far from the threshold is a
    failing row."""
    import numpy as np

    import bench
    from svsa_synth import get_config, make_inputs
    cfg = get_config("small")
    inp = make_inputs(cfg, seed=0)
    tp = np.full(cfg.heads, 0.9, np.float32)
    rp, ci, out = _oracle_step(cfg, inp, tp)
    cpu, rep = bench.oracle_leg(cfg, inp, tp, None, rp, ci, out, 2.0, 1e9)
    assert rep["pass"] and rep["mask"]["identical"] == cfg.heads * cfg.nb
    assert rep["mask"]["failing"] == 0 and rep["mask"]["tolerated_near_threshold"] == 0
    assert rep["attention"]["query_blocks"] >= 4 * cfg.heads
    assert 0 < rep["attention"]["rel_l2"] < 3e-3 and rep["attention"]["max_abs"] < 1e-2
    assert cpu["kind"] == "oracle" and cpu["value"] > 0
    # drop one kept block (not in the band) of a row that keeps several
    r = next(r for r in range(cfg.heads * cfg.nb) if rp[r + 1] - rp[r] >= 3)
    i = r % cfg.nb
    row = [j for j in ci[rp[r]: rp[r + 1]] if abs(int(j) - i) >= 1]
    drop = row[0]
    ci2 = np.concatenate([ci[: rp[r]], [j for j in ci[rp[r]: rp[r + 1]] if j != drop],
                          ci[rp[r + 1]:]]).astype(ci.dtype)
    rp2 = rp.copy()
    rp2[r + 1:] -= 1
    _, rep2 = bench.oracle_leg(cfg, inp, tp, None, rp2, ci2, out, 0.5, 1e9)
    assert rep2["mask"]["failing"] == 1 and not rep2["pass"]
