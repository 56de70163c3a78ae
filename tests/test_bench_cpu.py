"""Host logic of bench.py: the closed-form work counts behind the roofline
figures (checked against the oracle's own counting and against brute-force
enumeration of the selections), the traffic-record gate, and the one-GPU
guard.  No GPU is touched."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from hierarchical_index_sparse_amd import datagen
from hierarchical_index_sparse_amd.workloads import WORKLOADS, Workload
from oracle import hisa_oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("B,m,k,L,nq", [(64, 8, 256, 4096, 4096), (16, 5, 40, 700, 300), (128, 64, 2048, 20000, 5)])
def test_per_query_counts_match_the_oracle(B, m, k, L, nq):
    w = Workload(name="c", batch=1, seq_len=L, n_q=nq, d_index=64, block=B, top_m=m, top_k=k, n_heads_q=1,
                 n_heads_kv=1)
    sb, st, kept = bench.per_query_counts(w)
    for i in range(0, nq, max(1, nq // 97)):
        t = w.query_pos(i)
        assert sb[i] + st[i] == orc.scored_items(t, B, m, k), (i, t)
        # kept = number of valid entries of the token list the oracle builds
        blk = np.arange(min(t // B + 1, m))  # which blocks does not change the count
        blk = np.concatenate([blk[:-1], [t // B]]) if t // B + 1 > m else blk
        assert kept[i] == min(orc.candidate_tokens(blk, t, B).size, k)


def test_three_level_counts_by_enumeration():
    # candidate blocks at level 2 = blocks j <= c of the kept super-blocks,
    # whichever super-blocks are kept; enumerate with the oracle's selection
    w = Workload(name="c3", batch=1, seq_len=3000, n_q=1, d_index=16, block=8, top_m=6, top_k=40, n_heads_q=1,
                 n_heads_kv=1, group=4, top_m2=5)
    inp = datagen.make_inputs(w, attention=False, q_range=2, centre_range=1, noise_range=1)
    S = orc.block_summary(inp["kI"][0], w.block)
    S2 = orc.super_summary(S, w.group)
    rng = np.random.default_rng(0)
    for t in sorted(set(rng.integers(0, w.seq_len, 60).tolist() + [0, 7, 31, 32, 159, 160, 2999])):
        scored_super, scored_blocks = bench.level1_counts(w, np.array([t]))
        c, C = t // w.block, t // (w.block * w.group)
        sup = orc.select_blocks(inp["qI"][0, 0], S2, t, w.block * w.group, w.top_m2)
        cand = [j for J in sup[sup >= 0] for j in range(J * w.group, J * w.group + w.group) if j <= c]
        assert scored_super[0] == (0 if C + 1 <= w.top_m2 else C - 1)
        assert scored_blocks[0] == (0 if len(cand) <= w.top_m else len(cand)), t


def test_head_work_counts():
    w = WORKLOADS["head_decode_512k"]
    work = bench.head_work(w)
    t = w.seq_len - 1
    c = t // w.block
    # scored chunk rows: per sequence and kv head, (c - 1) chunks x nL landmark rows
    rows = w.batch * w.n_heads_kv * (c - 1) * w.n_landmarks
    assert work["block_topm"]["bytes"] >= rows * w.head_dim * 2
    # attended tokens: every causal token of m chunks per head
    tokens = w.batch * w.n_heads_q * ((w.top_m - 1) * w.block + (t - c * w.block + 1))
    assert work["sparse_attn"]["flops"] == 4.0 * w.head_dim * tokens
    assert work["token_topk"]["bytes"] == 0.0


def test_kernel_work_splits_a_stage_in_two():
    # a scorer and its select hand over 4-byte scores: the two kernels'
    # bytes add up to the stage's plus twice the scores
    w = WORKLOADS["decode_128k"]
    st = bench.algorithmic_work(w)["token_topk"]["bytes"]
    a = bench.kernel_work(w, "k_token_scores")["bytes"]
    b = bench.kernel_work(w, "k_token_select")["bytes"]
    _, scored, _ = bench.per_query_counts(w)
    scores = float(scored.sum()) * w.batch * 4
    assert a + b == pytest.approx(st + 2 * scores - w.batch * w.n_q * w.top_m * 4 + w.batch * w.n_q * w.d_index * 2)
    assert bench.kernel_work(w, "k_block_scores_mfma")["bound"] == "mfma"
    for name in bench.KERNEL_STAGE:
        kw = bench.kernel_work(w, name)
        assert kw["bytes"] >= 0 and kw["flops"] >= 0


def test_traffic_record_gate(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    good = bench.kernel_source_hash("k_sparse_attn")
    text = ("kernel: k_sparse_attn\nsource_sha256: {h}\nfetch_size_kib_per_dispatch: 1024.0\n"
            "write_size_kib_per_dispatch: 512.0\ncopy_bytes: 1073741824\ncopy_fetch_size_kib: 524288.0\n"
            "copy_write_size_kib: 1048576.0\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (prof / "wl_traffic.txt").write_text(text.format(h=good))
    # FETCH counts half the bytes of the calibration copy, WRITE all of them
    assert bench.recorded_traffic("wl", "k_sparse_attn") == pytest.approx(1024 * (1024.0 * 2 + 512.0))
    assert bench.recorded_traffic("wl", "k_token_scores") is None
    (prof / "wl_traffic.txt").write_text(text.format(h="0" * 64))
    assert bench.recorded_traffic("wl", "k_sparse_attn") is None
    assert bench.recorded_traffic("other", "k_sparse_attn") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_parity_check_flags_differences():
    w = Workload(name="p", batch=2, seq_len=700, n_q=5, d_index=16, block=16, top_m=4, top_k=30, n_heads_q=4,
                 n_heads_kv=2)
    inp = datagen.make_inputs(w)
    S = [orc.block_summary(inp["kI"][b], w.block) for b in range(w.batch)]
    pairs = [(0, 0), (1, 4)]
    rows = {key: [] for key in ("blk", "tok", "O", "lse")}
    for b, i in pairs:
        r = orc.forward_query(inp, b, i, w.query_pos(i), w.block, w.top_m, w.top_k, w.scale, S_bits=S[b])
        for key in rows:
            rows[key].append(np.asarray(r[key], dtype=np.float32 if key in ("O", "lse") else np.int32))
    rows = {key: np.stack(v) for key, v in rows.items()}
    good = bench.parity_check(w, inp, S, None, rows, pairs)
    assert good["pass"] and good["index_sets_exact"] and good["max_abs_err_O"] < 1e-6
    bad = dict(rows, tok=rows["tok"].copy())
    bad["tok"][1, 0] += 1
    assert not bench.parity_check(w, inp, S, None, bad, pairs)["index_sets_exact"]
    off = bench.parity_check(w, inp, S, None, dict(rows, O=rows["O"] + 3e-3), pairs)
    assert off["index_sets_exact"] and not off["pass"]


def test_rooflines_are_fractions():
    # no HBM fraction above 1 is printed: prefill stages (rows shared by many
    # queries) report rates only, and the prefill attention and scorers are
    # measured against the bf16 MFMA roof with the method's flops
    w = WORKLOADS["prefill_64k"]
    work = bench.algorithmic_work(w)
    rates = bench.stage_rates(w, work, {"block_summary": 0.008, "block_topm": 0.12, "token_topk": 1.45,
                                        "sparse_attn": 5.5})
    for name, r in rates.items():
        assert r["hbm_frac"] is None or r["hbm_frac"] <= 1.0, name
        assert r.get("mfma_frac", 0.0) <= 1.0, name
    assert rates["sparse_attn"]["hbm_frac"] is None
    roof = bench.roofline_entry(w, "k_sparse_attn", 5.5, 32, None, None)
    assert roof["bound"] == "mfma" and 0 < roof["frac"] < 1
    assert roof["achieved"] == pytest.approx(4.0 * 128 * 16 * 132_121_600 / 5.5e-3 / 1e12)
    # 32 launches of 2048 queries: the same rate, the work and time split over them
    assert roof["algorithmic_per_launch"] == pytest.approx(4.0 * 128 * 16 * 132_121_600 / 32)
    assert roof["avg_launch_us"] == pytest.approx(5500.0 / 32)
    # decode streams its rows once: HBM roof
    wd = WORKLOADS["decode_128k"]
    assert bench.roofline_entry(wd, "k_sparse_attn", 0.0097, 1, None, None)["bound"] == "hbm"
    assert bench.kernel_work(w, "k_block_scores_max")["bytes"] == 4.0 * w.n_q
