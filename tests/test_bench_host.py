"""Host-side pieces of bench.py that need no GPU: the oracle-sample
comparison counts what it claims, and the CPU baseline reports the fields
the bench line promises, on one thread and on several."""
import numpy as np

import bench
import oracle
import workloads


def _oracle_outputs(cfg, wl):
    res = [oracle.verify(wl.target[b:b + 1], None if wl.draft is None else wl.draft[b:b + 1], wl.tokens[b:b + 1],
                         wl.uniforms[b:b + 1], cfg.T, onehot=cfg.onehot) for b in range(wl.n)]
    acc = np.array([r.accepted_len[0] for r in res], np.int32)
    out = np.concatenate([r.out_tokens for r in res]).astype(np.int32)
    return acc, out


def test_sample_parity_counts_mismatches_not_agreement():
    cfg = workloads.get_config("selfdraft").scaled(B=6, V=3000)
    wl = workloads.generate(cfg)
    acc, out = _oracle_outputs(cfg, wl)
    rep = bench.sample_parity(cfg, wl, acc, out, threads=3)
    assert rep["sequences"] == 6 and rep["mismatches"] == 0
    # a different committed token at r in one sequence, an accepted length
    # off by one in another: two mismatches (unless a band excuses them)
    bad_out = out.copy()
    bad_out[0, acc[0]] = (bad_out[0, acc[0]] + 1) % cfg.V
    bad_acc = acc.copy()
    bad_acc[1] = acc[1] - 1 if acc[1] > 0 else 1
    rep2 = bench.sample_parity(cfg, wl, bad_acc, bad_out, threads=2)
    excused = rep2["ambiguous_accept"] + rep2["ambiguous_draw"]
    assert rep2["mismatches"] + excused >= 2 and rep2["mismatches"] >= 2 - excused


def test_sample_parity_greedy_has_no_ambiguity():
    cfg = workloads.get_config("grpo_greedy").scaled(B=5, V=2000)
    wl = workloads.generate(cfg)
    acc, out = _oracle_outputs(cfg, wl)
    rep = bench.sample_parity(cfg, wl, acc, out, threads=2)
    assert rep["ambiguous_accept"] == rep["ambiguous_draw"] == rep["mismatches"] == 0


def test_cpu_baseline_fields_one_and_several_threads():
    cfg = workloads.get_config("ngram_tail").scaled(B=4, V=5000)
    one = bench.cpu_baseline(cfg, 0.3, threads=1)
    two = bench.cpu_baseline(cfg, 0.3, threads=2)
    for r, n in ((one, 1), (two, 2)):
        assert r["kind"] == "oracle" and r["unit"] == "positions/s" and r["cores"] == n
        assert r["value"] > 0 and "sample" in r and r["host_nproc"] >= 1
    assert 1 <= bench.host_threads() <= bench.HOST_THREADS_MAX
