"""GPU parity of the fixed-interval refresh schedule against the oracle's loop.

The driver (sparse_kv_cache_sfi_amd.schedule.RefreshSchedule) runs slow steps every
``interval`` steps and fast steps between on a run whose planted heavy hitters shift
every 16 steps.  The oracle's refresh_loop runs the same schedule in fp64, selecting
from the very logits the GPU produced (checked against its own within the fp32 bound),
so the selections must match bit for bit and every step's output within tolerance.
"""
import numpy as np
import pytest
import torch

import oracle as O
from sfi_synth import drifting_case
from _gpu import DEV, LSE_TOL, OUT_TOL, DevCase, assert_close, dev_array, score_bound

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("interval", [1, 8, 13])
def test_refresh_schedule_matches_the_oracle_loop(gpu_lib, interval):
    from sparse_kv_cache_sfi_amd.schedule import RefreshSchedule
    steps, k = 40, 48
    dc = drifting_case(61, B=2, Hq=8, Hkv=2, d=128, dtype="bf16", L0=[1500, 2600], steps=steps, period=16,
                       hh=16, n_sink=4, n_recent=32, k_sel=k)
    c = dc.case
    dev = DevCase(c)
    L0 = c.seq_lens.astype(np.int64)
    q = torch.empty((c.B, c.Hq, c.d), dtype=torch.bfloat16, device=DEV)
    lens = torch.empty((c.B,), dtype=torch.int32, device=DEV)
    sched = RefreshSchedule(dev.k, dev.v, dev.bt, q, lens, max_seq_len=dev.max_seq_len, n_sink=4, n_recent=32,
                            k=k, interval=interval)
    outs, lses, sels, scores = [], [], {}, {}
    for t in range(steps):
        q.copy_(dev_array(dc.q_steps[t]))
        lens.copy_(torch.from_numpy((L0 + t + 1).astype(np.int32)))
        slow = sched.step()
        torch.cuda.synchronize()
        outs.append(sched.out.cpu().numpy().copy())
        lses.append(sched.lse.cpu().numpy().copy())
        if slow:
            sels[t] = sched.sel.cpu().numpy().copy()
            scores[t] = sched.scores.cpu().numpy().copy()
    qv = dc.q_step_values()
    for b in range(c.B):
        res = O.refresh_loop(qv[:, b], c.kv.k, c.kv.v, c.kv.block_table[b], int(L0[b]), c.Hkv, 4, 32, k, interval,
                             c.scale, 4 + k, kv_dtype="bf16", scores_at=lambda t: scores[t][b].astype(np.float64))
        for t, (out, lse, sel, S) in enumerate(res):
            assert_close(outs[t][b], out, OUT_TOL, f"out t={t} b={b}")
            assert_close(lses[t][b], lse, LSE_TOL, f"lse t={t} b={b}")
            if sel is None:
                continue
            assert np.array_equal(sels[t][b], sel), (t, b)
            L = int(L0[b]) + t + 1
            lo, hi = O.candidate_range(L, 1, 4, 32)
            for g in range(c.Hkv):
                rows = O.paged_rows(c.kv.k_values(), c.kv.block_table[b], g, np.arange(lo, hi))
                bound = score_bound(qv[t, b, g * c.G:(g + 1) * c.G], rows, c.scale)
                assert_close(scores[t][b, g, lo:hi], S[g, lo:hi], bound, f"scores t={t} b={b} g={g}")
                # the refresh finds the current epoch's planted support
                assert set(dc.support[t // 16, b, g].tolist()) <= set(sels[t][b, g].tolist()), (t, b, g)
