"""The library keeps no state between calls and is reentrant: several host
threads, each on its own stream, call the entry points (quantization and the
scale re-layout) at the same time and every result equals the oracle's."""
import threading

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import (CANARY, DEV, adversarial, assert_same_bytes, bf16_dev, i32_dev,
                         jagged_colwise, jagged_mx_rowwise, jagged_rowwise, mx_3d_colwise,
                         random_offsets, relayout)

pytestmark = pytest.mark.gpu


def test_concurrent_calls_on_separate_streams():
    cases = []
    for k in range(6):
        bits = adversarial((300 + 37 * k, 2048 + 8 * k), 900 + k)
        offs = random_offsets(bits.shape[1], 3 + k, 900 + k, short_tail=k)
        cases.append((bits, offs))
    col = adversarial((3000, 64), 990)
    col_offs = random_offsets(3000, 5, 990)
    w = np.stack([workloads.mx3d_sweep_expert(e, N=256, K=512) for e in range(2)])
    rl_offs = random_offsets(40000, 6, 995, short_tail=11)
    rl = workloads.e8m0_bytes((200, oracle.jagged_mx_scale_capacity(40000, 6)), 995)

    want = {}
    for k, (bits, offs) in enumerate(cases):
        want[("row", k)] = oracle.quantize_jagged_rowwise(bits, offs, canary=CANARY)
        want[("mx", k)] = oracle.quantize_jagged_mx_rowwise(bits, offs, canary=CANARY)
    want["col"] = oracle.quantize_jagged_colwise(col, col_offs, canary=CANARY)
    want["mx3d"] = oracle.quantize_mx_3d_colwise(w)
    want["relayout"] = oracle.relayout_mx_scales_grouped(rl, rl_offs, 40000, canary=CANARY)

    dev_cases = [(bf16_dev(b), i32_dev(o)) for b, o in cases]
    dev_col, dev_col_offs, dev_w = bf16_dev(col), i32_dev(col_offs), bf16_dev(w)
    dev_rl = torch.from_numpy(rl).to(DEV)
    torch.cuda.synchronize()

    got, errors = {}, []

    def worker(k):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for rep in range(3):
                    x, o = dev_cases[k]
                    got[("row", k, rep)] = jagged_rowwise(x, o, stream=stream)
                    got[("mx", k, rep)] = jagged_mx_rowwise(x, o, stream=stream)
                    if k == 0:
                        got[("col", rep)] = jagged_colwise(dev_col, dev_col_offs, stream=stream)
                    if k == 1:
                        got[("mx3d", rep)] = mx_3d_colwise(dev_w, stream=stream)
                    if k == 2:
                        got[("relayout", rep)] = relayout(dev_rl, rl_offs, 40000, stream=stream)
        except Exception as e:   # surfaced below
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(len(cases))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors

    for rep in range(3):
        for k in range(len(cases)):
            for kind in ("row", "mx"):
                q, s = got[(kind, k, rep)]
                oq, os_ = want[(kind, k)]
                assert_same_bytes(q, oq, f"{kind} case {k} rep {rep} q")
                assert_same_bytes(s, os_, f"{kind} case {k} rep {rep} scales")
        q, s = got[("col", rep)]
        assert_same_bytes(q, want["col"][0], f"colwise rep {rep} q")
        assert_same_bytes(s, want["col"][1], f"colwise rep {rep} scales")
        q, s = got[("mx3d", rep)]
        assert_same_bytes(q, want["mx3d"][0], f"mx3d rep {rep} q")
        assert_same_bytes(s, want["mx3d"][1], f"mx3d rep {rep} scales")
        t, st = got[("relayout", rep)]
        assert np.array_equal(t, want["relayout"][0]), f"relayout rep {rep} tiles"
        assert np.array_equal(st, want["relayout"][1]), f"relayout rep {rep} tile starts"
