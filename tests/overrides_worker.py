"""Run by tests/test_gpu_overrides.py in a process of its own, with the
test-only overrides PA_TEST_SPLIT_KEYS / PA_TEST_PATH set in its
environment (the library reads them once per process).

For a set of batches built around the split length in force, it checks
through the C ABI:
* every output within the fp16 / bf16 bar of the fp64 oracle (also over
  fp8 caches, for decode-shaped batches);
* batch invariance: each sequence's rows computed in a call of its own
  (same cache, same table row) equal its rows in the whole batch bitwise.
Prints one JSON line and exits 0 when everything holds, 1 otherwise.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

import numpy as np  # noqa: E402
import torch  # noqa: E402

import paged_kv_cache_pa_amd as pa  # noqa: E402
from paged_kv_cache_pa_amd import workloads as W  # noqa: E402
from gpu_util import (TOL, device_inputs, device_inputs_fp8, max_err, oracle_full,  # noqa: E402
                      oracle_full_fp8, run_attention_fp8)


def one_sequence(wl, d, b, **opts):
    """Sequence b alone: its query rows and metadata over the same cache."""
    cu = wl.cu_seqlens_q
    q = d["q"][cu[b]:cu[b + 1]].contiguous()
    c1 = torch.tensor([0, int(cu[b + 1] - cu[b])], dtype=torch.int32, device="cuda")
    lens = d["lens"][b:b + 1].contiguous()
    table = d["table"][b:b + 1].contiguous()
    out = pa.pa_attention(q, c1, lens, table, d["kc"], d["vc"], wl.scale, wl.num_heads,
                          wl.num_kv_heads, **opts)
    torch.cuda.synchronize()
    return out


def main():
    S = int(os.environ.get("PA_TEST_SPLIT_KEYS", "1024"))
    path = os.environ.get("PA_TEST_PATH", "auto")
    bs_list = [16, 32]    # a 2048-key split spans 128 blocks of 16, the most a split may
    cases = []
    for bs in bs_list:
        # Decode columns around split boundaries (q_len 1 and 2, G 8: 8 and
        # 16 columns), a prefill chunk, MHA and G = 4.
        cases.append((W.custom([1, 1, 1, 2, 1, 40], [S - 1, S, S + 1, 2 * S + 7, 5 * S + 3, S + 60],
                               32, 4, 128, bs, seed=61), {}))
        cases.append((W.custom([1, 2, 17, 1], [3 * S, S + 2, 2 * S - 5, 1], 64, 8, 128, bs,
                               dtype="bf16", seed=62), {}))
        cases.append((W.custom([1, 3, 1], [2 * S + 1, S - 3, 4 * S], 8, 8, 64, bs, seed=63), {}))
        cases.append((W.custom([1, 1, 9], [3 * S + 5, S, 2 * S], 32, 8, 128, bs, seed=64),
                      dict(softcap=20.0, local_window_size=S + 100)))
    worst, invariant, n = 0.0, True, 0
    for wl, opts in cases:
        d = device_inputs(wl)
        out = pa.pa_attention(d["q"], d["cu"], d["lens"], d["table"], d["kc"], d["vc"], wl.scale,
                              wl.num_heads, wl.num_kv_heads, **opts)
        torch.cuda.synchronize()
        err = max_err(out, oracle_full(wl, d, **opts))
        worst = max(worst, err)
        if not err <= TOL[wl.dtype]:
            print(json.dumps({"fail": wl.name, "err": err, "opts": opts}), flush=True)
            return 1
        cu = wl.cu_seqlens_q
        for b in range(wl.num_seqs):
            if cu[b + 1] == cu[b]:
                continue
            alone = one_sequence(wl, d, b, **opts)
            if not torch.equal(alone, out[cu[b]:cu[b + 1]]):
                invariant = False
                print(json.dumps({"not invariant": wl.name, "seq": b}), flush=True)
        n += 1
    # fp8 caches (decode-shaped batches; the forced prefill path does not
    # apply to them): the same split boundaries through the fp8 decode items.
    for bs in bs_list:
        wl = W.custom([1, 2, 1, 1], [S - 1, 2 * S + 5, S + 1, 3 * S + 7], 32, 8, 128, bs,
                      seed=65)
        d = device_inputs_fp8(wl)
        err = max_err(run_attention_fp8(wl, d), oracle_full_fp8(wl, d))
        worst = max(worst, err)
        if not err <= TOL[wl.dtype]:
            print(json.dumps({"fail": "fp8 " + wl.name, "err": err}), flush=True)
            return 1
        n += 1
    print(json.dumps({"split_keys": S, "path": path, "batches": n, "worst_err": worst,
                      "batch_invariant": invariant}), flush=True)
    return 0 if invariant else 1


if __name__ == "__main__":
    sys.exit(main())
