"""GPU checks of the arithmetic at unusual score ranges, against the fp64
oracle (max|err| <= 1e-2, relative RMS <= 2e-3, f32 output): a zero scale
(every score 0, so each output is the plain mean of V), a negative scale, and
a scale 30 times the usual one (scores with a spread of about 30, so the
softmax is nearly one-hot and the running maximum jumps by far more than the
lazy rescale's threshold).  Every schedule runs: the fused one-launch step,
unsplit MFMA, partitions, stream-K, the host-length split step, the
partitioned step whose shared-partition kernel takes the append (the new
token folded in from k / v), and VALU."""

import dataclasses
import math

import numpy as np
import pytest

from gpu_util import assert_close, need_gpu, oracle_step
from paged_kv_cache_122_amd import workloads

pytestmark = pytest.mark.gpu

LENS = [1, 17, 300, 1024, 2049, 3000, 40, 999]
SCALES = {"zero": 0.0, "negative": -1.0, "sharp": 30.0}  # times 1/sqrt(D)


def _workload(hq, hkv, scale_mult):
    w = workloads.random_workload(7300 + hq, LENS, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, block_size=16,
                                  name=f"numerics_g{hq // hkv}")
    return dataclasses.replace(w, scale=scale_mult / math.sqrt(w.head_dim))


@pytest.mark.parametrize("which", list(SCALES), ids=list(SCALES))
def test_score_ranges_every_schedule(which):
    torch = need_gpu()
    from paged_kv_cache_122_amd import _lib as pa
    from paged_kv_cache_122_amd import device as dev

    for hq, hkv, runs in ((32, 8, ("fused", "unsplit", "parts", "stream", "host_split", "shared_step")),
                          (16, 8, ("valu",))):
        w = _workload(hq, hkv, SCALES[which])
        print(f"[{which} G={hq // hkv}] scale {w.scale:+.4f}", flush=True)
        _, _, ref = oracle_step(w)
        dw = dev.upload(w)
        maxlen = w.table_width * w.block_size
        hl = np.asarray(w.context_lens, dtype=np.int32)
        for run in runs:
            part = {"parts": 512, "stream": -2, "shared_step": 512}.get(run, 0)
            nb = pa.workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, maxlen, part)
            ws = pa.alloc_workspace(nb, "cuda") if nb else None
            out = torch.empty(dw.q.shape, dtype=torch.float32, device="cuda")
            if run in ("fused", "host_split", "shared_step"):
                # fused: the unsplit MFMA schedule (one launch); host_split: the automatic
                # schedule of this batch splits, which host lengths turn into partitions;
                # shared_step: partitions of 512 tokens, the append in the decode launch
                opts = {"fused": {"partition_tokens": -1, "path": 2},
                        "shared_step": {"partition_tokens": 512}}.get(run, {})
                assert run != "host_split" or pa.schedule(w.num_seqs, w.num_q_heads, w.num_kv_heads, maxlen) in (-2, 512)
                pa.append_decode(out, dw.q, dw.k_new, dw.v_new, dw.slot_mapping, dw.k_cache, dw.v_cache,
                                 dw.block_tables, dw.context_lens, w.scale, w.block_size, workspace=ws,
                                 host_context_lens=hl, **opts)
            else:
                pa.cache_append(dw.k_new, dw.v_new, dw.slot_mapping, dw.k_cache, dw.v_cache)
                path = 1 if run == "valu" else 2
                pa.decode_ex(out, dw.q, dw.k_cache, dw.v_cache, dw.block_tables, dw.context_lens, w.scale,
                             w.block_size, partition_tokens=-1 if run in ("unsplit", "valu") else part, path=path,
                             workspace=ws)
            torch.cuda.synchronize()
            a, r = assert_close(out.double().cpu().numpy(), ref, f"{which} {run}")
            print(f"[{which} {run}] max|err| {a:.2e} rel RMS {r:.2e}", flush=True)
        del dw
        torch.cuda.empty_cache()
