"""GPU check that the entry points which take the caller's workspace allocate
nothing and can be captured into a HIP graph: pa_append_decode (the fused
one-launch step, the host-length split step with its row combine, and the
partitioned step whose shared-partition kernel takes the new token, with the
combine that stores it), pa_decode_ex (stream-K) and pa_decode_multi_ex
(several new tokens, split, with the row combine).
Each graph is replayed several times, with eager work and a synchronisation
between replays, and every replay's output must equal the eager call's bit for
bit (the kernels are deterministic and the step's append is idempotent)."""

import numpy as np
import pytest

from gpu_util import need_gpu
from paged_kv_cache_122_amd import workloads

pytestmark = pytest.mark.gpu

CASES = [
    ("llama3_8b_b64", "append_decode"),           # one fused launch
    ("long32k_b16", "append_decode"),             # host-length partitions + row combine
    ("opt13b_mha_prefix_b128", "append_decode"),  # shared partitions (new token from k / v), combine + append
    ("long32k_b16", "decode_ex"),                 # stream-K + its combine
    ("long32k_verify5_b16", "decode_multi_ex"),   # several new tokens, split + row combine
]


@pytest.mark.parametrize("name,call", CASES, ids=[f"{c[0]}-{c[1]}" for c in CASES])
def test_graph_replay_matches_eager(name, call):
    torch = need_gpu()
    from paged_kv_cache_122_amd import _lib as pa
    from paged_kv_cache_122_amd import device as dev

    w = workloads.make(name)
    print(f"[{name} {call}] S={w.num_seqs}", flush=True)
    dw = dev.upload(w)
    maxlen = w.table_width * w.block_size
    if call == "decode_multi_ex":
        mql = int(np.diff(w.query_start).max())
        nb = pa.multi_workspace_bytes(w.q.shape[0], w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, mql,
                                      maxlen, 0)
    else:
        nb = pa.workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, maxlen, 0)
    ws = pa.alloc_workspace(nb, "cuda") if nb else None
    hl = np.asarray(w.context_lens, dtype=np.int32)
    out = torch.empty(dw.q.shape, dtype=torch.float32, device="cuda")

    def run():
        if call == "append_decode":
            pa.append_decode(out, dw.q, dw.k_new, dw.v_new, dw.slot_mapping, dw.k_cache, dw.v_cache,
                             dw.block_tables, dw.context_lens, w.scale, w.block_size, workspace=ws,
                             host_context_lens=hl)
        elif call == "decode_multi_ex":
            pa.decode_multi_ex(out, dw.q, dw.k_new, dw.v_new, dw.slot_mapping, dw.query_start, dw.k_cache,
                               dw.v_cache, dw.block_tables, dw.context_lens, w.scale, w.block_size, mql,
                               workspace=ws)
        else:
            pa.decode_ex(out, dw.q, dw.k_cache, dw.v_cache, dw.block_tables, dw.context_lens, w.scale,
                         w.block_size, workspace=ws)

    if call == "decode_ex":  # the pools hold this step's token before the decode
        pa.cache_append(dw.k_new, dw.v_new, dw.slot_mapping, dw.k_cache, dw.v_cache)
    run()
    torch.cuda.synchronize()
    ref = out.clone()
    assert not torch.isnan(ref).any()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for i in range(3):
        out.fill_(float("nan"))  # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), f"{name} {call}: replay {i} differs"
    del graph, dw
    torch.cuda.empty_cache()
