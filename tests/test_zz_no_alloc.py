"""The allocation-free attention entry point (needs an MI355X).

wf_chunk_attn_fwd_noalloc must give exactly what wf_chunk_attn_fwd gives with a
caller workspace, call after call on one GPU: the scratch array inside the
library keeps the previous call's partial results, and every slot the merge
reads must have been rewritten by the current call.  Two calls in a row, the
second smaller, on the split schedule (bf16 and E4M3FN caches) and on the
per-tile schedule, compared bitwise; the first call is also checked against the
float64 oracle at the bf16 bars.
"""
import numpy as np
import pytest
import torch

import chunk_causal_dit_wf_amd as wf
import synth
from gpu_util import Pair, dev, errors, host_codes, host_values, values_of

pytestmark = pytest.mark.gpu

H, D, N_KEYS = 2, 128, 6400
CALLS = [  # (q_off, kv_begin, kv_end): the second call is smaller
    ([0, 37, 300, 301], [5, 0, 0], [6395, 6400, 6340]),
    ([0, 100], [64], [3264]),
]


def make_pair(dtype, P, seed):
    rng = np.random.default_rng(seed)
    T = N_KEYS // P
    pair = Pair(T + 2, P, H, D, dtype, list(rng.permutation(T + 2)[:T]), fill_seed=seed + 1)
    std = 0.5 if dtype == "bf16" else 1.0
    k = synth.normal_f32((N_KEYS, H, D), std, 90, seed, 1)
    v = synth.normal_f32((N_KEYS, H, D), std, 90, seed, 2)
    if dtype == "fp8":
        kc, ks = synth.quantize_e4m3_pages(k, P)
        vc, vs = synth.quantize_e4m3_pages(v, P)
        pair.append(0, kc, vc, ks, vs)
    else:
        pair.append(0, synth.bf16_codes(k), synth.bf16_codes(v))
    q = synth.bf16_codes(synth.normal_f32((301, H, D), std, 90, seed, 0) * np.float32(2.0))
    return pair, q


@pytest.mark.parametrize("dtype,P,sched", [("bf16", 256, "split"), ("fp8", 256, "split"), ("bf16", 40, "per_tile")])
def test_noalloc_equals_workspace_entry_point(dtype, P, sched):
    print("case: noalloc", dtype, P, sched, flush=True)
    pair, qc = make_pair(dtype, P, 91)
    ws = wf.workspace_for(pair.gpu, "cuda")
    for i, (q_off, kb, ke) in enumerate(CALLS):
        pl = wf.wf_chunk_attn_plan(pair.gpu, q_off, kb, ke, "bf16", 0 if ws is None else ws.numel())
        print("call %d plan %s" % (i, pl), flush=True)
        assert pl["schedule"] == sched
        q = dev(qc[:q_off[-1]], "bf16")
        o_ref, l_ref = wf.wf_chunk_attn_fwd(pair.gpu, q, q_off, kb, ke, return_lse=True, workspace=ws)
        o = torch.full_like(q, float("nan"))
        lse = torch.full((H, q_off[-1]), float("nan"), dtype=torch.float32, device="cuda")
        wf.wf_chunk_attn_fwd_noalloc(pair.gpu, q, q_off, kb, ke, o, lse)
        torch.cuda.synchronize()
        assert np.array_equal(host_codes(o), host_codes(o_ref)), "call %d: O differs" % i
        assert np.array_equal(lse.cpu().numpy(), l_ref.cpu().numpy()), "call %d: LSE differs" % i
        if i == 0:
            ro, _ = pair.reference(values_of(qc[:q_off[-1]], "bf16"), q_off, kb, ke)
            mx, mean, rel = errors(host_values(o), ro)
            print("vs oracle: max-abs %.3e mean-abs %.3e rel-L2 %.3e" % (mx, mean, rel), flush=True)
            if dtype == "bf16":
                assert mx <= 1e-2 and mean <= 1e-3 and rel <= 1e-2
            else:
                assert mx <= 5e-2 and rel <= 6e-2


def test_noalloc_validates_before_launch():
    pair, qc = make_pair("bf16", 256, 92)
    q = dev(qc[:10], "bf16")
    o = torch.empty_like(q)
    with pytest.raises(wf.WfError) as e:
        wf.wf_chunk_attn_fwd_noalloc(pair.gpu, q, [0, 10], [0], [N_KEYS + 1], o)
    assert e.value.status == wf.WF_ERR_RANGE
