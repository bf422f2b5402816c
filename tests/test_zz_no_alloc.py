"""The allocation-free decode entry point, on the GPU, through the C ABI: its
outputs equal those of mla_decode_attention with a caller workspace bit for
bit, on two calls in a row (the second with a smaller input, so it runs on
the scratch the first one left behind), on both decode kernels (128 query
rows per request and 64)."""
import numpy as np
import pytest
import torch

import mla_inputs as mi
import mla_latent_cache_amd as mla
from gpu_util import DeviceCase, dims_tuple, run

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on a GPU machine only
    pytest.skip("no GPU", allow_module_level=True)


def noalloc(dc, num_splits, out_dtype):
    case, s = dc.case, dc.case.spec
    q_abs = run(dc, num_splits=num_splits, out_dtype=out_dtype, decompress=False)["q_abs"]
    out = torch.full((s.batch, s.t_q, s.n_head, s.kv_rank), 7.0, dtype=out_dtype, device="cuda")
    lse = torch.full((s.batch, s.t_q, s.n_head), 7.0, dtype=torch.float32, device="cuda")
    mla.mla_decode_attention_noalloc(dims_tuple(s), case.scale, q_abs, dc.kv, dc.bt, dc.sl, out, lse, num_splits)
    torch.cuda.synchronize()
    return out, lse


def test_noalloc_matches_workspace_call_twice_second_smaller():
    big = mi.with_spec(mi.SPECS["dsv3_ragged"], name="dsv3_noalloc", batch=6, fixed_lens=(900, 0, 5000, 33, 1, 2100),
                       max_blocks=320, lengths="fixed", zero_requests=())
    small = mi.with_spec(mi.SPECS["glm52_decode"], name="glm52_noalloc", batch=3, fixed_lens=(77, 300, 16),
                         max_blocks=19)
    for spec, k, odt in ((big, 0, torch.bfloat16), (small, 3, torch.float32)):
        dc = DeviceCase(mi.make_case(spec))
        ref = run(dc, num_splits=k, out_dtype=odt, decompress=False)
        assert ref["status"] == 0
        out, lse = noalloc(dc, k, odt)
        assert torch.equal(out, ref["o_lat"]), spec.name
        assert torch.equal(lse, ref["lse"]), spec.name
        assert np.isfinite(out[dc.sl.cpu().numpy() > 0].float().cpu().numpy()).all()
