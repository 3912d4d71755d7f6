"""bigram_bwd_update_noalloc (the table update with library-owned scratch) against
bigram_bwd_update (caller workspace) through the C ABI: the same kernels run on the same inputs,
so tables and second moments must agree bit for bit, on two calls in a row (the second smaller,
so it runs over scratch the first call left behind), and sizes above the scratch are refused
before any launch."""
import numpy as np
import pytest
import torch

from gpt_lm_step_amd import binding as B
from gpt_lm_step_amd import configs, inputs
from oracle import tables as ot

from gpu_util import dev

pytestmark = pytest.mark.gpu


def _case(seed, n, R, D, zipf):
    rng = np.random.default_rng(seed)
    if zipf:
        tok = inputs.zipf_tokens(seed, (n // 1024, 1024), configs.TABLES.vocab)
        h = ot.hash_indices(tok, 2, configs.TABLES.vocab, R).reshape(-1).astype(np.int32)
    else:
        h = rng.integers(0, R, n).astype(np.int32)
        h[: n // 4] = 7                       # one long segment across many tiles
    dy = inputs.normal(seed + 1, (n, D), 1.0, True)
    table = inputs.normal(seed + 2, (R, D), 0.02, True)
    v = (np.abs(rng.standard_normal(R)) * 1e-3).astype(np.float32)
    return h, dy, table, v


def test_noalloc_update_equals_workspace_update_twice():
    cases = [(61, configs.TABLES.n_tokens, 1 << 21, 768, True),   # the tables workload
             (71, 3000, 5003, 768, False)]                         # then a smaller call
    for seed, n, R, D, zipf in cases:
        h, dy, table0, v0 = _case(seed, n, R, D, zipf)
        th, tdy = dev(h), dev(dy, torch.bfloat16)
        t_ref, v_ref = dev(table0, torch.bfloat16), dev(v0)
        t_na, v_na = t_ref.clone(), v_ref.clone()
        B.bigram_bwd_update(th, tdy, t_ref, v_ref, 1e-2)
        B.bigram_bwd_update_noalloc(th, tdy, t_na, v_na, 1e-2)
        torch.cuda.synchronize()
        assert torch.equal(t_na.view(torch.int16), t_ref.view(torch.int16)), (seed, n)
        assert torch.equal(v_na.view(torch.int32), v_ref.view(torch.int32)), (seed, n)
        assert not torch.equal(t_na, dev(table0, torch.bfloat16))    # rows did move


def test_noalloc_update_refuses_sizes_above_its_scratch():
    D = 768
    n = 400_000
    assert B.bigram_workspace_bytes(n, D) > 32 << 20
    h = torch.zeros(n, dtype=torch.int32, device="cuda")
    dy = torch.zeros(n, D, dtype=torch.bfloat16, device="cuda")
    table = torch.zeros(16, D, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(16, device="cuda")
    with pytest.raises(B.GptError) as e:
        B.bigram_bwd_update_noalloc(h, dy, table, v, 1e-2)
    assert e.value.status == B.GPT_ESHAPE and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.count_nonzero(v) == 0
