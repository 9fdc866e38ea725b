"""lightning_attn_decode_noalloc, the decode entry point that allocates
nothing, against lightning_attn_decode (needs an MI355X).

Both run the same kernels in the same order; the no-allocation one keeps the
two-kernel path's y and sums of squares in the library's fixed device array
instead of the caller's workspace, so outputs and updated states must be
identical bit for bit.  Two calls in a row (the second smaller) use the
array, a third shape needs none, and a shape beyond the array is refused
with nothing enqueued."""
import numpy as np
import pytest
import torch

from gpu_util import dev, inputs, say
import long_context_attn_amd as la

pytestmark = pytest.mark.gpu


def _case(S, H, D, dtype, key):
    q, k, v, g, w = inputs(S, H, D, "unit", bf16=dtype == torch.bfloat16, key=key)
    st = np.random.default_rng(key).standard_normal((S, H, D, D)).astype(np.float32)
    args = [dev(a, dtype) for a in (q, k, v, g, w)]
    return args, torch.from_numpy(st).cuda()


@pytest.mark.parametrize("S,H,D,dtype", [
    (120, 64, 128, torch.bfloat16),   # scratch: 3.75 MiB of y
    (37, 8, 64, torch.float32),       # the second call, smaller
    (256, 4, 128, torch.bfloat16),    # one kernel per sequence: no scratch
])
def test_noalloc_decode_matches_decode(S, H, D, dtype):
    args, st = _case(S, H, D, dtype, key=600 + S)
    st_ref, st_na = st.clone(), st.clone()
    say("noalloc decode S", S, "H", H, "D", D, dtype)
    for step in range(2):
        ref = la.decode(*args, st_ref)
        out = la.decode_noalloc(*args, st_na)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), step
        assert torch.equal(st_na, st_ref), step


def test_noalloc_decode_refuses_beyond_its_scratch():
    S, H, D = 255, 64, 128  # y alone is 8.2 MB: more than the 4 MiB + 64 KiB array
    args, st = _case(S, H, D, torch.bfloat16, key=700)
    out = torch.full((S, H, D), 5.0, dtype=torch.bfloat16, device="cuda")
    st0 = st.clone()
    with pytest.raises(la.LightningAttnError) as e:
        la.decode_noalloc(*args, st, out=out)
    assert e.value.status == 7
    torch.cuda.synchronize()
    assert torch.all(out == 5.0) and torch.equal(st, st0)
