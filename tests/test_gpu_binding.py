"""The Python binding's argument checks on real device tensors: a call whose
tensors are of the wrong dtype, size or device kind, or not contiguous,
raises before anything is launched (the outputs keep their contents), and
names the offending argument."""
import pytest
import torch

import tensor_all_reduce_ar_amd as ar

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

H, ROWS = 256, 4
N = H * ROWS


def _fused_args():
    g = torch.Generator(device="cpu").manual_seed(77)
    parts = [torch.randn(N, generator=g).half().cuda() for _ in range(3)]
    weight = torch.randn(H, generator=g).half().cuda()
    residual = torch.randn(N, generator=g).half().cuda()
    bias = torch.randn(H, generator=g).half().cuda()
    out = torch.full((N,), 7.0, dtype=torch.float16, device="cuda")
    inter = torch.full((N,), 7.0, dtype=torch.float16, device="cuda")
    return dict(partials=parts, weight=weight, eps=1e-6, out=out, intermediate=inter, bias=bias,
                residual=residual)


def _untouched(*ts):
    torch.cuda.synchronize()
    return all(bool((t == 7.0).all()) for t in ts)


@pytest.mark.parametrize("field,bad,err,name", [
    ("partial", lambda t: t.float(), TypeError, "partial 1"),                     # dtype
    ("partial", lambda t: t[: N - 8], ValueError, "partial 1"),                   # size
    ("partial", lambda t: t.cpu(), ValueError, "partial 1"),                      # host tensor
    ("partial", lambda t: t.view(ROWS, H).t(), ValueError, "partial 1"),          # not contiguous
    ("weight", lambda t: t.float(), TypeError, "weight"),
    ("bias", lambda t: t.bfloat16(), TypeError, "bias"),
    ("residual", lambda t: t.cpu(), ValueError, "residual"),
    ("intermediate", lambda t: t.view(ROWS, H).t(), ValueError, "intermediate"),
])
def test_fused_call_rejects_bad_tensors(field, bad, err, name):
    a = _fused_args()
    if field == "partial":
        a["partials"][1] = bad(a["partials"][1])
    else:
        a[field] = bad(a[field])
    with pytest.raises(err, match=name):
        ar.ar_residual_rmsnorm(**a)
    with pytest.raises(err, match=name):
        ar.prepare_residual_rmsnorm(**a)
    outs = [a["out"]] + ([a["intermediate"]] if a["intermediate"].is_cuda and a["intermediate"].is_contiguous()
                         else [])
    assert _untouched(*outs)


def test_weight_shorter_than_the_given_row_width():
    """hidden_size defaults to the weight's length; given explicitly, a
    shorter weight is an error."""
    a = _fused_args()
    a["weight"] = a["weight"][:-1]
    with pytest.raises(ValueError, match="weight has 255 elements, expected 256"):
        ar.ar_residual_rmsnorm(**a, hidden_size=H)
    assert _untouched(a["out"], a["intermediate"])


def test_sum_call_rejects_bad_tensors():
    parts = [torch.ones(N, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    out = torch.full((N,), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(TypeError, match="partial 0"):
        ar.ar_sum([parts[0].half(), parts[1]], out)
    with pytest.raises(ValueError, match="partial 1"):
        ar.ar_sum([parts[0], parts[1][1:]], out)
    with pytest.raises(ValueError, match="out must be a device tensor"):
        ar.ar_sum(parts, out.cpu())
    with pytest.raises(ValueError, match="need 1..8 partials"):
        ar.ar_sum([], out)
    assert _untouched(out)
    ar.ar_sum(parts, out)  # and the good call still runs
    torch.cuda.synchronize()
    assert bool((out == 2.0).all())
