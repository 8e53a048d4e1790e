"""The binding rejects caller buffers that do not fit the launch (GPU)."""
import pytest
import torch

import exact_attention_forward_04_amd as fa

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load()
    yield
    torch.cuda.synchronize()


def _inputs(B=1, S=64, H=2, D=64):
    g = torch.Generator().manual_seed(0)
    mk = lambda: torch.randn(B, S, H, D, generator=g).to(torch.bfloat16).cuda()  # noqa: E731
    return mk(), mk(), mk()


def test_attention_rejects_bad_lse_and_out():
    q, k, v = _inputs()
    dev = q.device
    for lse in (torch.empty(1, 2, 32, device=dev),                          # smaller
                torch.empty(1, 2, 64, device=dev, dtype=torch.float16),     # dtype
                torch.empty(1, 64, 2, device=dev).transpose(1, 2),          # layout
                torch.empty(1, 2, 64)):                                     # host memory
        with pytest.raises(ValueError):
            fa.attention(q, k, v, causal=True, lse_out=lse)
    for out in (torch.empty(1, 64, 2, 32, dtype=torch.bfloat16, device=dev),
                torch.empty(1, 64, 2, 64, dtype=torch.float32, device=dev),
                torch.empty(1, 2, 64, 64, dtype=torch.bfloat16, device=dev).transpose(1, 2)):
        with pytest.raises(ValueError):
            fa.attention(q, k, v, causal=True, out=out)
    # the right buffers are accepted and written
    o = torch.empty(1, 64, 2, 64, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(1, 2, 64, device=dev)
    o2, lse2 = fa.attention(q, k, v, causal=True, out=o, lse_out=lse)
    torch.cuda.synchronize()
    assert o2.data_ptr() == o.data_ptr() and lse2.data_ptr() == lse.data_ptr()
    assert torch.isfinite(lse).all()


def test_splits_with_tuning_rejected():
    q, k, v = _inputs()
    with pytest.raises(ValueError):
        fa.attention(q, k, v, causal=True, num_splits=2, tuning=fa.default_tuning())


def test_backward_rejects_bad_buffers():
    q, k, v = _inputs()
    o, lse = fa.attention(q, k, v, causal=True)
    do = torch.randn_like(q.float()).to(torch.bfloat16)
    dev = q.device
    with pytest.raises(ValueError):
        fa.attention_backward(q, k, v, o, lse, do, causal=True,
                              dq=torch.empty(1, 2, 64, 64, dtype=torch.bfloat16,
                                             device=dev).transpose(1, 2))
    with pytest.raises(ValueError):
        fa.attention_backward(q, k, v, o, lse, do, causal=True, delta=torch.empty(1, 2, 64))


def test_fa_log_lines():
    """FA_LOG=1: each launch writes one "[fa] ..." line naming its kernel,
    grid and LDS to stderr (checked in a child process, which reads the
    variable at its first launch); without it nothing is written."""
    import os
    import subprocess
    import sys as _sys
    code = ("import torch, exact_attention_forward_04_amd as fa\n"
            "q = torch.randn(1, 300, 2, 128, device='cuda').to(torch.bfloat16)\n"
            "o, lse = fa.attention(q, q, q, causal=True)\n"
            "fa.attention(q[:, :1].contiguous(), q, q, causal=True, num_splits=2)\n"
            "fa.attention_backward(q, q, q, o, lse, q.clone(), causal=True)\n"
            "torch.cuda.synchronize()\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for val, expect in (("1", True), ("0", False)):
        env = dict(os.environ, FA_LOG=val, PYTHONPATH=root)
        r = subprocess.run([_sys.executable, "-c", code], env=env, capture_output=True, text=True,
                           timeout=300)
        assert r.returncode == 0, r.stderr[-2000:]
        lines = [l for l in r.stderr.splitlines() if l.startswith("[fa] ")]
        if expect:
            text = "\n".join(lines)
            assert "fa_fwd_persistent<D=128 causal=1" in text, text
            assert "fa_fwd_split<D=128" in text and "fa_split_combine" in text, text
            assert "fa_bwd_dq<D=128" in text, text
            assert "B LDS" in text
        else:
            assert lines == []
