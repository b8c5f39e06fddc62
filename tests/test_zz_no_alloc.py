"""gpt2_forward_noalloc (the forward on the library's fixed scratch, for callers that cannot
allocate) against gpt2_forward on a caller workspace: same kernels, same inputs, so logits and
argmax must be bit-identical. Two calls in a row, the second smaller, then a size past the
scratch's 80 MiB, which must be refused without touching the outputs."""
import numpy as np
import pytest
import torch

from decoder_only_transformer_gpt2_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def small_bf16():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from decoder_only_transformer_gpt2_amd import gpt2
    gpt2.lib()  # raises when the library has not been built
    m = gpt2.GPT2(gpt2.ModelConfig(dtype="bf16"))
    m.load_numpy(synth.make_weights(synth.GPT2_SMALL, bf16=True))
    return gpt2, m


def _both(m, B, T, seed):
    tok = torch.from_numpy(synth.make_tokens(B, T, seed=seed)).cuda()
    ref_l, ref_a = m.forward(tok)
    logits = torch.full((B, T, 50257), float("nan"), dtype=torch.float32, device="cuda")
    am = torch.full((B, T), -7, dtype=torch.int32, device="cuda")
    print(f"noalloc forward B={B} T={T}", flush=True)
    m.forward_noalloc(tok, logits, am)
    torch.cuda.synchronize()
    return ref_l, ref_a, logits, am


def test_noalloc_matches_forward_twice_then_smaller(small_bf16):
    g, m = small_bf16
    for B, T, seed in ((4, 1024, 1), (2, 77, 9)):
        ref_l, ref_a, logits, am = _both(m, B, T, seed)
        assert torch.equal(logits.view(torch.int32), ref_l.view(torch.int32)), (B, T)
        assert torch.equal(am, ref_a), (B, T)


def test_noalloc_rejects_past_scratch(small_bf16):
    g, m = small_bf16
    tok = torch.from_numpy(synth.make_tokens(8, 1024)).cuda()
    logits = torch.zeros((1,), dtype=torch.float32, device="cuda")
    with pytest.raises(g.GPT2Error) as e:
        m.forward_noalloc(tok, logits, None)
    assert e.value.status == g.EWORKSPACE
    assert logits.item() == 0.0
