"""GPU parity at component counts above 128, up to the library's bound K = 256
(the language model of the technical summary "Resumo Técnico: Atenção de
Mistura Gaussiana (GMA)", section "Resultados e Desempenho", uses K = 256).

Both variants and both input types.  Where the causal scan kernel's tiles do
not fit in LDS (fp32 and bf16 at the larger K x d_v), the causal forward runs
as a chain of fp32 products over stored responsibilities; the parity bar is
the same.
"""
import pytest
import torch

from gaussian_mixture_sequence_gma_amd import binding as B, inputs
from tests.parity import run_and_compare

pytestmark = pytest.mark.gpu

W = inputs.WORKLOADS


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("K", [129, 200, 256])
def test_wide_component_counts(K, dtype, causal):
    w = W["tiny_bidir_f32"].with_(K=K, d_r=32, d_v=64, N=300, H=2, dtype=dtype, causal=causal)
    run_and_compare(w)


@pytest.mark.parametrize("causal", [False, True])
def test_language_model_k256(causal):
    """K = 256 at the language-model head shape (d_r = d_v = 64), bf16, with
    several 64-token chunks and tiles and a ragged tail."""
    w = W["lm_causal_bf16"].with_(B=1, H=3, N=1500, K=256, causal=causal)
    run_and_compare(w)


@pytest.mark.parametrize("causal", [False, True])
def test_long_head_k256(causal):
    """K = 256 with the long-context head's d_v = 128 and skewed parameters."""
    w = W["long_bidir_bf16"].with_(H=2, N=2000, K=256, causal=causal)
    run_and_compare(w)
