"""The measurement helpers behind bench.py's measured peaks and GEMM-tile probe:
the shared GEMM tile on its own (ttt_probe_gemm_bf16) against an fp32 product
of the same bf16 values, for each operand layout, and the MFMA loop's
argument checks."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,groups", [(128, 1), (256, 1), (64, 1), (128, 2)])
@pytest.mark.parametrize("ak,bk", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_gemm_tile_probe_matches_fp32_product(ak, bk, rows, groups):
    import chunked_linear_attention_amd._lib as L
    lib = L.load()
    # K = 448: seven 64-deep steps, so the eight-wave tile's second group has
    # one step fewer than the first
    M, N, K = 512 if rows == 256 else 384, 256, 448
    g = torch.Generator(device="cuda").manual_seed(11 + 2 * ak + bk)
    a = torch.randn((K, M) if ak else (M, K), device="cuda", generator=g).to(torch.bfloat16)
    b = torch.randn((K, N) if bk else (N, K), device="cuda", generator=g).to(torch.bfloat16)
    c = torch.full((M, N), float("nan"), device="cuda")
    st = torch.cuda.current_stream()
    assert lib.ttt_probe_gemm_bf16(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, ak, bk, rows, groups,
                                   st.cuda_stream) == 0
    ref = (a.float().t() if ak else a.float()) @ (b.float() if bk else b.float().t())
    torch.cuda.synchronize()
    assert torch.isfinite(c).all()
    assert float((c - ref).abs().max() / ref.abs().max()) < 1e-5


def test_probe_argument_checks():
    import chunked_linear_attention_amd._lib as L
    lib = L.load()
    x = torch.empty(128 * 128, device="cuda", dtype=torch.bfloat16)
    c = torch.empty(128 * 128, device="cuda")
    assert lib.ttt_probe_gemm_bf16(x.data_ptr(), x.data_ptr(), c.data_ptr(), 100, 128, 64, 0, 0, 128, 1, None) == L.TTT_EINVAL
    assert lib.ttt_probe_gemm_bf16(x.data_ptr(), x.data_ptr(), c.data_ptr(), 128, 128, 96, 0, 0, 128, 1, None) == L.TTT_EINVAL
    assert lib.ttt_probe_gemm_bf16(x.data_ptr(), x.data_ptr(), c.data_ptr(), 128, 128, 64, 0, 0, 256, 1, None) == L.TTT_EINVAL
    assert lib.ttt_probe_gemm_bf16(x.data_ptr(), x.data_ptr(), c.data_ptr(), 128, 128, 64, 0, 0, 96, 1, None) == L.TTT_EINVAL
    assert lib.ttt_probe_gemm_bf16(x.data_ptr(), x.data_ptr(), c.data_ptr(), 128, 128, 64, 0, 0, 64, 2, None) == L.TTT_EINVAL
    assert lib.ttt_probe_gemm_bf16(x.data_ptr(), x.data_ptr(), c.data_ptr(), 128, 128, 64, 0, 0, 128, 3, None) == L.TTT_EINVAL
    assert lib.ttt_probe_gemm_bf16(x.data_ptr(), x.data_ptr(), c.data_ptr(), 256, 128, 64, 0, 0, 256, 2, None) == L.TTT_EINVAL
    assert lib.ttt_probe_mfma_bf16(c.data_ptr(), 0, 1, None) == L.TTT_EINVAL
