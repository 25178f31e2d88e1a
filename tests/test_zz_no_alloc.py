"""vc_quantize_noalloc (the quantiser for callers that cannot allocate: its scratch is the
library's own device array) against vc_quantize with a caller workspace, through the C ABI:
every output bit-identical, on two calls in a row, the second on a smaller input (other head
size, no permutation, other flags), so the second call runs on the array the first one left."""
import pytest
import torch

pytestmark = pytest.mark.gpu

vc = pytest.importorskip("bit_attention_video_online_amd")


def _inputs(B, H, N, d, seed, perm):
    g = torch.Generator(device="cuda").manual_seed(seed)
    Q = torch.randn((B, H, N, d), generator=g, device="cuda").to(torch.bfloat16)
    K = (torch.randn((B, H, N, d), generator=g, device="cuda") + 1.5).to(torch.bfloat16)
    V = (torch.randn((B, H, N, d), generator=g, device="cuda") * 2.0).to(torch.bfloat16)
    P = None
    if perm:
        P = torch.stack([torch.stack([torch.randperm(N, generator=g, device="cuda") for _ in range(H)])
                         for _ in range(B)]).to(torch.int32).contiguous()
    return Q, K, V, P


@pytest.mark.parametrize("case", [0, 1])
def test_noalloc_quantize_equals_workspace_path(case):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # the video workload's size (59.1 MiB of the 64 MiB scratch), then a smaller head size
    shapes = [((1, 40, 70400, 128), vc.VC_F_KSMOOTH | vc.VC_F_VSMOOTH, True),
              ((2, 3, 1024, 64), vc.VC_F_KSMOOTH, False)]
    for i, ((B, H, N, d), flags, perm) in enumerate(shapes if case == 0 else shapes[::-1][:1] + shapes[:1]):
        print("[noalloc] call %d: B=%d H=%d N=%d d=%d flags=%d" % (i, B, H, N, d, flags), flush=True)
        Q, K, V, P = _inputs(B, H, N, d, 100 + i, perm)
        ref = vc.quantize_outputs(B, H, N, d)
        vc.vc_quantize(Q, K, V, P, flags, ref)
        got = vc.quantize_outputs(B, H, N, d)
        for t in got.values():
            t.fill_(0)  # torch's fill kernel, not a memset: outputs start from known bytes
        vc.vc_quantize_noalloc(Q, K, V, P, flags, got)
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(got[k].view(torch.uint8), ref[k].view(torch.uint8)), (i, k)
        del Q, K, V, P, ref, got
        torch.cuda.empty_cache()
