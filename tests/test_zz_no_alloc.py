"""hq_encode_noalloc (the encode whose workspace is the library's static
device scratch) against hq_encode (a caller workspace), through the C ABI.

Two calls in a row on one stream, the second on a smaller input: the second
must not see anything the first left in the shared scratch.  Stream words,
offsets and Rice parameters must equal hq_encode's bit for bit (integer
outputs), including the words past the stream's end, which neither writes.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

SEED = 0x5EED0001


def _enc_pair(hq, plan, x, ws, status):
    n = x.numel() // 128
    nw = plan.bound_words(n)
    fill = torch.tensor(0x5A5A5A5A, dtype=torch.int64).to(torch.int32).item()
    ref = (torch.full((nw,), fill, dtype=torch.int32, device="cuda"),
           torch.full((n + 1,), -7, dtype=torch.int64, device="cuda"),
           torch.full((n,), 0xEE, dtype=torch.uint8, device="cuda"))
    got = tuple(t.clone() for t in ref)
    hq.encode(plan, x, ws, out=ref)
    hq.encode_noalloc(plan, x, status, out=got)
    hq.check(ws)
    hq.check(status)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("lat", ["E8", "D4", "A2", "Z"])
def test_noalloc_equals_encode_twice_second_smaller(lat):
    import lattice_vq_entropy_amd as hq
    from lattice_vq_entropy_amd import workloads as W
    print(f"noalloc: lattice {lat}", flush=True)
    plan = hq.Plan(lat, 4.0, SEED).set_alpha(0.004)
    status = hq.status_block()
    ws = plan.workspace(hq.NOALLOC_MAX_TILES)
    # a large call (the size limit, bf16) then a smaller ragged one (fp32)
    x1 = W.c2("cuda", rows=hq.NOALLOC_MAX_TILES // 8, cols=1024, seed=11)
    x2 = W.c2("cuda", rows=333, cols=384, seed=12).float()
    for x in (x1, x2):
        ref, got = _enc_pair(hq, plan, x, ws, status)
        for a, b in zip(ref, got):
            assert torch.equal(a, b)
        n = x.numel() // 128
        assert int(got[1][n].item()) > 0


def test_noalloc_reports_data_errors_in_the_status_block():
    import lattice_vq_entropy_amd as hq
    plan = hq.Plan("E8", 4.0, SEED).set_alpha(0.004)
    status = hq.status_block()
    x = torch.randn(64 * 128, device="cuda") * 0.02
    x[1000] = float("nan")
    n = x.numel() // 128
    out = hq.alloc_stream(plan, n)
    hq.encode_noalloc(plan, x, status, out=out)
    assert hq.status_sync(status) == hq.ERR_NONFINITE
    assert hq.status_sync(status) == hq.OK  # read and cleared
    # a clean call afterwards reports nothing
    x[1000] = 0.0
    hq.encode_noalloc(plan, x, status, out=out)
    assert hq.status_sync(status) == hq.OK


def test_noalloc_rejects_more_tiles_than_the_scratch_holds():
    import lattice_vq_entropy_amd as hq
    plan = hq.Plan("E8", 4.0, SEED).set_alpha(0.004)
    status = hq.status_block()
    n = hq.NOALLOC_MAX_TILES + 1
    x = torch.zeros(n * 128, dtype=torch.bfloat16, device="cuda")
    out = hq.alloc_stream(plan, n)
    with pytest.raises(hq.HQError) as e:
        hq.encode_noalloc(plan, x, status, out=out)
    assert e.value.code == hq.ERR_ARG
