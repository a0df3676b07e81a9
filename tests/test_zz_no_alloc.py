"""attn_verify_noalloc (the allocation-free variant of attn_verify) through
the C ABI: on the verify workload and then on a smaller input, each result
must equal attn_verify's with a caller workspace bit for bit (same kernels,
same arithmetic) and match the fp64 oracle within the bf16 tolerance.  The
second call reuses the static scratch the first one left behind."""
import numpy as np
import pytest
import torch

from exact_attention_04_amd import synth
from oracle import ref_attention as ref
from tests import parity as P

pytestmark = pytest.mark.gpu


def raw_noalloc(q, k, v, sl, max_len, scale):
    from exact_attention_04_amd import binding as bd
    B, H, kq, d = q.shape
    Hkv, stride = k.shape[1], k.shape[2]
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, kq), float("nan"), dtype=torch.float32, device=q.device)
    rc = bd.attn_verify_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), sl.data_ptr(), max_len, stride,
                                o.data_ptr(), lse.data_ptr(), B, H, Hkv, kq, d, scale, bd.ATTN_BF16,
                                torch.cuda.current_stream().cuda_stream)
    assert rc == bd.ATTN_OK, bd.attn_strerror(rc)
    torch.cuda.synchronize()
    return o, lse


def check_against_workspace_call(q, k, v, sl, scale, what):
    from exact_attention_04_amd import binding as bd
    max_len = int(sl.max())
    P.log(f"[noalloc] {what} B={q.shape[0]} H={q.shape[1]} Hkv={k.shape[1]} kq={q.shape[2]} "
          f"lengths={sl.tolist()}")
    o_n, l_n = raw_noalloc(q, k, v, sl, max_len, scale)
    o_w, l_w = bd.verify(q, k, v, sl, max_len, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o_n, o_w) and torch.equal(l_n, l_w), what
    o_ref, l_ref = ref.verify(synth.to_f64(q), synth.to_f64(k), synth.to_f64(v), sl.cpu().numpy(), scale)
    P.log(f"    ok bitwise equal to attn_verify; {P.compare(synth.to_f64(o_n), synth.to_f64(l_n), o_ref, l_ref, 'bf16', what)}")


def test_noalloc_twice_second_smaller():
    w = synth.VERIFY_BF16
    q, k, v, sl = synth.verify_inputs(w, "cuda")
    check_against_workspace_call(q, k, v, sl, w.scale, w.name)
    rng = np.random.default_rng(31)
    lengths = torch.tensor([1500, 7, 3000], dtype=torch.int32, device="cuda")
    qs = synth.normal(rng, (3, 32, 5, 128), "bf16").cuda()
    ks = synth.normal(rng, (3, 8, 3000, 128), "bf16").cuda()
    vs = synth.normal(rng, (3, 8, 3000, 128), "bf16").cuda()
    check_against_workspace_call(qs, ks, vs, lengths, w.scale, "smaller")


def test_noalloc_in_a_captured_graph():
    """The callers this entry point is for: a call captured into a HIP graph
    (it allocates nothing, so capture needs no memory pool), replayed three
    times with eager work in between; every replay equals the eager
    workspace call bit for bit."""
    from exact_attention_04_amd import binding as bd
    w = synth.VERIFY_BF16
    q, k, v, sl = synth.verify_inputs(w, "cuda")
    max_len = int(sl.max())
    o_w, l_w = bd.verify(q, k, v, sl, max_len, scale=w.scale)
    torch.cuda.synchronize()
    o = torch.full_like(q, float("nan"))
    lse = torch.full((w.B, w.H, w.kq), float("nan"), dtype=torch.float32, device="cuda")

    def call():
        rc = bd.attn_verify_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), sl.data_ptr(), max_len, k.shape[2],
                                    o.data_ptr(), lse.data_ptr(), w.B, w.H, w.Hkv, w.kq, w.d, w.scale, bd.ATTN_BF16,
                                    torch.cuda.current_stream().cuda_stream)
        assert rc == bd.ATTN_OK, bd.attn_strerror(rc)
    call()  # the first call on the device locates the static scratch: outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        P.log(f"[noalloc] graph replay {rep}")
        assert torch.equal(o, o_w) and torch.equal(lse, l_w), rep
        o_e, l_e = bd.verify(q, k, v, sl, max_len, scale=w.scale)  # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(o_e, o_w) and torch.equal(l_e, l_w), rep
