"""The Python binding's argument checks: every tensor a call takes (inputs,
caller-provided outputs, gradients, workspace, offsets) must have its shape,
dtype and layout and sit on the device of q, else the call raises before
anything reaches the library (a kernel given a host pointer or a short
buffer would fault).  The CPU tests pass host tensors to every entry point;
the GPU tests change one argument of a valid call at a time."""
import pytest
import torch

import long_sequence_block_amd as lsb

T, H, D, B, W = 100, 2, 64, 32, 2
NB = -(-T // 32) + 2   # token blocks for two users


def _host_args():
    x = torch.zeros(T, H, D, dtype=torch.bfloat16)
    u8 = torch.zeros(T, H, D, dtype=torch.uint8)
    sc = torch.full((H, T, D // 32), 127, dtype=torch.uint8)
    tok = torch.zeros(H, D, 32 * NB, dtype=torch.uint8)
    tsc = torch.full((H, NB, D), 127, dtype=torch.uint8)
    lse = torch.zeros(H, T)
    off = torch.tensor([0, 40, T], dtype=torch.int32)
    return x, u8, sc, tok, tsc, lse, off


def _calls(x, u8, sc, tok, tsc, lse, off):
    s = 0.125
    return {
        "fwd": lambda: lsb.fwd(x, x, x, off, B, W, s),
        "bwd": lambda: lsb.bwd(x, x, x, x, x, lse, off, B, W, s),
        "bwd_noalloc": lambda: lsb.bwd_noalloc(x, x, x, x, x, lse, off, B, W, s),
        "swa_fwd": lambda: lsb.swa_fwd(x, x, x, off, 37, s),
        "swa_bwd": lambda: lsb.swa_bwd(x, x, x, x, x, lse, off, 37, s),
        "rope": lambda: lsb.rope(x, x, off),
        "rope_bwd": lambda: lsb.rope_bwd(x, x, x, x, x, lse, off, B, W, s),
        "gdpa_fwd": lambda: lsb.gdpa_fwd(x, x, x, off, B, W, s, lsb.GDPA_SILU),
        "gdpa_bwd": lambda: lsb.gdpa_bwd(x, x, x, x, off, B, W, s, lsb.GDPA_SILU),
        "mx_fwd": lambda: lsb.mx_fwd(u8, sc, u8, sc, x, off, B, W, s),
        "mxpv_fwd": lambda: lsb.mxpv_fwd(u8, sc, u8, sc, tok, tsc, off, B, W, s),
        "mx_bwd": lambda: lsb.mx_bwd(u8, sc, u8, sc, u8, sc, u8, sc, tok, tsc, tok, tsc, tok,
                                     tsc, x, lse, off, B, W, s),
    }


@pytest.mark.parametrize("name", sorted(_calls(*_host_args())))
def test_host_tensors_are_rejected(name):
    with pytest.raises(ValueError):
        _calls(*_host_args())[name]()


@pytest.mark.gpu
def test_each_wrong_argument_is_rejected():
    dev = torch.device("cuda:0")
    x, u8, sc, tok, tsc, lse, off = (t.to(dev) for t in _host_args())
    s = 0.125
    # valid calls first: the checks accept what the library takes
    out, l = lsb.fwd(x, x, x, off, B, W, s)
    lsb.bwd(x, x, x, out, x, l, off, B, W, s)
    torch.cuda.synchronize()
    short = torch.zeros(T - 1, H, D, dtype=torch.bfloat16, device=dev)
    f32 = torch.zeros(T, H, D, device=dev)
    strided = torch.zeros(T, H, 2 * D, dtype=torch.bfloat16, device=dev)[:, :, :D]
    bad = {
        "out too short": lambda: lsb.fwd(x, x, x, off, B, W, s, out=short),
        "out of another dtype": lambda: lsb.fwd(x, x, x, off, B, W, s, out=f32),
        "lse transposed": lambda: lsb.fwd(x, x, x, off, B, W, s,
                                          lse=torch.zeros(T, H, device=dev)),
        "lse on the host": lambda: lsb.bwd(x, x, x, out, x, l.cpu(), off, B, W, s),
        "strided k": lambda: lsb.fwd(x, strided, x, off, B, W, s),
        "offsets on the host": lambda: lsb.fwd(x, x, x, off.cpu(), B, W, s),
        "int64 offsets": lambda: lsb.fwd(x, x, x, off.long(), B, W, s),
        "two grads": lambda: lsb.bwd(x, x, x, out, x, l, off, B, W, s, grads=(x, x)),
        "short grad": lambda: lsb.bwd(x, x, x, out, x, l, off, B, W, s,
                                      grads=(torch.empty_like(x), short, torch.empty_like(x))),
        "workspace on the host": lambda: lsb.bwd(x, x, x, out, x, l, off, B, W, s,
                                                 workspace=torch.empty(1 << 20,
                                                                       dtype=torch.uint8)),
        "gdpa out too short": lambda: lsb.gdpa_fwd(x, x, x, off, B, W, s, lsb.GDPA_SILU,
                                                   out=short),
        "mx scale transposed": lambda: lsb.mx_fwd(u8, sc.transpose(0, 1).contiguous(), u8, sc,
                                                  x, off, B, W, s),
        "mxpv v_t one block short": lambda: lsb.mxpv_fwd(u8, sc, u8, sc,
                                                         tok[:, :, 32:].contiguous(), tsc, off,
                                                         B, W, s),
        "mx_bwd grads in fp32": lambda: lsb.mx_bwd(u8, sc, u8, sc, u8, sc, u8, sc, tok, tsc, tok,
                                                   tsc, tok, tsc, out, l, off, B, W, s,
                                                   grads=(f32, f32, f32)),
        "mx_bwd out in fp32": lambda: lsb.mx_bwd(u8, sc, u8, sc, u8, sc, u8, sc, tok, tsc, tok,
                                                 tsc, tok, tsc, f32, l, off, B, W, s),
    }
    for what, call in bad.items():
        print(what, flush=True)
        with pytest.raises(ValueError):
            call()
    torch.cuda.synchronize()


@pytest.mark.gpu
def test_caller_buffers_give_the_same_results():
    """out, lse, grads and workspace passed in are used as they are: the
    results equal those of a call that allocates them."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    x, k, v, do = (torch.randn(T, H, D, device=dev, generator=g).to(torch.bfloat16)
                   for _ in range(4))
    off = torch.tensor([0, 40, T], dtype=torch.int32, device=dev)
    s = 0.125
    out, lse = lsb.fwd(x, k, v, off, B, W, s)
    out2, lse2 = torch.empty_like(out), torch.empty_like(lse)
    r = lsb.fwd(x, k, v, off, B, W, s, out=out2, lse=lse2)
    assert r[0] is out2 and r[1] is lse2
    grads = lsb.bwd(x, k, v, out, do, lse, off, B, W, s)
    mine = tuple(torch.empty_like(x) for _ in range(3))
    ws = torch.empty(lsb.blockattn_bwd_workspace_size(T, 2, H, lsb.BF16), dtype=torch.uint8,
                     device=dev)
    r2 = lsb.bwd(x, k, v, out, do, lse, off, B, W, s, grads=mine, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse, lse2)
    for a, b, c in zip(grads, mine, r2):
        assert b is c
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
