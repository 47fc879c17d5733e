"""The library's calls inside a captured HIP graph: a split-K GEMM (its
partial-sum workspace and reduce kernel), an im2col + GEMM convolution, and an
implicit-GEMM convolution with table address terms (its table kernel and
buffer), one over the zero-bordered image copy (its pad kernel and buffer),
and, on a wide filter, both products from image windows (the filter copy,
the padded output-gradient copy, the padded gradient accumulator and their
kernels) are captured once on a stream that has run them before (so every
library-owned buffer already exists and nothing is allocated during capture),
then replayed several times with new inputs written eagerly in between.
Every replay must equal the eager calls bit for bit (the library is
deterministic: fixed tile plans, fixed slice order).
"""
from __future__ import annotations

import numpy as np
import pytest

import dense_gemm_03_amd as dg
from dense_gemm_03_amd import workloads as wl
from tests.gpu_util import log, to_device

pytestmark = pytest.mark.gpu


def test_graph_replays_equal_eager_calls():
    import torch
    M, N, K = 64, 4096, 8192                       # the wide class: split into K slices
    dt = dg.GEMM_DTYPE_F32
    cfg = dg.gemm_select_config_ex(dt, 0, 0, M, N, K)
    assert dg.gemm_split_k_ex(dt, cfg, 0, 0, M, N, K) > 1
    A = to_device(wl.uniform_f32((M, K), 1))
    B = to_device(wl.uniform_f32((K, N), 2))
    C = torch.empty((M, N), device="cuda:0")
    cs = (2, 6, 30, 33, 8, 5, 5, 2)                # batch, cin, h, w, cout, r, s, pad
    x = to_device(wl.uniform_f32((cs[0], cs[1], cs[2], cs[3]), 3))
    w = to_device(wl.uniform_f32((cs[4], cs[1], cs[5], cs[6]), 4))
    params = dg.conv2d_params(cs[0], cs[1], cs[2], cs[3], cs[4], cs[5], cs[6], (cs[7], cs[7]))
    rc, P, Q = dg.conv2d_output_size(params)
    assert rc == dg.GEMM_OK
    need = dg.conv2d_workspace_size(dt, params)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    y1 = torch.empty((cs[0], cs[4], P, Q), device="cuda:0")
    y2 = torch.empty_like(y1)
    y3 = torch.empty_like(y1)
    # wide filter (1 x 31): the image-window forms
    ws_ = (2, 3, 6, 200, 8, 1, 31, 0, 15)          # batch, cin, h, w, cout, r, s, ph, pw
    xw = to_device(wl.uniform_f32((ws_[0], ws_[1], ws_[2], ws_[3]), 5))
    ww = to_device(wl.uniform_f32((ws_[4], ws_[1], ws_[5], ws_[6]), 6))
    pw_ = dg.conv2d_params(ws_[0], ws_[1], ws_[2], ws_[3], ws_[4], ws_[5], ws_[6], (ws_[7], ws_[8]))
    rc, Pw, Qw = dg.conv2d_output_size(pw_)
    assert rc == dg.GEMM_OK
    dyw = to_device(wl.uniform_f32((ws_[0], ws_[4], Pw, Qw), 7))
    y4 = torch.empty((ws_[0], ws_[4], Pw, Qw), device="cuda:0")
    dw4 = torch.empty((ws_[4], ws_[1], ws_[5], ws_[6]), device="cuda:0")

    def calls(stream):
        sp = stream.cuda_stream
        dg.gemm(A, B, out=C, stream=sp)
        assert dg.conv2d_fwd(dt, dt, params, x.data_ptr(), w.data_ptr(), y1.data_ptr(),
                             ws.data_ptr(), need, sp) == dg.GEMM_OK
        assert dg.conv2d_fwd_implicit_ex(dt, dt, params, dg.CONV_ADDR_TABLE, x.data_ptr(),
                                         w.data_ptr(), y2.data_ptr(), sp) == dg.GEMM_OK
        assert dg.conv2d_fwd_implicit_ex(dt, dt, params, dg.CONV_ADDR_PADDED, x.data_ptr(),
                                         w.data_ptr(), y3.data_ptr(), sp) == dg.GEMM_OK
        assert dg.conv2d_fwd_implicit_ex(dt, dt, pw_, dg.CONV_ADDR_WINDOW, xw.data_ptr(),
                                         ww.data_ptr(), y4.data_ptr(), sp) == dg.GEMM_OK
        assert dg.conv2d_bwd_weight_implicit_ex(dt, pw_, dg.CONV_ADDR_WINDOW, xw.data_ptr(),
                                                dyw.data_ptr(), dw4.data_ptr(), sp) == dg.GEMM_OK

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls(s)                                   # creates the per-stream buffers
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        calls(s)
    torch.cuda.synchronize()

    for rep in range(3):
        A.copy_(to_device(wl.uniform_f32((M, K), 10 + rep)))
        x.copy_(to_device(wl.uniform_f32((cs[0], cs[1], cs[2], cs[3]), 20 + rep)))
        xw.copy_(to_device(wl.uniform_f32((ws_[0], ws_[1], ws_[2], ws_[3]), 30 + rep)))
        dyw.copy_(to_device(wl.uniform_f32((ws_[0], ws_[4], Pw, Qw), 40 + rep)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        C_eager = dg.gemm(A, B)
        y1_eager = dg.conv2d(x, w, padding=cs[7])
        y2_eager = dg.conv2d(x, w, padding=cs[7], implicit="table")
        y3_eager = dg.conv2d(x, w, padding=cs[7], implicit="padded")
        y4_eager = dg.conv2d(xw, ww, padding=(ws_[7], ws_[8]), implicit="window")
        dw4_eager = dg.conv2d_weight_grad(xw, dyw, tuple(ww.shape), padding=(ws_[7], ws_[8]),
                                          implicit="window")
        torch.cuda.synchronize()
        log("replay %d: gemm %s, conv %s, implicit conv %s, padded %s, window %s %s" % (
            rep, torch.equal(C, C_eager), torch.equal(y1, y1_eager), torch.equal(y2, y2_eager),
            torch.equal(y3, y3_eager), torch.equal(y4, y4_eager), torch.equal(dw4, dw4_eager)))
        assert torch.equal(C, C_eager)
        assert torch.equal(y1, y1_eager)
        assert torch.equal(y2, y2_eager)
        assert torch.equal(y3, y3_eager)
        assert torch.equal(y4, y4_eager)
        assert torch.equal(dw4, dw4_eager)
        # the replay computed the new inputs, not a stale result
        assert not np.array_equal(C.cpu().numpy(), 0)
