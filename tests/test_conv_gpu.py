"""GPU parity of the scan fed through the causal depthwise convolution + SiLU (ssm_conv_scan_fwd) and of its decode
step (ssm_conv_state_update), against the fp64 oracle: oracle.conv1d followed by oracle.scan on its output."""
import numpy as np
import pytest

import oracle
import selective_state_space_57_amd as ssm
from selective_state_space_57_amd import inputs as I
import gpu_util as G

pytestmark = pytest.mark.gpu


def ref_conv_scan(d, cv, disc=0, silu=True, softplus=True):
    f = I.as_f64(d)
    st = None if cv["conv_state"] is None else cv["conv_state"].astype(np.float64)
    u, so = oracle.conv1d(f["x"], cv["conv_w"].astype(np.float64), bias=cv["conv_b"].astype(np.float64),
                          state_in=st, silu=silu)
    y, h = oracle.scan(u, f["dt"], f["A"], f["B"], f["C"], dt_bias=f["dt_bias"], Dskip=f["Dskip"], z=f["z"],
                       h0=f["h0"], disc=disc, softplus=softplus)
    return y, h, so


def run_conv_scan(dd, dc, disc=0, silu=True, segments=0, state_out=None):
    torch = G.torch_dev()
    y, hf = ssm.conv_scan_fwd(dd["x"], dc["conv_w"], dd["dt"], dd["A"], dd["B"], dd["C"], dt_bias=dd["dt_bias"],
                              Dskip=dd["Dskip"], z=dd["z"], h0=dd["h0"], conv_bias=dc["conv_b"],
                              conv_state=dc["conv_state"], conv_state_out=state_out, activation=silu,
                              y_dtype=torch.float32, disc=disc, segments=segments)
    torch.cuda.synchronize()
    return y, hf


@pytest.mark.parametrize("seed,b,D,L,N,io,width,state,silu,disc,segments", [
    (1, 1, 16, 64, 16, "f32", 4, False, True, 0, 0),
    (2, 2, 17, 100, 16, "f32", 4, True, True, 0, 0),
    (3, 2, 33, 257, 16, "bf16", 4, True, True, 0, 0),
    (4, 1, 5, 1, 16, "f32", 4, True, True, 0, 0),      # one step: the whole window comes from the state
    (5, 2, 9, 2, 16, "f32", 3, True, True, 1, 0),      # shorter than the window, ZOH
    (6, 1, 20, 130, 5, "f32", 2, True, False, 0, 0),   # width 2, no activation, N = 5
    (7, 3, 12, 77, 16, "bf16", 1, False, True, 0, 0),  # width 1: a per-channel scale + bias + SiLU
    (8, 2, 19, 700, 16, "f32", 4, True, True, 0, 4),   # four L-segments: windows across segment starts
    (9, 1, 64, 1500, 16, "bf16", 4, False, True, 1, 3),
])
def test_conv_scan_random(seed, b, D, L, N, io, width, state, silu, disc, segments):
    torch = G.torch_dev()
    d = I.random_small(seed, b, D, L, N, io=io, h0=True)
    cv = I.random_small_conv(seed, b, D, N, width=width, with_state=state)
    dd, dc = G.to_dev(d), G.to_dev(cv)
    so = torch.empty((b, D, width - 1), dtype=torch.float32, device="cuda") if width > 1 else None
    y, hf = run_conv_scan(dd, dc, disc=disc, silu=silu, segments=segments, state_out=so)
    yr, hr, sr = ref_conv_scan(d, cv, disc=disc, silu=silu)
    tol = G.tol_for(io)
    assert G.rel_max(G.to_np64(y), yr) <= tol
    assert G.rel_max(G.to_np64(hf), hr) <= tol
    if so is not None:
        assert np.array_equal(so.cpu().numpy().astype(np.float64), sr)  # the window is copied, not computed


def test_conv_state_out_may_alias_state_in():
    torch = G.torch_dev()
    d = I.random_small(20, 2, 11, 50, 16, io="f32", h0=True)
    cv = I.random_small_conv(20, 2, 11, 16, width=4, with_state=True)
    dd, dc = G.to_dev(d), G.to_dev(cv)
    yr, hr, sr = ref_conv_scan(d, cv)
    y, _ = run_conv_scan(dd, dc, state_out=dc["conv_state"])  # in place
    assert G.rel_max(G.to_np64(y), yr) <= G.TOL_F32
    assert np.array_equal(dc["conv_state"].cpu().numpy().astype(np.float64), sr)


def test_conv_split_sequence_hand_off():
    # two calls with the windows and states handed over equal one call over the whole sequence
    torch = G.torch_dev()
    d = I.random_small(21, 2, 24, 300, 16, io="f32", h0=True)
    cv = I.random_small_conv(21, 2, 24, 16, width=4, with_state=True)
    dd, dc = G.to_dev(d), G.to_dev(cv)
    y_full, h_full = run_conv_scan(dd, dc)
    first = {k: (v[:, :, :128].contiguous() if k in ("x", "dt", "z", "B", "C") else v) for k, v in dd.items()}
    second = {k: (v[:, :, 128:].contiguous() if k in ("x", "dt", "z", "B", "C") else v) for k, v in dd.items()}
    mid = torch.empty_like(dc["conv_state"])
    y1, h1 = run_conv_scan(first, dc, state_out=mid)
    second["h0"] = h1
    y2, h2 = run_conv_scan(second, dict(dc, conv_state=mid))
    yy = torch.cat([y1, y2], dim=2)
    assert G.rel_max(G.to_np64(yy), G.to_np64(y_full)) <= 1e-6
    assert G.rel_max(G.to_np64(h2), G.to_np64(h_full)) <= 1e-6


@pytest.mark.parametrize("io,width,disc", [("f32", 4, 0), ("bf16", 4, 1), ("f32", 2, 0)])
def test_conv_decode_equals_conv_scan(io, width, disc):
    torch = G.torch_dev()
    T = 40
    d = I.random_small(30 + width, 3, 45, T, 16, io=io, h0=True)
    cv = I.random_small_conv(30 + width, 3, 45, 16, width=width, with_state=True)
    dd, dc = G.to_dev(d), G.to_dev(cv)
    y_scan, h_scan = run_conv_scan(dd, dc, disc=disc)
    state = dd["h0"].clone()
    win = dc["conv_state"].clone()
    ys = []
    for t in range(T):
        sl = lambda k: dd[k][:, :, t].contiguous()
        ys.append(ssm.conv_state_update(state, win, sl("x"), dc["conv_w"], sl("dt"), dd["A"], sl("B"), sl("C"),
                                        dt_bias=dd["dt_bias"], Dskip=dd["Dskip"], z=sl("z"), conv_bias=dc["conv_b"],
                                        y_dtype=torch.float32, disc=disc))
    torch.cuda.synchronize()
    yd = torch.stack(ys, dim=2)
    assert G.rel_max(G.to_np64(yd), G.to_np64(y_scan)) <= 1e-5
    assert G.rel_max(G.to_np64(state), G.to_np64(h_scan)) <= 1e-5
    yr, hr, sr = ref_conv_scan(d, cv, disc=disc)
    assert G.rel_max(G.to_np64(yd), yr) <= G.tol_for(io)
    assert np.array_equal(win.cpu().numpy().astype(np.float64), sr)


def test_conv_scan_full_size():
    """The 2.8B layer with the width-4 convolution and SiLU, in the benchmark's launch configuration: every output and
    final state against the oracle's convolution then scan (multithreaded)."""
    torch = G.torch_dev()
    w = I.WORKLOADS[2]
    d = I.scan_inputs(w)
    cv = I.conv_params(w, 4)
    dd, dc = G.to_dev(d), G.to_dev(cv)
    y, hf = run_conv_scan(dd, dc)
    yr, hr, _ = ref_conv_scan(d, dict(cv, conv_state=None))
    ey, eh = G.rel_max(G.to_np64(y), yr), G.rel_max(G.to_np64(hf), hr)
    print("conv scan full size: y err %.2e, h err %.2e" % (ey, eh), flush=True)
    assert ey <= G.TOL_BF16 and eh <= G.TOL_BF16, (ey, eh)


# ---- the convolution on its own (recompute for training) and its backward

@pytest.mark.parametrize("seed,b,D,L,io,width,state,silu", [
    (21, 2, 17, 100, "f32", 4, True, True),
    (22, 1, 9, 2, "f32", 4, True, True),        # shorter than the window
    (23, 3, 12, 77, "bf16", 3, False, True),
    (24, 2, 8, 130, "f32", 1, False, False),    # width 1, no activation
    (25, 2, 64, 1000, "bf16", 4, True, True),
    # rows of a multiple of 8 steps take the 16-byte path: first block (window), interior blocks, last block
    (26, 3, 10, 256, "f32", 2, True, True),
    (27, 1, 5, 8, "bf16", 4, True, True),       # one block
    (28, 2, 7, 24, "f32", 3, True, False),      # first, one interior, last
    (29, 2, 6, 64, "bf16", 1, False, True),
    (30, 1, 3, 1, "f32", 4, True, True),        # a single step
    (31, 2, 3, 2048, "bf16", 4, True, True),    # rows of 128 forward blocks: a wave shares one row
    (32, 1, 4, 1040, "f32", 3, True, True),     # 16-step forward blocks, ragged 8-step backward tail
])
def test_conv1d_fwd_and_bwd(seed, b, D, L, io, width, state, silu):
    torch = G.torch_dev()
    d = I.random_small(seed, b, D, L, 16, io=io)
    cv = I.random_small_conv(seed, b, D, 16, width=width, with_state=state)
    cots = I.random_small_cotangents(seed, b, D, L, 16, io="f32")
    dd, dc = G.to_dev(d), G.to_dev(cv)
    f = I.as_f64(d)
    st = None if cv["conv_state"] is None else cv["conv_state"].astype(np.float64)
    w64, b64 = cv["conv_w"].astype(np.float64), cv["conv_b"].astype(np.float64)
    # forward
    u = ssm.conv1d_fwd(dd["x"], dc["conv_w"], dc["conv_b"], dc["conv_state"], activation=silu, u_dtype=torch.float32)
    torch.cuda.synchronize()
    ur, _ = oracle.conv1d(f["x"], w64, bias=b64, state_in=st, silu=silu)
    assert G.rel_max(G.to_np64(u), ur) <= 1e-6
    # backward, with a gradient for the returned window too
    du = torch.from_numpy(cots["dy"]).cuda()
    dso = (torch.from_numpy(np.random.default_rng(seed).standard_normal((b, D, width - 1)).astype(np.float32)).cuda()
           if width > 1 else None)
    g = ssm.conv1d_bwd(dd["x"], dc["conv_w"], du, dc["conv_b"], dc["conv_state"], dso, activation=silu)
    torch.cuda.synchronize()
    gr = oracle.conv1d_bwd(f["x"], w64, cots["dy"].astype(np.float64), bias=b64, state_in=st,
                           dstate_out=None if dso is None else dso.cpu().numpy().astype(np.float64), silu=silu)
    for k, tol in (("dx", 1e-5), ("dweight", 1e-5), ("dbias", 1e-5), ("dstate_in", 1e-5)):
        rk = {"dweight": "dw"}.get(k, k)
        if gr[rk].size == 0:
            continue
        e = G.rel_max(G.to_np64(g[k]), gr[rk])
        assert e <= tol, (k, e)
    # deterministic
    g2 = ssm.conv1d_bwd(dd["x"], dc["conv_w"], du, dc["conv_b"], dc["conv_state"], dso, activation=silu)
    torch.cuda.synchronize()
    assert all(torch.equal(g[k], g2[k]) for k in g)


@pytest.mark.parametrize("L", [96, 101])
def test_conv1d_bf16_outputs(L):
    # u and dx in bf16 are the round-to-nearest-even of the fp32 results on the same inputs (vector and scalar paths)
    torch = G.torch_dev()
    b, D = 2, 11
    d = I.random_small(41, b, D, L, 16, io="bf16")
    cv = I.random_small_conv(41, b, D, 16, width=4, with_state=True)
    dd, dc = G.to_dev(d), G.to_dev(cv)
    u32 = ssm.conv1d_fwd(dd["x"], dc["conv_w"], dc["conv_b"], dc["conv_state"], u_dtype=torch.float32)
    u16 = ssm.conv1d_fwd(dd["x"], dc["conv_w"], dc["conv_b"], dc["conv_state"], u_dtype=torch.bfloat16)
    du16 = torch.randn((b, D, L), generator=torch.Generator().manual_seed(41)).to(torch.bfloat16).cuda()
    g32 = ssm.conv1d_bwd(dd["x"], dc["conv_w"], du16.float(), dc["conv_b"], dc["conv_state"])
    g16 = ssm.conv1d_bwd(dd["x"], dc["conv_w"], du16, dc["conv_b"], dc["conv_state"])
    torch.cuda.synchronize()
    assert torch.equal(u16.view(torch.int16), u32.to(torch.bfloat16).view(torch.int16))
    assert torch.equal(g16["dx"].view(torch.int16), g32["dx"].to(torch.bfloat16).view(torch.int16))
    for k in ("dweight", "dbias", "dstate_in"):
        assert torch.equal(g16[k], g32[k]), k


def test_conv_scan_training_chain():
    # forward through the fused convolution + scan; backward: recompute u, scan backward (dL/du), convolution backward.
    # Against the oracle composition: conv1d -> scan_bwd on its output -> conv1d_bwd.
    torch = G.torch_dev()
    b, D, L, N, width = 2, 24, 300, 16, 4
    d = I.random_small(31, b, D, L, N, io="f32", h0=True)
    cv = I.random_small_conv(31, b, D, N, width=width, with_state=True)
    cots = I.random_small_cotangents(31, b, D, L, N, io="f32", dh_final=True)
    dd, dc = G.to_dev(d), G.to_dev(cv)
    u = ssm.conv1d_fwd(dd["x"], dc["conv_w"], dc["conv_b"], dc["conv_state"], u_dtype=torch.float32)
    dy, dhf = torch.from_numpy(cots["dy"]).cuda(), torch.from_numpy(cots["dh_final"]).cuda()
    gs = ssm.scan_bwd(u, dd["dt"], dd["A"], dd["B"], dd["C"], dy, dt_bias=dd["dt_bias"], Dskip=dd["Dskip"],
                      z=dd["z"], h0=dd["h0"], dh_final=dhf)
    gc = ssm.conv1d_bwd(dd["x"], dc["conv_w"], gs["dx"], dc["conv_b"], dc["conv_state"])
    torch.cuda.synchronize()
    f = I.as_f64(d)
    w64, b64, st = (cv["conv_w"].astype(np.float64), cv["conv_b"].astype(np.float64),
                    cv["conv_state"].astype(np.float64))
    ur, _ = oracle.conv1d(f["x"], w64, bias=b64, state_in=st)
    gsr = oracle.scan_bwd(ur, f["dt"], f["A"], f["B"], f["C"], cots["dy"].astype(np.float64), dt_bias=f["dt_bias"],
                          Dskip=f["Dskip"], z=f["z"], h0=f["h0"], dh_final=cots["dh_final"].astype(np.float64))
    gcr = oracle.conv1d_bwd(f["x"], w64, gsr["dx"], bias=b64, state_in=st)
    for k, rk in (("dx", "dx"), ("dweight", "dw"), ("dbias", "dbias"), ("dstate_in", "dstate_in")):
        e = G.rel_max(G.to_np64(gc[k]), gcr[rk])
        assert e <= 1e-4, (k, e)
    assert G.rel_max(G.to_np64(gs["dA"]), gsr["dA"]) <= 1e-4


def test_conv1d_full_size():
    """The convolution on its own and its backward at the size the benchmark times (4 x 5120 x 4096, width 4, SiLU,
    bf16 x, u, du and dx, the same launch configurations): fp32-output runs against the oracle over the whole tensors,
    and the bf16 outputs equal to their round-to-nearest-even."""
    torch = G.torch_dev()
    w = I.WORKLOADS[2]
    x = I.scan_inputs(w)["x"]
    cv = I.conv_params(w, 4)
    du_bits = I.cotangents(w)["dy"]   # bf16, as the benchmark's du
    dd = G.to_dev({"x": x, "du": du_bits})
    dc = G.to_dev(cv)
    u32 = ssm.conv1d_fwd(dd["x"], dc["conv_w"], dc["conv_b"], None, activation=True, u_dtype=torch.float32)
    u16 = ssm.conv1d_fwd(dd["x"], dc["conv_w"], dc["conv_b"], None, activation=True, u_dtype=torch.bfloat16)
    g32 = ssm.conv1d_bwd(dd["x"], dc["conv_w"], dd["du"].to(torch.float32), dc["conv_b"], None, None, activation=True)
    g16 = ssm.conv1d_bwd(dd["x"], dc["conv_w"], dd["du"], dc["conv_b"], None, None, activation=True)
    torch.cuda.synchronize()
    assert np.array_equal(u16.to(torch.float32).cpu().numpy(), G.bf16_rne(u32.cpu().numpy()))
    assert np.array_equal(g16["dx"].to(torch.float32).cpu().numpy(), G.bf16_rne(g32["dx"].cpu().numpy()))
    assert torch.equal(g16["dweight"], g32["dweight"]) and torch.equal(g16["dbias"], g32["dbias"])
    x64, du64 = I.to_f64(x, w.io), I.to_f64(du_bits, w.io)
    w64, b64 = cv["conv_w"].astype(np.float64), cv["conv_b"].astype(np.float64)
    ur, _ = oracle.conv1d(x64, w64, bias=b64, silu=True)
    gr = oracle.conv1d_bwd(x64, w64, du64, bias=b64, silu=True)
    # fp32 evaluation: four products, the bias, SiLU's exponential and reciprocal, about an ulp each, so up to about
    # 8 x 2^-24 of |u|; over millions of outputs the largest |u| are several times rms(u): the fp32 bar, 1e-5 of rms
    e = {"u": G.rel_max(G.to_np64(u32), ur), "dx": G.rel_max(G.to_np64(g32["dx"]), gr["dx"]),
         "dw": G.rel_max(G.to_np64(g32["dweight"]), gr["dw"]), "dbias": G.rel_max(G.to_np64(g32["dbias"]), gr["dbias"])}
    print("conv1d full size:", {k: "%.2e" % v for k, v in e.items()}, flush=True)
    assert e["u"] <= G.TOL_F32 and e["dx"] <= 1e-5 and e["dw"] <= 1e-5 and e["dbias"] <= 1e-5, e
