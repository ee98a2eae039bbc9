"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same seeded, rounded inputs.

Tolerances (max |y - y_ref| / rms(y_ref), likewise for the final state): 1e-5 with fp32 I/O; 3e-3 with bf16 I/O and
fp32 state, measured with fp32 y.  bf16 y is checked to be bit-identical to round-to-nearest-even of the fp32-y run.
"""
import numpy as np
import pytest

from selective_state_space_57_amd import inputs as I
import gpu_util as G

pytestmark = pytest.mark.gpu


def _check(d, io, disc=0, softplus=True, segments=0, chans=None, y_dtype="f32"):
    torch = G.torch_dev()
    dd = G.to_dev(d)
    y, hf = G.run_gpu(dd, disc=disc, y_dtype=torch.float32, segments=segments, softplus=softplus)
    yr, hr = G.oracle_ref(d, disc=disc, softplus=softplus, chans=chans)
    yg, hg = G.to_np64(y), G.to_np64(hf)
    if chans is not None:
        yg = np.stack([yg[b, dd_] for b, dd_ in chans])
        hg = np.stack([hg[b, dd_] for b, dd_ in chans])
    tol = G.tol_for(io)
    ey, eh = G.rel_max(yg, yr), G.rel_max(hg, hr)
    assert ey <= tol, ("y", ey, tol)
    assert eh <= tol, ("h_final", eh, tol)
    return y, dd, ey, eh


def test_tiny_fp32_workload():
    w = I.WORKLOADS[0]
    d = I.scan_inputs(w)
    _check(d, w.io)


# (seed, b, D, L, N, io, disc, gate, dskip, bias, h0, segments)
CASES = [
    (1, 1, 1, 1, 16, "f32", 0, True, True, True, False, 0),
    (2, 1, 1, 1, 1, "f32", 1, False, False, False, True, 0),
    (3, 1, 5, 7, 16, "f32", 0, True, True, True, True, 0),
    (4, 2, 17, 63, 16, "f32", 0, True, False, True, True, 0),
    (5, 3, 16, 64, 16, "f32", 1, True, True, True, True, 0),
    (6, 2, 33, 65, 8, "f32", 0, False, True, True, False, 0),
    (7, 1, 31, 200, 4, "f32", 1, True, True, False, True, 0),
    (8, 2, 20, 333, 2, "f32", 0, True, True, True, True, 0),
    (9, 1, 48, 129, 1, "f32", 1, False, False, True, True, 0),
    (10, 2, 16, 257, 3, "f32", 0, True, True, True, True, 0),
    (11, 1, 9, 1000, 7, "f32", 1, True, False, True, False, 0),
    (12, 2, 40, 777, 16, "f32", 0, True, True, True, True, 3),
    (13, 1, 17, 1500, 16, "f32", 1, True, True, True, True, 7),
    (14, 3, 5, 130, 16, "f32", 0, False, False, False, True, 2),
    (15, 1, 64, 4096, 16, "f32", 0, True, True, True, True, 64),
    (16, 1, 1, 65, 16, "f32", 0, True, True, True, True, 2),
    (21, 2, 17, 63, 16, "bf16", 0, True, True, True, True, 0),
    (22, 1, 33, 500, 16, "bf16", 1, True, True, True, True, 0),
    (23, 4, 50, 129, 8, "bf16", 0, False, True, True, False, 0),
    (24, 1, 16, 2048, 16, "bf16", 0, True, True, True, True, 5),
    (25, 2, 7, 99, 1, "bf16", 1, True, False, False, True, 0),
    (26, 1, 130, 1024, 16, "bf16", 0, True, True, True, True, 16),
]


@pytest.mark.parametrize("case", CASES, ids=["s%d" % c[0] for c in CASES])
def test_random_small(case):
    seed, b, D, L, N, io, disc, gate, dskip, bias, h0, seg = case
    d = I.random_small(seed, b, D, L, N, io=io, gate=gate, dskip=dskip, bias=bias, h0=h0)
    _check(d, io, disc=disc, segments=seg)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_no_softplus(io):
    # Delta = dt directly (positive values), no bias
    r = np.random.default_rng(77)
    d = I.random_small(30, 2, 19, 150, 16, io=io, bias=False, h0=True)
    d["dt"] = I.to_storage(np.exp(r.uniform(np.log(1e-3), np.log(0.5), d["x"].shape)), io)
    _check(d, io, softplus=False)
    _check(d, io, softplus=False, disc=1)


def test_bf16_output_is_rne_of_fp32_output():
    torch = G.torch_dev()
    d = I.random_small(40, 2, 37, 301, 16, io="bf16", h0=True)
    dd = G.to_dev(d)
    y32, h32 = G.run_gpu(dd, y_dtype=torch.float32)
    y16, h16 = G.run_gpu(dd, y_dtype=torch.bfloat16)
    a = y32.cpu().numpy()
    want = G.bf16_rne(a)
    got = y16.to(torch.float32).cpu().numpy()
    assert np.array_equal(got, want)
    assert torch.equal(h32, h16)


def test_deterministic():
    torch = G.torch_dev()
    d = I.random_small(41, 3, 70, 700, 16, io="bf16", h0=True)
    dd = G.to_dev(d)
    y1, h1 = G.run_gpu(dd)
    y2, h2 = G.run_gpu(dd)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    y3, h3 = G.run_gpu(dd, segments=4)
    y4, h4 = G.run_gpu(dd, segments=4)
    assert torch.equal(y3, y4) and torch.equal(h3, h4)


def test_reset_makes_output_independent_of_the_past():
    # paper section 3.5.2 (boundary reset): Delta -> infinity at t* forgets everything before t*
    torch = G.torch_dev()
    d = I.random_small(42, 2, 21, 160, 16, io="f32", h0=True)
    ts = 77
    d["dt"] = d["dt"].copy()
    d["dt"][:, :, ts] = 1e4
    y1, h1 = G.run_gpu(G.to_dev(d))
    d2 = dict(d)
    r = np.random.default_rng(3)
    d2["x"] = d["x"].copy()
    d2["x"][:, :, :ts] = r.standard_normal(d["x"][:, :, :ts].shape).astype(np.float32)
    d2["h0"] = r.standard_normal(d["h0"].shape).astype(np.float32)
    y2, h2 = G.run_gpu(G.to_dev(d2))
    assert torch.equal(y1[:, :, ts:], y2[:, :, ts:])
    assert torch.equal(h1, h2)


def test_host_split_with_state_handoff():
    torch = G.torch_dev()
    d = I.random_small(43, 2, 24, 1000, 16, io="f32", h0=True)
    dd = G.to_dev(d)
    y, hf = G.run_gpu(dd)
    cuts = [0, 1, 64, 65, 400, 999, 1000]
    h = dd["h0"]
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        sub = dict(dd)
        for k in ("x", "dt", "z", "B", "C"):
            sub[k] = dd[k][:, :, a:b].contiguous()
        ys, h = G.run_gpu(sub, h0=h)
        parts.append(ys)
    yc = torch.cat(parts, dim=2)
    assert G.rel_max(G.to_np64(yc), G.to_np64(y)) <= 1e-5
    assert G.rel_max(G.to_np64(h), G.to_np64(hf)) <= 1e-5


@pytest.mark.parametrize("cfg", [1, 2])
def test_layer_workload_full(cfg):
    # the full-size launch the benchmark times, every output element and every final state against the oracle
    torch = G.torch_dev()
    w = I.WORKLOADS[cfg]
    d = I.scan_inputs(w)
    print("%s: scan + oracle on all %d channels" % (w.name, w.batch * w.dim), flush=True)
    y, dd, ey, eh = _check(d, w.io)
    print("%s: err y %.3e h %.3e (of rms)" % (w.name, ey, eh), flush=True)
    y16, _ = G.run_gpu(dd, y_dtype=torch.bfloat16)
    assert np.array_equal(y16.to(torch.float32).cpu().numpy(), G.bf16_rne(y.cpu().numpy()))


def test_million_length_zoh_sampled():
    """The million-step layer under ZOH through the planner (32 segments: the ZOH kernel keeps four waves per SIMD
    resident), in the launch configuration the benchmark times for its Euler leg: two blocks of 64 channels (the first
    and the last workgroups' channels) against the oracle run on them, every output and final state."""
    torch = G.torch_dev()
    import selective_state_space_57_amd as ssm
    ZOH = ssm.ZOH
    w = I.WORKLOADS[3]
    assert ssm.plan_segments(ssm.make_params(w.batch, w.dim, w.seqlen, w.dstate, ssm.SSM_BF16, disc=ssm.ZOH)) == 32
    print("million-length ZOH: generating inputs", flush=True)
    d = I.scan_inputs(w)
    y, hf = G.run_gpu(G.to_dev(d), disc=ZOH, y_dtype=torch.float32)
    yg = y.cpu().numpy()
    hg = hf.cpu().numpy().astype(np.float64)
    del y
    for c0 in (0, w.dim - 64):
        sub = {k: v for k, v in d.items()}
        for k in ("x", "dt", "z"):
            sub[k] = d[k][:, c0:c0 + 64]
        for k in ("A", "dt_bias", "Dskip"):
            sub[k] = d[k][c0:c0 + 64]
        yr, hr = G.oracle_ref(sub, disc=ZOH)
        ey = G.rel_max(yg[:, c0:c0 + 64].astype(np.float64), yr)
        eh = G.rel_max(hg[:, c0:c0 + 64], hr)
        print("million-length ZOH: channels %d..%d: err y %.3e h %.3e (of rms)" % (c0, c0 + 63, ey, eh), flush=True)
        assert ey <= G.TOL_BF16 and eh <= G.TOL_BF16, (c0, ey, eh)


def test_million_length_full_and_16_segment_handoff():
    # one batch element, 512 channels, 2^20 steps: the planner's segmented path (segments pass, carry, correction).
    # Every output and final state is compared with the oracle, 64 channels at a time (fp64 copies of one block
    # of x, dt, z and y hold 2 GB).
    torch = G.torch_dev()
    w = I.WORKLOADS[3]
    print("million-length: generating inputs", flush=True)
    d = I.scan_inputs(w)
    dd = G.to_dev(d)
    y, hf = G.run_gpu(dd, y_dtype=torch.float32)
    yg = y.cpu().numpy()
    hg = hf.cpu().numpy().astype(np.float64)
    del y
    blk = 64
    num_y, num_h, ss_y, ss_h, cnt = 0.0, 0.0, 0.0, 0.0, 0
    for c0 in range(0, w.dim, blk):
        sub = {k: v for k, v in d.items()}
        for k in ("x", "dt", "z"):
            sub[k] = d[k][:, c0:c0 + blk]
        for k in ("A", "dt_bias", "Dskip"):
            sub[k] = d[k][c0:c0 + blk]
        yr, hr = G.oracle_ref(sub)
        num_y = max(num_y, float(np.max(np.abs(yg[:, c0:c0 + blk].astype(np.float64) - yr))))
        num_h = max(num_h, float(np.max(np.abs(hg[:, c0:c0 + blk] - hr))))
        ss_y += float(np.sum(yr * yr))
        ss_h += float(np.sum(hr * hr))
        cnt += yr.size
        print("million-length: channels %d..%d checked" % (c0, c0 + blk - 1), flush=True)
    ey = num_y / np.sqrt(ss_y / cnt)
    eh = num_h / np.sqrt(ss_h / (w.batch * w.dim * w.dstate))
    print("million-length: err y %.3e h %.3e (of rms); 16-segment hand-off" % (ey, eh), flush=True)
    assert ey <= G.TOL_BF16, ("y", ey)
    assert eh <= G.TOL_BF16, ("h_final", eh)
    # the same sequence as 16 host-level segments of 65,536 steps with the state handed over
    seg = w.seqlen // 16
    h = None
    parts = []
    for s in range(16):
        sub = dict(dd)
        for k in ("x", "dt", "z", "B", "C"):
            sub[k] = dd[k][:, :, s * seg:(s + 1) * seg].contiguous()
        ys, h = G.run_gpu(sub, y_dtype=torch.float32, h0=h)
        parts.append(ys)
    yc = torch.cat(parts, dim=2)
    assert G.rel_max(G.to_np64(yc), yg.astype(np.float64)) <= G.TOL_BF16
    assert G.rel_max(G.to_np64(h), hg) <= G.TOL_BF16
