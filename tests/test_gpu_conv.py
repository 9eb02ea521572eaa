"""GPU parity of the short causal conv (gdn_conv1d, gdn_conv1d_update) against the oracle.

Bars: the conv states are inputs moved between buffers, so the pool is compared bit
for bit (and untouched slots / skipped rows keep their bytes).  The outputs are the
fp32 sum of K products and the bias, then silu, rounded to bf16: each element is
within one bf16 ulp of the float64 oracle (|d| <= 2^-8 |ref| + 1e-5, the 1e-5 covering
the fp32 sum and the hardware exp / reciprocal in silu), which also implies the
rel-L2 <= 2e-3 bar of the layer.
"""
import numpy as np
import pytest
import torch

import oracle
from hybrid_model_linear_amd import synth
from gpu_util import assert_close, upload

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _dev(x, dt=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dt)


def _check_out(got, ref, what):
    got = np.asarray(got, np.float64)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5
    bad = np.abs(got - ref) > bound
    assert not bad.any(), (what, int(bad.sum()), np.argwhere(bad)[:5], got[bad][:5], ref[bad][:5])
    num = np.linalg.norm(got - ref)
    den = np.linalg.norm(ref)
    assert num <= 2e-3 * max(den, 1e-30), (what, num / den)


def _upload_conv(c):
    return dict(x=_dev(c.x), w=_dev(c.weight), b=_dev(c.bias), cu=_dev(c.cu_seqlens, torch.int32),
                slot=_dev(c.slot, torch.int32), has_init=_dev(c.has_init, torch.int32),
                pool=_dev(c.pool))


def _run_and_check(gdn, c, K, act, use_bias, keep_pool=False):
    d = _upload_conv(c)
    out = torch.randn((c.T, c.x.shape[1]), device="cuda").to(torch.bfloat16)
    out_before = out.clone()
    pool_before = d["pool"].clone()
    gdn.conv1d(d["x"], d["w"], d["b"] if use_bias else None, d["cu"], d["slot"], d["pool"],
               has_init=d["has_init"], activation=act, out=out, keep_pool=keep_pool)
    torch.cuda.synchronize()
    ref, states = oracle.causal_conv1d(c.x, c.weight, c.bias if use_bias else None, c.cu_seqlens,
                                       c.slot, c.has_init, c.pool, activation=act)
    got = out.float().cpu().numpy()
    live = ~np.isnan(ref[:, 0])
    _check_out(got[live], ref[live], f"conv K={K} act={act}")
    # rows of skipped sequences keep their bytes
    assert torch.equal(out[torch.from_numpy(~live).cuda()], out_before[torch.from_numpy(~live).cuda()])
    pool = d["pool"].cpu()
    if keep_pool:
        assert torch.equal(pool, pool_before.cpu())
        return got
    touched = np.zeros(c.pool.shape[0], bool)
    for s, st in states.items():
        touched[s] = True
        want = torch.from_numpy(st.astype(np.float32)).to(torch.bfloat16)
        assert torch.equal(pool[s], want), f"conv state of slot {s}"
    assert torch.equal(pool[torch.from_numpy(~touched)], pool_before.cpu()[torch.from_numpy(~touched)])
    return got


# lengths: empty, shorter than K - 1, tile-crossing (64-token tiles), several
# sequences inside one tile, one skipped; D = 1032 leaves a ragged channel block
LENS = (0, 1, 2, 3, 31, 33, 70, 5, 100, 0, 64, 9)
INIT = (1, 1, 0, 1, 1, 0, 1, 1, 1, 0, 1, 0)


@pytest.mark.parametrize("K,act,use_bias", [(2, True, True), (3, True, True), (4, True, True),
                                            (4, False, False)])
def test_conv1d_varlen(gdn_lib, K, act, use_bias):
    _announce(f"conv1d varlen K={K} act={act} bias={use_bias}")
    c = synth.make_conv_case(seed=300 + K, lens=LENS, D=1032, K=K, has_init=INIT, num_slots=16)
    c.slot[7] = -1
    _run_and_check(gdn_lib, c, K, act, use_bias)


def test_conv1d_keep_pool(gdn_lib):
    _announce("conv1d keep_pool")
    c = synth.make_conv_case(seed=311, lens=LENS, D=1032, K=4, has_init=INIT, num_slots=16)
    a = _run_and_check(gdn_lib, c, 4, True, True, keep_pool=True)
    b = _run_and_check(gdn_lib, c, 4, True, True, keep_pool=False)
    live = ~np.isnan(oracle.causal_conv1d(c.x, c.weight, c.bias, c.cu_seqlens, c.slot, c.has_init,
                                          c.pool)[0][:, 0])
    assert np.array_equal(a[live], b[live])


@pytest.mark.parametrize("cut", [1, 2, 31, 32, 45])
def test_conv1d_split_resume_and_decode(gdn_lib, cut):
    """One call over a sequence == two calls through the conv state == a prefix call then
    one decode step per token: same windows, same fp32 arithmetic, bit for bit."""
    gdn = gdn_lib
    _announce(f"conv1d split at {cut}")
    L, D = 70, 2048
    c = synth.make_conv_case(seed=320, lens=(L,), D=D, K=4, has_init=1, num_slots=4)
    d = _upload_conv(c)
    one = gdn.conv1d(d["x"], d["w"], d["b"], d["cu"], d["slot"], d["pool"].clone(), has_init=d["has_init"])
    pool = d["pool"].clone()
    parts = []
    for a0, a1 in ((0, cut), (cut, L)):
        cu = torch.tensor([0, a1 - a0], dtype=torch.int32, device="cuda")
        parts.append(gdn.conv1d(d["x"][a0:a1], d["w"], d["b"], cu, d["slot"], pool, has_init=d["has_init"]))
    assert torch.equal(torch.cat(parts), one)
    pool2 = d["pool"].clone()
    cu = torch.tensor([0, cut], dtype=torch.int32, device="cuda")
    rows = [gdn.conv1d(d["x"][:cut], d["w"], d["b"], cu, d["slot"], pool2, has_init=d["has_init"])]
    for t in range(cut, L):
        rows.append(gdn.conv1d_update(d["x"][t:t + 1], d["w"], d["b"], d["slot"], pool2))
    assert torch.equal(torch.cat(rows), one)
    assert torch.equal(pool2, pool)
    ref, _ = oracle.causal_conv1d(c.x, c.weight, c.bias, c.cu_seqlens, c.slot, c.has_init, c.pool)
    _check_out(one.float().cpu().numpy(), ref, "conv one call")


@pytest.mark.parametrize("inplace", [False, True])
def test_conv1d_update(gdn_lib, inplace):
    """Decode: 256 rows of 8192 channels (one token per sequence), padding rows skipped."""
    gdn = gdn_lib
    _announce(f"conv1d_update inplace={inplace}")
    B, D = 256, 8192
    c = synth.make_conv_case(seed=330, lens=(1,) * B, D=D, K=4, has_init=1, num_slots=300)
    c.slot[5] = c.slot[77] = -1
    d = _upload_conv(c)
    pool_before = d["pool"].clone()
    x_before = d["x"].clone()
    out = d["x"] if inplace else torch.randn((B, D), device="cuda").to(torch.bfloat16)
    out_before = out.clone()
    gdn.conv1d_update(d["x"], d["w"], d["b"], d["slot"], d["pool"], out=out)
    torch.cuda.synchronize()
    ref, states = oracle.causal_conv1d(c.x, c.weight, c.bias, c.cu_seqlens, c.slot, c.has_init, c.pool)
    live = c.slot >= 0
    _check_out(out.float().cpu().numpy()[live], ref[live], "conv update")
    assert torch.equal(out[~torch.from_numpy(live).cuda()], out_before[~torch.from_numpy(live).cuda()])
    if not inplace:
        assert torch.equal(d["x"], x_before)
    pool = d["pool"].cpu()
    touched = np.zeros(c.pool.shape[0], bool)
    for s, st in states.items():
        touched[s] = True
        assert torch.equal(pool[s], torch.from_numpy(st.astype(np.float32)).to(torch.bfloat16))
    assert torch.equal(pool[torch.from_numpy(~touched)], pool_before.cpu()[torch.from_numpy(~touched)])


def test_conv1d_prefill_full_size(gdn_lib):
    """8 sequences x 4096 tokens, 8192 channels (the q | k | v width of 16 qk-heads and
    32 v-heads of 128), width 4, from earlier states: every output and state."""
    gdn = gdn_lib
    _announce("conv1d 8x4096 x 8192")
    c = synth.make_conv_case(seed=340, lens=(4096,) * 8, D=8192, K=4, has_init=1, num_slots=16)
    _run_and_check(gdn, c, 4, True, True)


def test_forward_gdn_with_conv(gdn_lib):
    """forward_gdn with the short conv in front: extend then one decode token per
    sequence.  The oracle convolves in float64, stores the result as the layer's bf16
    mixed_qkv (the storage type of the layer input) and runs the GDN oracle on it."""
    from types import SimpleNamespace
    gdn = gdn_lib
    _announce("forward_gdn with conv: extend + decode")
    case = synth.edge_case("fwd-conv", (30, 70, 2), has_init=(1, 0, 1), seed=35, num_slots=6)
    D = case.mixed_qkv.shape[1]
    cc = synth.make_conv_case(seed=36, lens=(30, 70, 2), D=D, K=4, has_init=(1, 0, 1), num_slots=6,
                              slot=case.slot)
    d = upload(case)
    raw = _dev(cc.x)
    cpool = _dev(cc.pool)
    layer = SimpleNamespace(num_k_heads=case.H_qk, num_v_heads=case.H_v, head_k_dim=case.d_k,
                            head_v_dim=case.d_v, A_log=d["A_log"], dt_bias=d["dt_bias"],
                            scale=case.scale, layer_id=0, conv_weight=_dev(cc.weight)[:, None, :],
                            conv_bias=_dev(cc.bias))
    fb = SimpleNamespace(forward_mode="extend", state_pool=[d["pool"]], conv_pool=[cpool],
                         state_slots=d["slot"], cu_seqlens=d["cu"], has_initial_state=d["has_init"],
                         max_seqlen=70)
    out = gdn.forward_gdn(layer, fb, raw, d["a"], d["b"])
    conv_ref, cstates = oracle.causal_conv1d(cc.x, cc.weight, cc.bias, cc.cu_seqlens, cc.slot,
                                             cc.has_init, cc.pool)
    mixed = synth.bf16_round(conv_ref.astype(np.float32))
    Hk = case.H_qk * case.d_k
    q = mixed[:, :Hk].reshape(-1, case.H_qk, case.d_k)
    k = mixed[:, Hk:2 * Hk].reshape(-1, case.H_qk, case.d_k)
    v = mixed[:, 2 * Hk:].reshape(-1, case.H_v, case.d_v)
    ref, _, fin = oracle.gdn_extend(q, k, v, case.a, case.b, case.A_log, case.dt_bias, case.cu_seqlens,
                                    case.slot, case.has_init, case.pool, case.scale)
    assert_close(out.float().cpu().numpy().reshape(ref.shape), ref, "forward_gdn+conv extend")
    # decode: one more token per sequence through both pools
    N = case.N
    rng = np.random.default_rng(37)
    x1 = synth.bf16_round(rng.standard_normal((N, D), dtype=np.float32))
    a1 = synth.bf16_round(rng.standard_normal((N, case.H_v), dtype=np.float32))
    b1 = synth.bf16_round(rng.standard_normal((N, case.H_v), dtype=np.float32))
    fb.forward_mode = "decode"
    out1 = gdn.forward_gdn(layer, fb, _dev(x1), _dev(a1), _dev(b1))
    cpool_ref = cc.pool.copy()
    for s, st in cstates.items():
        cpool_ref[s] = st
    c1, _ = oracle.causal_conv1d(x1, cc.weight, cc.bias, np.arange(N + 1), case.slot, None, cpool_ref)
    m1 = synth.bf16_round(c1.astype(np.float32))
    pool_ref = oracle.apply_final_states(case.pool, fin)
    ref1, _, _ = oracle.gdn_decode(m1[:, :Hk].reshape(N, case.H_qk, case.d_k),
                                m1[:, Hk:2 * Hk].reshape(N, case.H_qk, case.d_k),
                                m1[:, 2 * Hk:].reshape(N, case.H_v, case.d_v), a1, b1, case.A_log,
                                case.dt_bias, case.slot, pool_ref, case.scale)
    assert_close(out1.float().cpu().numpy().reshape(ref1.shape), ref1, "forward_gdn+conv decode")
