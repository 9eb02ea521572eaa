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


@pytest.mark.parametrize("K,D,inplace", [(4, 8192, False), (4, 8192, True), (2, 1032, False),
                                         (3, 1032, True)])
def test_conv1d_update(gdn_lib, K, D, inplace):
    """Decode: 256 rows (one token per sequence) of 8192 channels, or 1032 (a ragged
    channel block) for the narrower widths; padding rows skipped."""
    gdn = gdn_lib
    _announce(f"conv1d_update K={K} D={D} inplace={inplace}")
    B = 256
    c = synth.make_conv_case(seed=330 + K, lens=(1,) * B, D=D, K=K, has_init=1, num_slots=300)
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


def test_forward_gdn_conv_decode_graph(gdn_lib):
    """forward_gdn decode with the short conv in front, captured once in a HIP graph over
    static buffers of 32 rows of which 20 are live (slot -1 pads the rest), replayed three
    times with new raw inputs and eager work in between.  Every replay is checked against
    the oracle (conv from the previous conv states, stored as bf16, then the GDN step from
    the previous states); padded rows' conv and GDN state slots stay untouched."""
    from types import SimpleNamespace
    gdn = gdn_lib
    _announce("forward_gdn + conv decode graph capture, 20 live of 32 static rows")
    rows, live, H_qk, H_v, d, K, nslot = 32, 20, 2, 4, 128, 4, 40
    D = 2 * H_qk * d + H_v * d
    rng = np.random.default_rng(93)
    pool = torch.from_numpy(rng.normal(0, 0.1, (nslot, H_v, d, d)).astype(np.float32)).cuda()
    cpool_h = synth.bf16_round(rng.standard_normal((nslot, D, K - 1)).astype(np.float32))
    cpool = _dev(cpool_h)
    slot_h = np.full(rows, -1, np.int32)
    slot_h[:live] = rng.permutation(nslot)[:live]
    lim = 1.0 / np.sqrt(K)
    w_h = synth.bf16_round(rng.uniform(-lim, lim, (D, K)).astype(np.float32))
    b_h = synth.bf16_round(rng.uniform(-lim, lim, D).astype(np.float32))
    A_log = np.log(rng.uniform(1, 16, H_v)).astype(np.float32)
    dt_bias = rng.normal(0, 0.5, H_v).astype(np.float32)
    layer = SimpleNamespace(num_k_heads=H_qk, num_v_heads=H_v, head_k_dim=d, head_v_dim=d,
                            A_log=torch.from_numpy(A_log).cuda(), dt_bias=torch.from_numpy(dt_bias).cuda(),
                            scale=d ** -0.5, layer_id=0, conv_weight=_dev(w_h), conv_bias=_dev(b_h))
    fb = SimpleNamespace(forward_mode="decode", state_pool=[pool], conv_pool=[cpool],
                         state_slots=torch.from_numpy(slot_h).cuda())
    raw = torch.zeros((rows, D), dtype=torch.bfloat16, device="cuda")
    a = torch.zeros((rows, H_v), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((rows, H_v), dtype=torch.bfloat16, device="cuda")
    pool_pad = pool.clone()
    cpool_pad = cpool.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            out = gdn.forward_gdn(layer, fb, raw, a, b)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(cpool, cpool_pad) and torch.equal(pool, pool_pad), "capture must not run kernels"
    states = pool.cpu().numpy().astype(np.float64)
    cstates = cpool_h.astype(np.float64)
    nq = H_qk * d
    for rep in range(3):
        x = synth.bf16_round(rng.standard_normal((rows, D)).astype(np.float32))
        av = synth.bf16_round(rng.standard_normal((rows, H_v)).astype(np.float32))
        bv = synth.bf16_round(rng.standard_normal((rows, H_v)).astype(np.float32))
        raw.copy_(_dev(x))
        a.copy_(_dev(av))
        b.copy_(_dev(bv))
        _ = (raw.float() * 2).sum()            # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        c, cfin = oracle.causal_conv1d(x[:live], w_h, b_h, np.arange(live + 1), slot_h[:live], None, cstates)
        m = synth.bf16_round(c.astype(np.float32))
        ref, _, fin = oracle.gdn_decode(m[:, :nq].reshape(live, H_qk, d), m[:, nq:2 * nq].reshape(live, H_qk, d),
                                        m[:, 2 * nq:].reshape(live, H_v, d), av[:live], bv[:live], A_log,
                                        dt_bias, slot_h[:live], states, d ** -0.5)
        assert_close(out[:live].float().cpu().numpy().reshape(ref.shape), ref, f"replay {rep} out")
        for s, st in cfin.items():
            cstates[s] = st
        states = oracle.apply_final_states(states, fin)
        got_c = cpool.cpu()
        assert torch.equal(got_c, torch.from_numpy(cstates.astype(np.float32)).to(torch.bfloat16)), \
            f"replay {rep} conv states"
        assert_close(pool.cpu().numpy()[slot_h[:live]], states[slot_h[:live]], f"replay {rep} states")
        unused = np.setdiff1d(np.arange(nslot), slot_h[:live])
        assert torch.equal(pool[unused], pool_pad[unused])


@pytest.mark.parametrize("K", [2, 3, 4])
def test_conv1d_token_tree(gdn_lib, K):
    """Target verify with token trees: each token's window follows its parents and then
    the slot's state; a chain given as a tree gives the plain conv's bits; the pool is
    only read."""
    gdn = gdn_lib
    _announce(f"conv1d token tree K={K}")
    lens = (5, 1, 0, 8, 4, 6)
    c = synth.make_conv_case(seed=350 + K, lens=lens, D=1032, K=K, has_init=(1, 0, 1, 1, 1, 0),
                             num_slots=12)
    c.slot[4] = -1
    rng = np.random.default_rng(K)
    tree = np.concatenate([[-1] + [int(rng.integers(-1, i)) for i in range(1, L)] for L in lens if L])
    chain = np.concatenate([np.arange(-1, L - 1) for L in lens if L])
    d = _upload_conv(c)
    pool_before = d["pool"].clone()
    outs = {}
    for name, par in (("tree", tree), ("chain", chain)):
        out = torch.randn((c.T, c.x.shape[1]), device="cuda").to(torch.bfloat16)
        out_before = out.clone()
        gdn.conv1d(d["x"], d["w"], d["b"], d["cu"], d["slot"], d["pool"], has_init=d["has_init"],
                   out=out, keep_pool=True, parent=_dev(par, torch.int32))
        torch.cuda.synchronize()
        ref, st = oracle.causal_conv1d(c.x, c.weight, c.bias, c.cu_seqlens, c.slot, c.has_init, c.pool,
                                       parent=par)
        live = ~np.isnan(ref[:, 0])
        _check_out(out.float().cpu().numpy()[live], ref[live], f"conv {name} K={K}")
        assert torch.equal(out[torch.from_numpy(~live).cuda()], out_before[torch.from_numpy(~live).cuda()])
        assert torch.equal(d["pool"], pool_before)
        outs[name] = out[torch.from_numpy(live).cuda()]
    plain = gdn.conv1d(d["x"], d["w"], d["b"], d["cu"], d["slot"], d["pool"], has_init=d["has_init"],
                       keep_pool=True)
    live_t = torch.from_numpy(live).cuda()
    assert torch.equal(outs["chain"], plain[live_t])


def test_forward_gdn_conv_target_verify_tree(gdn_lib):
    """forward_gdn in TARGET_VERIFY mode with the short conv and a token tree: the conv
    windows and the GDN states both follow the tree; both pools are left unwritten."""
    from types import SimpleNamespace
    gdn = gdn_lib
    _announce("forward_gdn + conv target verify, token tree")
    N, L = 3, 5
    case = synth.edge_case("fwd-conv-tree", (L,) * N, has_init=1, seed=83, num_slots=6)
    D = case.mixed_qkv.shape[1]
    cc = synth.make_conv_case(seed=84, lens=(L,) * N, D=D, K=4, has_init=1, num_slots=6, slot=case.slot)
    tree = np.array([-1, 0, 0, 1, 2] * N, np.int32)
    d = upload(case)
    cpool = _dev(cc.pool)
    pool_before, cpool_before = d["pool"].clone(), cpool.clone()
    rows = torch.tensor([2, 0, 1], dtype=torch.int32, device="cuda")
    buf = torch.zeros((N, L, case.H_v, case.d_v, case.d_k), dtype=torch.float32, device="cuda")
    layer = SimpleNamespace(num_k_heads=case.H_qk, num_v_heads=case.H_v, head_k_dim=case.d_k,
                            head_v_dim=case.d_v, A_log=d["A_log"], dt_bias=d["dt_bias"], scale=case.scale,
                            layer_id=0, conv_weight=_dev(cc.weight), conv_bias=_dev(cc.bias))
    fb = SimpleNamespace(forward_mode="TARGET_VERIFY", state_slots=d["slot"], state_pool=[d["pool"]],
                         conv_pool=[cpool], cu_seqlens=d["cu"], has_initial_state=d["has_init"],
                         max_seqlen=L, spec_states=[buf], spec_state_slots=rows,
                         spec_parents=_dev(tree, torch.int32))
    out = gdn.forward_gdn(layer, fb, _dev(cc.x), d["a"], d["b"])
    torch.cuda.synchronize()
    conv_ref, _ = oracle.causal_conv1d(cc.x, cc.weight, cc.bias, cc.cu_seqlens, cc.slot, cc.has_init,
                                       cc.pool, parent=tree)
    m = synth.bf16_round(conv_ref.astype(np.float32))
    Hk = case.H_qk * case.d_k
    spec = {}
    ref, _, _ = oracle.gdn_extend(m[:, :Hk].reshape(-1, case.H_qk, case.d_k),
                                  m[:, Hk:2 * Hk].reshape(-1, case.H_qk, case.d_k),
                                  m[:, 2 * Hk:].reshape(-1, case.H_v, case.d_v), case.a, case.b, case.A_log,
                                  case.dt_bias, case.cu_seqlens, case.slot, case.has_init, case.pool,
                                  case.scale, spec_slot=rows.cpu().numpy(), spec_parent=tree, spec=spec)
    assert_close(out.float().cpu().numpy().reshape(ref.shape), ref, "forward_gdn+conv tree out")
    got = buf.cpu().numpy()
    for (r, i), S in spec.items():
        assert_close(got[r, i], S, f"tree state {r},{i}")
    assert torch.equal(d["pool"], pool_before) and torch.equal(cpool, cpool_before)


def test_forward_gdn_conv_extend_graph_static_buffer(gdn_lib):
    """The split-op extend case of the SGLang GDN test article (prefixes 0, 8, 16; extends
    15, 8, 1; a static token buffer of 32): forward_gdn with the short conv captured once
    in a HIP graph over the static buffer, replayed with those live lengths and then with
    (10, 3, 9) written into the same cu_seqlens.  Tokens after the last sequence are
    padding: their output rows stay untouched.  Every replay continues from the pools
    the previous one left and is checked against the oracle."""
    from types import SimpleNamespace
    gdn = gdn_lib
    _announce("forward_gdn + conv extend graph over a static 32-token buffer")
    Tst, N, H_qk, H_v, d, K, nslot = 32, 3, 2, 4, 128, 4, 8
    D = 2 * H_qk * d + H_v * d
    rng = np.random.default_rng(97)
    slot_h = rng.permutation(nslot)[:N].astype(np.int32)
    has_init_h = np.array([0, 1, 1], np.int32)                # prefix 0 has no state
    pool = torch.from_numpy(rng.normal(0, 0.1, (nslot, H_v, d, d)).astype(np.float32)).cuda()
    cpool_h = synth.bf16_round(rng.standard_normal((nslot, D, K - 1)).astype(np.float32))
    cpool = _dev(cpool_h)
    lim = 1.0 / np.sqrt(K)
    w_h = synth.bf16_round(rng.uniform(-lim, lim, (D, K)).astype(np.float32))
    b_h = synth.bf16_round(rng.uniform(-lim, lim, D).astype(np.float32))
    A_log = np.log(rng.uniform(1, 16, H_v)).astype(np.float32)
    dt_bias = rng.normal(0, 0.5, H_v).astype(np.float32)
    layer = SimpleNamespace(num_k_heads=H_qk, num_v_heads=H_v, head_k_dim=d, head_v_dim=d,
                            A_log=torch.from_numpy(A_log).cuda(), dt_bias=torch.from_numpy(dt_bias).cuda(),
                            scale=d ** -0.5, layer_id=0, conv_weight=_dev(w_h), conv_bias=_dev(b_h))
    cu = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    fb = SimpleNamespace(forward_mode="extend", state_pool=[pool], conv_pool=[cpool],
                         state_slots=torch.from_numpy(slot_h).cuda(), cu_seqlens=cu,
                         has_initial_state=torch.from_numpy(has_init_h).cuda(), max_seqlen=0)
    raw = torch.zeros((Tst, D), dtype=torch.bfloat16, device="cuda")
    a = torch.zeros((Tst, H_v), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((Tst, H_v), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            out = gdn.forward_gdn(layer, fb, raw, a, b)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    out.fill_(SENT := -7.0)
    states = pool.cpu().numpy().astype(np.float64)
    cstates = cpool_h.astype(np.float64)
    nq = H_qk * d
    for rep, lens in enumerate([(15, 8, 1), (10, 3, 9)]):
        cu_h = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        live = int(cu_h[-1])
        x = synth.bf16_round(rng.standard_normal((Tst, D)).astype(np.float32))
        av = synth.bf16_round(rng.standard_normal((Tst, H_v)).astype(np.float32))
        bv = synth.bf16_round(rng.standard_normal((Tst, H_v)).astype(np.float32))
        cu.copy_(torch.from_numpy(cu_h))
        raw.copy_(_dev(x))
        a.copy_(_dev(av))
        b.copy_(_dev(bv))
        _ = (raw.float() * 2).sum()            # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        c, cfin = oracle.causal_conv1d(x[:live], w_h, b_h, cu_h, slot_h, has_init_h, cstates)
        m = synth.bf16_round(c.astype(np.float32))
        ref, _, fin = oracle.gdn_extend(m[:, :nq].reshape(live, H_qk, d), m[:, nq:2 * nq].reshape(live, H_qk, d),
                                        m[:, 2 * nq:].reshape(live, H_v, d), av[:live], bv[:live], A_log,
                                        dt_bias, cu_h, slot_h, has_init_h, states, d ** -0.5)
        got = out.float().cpu().numpy()
        assert_close(got[:live].reshape(ref.shape), ref, f"replay {rep} out")
        assert (got[live:] == SENT).all(), f"replay {rep}: padding rows were written"
        for s, st in cfin.items():
            cstates[s] = st
        states = oracle.apply_final_states(states, fin)
        assert torch.equal(cpool.cpu(), torch.from_numpy(cstates.astype(np.float32)).to(torch.bfloat16)), \
            f"replay {rep} conv states"
        assert_close(pool.cpu().numpy()[slot_h], states[slot_h], f"replay {rep} states")
        out.fill_(SENT)


def test_conv1d_empty_batches(gdn_lib):
    """T = 0 with sequences: only the state pass runs; an empty sequence keeps its slot
    (has_init) or clears it (no initial state), a skipped one touches nothing.  An empty
    decode batch is a no-op."""
    gdn = gdn_lib
    _announce("conv1d empty batches")
    D, K = 1032, 4
    c = synth.make_conv_case(seed=360, lens=(0, 0, 0), D=D, K=K, has_init=(1, 0, 0), num_slots=6,
                             slot=np.array([4, 1, -1]))
    d = _upload_conv(c)
    before = d["pool"].clone()
    x = torch.empty((0, D), dtype=torch.bfloat16, device="cuda")
    out = gdn.conv1d(x, d["w"], d["b"], d["cu"], d["slot"], d["pool"], has_init=d["has_init"])
    torch.cuda.synchronize()
    assert out.shape == (0, D)
    _, states = oracle.causal_conv1d(np.zeros((0, D)), c.weight, c.bias, c.cu_seqlens, c.slot, c.has_init,
                                     c.pool)
    pool = d["pool"].cpu()
    assert torch.equal(pool[4], before.cpu()[4]) and torch.equal(pool[1], torch.zeros_like(pool[1]))
    for s, st in states.items():
        assert torch.equal(pool[s], torch.from_numpy(st.astype(np.float32)).to(torch.bfloat16))
    for s in (0, 2, 3, 5):
        assert torch.equal(pool[s], before.cpu()[s])
    empty = torch.empty(0, dtype=torch.int32, device="cuda")
    o = gdn.conv1d_update(x, d["w"], d["b"], empty, d["pool"])
    torch.cuda.synchronize()
    assert o.shape == (0, D) and torch.equal(d["pool"].cpu(), pool)
