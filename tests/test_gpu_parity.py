"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: slot / index handling bit-exact (untouched pool slots and skipped rows keep
their bytes); outputs and final states within rel-L2 <= 2e-3 and max-abs <= 1e-2
of the float64 oracle for bf16 inputs with fp32 state.  fp32 paths are held to a
much tighter bound as a regression guard.
"""
import numpy as np
import pytest
import torch

import oracle
from hybrid_model_linear_amd import synth
from gpu_util import assert_close, host_rows, oracle_seq, rel_l2, run_extend, upload

pytestmark = pytest.mark.gpu

SENTINEL = -12345.0


def _announce(msg):
    print(f"[case] {msg}", flush=True)


# ------------------------------------------------------------------ gate
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gate_parity(gdn_lib, dtype):
    gdn = gdn_lib
    _announce(f"gate {dtype}")
    rng = np.random.default_rng(11)
    T, H = 1000, 32
    a = rng.standard_normal((T, H)).astype(np.float32) * 4
    b = rng.standard_normal((T, H)).astype(np.float32) * 8
    a[0, :4] = [-80.0, 80.0, 0.0, 30.0]
    b[0, :4] = [-90.0, 90.0, 0.0, 1e-3]
    if dtype == "bf16":
        a, b = synth.bf16_round(a), synth.bf16_round(b)
    A_log = np.log(rng.uniform(1, 16, H)).astype(np.float32)
    bias = (rng.standard_normal(H) * 0.5).astype(np.float32)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    ta = torch.from_numpy(a).to("cuda", tdt)
    tb = torch.from_numpy(b).to("cuda", tdt)
    lg, bt = gdn.gate(ta, tb, torch.from_numpy(A_log).cuda(), torch.from_numpy(bias).cuda())
    rlg, rbt = oracle.gdn_gate(a, b, A_log, bias)
    lg, bt = lg.cpu().numpy(), bt.cpu().numpy()
    assert np.allclose(lg, rlg, rtol=2e-6, atol=1e-7), np.max(np.abs(lg - rlg) / (np.abs(rlg) + 1e-7))
    assert np.allclose(bt, rbt, rtol=2e-6, atol=1e-7)
    # ssd mode with a clamp
    dt = synth.bf16_round(rng.standard_normal((T, H)).astype(np.float32))
    A = (-rng.uniform(1, 16, H)).astype(np.float32)
    for sp, lim in ((True, (0.0, float("inf"))), (False, (0.05, 0.5)), (True, (0.2, 1.5))):
        lg, dtp = gdn.ssd_gate(torch.from_numpy(dt).to("cuda", torch.bfloat16), torch.from_numpy(A).cuda(),
                               torch.from_numpy(bias).cuda(), sp, lim)
        rlg, rdt = oracle.ssd_gate(dt, A, bias, sp, lim)
        assert np.allclose(dtp.cpu().numpy(), rdt, rtol=2e-6, atol=1e-7)
        assert np.allclose(lg.cpu().numpy(), rlg, rtol=2e-6, atol=1e-6)


# ------------------------------------------------------------------ gate folded into the kernels
# The gated calls take the raw a, b (dt) and compute log g, beta with the gate
# kernel's own arithmetic, so they must reproduce gate + extend / decode exactly.
@pytest.mark.parametrize("dtype,max_seqlen", [("bf16", 0), ("bf16", 8), ("f32", 0)])
def test_gate_folded_extend_matches_separate(gdn_lib, dtype, max_seqlen):
    gdn = gdn_lib
    _announce(f"gate folded into extend {dtype} max_seqlen={max_seqlen}")
    lens = (5, 64, 65, 130) if max_seqlen == 0 else (3, 8, 1, 7)
    case = synth.make_gdn_case("fold", seed=21, lens=lens, has_init=(1, 0, 1, 1), H_qk=2, H_v=4,
                               d_k=128, d_v=128, dtype=dtype, num_slots=6, pool_sigma=0.05)
    d = upload(case)
    q, k, v = gdn.split_mixed_qkv(d["mixed"], case.H_qk, case.H_v, case.d_k, case.d_v)
    runs = []
    for folded in (False, True):
        pool = d["pool"].clone()
        if folded:
            lg = bt = None
            g = gdn.gdn_gate_inputs(d["a"], d["b"], d["A_log"], d["dt_bias"])
        else:
            lg, bt = gdn.gate(d["a"], d["b"], d["A_log"], d["dt_bias"])
            g = None
        out = gdn.extend(q, k, v, lg, bt, d["cu"], d["slot"], pool, has_init=d["has_init"],
                         scale=case.scale, max_seqlen=max_seqlen, gate=g)
        runs.append((out, pool))
    torch.cuda.synchronize()
    assert torch.equal(runs[0][0].view(torch.int16 if dtype == "bf16" else torch.int32),
                       runs[1][0].view(torch.int16 if dtype == "bf16" else torch.int32)), "outputs differ"
    assert torch.equal(runs[0][1].view(torch.int32), runs[1][1].view(torch.int32)), "states differ"
    ref, _, fin = oracle.gdn_extend(case.q, case.k, case.v, case.a, case.b, case.A_log, case.dt_bias,
                                    case.cu_seqlens, case.slot, case.has_init, case.pool, case.scale)
    bar = (2e-3, 1e-2) if dtype == "bf16" else (1e-3, 2e-3)
    assert_close(runs[1][0].float().cpu().numpy(), ref, "folded out", *bar)


def test_gate_folded_decode_and_ssd_match_separate(gdn_lib):
    gdn = gdn_lib
    _announce("gate folded into decode and delta-off extend")
    case = synth.make_gdn_case("fold-dec", seed=23, lens=(1,) * 9, has_init=1, H_qk=2, H_v=4,
                               d_k=128, d_v=128, dtype="bf16", num_slots=12, pool_sigma=0.05)
    d = upload(case)
    q, k, v = gdn.split_mixed_qkv(d["mixed"], case.H_qk, case.H_v, case.d_k, case.d_v)
    outs = []
    for folded in (False, True):
        pool = d["pool"].clone()
        if folded:
            out = gdn.decode(q, k, v, None, None, d["slot"], pool, scale=case.scale,
                             gate=gdn.gdn_gate_inputs(d["a"], d["b"], d["A_log"], d["dt_bias"]))
        else:
            lg, bt = gdn.gate(d["a"], d["b"], d["A_log"], d["dt_bias"])
            out = gdn.decode(q, k, v, lg, bt, d["slot"], pool, scale=case.scale)
        outs.append((out, pool))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16)), "decode outputs differ"
    assert torch.equal(outs[0][1].view(torch.int32), outs[1][1].view(torch.int32)), "decode states differ"
    # delta-off: ssd_combined_fwd (gate folded) against ssd_gate + extend
    c = synth.config4_ssd(seed=5, batch=2, L=100, H=6, P=64, G=2, Nst=128, initial=True)
    tb = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda", torch.bfloat16)
    tf = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda", torch.float32)
    lim = (0.05, 2.0)
    out, fin = gdn.ssd_combined_fwd(tb(c.x), tb(c.dt), tf(c.A), tb(c.B), tb(c.C), tb(c.D), tb(c.z),
                                    tf(c.dt_bias), True, lim, tf(c.initial_states))
    batch, L, H, P = c.x.shape
    G, Nst = c.B.shape[2], c.B.shape[3]
    T = batch * L
    lg, dtp = gdn.ssd_gate(tb(c.dt).view(T, H), tf(c.A), tf(c.dt_bias), True, lim)
    pool = tf(c.initial_states).contiguous().clone()
    cu = torch.arange(0, T + 1, L, dtype=torch.int32, device="cuda")
    slot = torch.arange(batch, dtype=torch.int32, device="cuda")
    hi = torch.ones(batch, dtype=torch.int32, device="cuda")
    out2 = gdn.extend(tb(c.C).view(T, G, Nst), tb(c.B).view(T, G, Nst), tb(c.x).view(T, H, P), lg, dtp,
                      cu, slot, pool, has_init=hi, mode="ssd", D=tb(c.D), z=tb(c.z).view(T, H, P),
                      max_seqlen=L)
    torch.cuda.synchronize()
    assert torch.equal(out.view(T, H, P).view(torch.int16), out2.view(torch.int16)), "ssd outputs differ"
    assert torch.equal(fin.view(torch.int32), pool.view(torch.int32)), "ssd states differ"


# ------------------------------------------------------------------ tiny fp32 (extend + decode)
def test_config0_tiny_fp32_extend_then_decode(gdn_lib):
    gdn = gdn_lib
    _announce("config0 tiny fp32")
    ext, dec = synth.config0_tiny()
    d = upload(ext)
    pool_before = d["pool"].clone()
    out = run_extend(gdn, ext, d)
    ref, written, fin = oracle.gdn_extend(ext.q, ext.k, ext.v, ext.a, ext.b, ext.A_log, ext.dt_bias,
                                          ext.cu_seqlens, ext.slot, ext.has_init, ext.pool, ext.scale)
    assert_close(out.cpu().numpy(), ref, "extend out", rel=1e-5, mx=1e-5)
    pool1 = oracle.apply_final_states(ext.pool, fin)
    got_pool = d["pool"].cpu().numpy()
    assert_close(got_pool[ext.slot], pool1[ext.slot], "extend states", rel=1e-5, mx=1e-5)
    untouched = np.setdiff1d(np.arange(ext.num_slots), ext.slot)
    assert torch.equal(d["pool"][untouched], pool_before[untouched])
    # one decode token per sequence from the extend's states
    dd = upload(dec, pool=d["pool"])
    q, k, v = gdn.split_mixed_qkv(dd["mixed"], 2, 2, 64, 64)
    lg, bt = gdn.gate(dd["a"], dd["b"], dd["A_log"], dd["dt_bias"])
    o = gdn.decode(q, k, v, lg, bt, dd["slot"], dd["pool"], scale=dec.scale)
    ref2, _, fin2 = oracle.gdn_decode(dec.q, dec.k, dec.v, dec.a, dec.b, dec.A_log, dec.dt_bias,
                                      dec.slot, pool1, dec.scale)
    assert_close(o.cpu().numpy(), ref2, "decode out", rel=1e-5, mx=1e-5)
    pool2 = oracle.apply_final_states(pool1, fin2)
    assert_close(d["pool"].cpu().numpy()[dec.slot], pool2[dec.slot], "decode states", rel=1e-5, mx=1e-5)


# ------------------------------------------------------------------ bf16 extend edge shapes
EDGE = [
    ("ragged-page", (15, 8, 1), (0, 1, 1)),
    ("exact-page", (16,), (0,)),
    ("chunk-boundary", (64, 65, 129), (0, 1, 1)),
    ("lengths", (1, 63, 64, 65, 127, 128, 129), (1, 0, 1, 0, 1, 0, 1)),
    ("batch1-long", (300,), (1,)),
    ("with-empty", (5, 0, 70, 0, 1), (1, 1, 0, 0, 1)),
]


@pytest.mark.parametrize("name,lens,has_init", EDGE, ids=[e[0] for e in EDGE])
@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_extend_edges(gdn_lib, name, lens, has_init, out_dtype):
    gdn = gdn_lib
    _announce(f"extend edge {name} out={out_dtype}")
    case = synth.edge_case(name, lens, has_init=has_init, seed=sum(lens) + 3, num_slots=2 * len(lens) + 3)
    d = upload(case)
    pool_before = d["pool"].clone()
    odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    out = torch.full((case.T, case.H_v, case.d_v), SENTINEL, dtype=odt, device="cuda")
    run_extend(gdn, case, d, out=out)
    torch.cuda.synchronize()
    ref, written, fin = oracle.gdn_extend(case.q, case.k, case.v, case.a, case.b, case.A_log,
                                          case.dt_bias, case.cu_seqlens, case.slot, case.has_init,
                                          case.pool, case.scale)
    bar = (2e-3, 1e-2) if out_dtype == "bf16" else (1e-3, 2e-3)
    if case.T:
        assert_close(out.float().cpu().numpy(), ref, "out", *bar)
    newpool = oracle.apply_final_states(case.pool, fin)
    assert_close(d["pool"].cpu().numpy()[case.slot], newpool[case.slot], "states", 2e-3 if out_dtype == "bf16" else 1e-3, 1e-2)
    untouched = np.setdiff1d(np.arange(case.num_slots), case.slot)
    assert torch.equal(d["pool"][untouched], pool_before[untouched]), "untouched slots changed"


SHORT = [
    ("short-tails", (8, 5, 1, 4, 0, 7, 3), 8),      # past the four tokens loaded up front
    ("short-wrong-hint", (4, 9, 2, 6), 4),          # a hint below the longest sequence
]


@pytest.mark.parametrize("name,lens,hint", SHORT, ids=[e[0] for e in SHORT])
@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_short_extend_token_recurrent(gdn_lib, name, lens, hint, out_dtype):
    """Short extends (host hint <= 8 tokens) take the token-recurrent kernel that loads
    its first four tokens' inputs with the state: sequences longer than four (and longer
    than the hint) continue token by token; outputs and states against the oracle."""
    gdn = gdn_lib
    _announce(f"short extend {name} out={out_dtype}")
    case = synth.edge_case(name, lens, has_init=(1,) * len(lens), seed=sum(lens) + 11,
                           num_slots=len(lens) + 3)
    d = upload(case)
    q, k, v = gdn.split_mixed_qkv(d["mixed"], case.H_qk, case.H_v, case.d_k, case.d_v)
    lg, bt = gdn.gate(d["a"], d["b"], d["A_log"], d["dt_bias"])
    assert gdn.extend_kernel(q, k, v, lg, bt, d["cu"], d["slot"], d["pool"], has_init=d["has_init"],
                             scale=case.scale, max_seqlen=hint)[0] == "recurrent"
    odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    out = run_extend(gdn, case, d, out_dtype=odt, max_seqlen=hint)
    torch.cuda.synchronize()
    ref, written, fin = oracle.gdn_extend(case.q, case.k, case.v, case.a, case.b, case.A_log,
                                          case.dt_bias, case.cu_seqlens, case.slot, case.has_init,
                                          case.pool, case.scale)
    bar = (2e-3, 1e-2) if out_dtype == "bf16" else (1e-3, 2e-3)
    assert_close(out.float().cpu().numpy(), ref, "out", *bar)
    newpool = oracle.apply_final_states(case.pool, fin)
    assert_close(d["pool"].cpu().numpy()[case.slot], newpool[case.slot], "states", 1e-3, 1e-2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_short_extend_head_dim_64(gdn_lib, dtype):
    """Short extends (hint 8) at d_k = d_v = 64, the tiny workload's head size: the
    token-recurrent kernel's short-extend layout with one float4 per lane of a 16-lane
    row, against the oracle (the fp32 inputs to the fp32 bar)."""
    gdn = gdn_lib
    _announce(f"short extend d=64 {dtype}")
    lens = (8, 3, 1, 6, 0, 5)
    case = synth.edge_case("short-d64", lens, has_init=(1, 0, 1, 1, 1, 0), seed=61, H_qk=2, H_v=4,
                           d_k=64, d_v=64, dtype=dtype, num_slots=len(lens) + 2)
    d = upload(case)
    q, k, v = gdn.split_mixed_qkv(d["mixed"], case.H_qk, case.H_v, case.d_k, case.d_v)
    lg, bt = gdn.gate(d["a"], d["b"], d["A_log"], d["dt_bias"])
    assert gdn.extend_kernel(q, k, v, lg, bt, d["cu"], d["slot"], d["pool"], has_init=d["has_init"],
                             scale=case.scale, max_seqlen=8)[0] == "recurrent"
    out = run_extend(gdn, case, d, max_seqlen=8)
    torch.cuda.synchronize()
    ref, written, fin = oracle.gdn_extend(case.q, case.k, case.v, case.a, case.b, case.A_log,
                                          case.dt_bias, case.cu_seqlens, case.slot, case.has_init,
                                          case.pool, case.scale)
    bar = (2e-3, 1e-2) if dtype == "bf16" else (1e-3, 1e-3)
    assert_close(out.float().cpu().numpy(), ref, "out", *bar)
    newpool = oracle.apply_final_states(case.pool, fin)
    assert_close(d["pool"].cpu().numpy()[case.slot], newpool[case.slot], "states", *bar)


def test_skipped_sequences_and_sentinels(gdn_lib):
    gdn = gdn_lib
    _announce("skipped sequences")
    case = synth.edge_case("skip", (20, 70, 3, 66), has_init=(1, 1, 0, 1), seed=5, num_slots=9)
    case.slot[:] = [4, -1, 7, -1]
    d = upload(case)
    pool_before = d["pool"].clone()
    out = torch.full((case.T, case.H_v, case.d_v), SENTINEL, dtype=torch.bfloat16, device="cuda")
    out_before = out.clone()
    run_extend(gdn, case, d, out=out)
    ref, written, fin = oracle.gdn_extend(case.q, case.k, case.v, case.a, case.b, case.A_log,
                                          case.dt_bias, case.cu_seqlens, case.slot, case.has_init,
                                          case.pool, case.scale)
    o = out.float().cpu().numpy()
    skipped = torch.from_numpy(~written).cuda()
    assert torch.equal(out[skipped].view(torch.int16), out_before[skipped].view(torch.int16)), \
        "rows of skipped sequences were written"
    assert_close(o[written], ref[written], "out")
    keep = np.setdiff1d(np.arange(9), [4, 7])
    assert torch.equal(d["pool"][keep], pool_before[keep])
    got = d["pool"].cpu().numpy()
    assert_close(got[[4, 7]], np.stack([fin[4], fin[7]]), "states")


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_extend_many_sequences(gdn_lib, out_dtype):
    """150 packed sequences (log-uniform lengths up to ~300, every 23rd empty, two
    skipped, mixed initial states): more sequences than the longest-first ordering takes,
    so workgroups follow the plain order with the qk-head pairs grouped per XCD; every
    written row and state against the oracle, untouched slots and skipped rows
    bit-exact."""
    gdn = gdn_lib
    _announce(f"extend many sequences out={out_dtype}")
    rng = np.random.default_rng(8)
    lens = np.exp(rng.uniform(0, np.log(300), 150)).astype(np.int64)
    lens[::23] = 0
    hi = (rng.random(150) < 0.6).astype(np.int32)
    case = synth.edge_case("many", tuple(int(x) for x in lens), has_init=tuple(int(x) for x in hi), seed=77,
                           H_qk=4, H_v=8, num_slots=160)
    case.slot[[12, 99]] = -1
    d = upload(case)
    q, k, v = gdn.split_mixed_qkv(d["mixed"], case.H_qk, case.H_v, case.d_k, case.d_v)
    lg, bt = gdn.gate(d["a"], d["b"], d["A_log"], d["dt_bias"])
    assert gdn.extend_kernel(q, k, v, lg, bt, d["cu"], d["slot"], d["pool"], has_init=d["has_init"],
                             scale=case.scale)[0] == "chunked64"
    pool_before = d["pool"].clone()
    odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    out = torch.full((case.T, case.H_v, case.d_v), SENTINEL, dtype=odt, device="cuda")
    out_before = out.clone()
    run_extend(gdn, case, d, out=out)
    torch.cuda.synchronize()
    ref, written, fin = oracle.gdn_extend(case.q, case.k, case.v, case.a, case.b, case.A_log,
                                          case.dt_bias, case.cu_seqlens, case.slot, case.has_init,
                                          case.pool, case.scale)
    bar = (2e-3, 1e-2) if out_dtype == "bf16" else (1e-3, 2e-3)
    assert_close(out.float().cpu().numpy()[written], ref[written], "out", *bar)
    skipped = torch.from_numpy(~written).cuda()
    assert torch.equal(out[skipped].view(torch.int16 if out_dtype == "bf16" else torch.int32),
                       out_before[skipped].view(torch.int16 if out_dtype == "bf16" else torch.int32)), \
        "rows of skipped sequences were written"
    used = case.slot[case.slot >= 0]
    newpool = oracle.apply_final_states(case.pool, fin)
    assert_close(d["pool"].cpu().numpy()[used], newpool[used], "states", *bar)
    untouched = np.setdiff1d(np.arange(case.num_slots), used)
    assert torch.equal(d["pool"][untouched], pool_before[untouched]), "untouched slots changed"


@pytest.mark.parametrize("decay", [1e-2, 1e-3])
@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_extend_long_memory(gdn_lib, decay, out_dtype):
    """Weak decay (A_log shifted by log(decay)): the state keeps its history for
    thousands of tokens, so the precision of the state operand of every chunk shows
    in the outputs.  Both output types are held to the general float bar."""
    gdn = gdn_lib
    _announce(f"long memory decay x{decay} out={out_dtype}")
    rng = np.random.default_rng(5)
    A_log = (np.log(rng.uniform(1, 16, 4)) + np.log(decay)).astype(np.float32)
    case = synth.make_gdn_case("long-memory", seed=11, lens=(1000, 777), has_init=(1, 1), H_qk=2, H_v=4,
                               d_k=128, d_v=128, A_log=A_log, num_slots=5)
    d = upload(case)
    odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    out = run_extend(gdn, case, d, out_dtype=odt)
    torch.cuda.synchronize()
    ref, _, fin = oracle.gdn_extend(case.q, case.k, case.v, case.a, case.b, case.A_log, case.dt_bias,
                                    case.cu_seqlens, case.slot, case.has_init, case.pool, case.scale)
    assert_close(out.float().cpu().numpy(), ref, "out")
    assert_close(d["pool"].cpu().numpy()[case.slot], np.stack([fin[s] for s in case.slot]), "states")


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_extend_precision_at_length(gdn_lib, out_dtype):
    """One 8192-token sequence at the layer's shape (H_qk 16, H_v 32, d 128) with weak
    decay (A_log shifted by log 1e-3: the state keeps thousands of tokens of history)
    through the gated chunked kernel, from a nonzero pool state; sampled v-heads
    (both v-heads of one qk-head, and heads at either end) against the float64 oracle.
    The fp32 output is held to rel-L2 1e-3, the bf16 output to 2e-3; final states to
    the output's bar."""
    gdn = gdn_lib
    _announce(f"precision at length 8192 out={out_dtype}")
    rng = np.random.default_rng(23)
    A_log = (np.log(rng.uniform(1, 16, 32)) + np.log(1e-3)).astype(np.float32)
    case = synth.make_gdn_case("length-8192", seed=31, lens=(8192,), has_init=(1,), H_qk=16, H_v=32,
                               d_k=128, d_v=128, A_log=A_log, num_slots=3)
    d = upload(case)
    init = case.pool[case.slot[0]].copy()
    q, k, v = gdn.split_mixed_qkv(d["mixed"], 16, 32, 128, 128)
    g = gdn.gdn_gate_inputs(d["a"], d["b"], d["A_log"], d["dt_bias"])
    odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    assert gdn.extend_kernel(q, k, v, None, None, d["cu"], d["slot"], d["pool"], has_init=d["has_init"],
                             scale=case.scale, out_dtype=odt, max_seqlen=8192, gate=g) == ("chunked64", [])
    out = gdn.extend(q, k, v, None, None, d["cu"], d["slot"], d["pool"], has_init=d["has_init"],
                     scale=case.scale, out_dtype=odt, max_seqlen=8192, gate=g)
    torch.cuda.synchronize()
    heads = [0, 6, 7, 31]
    ref, fin = oracle_seq(case, 0, heads, init)
    rel = 2e-3 if out_dtype == "bf16" else 1e-3
    got = out.float().cpu().numpy()[:, heads]
    assert_close(got, ref, "out", rel=rel)
    for i in (0, 4095, 8191):   # the rows at the start, middle and end, each on its own
        assert rel_l2(got[i], ref[i]) <= 2 * rel, f"row {i}: rel-L2 {rel_l2(got[i], ref[i]):.3e}"
    assert_close(d["pool"].cpu().numpy()[case.slot[0]][heads], fin, "state", rel=rel)


def test_has_init_zero_ignores_pool_content(gdn_lib):
    gdn = gdn_lib
    _announce("has_init=0 ignores pool")
    case = synth.edge_case("noinit", (40, 90), has_init=(0, 0), seed=9, num_slots=4)
    d = upload(case)
    d["pool"].fill_(float("nan"))
    out = run_extend(gdn, case, d)
    ref, _, fin = oracle.gdn_extend(case.q, case.k, case.v, case.a, case.b, case.A_log, case.dt_bias,
                                    case.cu_seqlens, case.slot, case.has_init,
                                    np.zeros_like(case.pool), case.scale)
    assert_close(out.float().cpu().numpy(), ref, "out")
    assert_close(d["pool"].cpu().numpy()[case.slot], np.stack([fin[s] for s in case.slot]), "states")


@pytest.mark.parametrize("cut", [1, 37, 64, 100, 128])
def test_split_resume(gdn_lib, cut):
    """extend(A||B) == extend(A) then extend(B), and == extend(A) then decode per token."""
    gdn = gdn_lib
    _announce(f"split/resume cut={cut}")
    L = 150
    case = synth.edge_case("split", (L,), has_init=(1,), seed=21, num_slots=3)
    full = upload(case)
    out_full = run_extend(gdn, case, full, out_dtype=torch.float32)
    # A then B
    d = upload(case)
    q, k, v = gdn.split_mixed_qkv(d["mixed"], case.H_qk, case.H_v, case.d_k, case.d_v)
    lg, bt = gdn.gate(d["a"], d["b"], d["A_log"], d["dt_bias"])
    one = torch.ones(1, dtype=torch.int32, device="cuda")
    oA = gdn.extend(q[:cut], k[:cut], v[:cut], lg[:cut].contiguous(), bt[:cut].contiguous(),
                    torch.tensor([0, cut], dtype=torch.int32, device="cuda"), d["slot"], d["pool"],
                    has_init=one, scale=case.scale, out_dtype=torch.float32)
    oB = gdn.extend(q[cut:], k[cut:], v[cut:], lg[cut:].contiguous(), bt[cut:].contiguous(),
                    torch.tensor([0, L - cut], dtype=torch.int32, device="cuda"), d["slot"], d["pool"],
                    has_init=one, scale=case.scale, out_dtype=torch.float32)
    got = torch.cat([oA, oB]).cpu().numpy()
    ref, _, fin = oracle.gdn_extend(case.q, case.k, case.v, case.a, case.b, case.A_log, case.dt_bias,
                                    case.cu_seqlens, case.slot, case.has_init, case.pool, case.scale)
    assert_close(got, ref, "A|B out", 2e-4, 2e-3)
    assert_close(d["pool"].cpu().numpy()[case.slot[0]], fin[case.slot[0]], "A|B state", 2e-4, 2e-3)
    assert rel_l2(got, out_full.cpu().numpy()) < 2e-4
    # A then per-token decode
    d2 = upload(case)
    gdn.extend(q[:cut], k[:cut], v[:cut], lg[:cut].contiguous(), bt[:cut].contiguous(),
               torch.tensor([0, cut], dtype=torch.int32, device="cuda"), d2["slot"], d2["pool"],
               has_init=one, scale=case.scale, out_dtype=torch.float32)
    outs = []
    for t in range(cut, min(L, cut + 12)):
        outs.append(gdn.decode(q[t:t + 1], k[t:t + 1], v[t:t + 1], lg[t:t + 1].contiguous(),
                               bt[t:t + 1].contiguous(), d2["slot"], d2["pool"], scale=case.scale,
                               out_dtype=torch.float32))
    got2 = torch.cat(outs).cpu().numpy()
    assert_close(got2, ref[cut:cut + len(outs)], "A|decode out", 2e-4, 2e-3)


# ------------------------------------------------------------------ full-size configurations
def test_config1_decode_full(gdn_lib):
    gdn = gdn_lib
    _announce("config1 decode 256 x [1024,32,128,128]")
    case = synth.device_config1_decode()
    pool = synth.device_pool(case)
    d = upload(case, pool=pool)
    before = pool.clone()
    init = pool[torch.from_numpy(case.slot).long().cuda()].cpu().numpy()
    q, k, v = gdn.split_mixed_qkv(d["mixed"], 16, 32, 128, 128)
    lg, bt = gdn.gate(d["a"], d["b"], d["A_log"], d["dt_bias"])
    out = gdn.decode(q, k, v, lg, bt, d["slot"], pool, scale=case.scale)
    torch.cuda.synchronize()
    mixed = host_rows(case.mixed_qkv, 0, 256)
    nq = 16 * 128
    ref, _, fin = oracle.gdn_decode(mixed[:, :nq].reshape(256, 16, 128), mixed[:, nq:2 * nq].reshape(256, 16, 128),
                                    mixed[:, 2 * nq:].reshape(256, 32, 128), host_rows(case.a, 0, 256),
                                    host_rows(case.b, 0, 256), case.A_log, case.dt_bias,
                                    np.arange(256), {i: init[i] for i in range(256)}, case.scale)
    assert_close(out.float().cpu().numpy(), ref, "decode out")
    got = pool[torch.from_numpy(case.slot).long().cuda()].cpu().numpy()
    assert_close(got, np.stack([fin[i] for i in range(256)]), "decode states")
    mask = torch.ones(1024, dtype=torch.bool, device="cuda")
    mask[torch.from_numpy(case.slot).long().cuda()] = False
    assert torch.equal(pool[mask], before[mask]), "untouched slots changed"


@pytest.mark.slow
def test_config2_prefill_sampled(gdn_lib):
    gdn = gdn_lib
    _announce("config2 prefill 8x4096 (sampled oracle)")
    case = synth.device_config2_prefill()
    pool = synth.device_pool(case)
    d = upload(case, pool=pool)
    out = run_extend(gdn, case, d)
    torch.cuda.synchronize()
    heads = [0, 1, 17, 31]
    for n in (0, 5):
        t0, t1 = int(case.cu_seqlens[n]), int(case.cu_seqlens[n + 1])
        ref, fin = oracle_seq(case, n, heads, None)
        assert_close(out[t0:t1, heads].float().cpu().numpy(), ref, f"seq {n} out")
        assert_close(pool[int(case.slot[n])][heads].cpu().numpy(), fin, f"seq {n} state")


@pytest.mark.slow
def test_config3_ragged_sampled_and_verify(gdn_lib):
    gdn = gdn_lib
    _announce("config3 ragged 64 seqs (sampled oracle) + verify 32x4")
    case = synth.device_config3_ragged()
    pool = synth.device_pool(case)
    d = upload(case, pool=pool)
    lens = np.diff(case.cu_seqlens)
    picks = [int(np.argmax(lens)), int(np.argmin(lens)), 7, 40]
    inits = {n: pool[int(case.slot[n])].cpu().numpy() for n in picks}
    before = pool.clone()
    out = run_extend(gdn, case, d, max_seqlen=int(lens.max()))
    torch.cuda.synchronize()
    heads = [0, 13, 31]
    for n in picks:
        t0, t1 = int(case.cu_seqlens[n]), int(case.cu_seqlens[n + 1])
        ref, fin = oracle_seq(case, n, heads, inits[n])
        assert_close(out[t0:t1, heads].float().cpu().numpy(), ref, f"seq {n} (len {t1 - t0}) out")
        assert_close(pool[int(case.slot[n])][heads].cpu().numpy(), fin, f"seq {n} state")
    mask = torch.ones(512, dtype=torch.bool, device="cuda")
    mask[torch.from_numpy(case.slot).long().cuda()] = False
    assert torch.equal(pool[mask], before[mask])
    # verify-style batch on other slots of the same pool
    ver = synth.device_config3_verify()
    dv = upload(ver, pool=pool)
    vinit = {n: pool[int(ver.slot[n])].cpu().numpy() for n in range(32)}
    vout = run_extend(gdn, ver, dv, max_seqlen=4)
    torch.cuda.synchronize()
    for n in (0, 9, 31):
        ref, fin = oracle_seq(ver, n, list(range(32)), vinit[n])
        assert_close(vout[4 * n:4 * n + 4].float().cpu().numpy(), ref, f"verify seq {n} out")
        assert_close(pool[int(ver.slot[n])].cpu().numpy(), fin, f"verify seq {n} state")


# ------------------------------------------------------------------ delta-off (SSD)
@pytest.mark.parametrize("shape", [(2, 150, 6, 64, 2, 128, False), (1, 64, 4, 64, 1, 128, True),
                                   (3, 33, 8, 64, 4, 128, True)])
@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_ssd_small(gdn_lib, shape, out_dtype):
    gdn = gdn_lib
    batch, L, H, P, G, Nst, init = shape
    _announce(f"ssd small {shape} out={out_dtype}")
    c = synth.config4_ssd(seed=L + H, batch=batch, L=L, H=H, P=P, G=G, Nst=Nst, initial=init)
    tb = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda", torch.bfloat16)
    tf = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda", torch.float32)
    out, fin = gdn.ssd_combined_fwd(tb(c.x), tb(c.dt), tf(c.A), tb(c.B), tb(c.C), tb(c.D), tb(c.z),
                                    tf(c.dt_bias), True, (0.0, float("inf")),
                                    None if c.initial_states is None else tf(c.initial_states),
                                    out_dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32)
    ref, rfin = oracle.ssd_combined(c.x, c.dt, c.A, c.B, c.C, c.D, c.z, c.dt_bias, True,
                                    (0.0, float("inf")), c.initial_states, True)
    bar = (2e-3, 1e-2) if out_dtype == "bf16" else (1e-3, 2e-3)
    assert_close(out.float().cpu().numpy(), ref, "ssd out", *bar, peak_rel=True)
    assert_close(fin.cpu().numpy(), rfin, "ssd states", *bar, peak_rel=True)


@pytest.mark.slow
def test_config4_ssd_sampled(gdn_lib):
    gdn = gdn_lib
    _announce("config4 ssd [2,8192,80,64] (sampled oracle)")
    c = synth.device_config4_ssd()
    out, fin = gdn.ssd_combined_fwd(c.x, c.dt, c.A, c.B, c.C, c.D, c.z, c.dt_bias, True,
                                    (0.0, float("inf")))
    torch.cuda.synchronize()
    heads = [0, 41, 79]
    h = lambda t: t.float().cpu().numpy()
    ref, rfin = oracle.ssd_combined(h(c.x), h(c.dt), h(c.A), h(c.B), h(c.C), h(c.D), h(c.z),
                                    h(c.dt_bias), True, (0.0, float("inf")), None, True, heads=heads)
    assert_close(h(out[:, :, heads]), ref, "ssd out", peak_rel=True)
    assert_close(h(fin[:, heads]), rfin, "ssd states", peak_rel=True)


# ------------------------------------------------------------------ adapter and helpers
def test_forward_gdn_end_to_end(gdn_lib):
    gdn = gdn_lib
    _announce("forward_gdn extend + decode")
    from types import SimpleNamespace
    case = synth.edge_case("fwd", (30, 70), has_init=(1, 0), seed=33, num_slots=6)
    d = upload(case)
    layer = SimpleNamespace(num_k_heads=case.H_qk, num_v_heads=case.H_v, head_k_dim=case.d_k,
                            head_v_dim=case.d_v, A_log=d["A_log"], dt_bias=d["dt_bias"],
                            scale=case.scale, layer_id=0)
    fb = SimpleNamespace(forward_mode="extend", state_pool=[d["pool"]], state_slots=d["slot"],
                         cu_seqlens=d["cu"], has_initial_state=d["has_init"], max_seqlen=70)
    out = gdn.forward_gdn(layer, fb, d["mixed"], d["a"], d["b"])
    ref, _, fin = oracle.gdn_extend(case.q, case.k, case.v, case.a, case.b, case.A_log, case.dt_bias,
                                    case.cu_seqlens, case.slot, case.has_init, case.pool, case.scale)
    assert out.shape == (case.T, case.H_v * case.d_v)
    assert_close(out.float().cpu().numpy().reshape(ref.shape), ref, "forward_gdn extend")


def test_validate_slots(gdn_lib):
    gdn = gdn_lib
    _announce("validate_slots")
    s = lambda v: torch.tensor(v, dtype=torch.int32, device="cuda")
    assert gdn.validate_slots(s([3, 1, -1, -1, 0]), 4) == 0
    assert gdn.validate_slots(s([3, 4]), 4) == 1
    assert gdn.validate_slots(s([2, 1, 2]), 4) == 2
    assert gdn.validate_slots(s([9, 9]), 4) == 3
    assert gdn.validate_slots(s([]), 4) == 0


# ------------------------------------------------------------------ state checkpoints
# One sequence per boundary kind: a chunk boundary, the start (zero state), inside the
# first chunk, the end of a one-chunk sequence, inside a later chunk, the first token of
# a chunk (m = 1), disabled (negative boundary), outside the sequence.
CKPT_LENS = (150, 64, 200, 7, 90, 130, 20, 30)
CKPT_INIT = (1, 0, 1, 1, 1, 0, 1, 1)
CKPT_REL = (64, 0, 37, 7, 70, 129, -1, 31)
CKPT_SLOT = (3, 0, 5, 1, 4, 2, 6, 6)


def _ckpt_args(case, relative):
    cu = case.cu_seqlens
    tok = np.array([r if (relative or r < 0) else cu[n] + r for n, r in enumerate(CKPT_REL)], np.int32)
    return tok, np.array(CKPT_SLOT, np.int32)


@pytest.mark.parametrize("path", ["chunked-bf16out", "chunked-f32out", "recurrent", "recurrent-short"])
def test_extend_checkpoints(gdn_lib, path):
    """Checkpoint states against the oracle's; outputs, final states and untouched
    checkpoint rows unchanged by the capture.  recurrent-short: the token-recurrent
    kernel's short-extend layout (host hint 8; the longer sequences continue past the
    four staged tokens)."""
    gdn = gdn_lib
    _announce(f"extend checkpoints {path}")
    rec = path.startswith("recurrent")
    hint = 8 if path == "recurrent-short" else 0
    dtype = "f32" if rec else "bf16"
    case = synth.edge_case("ckpt", CKPT_LENS, has_init=CKPT_INIT, seed=31, num_slots=11, dtype=dtype)
    odt = torch.float32 if path == "chunked-f32out" else None
    relative = rec
    tok, cks = _ckpt_args(case, relative)
    d = upload(case)
    base = run_extend(gdn, case, d, out_dtype=odt, max_seqlen=hint)
    pool_base = d["pool"].clone()
    d2 = upload(case)
    states = torch.full((8, case.H_v, case.d_v, case.d_k), SENTINEL, dtype=torch.float32, device="cuda")
    q, k, v = gdn.split_mixed_qkv(d2["mixed"], case.H_qk, case.H_v, case.d_k, case.d_v)
    lg, bt = gdn.gate(d2["a"], d2["b"], d2["A_log"], d2["dt_bias"])
    ti = lambda x: torch.from_numpy(x).to("cuda")
    out = gdn.extend(q, k, v, lg, bt, d2["cu"], d2["slot"], d2["pool"], has_init=d2["has_init"],
                     scale=case.scale, out_dtype=odt, ckpt_token=ti(tok), ckpt_slot=ti(cks),
                     ckpt_states=states, ckpt_relative=relative, max_seqlen=hint)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32 if out.dtype == torch.float32 else torch.int16),
                       base.view(torch.int32 if base.dtype == torch.float32 else torch.int16)), "outputs changed"
    assert torch.equal(d2["pool"], pool_base), "final states changed"
    ck = {}
    abs_tok = np.array([r if r < 0 else case.cu_seqlens[n] + r for n, r in enumerate(CKPT_REL)])
    oracle.gdn_extend(case.q, case.k, case.v, case.a, case.b, case.A_log, case.dt_bias,
                      case.cu_seqlens, case.slot, case.has_init, case.pool, case.scale,
                      ckpt_token=abs_tok, ckpt_slot=np.array(CKPT_SLOT), ckpts=ck)
    assert sorted(ck) == [0, 1, 2, 3, 4, 5]
    got = states.cpu().numpy()
    bar = (2e-3, 1e-2) if path == "chunked-bf16out" else (1e-3, 2e-3)
    for s in ck:
        assert_close(got[s], ck[s], f"checkpoint row {s}", *bar)
    assert (got[6:] == SENTINEL).all(), "rows without a capture were written"


def test_ssd_checkpoints(gdn_lib):
    """ssd_combined_fwd checkpoint arguments (batched: boundaries relative to each batch
    element) against the oracle."""
    gdn = gdn_lib
    _announce("ssd checkpoints")
    c = synth.config4_ssd(seed=41, batch=4, L=150, H=6, P=64, G=2, Nst=128, initial=True)
    tb = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda", torch.bfloat16)
    tf = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda", torch.float32)
    rel = np.array([37, 64, 150, 0], np.int32)
    cks = np.array([2, 0, 3, 1], np.int32)
    states = torch.full((5, 6, 64, 128), SENTINEL, dtype=torch.float32, device="cuda")
    out, fin = gdn.ssd_combined_fwd(tb(c.x), tb(c.dt), tf(c.A), tb(c.B), tb(c.C), tb(c.D), tb(c.z),
                                    tf(c.dt_bias), True, (0.0, float("inf")), tf(c.initial_states),
                                    checkpoint_token_indices=torch.from_numpy(rel).cuda(),
                                    checkpoint_state_slots=torch.from_numpy(cks).cuda(),
                                    checkpoint_states=states)
    ck = {}
    oracle.ssd_combined(c.x, c.dt, c.A, c.B, c.C, c.D, c.z, c.dt_bias, True, (0.0, float("inf")),
                        c.initial_states, True, ckpt_token=rel, ckpt_slot=cks, ckpts=ck)
    got = states.cpu().numpy()
    for s in ck:
        assert_close(got[s], ck[s], f"ssd checkpoint row {s}", peak_rel=True)
    assert (got[4] == SENTINEL).all()


# ------------------------------------------------------------------ target verify
@pytest.mark.parametrize("tree", [False, True], ids=["chain", "tree"])
@pytest.mark.parametrize("keep_pool", [True, False])
def test_target_verify_states(gdn_lib, tree, keep_pool):
    """Verify batches (4 draft tokens per sequence, 8 sequences, one without a row):
    outputs and the state after every draft token against the oracle, for a chain and
    for a token tree (EAGLE topk = 2 shape: parents -1, 0, 0, 1); keep_pool leaves the
    pool untouched."""
    gdn = gdn_lib
    _announce(f"target verify tree={tree} keep_pool={keep_pool}")
    N, L = 8, 4
    case = synth.edge_case("verify", (L,) * N, has_init=1, seed=77, num_slots=12)
    rows = np.array([3, 0, 7, -1, 5, 1, 6, 2], np.int32)
    parents = np.tile(np.array([-1, 0, 0, 1], np.int32), N) if tree else None
    if tree:
        rows[3] = 4                                        # a tree needs every sequence's row
    d = upload(case)
    pool_before = d["pool"].clone()
    states = torch.full((9, L, case.H_v, case.d_v, case.d_k), SENTINEL, dtype=torch.float32, device="cuda")
    q, k, v = gdn.split_mixed_qkv(d["mixed"], case.H_qk, case.H_v, case.d_k, case.d_v)
    lg, bt = gdn.gate(d["a"], d["b"], d["A_log"], d["dt_bias"])
    out = gdn.extend(q, k, v, lg, bt, d["cu"], d["slot"], d["pool"], has_init=d["has_init"],
                     scale=case.scale, max_seqlen=L, spec_states=states,
                     spec_slot=torch.from_numpy(rows).cuda(),
                     spec_parent=None if parents is None else torch.from_numpy(parents).cuda(),
                     keep_pool=keep_pool)
    torch.cuda.synchronize()
    spec = {}
    ref, _, fin = oracle.gdn_extend(case.q, case.k, case.v, case.a, case.b, case.A_log, case.dt_bias,
                                    case.cu_seqlens, case.slot, case.has_init, case.pool, case.scale,
                                    spec_slot=rows, spec_parent=parents, spec=spec)
    assert_close(out.float().cpu().numpy(), ref, "verify out")
    got = states.cpu().numpy()
    for (r, i), S in spec.items():
        assert_close(got[r, i], S, f"verify state row {r} step {i}")
    if not tree:
        assert (got[8] == SENTINEL).all() and (got[4] == SENTINEL).all(), "row without a sequence written"
    if keep_pool:
        assert torch.equal(d["pool"], pool_before), "keep_pool: the pool changed"
    else:
        newpool = oracle.apply_final_states(case.pool, fin)
        assert_close(d["pool"].cpu().numpy()[case.slot], newpool[case.slot], "verify final states")


def test_target_verify_tree_forward_parents(gdn_lib):
    """Token trees whose parents point forward or at the token itself (inside the
    recorded rows, so a kernel that followed them would read rows not yet written): such
    a parent counts as -1 and the token starts from the sequence's start state."""
    gdn = gdn_lib
    _announce("target verify tree with forward parents")
    N, L = 6, 4
    case = synth.edge_case("verify-fwd", (L,) * N, has_init=1, seed=81, num_slots=10)
    rows = np.array([2, 0, 5, 1, 4, 3], np.int32)
    per_seq = [[-1, 2, 3, 1], [-1, 1, 0, 3], [3, 0, 1, 2], [-1, 0, 0, 1], [0, 3, 1, 2], [-1, 2, 2, 0]]
    parents = np.array(per_seq, np.int32).reshape(-1)
    d = upload(case)
    pool_before = d["pool"].clone()
    states = torch.full((6, L, case.H_v, case.d_v, case.d_k), SENTINEL, dtype=torch.float32, device="cuda")
    q, k, v = gdn.split_mixed_qkv(d["mixed"], case.H_qk, case.H_v, case.d_k, case.d_v)
    lg, bt = gdn.gate(d["a"], d["b"], d["A_log"], d["dt_bias"])
    out = gdn.extend(q, k, v, lg, bt, d["cu"], d["slot"], d["pool"], has_init=d["has_init"],
                     scale=case.scale, max_seqlen=L, spec_states=states,
                     spec_slot=torch.from_numpy(rows).cuda(), spec_parent=torch.from_numpy(parents).cuda(),
                     keep_pool=True)
    torch.cuda.synchronize()
    spec = {}
    ref, _, _ = oracle.gdn_extend(case.q, case.k, case.v, case.a, case.b, case.A_log, case.dt_bias,
                                  case.cu_seqlens, case.slot, case.has_init, case.pool, case.scale,
                                  spec_slot=rows, spec_parent=parents, spec=spec, spec_steps=L)
    assert_close(out.float().cpu().numpy(), ref, "verify out")
    got = states.cpu().numpy()
    for (r, i), S in spec.items():
        assert_close(got[r, i], S, f"verify state row {r} step {i}")
    assert torch.equal(d["pool"], pool_before), "keep_pool: the pool changed"


def test_forward_gdn_target_verify(gdn_lib):
    """forward_gdn in TARGET_VERIFY mode with a speculative state buffer: states per draft
    token recorded, pool untouched."""
    from types import SimpleNamespace
    gdn = gdn_lib
    _announce("forward_gdn target verify")
    N, L = 4, 3
    case = synth.edge_case("fwd-verify", (L,) * N, has_init=1, seed=79, num_slots=6)
    d = upload(case)
    pool_before = d["pool"].clone()
    rows = torch.tensor([1, 0, 3, 2], dtype=torch.int32, device="cuda")
    buf = torch.zeros((4, L, case.H_v, case.d_v, case.d_k), dtype=torch.float32, device="cuda")
    layer = SimpleNamespace(num_k_heads=case.H_qk, num_v_heads=case.H_v, head_k_dim=case.d_k,
                            head_v_dim=case.d_v, A_log=d["A_log"], dt_bias=d["dt_bias"], scale=case.scale,
                            layer_id=0)
    fb = SimpleNamespace(forward_mode="TARGET_VERIFY", state_slots=d["slot"], state_pool=[d["pool"]],
                         cu_seqlens=d["cu"], has_initial_state=d["has_init"], max_seqlen=L,
                         spec_states=[buf], spec_state_slots=rows)
    out = gdn.forward_gdn(layer, fb, d["mixed"], d["a"], d["b"])
    torch.cuda.synchronize()
    spec = {}
    ref, _, _ = oracle.gdn_extend(case.q, case.k, case.v, case.a, case.b, case.A_log, case.dt_bias,
                                  case.cu_seqlens, case.slot, case.has_init, case.pool, case.scale,
                                  spec_slot=rows.cpu().numpy(), spec=spec)
    assert_close(out.float().cpu().numpy().reshape(ref.shape), ref, "forward_gdn verify out")
    got = buf.cpu().numpy()
    for (r, i), S in spec.items():
        assert_close(got[r, i], S, f"forward_gdn verify state {r},{i}")
    assert torch.equal(d["pool"], pool_before)


# ------------------------------------------------------------------ graph-captured decode
def test_decode_graph_capture_padded(gdn_lib):
    """gdn_decode (gate folded in) captured once in a HIP graph over static buffers of 32
    rows of which 20 are live (slot -1 pads the rest), then replayed three times with new
    inputs copied into the static buffers and eager work in between.  Every replay is
    checked against the oracle step from the previous states; padded rows stay untouched."""
    gdn = gdn_lib
    _announce("decode graph capture, 20 live of 32 static rows")
    rows, live, H_qk, H_v, d = 32, 20, 2, 4, 128
    width = 2 * H_qk * d + H_v * d
    rng = np.random.default_rng(91)
    pool = torch.from_numpy(rng.normal(0, 0.1, (40, H_v, d, d)).astype(np.float32)).cuda()
    slot_h = np.full(rows, -1, np.int32)
    slot_h[:live] = rng.permutation(40)[:live]
    slot = torch.from_numpy(slot_h).cuda()
    A_log = torch.from_numpy(np.log(rng.uniform(1, 16, H_v)).astype(np.float32)).cuda()
    dt_bias = torch.from_numpy(rng.normal(0, 0.5, H_v).astype(np.float32)).cuda()
    mixed = torch.zeros((rows, width), dtype=torch.bfloat16, device="cuda")
    a = torch.zeros((rows, H_v), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((rows, H_v), dtype=torch.bfloat16, device="cuda")
    out = torch.full((rows, H_v, d), SENTINEL, dtype=torch.bfloat16, device="cuda")
    out0 = out.clone()
    q, k, v = gdn.split_mixed_qkv(mixed, H_qk, H_v, d, d)
    g_in = gdn.gdn_gate_inputs(a, b, A_log, dt_bias)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # (capture happens off the default stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            gdn.decode(q, k, v, None, None, slot, pool, scale=d ** -0.5, out=out, gate=g_in)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(out, out0), "capture must not run the kernel"
    states = pool.cpu().numpy().astype(np.float64)
    for rep in range(3):
        m = rng.standard_normal((rows, width)).astype(np.float32)
        av = rng.standard_normal((rows, H_v)).astype(np.float32)
        bv = rng.standard_normal((rows, H_v)).astype(np.float32)
        mixed.copy_(torch.from_numpy(m).to(torch.bfloat16))
        a.copy_(torch.from_numpy(av).to(torch.bfloat16))
        b.copy_(torch.from_numpy(bv).to(torch.bfloat16))
        _ = (mixed.float() * 2).sum()          # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        mh = mixed[:live].float().cpu().numpy()
        nq = H_qk * d
        ref, _, fin = oracle.gdn_decode(mh[:, :nq].reshape(live, H_qk, d), mh[:, nq:2 * nq].reshape(live, H_qk, d),
                                        mh[:, 2 * nq:].reshape(live, H_v, d), a[:live].float().cpu().numpy(),
                                        b[:live].float().cpu().numpy(), A_log.cpu().numpy(),
                                        dt_bias.cpu().numpy(), slot_h[:live], states, d ** -0.5)
        assert_close(out[:live].float().cpu().numpy(), ref, f"replay {rep} out")
        assert torch.equal(out[live:], out0[live:]), "padded rows were written"
        states = oracle.apply_final_states(states, fin)
        assert_close(pool.cpu().numpy()[slot_h[:live]], states[slot_h[:live]], f"replay {rep} states")


@pytest.mark.parametrize("with_init", [True, False])
def test_ssd_packed_varlen(gdn_lib, with_init):
    """ssd_combined_fwd in packed-varlen mode (seq_idx): three sequences of 100, 37 and 200
    tokens packed in one row (chunk boundaries inside and across sequences), each from its
    own initial state, with an absolute checkpoint boundary per sequence; against the
    oracle run on each sequence as a batch of one."""
    gdn = gdn_lib
    _announce(f"ssd packed varlen init={with_init}")
    lens, H, P, G, Nst = (100, 37, 200), 4, 64, 1, 128
    L = sum(lens)
    c = synth.config4_ssd(seed=123, batch=1, L=L, H=H, P=P, G=G, Nst=Nst, initial=False)
    rng = np.random.default_rng(124)
    init = rng.normal(0, 0.1, (3, H, P, Nst)).astype(np.float32) if with_init else None
    seq_idx = np.repeat(np.arange(3), lens)[None].astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(lens)])
    bnd = np.array([cu[0] + 64, cu[1] + 37, cu[2] + 150], np.int32)    # absolute boundaries
    tb = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda", torch.bfloat16)
    tf = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda", torch.float32)
    ck = torch.zeros((3, H, P, Nst), dtype=torch.float32, device="cuda")
    out, fin = gdn.ssd_combined_fwd(tb(c.x), tb(c.dt), tf(c.A), tb(c.B), tb(c.C), tb(c.D), tb(c.z),
                                    tf(c.dt_bias), True, (0.0, float("inf")),
                                    None if init is None else tf(init),
                                    seq_idx=torch.from_numpy(seq_idx).cuda(),
                                    checkpoint_token_indices=torch.from_numpy(bnd).cuda(),
                                    checkpoint_state_slots=torch.tensor([2, 0, 1], dtype=torch.int32,
                                                                        device="cuda"),
                                    checkpoint_states=ck)
    assert out.shape == (1, L, H, P) and fin.shape == (3, H, P, Nst)
    got, gfin, gck = out.float().cpu().numpy(), fin.cpu().numpy(), ck.cpu().numpy()
    for n, row in enumerate((2, 0, 1)):
        t0, t1 = cu[n], cu[n + 1]
        sl = lambda a: None if a is None else a[:, t0:t1]
        i0 = None if init is None else init[n:n + 1]
        ref, rfin = oracle.ssd_combined(sl(c.x), sl(c.dt), c.A, sl(c.B), sl(c.C), c.D, sl(c.z), c.dt_bias,
                                        True, (0.0, float("inf")), i0, True)
        assert_close(got[:, t0:t1], ref, f"ssd packed out seq {n}", peak_rel=True)
        assert_close(gfin[n], rfin[0], f"ssd packed final seq {n}", peak_rel=True)
        b = int(bnd[n] - t0)                    # the state after the first b tokens
        _, rck = oracle.ssd_combined(sl(c.x)[:, :b], sl(c.dt)[:, :b], c.A, sl(c.B)[:, :b], sl(c.C)[:, :b],
                                     c.D, sl(c.z)[:, :b], c.dt_bias, True, (0.0, float("inf")), i0, True)
        assert_close(gck[row], rck[0], f"ssd packed checkpoint seq {n}", peak_rel=True)
