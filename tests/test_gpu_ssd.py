"""GPU parity of the chunk-128 delta-off kernel (the Mamba2 SSD mode behind
ssd_combined_fwd) against the float64 oracle: segment-parallel scans of ragged
sequences (lengths around the chunk and segment sizes, zero-length sequences, a length
hint that is too small), initial states, checkpoints at and between segment
boundaries, workspace sizes, long memory, and the kernel choice itself.

Bars: rel-L2 <= 2e-3 (bf16 output) or 1e-3 (fp32 output) on outputs and states, the
max-abs bound relative to the peak for these delta-off tensors; untouched pool slots
and skipped rows bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
from hybrid_model_linear_amd import synth
from gpu_util import assert_close

pytestmark = pytest.mark.gpu

SENTINEL = -12345.0


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _tb(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda", torch.bfloat16)


def _tf(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda", torch.float32)


def _ragged_case(seed, lens, H=6, G=2, P=64, N=128, A_scale=1.0):
    """Packed delta-off inputs for ragged sequences (one row of batch 1) with the
    workload's value distributions: x, dt, B, C, D, z ~ N(0, 1) bf16, A = -U(1, 16) (times
    A_scale), dt_bias ~ N(0, 0.5)."""
    L = int(sum(lens))
    c = synth.config4_ssd(seed=seed, batch=1, L=max(L, 1), H=H, P=P, G=G, Nst=N, initial=False)
    c.A = (c.A * A_scale).astype(np.float32)
    return c


def _run_extend(c, lens, *, slot, has_init, pool, max_seqlen, out_dtype=torch.bfloat16, chunk=0,
                workspace=None, ckpt=None, gdn=None):
    L = int(sum(lens))
    H, P = c.x.shape[2], c.x.shape[3]
    G, N = c.B.shape[2], c.B.shape[3]
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
    g = gdn.ssd_gate_inputs(_tb(c.dt[0, :L]), _tf(c.A), _tf(c.dt_bias), True, (0.0, float("inf")))
    kw = dict(has_init=torch.from_numpy(np.asarray(has_init, np.int32)).cuda(), mode="ssd",
              D=_tb(c.D), z=_tb(c.z[0, :L]), max_seqlen=max_seqlen, out_dtype=out_dtype, chunk=chunk,
              gate=g)
    if ckpt is not None:
        kw.update(ckpt_token=ckpt[0], ckpt_slot=ckpt[1], ckpt_states=ckpt[2])
    args = (_tb(c.C[0, :L]), _tb(c.B[0, :L]), _tb(c.x[0, :L]), None, None, cu,
            torch.from_numpy(np.asarray(slot, np.int32)).cuda(), pool)
    kern = gdn.extend_kernel(*args, workspace=workspace, **kw)
    out = gdn.extend(*args, workspace=workspace, **kw)
    return out, kern


def _oracle_seq(c, lens, n, init, ckpt_rel=None):
    cu = np.concatenate([[0], np.cumsum(lens)])
    t0, t1 = int(cu[n]), int(cu[n + 1])
    sl = lambda a: a[:, t0:t1]
    i0 = None if init is None else init[None]
    ck = {}
    kw = {}
    if ckpt_rel is not None:
        kw = dict(ckpt_token=np.array([ckpt_rel]), ckpt_slot=np.array([0]), ckpts=ck)
    ref, fin = oracle.ssd_combined(sl(c.x), sl(c.dt), c.A, sl(c.B), sl(c.C), c.D, sl(c.z), c.dt_bias,
                                   True, (0.0, float("inf")), i0, True, **kw)
    return ref[0], fin[0], ck.get(0)


# lengths around the chunk (128) and the segment sizes the host picks, an empty
# sequence and a skipped one
LENS = (1, 127, 128, 129, 300, 0, 700, 256, 513)


@pytest.mark.parametrize("hint", ["exact", "small", "none"])
@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_ssd_chunk128_ragged_segments(gdn_lib, hint, out_dtype):
    """Ragged packed sequences through the segment-parallel chunk-128 kernel, against the
    oracle per sequence: the exact length hint (several segments for the long ones), a
    hint below the longest length (its last segment takes the rest) and no hint (one
    segment per sequence).  Pool slots of skipped sequences and untouched slots keep
    their bytes; skipped rows of the output keep the sentinel."""
    gdn = gdn_lib
    _announce(f"ssd chunk128 ragged hint={hint} out={out_dtype}")
    lens = LENS
    c = _ragged_case(17, lens)
    H, P, N = 6, 64, 128
    rng = np.random.default_rng(3)
    nseq = len(lens)
    pool0 = rng.normal(0, 0.3, (nseq + 4, H, P, N)).astype(np.float32)
    slot = rng.permutation(nseq + 4)[:nseq].astype(np.int32)
    slot[3] = -1                                             # skipped
    has_init = np.array([1, 0, 1, 1, 0, 1, 1, 0, 1], np.int32)
    pool = _tf(pool0)
    odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    max_seqlen = {"exact": max(lens), "small": 200, "none": 0}[hint]
    out, kern = _run_extend(c, lens, slot=slot, has_init=has_init, pool=pool, max_seqlen=max_seqlen,
                            out_dtype=odt, gdn=gdn)
    assert kern == ("ssd_chunked128", []), kern
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    gpool = pool.cpu().numpy()
    cu = np.concatenate([[0], np.cumsum(lens)])
    bar = (2e-3, 1e-2) if out_dtype == "bf16" else (1e-3, 2e-3)
    for n in range(nseq):
        if slot[n] < 0:
            continue
        init = pool0[slot[n]] if has_init[n] else None
        ref, fin, _ = _oracle_seq(c, lens, n, init)
        if lens[n]:
            assert_close(got[cu[n]:cu[n + 1]], ref, f"seq {n} (len {lens[n]}) out", *bar, peak_rel=True)
        assert_close(gpool[slot[n]], fin, f"seq {n} state", *bar, peak_rel=True)
    untouched = np.setdiff1d(np.arange(nseq + 4), slot[slot >= 0])
    assert np.array_equal(gpool[untouched], pool0[untouched]), "untouched slots changed"


def test_ssd_chunk128_many_sequences(gdn_lib):
    """A hundred packed sequences (log-uniform lengths up to ~600, every 17th empty, one
    skipped, random initial states for most) with an odd number of heads per group: every
    chunk slot of the per-chunk preparation finds its sequence; the outputs of all
    written rows together and every final state match the oracle, untouched slots keep
    their bytes.  (Outputs are held to the bar as one tensor: for a one-token sequence
    the bf16 rounding of the exact result alone reaches rel-L2 2.07e-3 here, 1.64e-3 over
    all rows.)"""
    gdn = gdn_lib
    _announce("ssd chunk128 many sequences")
    rng = np.random.default_rng(5)
    lens = np.exp(rng.uniform(0, np.log(600), 100)).astype(np.int64)
    lens[::17] = 0
    lens = tuple(int(v) for v in lens)
    nseq, H, P, N = len(lens), 3, 64, 128
    c = _ragged_case(51, lens, H=H, G=1)
    pool0 = rng.normal(0, 0.3, (nseq + 8, H, P, N)).astype(np.float32)
    slot = rng.permutation(nseq + 8)[:nseq].astype(np.int32)
    slot[41] = -1
    has_init = (rng.random(nseq) < 0.7).astype(np.int32)
    pool = _tf(pool0)
    out, kern = _run_extend(c, lens, slot=slot, has_init=has_init, pool=pool, max_seqlen=max(lens), gdn=gdn)
    assert kern == ("ssd_chunked128", []), kern
    torch.cuda.synchronize()
    got, gpool = out.float().cpu().numpy(), pool.cpu().numpy()
    cu = np.concatenate([[0], np.cumsum(lens)])
    outs, refs = [], []
    for n in range(nseq):
        if slot[n] < 0:
            continue
        ref, fin, _ = _oracle_seq(c, lens, n, pool0[slot[n]] if has_init[n] else None)
        outs.append(got[cu[n]:cu[n + 1]])
        refs.append(ref)
        assert_close(gpool[slot[n]], fin, f"seq {n} state", peak_rel=True)
    assert_close(np.concatenate(outs), np.concatenate(refs), "outputs of all written rows", peak_rel=True)
    untouched = np.setdiff1d(np.arange(nseq + 8), slot[slot >= 0])
    assert np.array_equal(gpool[untouched], pool0[untouched]), "untouched slots changed"


def test_ssd_chunk128_skipped_rows_keep_sentinel(gdn_lib):
    gdn = gdn_lib
    _announce("ssd chunk128 skipped rows")
    lens = (200, 150, 90)
    c = _ragged_case(23, lens)
    L = sum(lens)
    out = torch.full((L, 6, 64), SENTINEL, dtype=torch.bfloat16, device="cuda")
    before = out.clone()
    pool = torch.zeros((3, 6, 64, 128), dtype=torch.float32, device="cuda")
    cu = torch.tensor([0, 200, 350, 440], dtype=torch.int32, device="cuda")
    g = gdn.ssd_gate_inputs(_tb(c.dt[0]), _tf(c.A), _tf(c.dt_bias), True, (0.0, float("inf")))
    gdn.extend(_tb(c.C[0]), _tb(c.B[0]), _tb(c.x[0]), None, None, cu,
               torch.tensor([0, -1, 2], dtype=torch.int32, device="cuda"), pool,
               has_init=torch.zeros(3, dtype=torch.int32, device="cuda"), mode="ssd", D=_tb(c.D),
               z=_tb(c.z[0]), max_seqlen=200, out=out, gate=g)
    torch.cuda.synchronize()
    assert torch.equal(out[200:350].view(torch.int16), before[200:350].view(torch.int16)), \
        "rows of the skipped sequence were written"
    assert (pool[1] == 0).all(), "the skipped sequence's slot was written"
    ref, fin, _ = _oracle_seq(c, lens, 2, None)
    assert_close(out[350:].float().cpu().numpy(), ref, "seq 2 out", peak_rel=True)


def test_ssd_short_extend_token_recurrent(gdn_lib):
    """Short delta-off extends (host hint 8) take the token-recurrent kernel, which loads
    the first four tokens' inputs with the state and continues token by token past
    them: outputs and final states from random initial states against the oracle."""
    gdn = gdn_lib
    _announce("ssd short extend (token-recurrent)")
    lens = (6, 3, 8, 1, 0, 5)
    c = _ragged_case(41, lens, H=4, G=1)
    rng = np.random.default_rng(41)
    init = rng.standard_normal((len(lens), 4, 64, 128)).astype(np.float32)
    pool = torch.from_numpy(init.copy()).cuda()
    out, kern = _run_extend(c, lens, slot=list(range(len(lens))), has_init=[1] * len(lens), pool=pool,
                            max_seqlen=8, gdn=gdn)
    torch.cuda.synchronize()
    assert kern[0] == "recurrent", kern
    cu = np.concatenate([[0], np.cumsum(lens)])
    got, st = out.float().cpu().numpy(), pool.cpu().numpy()
    for n in range(len(lens)):
        ref, fin, _ = _oracle_seq(c, lens, n, init[n])
        if lens[n]:
            assert_close(got[cu[n]:cu[n + 1]], ref, f"seq {n} out", peak_rel=True)
        assert_close(st[n], fin, f"seq {n} state", peak_rel=True)


@pytest.mark.parametrize("ws", ["full", "one_segment"])
def test_ssd_chunk128_workspace_sizes(gdn_lib, ws):
    """A caller-given workspace: the size the library asks for (several segments) and the
    smallest one it accepts (one segment per sequence) give the same results up to
    rounding, both within the bar."""
    gdn = gdn_lib
    _announce(f"ssd chunk128 workspace {ws}")
    lens = (1000, 600)
    c = _ragged_case(29, lens)
    pool = torch.zeros((2, 6, 64, 128), dtype=torch.float32, device="cuda")
    # one segment per sequence: fp16 B and C copies and the raw C B^T tiles of the
    # T / 128 + N chunk slots (ten 32 x 32 fp16 tiles per slot and group), G = 2
    need = 2 * sum(lens) * 2 * 128 * 2 + (sum(lens) // 128 + 2) * 2 * 10 * 32 * 32 * 2
    if ws == "full":
        cu = torch.tensor([0, 1000, 1600], dtype=torch.int32, device="cuda")
        g = gdn.ssd_gate_inputs(_tb(c.dt[0]), _tf(c.A), _tf(c.dt_bias), True, (0.0, float("inf")))
        need = gdn.extend_workspace_size(_tb(c.C[0]), _tb(c.B[0]), _tb(c.x[0]), None, None, cu,
                                         torch.tensor([0, 1], dtype=torch.int32, device="cuda"), pool,
                                         mode="ssd", max_seqlen=1000, gate=g, D=_tb(c.D), z=_tb(c.z[0]))
        assert need > 2 * sum(lens) * 2 * 128 * 2 + (sum(lens) // 128 + 2) * 2 * 10 * 32 * 32 * 2
    workspace = torch.empty(need, dtype=torch.uint8, device="cuda")
    out, kern = _run_extend(c, lens, slot=[0, 1], has_init=[0, 0], pool=pool, max_seqlen=1000,
                            workspace=workspace, gdn=gdn)
    assert kern == ("ssd_chunked128", [])
    torch.cuda.synchronize()
    for n in range(2):
        ref, fin, _ = _oracle_seq(c, lens, n, None)
        t0 = sum(lens[:n])
        assert_close(out[t0:t0 + lens[n]].float().cpu().numpy(), ref, f"seq {n} out", peak_rel=True)
        assert_close(pool[n].cpu().numpy(), fin, f"seq {n} state", peak_rel=True)


# boundaries (relative): start, inside the first chunk, a chunk boundary, inside a later
# chunk, the start of a later segment, the end, outside, disabled
CK_REL = (0, 37, 256, 610, 1024, 1100, 1201, -1)
CK_SLOT = (5, 0, 3, 1, 6, 2, 4, 7)


def test_ssd_chunk128_checkpoints(gdn_lib):
    """One checkpoint per sequence at every kind of boundary, with eight sequences of
    1100 tokens split into segments: the state after the tokens before each boundary
    against the oracle's; rows without a capture keep the sentinel."""
    gdn = gdn_lib
    _announce("ssd chunk128 checkpoints")
    lens = (1100,) * 8
    c = _ragged_case(31, lens, H=4, G=1)
    rng = np.random.default_rng(9)
    pool0 = rng.normal(0, 0.3, (8, 4, 64, 128)).astype(np.float32)
    pool = _tf(pool0)
    states = torch.full((8, 4, 64, 128), SENTINEL, dtype=torch.float32, device="cuda")
    cu = np.concatenate([[0], np.cumsum(lens)])
    tok = torch.from_numpy(np.array([r if r < 0 else cu[n] + r for n, r in enumerate(CK_REL)], np.int32)).cuda()
    cks = torch.from_numpy(np.array(CK_SLOT, np.int32)).cuda()
    out, kern = _run_extend(c, lens, slot=list(range(8)), has_init=[1] * 8, pool=pool, max_seqlen=1100,
                            ckpt=(tok, cks, states), gdn=gdn)
    assert kern[0] == "ssd_chunked128"
    torch.cuda.synchronize()
    got = states.cpu().numpy()
    for n, r in enumerate(CK_REL):
        ref, fin, ck = _oracle_seq(c, lens, n, pool0[n], ckpt_rel=r if r <= 1100 else None)
        if 0 <= r <= 1100:
            assert_close(got[CK_SLOT[n]], ck, f"seq {n} checkpoint at {r}", peak_rel=True)
        else:
            assert (got[CK_SLOT[n]] == SENTINEL).all(), f"seq {n}: a row without a capture was written"
        if n == 2:
            assert_close(out[cu[n]:cu[n + 1]].float().cpu().numpy(), ref, "seq 2 out", peak_rel=True)
            assert_close(pool[n].cpu().numpy(), fin, "seq 2 state", peak_rel=True)


@pytest.mark.parametrize("scale", [1e-2, 1e-3])
def test_ssd_chunk128_long_memory(gdn_lib, scale):
    """Weak decay (A scaled by 1e-2, 1e-3): the state carries thousands of tokens, so the
    precision of the state operand of every chunk and of the segment combination shows;
    both output types held to their bars."""
    gdn = gdn_lib
    _announce(f"ssd chunk128 long memory A x{scale}")
    lens = (3000, 1500)
    c = _ragged_case(37, lens, A_scale=scale)
    refs = [_oracle_seq(c, lens, n, None) for n in range(2)]
    for odt, bar in ((torch.bfloat16, (2e-3, 1e-2)), (torch.float32, (1e-3, 2e-3))):
        pool = torch.zeros((2, 6, 64, 128), dtype=torch.float32, device="cuda")
        out, kern = _run_extend(c, lens, slot=[0, 1], has_init=[0, 0], pool=pool, max_seqlen=3000,
                                out_dtype=odt, gdn=gdn)
        assert kern[0] == "ssd_chunked128"
        torch.cuda.synchronize()
        for n in range(2):
            ref, fin, _ = refs[n]
            t0 = sum(lens[:n])
            assert_close(out[t0:t0 + lens[n]].float().cpu().numpy(), ref, f"{odt} seq {n} out", *bar,
                         peak_rel=True)
            assert_close(pool[n].cpu().numpy(), fin, f"{odt} seq {n} state", *bar, peak_rel=True)


def test_ssd_chunk64_still_available(gdn_lib):
    """chunk=64 selects the chunk-64 kernel (no workspace), with the same results up to
    rounding."""
    gdn = gdn_lib
    _announce("ssd chunk64 explicit")
    lens = (300, 129)
    c = _ragged_case(41, lens)
    pool = torch.zeros((2, 6, 64, 128), dtype=torch.float32, device="cuda")
    out, kern = _run_extend(c, lens, slot=[0, 1], has_init=[0, 0], pool=pool, max_seqlen=300, chunk=64,
                            gdn=gdn)
    assert kern == ("chunked64", ["chunk64_requested"])
    torch.cuda.synchronize()
    for n in range(2):
        ref, fin, _ = _oracle_seq(c, lens, n, None)
        t0 = sum(lens[:n])
        assert_close(out[t0:t0 + lens[n]].float().cpu().numpy(), ref, f"seq {n} out", peak_rel=True)


def test_ssd_combined_fwd_runs_chunk128(gdn_lib):
    """ssd_combined_fwd (batched mode) takes the chunk-128 kernel with its own workspace."""
    gdn = gdn_lib
    _announce("ssd_combined_fwd kernel choice")
    c = synth.config4_ssd(seed=5, batch=2, L=300, H=4, P=64, G=1, Nst=128, initial=False)
    T = 600
    cu = torch.tensor([0, 300, 600], dtype=torch.int32, device="cuda")
    g = gdn.ssd_gate_inputs(_tb(c.dt).view(T, 4), _tf(c.A), _tf(c.dt_bias), True, (0.0, float("inf")))
    pool = torch.zeros((2, 4, 64, 128), dtype=torch.float32, device="cuda")
    kern = gdn.extend_kernel(_tb(c.C).view(T, 1, 128), _tb(c.B).view(T, 1, 128), _tb(c.x).view(T, 4, 64),
                             None, None, cu, torch.arange(2, dtype=torch.int32, device="cuda"), pool,
                             has_init=torch.zeros(2, dtype=torch.int32, device="cuda"), mode="ssd",
                             D=_tb(c.D), z=_tb(c.z).view(T, 4, 64), max_seqlen=300, gate=g)
    assert kern == ("ssd_chunked128", [])
    out, fin = gdn.ssd_combined_fwd(_tb(c.x), _tb(c.dt), _tf(c.A), _tb(c.B), _tb(c.C), _tb(c.D), _tb(c.z),
                                    _tf(c.dt_bias), True, (0.0, float("inf")))
    ref, rfin = oracle.ssd_combined(c.x, c.dt, c.A, c.B, c.C, c.D, c.z, c.dt_bias, True, (0.0, float("inf")),
                                    None, True)
    assert_close(out.float().cpu().numpy(), ref, "out", peak_rel=True)
    assert_close(fin.cpu().numpy(), rfin, "states", peak_rel=True)
