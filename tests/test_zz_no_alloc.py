"""gdn_extend_noalloc against gdn_extend_gated: the same delta-off extend, once with a
workspace the caller allocated and once with the library's static scratch, on two
calls in a row, the second with a smaller input (it finds the first call's contents in
the scratch).  Both take the chunk-128 kernel with the same segment plan, so outputs
and pool slots must agree bit for bit."""
import numpy as np
import pytest
import torch

from hybrid_model_linear_amd import synth

pytestmark = pytest.mark.gpu


def _tb(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda", torch.bfloat16)


def _tf(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda", torch.float32)


def _i32(x):
    return torch.from_numpy(np.asarray(x, np.int32)).cuda()


def _call(gdn, lens, seed, out_dtype, noalloc):
    """One ragged delta-off extend (H=6 heads of headdim 64, 2 groups of dstate 128):
    returns (out, pool, kernel)."""
    H, P, G, N = 6, 64, 2, 128
    L = int(sum(lens))
    c = synth.config4_ssd(seed=seed, batch=1, L=L, H=H, P=P, G=G, Nst=N, initial=False)
    rng = np.random.default_rng(seed + 1)
    nseq = len(lens)
    pool = _tf(rng.normal(0, 0.3, (nseq + 2, H, P, N)).astype(np.float32))
    slot = rng.permutation(nseq + 2)[:nseq]
    has_init = (np.arange(nseq) % 2).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(lens)])
    g = gdn.ssd_gate_inputs(_tb(c.dt[0]), _tf(c.A), _tf(c.dt_bias), True, (0.0, float("inf")))
    args = (_tb(c.C[0]), _tb(c.B[0]), _tb(c.x[0]), None, None, _i32(cu), _i32(slot), pool)
    kw = dict(has_init=_i32(has_init), mode="ssd", D=_tb(c.D), z=_tb(c.z[0]),
              max_seqlen=max(lens), gate=g)
    kern = gdn.extend_kernel(*args, out_dtype=out_dtype, **kw)
    out = torch.full((L, H, P), -7.0, dtype=out_dtype, device="cuda")
    if noalloc:
        gdn.extend_noalloc(*args, out=out, **kw)
    else:
        gdn.extend(*args, out=out, **kw)
    torch.cuda.synchronize()
    return out, pool, kern


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_the_allocating_entry_point(gdn_lib, out_dtype):
    gdn = gdn_lib
    for step, (lens, seed) in enumerate([((700, 129, 1500, 0, 256, 1), 41), ((300, 5), 42)]):
        print(f"[case] noalloc step {step} lens={lens} out={out_dtype}", flush=True)
        ref, ref_pool, kern = _call(gdn, lens, seed, out_dtype, noalloc=False)
        assert kern == ("ssd_chunked128", []), kern
        got, got_pool, _ = _call(gdn, lens, seed, out_dtype, noalloc=True)
        assert torch.equal(got.view(torch.int16) if out_dtype == torch.bfloat16 else got.view(torch.int32),
                           ref.view(torch.int16) if out_dtype == torch.bfloat16 else ref.view(torch.int32)), \
            f"step {step}: outputs differ"
        assert torch.equal(got_pool.view(torch.int32), ref_pool.view(torch.int32)), f"step {step}: pools differ"
        assert torch.isfinite(got.float()).all()


def test_noalloc_needs_a_caller_out(gdn_lib):
    with pytest.raises(ValueError, match="caller-given out"):
        gdn_lib.extend_noalloc(*(torch.empty(0),) * 8, out=None)
