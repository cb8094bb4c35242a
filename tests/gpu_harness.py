"""Helpers for the GPU parity tests: run a workload through the C ABI and
compare it with the CPU oracle on the same seeded inputs."""
import numpy as np

from oracle.attention import attend_case

O_TOL = {"bf16": 1e-2, "fp8": 4e-2}
LSE_TOL = 2e-3


def run_gpu(case, mode=0, num_cus=None, kv_indices=None, decoder=None, words=None):
    import torch
    import paged_mla_decode_02_amd as mla
    inputs = mla.device_inputs(case.q_codes, case.q_scale, case.pool_codes, case.kv_scale,
                               case.qo_indptr, case.kv_indptr,
                               case.kv_indices if kv_indices is None else kv_indices)
    dec = decoder or mla.MlaDecoder(case.heads, case.q_len, case.q_dtype, case.kv_dtype, case.causal,
                                    float(case.sm_scale), mode, num_cus)
    T = case.num_tokens
    o = torch.full((max(T, 1), case.heads, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((max(T, 1), case.heads), float("nan"), dtype=torch.float32, device="cuda")
    words = dec.run(inputs, case.kv_lens, o, lse, words)
    torch.cuda.synchronize()
    return o[:T].float().cpu().numpy(), lse[:T].cpu().numpy(), words


def tolerance(case):
    return O_TOL["fp8"] if "fp8" in (case.q_dtype, case.kv_dtype) else O_TOL["bf16"]


def compare(case, O, LSE, rows=None, ref=None):
    """Max |O - O_ref| / max |O_ref| over the compared rows, and max |dLSE| over
    finite entries; -inf entries must match exactly. Returns (ratio, lse_err)."""
    if ref is None:
        ref = attend_case(case, rows)
    errs, refmax, lse_err = 0.0, 0.0, 0.0
    for b, (Ob, Lb) in ref.items():
        t0, t1 = int(case.qo_indptr[b]), int(case.qo_indptr[b + 1])
        got_o, got_l = O[t0:t1], LSE[t0:t1]
        assert not np.isnan(got_o).any(), f"row {b}: NaN (unwritten?) output"
        assert not np.isnan(got_l).any(), f"row {b}: NaN LSE"
        errs = max(errs, float(np.abs(got_o - Ob).max(initial=0.0)))
        refmax = max(refmax, float(np.abs(Ob).max(initial=0.0)))
        ninf = np.isneginf(Lb)
        assert np.array_equal(np.isneginf(got_l), ninf), f"row {b}: -inf LSE pattern differs"
        if (~ninf).any():
            lse_err = max(lse_err, float(np.abs(got_l[~ninf] - Lb[~ninf]).max()))
    ratio = errs / refmax if refmax > 0 else (0.0 if errs == 0 else np.inf)
    return ratio, lse_err


def assert_parity(case, O, LSE, rows=None, ref=None):
    ratio, lse_err = compare(case, O, LSE, rows, ref)
    tol = tolerance(case)
    assert ratio <= tol, f"{case.name}: max|err|/max|O_ref| = {ratio:.3e} > {tol}"
    assert lse_err <= LSE_TOL, f"{case.name}: max|dLSE| = {lse_err:.3e} > {LSE_TOL}"
    return ratio, lse_err
