"""gemm_f16_f32acc_noalloc, the entry point that allocates nothing, against
gemm_f16_f32acc, both called through the C ABI.

Two calls in a row, the second with a smaller problem, each of a shape whose
128x128 tiles split K over several workgroups (so the static scratch buffer
holds the partial tiles and counters): the two entry points run the same plan
and kernels, so C must agree bit for bit, and within the normalized error bound
of the oracle (bit-exact with small-integer inputs).  A first call on a fresh
stream must not take device memory (free memory unchanged once the library's
code is loaded), where the allocating entry point allocates that stream's
scratch."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import dense_gemm_optimisation_f32_amd as dg
import oracle
import seeded_inputs as si

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _dev(buf):
    return torch.from_numpy(np.ascontiguousarray(buf)).to("cuda")


def _free_bytes():
    hip = ctypes.CDLL("libamdhip64.so")
    free, total = ctypes.c_size_t(), ctypes.c_size_t()
    assert hip.hipMemGetInfo(ctypes.byref(free), ctypes.byref(total)) == 0
    return free.value


@pytest.mark.parametrize("kind_vals", ["pm1", "int4"])
def test_noalloc_matches_allocating_entry_point(kind_vals):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = dg.load_library()
    # The static buffer is a device global of the library: the runtime places
    # it in device memory when the code holding it is first used on the GPU and
    # keeps it until the process ends.  A first small call (no K split) does
    # that, so the memory checks below see the calls alone.
    t = _dev(np.zeros(64 * 64, np.float16))
    out = torch.zeros(64 * 64, dtype=torch.float32, device="cuda")
    assert lib.gemm_f16_f32acc_noalloc(64, 64, 64, 1.0, t.data_ptr(), 64, t.data_ptr(), 64, 0.0, out.data_ptr(),
                                       64, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    # 512^2 x 8192: 16 tiles x 8 splits (the whole static buffer); 300 x 200 x 6000: 6 tiles x 5 splits
    for i, ((M, N, K), seed) in enumerate((((512, 512, 8192), 201), ((300, 200, 6000), 202))):
        print(f"[noalloc] {kind_vals} M={M} N={N} K={K}", flush=True)
        stream = torch.cuda.Stream()   # a stream no call has used: the allocating entry point allocates for it
        h = stream.cuda_stream
        p = si.gemm_problem(M, N, K, in_dtype=np.float16, kind=kind_vals, seed=seed)
        dA, dB = _dev(p["A"]), _dev(p["B"])
        c_new, c_ref = _dev(p["C"]), _dev(p["C"])
        torch.cuda.synchronize()
        f0 = _free_bytes()
        rc_new = lib.gemm_f16_f32acc_noalloc(M, N, K, 1.5, dA.data_ptr(), K, dB.data_ptr(), N, -0.5,
                                             c_new.data_ptr(), N, h)
        stream.synchronize()
        f1 = _free_bytes()
        rc_ref = lib.gemm_f16_f32acc(M, N, K, 1.5, dA.data_ptr(), K, dB.data_ptr(), N, -0.5, c_ref.data_ptr(), N, h)
        stream.synchronize()
        f2 = _free_bytes()
        assert rc_new == 0 and rc_ref == 0, (rc_new, rc_ref)
        assert f0 - f1 < (1 << 20), f"the no-allocation call took {f0 - f1} bytes of device memory"
        if i == 0:   # the check can see an allocation: the allocating entry point's first split on the stream
            assert f1 - f2 >= (16 << 20), f1 - f2
        assert torch.equal(c_new, c_ref)
        ref, bound = oracle.gemm_ref(M, N, K, 1.5, p["A"], K, p["B"], N, -0.5, p["C"], N)
        got = c_new.view(M, N).cpu().numpy()
        if kind_vals == "int4":
            assert np.array_equal(got, ref.astype(np.float32))
        assert oracle.normalized_error(got, ref, bound) <= 1e-5
