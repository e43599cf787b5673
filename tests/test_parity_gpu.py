"""Parity of the HIP library with the CPU oracle, element by element (GPU).

Acceptance (for every entry point):
  * normalized error  max |C - ref| / (|alpha| sum_k |a_ik||b_kj| + |beta||c_ij|) <= 1e-5,
    with ref and bound from the fp64 oracle on the very values the GPU received;
  * bit-exact C == float32(ref) when every entry is a small integer, because then
    every partial sum, alpha*acc, beta*c and their sum is an exact fp32 value and
    the summation order cannot matter;
  * bit-identical results from two calls with the same arguments.
Workloads are the five benchmark configurations (SGEMM 512^3; the 1001x777x513
non-multiple shape and 1024x1024x512; the M = N sweep at K = 1024; HGEMM 2048^3 and
4096^3; 16 batched 1024^3 HGEMMs with beta = 1) plus ragged, padded, misaligned and
degenerate cases.  Every benchmark configuration up to 4096 is compared in full; the
larger sweep points and some large edge cases compare 64 seeded rows (always the first
and last).
"""
from __future__ import annotations

import numpy as np
import pytest

import dense_gemm_optimisation_f32_amd as dg
import oracle
import seeded_inputs as si

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dg.load_library()
    yield
    torch.cuda.synchronize()


def note(msg: str):
    print(f"[parity] {msg}", flush=True)


def to_dev(buf):
    buf = np.ascontiguousarray(buf)
    if buf.dtype == np.uint16:   # bfloat16 bit patterns
        return torch.from_numpy(buf.view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(buf).to("cuda")


IN_DTYPE = {"f32": np.float32, "f16": np.float16, "bf16": "bf16"}


def call(kind, p, alpha, beta, dA, dB, dC, stream=None):
    M, N, K = p["M"], p["N"], p["K"]
    tA, tB = int(p.get("transA", False)), int(p.get("transB", False))
    if tA or tB:   # the op(A)/op(B) entry points
        fn = {"f32": dg.gemm_f32_ex, "f16": dg.gemm_f16_f32acc_ex, "bf16": dg.gemm_bf16_f32acc_ex}[kind]
        fn(tA, tB, M, N, K, alpha, dA, p["lda"], dB, p["ldb"], beta, dC, p["ldc"], stream)
    else:
        fn = {"f32": dg.gemm_f32, "f16": dg.gemm_f16_f32acc, "bf16": dg.gemm_bf16_f32acc}[kind]
        fn(M, N, K, alpha, dA, p["lda"], dB, p["ldb"], beta, dC, p["ldc"], stream)


def rows_of(dC, M, N, ldc, rows=None):
    """Rows of the device C (all when rows is None) as a float32 host array.
    ``dC`` is a flat buffer of at least M*ldc elements."""
    full = dC[: M * ldc].view(M, ldc)[:, :N]
    if rows is not None:
        full = full[torch.as_tensor(rows, device="cuda", dtype=torch.long)]
    return full.cpu().numpy()


def to_dev_offset(buf, offset):
    """``buf`` on the device starting ``offset`` elements into a fresh allocation
    (offset 1 puts an fp32 array, offset 2 an fp16 one, 4 bytes past a 16-byte
    boundary)."""
    if offset == 0:
        return to_dev(buf)
    return to_dev(np.concatenate([np.zeros(offset, buf.dtype), buf]))[offset:]


def run_and_check(kind, M, N, K, alpha, beta, *, kind_vals="pm1", lda=None, ldb=None, ldc=None,
                  sample=None, exact=False, seed=42, c_nan=False, transA=False, transB=False, offset=0):
    in_dtype = IN_DTYPE[kind]
    note(f"{kind} M={M} N={N} K={K} alpha={alpha} beta={beta} vals={kind_vals} lda={lda} ldb={ldb} "
         f"ldc={ldc} sample={sample} seed={seed} transA={int(transA)} transB={int(transB)} offset={offset}")
    p = si.gemm_problem(M, N, K, lda=lda, ldb=ldb, ldc=ldc, in_dtype=in_dtype, kind=kind_vals, seed=seed,
                        with_c=not c_nan, transA=transA, transB=transB)
    dA, dB = to_dev_offset(p["A"], offset), to_dev_offset(p["B"], offset)
    if c_nan:   # beta = 0: C must be written without being read
        dC = torch.full((M * p["ldc"],), float("nan"), dtype=torch.float32, device="cuda")
    else:
        dC = to_dev(p["C"])
    call(kind, p, alpha, beta, dA, dB, dC)
    torch.cuda.synchronize()
    rows = si.sample_rows(seed, M, sample) if sample else None
    got = rows_of(dC, M, N, p["ldc"], rows)
    ref, bound = oracle.gemm_ref(M, N, K, alpha, p["A"], p["lda"], p["B"], p["ldb"], beta,
                                 None if beta == 0 else p["C"], p["ldc"], rows=rows, transA=transA, transB=transB,
                                 bf16=kind == "bf16")
    if exact:
        want = ref.astype(np.float32)
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{len(bad)} elements differ, first {bad[:3].tolist()}"
    err = oracle.normalized_error(got, ref, bound)
    assert err <= TOL, f"normalized error {err:.3e} > {TOL}"
    # the pad columns of C (ldc > N, NaN in the input) are never written
    if p["ldc"] > N and M > 0:
        assert bool(torch.isnan(dC[: M * p["ldc"]].view(M, p["ldc"])[:, N:]).all())
    return err


# ------------------------------------------------------------------ configurations
def test_cfg1_sgemm_512():
    run_and_check("f32", 512, 512, 512, 1.0, 0.0, c_nan=True)
    run_and_check("f32", 512, 512, 512, 1.0, 0.0, kind_vals="int4", exact=True)


@pytest.mark.parametrize("alpha,beta", [(1.5, -0.5), (1.0, 0.0)])
@pytest.mark.parametrize("M,N,K", [(1001, 777, 513), (1024, 1024, 512)])
def test_cfg2_sgemm_odd_and_regular(M, N, K, alpha, beta):
    run_and_check("f32", M, N, K, alpha, beta)
    run_and_check("f32", M, N, K, alpha, beta, kind_vals="int4", exact=True, seed=7)


@pytest.mark.parametrize("n", [128, 256, 512, 1024, 2048, 4096])
def test_cfg3_sgemm_sweep_full(n):
    run_and_check("f32", n, n, 1024, 1.0, 0.0, c_nan=True)


@pytest.mark.parametrize("n", [8192, 16384])
def test_cfg3_sgemm_sweep_sampled(n):
    run_and_check("f32", n, n, 1024, 1.0, 0.0, sample=64, c_nan=True)


def test_cfg3_sgemm_int_exact():
    run_and_check("f32", 2048, 2048, 1024, 1.0, 0.0, kind_vals="int4", exact=True, seed=3)
    run_and_check("f32", 16384, 16384, 1024, 1.0, 0.0, kind_vals="int4", exact=True, sample=64, seed=4)


@pytest.mark.parametrize("n", [2048, 4096])
def test_cfg4_hgemm(n):
    # the whole C in both cases: the oracle takes a few seconds at 4096^3 on the host's cores
    run_and_check("f16", n, n, n, 1.0, 0.0, c_nan=True)
    run_and_check("f16", n, n, n, 1.0, 0.0, kind_vals="int4", exact=True, seed=5)


def batched_check(M, N, K, nb, alpha, beta, *, kind_vals="pm1", sample=None, exact=False, seed=42,
                  pad=0, share_a=False, transA=False, transB=False, fmt="f16"):
    note(f"batched {fmt} M={M} N={N} K={K} batch={nb} alpha={alpha} beta={beta} vals={kind_vals} "
         f"sample={sample} pad={pad} share_a={share_a} transA={int(transA)} transB={int(transB)}")
    bf = fmt == "bf16"
    in_np = np.uint16 if bf else np.float16
    a_rows, a_cols = (K, M) if transA else (M, K)
    b_rows, b_cols = (N, K) if transB else (K, N)
    lda, ldb, ldc = a_cols + pad, b_cols + pad, N + pad
    probs = [si.gemm_problem(M, N, K, lda=lda, ldb=ldb, ldc=ldc, in_dtype=IN_DTYPE[fmt], kind=kind_vals,
                             seed=seed, batch=b, transA=transA, transB=transB) for b in range(nb)]
    sA = 0 if share_a else a_rows * lda + 8 * pad
    sB, sC = b_rows * ldb + 8 * pad, M * ldc + 8 * pad

    def pack(key, stride, n_el, dtype):
        fill = 0x7FC0 if dtype == np.uint16 else np.nan   # NaN between members
        buf = np.full(stride * (nb - 1) + n_el if stride else n_el, fill, dtype=dtype)
        for b in range(nb if stride else 1):
            buf[b * stride: b * stride + n_el] = probs[b][key]
        return buf

    A = pack("A", sA, a_rows * lda, in_np)
    B = pack("B", sB, b_rows * ldb, in_np)
    C = pack("C", sC, M * ldc, np.float32)
    dA, dB, dC = to_dev(A), to_dev(B), to_dev(C)
    if transA or transB:
        fn = dg.gemm_batched_bf16_f32acc_ex if bf else dg.gemm_batched_f16_f32acc_ex
        fn(int(transA), int(transB), M, N, K, alpha, dA, lda, sA, dB, ldb, sB, beta, dC, ldc, sC, nb)
    else:
        fn = dg.gemm_batched_bf16_f32acc if bf else dg.gemm_batched_f16_f32acc
        fn(M, N, K, alpha, dA, lda, sA, dB, ldb, sB, beta, dC, ldc, sC, nb)
    torch.cuda.synchronize()
    rows = si.sample_rows(seed, M, sample) if sample else None
    worst = 0.0
    for b in range(nb):
        got = rows_of(dC[b * sC:], M, N, ldc, rows)
        ref, bound = oracle.gemm_ref(M, N, K, alpha, A[b * sA:], lda, B[b * sB:], ldb, beta,
                                     C[b * sC: b * sC + M * ldc], ldc, rows=rows, transA=transA, transB=transB,
                                     bf16=bf)
        if exact:
            assert np.array_equal(got, ref.astype(np.float32)), f"member {b} not bit-exact"
        e = oracle.normalized_error(got, ref, bound)
        assert e <= TOL, f"member {b}: normalized error {e:.3e}"
        worst = max(worst, e)
    return worst


def test_cfg5_batched_hgemm():
    # every element of all 16 members, random and small-integer inputs
    batched_check(1024, 1024, 1024, 16, 1.0, 1.0)
    batched_check(1024, 1024, 1024, 16, 1.0, 1.0, kind_vals="int4", exact=True, seed=9)


def test_batched_small_full_and_shared_operand():
    batched_check(200, 136, 72, 5, 1.5, -0.5, pad=3)
    batched_check(64, 96, 130, 3, 1.0, 1.0, share_a=True)
    batched_check(33, 65, 17, 4, 1.0, 0.0, kind_vals="int4", exact=True, pad=1)


@pytest.mark.parametrize("kind", ["f32", "f16"])
def test_fast_paths_with_padded_leading_dimensions(kind):
    # whole tiles and 16-byte aligned rows, but every leading dimension larger than
    # the logical width: the direct-to-LDS kernels must honour lda/ldb/ldc
    # (the SGEMM case needs enough tiles to leave the split-K small-problem kernel)
    if kind == "f32":
        run_and_check(kind, 2048, 2048, 320, 1.5, -0.5, lda=328, ldb=2056, ldc=2060, sample=128)
    else:
        run_and_check(kind, 512, 384, 320, 1.5, -0.5, lda=328, ldb=392, ldc=400)
    run_and_check(kind, 4096, 4096, 256, 1.0, 0.0, lda=264, ldb=4104, ldc=4100, sample=64, c_nan=True)


@pytest.mark.parametrize("M,N,K", [(512, 512, 512), (64, 64, 4096), (1000, 100, 3000), (96, 1024, 40)])
def test_small_problem_split_k(M, N, K):
    # grids too small for the 64x64 direct-to-LDS tile: the eight waves of a
    # workgroup split K and their partial tiles are summed in a fixed order --
    # check values and bits
    run_and_check("f32", M, N, K, 1.5, -0.5, lda=K + 1)
    run_and_check("f32", M, N, K, 1.0, 1.0, kind_vals="int4", exact=True, seed=11)


@pytest.mark.parametrize("K", [256, 320, 384, 512, 1024])
def test_hgemm_128_ring_lengths(K):
    # 128x128 direct-to-LDS HGEMM, four-slice ring with staggered refills: K/64 slices
    # from exactly the ring (no refill) through the tail-only refill to a steady loop
    run_and_check("f16", 256, 384, K, 1.5, -0.5)
    run_and_check("f16", 256, 384, K, 1.0, 1.0, kind_vals="int4", exact=True, seed=29)
    run_and_check("f16", 384, 256, K, 1.0, 0.0, kind_vals="int4", exact=True, seed=31, transA=True, transB=True)


def test_batched_whole_tiles_mid_size():
    # 128x128 whole tiles with K a multiple of 64 (the mid-size direct-to-LDS path), 3 members
    batched_check(384, 256, 320, 3, 1.5, -0.5)
    batched_check(256, 384, 512, 2, 1.0, 1.0, kind_vals="int4", exact=True)


# ------------------------------------------------------------------ edge cases
RAGGED = [(1, 1, 1), (1, 7, 3), (3, 1, 5), (2, 3, 1), (33, 65, 17), (127, 129, 63), (129, 127, 65),
          (257, 255, 129), (31, 33, 300), (300, 17, 1000), (17, 300, 8), (65, 64, 9)]


@pytest.mark.parametrize("kind", ["f32", "f16"])
@pytest.mark.parametrize("M,N,K", RAGGED)
def test_ragged_shapes(kind, M, N, K):
    run_and_check(kind, M, N, K, 1.5, -0.5)
    run_and_check(kind, M, N, K, 1.5, -0.5, lda=K + 3, ldb=N + 5, ldc=N + 1, kind_vals="int4", exact=True)


@pytest.mark.parametrize("kind", ["f32", "f16"])
def test_aligned_lds_with_ragged_tails(kind):
    # leading dimensions that keep the vector path while M, N, K end mid-tile and mid-vector
    run_and_check(kind, 300, 260, 203, 1.0, 1.0, lda=208, ldb=264, ldc=264)
    run_and_check(kind, 513, 515, 517, 1.5, -0.5, lda=520, ldb=520, ldc=520, kind_vals="int4", exact=True)


@pytest.mark.parametrize("kind", ["f32", "f16", "bf16"])
def test_beta_zero_does_not_read_c(kind):
    run_and_check(kind, 130, 70, 40, 1.0, 0.0, c_nan=True)


def nan_like(buf):
    """A buffer of the same shape and element type holding NaN (0x7FC0 for bf16 patterns)."""
    return np.full_like(buf, 0x7FC0) if buf.dtype == np.uint16 else np.full_like(buf, np.nan)


@pytest.mark.parametrize("kind", ["f32", "f16", "bf16"])
def test_quick_returns(kind):
    note(f"{kind} quick returns")
    M, N = 37, 45
    for K, alpha, beta in [(0, 1.0, -0.5), (16, 0.0, 1.5), (0, 1.0, 0.0), (16, 0.0, 0.0)]:
        p = si.gemm_problem(M, N, max(K, 1), in_dtype=IN_DTYPE[kind])
        p["K"] = K
        C0 = p["C"].copy()
        dC = to_dev(C0 if beta != 0 else np.full_like(C0, np.nan))
        dA = to_dev(nan_like(p["A"]))   # A and B must not be read
        dB = to_dev(nan_like(p["B"]))
        call(kind, dict(p, lda=max(K, 1)), alpha, beta, dA, dB, dC)
        torch.cuda.synchronize()
        got = dC.cpu().numpy()
        want = (np.float32(beta) * C0) if beta != 0 else np.zeros_like(C0)
        assert np.array_equal(got, want)
    # empty problems leave C untouched
    dC = to_dev(np.arange(12, dtype=np.float32))
    call(kind, dict(M=0, N=3, K=4, lda=4, ldb=3, ldc=3), 1.0, 1.0, None, None, dC)
    call(kind, dict(M=3, N=0, K=4, lda=4, ldb=1, ldc=1), 1.0, 1.0, None, None, dC)
    torch.cuda.synchronize()
    assert np.array_equal(dC.cpu().numpy(), np.arange(12, dtype=np.float32))


@pytest.mark.parametrize("kind", ["f32", "f16", "bf16"])
def test_misaligned_pointers(kind):
    note(f"{kind} operands offset by one element from a 16-byte boundary")
    M, N, K = 190, 210, 150
    p = si.gemm_problem(M, N, K, in_dtype=IN_DTYPE[kind], seed=21)
    dA = to_dev(np.concatenate([np.zeros(1, p["A"].dtype), p["A"]]))[1:]
    dB = to_dev(np.concatenate([np.zeros(1, p["B"].dtype), p["B"]]))[1:]
    dC = to_dev(np.concatenate([np.zeros(1, np.float32), p["C"]]))[1:]
    call(kind, p, 1.5, -0.5, dA, dB, dC)
    torch.cuda.synchronize()
    ref, bound = oracle.gemm_ref(M, N, K, 1.5, p["A"], K, p["B"], N, -0.5, p["C"], N, bf16=kind == "bf16")
    assert oracle.normalized_error(rows_of(dC, M, N, N), ref, bound) <= TOL


@pytest.mark.parametrize("kind,M,N,K", [("f32", 1001, 777, 513), ("f16", 4096, 4096, 4096),
                                        ("f32", 4096, 4096, 1024), ("bf16", 2048, 2048, 2048)])
def test_deterministic(kind, M, N, K):
    note(f"{kind} determinism M={M} N={N} K={K}")
    p = si.gemm_problem(M, N, K, in_dtype=IN_DTYPE[kind], seed=33)
    dA, dB = to_dev(p["A"]), to_dev(p["B"])
    outs = []
    for _ in range(2):
        dC = to_dev(p["C"])
        call(kind, p, 1.5, -0.5, dA, dB, dC)
        outs.append(dC)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


def test_runs_on_the_given_stream():
    note("f32 and f16 on a side stream")
    s = torch.cuda.Stream()
    for kind in ("f32", "f16"):
        in_dtype = np.float32 if kind == "f32" else np.float16
        p = si.gemm_problem(256, 192, 320, in_dtype=in_dtype, seed=44)
        dA, dB, dC = to_dev(p["A"]), to_dev(p["B"]), to_dev(p["C"])
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            call(kind, p, 1.0, 1.0, dA, dB, dC, stream=s)
        s.synchronize()
        ref, bound = oracle.gemm_ref(256, 192, 320, 1.0, p["A"], 320, p["B"], 192, 1.0, p["C"], 192)
        assert oracle.normalized_error(rows_of(dC, 256, 192, 192), ref, bound) <= TOL


def test_concurrent_streams():
    # the library keeps no state between calls: four different kernels enqueued on four
    # streams at once (SGEMM 256x256 direct-to-LDS, HGEMM 128x128 direct-to-LDS, the
    # split-K SGEMM, a batched HGEMM) each give their own oracle result
    note("four kernels on four streams at once")
    cases = [("f32", 4096, 4096, 512, 64), ("f16", 2048, 2048, 512, 64), ("f32", 300, 260, 700, None)]
    probs, devs = [], []
    for i, (kind, M, N, K, sample) in enumerate(cases):
        p = si.gemm_problem(M, N, K, in_dtype=np.float32 if kind == "f32" else np.float16, seed=80 + i)
        probs.append(p)
        devs.append((to_dev(p["A"]), to_dev(p["B"]), to_dev(p["C"])))
    nb, bm, bn, bk = 3, 128, 136, 320
    bp = [si.gemm_problem(bm, bn, bk, in_dtype=np.float16, seed=90, batch=b) for b in range(nb)]
    bA = to_dev(np.concatenate([q["A"] for q in bp]))
    bB = to_dev(np.concatenate([q["B"] for q in bp]))
    bC = to_dev(np.concatenate([q["C"] for q in bp]))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(4)]
    for s, (kind, M, N, K, _), p, (dA, dB, dC) in zip(streams, cases, probs, devs):
        call(kind, p, 1.5, -0.5, dA, dB, dC, stream=s)
    dg.gemm_batched_f16_f32acc(bm, bn, bk, 1.0, bA, bk, bm * bk, bB, bn, bk * bn, 1.0, bC, bn, bm * bn, nb,
                               streams[3])
    torch.cuda.synchronize()
    for i, ((kind, M, N, K, sample), p, (_, _, dC)) in enumerate(zip(cases, probs, devs)):
        rows = si.sample_rows(80 + i, M, sample) if sample else None
        ref, bound = oracle.gemm_ref(M, N, K, 1.5, p["A"], p["lda"], p["B"], p["ldb"], -0.5, p["C"], p["ldc"],
                                     rows=rows)
        assert oracle.normalized_error(rows_of(dC, M, N, p["ldc"], rows), ref, bound) <= TOL, kind
    for b in range(nb):
        q = bp[b]
        ref, bound = oracle.gemm_ref(bm, bn, bk, 1.0, q["A"], bk, q["B"], bn, 1.0, q["C"], bn)
        assert oracle.normalized_error(rows_of(bC[b * bm * bn:], bm, bn, bn), ref, bound) <= TOL, f"member {b}"


# ------------------------------------------------------------------ op(A) / op(B)
# C = alpha*op(A)op(B) + beta*C with A stored K x M (transA) and/or B stored
# N x K (transB).  Each case names the kernel it reaches; the int4 runs are
# bit-exact, which also proves that no element is read from the wrong place.
OPS = [(True, False), (False, True), (True, True)]


@pytest.mark.parametrize("kind", ["f32", "f16"])
@pytest.mark.parametrize("tA,tB", OPS)
@pytest.mark.parametrize("M,N,K", [(1, 7, 3), (33, 65, 17), (127, 129, 63), (257, 255, 129), (300, 17, 1000)])
def test_transposed_ragged(kind, tA, tB, M, N, K):
    # SGEMM: split-K small-problem kernel; HGEMM: masked register-staged kernel
    run_and_check(kind, M, N, K, 1.5, -0.5, transA=tA, transB=tB)
    a_cols, b_cols = (M if tA else K), (K if tB else N)
    run_and_check(kind, M, N, K, 1.5, -0.5, lda=a_cols + 3, ldb=b_cols + 5, ldc=N + 1, kind_vals="int4",
                  exact=True, transA=tA, transB=tB, seed=13)


@pytest.mark.parametrize("tA,tB", [(False, False)] + OPS)
def test_sgemm_register_kernel(tA, tB):
    # >= 256 tiles of 128x128 with K below two slices, which the direct-to-LDS
    # kernel cannot take (ragged edges -> masked register kernel, whole tiles ->
    # unmasked)
    run_and_check("f32", 2100, 2100, 40, 1.5, -0.5, sample=64, transA=tA, transB=tB)
    run_and_check("f32", 2100, 2100, 40, 1.0, 1.0, sample=64, kind_vals="int4", exact=True, transA=tA,
                  transB=tB, seed=5)
    run_and_check("f32", 2048, 2048, 48, 1.0, 0.0, sample=64, c_nan=True, transA=tA, transB=tB)


@pytest.mark.parametrize("kind", ["f32", "f16"])
@pytest.mark.parametrize("tA,tB", [(False, False)] + OPS)
def test_direct_to_lds_straddling_chunks(kind, tA, tB):
    # an MN-contiguous operand whose M or N is not a multiple of the 16-byte
    # chunk (4 floats, 8 halves): the direct-to-LDS slices stop before row K-1
    # and the K tail takes up to a whole slice; int4 runs prove that no element
    # comes from the wrong place
    if kind == "f32":
        cases = [(2050, 2046, 300), (1001, 1003, 1024), (4095, 4093, 256), (1002, 998, 65)]
    else:
        cases = [(1500, 1500, 1536), (2050, 2046, 320), (1001, 1003, 1024), (4100, 4092, 512), (1500, 1500, 257)]
    for idx, (M, N, K) in enumerate(cases):
        run_and_check(kind, M, N, K, 1.5, -0.5, ldc=N + 1, sample=48, transA=tA, transB=tB, seed=61 + idx)
        run_and_check(kind, M, N, K, 1.0, 1.0, sample=48, kind_vals="int4", exact=True, transA=tA, transB=tB,
                      seed=71 + idx)


@pytest.mark.parametrize("tA,tB", [(False, False)] + OPS)
def test_direct_to_lds_dword_aligned_rows(tA, tB):
    # rows that start 4-byte but not 16-byte aligned (odd fp32 leading dimensions,
    # fp16 ones of 2 or 6 mod 8, base pointers 4 bytes past a 16-byte boundary)
    # still take the direct-to-LDS kernels: whole 256x256 tiles, then ragged tiles
    for kind, pa, pb, off, ragged in [("f32", 1, 3, 1, (1000, 1000, 300)), ("f16", 2, 6, 2, (3000, 3000, 320))]:
        M, N, K = 4096, 4096, 256
        a_cols, b_cols = (M if tA else K), (K if tB else N)
        run_and_check(kind, M, N, K, 1.5, -0.5, lda=a_cols + pa, ldb=b_cols + pb, ldc=N + 1, sample=64,
                      transA=tA, transB=tB, offset=off)
        M, N, K = ragged
        a_cols, b_cols = (M if tA else K), (K if tB else N)
        run_and_check(kind, M, N, K, 1.0, 1.0, lda=a_cols + pb, ldb=b_cols + pa, ldc=N + 2, sample=96,
                      kind_vals="int4", exact=True, transA=tA, transB=tB, offset=off, seed=29)


@pytest.mark.parametrize("kind", ["f32", "f16"])
@pytest.mark.parametrize("tA,tB", OPS)
def test_transposed_fast_paths(kind, tA, tB):
    # whole tiles, 16-byte aligned rows, padded leading dimensions: the direct-to-LDS
    # kernels (256x256 tiles at 4096^2, 128x128 below)
    M = N = 4096
    K = 256
    a_cols, b_cols = (M if tA else K), (K if tB else N)
    run_and_check(kind, M, N, K, 1.5, -0.5, lda=a_cols + 8, ldb=b_cols + 16, ldc=N + 4, sample=64,
                  transA=tA, transB=tB)
    run_and_check(kind, M, N, K, 1.0, 0.0, sample=32, kind_vals="int4", exact=True, transA=tA, transB=tB,
                  seed=17)
    if kind == "f32":
        M, N, K = 2048, 2048, 320
    else:
        M, N, K = 512, 384, 320
    a_cols, b_cols = (M if tA else K), (K if tB else N)
    run_and_check(kind, M, N, K, 1.5, -0.5, lda=a_cols + 8, ldb=b_cols + 8, ldc=N + 4, sample=128,
                  transA=tA, transB=tB)
    run_and_check(kind, M, N, K, 1.0, 1.0, sample=64, kind_vals="int4", exact=True, transA=tA, transB=tB,
                  seed=19)


@pytest.mark.parametrize("tA,tB", [(False, False)] + OPS)
def test_sgemm_64_tiles_direct_to_lds(tA, tB):
    # fewer than 256 tiles of 128x128 but at least 256 whole 64x64 tiles: the
    # 64x64 direct-to-LDS kernel, whose four K groups take one eight-k step of
    # each slice and run the slices in pairs, with a two-slice ring (A stored
    # K x M, or K below four slices) or a four-slice one.  K = 64 .. 224 give two
    # to seven slices (every ring ending in both buffer parities); 120 and 136
    # add tails of three steps and of one, split over the groups; 416 is a
    # longer run.
    for M, N, K in [(1024, 1024, 64), (1024, 1024, 96), (1024, 1024, 128), (1024, 1024, 160),
                    (1024, 1024, 192), (1024, 1024, 224), (1024, 1024, 120), (1024, 1024, 136),
                    (1024, 2048, 416)]:
        a_cols, b_cols = (M if tA else K), (K if tB else N)
        run_and_check("f32", M, N, K, 1.5, -0.5, lda=a_cols + 4, ldb=b_cols + 12, ldc=N + 3, sample=128,
                      transA=tA, transB=tB)
        run_and_check("f32", M, N, K, 1.0, 1.0, sample=64, kind_vals="int4", exact=True, transA=tA, transB=tB,
                      seed=23)


def _ld4(cols, pad):
    # a leading dimension that keeps rows 16-byte aligned (a multiple of four floats)
    return cols + (-cols) % 4 + pad


@pytest.mark.parametrize("tA,tB", [(False, False)] + OPS)
@pytest.mark.parametrize("M,N,K", [(1000, 1000, 1000), (1000, 1000, 64), (996, 1204, 2000), (2052, 2100, 333),
                                   (4000, 4000, 95), (4000, 4000, 1024)])
def test_sgemm_ragged_direct_to_lds(M, N, K, tA, tB):
    # M, N not multiples of the tile and K not of 32, 16-byte aligned rows: the
    # direct-to-LDS kernels with clamped loads, the K tail from global memory and
    # masked stores (64x64 tiles up to 1000^2, 128x128 at 2052x2100, 256x256 at
    # 4000^2, one round of 256 such tiles)
    a_cols, b_cols = (M if tA else K), (K if tB else N)
    sample = 64 if M * N > 2_000_000 else 128
    run_and_check("f32", M, N, K, 1.5, -0.5, lda=_ld4(a_cols, 4), ldb=_ld4(b_cols, 8), ldc=N + 3, sample=sample,
                  transA=tA, transB=tB)
    run_and_check("f32", M, N, K, 1.0, 1.0, sample=sample, kind_vals="int4", exact=True, transA=tA, transB=tB,
                  lda=_ld4(a_cols, 0), ldb=_ld4(b_cols, 0), seed=37)


@pytest.mark.parametrize("tA,tB", [(False, False), (False, True)])
def test_sgemm_ragged_direct_to_lds_rows(tA, tB):
    # M not a multiple of four is fine while A is K-contiguous (its chunks run along k)
    N = 1200 if not tB else 1201
    run_and_check("f32", 999, N, 2000, 1.5, -0.5, lda=2004, ldb=_ld4(2000 if tB else N, 4), ldc=N + 1, sample=128,
                  transA=tA, transB=tB)
    run_and_check("f32", 999, N, 2000, 1.0, 0.0, c_nan=True, sample=64, kind_vals="int4", exact=True,
                  transA=tA, transB=tB, seed=41)


def _ld8(cols, pad):
    # a leading dimension that keeps rows 16-byte aligned (a multiple of eight halves)
    return cols + (-cols) % 8 + pad


@pytest.mark.parametrize("tA,tB", [(False, False)] + OPS)
@pytest.mark.parametrize("M,N,K", [(1000, 1000, 300), (1000, 1000, 256), (2000, 2000, 2000), (3000, 3000, 320),
                                   (4000, 4000, 1000), (4104, 4104, 333)])
def test_hgemm_ragged_direct_to_lds(M, N, K, tA, tB):
    # M, N not multiples of the tile and K not of 64, 16-byte aligned rows: the
    # direct-to-LDS kernels with clamped loads, the K tail from global memory and
    # masked stores (128x128 tiles up to 2000^2; 256x256 from 3000^2, where one
    # round of 144 such tiles beats three rounds of 128x128 ones)
    a_cols, b_cols = (M if tA else K), (K if tB else N)
    sample = 64 if M * N > 2_000_000 else 128
    run_and_check("f16", M, N, K, 1.5, -0.5, lda=_ld8(a_cols, 8), ldb=_ld8(b_cols, 16), ldc=N + 3, sample=sample,
                  transA=tA, transB=tB)
    run_and_check("f16", M, N, K, 1.0, 1.0, sample=sample, kind_vals="int4", exact=True, transA=tA, transB=tB,
                  lda=_ld8(a_cols, 0), ldb=_ld8(b_cols, 0), seed=43)


@pytest.mark.parametrize("tA,tB", [(False, False), (True, True)])
def test_hgemm_256_short_k(tA, tB):
    # 256x256 direct-to-LDS tiles with the shortest rings: three whole slices of 64, and
    # two plus a 32-k tail on a ragged grid (too short for the 128x128 four-slot ring)
    for M, N, K in [(4096, 4096, 192), (4000, 4000, 160)]:
        run_and_check("f16", M, N, K, 1.5, -0.5, sample=64, transA=tA, transB=tB)
        run_and_check("f16", M, N, K, 1.0, 1.0, sample=32, kind_vals="int4", exact=True, transA=tA, transB=tB,
                      seed=59)


def test_hgemm_ragged_direct_to_lds_rows_and_batch():
    # M not a multiple of eight with A K-contiguous; a ragged strided batch
    run_and_check("f16", 1001, 1000, 500, 1.5, -0.5, lda=504, ldb=1008, ldc=1001, sample=128)
    run_and_check("f16", 1001, 1000, 500, 1.0, 0.0, c_nan=True, kind_vals="int4", exact=True, sample=64, seed=47)
    batched_check(200, 136, 304, 3, 1.5, -0.5)
    batched_check(200, 136, 304, 3, 1.0, 1.0, kind_vals="int4", exact=True, seed=53)
    # leading dimensions and batch strides of 2 or 6 mod 8 halves (4-byte aligned rows)
    batched_check(256, 264, 320, 3, 1.5, -0.5, pad=2)
    batched_check(200, 136, 304, 3, 1.0, 1.0, kind_vals="int4", exact=True, pad=6, seed=59)
    # N not a multiple of eight (a chunk of B straddles N), the last member ending the buffer
    batched_check(200, 140, 320, 3, 1.0, 1.0, kind_vals="int4", exact=True, seed=67)
    batched_check(200, 140, 320, 3, 1.5, -0.5, pad=2, seed=68)


@pytest.mark.parametrize("tA,tB", [(False, False)] + OPS)
def test_hgemm_odd_leading_dimensions(tA, tB):
    # odd fp16 leading dimensions (rows alternately 2 bytes past a dword) and a
    # base pointer one half past a dword: the register-staged kernel's eight-half
    # loads from two dword-aligned loads and a shift, edges element by element
    M, N, K = 1000, 1001, 1003
    a_cols, b_cols = (M if tA else K), (K if tB else N)
    run_and_check("f16", M, N, K, 1.5, -0.5, lda=a_cols + 1 - a_cols % 2 + 2, ldb=b_cols + 1 - b_cols % 2,
                  ldc=N, sample=64, transA=tA, transB=tB)
    run_and_check("f16", M, N, K, 1.0, 1.0, lda=a_cols + 1 - a_cols % 2, ldb=b_cols + 3 - b_cols % 2,
                  sample=64, kind_vals="int4", exact=True, transA=tA, transB=tB, offset=1, seed=97)


@pytest.mark.parametrize("tA,tB", OPS)
def test_transposed_hgemm_register_whole_tiles(tA, tB):
    # whole 128x128 tiles but K too short for the direct-to-LDS ring: unmasked register kernel
    run_and_check("f16", 256, 256, 128, 1.5, -0.5, transA=tA, transB=tB)
    run_and_check("f16", 256, 256, 128, 1.0, 0.0, kind_vals="int4", exact=True, transA=tA, transB=tB)


@pytest.mark.parametrize("tA,tB", OPS)
def test_transposed_batched(tA, tB):
    batched_check(384, 256, 320, 3, 1.5, -0.5, transA=tA, transB=tB)
    batched_check(33, 65, 17, 4, 1.0, 0.0, kind_vals="int4", exact=True, pad=1, transA=tA, transB=tB)
    batched_check(200, 136, 72, 3, 1.0, 1.0, pad=3, share_a=True, transA=tA, transB=tB)


@pytest.mark.parametrize("kind", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("tA,tB", OPS)
def test_transposed_matches_untransposed(kind, tA, tB):
    # the same logical product through the plain and the op() entry points gives
    # the same bits (all four combinations use one k order)
    M, N, K = (4096, 4096, 512)
    note(f"{kind} op() vs plain M={M} N={N} K={K} transA={int(tA)} transB={int(tB)}")
    p = si.gemm_problem(M, N, K, in_dtype=IN_DTYPE[kind], seed=61)
    A2 = si.logical_transpose(p["A"], M, K) if tA else p["A"]
    B2 = si.logical_transpose(p["B"], K, N) if tB else p["B"]
    q = dict(p, transA=tA, transB=tB, lda=(M if tA else K), ldb=(K if tB else N))
    dA, dB, dA2, dB2 = to_dev(p["A"]), to_dev(p["B"]), to_dev(A2), to_dev(B2)
    dC1, dC2 = to_dev(p["C"]), to_dev(p["C"])
    call(kind, p, 1.5, -0.5, dA, dB, dC1)
    call(kind, q, 1.5, -0.5, dA2, dB2, dC2)
    torch.cuda.synchronize()
    assert torch.equal(dC1, dC2)


# ------------------------------------------------------------------ maximum sizes
def test_batched_beyond_one_launch():
    # more members than one launch's grid z holds (65535): the host splits the batch;
    # members on both sides of the split are checked against the oracle
    M, N, K, nb = 3, 5, 4, 70001
    note(f"batched M={M} N={N} K={K} batch={nb} (split over launches)")
    A = si.draw(101, nb * M * K).astype(np.float16)
    B = si.draw(102, nb * K * N).astype(np.float16)
    C = si.draw(103, nb * M * N)
    dA, dB, dC = to_dev(A), to_dev(B), to_dev(C)
    dg.gemm_batched_f16_f32acc(M, N, K, 1.5, dA, K, M * K, dB, N, K * N, -0.5, dC, N, M * N, nb)
    torch.cuda.synchronize()
    got = dC.cpu().numpy()
    members = sorted({0, 1, 65533, 65534, 65535, 65536, 65537, nb - 1} |
                     {int(x) % nb for x in si.splitmix64(7, 24)})
    for b in members:
        ref, bound = oracle.gemm_ref(M, N, K, 1.5, A[b * M * K:], K, B[b * K * N:], N, -0.5,
                                     C[b * M * N: (b + 1) * M * N], N)
        e = oracle.normalized_error(got[b * M * N: (b + 1) * M * N].reshape(M, N), ref, bound)
        assert e <= TOL, f"member {b}: normalized error {e:.3e}"


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (100, 70, 40)])
def test_batched_offsets_beyond_32_bits(M, N, K):
    # member 1 of each operand starts 2^31 + 64 elements after member 0: every
    # batch offset must be formed in 64 bits (the gap is NaN, so a wrapped offset
    # shows up as NaN or as a wrong value)
    stride = (1 << 31) + 64
    note(f"batched M={M} N={N} K={K} strides {stride} (64-bit member offsets)")
    probs = [si.gemm_problem(M, N, K, in_dtype=np.float16, seed=300, batch=b) for b in range(2)]
    dA = torch.full((stride + M * K,), float("nan"), dtype=torch.float16, device="cuda")
    dB = torch.full((stride + K * N,), float("nan"), dtype=torch.float16, device="cuda")
    dC = torch.full((stride + M * N,), float("nan"), dtype=torch.float32, device="cuda")
    for b in range(2):
        dA[b * stride: b * stride + M * K] = to_dev(probs[b]["A"])
        dB[b * stride: b * stride + K * N] = to_dev(probs[b]["B"])
        dC[b * stride: b * stride + M * N] = to_dev(probs[b]["C"])
    dg.gemm_batched_f16_f32acc(M, N, K, 1.0, dA, K, stride, dB, N, stride, 1.0, dC, N, stride, 2)
    torch.cuda.synchronize()
    for b in range(2):
        got = dC[b * stride: b * stride + M * N].view(M, N).cpu().numpy()
        ref, bound = oracle.gemm_ref(M, N, K, 1.0, probs[b]["A"], K, probs[b]["B"], N, 1.0, probs[b]["C"], N)
        e = oracle.normalized_error(got, ref, bound)
        assert e <= TOL, f"member {b}: normalized error {e:.3e}"
    # the gap after member 0's C is untouched
    assert bool(torch.isnan(dC[M * N: M * N + 4096]).all())
    del dA, dB, dC
    torch.cuda.empty_cache()


@pytest.mark.parametrize("transA", [False, True])
def test_row_offsets_beyond_32_bits(transA):
    # a leading dimension of 2^29 + 4 floats: row starts lie beyond 2^31 elements
    # (an 8 GiB operand of five stored rows), so row offsets are formed in 64 bits
    M, N, K = 5, 40, 5
    ld = (1 << 29) + 4
    note(f"f32 M={M} N={N} K={K} lda={ld} transA={int(transA)} (64-bit row offsets)")
    a_rows, a_cols = (K, M) if transA else (M, K)
    p = si.gemm_problem(M, N, K, in_dtype=np.float32, seed=310, transA=transA)
    dA = torch.full(((a_rows - 1) * ld + a_cols,), float("nan"), dtype=torch.float32, device="cuda")
    for r in range(a_rows):
        dA[r * ld: r * ld + a_cols] = to_dev(p["A"][r * a_cols: (r + 1) * a_cols])
    dB, dC = to_dev(p["B"]), to_dev(p["C"])
    dg.gemm_f32_ex(int(transA), 0, M, N, K, 1.5, dA, ld, dB, N, -0.5, dC, N)
    torch.cuda.synchronize()
    ref, bound = oracle.gemm_ref(M, N, K, 1.5, p["A"], a_cols, p["B"], N, -0.5, p["C"], N, transA=transA)
    assert oracle.normalized_error(rows_of(dC, M, N, N), ref, bound) <= TOL
    del dA
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ seeded random sweep
def _sweep_cases(n):
    """n problems drawn from a counter-based stream: shapes, padding, flags, alpha/beta."""
    u = si.splitmix64(2024, 16 * n)
    pick = lambda k, lo, hi: lo + int(u[k] % np.uint64(hi - lo + 1))
    alphas, betas = [1.0, 1.5, -0.75, 0.0], [0.0, 1.0, -0.5, 2.0]
    cases = []
    for c in range(n):
        b = 16 * c
        cases.append(dict(kind="f32" if u[b] % np.uint64(2) == 0 else "f16",
                          M=pick(b + 1, 1, 700), N=pick(b + 2, 1, 700), K=pick(b + 3, 1, 600),
                          pa=pick(b + 4, 0, 9), pb=pick(b + 5, 0, 9), pc=pick(b + 6, 0, 9),
                          tA=bool(u[b + 7] % np.uint64(2)), tB=bool(u[b + 8] % np.uint64(2)),
                          alpha=alphas[int(u[b + 9] % np.uint64(4))], beta=betas[int(u[b + 10] % np.uint64(4))],
                          ints=bool(u[b + 11] % np.uint64(3) == 0), seed=500 + c))
    return cases


@pytest.mark.parametrize("case", _sweep_cases(48), ids=lambda c: f"{c['kind']}-{c['M']}x{c['N']}x{c['K']}"
                         f"-t{int(c['tA'])}{int(c['tB'])}")
def test_random_sweep(case):
    # alpha = 0 and beta = 0 combinations included: C <- beta*C without reading A, B
    c = case
    a_cols, b_cols = (c["M"] if c["tA"] else c["K"]), (c["K"] if c["tB"] else c["N"])
    run_and_check(c["kind"], c["M"], c["N"], c["K"], c["alpha"], c["beta"],
                  kind_vals="int4" if c["ints"] else "pm1", exact=c["ints"],
                  lda=a_cols + c["pa"], ldb=b_cols + c["pb"], ldc=c["N"] + c["pc"],
                  transA=c["tA"], transB=c["tB"], seed=c["seed"], c_nan=(c["beta"] == 0.0))


def _dma_sweep_cases(n):
    """n problems large enough for the direct-to-LDS kernels (grids of 64x64 to 256x256 tiles),
    with 16-byte aligned rows, ragged M, N, K and random storage orientations."""
    u = si.splitmix64(4242, 16 * n)
    pick = lambda k, lo, hi: lo + int(u[k] % np.uint64(hi - lo + 1))
    alphas, betas = [1.0, 1.5, -0.75], [0.0, 1.0, -0.5]
    cases = []
    for c in range(n):
        b = 16 * c
        kind = "f32" if u[b] % np.uint64(2) == 0 else "f16"
        lo, hi = [(900, 2000), (2000, 3500), (3900, 4400)][int(u[b + 12] % np.uint64(3))]
        M, N = pick(b + 1, lo, hi), pick(b + 2, lo, hi)
        if u[b + 13] % np.uint64(2) == 0:   # MN-contiguous operands can take the direct-to-LDS kernels
            M, N = M - M % 8, N - N % 8
        cases.append(dict(kind=kind, M=M, N=N, K=pick(b + 3, 64, 700),
                          pa=pick(b + 4, 0, 3), pb=pick(b + 5, 0, 3), pc=pick(b + 6, 0, 9),
                          tA=bool(u[b + 7] % np.uint64(2)), tB=bool(u[b + 8] % np.uint64(2)),
                          alpha=alphas[int(u[b + 9] % np.uint64(3))], beta=betas[int(u[b + 10] % np.uint64(3))],
                          ints=bool(u[b + 11] % np.uint64(3) == 0), seed=700 + c))
    return cases


@pytest.mark.parametrize("case", _dma_sweep_cases(24), ids=lambda c: f"{c['kind']}-{c['M']}x{c['N']}x{c['K']}"
                         f"-t{int(c['tA'])}{int(c['tB'])}")
def test_random_sweep_direct_to_lds(case):
    # leading dimensions rounded up to whole 16-byte chunks plus 0-3 chunks of padding
    c = case
    q = 4 if c["kind"] == "f32" else 8
    a_cols, b_cols = (c["M"] if c["tA"] else c["K"]), (c["K"] if c["tB"] else c["N"])
    lda = a_cols + (-a_cols) % q + q * c["pa"]
    ldb = b_cols + (-b_cols) % q + q * c["pb"]
    run_and_check(c["kind"], c["M"], c["N"], c["K"], c["alpha"], c["beta"],
                  kind_vals="int4" if c["ints"] else "pm1", exact=c["ints"], lda=lda, ldb=ldb,
                  ldc=c["N"] + c["pc"], transA=c["tA"], transB=c["tB"], seed=c["seed"], sample=64,
                  c_nan=(c["beta"] == 0.0))


# ------------------------------------------------------------------ 64x128 HGEMM tile
def test_hgemm_64x128_tiles():
    # grids that 128x128 tiles would fill to a quarter (or to half with K >= 4096)
    # run 64x128 tiles when A is stored M x K; A stored K x M keeps 128x128
    for tB in (False, True):
        run_and_check("f16", 512, 4096, 4096, 1.0, 0.0, transB=tB, sample=64, c_nan=True)
        run_and_check("f16", 1000, 1000, 2000, 1.5, -0.5, transB=tB)              # ragged edges and K tail
        run_and_check("f16", 1002, 998, 600, 1.0, 1.0, transB=tB)                 # chunks straddling N (NN)
        run_and_check("f16", 256, 2048, 1024, 1.0, 0.0, kind_vals="int4", exact=True, transB=tB)
        run_and_check("bf16", 640, 768, 512, 1.5, -0.5, transB=tB)
    run_and_check("f16", 1000, 1000, 2000, 1.5, -0.5, transA=True)                # stays on 128x128
    run_and_check("f16", 512, 4096, 4096, 1.0, 0.0, transA=True, transB=True, sample=64)
    batched_check(256, 512, 1024, 4, 1.0, 1.0, sample=32)
    batched_check(100, 300, 520, 3, 1.5, -0.5, pad=2, transB=True)


@pytest.mark.parametrize("M,N,K", [(1000, 1000, 2000), (512, 4096, 4096)])
def test_hgemm_64x128_matches_128x128_bits(M, N, K):
    # A stored M x K takes the 64x128 tile on these grids; the same A stored K x M
    # (transA) can only take the 128x128 tile.  Both tiles give each lane the same
    # eight k per MFMA in the same order, so C must agree bit for bit.
    note(f"64x128 vs 128x128 bits M={M} N={N} K={K}")
    p = si.gemm_problem(M, N, K, in_dtype=np.float16, seed=71, with_c=True)
    dA, dB = to_dev(p["A"]), to_dev(p["B"])
    dAt = to_dev(np.ascontiguousarray(p["A"].reshape(M, K).T))
    c0 = to_dev(p["C"])
    c1 = c0.clone()
    dg.gemm_f16_f32acc(M, N, K, 1.5, dA, K, dB, N, -0.5, c0, N)
    dg.gemm_f16_f32acc_ex(1, 0, M, N, K, 1.5, dAt, M, dB, N, -0.5, c1, N)
    torch.cuda.synchronize()
    assert torch.equal(c0, c1)


# ------------------------------------------------------------------ beta epilogue on whole tiles
# Whole tiles of the direct-to-LDS HGEMM kernels read C one block row ahead of
# their stores (the first block row before the last slice); tiles at the edge of
# C keep the plain order.  Whole-tile shapes of each tile and storage
# combination, beta != 0, int4 values: bit-exact against the oracle, so a block
# row read into the wrong buffer or combined with the wrong accumulators fails.
@pytest.mark.parametrize("tA,tB", [(False, False)] + OPS)
@pytest.mark.parametrize("M,N,K,tile", [
    (4096, 4096, 128, "256x256"),
    (4096, 4096, 192, "256x256, odd slice count"),
    (1536, 1536, 4096, "128x128"),
    (1024, 1024, 2048, "64x128 (128x128 when A is stored K x M)"),
])
def test_hgemm_beta_read_ahead(M, N, K, tile, tA, tB):
    note(f"beta read-ahead, {tile} tile")
    run_and_check("f16", M, N, K, 1.0, -0.5, kind_vals="int4", exact=True, sample=48, transA=tA, transB=tB,
                  seed=83)
    run_and_check("f16", M, N, K, 1.5, 2.0, sample=32, transA=tA, transB=tB, seed=84)
    # C rows only 4-byte aligned (odd ldc): the row-segment reads and writes take any dword offset
    run_and_check("f16", M, N, K, -0.75, 1.0, ldc=N + 1, kind_vals="int4", exact=True, sample=24, transA=tA,
                  transB=tB, seed=86)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("tA,tB", [(False, False)] + OPS)
@pytest.mark.parametrize("K", [128, 192])
def test_hgemm_256_beta_every_element(K, tA, tB, fmt):
    # Every element of a 4096x4096 C on 256x256 tiles (the block row that goes
    # through the freed LDS slot included), int4 values: the beta != 0 result
    # must equal the beta == 0 result plus beta*C exactly (all values are small
    # integers and halves, so no step rounds).  The beta == 0 path is checked
    # against the oracle by the other tests.
    M = N = 4096
    note(f"256x256 beta every element {fmt} K={K} transA={int(tA)} transB={int(tB)}")
    p = si.gemm_problem(M, N, K, in_dtype=IN_DTYPE[fmt], kind="int4", seed=89, transA=tA, transB=tB)
    dA, dB, c0 = to_dev(p["A"]), to_dev(p["B"]), to_dev(p["C"])
    d = torch.empty_like(c0)
    c = c0.clone()
    lda, ldb = p["lda"], p["ldb"]
    fn = dg.gemm_bf16_f32acc_ex if fmt == "bf16" else dg.gemm_f16_f32acc_ex
    fn(int(tA), int(tB), M, N, K, 1.0, dA, lda, dB, ldb, 0.0, d, N)
    fn(int(tA), int(tB), M, N, K, 1.0, dA, lda, dB, ldb, -0.5, c, N)
    torch.cuda.synchronize()
    assert torch.equal(c, d + (-0.5) * c0)


@pytest.mark.parametrize("nb,M,N,K", [(16, 1024, 1024, 1024), (12, 1024, 1024, 320)])
def test_batched_256_beta_every_element(nb, M, N, K):
    # The same on batched 256x256 tiles (member strides with a gap of 64
    # elements), every element of every member, and the gaps left untouched
    note(f"batched 256x256 beta every element batch={nb} M={M} N={N} K={K}")
    probs = [si.gemm_problem(M, N, K, in_dtype=np.float16, kind="int4", seed=91, batch=b) for b in range(nb)]
    sA, sB, sC = M * K + 64, K * N + 64, M * N + 64
    A = np.zeros(sA * nb, np.float16)
    B = np.zeros(sB * nb, np.float16)
    C = np.zeros(sC * nb, np.float32)
    for b, q in enumerate(probs):
        A[b * sA: b * sA + M * K] = q["A"]
        B[b * sB: b * sB + K * N] = q["B"]
        C[b * sC: b * sC + M * N] = q["C"]
    dA, dB, c0 = to_dev(A), to_dev(B), to_dev(C)
    d = torch.zeros_like(c0)
    c = c0.clone()
    dg.gemm_batched_f16_f32acc(M, N, K, 1.0, dA, K, sA, dB, N, sB, 0.0, d, N, sC, nb)
    dg.gemm_batched_f16_f32acc(M, N, K, 1.0, dA, K, sA, dB, N, sB, 2.0, c, N, sC, nb)
    torch.cuda.synchronize()
    for b in range(nb):
        got = c[b * sC: b * sC + M * N]
        want = d[b * sC: b * sC + M * N] + 2.0 * c0[b * sC: b * sC + M * N]
        assert torch.equal(got, want), f"member {b}"
        # the gaps between members are never written
        assert torch.equal(c[b * sC + M * N: (b + 1) * sC], c0[b * sC + M * N: (b + 1) * sC])


def test_batched_beta_read_ahead_bits():
    # the batched configuration's 256x256 tiles, beta = 1, int4 values
    batched_check(1024, 1024, 1024, 16, 1.0, 1.0, kind_vals="int4", exact=True, sample=16, seed=85)
    # whole 128x128 tiles of transposed members, beta != 0, bf16 and fp16
    batched_check(256, 384, 512, 3, 1.5, -0.5, transA=True, transB=True, seed=87)
    batched_check(256, 384, 512, 3, 1.0, 2.0, kind_vals="int4", exact=True, transA=True, seed=88, fmt="bf16")


# ------------------------------------------------------------------ bfloat16 inputs
# The bf16 entry points run the HGEMM kernels with the bf16 matrix-core op, so
# these cases cover each of those kernels once more with bfloat16 inputs.

@pytest.mark.parametrize("n", [2048, 4096])
def test_bf16_square(n):
    # 128x128 (2048) and 256x256 (4096) direct-to-LDS tiles
    run_and_check("bf16", n, n, n, 1.0, 0.0, c_nan=True, seed=n)
    run_and_check("bf16", n, n, n, 1.0, 0.0, kind_vals="int4", exact=True, seed=7)


@pytest.mark.parametrize("tA,tB", [(False, False)] + OPS)
def test_bf16_ragged_and_transposed(tA, tB):
    run_and_check("bf16", 1000, 1200, 776, 1.5, -0.5, transA=tA, transB=tB)              # masked tiles
    run_and_check("bf16", 2050, 2046, 320, 1.5, -0.5, transA=tA, transB=tB, sample=64)   # straddling chunks
    run_and_check("bf16", 300, 260, 700, 1.0, 1.0, transA=tA, transB=tB)
    run_and_check("bf16", 256, 256, 128, 1.0, 0.0, kind_vals="int4", exact=True, transA=tA, transB=tB)


def test_bf16_register_kernels():
    # odd leading dimensions, a 2-byte aligned pointer and K below the ring: the
    # register-staged kernel
    run_and_check("bf16", 500, 400, 300, 1.5, -0.5, lda=301, ldb=401)
    run_and_check("bf16", 384, 256, 260, 1.0, 0.0, offset=1)
    run_and_check("bf16", 1024, 1024, 64, 1.0, 0.0, kind_vals="int4", exact=True)


def test_bf16_batched():
    batched_check(1024, 1024, 1024, 16, 1.0, 1.0, fmt="bf16")
    batched_check(33, 65, 17, 4, 1.0, 0.0, kind_vals="int4", exact=True, pad=1, fmt="bf16")
    batched_check(200, 136, 72, 3, 1.0, 1.0, pad=3, share_a=True, transA=True, transB=True, fmt="bf16")


def test_bf16_and_fp16_agree_on_values_both_hold():
    # entries that are exact in both formats (small integers, and multiples of
    # 2**-7 below 1) give the same products, and the two paths add them in the
    # same order: identical bits
    M, N, K = 2048, 2048, 1024
    for kind_vals, seed in (("int4", 21), ("pm1", 22)):
        ph = si.gemm_problem(M, N, K, in_dtype=np.float16, kind=kind_vals, seed=seed)
        if kind_vals == "pm1":   # round to multiples of 2**-7, exact in both formats
            ph["A"] = (np.round(ph["A"].astype(np.float32) * 128) / 128).astype(np.float16)
            ph["B"] = (np.round(ph["B"].astype(np.float32) * 128) / 128).astype(np.float16)
        a_bf = si.to_bf16_bits(ph["A"].astype(np.float32))
        b_bf = si.to_bf16_bits(ph["B"].astype(np.float32))
        out = []
        for fn, a, b in ((dg.gemm_f16_f32acc, ph["A"], ph["B"]), (dg.gemm_bf16_f32acc, a_bf, b_bf)):
            dC = torch.zeros(M * N, dtype=torch.float32, device="cuda")
            fn(M, N, K, 1.0, to_dev(a), K, to_dev(b), N, 0.0, dC, N)
            torch.cuda.synchronize()
            out.append(dC.cpu())
        note(f"bf16 vs fp16 {kind_vals}: equal={torch.equal(out[0], out[1])}")
        assert torch.equal(out[0], out[1])


# ------------------------------------------------------------------ K split over workgroups (HGEMM)
# Shapes whose 128x128 tiles fill at most a quarter of the CUs and whose K holds
# at least 64 slices split each tile's K range over several workgroups; the last
# to finish adds the partial tiles in split order.  The split each shape gets is
# checked on the host by tests/test_plan16.py.

@pytest.mark.parametrize("M,N,K,tA,tB", [
    (512, 512, 8192, False, False),      # 8 splits of 16 slices
    (1000, 1000, 5000, False, False),    # 2 splits, ragged tiles and a K tail
    (300, 200, 6000, False, False),      # 5 splits of 18 or 19 slices, K tail
    (500, 1002, 8192, False, False),     # B chunks straddling N: the slices stop before row K-1
    (512, 768, 5000, True, True),
    (768, 768, 4096, True, False),
    (768, 768, 4096, False, True),
])
def test_split_k_parity(M, N, K, tA, tB):
    run_and_check("f16", M, N, K, 1.5, -0.5, transA=tA, transB=tB, seed=101)
    run_and_check("f16", M, N, K, 1.0, 1.0, kind_vals="int4", exact=True, transA=tA, transB=tB, seed=102)
    run_and_check("f16", M, N, K, 1.0, 0.0, c_nan=True, transA=tA, transB=tB, seed=103)


def test_split_k_bf16_and_batched():
    run_and_check("bf16", 512, 512, 8192, 1.5, -0.5, seed=104)
    run_and_check("bf16", 1000, 1000, 5000, 1.0, 1.0, kind_vals="int4", exact=True, seed=105)
    batched_check(256, 384, 4096, 3, 1.5, -0.5)                               # 18 tiles x 4 splits
    batched_check(256, 384, 4096, 3, 1.0, 1.0, kind_vals="int4", exact=True, seed=106)


def test_split_k_deterministic():
    # the partial tiles are added in split order whichever workgroup finishes last
    M, N, K = 512, 512, 8192
    p = si.gemm_problem(M, N, K, in_dtype=np.float16, seed=107)
    dA, dB = to_dev(p["A"]), to_dev(p["B"])
    outs = []
    for _ in range(4):
        dC = to_dev(p["C"])
        dg.gemm_f16_f32acc(M, N, K, 1.5, dA, K, dB, N, -0.5, dC, N)
        torch.cuda.synchronize()
        outs.append(dC)
    assert all(torch.equal(outs[0], o) for o in outs[1:])


def test_split_k_concurrent_streams():
    # each stream has its own scratch: split calls on four streams at once
    note("split-K HGEMM on four streams at once")
    shapes = [(512, 512, 8192), (1024, 1024, 8192), (300, 200, 6000), (256, 256, 8192)]
    probs = [si.gemm_problem(M, N, K, in_dtype=np.float16, seed=110 + i) for i, (M, N, K) in enumerate(shapes)]
    devs = [(to_dev(p["A"]), to_dev(p["B"]), to_dev(p["C"])) for p in probs]
    streams = [torch.cuda.Stream() for _ in shapes]
    torch.cuda.synchronize()
    for _ in range(3):   # repeated: the counters must be left zero by every call
        for (M, N, K), p, (dA, dB, dC), s in zip(shapes, probs, devs, streams):
            dC.copy_(to_dev(p["C"]))
            torch.cuda.synchronize()
        for (M, N, K), p, (dA, dB, dC), s in zip(shapes, probs, devs, streams):
            dg.gemm_f16_f32acc(M, N, K, 1.5, dA, K, dB, N, -0.5, dC, N, s)
        torch.cuda.synchronize()
        for (M, N, K), p, (_, _, dC) in zip(shapes, probs, devs):
            ref, bound = oracle.gemm_ref(M, N, K, 1.5, p["A"], K, p["B"], N, -0.5, p["C"], N)
            assert oracle.normalized_error(rows_of(dC, M, N, N), ref, bound) <= TOL


def test_split_k_graph_capture():
    # A stream that has already run a split call holds its scratch, so a graph
    # captured on it records the split kernel and replays it bit for bit.  A
    # stream that has not cannot allocate during capture: its graph records the
    # unsplit kernel, whose result is equally within tolerance.
    M, N, K = 512, 512, 8192
    p = si.gemm_problem(M, N, K, in_dtype=np.float16, seed=120)
    dA, dB, c0 = to_dev(p["A"]), to_dev(p["B"]), to_dev(p["C"])
    ref, bound = oracle.gemm_ref(M, N, K, 1.5, p["A"], K, p["B"], N, -0.5, p["C"], N)
    warm = torch.cuda.Stream()
    eager = c0.clone()
    with torch.cuda.stream(warm):
        dg.gemm_f16_f32acc(M, N, K, 1.5, dA, K, dB, N, -0.5, eager, N, warm)
    torch.cuda.synchronize()
    for stream, same_bits in ((warm, True), (torch.cuda.Stream(), False)):
        out = c0.clone()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            dg.gemm_f16_f32acc(M, N, K, 1.5, dA, K, dB, N, -0.5, out, N, stream)
        first = None
        for replay in range(3):
            out.copy_(c0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert oracle.normalized_error(rows_of(out, M, N, N), ref, bound) <= TOL
            if same_bits:
                assert torch.equal(out, eager), f"replay {replay} differs from the eager split result"
            first = out.clone() if first is None else first
            assert torch.equal(out, first)
            _ = (dA.float() * 2).sum().item()   # unrelated eager work between replays
        del g


# ------------------------------------------------------------------ graph capture
def test_graph_capture_replays_match_eager():
    # the library enqueues plain kernel launches on the caller's stream (no memset,
    # no allocation), so a captured sequence replays exactly; every replay is
    # checked, with eager work and synchronisation between replays
    note("graph capture of gemm_f32 + gemm_f16_f32acc + batched, 4 replays")
    ps = si.gemm_problem(1001, 777, 513, seed=71)
    ph = si.gemm_problem(512, 384, 320, in_dtype=np.float16, seed=72)
    sA, sB, hA, hB = to_dev(ps["A"]), to_dev(ps["B"]), to_dev(ph["A"]), to_dev(ph["B"])
    bA = to_dev(si.draw(73, 3 * 64 * 96).astype(np.float16))
    bB = to_dev(si.draw(74, 3 * 96 * 80).astype(np.float16))
    sC0, hC0 = to_dev(ps["C"]), to_dev(ph["C"])
    bC0 = to_dev(si.draw(75, 3 * 64 * 80))

    def work(sC, hC, bC, stream=None):
        dg.gemm_f32(1001, 777, 513, 1.5, sA, 513, sB, 777, -0.5, sC, 777, stream)
        dg.gemm_f16_f32acc(512, 384, 320, 1.0, hA, 320, hB, 384, 1.0, hC, 384, stream)
        dg.gemm_batched_f16_f32acc(64, 80, 96, 1.0, bA, 96, 64 * 96, bB, 80, 96 * 80, 0.5, bC, 80, 64 * 80, 3,
                                   stream)

    eager = [sC0.clone(), hC0.clone(), bC0.clone()]
    work(*eager)
    torch.cuda.synchronize()

    outs = [torch.empty_like(sC0), torch.empty_like(hC0), torch.empty_like(bC0)]
    for o, c0 in zip(outs, (sC0, hC0, bC0)):
        o.copy_(c0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        work(*outs, stream=side)
    for replay in range(4):
        for o, c0 in zip(outs, (sC0, hC0, bC0)):
            o.copy_(c0)        # beta != 0: every replay starts from the same C
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {replay} differs from the eager result"
        _ = (sA * 2).sum().item()   # unrelated eager work between replays
