"""Property test of the C-ABI's argument checks against the rules that
include/gemm.h states, on random sizes, leading dimensions (up to 2^63-1)
and fake pointers that often overlap.  Every case the rules accept with
work to do is skipped, so no call reaches a launch: CPU only."""
from hypothesis import HealthCheck, assume, given, settings
from hypothesis import strategies as st

from dense_gemm_row_amd import gemm

LIM = 2 ** 31 - 1
OK, INVALID, ALIAS = gemm.GEMM_OK, gemm.GEMM_ERR_INVALID_ARG, gemm.GEMM_ERR_ALIAS
IN_BYTES = {gemm.DTYPE_F32: 4, gemm.DTYPE_F16: 2, gemm.DTYPE_BF16: 2, gemm.DTYPE_F8: 1, gemm.DTYPE_E5M2: 1}
OUT_BYTES = {gemm.DTYPE_F32: 4, gemm.DTYPE_F16: 2, gemm.DTYPE_BF16: 2, gemm.DTYPE_F8: 2, gemm.DTYPE_E5M2: 2}


def rules(dt, M, N, K, A, lda, B, ldb, C, ldc, at, bt):
    """The status the header's rules give, in their order."""
    if min(M, N, K) < 0 or max(M, N, K) > LIM:
        return INVALID
    if lda < max(1, M if at else K) or ldb < max(1, K if bt else N) or ldc < max(1, N):
        return INVALID
    if (M > 0 and K > 0 and not A) or (K > 0 and N > 0 and not B) or (M > 0 and N > 0 and not C):
        return INVALID
    if -(-M // 64) * -(-N // 64) > LIM:
        return INVALID

    def span(rows, cols, ld, es):
        return 0 if rows <= 0 or cols <= 0 else ((rows - 1) * ld + cols) * es

    es = IN_BYTES[dt]
    sa = span(K, M, lda, es) if at else span(M, K, lda, es)
    sb = span(N, K, ldb, es) if bt else span(K, N, ldb, es)
    sc = span(M, N, ldc, OUT_BYTES[dt])
    if max(sa, sb, sc) >= 2 ** 63:
        return INVALID

    def overlap(p, n, q, m):
        return bool(p and q and n and m and p < q + m and q < p + n)

    return ALIAS if overlap(C, sc, A, sa) or overlap(C, sc, B, sb) else OK


dims = st.one_of(st.integers(-2, 300), st.sampled_from([0, 1, LIM, LIM + 1, 2 ** 40]))
lds = st.one_of(st.integers(-2, 400), st.sampled_from([LIM, 2 ** 40, 2 ** 61, 2 ** 62, 2 ** 63 - 1]))
bases = [2 ** 32, 2 ** 32 + 64, 2 ** 32 + 4096, 2 ** 33, 3 * 2 ** 32]
ptrs = st.one_of(st.just(0), st.sampled_from(bases), st.tuples(st.sampled_from(bases), st.integers(-512, 512))
                 .map(lambda t: t[0] + t[1]))


@settings(max_examples=4000, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.filter_too_much, HealthCheck.too_slow])
@given(dt=st.sampled_from(sorted(IN_BYTES)), M=dims, N=dims, K=dims, A=ptrs, lda=lds, B=ptrs, ldb=lds,
       C=ptrs, ldc=lds, at=st.booleans(), bt=st.booleans())
def test_checks_follow_the_stated_rules(dt, M, N, K, A, lda, B, ldb, C, ldc, at, bt):
    want = rules(dt, M, N, K, A, lda, B, ldb, C, ldc, at, bt)
    assume(not (want == OK and M > 0 and N > 0))   # would launch
    fn = gemm.entry(dt, "_trans")
    got = fn(M, N, K, A, lda, B, ldb, C, ldc, None, None, int(at), int(bt))
    assert got == want, (got, want, gemm.gemm_last_error())
    assert (gemm.gemm_last_error() == "") == (got == OK)


def test_workspace_size_overflow_is_refused():
    """S x M x N x 4 beyond int64 (M = N = 2^21, K = 2^31 - 1, 2^20 chunks
    of 2048) is refused, not wrapped to a small or zero size."""
    for dt in sorted(IN_BYTES):
        assert gemm.gemm_splitk_workspace_bytes(dt, 2 ** 21, 2 ** 21, LIM, 2 ** 20) == -1
        assert gemm.gemm_splitk_workspace_bytes(dt, 2 ** 21, 2 ** 21, LIM, 2 ** 19) == -1  # 2^63
        # 2^18 chunks of 8192 k: 2^18 * 2^42 * 4 = 2^62 bytes fits.
        assert gemm.gemm_splitk_workspace_bytes(dt, 2 ** 21, 2 ** 21, LIM, 2 ** 18) == 2 ** 62


def test_split_chunks_are_whole_slices_of_every_variant():
    """Chunks are multiples of 64 k, or of 128 k for the 8-bit types (whose
    LDS-direct slices are up to 128 k): K = 8192 with 12 requested splits
    gives chunks of 704 (12 planes) for 32- and 16-bit types and of 768
    (11 planes) for E4M3 and E5M2."""
    M, N = 512, 256
    for dt in sorted(IN_BYTES):
        planes = 11 if dt in (gemm.DTYPE_F8, gemm.DTYPE_E5M2) else 12
        assert gemm.gemm_splitk_workspace_bytes(dt, M, N, 8192, 12) == planes * M * N * 4, dt
