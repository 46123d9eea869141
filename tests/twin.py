"""An independent pure-Python statement of C = ReLU(A.B) for tiny inputs.

It uses numpy's own float16 <-> float32 conversions and float32 scalar
arithmetic, and shares nothing with the C oracle, so agreement between the
two pins the oracle's conversions and loop. Test-only.
"""
import numpy as np


def gemm_relu_twin(A, B):
    """fp16 A (M, K), B (K, N) -> uint16 bits of ReLU(A.B), fp32 accumulation in ascending k."""
    M, K = A.shape
    N = B.shape[1]
    C = np.zeros((M, N), np.uint16)
    for i in range(M):
        for j in range(N):
            acc = np.float32(0.0)
            for k in range(K):
                acc = np.float32(acc + np.float32(A[i, k]) * np.float32(B[k, j]))
            r = acc if acc > np.float32(0.0) else np.float32(0.0)
            C[i, j] = np.float16(r).view(np.uint16)
    return C


def relu_rne16_of_int(S):
    """Exact integer sums -> fp16 bits of ReLU, rounded to nearest even by numpy."""
    S = np.asarray(S, dtype=np.int64)
    with np.errstate(over="ignore"):
        return np.where(S > 0, S, 0).astype(np.float16).view(np.uint16)
