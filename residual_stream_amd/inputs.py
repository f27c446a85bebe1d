"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the method: it only draws random arrays and
rounds them to the storage dtype.  Both the fp64 oracle and the HIP path consume
exactly the arrays returned here.

Recipe (one ``numpy.random.default_rng(seed)``, draws in this order; the
activations are drawn directly in float32, phi and bias in float64):

* x[T,N,D] ~ N(0,1)        — the N-stream residual state
* y[T,D] ~ N(0,1)          — the sublayer output
* phi[N·D, N²+2N] ~ N(0, 1/(N·D))   (variance 1/(N·D), i.e. unit-variance raw logits)
* bias[N²+2N] ~ N(0, 0.1)  (variance 0.1; ``bias_std`` overrides the standard
  deviation, e.g. 3 for logits large enough that one Sinkhorn round is far
  from converged)
* dh[T,D] ~ N(0,1), dx_next[T,N,D] ~ N(0,1)   — upstream gradients (optional)

Inputs of the write-back calls that are not drawn above come from
``make_coefficients`` (a separate generator, so that the write-back can be
checked without running hc_pre): H_post[T,N] ~ U(0, 2) and H_res[T,N,N] ~
U(0, 1), in the ranges the maps take, with no normalisation; and from
``make_norm_weights``: learnable norm weights ~ U(0.5, 1.5), y_weight[D] and
out_weight[N·D].

x, y, dh and dx_next are rounded to the I/O dtype (fp32, or bf16 with
round-to-nearest-even); phi and bias are always fp32.  Every array is returned
as float32 numpy holding exactly the stored values, so upcasting to float64 is
exact.
"""

from __future__ import annotations

import dataclasses

import numpy as np

IO_F32 = "f32"
IO_BF16 = "bf16"


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32.

    NaN stays NaN; overflow goes to ±inf as IEEE rounding prescribes.
    """
    f = np.array(a, dtype=np.float32, copy=True, order="C")
    flat = f.reshape(-1)
    u_all = flat.view(np.uint32)
    step = 1 << 20
    for i in range(0, flat.size, step):
        u = u_all[i:i + step]
        nan = np.isnan(flat[i:i + step])
        # For every non-NaN word u + 0x7FFF + 1 stays below 2^32: uint32 arithmetic is exact.
        lsb = (u >> 16) & np.uint32(1)
        u += np.uint32(0x7FFF)
        u += lsb
        u &= np.uint32(0xFFFF0000)
        if nan.any():
            flat[i:i + step][nan] = np.float32("nan")
    return f


def to_io(a: np.ndarray, io: str) -> np.ndarray:
    """Cast to float32, then to the storage dtype's values (fp32 or bf16-RNE)."""
    f = np.asarray(a, dtype=np.float32)
    if io == IO_F32:
        return np.ascontiguousarray(f)
    if io == IO_BF16:
        return round_to_bf16(f)
    raise ValueError(f"unknown io dtype {io!r}")


@dataclasses.dataclass
class MhcInputs:
    T: int
    N: int
    D: int
    io: str
    x: np.ndarray
    y: np.ndarray
    phi: np.ndarray
    bias: np.ndarray
    alphas: tuple
    eps: float
    iters: int
    dh: np.ndarray | None = None
    dx_next: np.ndarray | None = None

    @property
    def K(self) -> int:
        return self.N * self.D

    @property
    def C(self) -> int:
        return self.N * self.N + 2 * self.N


def make_inputs(T: int, N: int, D: int, io: str = IO_F32, seed: int = 0,
                alpha: float | tuple = 0.01, eps: float = 1e-6, iters: int = 20,
                grads: bool = False, bias_std: float | None = None) -> MhcInputs:
    """Draw one seeded problem instance (see the module docstring for the recipe)."""
    rng = np.random.default_rng(seed)
    K = N * D
    C = N * N + 2 * N
    x = to_io(rng.standard_normal((T, N, D), dtype=np.float32), io)
    y = to_io(rng.standard_normal((T, D), dtype=np.float32), io)
    phi = (rng.standard_normal((K, C)) * (1.0 / np.sqrt(K))).astype(np.float32)
    bstd = np.sqrt(0.1) if bias_std is None else float(bias_std)
    bias = (rng.standard_normal(C) * bstd).astype(np.float32)
    dh = dxn = None
    if grads:
        dh = to_io(rng.standard_normal((T, D), dtype=np.float32), io)
        dxn = to_io(rng.standard_normal((T, N, D), dtype=np.float32), io)
    alphas = tuple(float(a) for a in alpha) if isinstance(alpha, (tuple, list)) else (float(alpha),) * 3
    return MhcInputs(T=T, N=N, D=D, io=io, x=x, y=y, phi=phi, bias=bias, alphas=alphas,
                     eps=float(eps), iters=int(iters), dh=dh, dx_next=dxn)


def make_coefficients(T: int, N: int, seed: int = 0):
    """Seeded H_post[T,N] ~ U(0,2) and H_res[T,N,N] ~ U(0,1), float32."""
    rng = np.random.default_rng(seed)
    H_post = rng.uniform(0.0, 2.0, (T, N)).astype(np.float32)
    H_res = rng.uniform(0.0, 1.0, (T, N, N)).astype(np.float32)
    return H_post, H_res


def make_norm_weights(N: int, D: int, seed: int = 0):
    """Seeded learnable norm weights ~ U(0.5, 1.5): y_weight[D], out_weight[N·D], float32."""
    rng = np.random.default_rng(seed)
    return (rng.uniform(0.5, 1.5, D).astype(np.float32),
            rng.uniform(0.5, 1.5, N * D).astype(np.float32))


# Named workloads: shapes of the pages' training activations (mHC with 4
# streams at the Pro hidden size 5120 and the Flash hidden size 2560, and the
# B=1, S=4096 long-sequence shape of the activation-memory discussion).
WORKLOADS = {
    "tiny_f32": dict(T=64, N=4, D=256, io=IO_F32),
    "pro_s1024_f32": dict(T=1024, N=4, D=5120, io=IO_F32),
    "flash_s2048_f32": dict(T=2048, N=4, D=2560, io=IO_F32),
    "pro_s4096_bf16": dict(T=4096, N=4, D=5120, io=IO_BF16),
}
