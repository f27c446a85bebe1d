"""torch.autograd integration of the mHC operator pair, with the recompute policy.

One residual block of a model that uses mHC (openPangu 2.0 analysis, §5.3 "mHC"
formula block) reads the N-stream state x through hc_pre, runs its sublayer F on
h, and writes back through hc_post:

    h, H_pre, H_post, H_res = hc_pre(x; φ, b, α)
    y = F(h)
    x_next = H_res · x + H_post ⊗ y

`MHCBlock` wraps that with the four C-ABI calls as autograd functions.  What the
backward keeps follows the intra-layer recompute paragraph of the Ascend mHC
Triton article: only the hc_pre input x and the sublayer output y (plus the
80 bytes per token of H_post / H_res); `mhc_pre_bwd` recomputes the norm, the
logits and the Sinkhorn rounds from x.  With ``recompute=True`` the sublayer is
checkpointed too, so not even h or the sublayer's own activations are kept.

The two backward nodes produce the state gradient together: the hc_post node
computes dy and the coefficient gradients only (`mhc_post_bwd` without dx) and
hands dx_next and H_res to the hc_pre node of the same block, whose
`mhc_pre_bwd_mix` forms dx = H_resᵀ·dx_next plus its own part in one pass, so
dx is written once instead of being written, read back and written again.
(With the stabilised write-back the hc_post node writes its dx and hands that
over; `mhc_pre_bwd` adds to it in place.)  The hc_post node therefore returns
no gradient for x; the hc_pre node returns the total.

openPangu's stabilised variant (openPangu 2.0 analysis, §5.4) is available
through three switches: ``sandwich_norm`` (an RMSNorm with a learnable weight
on y before H_post writes it back), ``post_norm`` (an RMSNorm with a learnable
weight over each token's flattened N·D state after the write-back: the
block-level post-norm, which a model enables on the first block and every
fifth) and ``pre_norm_weight`` (a learnable weight on the hc_pre RMSNorm).
The first two run in ``mhc_post_stable`` and its backward.  The hc_pre weight
w only scales the normalised state before the projection, so it is folded
into the projection's rows, φ' = diag(w)·φ, a [N·D, N²+2N] parameter product
computed once per step; the per-token work stays in the kernels.

`MHCStack` chains blocks so that each block's write-back and the next block's
read run as one fused call (`mhc_post_pre`, the pages' inference fusion),
with the same results as the blocks run one after another.

Every per-token step runs in the library's kernels; this module only wires
them into autograd.  It needs a GPU and the built library, like the binding.
"""

from __future__ import annotations

import torch
from torch.utils.checkpoint import checkpoint

from . import mhc


class _DxHandoff:
    """Carries hc_post's share of the state gradient to the hc_pre backward of
    the same block: either dx itself (stabilised write-back), or dx_next and
    H_res, from which mhc_pre_bwd_mix forms it (plain write-back: dx then
    crosses HBM once)."""

    __slots__ = ("dx", "mix")

    def __init__(self):
        self.dx = None
        self.mix = None


class _Pre(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, phi, bias, alpha, iters, eps, handoff):
        # alpha is a GPU tensor the kernels read on the device: no host round trip
        h, Hp, Hq, Hr = mhc.mhc_pre(x, phi, bias, iters=iters, eps=eps, alphas=alpha)
        ctx.save_for_backward(x, phi, bias, alpha)
        ctx.cfg = (iters, eps, alpha.requires_grad)
        ctx.handoff = handoff
        ctx.mark_non_differentiable(Hp)  # used only inside the collapse
        return h, Hp, Hq, Hr

    @staticmethod
    def backward(ctx, dh, _dHp, dHq, dHr):
        x, phi, bias, alphas = ctx.saved_tensors
        iters, eps, want_dalpha = ctx.cfg
        T, N, D = x.shape
        dx, mix = ctx.handoff.dx, ctx.handoff.mix
        ctx.handoff.dx = ctx.handoff.mix = None
        if dx is None and mix is None:  # hc_post's output took no gradient
            dx = torch.zeros_like(x)
        if dh is None:
            dh = torch.zeros((T, D), dtype=x.dtype, device=x.device)
        if dHq is None:
            dHq = torch.zeros((T, N), dtype=torch.float32, device=x.device)
        if dHr is None:
            dHr = torch.zeros((T, N, N), dtype=torch.float32, device=x.device)
        if mix is not None:
            dx_next, H_res = mix
            dx, dphi, dbias, dalpha = mhc.mhc_pre_bwd_mix(
                dh.contiguous(), x, phi, bias, dHq.contiguous(), dHr.contiguous(), dx_next, H_res,
                iters=iters, eps=eps, alphas=alphas, want_dalpha=want_dalpha)
        else:
            dx, dphi, dbias, dalpha = mhc.mhc_pre_bwd(
                dh.contiguous(), x, phi, bias, dHq.contiguous(), dHr.contiguous(), dx,
                iters=iters, eps=eps, alphas=alphas, want_dalpha=want_dalpha)
        return dx, dphi, dbias, (dalpha if want_dalpha else None), None, None, None


class _Post(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, y, H_post, H_res, y_weight, out_weight, eps, handoff):
        if y_weight is None and out_weight is None:
            x_next = mhc.mhc_post(x, y, H_post, H_res)
        else:
            x_next = mhc.mhc_post_stable(x, y, H_post, H_res, y_weight=y_weight,
                                         out_weight=out_weight, eps=eps)
        ctx.save_for_backward(x, y, H_post, H_res, y_weight, out_weight)
        ctx.eps = eps
        ctx.handoff = handoff
        return x_next

    @staticmethod
    def backward(ctx, dx_next):
        x, y, H_post, H_res, y_weight, out_weight = ctx.saved_tensors
        T, N, D = x.shape
        if y_weight is None and out_weight is None and mhc.mix_fuses(N, D, mhc._io_of(x)):
            # dx is formed by the hc_pre backward of this block from dx_next
            dx_next = dx_next.contiguous()
            _, dy, dHq, dHr = mhc.mhc_post_bwd(dx_next, x, y, H_post, H_res, want_dx=False)
            ctx.handoff.mix = (dx_next, H_res)
            dyw = dow = None
        elif y_weight is None and out_weight is None:
            dx, dy, dHq, dHr = mhc.mhc_post_bwd(dx_next.contiguous(), x, y, H_post, H_res)
            ctx.handoff.dx = dx  # the hc_pre backward of this block adds to it
            dyw = dow = None
        else:
            dx, dy, dHq, dHr, dyw, dow = mhc.mhc_post_stable_bwd(
                dx_next.contiguous(), x, y, H_post, H_res, y_weight=y_weight,
                out_weight=out_weight, eps=ctx.eps)
            ctx.handoff.dx = dx  # the hc_pre backward of this block adds to it
        return None, dy, dHq, dHr, dyw, dow, None, None


class MHCBlock(torch.nn.Module):
    """One mHC residual block around `sublayer` (a module mapping h[T, D] to
    y[T, D] in the I/O dtype).

    Parameters: φ[N·D, N²+2N] and b[N²+2N] (fp32, on the GPU) and the three gate
    scalars α = (α_pre, α_post, α_res), also a GPU tensor that the kernels
    read on the device (so neither the forward nor the backward waits for the
    host, and a captured graph follows the parameter's updates); with the
    stabilisation switches also y_weight[D], out_weight[N·D] and
    pre_weight[N·D] (fp32, initialised to one).  x is [T, N, D] or
    [B, S, N, D], fp32 or bf16, on the GPU.
    """

    def __init__(self, sublayer: torch.nn.Module, n_streams: int, hidden: int, *,
                 iters: int = 20, eps: float = 1e-6, alpha=(0.01, 0.01, 0.01),
                 train_alpha: bool = False, recompute: bool = False, sandwich_norm: bool = False,
                 post_norm: bool = False, pre_norm_weight: bool = False, device="cuda"):
        super().__init__()
        N, D = n_streams, hidden
        C = N * N + 2 * N
        self.sublayer = sublayer
        self.N, self.D, self.iters, self.eps, self.recompute = N, D, iters, eps, recompute
        self.phi = torch.nn.Parameter(torch.randn(N * D, C, device=device) / (N * D) ** 0.5)
        self.bias = torch.nn.Parameter(torch.zeros(C, device=device))
        self.alpha = torch.nn.Parameter(torch.tensor(alpha, dtype=torch.float32, device=device),
                                        requires_grad=train_alpha)
        ones = lambda n: torch.nn.Parameter(torch.ones(n, device=device))  # noqa: E731
        self.y_weight = ones(D) if sandwich_norm else None
        self.out_weight = ones(N * D) if post_norm else None
        self.pre_weight = ones(N * D) if pre_norm_weight else None

    def _phi(self):
        if self.pre_weight is None:
            return self.phi
        return (self.pre_weight[:, None] * self.phi).contiguous()

    def _pre_sub(self, x, handoff):
        h, _Hp, Hq, Hr = _Pre.apply(x, self._phi(), self.bias, self.alpha, self.iters, self.eps,
                                    handoff)
        return self.sublayer(h), Hq, Hr

    def forward(self, x):
        shape = x.shape
        if x.dim() == 4:
            x = x.reshape(-1, shape[-2], shape[-1])
        if x.shape[1:] != (self.N, self.D):
            raise ValueError(f"expected [..., {self.N}, {self.D}] state, got {tuple(shape)}")
        x = x.contiguous()
        handoff = _DxHandoff()
        if self.recompute and torch.is_grad_enabled():
            y, Hq, Hr = checkpoint(self._pre_sub, x, handoff, use_reentrant=False)
        else:
            y, Hq, Hr = self._pre_sub(x, handoff)
        x_next = _Post.apply(x, y.contiguous(), Hq, Hr, self.y_weight, self.out_weight, self.eps,
                             handoff)
        return x_next.reshape(shape)


class _PostPre(torch.autograd.Function):
    """hc_post of block l fused with hc_pre of block l + 1 (`mhc_post_pre`).

    Backward, in the order the separate blocks run it: hc_pre's backward of
    block l + 1 forms the gradient of x_{l+1} from the dx_next and H_res the
    next boundary handed over, then hc_post's backward of block l runs without
    dx and hands its own dx_next and H_res to the previous boundary (or block
    0's hc_pre) through ``handoff_out``.
    """

    @staticmethod
    def forward(ctx, x, y, H_post_in, H_res_in, phi, bias, alpha, iters, eps, handoff_in, handoff_out):
        x_next, h, Hp, Hq, Hr = mhc.mhc_post_pre(x, y, H_post_in, H_res_in, phi, bias, iters=iters,
                                                 eps=eps, alphas=alpha)
        ctx.save_for_backward(x, y, H_post_in, H_res_in, x_next, phi, bias, alpha)
        ctx.cfg = (iters, eps, alpha.requires_grad)
        ctx.handoff_in, ctx.handoff_out = handoff_in, handoff_out
        ctx.mark_non_differentiable(Hp)
        return x_next, h, Hp, Hq, Hr

    @staticmethod
    def backward(ctx, dxn, dh, _dHp, dHq, dHr):
        x, y, H_post_in, H_res_in, x_next, phi, bias, alphas = ctx.saved_tensors
        iters, eps, want_dalpha = ctx.cfg
        T, N, D = x.shape
        if dh is None:
            dh = torch.zeros((T, D), dtype=x.dtype, device=x.device)
        if dHq is None:
            dHq = torch.zeros((T, N), dtype=torch.float32, device=x.device)
        if dHr is None:
            dHr = torch.zeros((T, N, N), dtype=torch.float32, device=x.device)
        kw = dict(iters=iters, eps=eps, alphas=alphas, want_dalpha=want_dalpha)
        # hc_pre backward of block l + 1: the next boundary (or the last
        # block's hc_post) handed over its dx_next and H_res, from which the
        # state gradient of x_{l+1} is formed here
        mix, dx_in = ctx.handoff_in.mix, ctx.handoff_in.dx
        ctx.handoff_in.mix = ctx.handoff_in.dx = None
        if mix is not None:
            dx_next, dphi, dbias, dalpha = mhc.mhc_pre_bwd_mix(
                dh.contiguous(), x_next, phi, bias, dHq.contiguous(), dHr.contiguous(), mix[0], mix[1], **kw)
        else:
            dx_next, dphi, dbias, dalpha = mhc.mhc_pre_bwd(
                dh.contiguous(), x_next, phi, bias, dHq.contiguous(), dHr.contiguous(),
                dx_in if dx_in is not None else torch.zeros_like(x_next), **kw)
        if dxn is not None:  # x_{l+1} also used outside the stack
            dx_next = dx_next + dxn
        # hc_post backward of block l, its dx left to the previous boundary
        if mhc.mix_fuses(N, D, mhc._io_of(x)):
            _, dy, dHq_in, dHr_in = mhc.mhc_post_bwd(dx_next, x, y, H_post_in, H_res_in, want_dx=False)
            ctx.handoff_out.mix = (dx_next, H_res_in)
        else:
            dx, dy, dHq_in, dHr_in = mhc.mhc_post_bwd(dx_next, x, y, H_post_in, H_res_in)
            ctx.handoff_out.dx = dx
        return None, dy, dHq_in, dHr_in, dphi, dbias, (dalpha if want_dalpha else None), None, None, None, None


class MHCStack(torch.nn.Module):
    """Consecutive `MHCBlock`s run with each block's write-back fused to the
    next block's read (openPangu 2.0 analysis §11.3; `mhc_post_pre`): the state
    between two blocks is written once and not read back.

    Uses the blocks' own parameters and sublayers, so a stack and the same
    blocks applied one after another compute the same values (bit for bit:
    the fused forward equals hc_post followed by hc_pre, and the backward runs
    the same kernels in the same order).  For the plain write-back only: a
    block with a sandwich or post-norm, or with recompute, is rejected.
    """

    def __init__(self, blocks):
        super().__init__()
        self.blocks = torch.nn.ModuleList(blocks)
        if not len(self.blocks):
            raise ValueError("MHCStack needs at least one block")
        b0 = self.blocks[0]
        for b in self.blocks:
            if b.y_weight is not None or b.out_weight is not None:
                raise ValueError("MHCStack fuses the plain write-back only (no sandwich or post-norm)")
            if b.recompute:
                raise ValueError("MHCStack does not checkpoint sublayers")
            if (b.N, b.D, b.iters, b.eps) != (b0.N, b0.D, b0.iters, b0.eps):
                raise ValueError("all blocks of a stack need the same N, D, rounds and eps")

    def forward(self, x):
        blocks = self.blocks
        b0 = blocks[0]
        shape = x.shape
        if x.dim() == 4:
            x = x.reshape(-1, shape[-2], shape[-1])
        if x.shape[1:] != (b0.N, b0.D):
            raise ValueError(f"expected [..., {b0.N}, {b0.D}] state, got {tuple(shape)}")
        x = x.contiguous()
        handoff = _DxHandoff()
        h, _Hp, Hq, Hr = _Pre.apply(x, b0._phi(), b0.bias, b0.alpha, b0.iters, b0.eps, handoff)
        for i, b in enumerate(blocks):
            y = b.sublayer(h).contiguous()
            if i + 1 < len(blocks):
                nb = blocks[i + 1]
                nxt = _DxHandoff()
                x, h, _Hp, Hq, Hr = _PostPre.apply(x, y, Hq, Hr, nb._phi(), nb.bias, nb.alpha, nb.iters,
                                                   nb.eps, nxt, handoff)
                handoff = nxt
            else:
                x = _Post.apply(x, y, Hq, Hr, None, None, b.eps, handoff)
        return x.reshape(shape)
