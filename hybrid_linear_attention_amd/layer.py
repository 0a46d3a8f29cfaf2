"""The GDN layer block as a sequence of libgdn launches.

Order of operations (tutorial page "Qwen3.8-27B: from model structure to the
vLLM inference dataflow", section 01, per-layer operator table, GDN layer):

    U = RMSNorm(X)                                     gdn_rmsnorm
    [Q0|K0|V0|Z|b|a] = U W_in                          gdn_gemm_bf16
    conv + L2 norm -> gated delta rule -> RMSNorm(o) * SiLU(Z):
        prefill requests                               gdn_prefill_fused
        decode requests                                gdn_decode_fused
    Y = X + y W_o                                      gdn_gemm_bf16 (residual epilogue)

With fused=False the core runs as its separate entry points instead
(gdn_conv1d_update, gdn_prefill_varlen, gdn_decode_step, gdn_gated_norm), which
also leaves o in a buffer.

W_in stacks the in-projection's q | k | v | z columns and then b | a (the
dispatch page "How the 64 layers of Qwen3.8-27B are dispatched in vLLM", step 7,
stacks in_proj_qkv/z into in_proj_qkvz and in_proj_b/a into in_proj_ba); both are
stored output-major ([N, hidden]) so the GEMM reads both operands along K.  The
batch is mixed: prefill requests first, then one-token decode requests.  This
module only allocates buffers with torch and calls the C entry points; every
step of the arithmetic runs in libgdn's kernels.
"""
from dataclasses import dataclass

import torch

from . import gdn


@dataclass
class LayerWeights:
    W_in: torch.Tensor      # [2*Hk*dk + 2*Hv*dv + 2*Hv, hidden] bf16, rows q|k|v|z|b|a
    W_out: torch.Tensor     # [hidden, Hv*dv] bf16 (output-major)
    conv_w: torch.Tensor    # [Cqkv, taps]
    gamma_in: torch.Tensor  # [hidden]
    gamma_out: torch.Tensor  # [dv]


def stack_weights(dims, W_qkvz, W_ba, W_o, conv_w, gamma_in, gamma_out, device="cuda"):
    """Device weights from input-major host matrices (W_qkvz [hidden, q|k|v|z],
    W_ba [hidden, b|a], W_o [Hv*dv, hidden]): a one-time weight-loading step."""
    W_in = torch.cat([W_qkvz, W_ba], dim=1).t().contiguous()
    return LayerWeights(W_in=W_in.to(device), W_out=W_o.t().contiguous().to(device),
                        conv_w=conv_w.contiguous().to(device),
                        gamma_in=gamma_in.contiguous().to(device),
                        gamma_out=gamma_out.contiguous().to(device))


class GdnLayer:
    """Buffers for one mixed batch shape and the launch sequence over them."""

    def __init__(self, dims, weights: LayerWeights, num_tokens, num_prefill_reqs,
                 num_prefill_tokens, num_decode, norm_eps=1e-6, l2_eps=1e-6, device="cuda",
                 fused=True):
        self.dims = dims
        self.w = weights
        self.T = int(num_tokens)
        self.n_pf = int(num_prefill_reqs)
        self.T_pf = int(num_prefill_tokens)
        self.n_dec = int(num_decode)
        if self.T != self.T_pf + self.n_dec:
            raise ValueError("tokens must be the prefill tokens followed by one per decode request")
        self.norm_eps, self.l2_eps = norm_eps, l2_eps
        self.fused = fused
        Hk, Hv, dk, dv = dims.num_k_heads, dims.num_v_heads, dims.head_dim_k, dims.head_dim_v
        self.cq = 2 * Hk * dk + Hv * dv
        self.cz = Hv * dv
        hidden = weights.W_in.shape[1]
        n_in = weights.W_in.shape[0]
        if n_in != self.cq + self.cz + 2 * Hv:
            raise ValueError("W_in rows must be q|k|v|z|b|a")
        T = self.T
        self.U = torch.empty((T, hidden), dtype=torch.bfloat16, device=device)
        self.P = torch.empty((T, n_in), dtype=torch.bfloat16, device=device)
        self.y = torch.empty((T, Hv * dv), dtype=torch.bfloat16, device=device)
        self.Y = torch.empty((T, hidden), dtype=torch.bfloat16, device=device)
        if fused:
            nbytes = gdn.gdn_prefill_fused_workspace_bytes(dims, self.T_pf, self.n_pf) if self.n_pf else 0
        else:
            self.q = torch.empty((T, Hk, dk), device=device)
            self.k = torch.empty((T, Hk, dk), device=device)
            self.v = torch.empty((T, Hv, dv), device=device)
            self.o = torch.empty((T, Hv, dv), device=device)
            nbytes = gdn.gdn_prefill_workspace_bytes(dims, self.T_pf, self.n_pf) if self.n_pf else 0
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes else None
        # the projections' split-tail workspace (one buffer: the launches run in order)
        gb = max(gdn.gdn_gemm_bf16_workspace_bytes(T, n_in, hidden),
                 gdn.gdn_gemm_bf16_workspace_bytes(T, hidden, Hv * dv))
        self.gemm_ws = torch.empty(gb, dtype=torch.uint8, device=device) if gb else None

    # views of the projection output
    def x_qkv(self):
        return self.P[:, :self.cq]

    def z(self):
        return self.P[:, self.cq:self.cq + self.cz]

    def b(self):
        Hv = self.dims.num_v_heads
        return self.P[:, self.cq + self.cz:self.cq + self.cz + Hv]

    def a(self):
        Hv = self.dims.num_v_heads
        return self.P[:, self.cq + self.cz + Hv:]

    def stages(self, X, conv_pool, state_pool, qsl, slot_ids, has_initial, stream=None):
        """The launches in order, as (name, callable) pairs."""
        d, w = self.dims, self.w
        T_pf, n_pf = self.T_pf, self.n_pf
        a, b = self.a(), self.b()
        out = [
            ("rmsnorm", lambda: gdn.gdn_rmsnorm(X, w.gamma_in, self.U, self.norm_eps, stream)),
            ("in_proj", lambda: gdn.gdn_gemm_bf16(self.U, w.W_in, self.P, stream=stream,
                                                 workspace=self.gemm_ws)),
        ]
        if self.fused:
            x, z = self.x_qkv(), self.z()
            if n_pf:
                out.append(("prefill", lambda: gdn.gdn_prefill_fused(
                    d, x[:T_pf], z[:T_pf], a[:T_pf], b[:T_pf], w.conv_w, w.gamma_out, conv_pool,
                    state_pool, qsl[:n_pf + 1], slot_ids[:n_pf], has_initial[:n_pf], self.y[:T_pf],
                    self.ws, l2_eps=self.l2_eps, norm_eps=self.norm_eps, stream=stream)))
            if self.n_dec:
                out.append(("decode", lambda: gdn.gdn_decode_fused(
                    d, x[T_pf:], z[T_pf:], a[T_pf:], b[T_pf:], w.conv_w, w.gamma_out, conv_pool,
                    state_pool, slot_ids[n_pf:], self.y[T_pf:], has_initial=has_initial[n_pf:],
                    l2_eps=self.l2_eps, norm_eps=self.norm_eps, stream=stream)))
            out.append(("out_proj", lambda: gdn.gdn_gemm_bf16(self.y, w.W_out, self.Y, residual=X,
                                                              stream=stream, workspace=self.gemm_ws)))
            return out
        out += [
            ("conv1d", lambda: gdn.gdn_conv1d_update(
                d, self.x_qkv(), w.conv_w, conv_pool, qsl, slot_ids, has_initial, self.q, self.k,
                self.v, self.l2_eps, stream)),
        ]
        if n_pf:
            out.append(("prefill", lambda: gdn.gdn_prefill_varlen(
                d, self.q[:T_pf], self.k[:T_pf], self.v[:T_pf], a[:T_pf], b[:T_pf], state_pool,
                qsl[:n_pf + 1], slot_ids[:n_pf], has_initial[:n_pf], self.o[:T_pf], self.ws,
                stream)))
        if self.n_dec:
            out.append(("decode", lambda: gdn.gdn_decode_step(
                d, self.q[T_pf:], self.k[T_pf:], self.v[T_pf:], a[T_pf:], b[T_pf:], state_pool,
                slot_ids[n_pf:], self.o[T_pf:], stream)))
        out += [
            ("gated_norm", lambda: gdn.gdn_gated_norm(d, self.o, self.z(), w.gamma_out, self.y,
                                                      self.norm_eps, stream)),
            ("out_proj", lambda: gdn.gdn_gemm_bf16(self.y, w.W_out, self.Y, residual=X,
                                                   stream=stream, workspace=self.gemm_ws)),
        ]
        return out

    def forward(self, X, conv_pool, state_pool, qsl, slot_ids, has_initial, stream=None):
        """Run the layer on X [T, hidden] bf16; conv_pool and state_pool are updated in
        place; returns Y [T, hidden] bf16 (a buffer owned by this object)."""
        for _, fn in self.stages(X, conv_pool, state_pool, qsl, slot_ids, has_initial, stream):
            fn()
        return self.Y
