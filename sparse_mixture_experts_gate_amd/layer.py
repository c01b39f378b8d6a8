"""A DeepSeekMoE layer object over the C ABI: it owns the device weights (and
their FP8 copies), allocates outputs and the workspace with torch, and calls
the library. No arithmetic of the layer happens here."""
from __future__ import annotations

import torch

from . import _lib as L
from .workloads import Workload

_ACT = {"f32": L.MOE_DT_F32, "bf16": L.MOE_DT_BF16}
_W = {"f32": L.MOE_DT_F32, "bf16": L.MOE_DT_BF16, "fp8": L.MOE_DT_FP8_E4M3}


def make_desc(wl: Workload, T: int, near_tie_eps: float = 1e-6) -> L.MoeLayerDesc:
    return L.MoeLayerDesc(T=T, d=wl.d, n_experts=wl.E, top_k=wl.K, n_groups=wl.G,
                          topk_groups=wl.M, group_topn=wl.topn, inter=wl.I, shared_inter=wl.Is,
                          act_dtype=_ACT[wl.act], w_dtype=_W[wl.w], near_tie_eps=near_tie_eps,
                          out_dtype=_ACT[wl.out_dtype])


def quantize_fp8_blocks(w: torch.Tensor):
    """E4M3 codes and 128x128 block scales of w [n, rows, cols] (library)."""
    shp = w.shape if w.dim() == 3 else (1, *w.shape)
    q = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    s = torch.empty(shp[0], shp[1] // 128, shp[2] // 128, dtype=torch.float32, device=w.device)
    L.moe_quantize_fp8_blocks(w.contiguous(), q, s)
    if w.dim() == 2:
        s = s[0]
    return q, s


class MoELayer:
    def __init__(self, wl: Workload, params: dict):
        self.wl = wl
        self.w_router = params["w_router"]
        self.bias = params["bias"].clone()
        dev = self.w_router.device
        if wl.w == "fp8":
            self.w13, self.w13_scale = quantize_fp8_blocks(params["w13"])
            self.w2, self.w2_scale = quantize_fp8_blocks(params["w2"])
            self.ws13, self.ws13_scale = (quantize_fp8_blocks(params["ws13"]) if wl.Is else (None, None))
            self.ws2, self.ws2_scale = (quantize_fp8_blocks(params["ws2"]) if wl.Is else (None, None))
        else:
            self.w13, self.w2 = params["w13"], params["w2"]
            self.ws13, self.ws2 = params["ws13"], params["ws2"]
            self.w13_scale = self.w2_scale = self.ws13_scale = self.ws2_scale = None
        self.weights = L.make_weights(self.w13, self.w2, self.ws13, self.ws2, self.w13_scale,
                                      self.w2_scale, self.ws13_scale, self.ws2_scale)
        self._ws = torch.empty(0, dtype=torch.uint8, device=dev)
        self.device = dev

    def desc(self, T: int) -> L.MoeLayerDesc:
        return make_desc(self.wl, T)

    def workspace(self, T: int) -> torch.Tensor:
        need = L.moe_workspace_size(self.desc(T))
        if self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._ws

    def alloc_outputs(self, T: int) -> dict:
        wl, dev = self.wl, self.device
        ydt = torch.float32 if wl.out_dtype == "f32" else torch.bfloat16
        return {"y": torch.empty(T, wl.d, dtype=ydt, device=dev),
                "topk_idx": torch.empty(T, wl.K, dtype=torch.int32, device=dev),
                "topk_gate": torch.empty(T, wl.K, dtype=torch.float32, device=dev),
                "counts": torch.empty(wl.E, dtype=torch.int32, device=dev),
                "near_tie": torch.empty(1, dtype=torch.int32, device=dev),
                "logits": torch.empty(T, wl.E, dtype=torch.float32, device=dev)}

    def forward(self, x: torch.Tensor, out: dict | None = None, with_logits: bool = True,
                stream=None) -> dict:
        T = x.shape[0]
        out = self.alloc_outputs(T) if out is None else out
        ws = self.workspace(T)
        L.deepseek_moe_forward(self.desc(T), x, self.w_router, self.bias, self.weights, out["y"],
                               out["topk_idx"], out["topk_gate"], out["counts"], out["near_tie"],
                               out["logits"] if with_logits else None, ws, stream)
        return out

    def bias_update(self, counts: torch.Tensor, T: int, gamma: float | None = None, stream=None):
        L.moe_bias_update(self.desc(T), counts, self.wl.gamma if gamma is None else gamma,
                          self.bias, stream)

    # ---- training (bf16 activations and weights) ----------------------------
    def alloc_saved(self, T: int) -> dict:
        wl, dev = self.wl, self.device
        TK = T * wl.K
        ldh = max(wl.I, wl.Is)
        hrows = TK + (T if wl.Is else 0)
        i32, f32, bf = torch.int32, torch.float32, torch.bfloat16
        return {"logits": torch.empty(T, wl.E, dtype=f32, device=dev),
                "topk_idx": torch.empty(T, wl.K, dtype=i32, device=dev),
                "topk_gate": torch.empty(T, wl.K, dtype=f32, device=dev),
                "counts": torch.empty(wl.E, dtype=i32, device=dev),
                "offsets": torch.empty(wl.E + 1, dtype=i32, device=dev),
                "perm": torch.empty(TK, dtype=i32, device=dev),
                "inv": torch.empty(T, wl.K, dtype=i32, device=dev),
                "h": torch.empty(hrows, ldh, dtype=bf, device=dev),
                "gu": torch.empty(hrows, 2 * ldh, dtype=bf, device=dev),
                "y_perm": torch.empty(TK, wl.d, dtype=bf, device=dev)}

    def forward_train(self, x: torch.Tensor, saved: dict | None = None, stream=None) -> tuple:
        """y [T, d] and the tensors the backward needs (moe_forward_train)."""
        T = x.shape[0]
        saved = self.alloc_saved(T) if saved is None else saved
        ydt = torch.float32 if self.wl.out_dtype == "f32" else torch.bfloat16
        y = torch.empty(T, self.wl.d, dtype=ydt, device=self.device)
        near_tie = torch.empty(1, dtype=torch.int32, device=self.device)
        L.moe_forward_train(self.desc(T), x, self.w_router, self.bias, self.weights, y,
                            L.make_saved(**saved), near_tie, self.workspace(T), stream)
        return y, saved

    def alloc_grads(self) -> dict:
        wl, dev, f32 = self.wl, self.device, torch.float32
        return {"dw13": torch.empty(wl.E, 2 * wl.I, wl.d, dtype=f32, device=dev),
                "dw2": torch.empty(wl.E, wl.d, wl.I, dtype=f32, device=dev),
                "dws13": torch.empty(2 * wl.Is, wl.d, dtype=f32, device=dev) if wl.Is else None,
                "dws2": torch.empty(wl.d, wl.Is, dtype=f32, device=dev) if wl.Is else None,
                "dw_router": torch.empty(wl.E, wl.d, dtype=f32, device=dev)}

    def backward_workspace(self, T: int) -> torch.Tensor:
        need = L.moe_backward_workspace_size(self.desc(T))
        if getattr(self, "_bws", None) is None or self._bws.numel() < need:
            self._bws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._bws

    def weights_transposed(self) -> L.MoeWeights:
        """Transposed copies of the FP8 weights (codes and block scales) that
        the FP8 backward reads, made once by the library."""
        if getattr(self, "_wt", None) is None:
            wl, dev, u8, f32 = self.wl, self.device, torch.uint8, torch.float32

            def tr(q, sc):
                lead = q.shape[:-2]
                qt = torch.empty(*lead, q.shape[-1], q.shape[-2], dtype=u8, device=dev)
                st = torch.empty(*lead, sc.shape[-1], sc.shape[-2], dtype=f32, device=dev)
                L.moe_transpose_fp8_blocks(q, sc, qt, st)
                return qt, st

            w13t, s13t = tr(self.w13, self.w13_scale)
            w2t, s2t = tr(self.w2, self.w2_scale)
            ws13t = ws2t = ss13t = ss2t = None
            if wl.Is:
                ws13t, ss13t = tr(self.ws13, self.ws13_scale)
                ws2t, ss2t = tr(self.ws2, self.ws2_scale)
            self._wt_tensors = (w13t, w2t, ws13t, ws2t, s13t, s2t, ss13t, ss2t)
            self._wt = L.make_weights(*self._wt_tensors)
        return self._wt

    def backward(self, x: torch.Tensor, dy: torch.Tensor, saved: dict, grads: dict | None = None,
                 stream=None) -> tuple:
        """dx [T, d] bf16 and the fp32 weight gradients (moe_backward, or
        moe_backward_fp8 for FP8 weights)."""
        T = x.shape[0]
        grads = self.alloc_grads() if grads is None else grads
        dx = torch.empty(T, self.wl.d, dtype=torch.bfloat16, device=self.device)
        if self.wl.w == "fp8":
            L.moe_backward_fp8(self.desc(T), x, self.w_router, self.weights,
                               self.weights_transposed(), L.make_saved(**saved), dy, dx,
                               L.make_grads(**grads), self.backward_workspace(T), stream)
        else:
            L.moe_backward(self.desc(T), x, self.w_router, self.weights,
                           L.make_saved(**saved), dy, dx, L.make_grads(**grads),
                           self.backward_workspace(T), stream)
        return dx, grads

    def seq_balance_loss(self, x: torch.Tensor, saved: dict, seq_len: int, alpha: float,
                         want_dlogits: bool = False, stream=None) -> dict:
        """The sequence-level balance loss of the forward that wrote ``saved``
        (its logits and selection) over sequences of ``seq_len`` tokens, and
        its gradients (moe_seq_balance_loss): loss [T / seq_len], dx [T, d],
        dw_router [E, d] (fp32), dlogits [T, E] when asked for."""
        T, dev, f32 = x.shape[0], self.device, torch.float32
        need = L.moe_seq_balance_workspace_size(self.desc(T), seq_len)
        if getattr(self, "_sws", None) is None or self._sws.numel() < need:
            self._sws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        out = {"loss": torch.empty(T // seq_len, dtype=f32, device=dev),
               "dx": torch.empty(T, self.wl.d, dtype=f32, device=dev),
               "dw_router": torch.empty(self.wl.E, self.wl.d, dtype=f32, device=dev),
               "dlogits": (torch.empty(T, self.wl.E, dtype=f32, device=dev)
                           if want_dlogits else None)}
        L.moe_seq_balance_loss(self.desc(T), seq_len, alpha, x, self.w_router, saved["logits"],
                               saved["topk_idx"], out["loss"], out["dlogits"], out["dx"],
                               out["dw_router"], self._sws, stream)
        return out
