"""Thin Python binding of libmtp.so (include/mtp.h): ctypes structures and
argument marshalling from torch tensors.  Every computation runs in the HIP
library; this module only passes device pointers, sizes and the stream.

Loading fails loudly when the library is missing: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, List, Optional, Sequence

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmtp.so")

MTP_F32, MTP_BF16 = 0, 1
MTP_REDUCE_FIXED, MTP_REDUCE_VALID_MEAN = 0, 1
STATUS = {0: "MTP_OK", -1: "MTP_ERR_NULL", -2: "MTP_ERR_SHAPE", -3: "MTP_ERR_DEPTH",
          -4: "MTP_ERR_DTYPE", -5: "MTP_ERR_WORKSPACE", -6: "MTP_ERR_ARG", -7: "MTP_ERR_HIP",
          -8: "MTP_ERR_UNSUPPORTED", -9: "MTP_ERR_TOO_LARGE"}
EXPORTS = ("mtp_chain_forward", "mtp_head_ce_fwd_bwd", "mtp_verify", "mtp_propose_step", "mtp_round_commit",
           "mtp_chain_workspace_size", "mtp_ce_workspace_size", "mtp_verify_workspace_size",
           "mtp_propose_workspace_size", "mtp_strerror", "mtp_abi_version", "mtp_profile_stage",
           "mtp_profile_count", "mtp_verify_noalloc", "mtp_chain_backward",
           "mtp_chain_backward_workspace_size", "mtp_profile_all", "mtp_horizon_heads",
           "mtp_horizon_heads_workspace_size", "mtp_chain_saved_bytes")
BLOCK_FIELDS = ("g_a", "g_f", "Wqkv", "Wo", "Wgate", "Wup", "Wdown")
STAGES = ("ROWS", "DUAL_NORM", "EH_PROJ", "NORM_A", "QKV", "ATTN", "O_PROJ", "NORM_F", "GATE_UP",
          "DOWN", "OUT_NORM", "CE_FWD", "CE_REDUCE", "CE_GRAD", "CE_DX", "CE_NORM_BWD", "CE_DW",
          "VERIFY", "BWD_RECOMPUTE", "BWD_MLP", "BWD_ATTN_PROJ", "BWD_ATTN", "BWD_QKV", "BWD_EH")
GRAD_FIELDS = ("g_h", "g_e", "g_a", "g_f", "M", "Wqkv", "Wo", "Wgate", "Wup", "Wdown")

vp = C.c_void_p
fp = C.POINTER(C.c_float)


class DepthWeights(C.Structure):
    _fields_ = [("g_h", vp), ("g_e", vp), ("g_attn", vp), ("g_ffn", vp), ("M", vp), ("Wqkv", vp),
                ("Wo", vp), ("Wgate", vp), ("Wup", vp), ("Wdown", vp)]


class ChainArgs(C.Structure):
    _fields_ = [("B", C.c_int), ("T", C.c_int), ("d", C.c_int), ("n_heads", C.c_int),
                ("head_dim", C.c_int), ("ffn", C.c_int), ("V", C.c_int), ("D", C.c_int),
                ("dtype", C.c_int), ("eps", C.c_float), ("rope_theta", C.c_float),
                ("tokens", vp), ("segment_ids", vp), ("h0", vp), ("embed", vp),
                ("w", C.POINTER(DepthWeights)), ("h_out", C.POINTER(vp)),
                ("state_mask", vp), ("loss_mask", vp), ("labels", vp), ("counts", vp),
                ("device_error", vp), ("workspace", vp), ("workspace_bytes", C.c_size_t),
                ("saved", vp), ("saved_bytes", C.c_size_t)]


ABI_VERSION = 9     # the struct layouts below mirror include/mtp.h at this version


class DepthGrads(C.Structure):
    _fields_ = [("g_h", vp), ("g_e", vp), ("g_attn", vp), ("g_ffn", vp), ("M", vp), ("Wqkv", vp),
                ("Wo", vp), ("Wgate", vp), ("Wup", vp), ("Wdown", vp)]


class ChainBwdArgs(C.Structure):
    _fields_ = [("B", C.c_int), ("T", C.c_int), ("d", C.c_int), ("n_heads", C.c_int),
                ("head_dim", C.c_int), ("ffn", C.c_int), ("V", C.c_int), ("D", C.c_int),
                ("dtype", C.c_int), ("eps", C.c_float), ("rope_theta", C.c_float),
                ("tokens", vp), ("segment_ids", vp), ("h0", vp), ("embed", vp),
                ("w", C.POINTER(DepthWeights)), ("h", C.POINTER(vp)), ("dh", C.POINTER(vp)),
                ("dh0", vp), ("dE", vp), ("dw", C.POINTER(DepthGrads)), ("accumulate", C.c_int),
                ("device_error", vp), ("workspace", vp), ("workspace_bytes", C.c_size_t),
                ("saved", vp), ("saved_bytes", C.c_size_t)]


class BlockWeights(C.Structure):
    _fields_ = [("g_attn", vp), ("g_ffn", vp), ("Wqkv", vp), ("Wo", vp), ("Wgate", vp), ("Wup", vp), ("Wdown", vp)]


class BlockGrads(C.Structure):
    _fields_ = [("g_attn", vp), ("g_ffn", vp), ("Wqkv", vp), ("Wo", vp), ("Wgate", vp), ("Wup", vp), ("Wdown", vp)]


class HorizonArgs(C.Structure):
    _fields_ = [("B", C.c_int), ("T", C.c_int), ("d", C.c_int), ("n_heads", C.c_int), ("head_dim", C.c_int),
                ("ffn", C.c_int), ("V", C.c_int), ("K", C.c_int), ("dtype", C.c_int), ("eps", C.c_float),
                ("rope_theta", C.c_float), ("lambda_", C.c_float), ("tokens", vp), ("segment_ids", vp),
                ("h", vp), ("w", C.POINTER(BlockWeights)), ("W_out", vp), ("g_out", vp), ("loss", vp),
                ("counts", vp), ("loss_total", vp), ("dh", vp), ("dW_out", vp), ("dg_out", vp),
                ("dw", C.POINTER(BlockGrads)), ("accumulate", C.c_int), ("device_error", vp),
                ("workspace", vp), ("workspace_bytes", C.c_size_t)]


C_STRUCT_NAMES = {"DepthGrads": "mtp_depth_grads", "ChainBwdArgs": "mtp_chain_bwd_args",
                  "BlockWeights": "mtp_block_weights", "BlockGrads": "mtp_block_grads",
                  "HorizonArgs": "mtp_horizon_args"}


class CeArgs(C.Structure):
    _fields_ = [("B", C.c_int), ("T", C.c_int), ("d", C.c_int), ("V", C.c_int), ("D", C.c_int),
                ("dtype", C.c_int), ("eps", C.c_float), ("lambda_", C.c_float), ("reduce", C.c_int),
                ("denom", C.c_double), ("h", C.POINTER(vp)), ("labels", vp), ("W_out", vp),
                ("g_out", vp), ("loss_sum", vp), ("counts", vp), ("loss", vp), ("loss_mtp", vp),
                ("lse", vp), ("dh", C.POINTER(vp)), ("dW_out", vp), ("dg_out", vp),
                ("accumulate", C.c_int), ("device_error", vp), ("logit_slab_bytes", C.c_size_t),
                ("dh_accumulate", C.c_int), ("pred", vp), ("correct", vp), ("accuracy", vp),
                ("workspace", vp), ("workspace_bytes", C.c_size_t)]


class VerifyArgs(C.Structure):
    _fields_ = [("R", C.c_int), ("gamma", C.c_int), ("V", C.c_int), ("temperature", C.c_float),
                ("logits_dtype", C.c_int), ("target_logits", vp), ("draft_logits", vp),
                ("draft_tokens", vp), ("u_accept", vp), ("u_sample", vp), ("accepted_len", vp),
                ("next_token", vp), ("status", vp), ("margin", vp), ("workspace", vp),
                ("workspace_bytes", C.c_size_t)]


class ProposeArgs(C.Structure):
    _fields_ = [("R", C.c_int), ("L_max", C.c_int), ("d", C.c_int), ("n_heads", C.c_int),
                ("head_dim", C.c_int), ("ffn", C.c_int), ("V", C.c_int), ("dtype", C.c_int),
                ("eps", C.c_float), ("rope_theta", C.c_float), ("temperature", C.c_float),
                ("w", C.POINTER(DepthWeights)), ("embed", vp), ("W_out", vp), ("g_out", vp),
                ("h_prev", vp), ("tokens", vp), ("positions", vp), ("u_sample", vp), ("kv_cache", vp),
                ("h_out", vp), ("logits", vp), ("draft_token", vp), ("status", vp), ("margin", vp),
                ("workspace", vp), ("workspace_bytes", C.c_size_t)]


class RoundArgs(C.Structure):
    _fields_ = [("R", C.c_int), ("gamma", C.c_int), ("eos", C.c_int), ("draft_tokens", vp),
                ("accepted_len", vp), ("next_token", vp), ("status", vp), ("remaining", vp),
                ("new_tokens", vp), ("n_new", vp), ("rows_to_keep", vp), ("pending_frontier", vp),
                ("stopped", vp)]


_lib = None


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load libmtp.so (once).  Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"libmtp.so not found at {path}: build it with "
                               "`python -m deepseek_sequential_mtp_amd.build`")
        lib = C.CDLL(path)
        lib.mtp_chain_forward.argtypes = [C.POINTER(ChainArgs), vp]
        lib.mtp_chain_backward.argtypes = [C.POINTER(ChainBwdArgs), vp]
        lib.mtp_horizon_heads.argtypes = [C.POINTER(HorizonArgs), vp]
        lib.mtp_horizon_heads_workspace_size.argtypes = [C.POINTER(HorizonArgs)]
        lib.mtp_horizon_heads_workspace_size.restype = C.c_size_t
        lib.mtp_chain_backward_workspace_size.argtypes = [C.POINTER(ChainBwdArgs)]
        lib.mtp_chain_backward_workspace_size.restype = C.c_size_t
        lib.mtp_head_ce_fwd_bwd.argtypes = [C.POINTER(CeArgs), vp]
        lib.mtp_verify.argtypes = [C.POINTER(VerifyArgs), vp]
        lib.mtp_verify_noalloc.argtypes = [C.POINTER(VerifyArgs), vp]
        lib.mtp_propose_step.argtypes = [C.POINTER(ProposeArgs), vp]
        lib.mtp_round_commit.argtypes = [C.POINTER(RoundArgs), vp]
        lib.mtp_propose_workspace_size.argtypes = [C.POINTER(ProposeArgs)]
        lib.mtp_propose_workspace_size.restype = C.c_size_t
        lib.mtp_chain_workspace_size.argtypes = [C.POINTER(ChainArgs)]
        lib.mtp_chain_workspace_size.restype = C.c_size_t
        lib.mtp_chain_saved_bytes.argtypes = [C.POINTER(ChainArgs)]
        lib.mtp_chain_saved_bytes.restype = C.c_size_t
        lib.mtp_ce_workspace_size.argtypes = [C.POINTER(CeArgs)]
        lib.mtp_ce_workspace_size.restype = C.c_size_t
        lib.mtp_verify_workspace_size.argtypes = [C.POINTER(VerifyArgs)]
        lib.mtp_verify_workspace_size.restype = C.c_size_t
        lib.mtp_strerror.argtypes = [C.c_int]
        lib.mtp_strerror.restype = C.c_char_p
        lib.mtp_abi_version.restype = C.c_int
        lib.mtp_profile_stage.argtypes = [C.c_int, C.POINTER(vp), C.POINTER(vp), C.c_int]
        lib.mtp_profile_count.restype = C.c_int
        lib.mtp_profile_all.argtypes = [C.POINTER(vp), C.POINTER(vp), C.POINTER(C.c_int), C.c_int]
        if lib.mtp_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{path} has ABI version {lib.mtp_abi_version()}, this binding "
                               f"expects {ABI_VERSION}: rebuild it")
        _lib = lib
    return _lib


class MtpError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {load().mtp_strerror(status).decode()}")


def _check(status: int):
    if status != 0:
        raise MtpError(status)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MTP_BF16
    if t.dtype == torch.float32:
        return MTP_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream) -> C.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _workspace(nbytes: int, device, cache: Optional[Dict] = None, key: str = "ws") -> torch.Tensor:
    if cache is not None and key in cache and cache[key].numel() >= nbytes:
        return cache[key]
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    if cache is not None:
        cache[key] = ws
    return ws


# ---------------------------------------------------------------------------
def chain_forward(tokens: torch.Tensor, segment_ids: torch.Tensor, h0: torch.Tensor,
                  embed: torch.Tensor, depths: Sequence[Dict[str, torch.Tensor]], *, n_heads: int,
                  head_dim: int, eps: float = 1e-6, rope_theta: float = 10000.0,
                  out: Optional[Dict] = None, cache: Optional[Dict] = None, save: bool = False,
                  stream=None) -> Dict:
    """mtp_chain_forward.  tokens/segment_ids int32 [B,T]; h0 [B*T,d]; embed [V,d];
    depths: D dicts with g_h, g_e, M, g_a, Wqkv, Wo, g_f, Wgate, Wup, Wdown.
    Returns dict(h=[D x [B*T,d]], state_mask, loss_mask, labels, counts, device_error), and with
    save=True also ``saved`` (uint8, the activations chain_backward can take instead of
    recomputing them; allocated unless ``out`` already holds one)."""
    B, T = tokens.shape
    V, d = embed.shape
    D = len(depths)
    ffn = depths[0]["Wgate"].shape[0]
    dev = h0.device
    if out is None:
        out = dict(h=[torch.empty_like(h0) for _ in range(D)],
                   state_mask=torch.empty((D, B, T), dtype=torch.uint8, device=dev),
                   loss_mask=torch.empty((D, B, T), dtype=torch.uint8, device=dev),
                   labels=torch.empty((D, B, T), dtype=torch.int32, device=dev),
                   counts=torch.empty((D,), dtype=torch.int32, device=dev),
                   device_error=torch.empty((1,), dtype=torch.int32, device=dev))
    ws_arr = (DepthWeights * D)()
    for k, w in enumerate(depths):
        ws_arr[k] = DepthWeights(_p(w["g_h"]), _p(w["g_e"]), _p(w["g_a"]), _p(w["g_f"]), _p(w["M"]),
                                 _p(w["Wqkv"]), _p(w["Wo"]), _p(w["Wgate"]), _p(w["Wup"]),
                                 _p(w["Wdown"]))
    hout = (vp * D)(*[h.data_ptr() for h in out["h"]])
    a = ChainArgs(B, T, d, n_heads, head_dim, ffn, V, D, _dtype_code(h0), eps, rope_theta,
                  _p(tokens), _p(segment_ids), _p(h0), _p(embed), ws_arr, hout,
                  _p(out["state_mask"]), _p(out["loss_mask"]), _p(out["labels"]), _p(out["counts"]),
                  _p(out["device_error"]), None, 0, None, 0)
    lib = load()
    if save:
        need = lib.mtp_chain_saved_bytes(C.byref(a))
        if need == 0:
            raise ValueError("saved activations need a valid bf16 chain")
        if out.get("saved") is None or out["saved"].numel() < need:
            out["saved"] = torch.empty(need, dtype=torch.uint8, device=dev)
        a.saved, a.saved_bytes = _p(out["saved"]), out["saved"].numel()
    nbytes = lib.mtp_chain_workspace_size(C.byref(a))
    if nbytes == 0:
        _check(lib.mtp_chain_forward(C.byref(a), _stream(stream)))   # raises the shape error
    ws = _workspace(nbytes, dev, cache, "chain_ws")
    a.workspace, a.workspace_bytes = _p(ws), ws.numel()
    _check(lib.mtp_chain_forward(C.byref(a), _stream(stream)))
    out["_keep"] = (ws_arr, hout, ws)
    return out


def _depth_weights(depths) -> C.Array:
    arr = (DepthWeights * len(depths))()
    for k, w in enumerate(depths):
        arr[k] = DepthWeights(_p(w["g_h"]), _p(w["g_e"]), _p(w["g_a"]), _p(w["g_f"]), _p(w["M"]),
                              _p(w["Wqkv"]), _p(w["Wo"]), _p(w["Wgate"]), _p(w["Wup"]), _p(w["Wdown"]))
    return arr


def chain_backward(tokens: torch.Tensor, segment_ids: torch.Tensor, h0: torch.Tensor, embed: torch.Tensor,
                   depths: Sequence[Dict[str, torch.Tensor]], hs: Sequence[torch.Tensor],
                   dh: Sequence[torch.Tensor], *, n_heads: int, head_dim: int, eps: float = 1e-6,
                   rope_theta: float = 10000.0, accumulate: bool = False, out: Optional[Dict] = None,
                   cache: Optional[Dict] = None, saved: Optional[torch.Tensor] = None, stream=None) -> Dict:
    """mtp_chain_backward.  hs: h^(1..D) from chain_forward; dh: D f32 tensors [B*T,d] (the
    head's gradients).  Returns dict(dh0 f32 [B*T,d], dE f32 [V,d] (added to; zeros when
    ``out`` is not given), dw = D dicts of f32 gradients keyed like the weights, device_error).
    saved: chain_forward(save=True)'s ``saved`` for the same inputs (skips the recompute)."""
    B, T = tokens.shape
    V, d = embed.shape
    D = len(depths)
    ffn = depths[0]["Wgate"].shape[0]
    dev = h0.device
    if out is None:
        out = dict(dh0=torch.empty((B * T, d), dtype=torch.float32, device=dev),
                   dE=torch.zeros((V, d), dtype=torch.float32, device=dev),
                   dw=[{n: torch.empty(w[n].shape, dtype=torch.float32, device=dev) for n in GRAD_FIELDS}
                       for w in depths],
                   device_error=torch.empty(1, dtype=torch.int32, device=dev))
    warr = _depth_weights(depths)
    garr = (DepthGrads * D)()
    for k, g in enumerate(out["dw"]):
        garr[k] = DepthGrads(_p(g["g_h"]), _p(g["g_e"]), _p(g["g_a"]), _p(g["g_f"]), _p(g["M"]), _p(g["Wqkv"]),
                             _p(g["Wo"]), _p(g["Wgate"]), _p(g["Wup"]), _p(g["Wdown"]))
    hp = (vp * D)(*[x.data_ptr() for x in hs])
    dhp = (vp * D)(*[x.data_ptr() for x in dh])
    a = ChainBwdArgs(B, T, d, n_heads, head_dim, ffn, V, D, _dtype_code(h0), eps, rope_theta, _p(tokens),
                     _p(segment_ids), _p(h0), _p(embed), warr, hp, dhp, _p(out["dh0"]), _p(out["dE"]), garr,
                     1 if accumulate else 0, _p(out["device_error"]), None, 0,
                     _p(saved) if saved is not None else None, saved.numel() if saved is not None else 0)
    lib = load()
    nbytes = lib.mtp_chain_backward_workspace_size(C.byref(a))
    if nbytes == 0:
        _check(lib.mtp_chain_backward(C.byref(a), _stream(stream)))
    ws = _workspace(nbytes, dev, cache, "chain_bwd_ws")
    a.workspace, a.workspace_bytes = _p(ws), ws.numel()
    _check(lib.mtp_chain_backward(C.byref(a), _stream(stream)))
    out["_keep"] = (warr, garr, hp, dhp, ws)
    return out


def horizon_heads(tokens: torch.Tensor, segment_ids: torch.Tensor, h: torch.Tensor,
                  blocks: Sequence[Dict[str, torch.Tensor]], W_out: torch.Tensor, g_out: torch.Tensor, *,
                  n_heads: int, head_dim: int, lam: float, eps: float = 1e-6, rope_theta: float = 10000.0,
                  accumulate: bool = False, out: Optional[Dict] = None, cache: Optional[Dict] = None,
                  stream=None) -> Dict:
    """mtp_horizon_heads.  h [B*T,d] trunk state; blocks: K dicts with g_a, g_f, Wqkv, Wo, Wgate, Wup, Wdown.
    Returns dict(loss [K], counts [K], loss_total [1], dh f32 [B*T,d], dW_out, dg_out,
    dw = K dicts of f32 block gradients, device_error)."""
    B, T = tokens.shape
    V, d = W_out.shape
    K = len(blocks)
    ffn = blocks[0]["Wgate"].shape[0]
    dev = h.device
    if out is None:
        out = dict(loss=torch.empty(K, dtype=torch.float32, device=dev),
                   counts=torch.empty(K, dtype=torch.int32, device=dev),
                   loss_total=torch.empty(1, dtype=torch.float32, device=dev),
                   dh=torch.empty((B * T, d), dtype=torch.float32, device=dev),
                   dW_out=torch.empty((V, d), dtype=torch.float32, device=dev),
                   dg_out=torch.empty((d,), dtype=torch.float32, device=dev),
                   dw=[{n: torch.empty(b[n].shape, dtype=torch.float32, device=dev) for n in BLOCK_FIELDS}
                       for b in blocks],
                   device_error=torch.empty(1, dtype=torch.int32, device=dev))
    warr = (BlockWeights * K)()
    garr = (BlockGrads * K)()
    for k, (b, g) in enumerate(zip(blocks, out["dw"])):
        warr[k] = BlockWeights(*[_p(b[n]) for n in BLOCK_FIELDS])
        garr[k] = BlockGrads(*[_p(g[n]) for n in BLOCK_FIELDS])
    a = HorizonArgs(B, T, d, n_heads, head_dim, ffn, V, K, _dtype_code(h), eps, rope_theta, lam, _p(tokens),
                    _p(segment_ids), _p(h), warr, _p(W_out), _p(g_out), _p(out["loss"]), _p(out["counts"]),
                    _p(out["loss_total"]), _p(out["dh"]), _p(out["dW_out"]), _p(out["dg_out"]), garr,
                    1 if accumulate else 0, _p(out["device_error"]), None, 0)
    lib = load()
    nbytes = lib.mtp_horizon_heads_workspace_size(C.byref(a))
    if nbytes == 0:
        _check(lib.mtp_horizon_heads(C.byref(a), _stream(stream)))
    ws = _workspace(nbytes, dev, cache, "horizon_ws")
    a.workspace, a.workspace_bytes = _p(ws), ws.numel()
    _check(lib.mtp_horizon_heads(C.byref(a), _stream(stream)))
    out["_keep"] = (warr, garr, ws)
    return out


def head_ce_fwd_bwd(hs: Sequence[torch.Tensor], labels: torch.Tensor, W_out: torch.Tensor,
                    g_out: torch.Tensor, *, lam: float, eps: float = 1e-6, reduce: str = "fixed",
                    denom: float = 0.0, accumulate: bool = False, want_lse: bool = False,
                    want_accuracy: bool = False, dh_accumulate: bool = False, logit_slab_bytes: int = 0,
                    out: Optional[Dict] = None,
                    cache: Optional[Dict] = None, stream=None) -> Dict:
    """mtp_head_ce_fwd_bwd.  hs: D tensors [B*T,d]; labels int32 [D,B,T].  logit_slab_bytes
    bounds the kept logits of a slab (fp16 for bf16, fp32 for f32) and the dz row group
    (0: the library default, 1 GiB with at most half of the rows per slab).
    Returns dict(loss_sum, counts, loss, loss_mtp, lse, dh, dW_out, dg_out, device_error,
    pred, correct, accuracy); the last three (top-1 accuracy by depth) only with
    want_accuracy (or when ``out`` holds them)."""
    D, B, T = labels.shape
    V, d = W_out.shape
    dev = W_out.device
    if out is None:
        out = dict(loss_sum=torch.empty(D, dtype=torch.float32, device=dev),
                   counts=torch.empty(D, dtype=torch.int32, device=dev),
                   loss=torch.empty(D, dtype=torch.float32, device=dev),
                   loss_mtp=torch.empty(1, dtype=torch.float32, device=dev),
                   lse=torch.empty((D, B * T), dtype=torch.float32, device=dev) if want_lse else None,
                   dh=[torch.empty((B * T, d), dtype=torch.float32, device=dev) for _ in range(D)],
                   dW_out=torch.zeros((V, d), dtype=torch.float32, device=dev),
                   dg_out=torch.zeros((d,), dtype=torch.float32, device=dev),
                   device_error=torch.empty(1, dtype=torch.int32, device=dev))
        if want_accuracy:
            out.update(pred=torch.empty((D, B * T), dtype=torch.int32, device=dev),
                       correct=torch.empty(D, dtype=torch.int32, device=dev),
                       accuracy=torch.empty(D, dtype=torch.float32, device=dev))
    hp = (vp * D)(*[h.data_ptr() for h in hs])
    dhp = (vp * D)(*[x.data_ptr() for x in out["dh"]])
    red = {"fixed": MTP_REDUCE_FIXED, "valid_mean": MTP_REDUCE_VALID_MEAN}[reduce]
    a = CeArgs(B, T, d, V, D, _dtype_code(W_out), eps, lam, red, float(denom), hp, _p(labels),
               _p(W_out), _p(g_out), _p(out["loss_sum"]), _p(out["counts"]), _p(out["loss"]),
               _p(out["loss_mtp"]), _p(out["lse"]), dhp, _p(out["dW_out"]), _p(out["dg_out"]),
               1 if accumulate else 0, _p(out["device_error"]), int(logit_slab_bytes),
               1 if dh_accumulate else 0, _p(out.get("pred")), _p(out.get("correct")), _p(out.get("accuracy")), None, 0)
    lib = load()
    nbytes = lib.mtp_ce_workspace_size(C.byref(a))
    if nbytes == 0:
        _check(lib.mtp_head_ce_fwd_bwd(C.byref(a), _stream(stream)))
    ws = _workspace(nbytes, dev, cache, "ce_ws")
    a.workspace, a.workspace_bytes = _p(ws), ws.numel()
    _check(lib.mtp_head_ce_fwd_bwd(C.byref(a), _stream(stream)))
    out["_keep"] = (hp, dhp, ws)
    return out


def verify(target_logits: torch.Tensor, draft_logits: torch.Tensor, draft_tokens: torch.Tensor,
           u_accept: torch.Tensor, u_sample: torch.Tensor, *, temperature: float = 1.0,
           want_margin: bool = True, out: Optional[Dict] = None, cache: Optional[Dict] = None,
           stream=None) -> Dict:
    """mtp_verify.  target [R, g+1, V], draft [R, g, V] (bf16 or f32), draft_tokens int32
    [R, g], u_accept f32 [R, g], u_sample f32 [R, g+1]."""
    R, G1, V = target_logits.shape
    G = G1 - 1
    dev = target_logits.device
    if out is None:
        out = dict(accepted_len=torch.empty(R, dtype=torch.int32, device=dev),
                   next_token=torch.empty(R, dtype=torch.int32, device=dev),
                   status=torch.empty(R, dtype=torch.int32, device=dev),
                   margin=torch.empty(R, dtype=torch.float32, device=dev) if want_margin else None)
    a = VerifyArgs(R, G, V, temperature, _dtype_code(target_logits), _p(target_logits),
                   _p(draft_logits), _p(draft_tokens), _p(u_accept), _p(u_sample),
                   _p(out["accepted_len"]), _p(out["next_token"]), _p(out["status"]),
                   _p(out["margin"]), None, 0)
    lib = load()
    nbytes = lib.mtp_verify_workspace_size(C.byref(a))
    if nbytes == 0:
        _check(lib.mtp_verify(C.byref(a), _stream(stream)))
    ws = _workspace(nbytes, dev, cache, "verify_ws")
    a.workspace, a.workspace_bytes = _p(ws), ws.numel()
    _check(lib.mtp_verify(C.byref(a), _stream(stream)))
    out["_keep"] = (ws,)
    return out


def verify_noalloc(target_logits: torch.Tensor, draft_logits: torch.Tensor, draft_tokens: torch.Tensor,
                   u_accept: torch.Tensor, u_sample: torch.Tensor, *, temperature: float = 1.0,
                   out: Dict, stream=None) -> Dict:
    """mtp_verify_noalloc: as ``verify`` with caller-allocated outputs ``out``
    (accepted_len, next_token, status int32 [R]; margin f32 [R] or None) and
    the library's static scratch instead of a workspace."""
    R, G1, V = target_logits.shape
    a = VerifyArgs(R, G1 - 1, V, temperature, _dtype_code(target_logits), _p(target_logits),
                   _p(draft_logits), _p(draft_tokens), _p(u_accept), _p(u_sample),
                   _p(out["accepted_len"]), _p(out["next_token"]), _p(out["status"]),
                   _p(out.get("margin")), None, 0)
    _check(load().mtp_verify_noalloc(C.byref(a), _stream(stream)))
    return out


def propose_step(h_prev: torch.Tensor, tokens: torch.Tensor, positions: torch.Tensor,
                 u_sample: torch.Tensor, kv_cache: torch.Tensor, weights: Dict[str, torch.Tensor],
                 embed: torch.Tensor, W_out: torch.Tensor, g_out: torch.Tensor, *, n_heads: int,
                 head_dim: int, eps: float = 1e-6, rope_theta: float = 10000.0, temperature: float = 1.0,
                 want_margin: bool = True, out: Optional[Dict] = None, cache: Optional[Dict] = None,
                 stream=None) -> Dict:
    """mtp_propose_step.  h_prev [R,d]; tokens, positions int32 [R]; u_sample f32 [R];
    kv_cache [R, 2, L_max, n_heads*head_dim] (updated in place at each request's slot);
    weights: one module's dict (g_h, g_e, M, g_a, Wqkv, Wo, g_f, Wgate, Wup, Wdown).
    Returns dict(h_out, logits, draft_token, status, margin)."""
    R, d = h_prev.shape
    V = embed.shape[0]
    L_max = kv_cache.shape[2]
    dev = h_prev.device
    if out is None:
        out = dict(h_out=torch.empty_like(h_prev),
                   logits=torch.empty((R, V), dtype=h_prev.dtype, device=dev),
                   draft_token=torch.empty(R, dtype=torch.int32, device=dev),
                   status=torch.empty(R, dtype=torch.int32, device=dev),
                   margin=torch.empty(R, dtype=torch.float32, device=dev) if want_margin else None)
    w = weights
    warr = (DepthWeights * 1)()
    warr[0] = DepthWeights(_p(w["g_h"]), _p(w["g_e"]), _p(w["g_a"]), _p(w["g_f"]), _p(w["M"]),
                           _p(w["Wqkv"]), _p(w["Wo"]), _p(w["Wgate"]), _p(w["Wup"]), _p(w["Wdown"]))
    a = ProposeArgs(R, L_max, d, n_heads, head_dim, w["Wgate"].shape[0], V, _dtype_code(h_prev), eps,
                    rope_theta, temperature, warr, _p(embed), _p(W_out), _p(g_out), _p(h_prev),
                    _p(tokens), _p(positions), _p(u_sample), _p(kv_cache), _p(out["h_out"]),
                    _p(out["logits"]), _p(out["draft_token"]), _p(out["status"]), _p(out.get("margin")),
                    None, 0)
    lib = load()
    nbytes = lib.mtp_propose_workspace_size(C.byref(a))
    if nbytes == 0:
        _check(lib.mtp_propose_step(C.byref(a), _stream(stream)))
    ws = _workspace(nbytes, dev, cache, "propose_ws")
    a.workspace, a.workspace_bytes = _p(ws), ws.numel()
    _check(lib.mtp_propose_step(C.byref(a), _stream(stream)))
    out["_keep"] = (warr, ws)
    return out


def round_commit(draft_tokens: torch.Tensor, accepted_len: torch.Tensor, next_token: torch.Tensor,
                 status: torch.Tensor, remaining: torch.Tensor, *, eos: int = -1, out: Optional[Dict] = None,
                 stream=None) -> Dict:
    """mtp_round_commit.  draft_tokens int32 [R, gamma]; accepted_len, next_token, status,
    remaining int32 [R].  Returns dict(new_tokens [R, gamma+1], n_new, rows_to_keep,
    pending_frontier, stopped)."""
    R, G = draft_tokens.shape
    dev = draft_tokens.device
    if out is None:
        out = dict(new_tokens=torch.empty((R, G + 1), dtype=torch.int32, device=dev),
                   **{k: torch.empty(R, dtype=torch.int32, device=dev)
                      for k in ("n_new", "rows_to_keep", "pending_frontier", "stopped")})
    a = RoundArgs(R, G, eos, _p(draft_tokens), _p(accepted_len), _p(next_token), _p(status), _p(remaining),
                  _p(out["new_tokens"]), _p(out["n_new"]), _p(out["rows_to_keep"]), _p(out["pending_frontier"]),
                  _p(out["stopped"]))
    _check(load().mtp_round_commit(C.byref(a), _stream(stream)))
    return out


class StageTimer:
    """Arms mtp_profile_stage with ``n`` hipEvent pairs (torch CUDA events on
    the calling stream) around every launch of one stage."""

    def __init__(self, stage: str, n: int):
        self.stage = STAGES.index(stage)
        self.start = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        self.stop = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in self.start + self.stop:
            e.record()                       # materialise the hipEvent_t handles
        torch.cuda.synchronize()
        self._s = (vp * n)(*[e.cuda_event for e in self.start])
        self._e = (vp * n)(*[e.cuda_event for e in self.stop])
        self.n = n

    def __enter__(self):
        _check(load().mtp_profile_stage(self.stage, self._s, self._e, self.n))
        return self

    def __exit__(self, *exc):
        self.count = load().mtp_profile_count()
        load().mtp_profile_stage(-1, None, None, 0)

    def times_ms(self):
        torch.cuda.synchronize()
        k = min(self.count, self.n)
        return [self.start[i].elapsed_time(self.stop[i]) for i in range(k)]


class AllStageTimer:
    """Arms mtp_profile_all with ``n`` hipEvent pairs: every launch of every
    stage records a pair and its stage id.  ``by_stage()`` returns the launch
    times (ms) grouped by stage name (the first ``n`` launches)."""

    def __init__(self, n: int):
        self.start = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        self.stop = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in self.start + self.stop:
            e.record()
        torch.cuda.synchronize()
        self._s = (vp * n)(*[e.cuda_event for e in self.start])
        self._e = (vp * n)(*[e.cuda_event for e in self.stop])
        self._ids = (C.c_int * n)()
        self.n = n

    def __enter__(self):
        _check(load().mtp_profile_all(self._s, self._e, self._ids, self.n))
        return self

    def __exit__(self, *exc):
        self.count = load().mtp_profile_count()
        load().mtp_profile_stage(-1, None, None, 0)

    def by_stage(self):
        torch.cuda.synchronize()
        if self.count > self.n:
            raise RuntimeError(f"{self.count} launches recorded into {self.n} slots")
        out: Dict[str, List[float]] = {}
        for i in range(self.count):
            out.setdefault(STAGES[self._ids[i]], []).append(self.start[i].elapsed_time(self.stop[i]))
        return out
