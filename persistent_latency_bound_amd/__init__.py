"""Python binding of libpld.so, the persistent batch-1 decode library for MI355X.

Argument marshalling only: every step of the decode path runs in the HIP kernels of
libpld.so (C ABI in include/pld.h). torch is used for device memory and streams. There
is no fallback: if the library is missing, using it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpld.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "pld.h")

PLD_OK, PLD_E_INVALID, PLD_E_UNSUPPORTED, PLD_E_CAPACITY, PLD_E_HIP, PLD_E_DEVICE_TIMEOUT, PLD_E_STATE = 0, -1, -2, -3, -4, -5, -6
PLD_ATTN_GQA, PLD_ATTN_MLA, PLD_ATTN_KDA = 0, 1, 2
PLD_WFMT_BF16, PLD_WFMT_FP8_BLOCK128, PLD_WFMT_LUT3 = 0, 1, 2
PLD_FFN_DENSE, PLD_FFN_MOE = 0, 1
PLD_ROUTER_SOFTMAX_TOPK, PLD_ROUTER_SIGMOID_BIAS = 0, 1

# every entry point include/pld.h declares
EXPORTS = (
    "pld_workspace_bytes", "decode_layer_init", "decode_step", "decode_layers_persistent", "decode_poll_status",
    "decode_reset", "decode_layer_destroy", "pld_status_string", "pld_debug_buffer", "pld_launch_shape",
    "pld_set_watchdog_us", "pld_set_trace", "pld_set_test_hooks", "decode_layer_init_static", "decode_speculative",
    "pld_workspace_bytes_for_cus", "decode_verify_batched", "decode_batch",
)
PLD_HOOK_DROP_WG0, PLD_HOOK_DELAY = 1, 2

i32, vp, f64 = ctypes.c_int32, ctypes.c_void_p, ctypes.c_double


class PldConfig(ctypes.Structure):
    _fields_ = [(n, i32) for n in (
        "attn_kind", "wfmt", "hidden", "n_heads", "n_kv_heads", "head_dim", "q_lora", "kv_lora", "rope_dim",
        "nope_dim", "v_dim", "index_heads", "index_dim", "index_topk", "ffn_kind", "inter", "n_experts", "top_k",
        "n_shared", "router_kind", "max_seq")] + [("eps", f64), ("rope_base", f64), ("vocab", i32),
                                                   ("kda_rank", i32), ("conv_width", i32), ("expert_wfmt", i32),
                                                   ("max_query", i32), ("max_batch", i32)]


class PldMatrix(ctypes.Structure):
    _fields_ = [("data", vp), ("scales", vp)]


class PldLayerWeights(ctypes.Structure):
    _fields_ = [("attn_norm", vp), ("ffn_norm", vp), ("q_norm", vp), ("kv_norm", vp)] + \
               [(n, PldMatrix) for n in ("wq", "wk", "wv", "w_dq", "w_uq", "w_dkv", "w_uk", "w_uv", "w_qi", "w_w",
                                         "w_ki", "wo")] + \
               [("router", vp), ("router_bias", vp)] + [(n, PldMatrix) for n in ("w_gate", "w_up", "w_down")] + \
               [(n, PldMatrix) for n in ("w_g", "w_beta", "w_adown", "w_aup")] + [("conv_taps", vp), ("o_norm", vp)]


class PldKvCache(ctypes.Structure):
    _fields_ = [("k", vp), ("v", vp), ("latent", vp), ("index_codes", vp), ("index_scales", vp), ("kda_state", vp),
                ("conv_ring", vp)]


class PldHeadWeights(ctypes.Structure):
    _fields_ = [("embed", vp), ("final_norm", vp), ("head", PldMatrix)]


class PldDeviceStatus(ctypes.Structure):
    _fields_ = [("code", i32), ("stage", i32), ("layer", i32), ("token", i32), ("wg", i32), ("reserved", i32 * 3)]


class PldPersistentArgs(ctypes.Structure):
    _fields_ = [("start_pos", i32), ("n_tokens", i32), ("n_query", i32), ("in_token", i32), ("in_hidden", vp),
                ("draft_tokens", vp), ("out_hidden", vp), ("out_logits", vp), ("out_tokens", vp),
                ("out_accepted", vp), ("temperature", f64), ("sample_seed", ctypes.c_uint64)]


class PldSpecArgs(ctypes.Structure):
    _fields_ = [("start_pos", i32), ("in_token", i32), ("n_tokens", i32), ("n_draft", i32), ("temperature", f64),
                ("sample_seed", ctypes.c_uint64), ("out_tokens", vp), ("out_stats", vp)]


class PldBatchArgs(ctypes.Structure):
    _fields_ = [("n_seq", i32), ("n_tokens", i32), ("start_pos", i32 * 8), ("in_token", i32 * 8),
                ("out_logits", vp), ("out_tokens", vp), ("out_hidden", vp), ("temperature", f64),
                ("sample_seed", ctypes.c_uint64)]


# intermediates kept as LL words (32-bit payload, 32-bit epoch) in the workspace
LL_BUFFERS = ("q", "o", "h2", "logits", "m", "x", "cq", "ckv", "qrope", "qlat", "olat", "qi", "ixr", "isel", "ilist",
              "part", "kv", "amax",
              "vx", "vcq", "vckv", "vqlat", "volat", "vo", "vh2")

_lib = None


def lib():
    """Load libpld.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run python -m persistent_latency_bound_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        L.pld_workspace_bytes.argtypes = [ctypes.POINTER(PldConfig), i32]
        L.pld_workspace_bytes.restype = ctypes.c_size_t
        L.pld_workspace_bytes_for_cus.argtypes = [ctypes.POINTER(PldConfig), i32, i32]
        L.pld_workspace_bytes_for_cus.restype = ctypes.c_size_t
        L.decode_layer_init.argtypes = [ctypes.POINTER(PldConfig), i32, ctypes.POINTER(PldLayerWeights),
                                        ctypes.POINTER(PldKvCache), ctypes.POINTER(PldHeadWeights), vp,
                                        ctypes.c_size_t, ctypes.POINTER(vp)]
        L.decode_layer_init_static.argtypes = [ctypes.POINTER(PldConfig), i32, ctypes.POINTER(PldLayerWeights),
                                               ctypes.POINTER(PldKvCache), ctypes.POINTER(PldHeadWeights),
                                               ctypes.POINTER(vp)]
        L.decode_step.argtypes = [vp, i32, vp, i32, vp, vp]
        L.decode_speculative.argtypes = [vp, vp, ctypes.POINTER(PldSpecArgs), vp]
        L.decode_layers_persistent.argtypes = [vp, ctypes.POINTER(PldPersistentArgs), vp]
        L.decode_poll_status.argtypes = [vp, ctypes.POINTER(PldDeviceStatus)]
        L.decode_reset.argtypes = [vp]
        L.decode_layer_destroy.argtypes = [vp]
        L.decode_layer_destroy.restype = None
        L.pld_status_string.argtypes = [i32]
        L.pld_status_string.restype = ctypes.c_char_p
        L.pld_debug_buffer.argtypes = [vp, ctypes.c_char_p, ctypes.POINTER(vp), ctypes.POINTER(ctypes.c_size_t)]
        L.pld_launch_shape.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i32)]
        L.pld_set_watchdog_us.argtypes = [vp, ctypes.c_int64]
        L.pld_set_trace.argtypes = [vp, vp, ctypes.c_size_t]
        L.pld_set_test_hooks.argtypes = [vp, i32, ctypes.c_uint32]
        L.decode_verify_batched.argtypes = [vp, vp, vp]
        L.decode_batch.argtypes = [vp, vp, vp]
        for f in ("decode_layer_init", "decode_layer_init_static", "decode_speculative", "decode_step",
                  "decode_layers_persistent", "decode_verify_batched", "decode_batch", "decode_poll_status",
                  "decode_reset", "pld_debug_buffer", "pld_launch_shape", "pld_set_watchdog_us", "pld_set_trace",
                  "pld_set_test_hooks"):
            getattr(L, f).restype = i32
        _lib = L
    return _lib


class PldError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        msg = lib().pld_status_string(code).decode()
        super().__init__(f"{what}: {msg} ({code})")


def check(code: int, what: str):
    if code != PLD_OK:
        raise PldError(code, what)


def config_from_shape(s, vocab: int = 0, max_query: int = 0, max_batch: int = 0) -> PldConfig:
    """pld_config of a synth.configs.LayerShape."""
    c = PldConfig()
    c.attn_kind = {"gqa": PLD_ATTN_GQA, "mla": PLD_ATTN_MLA, "kda": PLD_ATTN_KDA}[s.attn]
    c.wfmt = PLD_WFMT_FP8_BLOCK128 if s.wfmt == "fp8" else PLD_WFMT_BF16
    c.hidden, c.n_heads, c.n_kv_heads, c.head_dim = s.hidden, s.n_heads, s.n_kv_heads, s.head_dim
    c.q_lora, c.kv_lora, c.rope_dim, c.nope_dim, c.v_dim = s.q_lora, s.kv_lora, s.rope_dim, s.nope_dim, s.v_dim
    c.index_heads, c.index_dim, c.index_topk = s.index_heads, s.index_dim, s.index_topk
    c.ffn_kind = PLD_FFN_MOE if s.ffn == "moe" else PLD_FFN_DENSE
    c.inter, c.n_experts, c.top_k, c.n_shared = s.inter, s.n_experts, s.top_k, s.n_shared
    c.router_kind = PLD_ROUTER_SIGMOID_BIAS if s.router == "sigmoid_bias" else PLD_ROUTER_SOFTMAX_TOPK
    c.max_seq, c.eps, c.rope_base, c.vocab = s.max_seq, s.eps, s.rope_base, vocab
    c.kda_rank, c.conv_width = s.kda_rank, s.conv_width
    c.expert_wfmt = PLD_WFMT_LUT3 if s.expert_fmt == "lut3" else 0
    c.max_query = int(max_query)
    c.max_batch = int(max_batch)
    return c


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _mat(m) -> PldMatrix:
    x = PldMatrix()
    if m is not None:
        x.data = m["data"].data_ptr()
        x.scales = _ptr(m.get("scales"))
    return x


def layer_struct(W: dict) -> PldLayerWeights:
    """pld_layer_weights from a dict of device tensors (as made by synth.device.layer_weights)."""
    L = PldLayerWeights()
    for n in ("attn_norm", "ffn_norm", "q_norm", "kv_norm", "router_bias", "conv_taps", "o_norm"):
        if n in W:
            setattr(L, n, W[n].data_ptr())
    for n in ("wq", "wk", "wv", "w_dq", "w_uq", "w_dkv", "w_uk", "w_uv", "w_qi", "w_w", "w_ki", "wo", "w_gate",
              "w_up", "w_down", "w_g", "w_beta", "w_adown", "w_aup"):
        if n in W:
            setattr(L, n, _mat(W[n]))
    if "router" in W:
        L.router = W["router"]["data"].data_ptr()
    return L


def cache_struct(C: dict) -> PldKvCache:
    K = PldKvCache()
    for n in ("k", "v", "latent", "index_codes", "index_scales", "kda_state", "conv_ring"):
        if n in C:
            setattr(K, n, C[n].data_ptr())
    return K


class Decoder:
    """One decode handle over a stack of layers (weights and caches are caller-owned torch tensors)."""

    def __init__(self, shape, layers: Sequence[dict], caches: Sequence[dict], head: Optional[dict] = None,
                 vocab: int = 0, static: bool = False, max_query: int = 0, max_batch: int = 0):
        """static=True: decode_layer_init_static (the library's own device array, no workspace
        allocation; one such handle per GPU, re-initialised by every such call).
        max_query >= 2: the workspace also holds the batched verify's buffers (verify_batched).
        max_batch >= 2: batch decode of up to max_batch sequences (batch); every layer's latent
        cache then holds max_batch sequences of max_seq rows back to back."""
        import torch

        self.shape = shape
        self.cfg = config_from_shape(shape, vocab, max_query, max_batch)
        n = len(layers)
        self._keep = (list(layers), list(caches), head)   # keep the tensors alive
        self.static = static
        if not static:
            ws = lib().pld_workspace_bytes(ctypes.byref(self.cfg), n)
            if ws == 0:
                raise PldError(PLD_E_UNSUPPORTED, "pld_workspace_bytes")
            self.workspace = torch.zeros(ws, dtype=torch.uint8, device="cuda")
        arr_w = (PldLayerWeights * n)(*[layer_struct(W) for W in layers])
        arr_c = (PldKvCache * n)(*[cache_struct(C) for C in caches])
        hp = None
        if head is not None:
            h = PldHeadWeights()
            h.embed = head["embed"].data_ptr()
            h.final_norm = head["final_norm"].data_ptr()
            h.head = _mat(head["head"])
            hp = ctypes.byref(h)
        self.handle = vp()
        if static:
            check(lib().decode_layer_init_static(ctypes.byref(self.cfg), n, arr_w, arr_c, hp,
                                                 ctypes.byref(self.handle)), "decode_layer_init_static")
        else:
            check(lib().decode_layer_init(ctypes.byref(self.cfg), n, arr_w, arr_c, hp, self.workspace.data_ptr(), ws,
                                          ctypes.byref(self.handle)), "decode_layer_init")

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value and _lib is not None:
            _lib.decode_layer_destroy(h)
            self.handle = None

    @staticmethod
    def _stream():
        import torch
        return vp(torch.cuda.current_stream().cuda_stream)

    def step(self, layer: int, x_in, pos: int, x_out):
        check(lib().decode_step(self.handle, layer, x_in.data_ptr(), pos, x_out.data_ptr(), self._stream()),
              "decode_step")

    def persistent(self, start_pos: int, in_hidden=None, out_hidden=None, n_tokens: int = 1, n_query: int = 1,
                   in_token: int = -1, draft_tokens=None, out_logits=None, out_tokens=None, out_accepted=None,
                   temperature: float = 0.0, sample_seed: int = 0):
        a = PldPersistentArgs()
        a.start_pos, a.n_tokens, a.n_query, a.in_token = start_pos, n_tokens, n_query, in_token
        a.temperature, a.sample_seed = float(temperature), int(sample_seed) & 0xFFFFFFFFFFFFFFFF
        a.in_hidden, a.out_hidden = _ptr(in_hidden), _ptr(out_hidden)
        a.draft_tokens, a.out_logits = _ptr(draft_tokens), _ptr(out_logits)
        a.out_tokens, a.out_accepted = _ptr(out_tokens), _ptr(out_accepted)
        check(lib().decode_layers_persistent(self.handle, ctypes.byref(a), self._stream()), "decode_layers_persistent")

    def verify_batched(self, start_pos: int, in_token: int, draft_tokens, out_hidden, out_logits=None,
                       out_tokens=None, out_accepted=None, temperature: float = 0.0, sample_seed: int = 0):
        """decode_verify_batched: 1 + len(draft_tokens) positions through the stack together."""
        a = PldPersistentArgs()
        a.start_pos, a.n_tokens, a.n_query, a.in_token = start_pos, 1, int(draft_tokens.numel()) + 1, in_token
        a.temperature, a.sample_seed = float(temperature), int(sample_seed) & 0xFFFFFFFFFFFFFFFF
        a.in_hidden, a.out_hidden = None, _ptr(out_hidden)
        a.draft_tokens, a.out_logits = _ptr(draft_tokens), _ptr(out_logits)
        a.out_tokens, a.out_accepted = _ptr(out_tokens), _ptr(out_accepted)
        check(lib().decode_verify_batched(self.handle, ctypes.byref(a), self._stream()), "decode_verify_batched")

    def batch(self, start_pos, in_token, n_tokens: int, out_tokens, out_hidden, out_logits=None,
              temperature: float = 0.0, sample_seed: int = 0):
        """decode_batch: len(start_pos) sequences, n_tokens steps."""
        a = PldBatchArgs()
        a.n_seq, a.n_tokens = len(start_pos), int(n_tokens)
        for b, (p, t) in enumerate(zip(start_pos, in_token)):
            a.start_pos[b], a.in_token[b] = int(p), int(t)
        a.out_logits, a.out_tokens, a.out_hidden = _ptr(out_logits), _ptr(out_tokens), _ptr(out_hidden)
        a.temperature, a.sample_seed = float(temperature), int(sample_seed) & 0xFFFFFFFFFFFFFFFF
        check(lib().decode_batch(self.handle, ctypes.byref(a), self._stream()), "decode_batch")

    def speculative(self, draft: "Decoder", start_pos: int, in_token: int, n_tokens: int, n_draft: int, out_tokens,
                    temperature: float = 0.0, sample_seed: int = 0):
        """decode_speculative with this decoder as the target; returns (verify launches, drafts kept)."""
        a = PldSpecArgs()
        a.start_pos, a.in_token, a.n_tokens, a.n_draft = start_pos, in_token, n_tokens, n_draft
        a.temperature, a.sample_seed = float(temperature), int(sample_seed) & 0xFFFFFFFFFFFFFFFF
        a.out_tokens = out_tokens.data_ptr()
        stats = (i32 * 2)()
        a.out_stats = ctypes.cast(stats, vp)
        check(lib().decode_speculative(self.handle, draft.handle, ctypes.byref(a), self._stream()),
              "decode_speculative")
        return stats[0], stats[1]

    def status(self) -> PldDeviceStatus:
        st = PldDeviceStatus()
        rc = lib().decode_poll_status(self.handle, ctypes.byref(st))
        if rc not in (PLD_OK, PLD_E_DEVICE_TIMEOUT):
            check(rc, "decode_poll_status")
        return st

    def reset(self):
        check(lib().decode_reset(self.handle), "decode_reset")

    def set_test_hooks(self, flags: int, seed: int = 0):
        check(lib().pld_set_test_hooks(self.handle, int(flags), int(seed) & 0xFFFFFFFF), "pld_set_test_hooks")

    def set_watchdog_us(self, us: int):
        check(lib().pld_set_watchdog_us(self.handle, int(us)), "pld_set_watchdog_us")

    def set_trace(self, buf):
        """Record per-stage wall-clock stamps into `buf` (int64 device tensor) on later launches; None stops."""
        if buf is None:
            check(lib().pld_set_trace(self.handle, None, 0), "pld_set_trace")
        else:
            check(lib().pld_set_trace(self.handle, buf.data_ptr(), buf.numel() * buf.element_size()), "pld_set_trace")
        self._trace = buf

    def launch_shape(self):
        n, b = i32(), i32()
        check(lib().pld_launch_shape(self.handle, ctypes.byref(n), ctypes.byref(b)), "pld_launch_shape")
        return n.value, b.value

    def debug_raw(self, name: str):
        """The workspace bytes of a named buffer as a uint8 view (not a copy)."""
        if self.static:
            raise RuntimeError("the workspace of a static handle is the library's own array; no debug view")
        p, nb = vp(), ctypes.c_size_t()
        check(lib().pld_debug_buffer(self.handle, name.encode(), ctypes.byref(p), ctypes.byref(nb)), "pld_debug_buffer")
        off = p.value - self.workspace.data_ptr()
        return self.workspace[off: off + nb.value]

    def debug(self, name: str, dtype=None):
        """Copy of an intermediate left in the workspace by the last launch (after a sync)."""
        import torch
        if self.static:
            raise RuntimeError("the workspace of a static handle is the library's own array; no debug view")
        p, nb = vp(), ctypes.c_size_t()
        check(lib().pld_debug_buffer(self.handle, name.encode(), ctypes.byref(p), ctypes.byref(nb)), "pld_debug_buffer")
        off = p.value - self.workspace.data_ptr()
        raw = self.workspace[off: off + nb.value].clone()
        if name in LL_BUFFERS:   # 8-byte LL words: keep the 32-bit payloads (low halves)
            raw = raw.view(torch.int32)[0::2].contiguous().view(torch.uint8)
        default = {"logits": torch.float64, "sel": torch.int32, "x": torch.int16, "qi": torch.int16,
                   "isel": torch.int32, "ikh": torch.int32, "ikl": torch.int32,
                   "ilist": torch.int32, "ilo": torch.int32, "itok": torch.int32,
                   "qlat": torch.int16, "qrope": torch.int16, "vx": torch.int16, "vqlat": torch.int16,
                   "vo": torch.int16, "vsel": torch.int32}   # bf16 bits
        if name == "cq" and getattr(self.shape, "index_topk", 0):
            default["cq"] = torch.float64   # the sparse layer passes c_q' in fp64 (word pairs)
        return raw.view(dtype or default.get(name, torch.float32))
