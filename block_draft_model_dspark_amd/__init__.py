"""DSpark draft round on MI355X (gfx950).

Thin ctypes binding of the HIP library `libdspark.so` (C ABI in
include/dspark.h).  Python only marshals arguments: device buffers and the
current stream come from PyTorch, every step of the round runs in the
library's kernels.  There is no CPU fallback: if the library is not built,
`load_library()` raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdspark.so")

F32, BF16, Q4 = 0, 1, 2
INPUT_CONTEXT_HIDDEN, INPUT_TARGET_FEATURES = 0, 1
TALL_ROWS_DEFAULT = 48  # dspark_model_set_tall_rows's default
_KIND = {"f32": F32, "bf16": BF16, "q4": Q4}

EXPORTED = ("dspark_model_create", "dspark_model_destroy", "dspark_model_set_tall_rows", "dspark_model_aux_bytes",
            "dspark_model_prepare",
            "dspark_project_workspace_bytes", "dspark_project_context_kv", "dspark_draft_workspace_bytes",
            "dspark_draft_rows", "dspark_draft_block", "dspark_profile_enable", "dspark_profile_read",
            "dspark_tall_tile_of", "dspark_stream_block_of", "dspark_draft_rows_noalloc", "dspark_draft_noalloc_max_bytes",
            "dspark_q4_address_check",
            "dspark_draft_rows_conf", "dspark_draft_rows_ex",
            "dspark_last_error")


class DsparkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"dspark status {status}: {msg}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("hidden_size", ctypes.c_int32), ("num_hidden_layers", ctypes.c_int32),
                ("num_attention_heads", ctypes.c_int32), ("global_head_dim", ctypes.c_int32),
                ("num_global_key_value_heads", ctypes.c_int32), ("intermediate_size", ctypes.c_int32),
                ("vocab_size", ctypes.c_int32), ("block_size", ctypes.c_int32), ("mask_token_id", ctypes.c_int32),
                ("markov_rank", ctypes.c_int32), ("attention_k_eq_v", ctypes.c_int32),
                ("markov_head_vanilla", ctypes.c_int32), ("activation_gelu_tanh", ctypes.c_int32),
                ("fc_in", ctypes.c_int32), ("rope_theta", ctypes.c_double),
                ("partial_rotary_factor", ctypes.c_double), ("rms_norm_eps", ctypes.c_double),
                ("final_logit_softcapping", ctypes.c_double), ("weight_dtype", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("enable_confidence_head", ctypes.c_int32), ("confidence_head_with_markov", ctypes.c_int32),
                ("confidence_threshold", ctypes.c_double), ("markov_head_rnn", ctypes.c_int32)]


class DraftArgs(ctypes.Structure):
    _fields_ = [("A", ctypes.c_int32), ("k_ctx_dev", ctypes.c_void_p), ("v_ctx_dev", ctypes.c_void_p),
                ("ctx_len_host", ctypes.c_void_p), ("ctx_pos0_host", ctypes.c_void_p),
                ("anchors_host", ctypes.c_void_p), ("positions_host", ctypes.c_void_p),
                ("thresholds_host", ctypes.c_void_p), ("tokens_dev", ctypes.c_void_p),
                ("logits_dev", ctypes.c_void_p), ("conf_dev", ctypes.c_void_p), ("lengths_dev", ctypes.c_void_p),
                ("aux_dev", ctypes.c_void_p), ("temperature", ctypes.c_float), ("seeds_host", ctypes.c_void_p)]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("launches", ctypes.c_int32), ("ms", ctypes.c_double)]


class Weight(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("dtype", ctypes.c_int32), ("data", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64)]


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libdspark.so (or `path`); raises if it is not built (no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run block_draft_model_dspark_amd/build.py")
    lib = ctypes.CDLL(path)
    P, I32, SZ, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_int64
    lib.dspark_model_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weight), ctypes.c_int,
                                        ctypes.POINTER(P)]
    lib.dspark_model_destroy.argtypes = [P]
    lib.dspark_model_destroy.restype = None
    lib.dspark_model_set_tall_rows.argtypes = [P, ctypes.c_int]
    lib.dspark_model_aux_bytes.argtypes = [P]
    lib.dspark_model_aux_bytes.restype = SZ
    lib.dspark_model_prepare.argtypes = [P, P, SZ, P]
    lib.dspark_project_workspace_bytes.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.dspark_project_workspace_bytes.restype = SZ
    lib.dspark_project_context_kv.argtypes = [P, ctypes.c_int, P, ctypes.c_int, ctypes.c_int,
                                              ctypes.POINTER(I32), ctypes.POINTER(P), ctypes.POINTER(P), P, SZ, P]
    lib.dspark_draft_workspace_bytes.argtypes = [P, ctypes.c_int, ctypes.c_int, I64]
    lib.dspark_draft_workspace_bytes.restype = SZ
    lib.dspark_draft_rows.argtypes = [P, ctypes.c_int, ctypes.POINTER(P), ctypes.POINTER(P), ctypes.POINTER(I32),
                                      ctypes.POINTER(I32), ctypes.POINTER(I32), P, P, P, P, SZ, P]
    lib.dspark_draft_block.argtypes = [P, ctypes.POINTER(P), ctypes.POINTER(P), I32, I32, I32, P, P, P, P, SZ, P]
    lib.dspark_draft_rows_noalloc.argtypes = [P, ctypes.c_int, ctypes.POINTER(P), ctypes.POINTER(P),
                                              ctypes.POINTER(I32), ctypes.POINTER(I32), ctypes.POINTER(I32), P, P, P,
                                              P]
    lib.dspark_draft_rows_conf.argtypes = [P, ctypes.c_int, ctypes.POINTER(P), ctypes.POINTER(P),
                                           ctypes.POINTER(I32), ctypes.POINTER(I32), ctypes.POINTER(I32),
                                           ctypes.POINTER(ctypes.c_float), P, P, P, P, P, P, SZ, P]
    lib.dspark_draft_rows_ex.argtypes = [P, ctypes.POINTER(DraftArgs), P, SZ, P]
    lib.dspark_draft_noalloc_max_bytes.argtypes = []
    lib.dspark_draft_noalloc_max_bytes.restype = SZ
    lib.dspark_profile_enable.argtypes = [ctypes.c_int]
    lib.dspark_profile_enable.restype = None
    lib.dspark_profile_read.argtypes = [ctypes.POINTER(KernelTime), ctypes.c_int]
    lib.dspark_profile_read.restype = ctypes.c_int
    lib.dspark_tall_tile_of.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                        ctypes.POINTER(ctypes.c_int)]
    lib.dspark_tall_tile_of.restype = ctypes.c_int
    lib.dspark_stream_block_of.argtypes = [ctypes.c_int] * 6 + [ctypes.POINTER(ctypes.c_int)] * 3
    lib.dspark_stream_block_of.restype = ctypes.c_int
    lib.dspark_q4_address_check.argtypes = [ctypes.POINTER(Config), ctypes.c_int, ctypes.POINTER(ctypes.c_int32),
                                            I64, ctypes.c_int, ctypes.POINTER(I64)]
    lib.dspark_q4_address_check.restype = ctypes.c_int
    lib.dspark_last_error.argtypes = []
    lib.dspark_last_error.restype = ctypes.c_char_p
    for fn in ("dspark_model_create", "dspark_model_set_tall_rows", "dspark_model_prepare",
               "dspark_project_context_kv", "dspark_draft_rows", "dspark_draft_block", "dspark_draft_rows_noalloc",
               "dspark_draft_rows_conf", "dspark_draft_rows_ex"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        raise DsparkError(status, _lib.dspark_last_error().decode())


def _stream_handle(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _keep_for(stream, *tensors) -> None:
    """Tensors allocated on the current stream but read or written by work
    enqueued on another `stream`: tell PyTorch's caching allocator not to
    hand their memory out again before that stream's work is done."""
    if stream is None:
        return
    import torch
    if stream == torch.cuda.current_stream():
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _torch_dtype(kind: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[kind]


def upload(stored: Dict[str, object], device="cuda") -> Dict[str, dict]:
    """Stored tensors (kind, shape, data, scales, biases) -> device tensors."""
    import torch
    out = {}
    for name, st in stored.items():
        if st.kind == "f32":
            d = torch.from_numpy(np.ascontiguousarray(st.data)).to(device)
            out[name] = {"kind": "f32", "data": d, "shape": st.shape}
        elif st.kind == "bf16":
            d = torch.from_numpy(np.ascontiguousarray(st.data).view(np.int16)).to(device).view(torch.bfloat16)
            out[name] = {"kind": "bf16", "data": d, "shape": st.shape}
        else:
            d = torch.from_numpy(np.ascontiguousarray(st.data).view(np.int32)).to(device)
            s = torch.from_numpy(np.ascontiguousarray(st.scales).view(np.int16)).to(device).view(torch.bfloat16)
            b = torch.from_numpy(np.ascontiguousarray(st.biases).view(np.int16)).to(device).view(torch.bfloat16)
            out[name] = {"kind": "q4", "data": d, "scales": s, "biases": b, "shape": st.shape}
    return out


def act_tensor(st, device="cuda"):
    """A stored activation (f32 or bf16) -> device tensor of the same shape."""
    import torch
    if st.kind == "f32":
        return torch.from_numpy(np.ascontiguousarray(st.data)).to(device)
    return torch.from_numpy(np.ascontiguousarray(st.data).view(np.int16)).to(device).view(torch.bfloat16)


def make_config(cfg, with_fc: bool) -> Config:
    """The library's config struct for a model config (fc / hidden_norm present
    or not)."""
    c = Config()
    c.hidden_size = cfg.hidden_size
    c.num_hidden_layers = cfg.num_hidden_layers
    c.num_attention_heads = cfg.num_attention_heads
    c.global_head_dim = cfg.global_head_dim
    c.num_global_key_value_heads = cfg.num_global_key_value_heads
    c.intermediate_size = cfg.intermediate_size
    c.vocab_size = cfg.vocab_size
    c.block_size = cfg.block_size
    c.mask_token_id = cfg.mask_token_id
    c.markov_rank = cfg.markov_rank
    c.attention_k_eq_v = int(getattr(cfg, "attention_k_eq_v", True))
    c.markov_head_vanilla = int(getattr(cfg, "markov_head_type", "vanilla") == "vanilla")
    c.activation_gelu_tanh = int(getattr(cfg, "hidden_activation", "gelu_pytorch_tanh") == "gelu_pytorch_tanh")
    c.fc_in = cfg.num_taps * cfg.target_hidden_size if with_fc else 0
    c.rope_theta = cfg.rope_theta
    c.partial_rotary_factor = cfg.partial_rotary_factor
    c.rms_norm_eps = cfg.rms_norm_eps
    c.final_logit_softcapping = cfg.final_logit_softcapping or 0.0
    c.weight_dtype = _KIND[cfg.weight_dtype]
    c.act_dtype = _KIND[cfg.act_dtype]
    c.group_size = cfg.group_size
    c.enable_confidence_head = int(bool(getattr(cfg, "enable_confidence_head", False)))
    c.confidence_head_with_markov = int(bool(getattr(cfg, "confidence_head_with_markov", False)))
    c.confidence_threshold = float(getattr(cfg, "confidence_threshold", 0.0) or 0.0)
    c.markov_head_rnn = int(getattr(cfg, "markov_head_type", "vanilla") == "rnn")
    return c


class Model:
    """A drafter whose weights live in device tensors owned by this object."""

    def __init__(self, cfg, weights: Dict[str, dict]):
        lib = load_library()
        self.cfg = cfg
        self.weights = weights  # keeps the device tensors alive
        c = make_config(cfg, "fc.weight" in weights)
        self._c = c
        names = list(weights)
        self._names = [n.encode() for n in names]
        table = (Weight * len(names))()
        for i, n in enumerate(names):
            w = weights[n]
            shape = w["shape"]
            table[i].name = self._names[i]
            table[i].dtype = _KIND[w["kind"]]
            table[i].data = w["data"].data_ptr()
            table[i].scales = _ptr(w.get("scales"))
            table[i].biases = _ptr(w.get("biases"))
            table[i].rows = shape[0]
            table[i].cols = shape[1] if len(shape) > 1 else 1
        h = ctypes.c_void_p()
        _check(lib.dspark_model_create(ctypes.byref(c), table, len(names), ctypes.byref(h)))
        self.handle = h
        self.aux = None

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.dspark_model_destroy(self.handle)
            self.handle = None

    def prepare(self, stream=None):
        import torch
        n = _lib.dspark_model_aux_bytes(self.handle)
        self.aux = torch.empty(n, dtype=torch.uint8, device="cuda")
        _check(_lib.dspark_model_prepare(self.handle, self.aux.data_ptr(), n, _stream_handle(stream)))
        _keep_for(stream, self.aux)
        return self

    def set_tall_rows(self, rows: int):
        """GEMMs over >= rows activation rows take the tiled MFMA path (0: never)."""
        _check(_lib.dspark_model_set_tall_rows(self.handle, int(rows)))
        return self

    @property
    def act_dtype(self):
        return _torch_dtype(self.cfg.act_dtype)


def profile_enable(on: bool = True) -> None:
    """Bracket every library kernel launch with HIP events (timing only)."""
    load_library().dspark_profile_enable(int(on))


def profile_read() -> Dict[str, tuple]:
    """{kernel role: (launches, total ms)} since the last read."""
    buf = (KernelTime * 64)()
    n = load_library().dspark_profile_read(buf, 64)
    return {buf[i].name.decode(): (buf[i].launches, buf[i].ms) for i in range(n)}


def project_workspace_bytes(model: Model, input_kind: int, B: int, L: int) -> int:
    return int(_lib.dspark_project_workspace_bytes(model.handle, input_kind, B, L))


def draft_workspace_bytes(model: Model, A: int, max_ctx: int, total_ctx: int) -> int:
    return int(_lib.dspark_draft_workspace_bytes(model.handle, A, max_ctx, total_ctx))


def project_context_kv(model: Model, x, pos0: Sequence[int], input_kind: int = INPUT_CONTEXT_HIDDEN,
                       k_out=None, v_out=None, workspace=None, stream=None, v_only: bool = False):
    """deepspec.ts, #projectContextKVRows.  x [B, L, H] (or [B, L, fc_in] for
    target features), act dtype, on the GPU.  Returns per-layer (K, V) lists,
    each [B, nKv, L, hd]; with v_only the K list is None (a V-only cache)."""
    import torch
    cfg = model.cfg
    B, L = int(x.shape[0]), int(x.shape[1])
    nL = cfg.num_hidden_layers
    if v_out is None:
        v_out = [torch.empty(B, cfg.nKv, L, cfg.hd, dtype=model.act_dtype, device=x.device) for _ in range(nL)]
    if k_out is None and not v_only:
        k_out = [torch.empty(B, cfg.nKv, L, cfg.hd, dtype=model.act_dtype, device=x.device) for _ in range(nL)]
    if v_only:
        k_out = None
    n = project_workspace_bytes(model, input_kind, B, L)
    if workspace is None or workspace.numel() < n:
        workspace = torch.empty(n, dtype=torch.uint8, device=x.device)
    pos = (ctypes.c_int32 * B)(*[int(p) for p in pos0])
    kp = None if k_out is None else (ctypes.c_void_p * nL)(*[t.data_ptr() for t in k_out])
    vp = (ctypes.c_void_p * nL)(*[t.data_ptr() for t in v_out])
    _check(_lib.dspark_project_context_kv(model.handle, input_kind, x.data_ptr(), B, L, pos, kp, vp,
                                          workspace.data_ptr(), n, _stream_handle(stream)))
    _keep_for(stream, workspace, *(k_out or []), *v_out)
    return k_out, v_out


class DraftCall:
    """Marshalled arguments of one dspark_draft_rows call, reusable so that a
    timing loop re-issues the same call without Python-side allocation."""

    def __init__(self, model: Model, k_rows, v_rows, ctx_lens: Sequence[int], anchors: Sequence[int],
                 positions: Sequence[int], collect_logits: bool = False, workspace=None, tokens=None):
        import torch
        cfg = model.cfg
        A = len(anchors)
        nL = cfg.num_hidden_layers
        self.model = model
        self.A = A
        self.keep = (k_rows, v_rows)
        self.kp = (ctypes.c_void_p * (nL * A))(*[k_rows[l][a].data_ptr() for l in range(nL) for a in range(A)])
        self.vp = (ctypes.c_void_p * (nL * A))(*[v_rows[l][a].data_ptr() for l in range(nL) for a in range(A)])
        self.lens = (ctypes.c_int32 * A)(*[int(v) for v in ctx_lens])
        self.anchors = (ctypes.c_int32 * A)(*[int(v) for v in anchors])
        self.positions = (ctypes.c_int32 * A)(*[int(v) for v in positions])
        self.tokens = tokens if tokens is not None else torch.empty(A, cfg.gamma, dtype=torch.int32, device="cuda")
        self.logits = (torch.empty(A, cfg.gamma, cfg.V, dtype=torch.float32, device="cuda")
                       if collect_logits else None)
        n = draft_workspace_bytes(model, A, max(ctx_lens), sum(ctx_lens))
        self.ws = workspace if workspace is not None and workspace.numel() >= n else torch.empty(
            n, dtype=torch.uint8, device="cuda")
        self.nbytes = n

    def __call__(self, stream=None):
        m = self.model
        _check(_lib.dspark_draft_rows(m.handle, self.A, self.kp, self.vp, self.lens, self.anchors, self.positions,
                                      self.tokens.data_ptr(), _ptr(self.logits),
                                      _ptr(m.aux), self.ws.data_ptr(), self.nbytes, _stream_handle(stream)))
        _keep_for(stream, self.ws, self.tokens, self.logits)
        return self.tokens


class DraftCallEx:
    """Marshalled arguments of one dspark_draft_rows_ex call (reusable, like
    DraftCall): k_rows None for a V-only cache; optional confidence outputs."""

    def __init__(self, model: Model, k_rows, v_rows, ctx_lens: Sequence[int], anchors: Sequence[int],
                 positions: Sequence[int], ctx_pos0: Optional[Sequence[int]] = None,
                 thresholds: Optional[Sequence[float]] = None, collect_logits: bool = False,
                 collect_conf: bool = False, lengths: bool = False, temperature: float = 0.0,
                 seeds: Optional[Sequence[int]] = None):
        import torch
        cfg = model.cfg
        A = len(anchors)
        nL = cfg.num_hidden_layers
        self.model = model
        self.keep_t = (k_rows, v_rows)
        self._keep = []

        def arr(ctype, vals):
            a = (ctype * len(vals))(*vals)
            self._keep.append(a)
            return ctypes.cast(a, ctypes.c_void_p)

        self.out = {"tokens": torch.empty(A, cfg.gamma, dtype=torch.int32, device="cuda"),
                    "logits": torch.empty(A, cfg.gamma, cfg.V, device="cuda") if collect_logits else None,
                    "conf": torch.empty(A, cfg.gamma, device="cuda") if collect_conf else None,
                    "lengths": torch.empty(A, dtype=torch.int32, device="cuda") if lengths else None}
        x = DraftArgs()
        x.A = A
        x.k_ctx_dev = None if k_rows is None else arr(ctypes.c_void_p, [k_rows[l][a].data_ptr() for l in range(nL)
                                                                        for a in range(A)])
        x.v_ctx_dev = arr(ctypes.c_void_p, [v_rows[l][a].data_ptr() for l in range(nL) for a in range(A)])
        x.ctx_len_host = arr(ctypes.c_int32, [int(v) for v in ctx_lens])
        x.ctx_pos0_host = None if ctx_pos0 is None else arr(ctypes.c_int32, [int(v) for v in ctx_pos0])
        x.anchors_host = arr(ctypes.c_int32, [int(v) for v in anchors])
        x.positions_host = arr(ctypes.c_int32, [int(v) for v in positions])
        x.thresholds_host = None if thresholds is None else arr(ctypes.c_float, [float(t) for t in thresholds])
        x.tokens_dev = self.out["tokens"].data_ptr()
        x.logits_dev = _ptr(self.out["logits"])
        x.conf_dev = _ptr(self.out["conf"])
        x.lengths_dev = _ptr(self.out["lengths"])
        x.aux_dev = _ptr(model.aux)
        x.temperature = float(temperature)
        x.seeds_host = None if seeds is None else arr(ctypes.c_uint64, [int(v) for v in seeds])
        self.args = x
        self.nbytes = draft_workspace_bytes(model, A, max(ctx_lens), sum(ctx_lens))
        self.ws = torch.empty(self.nbytes, dtype=torch.uint8, device="cuda")

    def __call__(self, stream=None):
        _check(_lib.dspark_draft_rows_ex(self.model.handle, ctypes.byref(self.args), self.ws.data_ptr(), self.nbytes,
                                         _stream_handle(stream)))
        _keep_for(stream, self.ws, *[t for t in self.out.values() if t is not None])
        return self.out


def draft_rows(model: Model, k_rows, v_rows, ctx_lens: Sequence[int], anchors: Sequence[int],
               positions: Sequence[int], collect_logits: bool = False, stream=None):
    """deepspec.ts, draftRows.  k_rows[l][a], v_rows[l][a]: row a's layer-l
    context K/V [nKv, ctx_len[a], hd] on the GPU.  Returns (tokens [A, gamma]
    int32 on the GPU, logits [A, gamma, V] fp32 or None)."""
    call = DraftCall(model, k_rows, v_rows, ctx_lens, anchors, positions, collect_logits)
    call(stream)
    return call.tokens, call.logits


def draft_rows_conf(model: Model, k_rows, v_rows, ctx_lens: Sequence[int], anchors: Sequence[int],
                    positions: Sequence[int], thresholds: Optional[Sequence[float]] = None,
                    collect_logits: bool = False, collect_conf: bool = True, stream=None):
    """deepspec.ts, draftRows with the confidence head: returns a dict of
    device tensors tokens [A, gamma] (the whole block), lengths [A] (each
    row's confident prefix), conf [A, gamma] (when collect_conf) and logits
    [A, gamma, V] (when collect_logits).  thresholds: gamma per-slot values,
    or None for the config's confidence_threshold."""
    import torch
    cfg = model.cfg
    A = len(anchors)
    nL = cfg.num_hidden_layers
    kp = (ctypes.c_void_p * (nL * A))(*[k_rows[l][a].data_ptr() for l in range(nL) for a in range(A)])
    vp = (ctypes.c_void_p * (nL * A))(*[v_rows[l][a].data_ptr() for l in range(nL) for a in range(A)])
    lens = (ctypes.c_int32 * A)(*[int(v) for v in ctx_lens])
    anc = (ctypes.c_int32 * A)(*[int(v) for v in anchors])
    pos = (ctypes.c_int32 * A)(*[int(v) for v in positions])
    thr = None if thresholds is None else (ctypes.c_float * cfg.gamma)(*[float(t) for t in thresholds])
    out = {"tokens": torch.empty(A, cfg.gamma, dtype=torch.int32, device="cuda"),
           "lengths": torch.empty(A, dtype=torch.int32, device="cuda")}
    out["conf"] = torch.empty(A, cfg.gamma, dtype=torch.float32, device="cuda") if collect_conf else None
    out["logits"] = torch.empty(A, cfg.gamma, cfg.V, dtype=torch.float32, device="cuda") if collect_logits else None
    n = draft_workspace_bytes(model, A, max(ctx_lens), sum(ctx_lens))
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    _check(_lib.dspark_draft_rows_conf(model.handle, A, kp, vp, lens, anc, pos, thr, out["tokens"].data_ptr(),
                                       _ptr(out["logits"]), _ptr(out["conf"]), out["lengths"].data_ptr(),
                                       _ptr(model.aux), ws.data_ptr(), n, _stream_handle(stream)))
    _keep_for(stream, ws, *[t for t in out.values() if t is not None])
    return out


def draft_rows_ex(model: Model, k_rows, v_rows, ctx_lens: Sequence[int], anchors: Sequence[int],
                  positions: Sequence[int], ctx_pos0: Optional[Sequence[int]] = None,
                  thresholds: Optional[Sequence[float]] = None, collect_logits: bool = False,
                  collect_conf: bool = False, lengths: bool = False, temperature: float = 0.0,
                  seeds: Optional[Sequence[int]] = None, stream=None):
    """deepspec.ts, draftRows through dspark_draft_rows_ex.  k_rows None: a
    V-only context cache (v_rows[l][a] only; the attention rebuilds the keys
    at positions ctx_pos0[a] + j).  temperature > 0 samples with the rows'
    key streams (seeds).  Returns a dict of device tensors: tokens, and
    logits / conf / lengths when asked for (None otherwise)."""
    return DraftCallEx(model, k_rows, v_rows, ctx_lens, anchors, positions, ctx_pos0, thresholds, collect_logits,
                       collect_conf, lengths, temperature, seeds)(stream)


def draft_rows_noalloc(model: Model, k_rows, v_rows, ctx_lens: Sequence[int], anchors: Sequence[int],
                       positions: Sequence[int], tokens, logits=None, stream=None):
    """draft_rows on the library's fixed per-GPU scratch array instead of a
    workspace (for callers that cannot allocate): the caller passes the
    outputs, tokens [A, gamma] int32 and optionally logits [A, gamma, V]
    fp32, both on the GPU.  Calls that overlap on one GPU race."""
    cfg = model.cfg
    A = len(anchors)
    nL = cfg.num_hidden_layers
    kp = (ctypes.c_void_p * (nL * A))(*[k_rows[l][a].data_ptr() for l in range(nL) for a in range(A)])
    vp = (ctypes.c_void_p * (nL * A))(*[v_rows[l][a].data_ptr() for l in range(nL) for a in range(A)])
    lens = (ctypes.c_int32 * A)(*[int(v) for v in ctx_lens])
    anc = (ctypes.c_int32 * A)(*[int(v) for v in anchors])
    pos = (ctypes.c_int32 * A)(*[int(v) for v in positions])
    _check(_lib.dspark_draft_rows_noalloc(model.handle, A, kp, vp, lens, anc, pos, tokens.data_ptr(), _ptr(logits),
                                          _ptr(model.aux), _stream_handle(stream)))
    return tokens, logits


def q4_address_check(cfg, A: int, anchors: Sequence[int], ctx_rows: int, input_kind: int = INPUT_CONTEXT_HIDDEN,
                     with_fc: bool = False) -> int:
    """Host replay of every 4-bit address a round and projection of these
    sizes form (dspark_q4_address_check); returns the number checked and
    raises DsparkError naming the first address out of range."""
    lib = load_library()
    c = make_config(cfg, with_fc)
    an = (ctypes.c_int32 * A)(*anchors)
    n = ctypes.c_int64()
    _check(lib.dspark_q4_address_check(ctypes.byref(c), A, an, ctx_rows, input_kind, ctypes.byref(n)))
    return n.value


def draft_noalloc_max_bytes() -> int:
    return int(load_library().dspark_draft_noalloc_max_bytes())


def draft_block(model: Model, k_ctx, v_ctx, anchor: int, position: int, collect_logits: bool = True,
                stream=None):
    """deepspec-module.ts, draftBlock: one row.  k_ctx[l], v_ctx[l]:
    [nKv, ctx_len, hd].  Returns (tokens [gamma], logits [gamma, V] or None)."""
    import torch
    cfg = model.cfg
    nL = cfg.num_hidden_layers
    L = int(k_ctx[0].shape[1])
    tokens = torch.empty(cfg.gamma, dtype=torch.int32, device="cuda")
    logits = torch.empty(cfg.gamma, cfg.V, dtype=torch.float32, device="cuda") if collect_logits else None
    n = draft_workspace_bytes(model, 1, L, L)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    kp = (ctypes.c_void_p * nL)(*[t.data_ptr() for t in k_ctx])
    vp = (ctypes.c_void_p * nL)(*[t.data_ptr() for t in v_ctx])
    _check(_lib.dspark_draft_block(model.handle, kp, vp, L, int(anchor), int(position), tokens.data_ptr(),
                                   _ptr(logits), _ptr(model.aux), ws.data_ptr(), n, _stream_handle(stream)))
    _keep_for(stream, ws, tokens, logits)
    return tokens, logits
