"""Thin ctypes binding of libofa.so (include/ofa.h), same names as the C ABI.

Argument marshalling only: every step of the method runs in the HIP kernels of
the library.  PyTorch is used for device memory and the stream.  Importing this
module fails loudly when libofa.so has not been built.
"""

from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libofa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m persistent_transformer_train_amd.build` "
        "(there is no CPU or PyTorch fallback)")

_lib = C.CDLL(LIB_PATH)

OFA_OK, OFA_E_ARG, OFA_E_HIP, OFA_E_NONFINITE, OFA_E_TIMEOUT, OFA_E_OVERFLOW, OFA_E_STATE = 0, -1, -2, -3, -4, -5, -6
OFA_DEBUG_SHUFFLE_TICKETS, OFA_DEBUG_SHORT_WATCHDOG, OFA_DEBUG_TRACE, OFA_DEBUG_TILE256, OFA_DEBUG_OCC1 = 1, 2, 4, 8, 16
OFA_DEBUG_PLAIN_TILES, OFA_DEBUG_WG_RELEASE, OFA_DEBUG_CE_UNFUSED = 32, 64, 128
OFA_TRACE_INSTANCES = 1024


class ofa_config(C.Structure):
    _fields_ = [
        ("n_layer", C.c_int32), ("d_model", C.c_int32), ("n_head", C.c_int32), ("d_ff", C.c_int32),
        ("vocab", C.c_int32), ("n_pos", C.c_int32),
        ("mlp_gated", C.c_int32), ("tied_head", C.c_int32), ("has_bias", C.c_int32),
        ("batch", C.c_int32), ("seq", C.c_int32), ("precision", C.c_int32),
        ("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float), ("eps", C.c_float),
        ("weight_decay", C.c_float),
        ("lr_schedule", C.c_int32), ("total_steps", C.c_int32),
        ("train_cus", C.c_int32), ("serve_cus", C.c_int32),
        ("decode_window", C.c_int32), ("prompt_len", C.c_int32), ("restart_every", C.c_int32),
        ("exec_mode", C.c_int32),
        ("debug_counter_base", C.c_uint64), ("debug_flags", C.c_int32),
        ("decode_batch", C.c_int32), ("reserved", C.c_int32 * 6),
    ]


class ofa_checkpoint_header(C.Structure):
    _fields_ = [
        ("magic", C.c_char * 8), ("n_params", C.c_uint64), ("steps_done", C.c_uint64), ("version", C.c_uint64),
        ("model_sha256", C.c_uint8 * 32), ("parent_sha256", C.c_uint8 * 32), ("note", C.c_uint8 * 32),
        ("reserved", C.c_uint8 * 128),
    ]


class ofa_stats(C.Structure):
    _fields_ = [
        ("status", C.c_int32), ("err_phase", C.c_int32), ("err_step", C.c_int64), ("err_info", C.c_int64),
        ("tickets_claimed", C.c_uint64), ("steps_done", C.c_uint64), ("version", C.c_uint64),
        ("last_call_ms", C.c_double), ("n_phases", C.c_int32), ("n_tiles_step", C.c_int32),
        ("grid", C.c_int32), ("n_tickets_step", C.c_int32), ("reserved", C.c_int32 * 4),
    ]


_H = C.c_void_p
_P = C.c_void_p
_sig = {
    "ofa_workspace_bytes": (C.c_size_t, [C.POINTER(ofa_config)]),
    "ofa_validate_config": (C.c_int, [C.POINTER(ofa_config), C.c_char_p, C.c_size_t]),
    "ofa_param_count": (C.c_int64, [C.POINTER(ofa_config)]),
    "ofa_param_tensor_count": (C.c_int32, [C.POINTER(ofa_config)]),
    "ofa_param_tensor": (C.c_int, [C.POINTER(ofa_config), C.c_int32, C.POINTER(C.c_int64), C.POINTER(C.c_int64),
                                   C.POINTER(C.c_int32), C.c_char_p, C.c_size_t]),
    "ofa_create": (C.c_int, [C.POINTER(ofa_config), _P, C.c_size_t, _P, _P, C.POINTER(_H)]),
    "ofa_create_static": (C.c_int, [C.POINTER(ofa_config), _P, _P, C.POINTER(_H)]),
    "ofa_train_step": (C.c_int, [_H, _P, C.c_int32, _P]),
    "ofa_publish_weights": (C.c_int, [_H, C.POINTER(C.c_uint64)]),
    "ofa_decode_token": (C.c_int, [_H, _P, C.c_int32, C.c_int32, _P, _P, _P]),
    "ofa_train_and_serve": (C.c_int, [_H, _P, C.c_int32, _P, _P, C.c_int32, _P, _P, C.c_int32, _P]),
    "ofa_decode_doorbell": (C.c_int, [_H, _P, C.c_int32, C.c_int32, _P, C.POINTER(C.c_double),
                                      C.POINTER(C.c_double)]),
    "ofa_get_params": (C.c_int, [_H, _P]),
    "ofa_set_params": (C.c_int, [_H, _P]),
    "ofa_get_grads": (C.c_int, [_H, _P]),
    "ofa_status_sync": (C.c_int, [_H, C.POINTER(ofa_stats)]),
    "ofa_phase_times": (C.c_int, [_H, C.POINTER(C.c_uint64), C.c_int32, C.POINTER(C.c_int32), C.c_char_p,
                                  C.c_size_t]),
    "ofa_decode_phase_times": (C.c_int, [_H, C.POINTER(C.c_uint64), C.c_int32, C.POINTER(C.c_int32), C.c_char_p,
                                         C.c_size_t]),
    "ofa_trace": (C.c_int, [_H, C.c_int32, C.POINTER(C.c_uint64), C.c_int64, C.POINTER(C.c_int64),
                            C.POINTER(C.c_int32)]),
    "ofa_task_budget": (C.c_int, [C.c_uint64, C.c_uint64, C.POINTER(C.c_uint64)]),
    "ofa_evaluate": (C.c_int, [_H, _P, C.c_int32, _P, _P, _P, C.c_int32, _P, _P]),
    "ofa_checkpoint_bytes": (C.c_size_t, [C.POINTER(ofa_config)]),
    "ofa_checkpoint_save": (C.c_int, [_H, _P, C.c_char_p, C.c_char_p]),
    "ofa_checkpoint_load": (C.c_int, [_H, _P, C.c_char_p]),
    "ofa_sha256": (C.c_int, [C.c_char_p, C.c_size_t, C.c_char_p]),
    "ofa_read_ceiling": (C.c_int, [C.c_int32, _P, C.c_int64, _P, C.c_int32, C.POINTER(C.c_double),
                                   C.POINTER(C.c_double)]),
    "ofa_sched_selftest": (C.c_int, [C.POINTER(ofa_config), C.c_int32, C.c_int32, C.c_int32, C.c_int64, C.c_uint64,
                                     C.c_int32, C.c_uint64, C.c_char_p, C.c_size_t]),
    "ofa_last_error": (C.c_char_p, [_H]),
    "ofa_status_string": (C.c_char_p, [C.c_int]),
    "ofa_destroy": (C.c_int, [_H]),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args
    globals()[_name] = _f

EXPORTED = tuple(_sig)


class OfaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ofa_status_string(code).decode()} ({code}): {msg}")
        self.code = code


def make_config(d: dict) -> ofa_config:
    c = ofa_config()
    for k, v in d.items():
        setattr(c, k, v)
    return c


def layout(cfg: ofa_config):
    """[(name, offset, numel, kind)] of the canonical parameter layout."""
    n = ofa_param_tensor_count(C.byref(cfg))
    if n < 0:
        buf = C.create_string_buffer(256)
        ofa_validate_config(C.byref(cfg), buf, 256)
        raise OfaError(OFA_E_ARG, buf.value.decode())
    out = []
    off, numel, kind = C.c_int64(), C.c_int64(), C.c_int32()
    name = C.create_string_buffer(64)
    kinds = {0: "normal", 1: "zeros", 2: "ones"}
    for i in range(n):
        ofa_param_tensor(C.byref(cfg), i, C.byref(off), C.byref(numel), C.byref(kind), name, 64)
        out.append((name.value.decode(), off.value, numel.value, kinds[kind.value]))
    return out


class Handle:
    """One model on one GPU: owns the torch-allocated workspace and the ofa handle."""

    # device -> the wrapper whose model the device's static handle holds: only that
    # wrapper retires it (an older wrapper of the same handle must not)
    _static_owner = {}

    def __init__(self, cfg_dict: dict, init_params, device="cuda:0", static=False):
        """static=True: ofa_create_static (the library's own workspace; no torch allocation
        of a workspace, and the device's one static handle is re-created)."""
        import torch
        self.torch = torch
        self.cfg_dict = dict(cfg_dict)
        self.cfg = make_config(cfg_dict)
        buf = C.create_string_buffer(256)
        if ofa_validate_config(C.byref(self.cfg), buf, 256) != OFA_OK:
            raise OfaError(OFA_E_ARG, buf.value.decode())
        self.device = torch.device(device)
        self.n_params = ofa_param_count(C.byref(self.cfg))
        init = torch.as_tensor(init_params, dtype=torch.float32).to(self.device).contiguous()
        assert init.numel() == self.n_params, (init.numel(), self.n_params)
        self.stream = torch.cuda.current_stream(self.device)
        self.h = _H()
        self.static = static
        if static:
            self.ws = None
            rc = ofa_create_static(C.byref(self.cfg), init.data_ptr(), self.stream.cuda_stream, C.byref(self.h))
            Handle._static_owner[self.device] = id(self)
        else:
            ws_bytes = ofa_workspace_bytes(C.byref(self.cfg))
            self.ws = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=self.device)
            base = self.ws.data_ptr()
            self.ws_ptr = (base + 255) // 256 * 256
            self.ws_bytes = ws_bytes
            rc = ofa_create(C.byref(self.cfg), self.ws_ptr, ws_bytes, init.data_ptr(), self.stream.cuda_stream,
                            C.byref(self.h))
        if rc != OFA_OK:
            msg = ofa_last_error(self.h).decode() if self.h.value else "create failed"
            raise OfaError(rc, msg)
        self.sync()
        del init

    # -- calls ---------------------------------------------------------------
    def _check(self, rc):
        if rc != OFA_OK:
            raise OfaError(rc, ofa_last_error(self.h).decode())

    def train_step(self, tokens, losses):
        """tokens: int32 cuda [n][B][T+1]; losses: float32 cuda [n]."""
        assert tokens.dtype == self.torch.int32 and tokens.is_cuda and tokens.is_contiguous()
        assert losses.dtype == self.torch.float32 and losses.is_cuda and losses.numel() >= tokens.shape[0]
        self._check(ofa_train_step(self.h, tokens.data_ptr(), tokens.shape[0], losses.data_ptr()))

    def publish(self) -> int:
        v = C.c_uint64()
        self._check(ofa_publish_weights(self.h, C.byref(v)))
        return v.value

    def decode(self, prompt, n_new, tokens_out, logits_out=None, versions_out=None):
        """prompt: int32 cuda [n_prompt], or [decode_batch][n_prompt] for several sequences
        (None continues); tokens_out [n_new] or [n_new][decode_batch]; logits_out
        [n_new][decode_batch][vocab]."""
        n_prompt = 0 if prompt is None else prompt.shape[-1]
        self._check(ofa_decode_token(self.h, 0 if prompt is None else prompt.data_ptr(), n_prompt, n_new,
                                     tokens_out.data_ptr(), 0 if logits_out is None else logits_out.data_ptr(),
                                     0 if versions_out is None else versions_out.data_ptr()))

    def decode_doorbell(self, prompt, n_new, tokens_out):
        """Batch-1 decode where each token waits for a host doorbell (rung inside the call);
        returns (ring-to-token microseconds on the host clock, wake-to-token microseconds on
        the device clock), one value per token."""
        host = (C.c_double * n_new)()
        dev = (C.c_double * n_new)()
        self._check(ofa_decode_doorbell(self.h, prompt.data_ptr(), prompt.shape[-1], n_new, tokens_out.data_ptr(),
                                        host, dev))
        return list(host), list(dev)

    def train_and_serve(self, tokens, losses, prompt, tokens_ring, versions_ring=None, n_generated=None):
        """Co-resident mode: train on tokens [n][B][T+1] on the train CUs while the
        serve CUs decode continuously from prompt (restarting every restart_every
        tokens); generated tokens go round-robin into tokens_ring, their weight
        versions into versions_ring, the count into n_generated (uint64 [1])."""
        assert tokens.dtype == self.torch.int32 and tokens.is_cuda and tokens.is_contiguous()
        assert losses.dtype == self.torch.float32 and losses.numel() >= tokens.shape[0]
        assert prompt.dtype == self.torch.int32 and tokens_ring.dtype == self.torch.int32
        self._check(ofa_train_and_serve(self.h, tokens.data_ptr(), tokens.shape[0], losses.data_ptr(),
                                        prompt.data_ptr(), prompt.numel(), tokens_ring.data_ptr(),
                                        0 if versions_ring is None else versions_ring.data_ptr(),
                                        tokens_ring.numel(), 0 if n_generated is None else n_generated.data_ptr()))

    def evaluate(self, tokens, losses, row_losses=None, probe_rows=None, probe_argmax=None, probe_entropy=None):
        """Forward-only scoring of tokens [n][B][T+1]: mean loss per batch into losses [n],
        per-row losses into row_losses [n][B*T], and at the flat rows probe_rows [k] the
        argmax token and prediction entropy into probe_argmax / probe_entropy [n][k]."""
        assert tokens.dtype == self.torch.int32 and tokens.is_cuda and tokens.is_contiguous()
        k = 0 if probe_rows is None else probe_rows.numel()
        p = lambda t: 0 if t is None else t.data_ptr()
        self._check(ofa_evaluate(self.h, tokens.data_ptr(), tokens.shape[0], losses.data_ptr(), p(row_losses),
                                 p(probe_rows), k, p(probe_argmax), p(probe_entropy)))

    def checkpoint_bytes(self) -> int:
        return ofa_checkpoint_bytes(C.byref(self.cfg))

    def checkpoint_save(self, dev_buf, note: bytes = None) -> bytes:
        """Training state into the uint8 device tensor dev_buf; returns its SHA-256."""
        assert dev_buf.is_cuda and dev_buf.numel() * dev_buf.element_size() >= self.checkpoint_bytes()
        out = C.create_string_buffer(32)
        self._check(ofa_checkpoint_save(self.h, dev_buf.data_ptr(), note, out))
        return out.raw

    def checkpoint_load(self, dev_buf) -> bytes:
        out = C.create_string_buffer(32)
        self._check(ofa_checkpoint_load(self.h, dev_buf.data_ptr(), out))
        return out.raw

    def get_params(self):
        out = self.torch.empty(self.n_params, dtype=self.torch.float32, device=self.device)
        self._check(ofa_get_params(self.h, out.data_ptr()))
        return out

    def set_params(self, p):
        p = p.to(self.device, self.torch.float32).contiguous()
        self._check(ofa_set_params(self.h, p.data_ptr()))
        self.sync()

    def get_grads(self):
        out = self.torch.empty(self.n_params, dtype=self.torch.float32, device=self.device)
        self._check(ofa_get_grads(self.h, out.data_ptr()))
        return out

    def sync(self) -> ofa_stats:
        st = ofa_stats()
        rc = ofa_status_sync(self.h, C.byref(st))
        self.last_stats = st
        self._check(rc)
        return st

    def phase_times(self, decode: bool = False):
        n = 512
        t = (C.c_uint64 * (2 * n))()
        names = C.create_string_buffer(32 * n)
        n_out = C.c_int32()
        fn = ofa_decode_phase_times if decode else ofa_phase_times
        self._check(fn(self.h, t, n, C.byref(n_out), names, 32))
        out = []
        for i in range(n_out.value):
            nm = names.raw[32 * i:32 * (i + 1)].split(b"\0", 1)[0].decode()
            out.append((nm, t[2 * i], t[2 * i + 1]))
        return out

    def trace(self, decode: bool = False):
        """(n_inst, n_phases, 4) device ticks of the last traced persistent call:
        first start, last start, last task end and last publication of every
        phase of every instance."""
        import numpy as np
        n = OFA_TRACE_INSTANCES * 512
        buf = (C.c_uint64 * (4 * n))()
        n_out, n_ph = C.c_int64(), C.c_int32()
        self._check(ofa_trace(self.h, 1 if decode else 0, buf, 2 * n, C.byref(n_out), C.byref(n_ph)))
        a = np.frombuffer(buf, dtype=np.uint64, count=4 * n_out.value).copy()
        return a.reshape(-1, n_ph.value, 4)

    def close(self):
        if self.h:
            if not getattr(self, "static", False) or Handle._static_owner.get(self.device) == id(self):
                ofa_destroy(self.h)
                Handle._static_owner.pop(self.device, None) if getattr(self, "static", False) else None
            self.h = _H()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def read_ceiling(n_wg: int, buf, sink, reps: int = 5):
    """ofa_read_ceiling over a device tensor buf (any dtype, only read) with a
    device int32 tensor sink of n_wg elements: (GB/s, fastest launch in us)."""
    g, us = C.c_double(), C.c_double()
    rc = ofa_read_ceiling(n_wg, C.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                          C.c_void_p(sink.data_ptr()), reps, C.byref(g), C.byref(us))
    if rc != OFA_OK:
        raise OfaError(rc, "read_ceiling")
    return g.value, us.value


def sha256(data: bytes) -> bytes:
    """The library's SHA-256 of a host byte string."""
    out = C.create_string_buffer(32)
    rc = ofa_sha256(data, len(data), out)
    if rc != OFA_OK:
        raise OfaError(rc, "sha256")
    return out.raw
