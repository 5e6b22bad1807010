"""Engine: one libspec context with a torch-owned workspace and stream."""

import numpy as np

from . import _lib as L


def make_config(model, max_requests=1, max_ctx=4096, max_nodes=17,
                max_rows=None, prefill_chunk=512, weight_format="native", kv_pages=0):
    """spec_config from a model-shape dict (keys as in synth.configs).
    weight_format: "native" (the model's dtype), "w12" or "w12_lowp" (W12 plus
    the 8-bit view read by verify(lowp=True)); the W12 formats need bf16.
    kv_pages: KV pool size in 16-token pages (0: every request at max_ctx)."""
    c = L.spec_config()
    c.n_layers = model["n_layers"]
    c.d_model = model["d_model"]
    c.n_heads = model["n_heads"]
    c.n_kv_heads = model["n_kv_heads"]
    c.head_dim = model["head_dim"]
    c.ffn_dim = model["ffn_dim"]
    c.vocab = model["vocab"]
    c.dtype = L.SPEC_DTYPE_BF16 if model["dtype"] == "bf16" else L.SPEC_DTYPE_FP32
    c.lr_state = model.get("lr_state", 0)
    for i, k in enumerate(model["layer_kinds"]):
        c.layer_kind[i] = L.SPEC_LAYER_LR if k == "L" else L.SPEC_LAYER_ATTN
    c.rms_eps = model["rms_eps"]
    c.rope_theta = model["rope_theta"]
    c.max_requests = max_requests
    c.max_ctx = max_ctx
    c.max_nodes = max_nodes
    c.max_rows = max_rows if max_rows is not None else max_nodes * max_requests
    c.prefill_chunk = prefill_chunk
    c.page_size = 16
    formats = {"native": L.SPEC_WEIGHTS_NATIVE, "w12": L.SPEC_WEIGHTS_W12,
               "w12_lowp": L.SPEC_WEIGHTS_W12_LOWP}
    if weight_format not in formats:
        raise ValueError(f"unknown weight format {weight_format!r}")
    c.weight_format = formats[weight_format]
    c.kv_pages = kv_pages
    return c


class Engine:
    """Owns a device workspace (a torch uint8 tensor), a HIP stream of its
    own (default priority; the library captures graphs on it) and a libspec
    context bound to that stream on `device`.  Every library call that hands
    results back synchronizes the stream first, so tensors it wrote may be
    read on torch's current stream afterwards."""

    def __init__(self, model, device=0, **caps):
        import torch
        L.lib()
        self.torch = torch
        self.model = model
        self.cfg = make_config(model, **caps)
        self.max_nodes = self.cfg.max_nodes
        self.device = torch.device("cuda", device)
        nbytes = L.spec_workspace_bytes(self.cfg)
        if nbytes == 0:
            raise ValueError("invalid spec_config")
        with torch.cuda.device(self.device):
            self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            self.stream = torch.cuda.Stream(device=self.device)
            torch.cuda.synchronize(self.device)
            self.ctx = L.spec_create(self.cfg, self.workspace.data_ptr(), nbytes,
                                     self.stream.cuda_stream)
        self.workspace_bytes = nbytes

    # -- weights -----------------------------------------------------------
    def load_weights(self, arrays):
        """arrays: weight tensors in tensor-id order (numpy float32, or
        uint16 bf16 bit patterns).  Each is staged on the device once."""
        torch = self.torch
        for tid, a in enumerate(arrays):
            a = np.ascontiguousarray(a)
            host = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
            dev = host.to(self.device, non_blocking=False)
            torch.cuda.synchronize(self.device)
            L.spec_load_weights(self.ctx, tid, dev.data_ptr(), a.nbytes, 1)
            del dev

    # -- decoding calls ----------------------------------------------------
    def prefill(self, req, prompt, logits=False):
        out = None
        if logits:
            out = self.torch.empty(self.model["vocab"], dtype=self.torch.float32,
                                   device=self.device)
        first = L.spec_prefill(self.ctx, req, [int(t) for t in prompt],
                               out.data_ptr() if out is not None else None)
        return (first, out) if logits else first

    def verify(self, reqs, drafts, parents, logits=False, lowp=False):
        """drafts/parents: one array per request.  Returns (paths, bonus
        [, logits tensor [rows, vocab]]).  The logits tensor is a view of one
        buffer owned by the engine (so repeated passes keep one launch
        shape): it is valid until the next verify.  lowp: the low-precision
        first round of two-level verification (accepts nothing)."""
        n_nodes = [len(d) for d in drafts]
        flat_d = [int(t) for d in drafts for t in d]
        flat_p = [int(p) for ps in parents for p in ps]
        out = None
        if logits:
            rows = sum(n + 1 for n in n_nodes)
            if getattr(self, "_logits", None) is None:
                self._logits = self.torch.empty((self.cfg.max_rows, self.model["vocab"]),
                                                dtype=self.torch.float32,
                                                device=self.device)
            out = self._logits[:rows]
        paths, bonus = L.spec_verify(self.ctx, list(reqs), n_nodes, flat_d, flat_p,
                                     self.max_nodes,
                                     out.data_ptr() if out is not None else None, lowp)
        return (paths, bonus, out) if logits else (paths, bonus)

    def commit(self, reqs, paths, next_roots):
        return L.spec_commit(self.ctx, list(reqs), paths, list(next_roots),
                             self.max_nodes)

    def release(self, req):
        return L.spec_release(self.ctx, req)

    def debug_flags(self, flags):
        L.spec_debug_flags(self.ctx, flags)

    def state(self, req):
        return L.spec_request_state(self.ctx, req)

    def force_root(self, req, token):
        return L.spec_force_root(self.ctx, req, token)

    def set_fault(self, token, bias, after_position):
        return L.spec_set_fault(self.ctx, token, bias, after_position)

    def use_graphs(self, enable):
        L.spec_use_graphs(self.ctx, enable)

    def timing(self, cls):
        L.spec_timing_enable(self.ctx, cls)

    def timing_read(self):
        return L.spec_timing_read(self.ctx)

    def close(self):
        if getattr(self, "ctx", None) is not None:
            L.spec_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
