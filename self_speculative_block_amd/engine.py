"""Python binding of the HIP engine: marshals arguments into the C ABI.

PyTorch only provides device memory (weights, KV page pool, prefixes,
logits buffers) and the current stream; every step of the decoding path
runs in the library's HIP kernels.  The calls mirror include/ssb.h.
"""

import ctypes

import numpy as np
import torch

from . import _lib as L

byref = ctypes.byref


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _i32(n):
    return (ctypes.c_int32 * max(n, 1))()


def torch_dtype(cfg):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


class Model:
    """A decoder on the GPU: packed weights plus the engine's fixed workspace."""

    def __init__(self, cfg, weights, block_B, max_rows=2048, max_positions=8192, device="cuda:0", max_batch=None,
                 sampling=True):
        """max_batch: requests per batched call (None: the library's limit); sampling: allocate the
        workspace of stochastic rounds."""
        self.lib = L.load()
        self.max_batch = max_batch or L.SSB_MAX_BATCH
        self.sampling = sampling
        self.cfg = cfg
        self.device = torch.device(device)
        self.block_B = block_B
        self.max_rows = max_rows
        self.max_positions = max_positions
        dt = torch_dtype(cfg)
        with torch.cuda.device(self.device):
            dev = lambda a, d=dt: torch.from_numpy(np.ascontiguousarray(a)).to(self.device).to(d)
            keep = []

            def put(name, d=dt):
                t = dev(weights[name], d)
                keep.append(t)
                return t.data_ptr()

            def arr(leaf, d=dt):
                return (ctypes.c_void_p * cfg.n_layers)(*[put(f"layers.{l}.{leaf}", d)
                                                          for l in range(cfg.n_layers)])

            w = L.SsbWeights()
            w.embed = put("embed")
            w.lm_head = put("lm_head")
            w.final_norm = put("final_norm", torch.float32)
            arrays = {k: arr(k, torch.float32 if k.endswith("norm") else dt)
                      for k in ("attn_norm", "mlp_norm", "wq", "wk", "wv", "wo", "wg", "wu", "wd")}
            for k, v in arrays.items():
                setattr(w, k, ctypes.cast(v, ctypes.POINTER(ctypes.c_void_p)))
            self.config = self.make_config(cfg, block_B, max_rows, max_positions, self.max_batch, sampling)
            h = ctypes.c_void_p()
            L.check(self.lib.ssb_init_model(byref(self.config), byref(w), _stream(), byref(h)))
            torch.cuda.current_stream().synchronize()
            del keep
        self.h = h

    @staticmethod
    def make_config(cfg, block_B, max_rows, max_positions, max_batch=0, sampling=False):
        c = L.SsbConfig()
        for k in ("n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim", "ffn", "vocab",
                  "mask_id", "eos_id"):
            setattr(c, k, getattr(cfg, k))
        c.block_B = block_B
        c.page_tokens = 16
        c.max_rows = max_rows
        c.max_positions = max_positions
        c.rms_eps = cfg.rms_eps
        c.rope_theta = cfg.rope_theta
        c.dtype = L.SSB_BF16 if cfg.dtype == "bf16" else L.SSB_F32
        c.max_batch = max_batch
        c.features = L.SSB_FEAT_SAMPLE if sampling else 0
        return c

    def prefix_tensor(self, prefix):
        """Upload prefix embeddings [P][hidden] in the model dtype."""
        return torch.from_numpy(np.ascontiguousarray(prefix, dtype=np.float32)).to(self.device).to(
            torch_dtype(self.cfg))

    def memory(self):
        """(packed weight bytes, workspace bytes) the model holds on the device."""
        wb, ws = ctypes.c_size_t(), ctypes.c_size_t()
        L.check(self.lib.ssb_model_memory(self.h, byref(wb), byref(ws)))
        return wb.value, ws.value

    def set_debug(self, poison, unfused=False):
        """poison: NaN-poison the KV slots no correct read reaches (window slots between draft and
        verify, rolled-back slots after accept); rounds then run without graph replay.
        unfused: run each layer's O, gate|up and down as three launches instead of the fused layer
        tail (bit-identical; a test and measurement switch)."""
        flags = (L.SSB_DEBUG_POISON if poison else 0) | (L.SSB_DEBUG_UNFUSED if unfused else 0)
        L.check(self.lib.ssb_set_debug(self.h, flags))

    def profile_kernel(self, kind, in_graph=False):
        """Start timing every launch of one kernel kind (name in KERNEL_KINDS), or stop (None).
        in_graph: rounds keep replaying launch graphs; a timed launch counts from the end of the launch
        before it to its own end (device real-time stamps)."""
        code = -1 if kind is None else L.KERNEL_KINDS[kind] | (L.SSB_PROFILE_IN_GRAPH if in_graph else 0)
        L.check(self.lib.ssb_profile_kernel(self.h, code))

    def profile_read(self, reset=True):
        us, n = ctypes.c_double(), ctypes.c_longlong()
        L.check(self.lib.ssb_profile_read(self.h, byref(us), byref(n), 1 if reset else 0))
        return us.value, n.value

    def close(self):
        if self.h:
            self.lib.ssb_free_model(self.h)
            self.h = None


class Pool:
    """KV page pool in a torch-owned device buffer."""

    def __init__(self, model, n_pages):
        self.model = model
        self.lib = model.lib
        nb = ctypes.c_size_t()
        L.check(self.lib.ssb_pool_bytes(model.h, n_pages, byref(nb)))
        self.buf = torch.empty(nb.value, dtype=torch.uint8, device=model.device)
        self.n_pages = n_pages
        h = ctypes.c_void_p()
        L.check(self.lib.ssb_pool_init(model.h, _ptr(self.buf), nb.value, n_pages, byref(h)))
        self.h = h

    def free_pages(self):
        n = ctypes.c_int()
        L.check(self.lib.ssb_pool_free_pages(self.h, byref(n)))
        return n.value

    def close(self):
        if self.h:
            self.lib.ssb_pool_free(self.h)
            self.h = None


class KV:
    """One sequence's KV cache and decode state."""

    def __init__(self, pool, max_tokens):
        self.pool = pool
        self.model = pool.model
        self.lib = pool.lib
        h = ctypes.c_void_p()
        L.check(self.lib.ssb_kv_create(pool.h, max_tokens, byref(h)))
        self.h = h

    def close(self):
        if self.h:
            self.lib.ssb_kv_free(self.h)
            self.h = None

    def reset(self):
        L.check(self.lib.ssb_kv_reset(self.h))

    def poison(self, lo, hi):
        """Debug: NaN into every layer's K and V at positions [lo, hi) of this kv's pages."""
        L.check(self.lib.ssb_kv_poison(self.h, lo, hi, _stream()))

    def rewind(self, n, x0):
        L.check(self.lib.ssb_kv_rewind(self.h, n, x0))

    def state(self):
        n, x0, pages = ctypes.c_int(), ctypes.c_int32(), ctypes.c_int()
        L.check(self.lib.ssb_kv_state(self.h, byref(n), byref(x0), byref(pages)))
        return n.value, x0.value, pages.value

    def prefill(self, prefix_dev):
        y = ctypes.c_int32()
        L.check(self.lib.ssb_prefill(self.model.h, self.h, _ptr(prefix_dev), prefix_dev.shape[0], byref(y),
                                     _stream()))
        return y.value

    def round(self, B, max_commit=None, planted_dev=None, want_logits=False):
        """One draft/verify/accept round; returns (committed, A, draft_logits, verify_logits)."""
        max_commit = B + 2 if max_commit is None else max_commit
        out = _i32(B + 2)
        n, A = ctypes.c_int32(), ctypes.c_int32()
        dl = vl = None
        if want_logits:
            V = self.model.cfg.vocab
            dl = torch.empty((B + 1, V), dtype=torch.float32, device=self.model.device)
            vl = torch.empty((B + 1, V), dtype=torch.float32, device=self.model.device)
        L.check(self.lib.ssb_round(self.model.h, self.h, B, max_commit, _ptr(planted_dev), out, byref(n),
                                   byref(A), _ptr(dl), _ptr(vl), _stream()))
        return list(out[: n.value]), A.value, dl, vl

    def round_noalloc(self, B, max_commit=None, planted_dev=None):
        """ssb_round_noalloc: the same round with its workspace in the library's scratch array."""
        max_commit = B + 2 if max_commit is None else max_commit
        out = _i32(B + 2)
        n = ctypes.c_int32()
        A = ctypes.c_int32()
        L.check(self.lib.ssb_round_noalloc(self.model.h, self.h, B, max_commit, _ptr(planted_dev), out, byref(n),
                                           byref(A), _stream()))
        return list(out[: n.value]), A.value

    def ar_step(self, want_logits=False):
        y = ctypes.c_int32()
        lg = None
        if want_logits:
            lg = torch.empty((self.model.cfg.vocab,), dtype=torch.float32, device=self.model.device)
        L.check(self.lib.ssb_ar_step(self.model.h, self.h, byref(y), _ptr(lg), _stream()))
        return y.value, lg

    def forward_tokens(self, tokens, p, want_logits=False):
        M = len(tokens)
        toks = (ctypes.c_int32 * M)(*[int(t) for t in tokens])
        am = _i32(M)
        t1 = (ctypes.c_float * M)()
        t2 = (ctypes.c_float * M)()
        lg = None
        if want_logits:
            lg = torch.empty((M, self.model.cfg.vocab), dtype=torch.float32, device=self.model.device)
        L.check(self.lib.ssb_forward_tokens(self.model.h, self.h, toks, M, p, _ptr(lg), am, t1, t2, _stream()))
        return list(am[:M]), np.array(t1[:M]), np.array(t2[:M]), lg

    def decode(self, prefix_dev, B, max_len, cont_dev=None, astar=None):
        out = _i32(max_len)
        n = ctypes.c_int32()
        st = L.SsbStats()
        na = 0 if astar is None else len(astar)
        astar_c = (ctypes.c_int32 * max(na, 1))(*([int(a) for a in astar] if astar is not None else [0]))
        L.check(self.lib.ssb_decode(self.model.h, self.h, _ptr(prefix_dev), prefix_dev.shape[0], B, max_len,
                                    _ptr(cont_dev), 0 if cont_dev is None else cont_dev.shape[0],
                                    astar_c if na else None, na, out, byref(n), byref(st), _stream()))
        return list(out[: n.value]), st

    def decode_ar(self, prefix_dev, max_len):
        out = _i32(max_len)
        n = ctypes.c_int32()
        st = L.SsbStats()
        L.check(self.lib.ssb_decode_ar(self.model.h, self.h, _ptr(prefix_dev), prefix_dev.shape[0], max_len, out,
                                       byref(n), byref(st), _stream()))
        return list(out[: n.value]), st


    def round_sample(self, B, u_dev, temperature=1.0, max_commit=None, want_logits=False):
        """One stochastic round driven by the device uniforms u_dev [2B+2];
        returns (committed, A, draft_logits, verify_logits)."""
        max_commit = B + 2 if max_commit is None else max_commit
        out = _i32(B + 2)
        n, A = ctypes.c_int32(), ctypes.c_int32()
        dl = vl = None
        if want_logits:
            V = self.model.cfg.vocab
            dl = torch.empty((B + 1, V), dtype=torch.float32, device=self.model.device)
            vl = torch.empty((B + 1, V), dtype=torch.float32, device=self.model.device)
        L.check(self.lib.ssb_round_sample(self.model.h, self.h, B, max_commit, float(temperature), _ptr(u_dev), out,
                                          byref(n), byref(A), _ptr(dl), _ptr(vl), _stream()))
        return list(out[: n.value]), A.value, dl, vl

    def decode_sample(self, prefix_dev, B, max_len, u_dev, temperature=1.0):
        out = _i32(max(max_len, 1))
        n = ctypes.c_int32()
        st = L.SsbStats()
        L.check(self.lib.ssb_decode_sample(self.model.h, self.h, _ptr(prefix_dev), prefix_dev.shape[0], B,
                                           float(temperature), max_len, _ptr(u_dev), u_dev.shape[0], out, byref(n),
                                           byref(st), _stream()))
        return list(out[: n.value]), st

    def decode_ar_sample(self, prefix_dev, max_len, u_dev, temperature=1.0):
        out = _i32(max(max_len, 1))
        n = ctypes.c_int32()
        st = L.SsbStats()
        L.check(self.lib.ssb_decode_ar_sample(self.model.h, self.h, _ptr(prefix_dev), prefix_dev.shape[0],
                                              float(temperature), max_len, _ptr(u_dev), out, byref(n), byref(st),
                                              _stream()))
        return list(out[: n.value]), st

    def round_multistep(self, B, steps, tau, max_commit=None, want_logits=False):
        """Greedy round with a draft schedule of at most `steps` forwards;
        returns (committed, A, draft_forwards, verify_logits)."""
        max_commit = B + 2 if max_commit is None else max_commit
        out = _i32(B + 2)
        n, A, k = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        vl = None
        if want_logits:
            vl = torch.empty((B + 1, self.model.cfg.vocab), dtype=torch.float32, device=self.model.device)
        L.check(self.lib.ssb_round_multistep(self.model.h, self.h, B, steps, float(tau), max_commit, out, byref(n),
                                             byref(A), byref(k), _ptr(vl), _stream()))
        return list(out[: n.value]), A.value, k.value, vl

    def decode_multistep(self, prefix_dev, B, steps, tau, max_len):
        out = _i32(max(max_len, 1))
        n = ctypes.c_int32()
        st = L.SsbStats()
        L.check(self.lib.ssb_decode_multistep(self.model.h, self.h, _ptr(prefix_dev), prefix_dev.shape[0], B, steps,
                                              float(tau), max_len, out, byref(n), byref(st), _stream()))
        return list(out[: n.value]), st

    def dd_block(self, B, tau, max_commit=None, write_cache=True, want_steps=False, want_logits=False):
        """One direct block-diffusion block.

        Returns (tokens, n_out, steps, extra): the B block tokens, how many of
        them belong to the output (EOS / budget cut), the denoising forwards,
        and, if asked, a dict with step_of, per-step confidences and greedy
        tokens of rows 0..B-1, and per-step logits.
        """
        max_commit = B if max_commit is None else max_commit
        toks, step_of = _i32(B), _i32(B)
        n, steps = ctypes.c_int32(), ctypes.c_int32()
        conf = (ctypes.c_float * (B * B))() if want_steps else None
        stok = _i32(B * B) if want_steps else None
        lg = None
        if want_logits:
            lg = torch.full((B, B + 1, self.model.cfg.vocab), float("nan"), dtype=torch.float32,
                            device=self.model.device)
        L.check(self.lib.ssb_dd_block(self.model.h, self.h, B, float(tau), max_commit, 1 if write_cache else 0,
                                      toks, byref(n), byref(steps), step_of, conf, stok, _ptr(lg), _stream()))
        extra = None
        if want_steps or want_logits:
            k = steps.value
            extra = {"step_of": list(step_of[:B])}
            if want_steps:
                extra["conf"] = np.array(conf[: k * B], dtype=np.float32).reshape(k, B)
                extra["tok"] = np.array(stok[: k * B], dtype=np.int64).reshape(k, B)
            if want_logits:
                extra["logits"] = lg[:k]
        return list(toks[:B]), n.value, steps.value, extra

    def decode_dd(self, prefix_dev, B, tau, max_len):
        out = _i32(max(max_len, 1))
        n = ctypes.c_int32()
        st = L.SsbStats()
        L.check(self.lib.ssb_decode_dd(self.model.h, self.h, _ptr(prefix_dev), prefix_dev.shape[0], B, float(tau),
                                       max_len, out, byref(n), byref(st), _stream()))
        return list(out[: n.value]), st


def round_batch(model, kvs, B, max_commit, planted_dev=None, want_logits=False):
    """One batched round over R requests; returns [(committed, A)] per request, and with
    want_logits also the draft and verify logits [R*(B+1), vocab] (request-major rows)."""
    R = len(kvs)
    hs = (ctypes.c_void_p * R)(*[kv.h.value for kv in kvs])
    mc = (ctypes.c_int32 * R)(*[int(x) for x in max_commit])
    out = _i32(R * (B + 2))
    n = _i32(R)
    A = _i32(R)
    dl = vl = None
    if want_logits:
        shape = (R * (B + 1), model.cfg.vocab)
        dl = torch.empty(shape, dtype=torch.float32, device=model.device)
        vl = torch.empty(shape, dtype=torch.float32, device=model.device)
    L.check(model.lib.ssb_round_batch(model.h, hs, R, B, mc, _ptr(planted_dev), out, n, A, _ptr(dl), _ptr(vl),
                                      _stream()))
    res = [(list(out[r * (B + 2): r * (B + 2) + n[r]]), A[r]) for r in range(R)]
    return (res, dl, vl) if want_logits else res


def ar_step_batch(model, kvs):
    """One greedy AR step for every kv in one launch per stage; returns the tokens."""
    R = len(kvs)
    hs = (ctypes.c_void_p * R)(*[kv.h.value for kv in kvs])
    out = _i32(R)
    L.check(model.lib.ssb_ar_step_batch(model.h, hs, R, out, _stream()))
    return list(out[:R])


def serve(model, pool, requests, max_running, mode, B=0, max_tokens=None):
    """Continuous batching over a queue of requests.

    requests: list of dicts with prefix_dev (device tensor [P][hidden]), max_len and, optionally,
    cont_dev (device int32 AR continuation) and astar (planted accept lengths per round).
    Returns (outputs, per-request info dicts, stats dict).
    """
    n = len(requests)
    reqs = (L.SsbRequest * max(n, 1))()
    outs, keep = [], []
    for i, q in enumerate(requests):
        r = reqs[i]
        r.prefix_dev = _ptr(q["prefix_dev"])
        r.P = q["prefix_dev"].shape[0]
        r.max_len = q["max_len"]
        o = _i32(max(q["max_len"], 1))
        outs.append(o)
        r.out = ctypes.cast(o, ctypes.c_void_p)
        if q.get("cont_dev") is not None:
            r.cont_dev = _ptr(q["cont_dev"])
            r.cont_len = q["cont_dev"].shape[0]
            a = (ctypes.c_int32 * max(len(q["astar"]), 1))(*[int(x) for x in q["astar"]])
            keep.append(a)
            r.astar = ctypes.cast(a, ctypes.c_void_p)
            r.n_astar = len(q["astar"])
    if max_tokens is None:
        max_tokens = max(q["prefix_dev"].shape[0] + q["max_len"] for q in requests) + 2 * B + 8
    st = L.SsbServeStats()
    L.check(model.lib.ssb_serve(model.h, pool.h, reqs, n, max_running, mode, B, max_tokens, byref(st), _stream()))
    res = [list(outs[i][: reqs[i].n_out]) for i in range(n)]
    info = [{"rounds": reqs[i].rounds, "finish_us": reqs[i].finish_us} for i in range(n)]
    stats = {k: getattr(st, k) for k, _ in L.SsbServeStats._fields_}
    return res, info, stats
