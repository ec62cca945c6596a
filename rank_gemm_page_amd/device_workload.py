"""Put a synthetic workload (``synth.Workload``) on the GPU through the C ABI.

Torch provides the device memory (page classes, x, y, metadata, workspace)
and the stream; every step of the LoRA delta runs in libslora.  Page memory
starts as NaN, so a read of any page that is not one of the batch's adapter
rows (KV filler, free pages, reserved adapters) turns into NaN in y.
"""
from __future__ import annotations

import numpy as np

from . import slora as S


class DeviceWorkload:
    def __init__(self, w, device="cuda:0", tuning=None, poison=True, load_all_weights=False,
                 load="sync"):
        """load: "sync" (slora_load_adapter) or "async" (packed pinned images
        fetched with slora_load_adapters_async on a second stream, which the
        current stream then waits for)."""
        import torch

        self.torch = torch
        self.w = w
        spec = w.spec
        self.device = torch.device(device)
        self.tdtype = torch.float16 if spec.dtype == "f16" else torch.float32
        self.dtype_code = S.SLORA_F16 if spec.dtype == "f16" else S.SLORA_F32
        n_classes = 2 if spec.two_classes else 1
        fill = float("nan") if poison else 0.0
        self.pages = [torch.full((int(w.n_pages[c]), w.page_elems(c)), fill, dtype=self.tdtype,
                                 device=self.device) for c in range(n_classes)]
        self.max_rank = int(max(int(w.ranks.max()), 1))
        self.pool = S.slora_pool_create(self.dtype_code, spec.h_in, spec.h_out, spec.n_proj,
                                        spec.n_adapters, self.max_rank, self.pages,
                                        [int(P) for P in w.n_pages], w.free_order)
        self.seg = None
        self.images = []          # pinned adapter images a queued load may still read
        self.stages = {}          # device staging buffer per fetch stream
        self.load_stream = None
        try:
            for key, value in (tuning or {}).items():
                S.slora_pool_set_tuning(self.pool, key, value)
            self.kv = [S.slora_alloc_pages(self.pool, c, int(n)) for c, n in enumerate(w.kv_pages)]
            stream = torch.cuda.current_stream(self.device)
            if load == "async":
                self.load_stream = torch.cuda.Stream(self.device)
            fetch = []
            for a in range(spec.n_adapters):
                r = int(w.ranks[a])
                if load_all_weights or w.has_weights(a):
                    if load == "async":
                        fetch.append(a)
                        continue
                    ws = [w.weights(a, p) for p in range(spec.n_proj)]
                    S.slora_load_adapter(self.pool, a, r, float(w.scales[a]), [m[0] for m in ws],
                                         [m[1] for m in ws], stream, h_in=spec.h_in,
                                         h_out=spec.h_out, dtype=w.np_dtype)
                else:
                    if fetch:   # pages are taken in id order, as the oracle's model does
                        self.load_async(fetch, self.load_stream)
                        fetch = []
                    S.slora_load_adapter(self.pool, a, r, float(w.scales[a]))
            if fetch:
                self.load_async(fetch, self.load_stream)
            if load == "async":
                done = torch.cuda.Event()
                done.record(self.load_stream)
                stream.wait_event(done)
            self.x = [torch.from_numpy(np.ascontiguousarray(x)).to(self.device) for x in w.x]
            self.y0 = [torch.from_numpy(np.ascontiguousarray(y)).to(self.device) for y in w.y]
            self.y = [t.clone() for t in self.y0]
            self.build(w.ids)
        except Exception:
            self.close()
            raise

    # -- adapter fetch ---------------------------------------------------------
    def pack(self, a):
        """Pinned host image of adapter a (the host-resident store's form)."""
        torch, w, spec = self.torch, self.w, self.w.spec
        r = int(w.ranks[a])
        nb = S.slora_adapter_image_bytes(self.pool, r)
        img = torch.empty(nb, dtype=torch.uint8, pin_memory=True)
        ws = [w.weights(a, p) for p in range(spec.n_proj)]
        S.slora_pack_adapter(self.pool, r, [m[0] for m in ws], [m[1] for m in ws], img, nb,
                             h_in=spec.h_in, h_out=spec.h_out, dtype=w.np_dtype)
        return img

    def stage_for(self, stream, nbytes):
        """Device staging of at least nbytes for fetches queued on `stream`:
        stream order lets every fetch on one stream reuse it."""
        key = int(stream.cuda_stream)
        if key not in self.stages or self.stages[key].numel() < nbytes:
            if key in self.stages:
                stream.synchronize()
            self.stages[key] = self.torch.empty(nbytes, dtype=self.torch.uint8, device=self.device)
        return self.stages[key]

    def load_async(self, adapters, stream, images=None):
        """Queue the fetch of `adapters` (one batch) on `stream`; return at once."""
        w = self.w
        adapters = [int(a) for a in adapters]
        imgs = [self.pack(a) for a in adapters] if images is None else list(images)
        self.images.extend(imgs)
        ranks = [int(w.ranks[a]) for a in adapters]
        need = sum(S.slora_adapter_image_bytes(self.pool, r) for r in ranks)
        stage = self.stage_for(stream, max(need, 256))
        S.slora_load_adapters_async(self.pool, adapters, ranks, [float(w.scales[a]) for a in adapters],
                                    imgs, stage, stage.numel(), stream)

    # -- segments --------------------------------------------------------------
    def build(self, ids):
        torch = self.torch
        if self.seg is not None:
            S.slora_segments_destroy(self.seg)
            self.seg = None
        self.seg = S.slora_build_segments(self.pool, ids)
        self.info = S.slora_segments_get_info(self.seg)
        self.meta = torch.empty(self.info["meta_bytes"], dtype=torch.uint8, device=self.device)
        self.workspace = torch.empty(self.info["workspace_bytes"], dtype=torch.uint8,
                                     device=self.device)
        self.upload()
        return self.info

    def upload(self, stream=None):
        stream = stream or self.torch.cuda.current_stream(self.device)
        S.slora_segments_upload(self.seg, self.meta, self.info["meta_bytes"], stream)

    # -- the hot path --------------------------------------------------------------
    def delta(self, proj=0, y=None, stream=None):
        stream = stream or self.torch.cuda.current_stream(self.device)
        x = self.x[self.w.spec.proj_x[proj]]
        S.slora_lora_delta(self.pool, self.seg, proj, x, self.y[proj] if y is None else y,
                           self.workspace, self.info["workspace_bytes"], stream)

    def ensure_workspace(self, n):
        """Workspace for n projections in one launch (slora_lora_delta_multi)."""
        need = n * self.info["workspace_bytes"]
        if self.workspace.numel() < need:
            self.workspace = self.torch.empty(need, dtype=self.torch.uint8, device=self.device)
        return need

    def delta_multi(self, projs=None, ys=None, stream=None, events=None):
        """Every projection in projs (all by default) in one slora_lora_delta_multi
        launch; events: (start, stop) raw hipEvent_t handles for the timed call."""
        stream = stream or self.torch.cuda.current_stream(self.device)
        projs = list(range(self.w.spec.n_proj)) if projs is None else list(projs)
        xs = [self.x[self.w.spec.proj_x[p]] for p in projs]
        ys = [self.y[p] for p in projs] if ys is None else list(ys)
        nbytes = self.ensure_workspace(len(projs))
        if events is None:
            S.slora_lora_delta_multi(self.pool, self.seg, projs, xs, ys, self.workspace, nbytes, stream)
        else:
            S.slora_lora_delta_multi_timed(self.pool, self.seg, projs, xs, ys, self.workspace, nbytes, stream,
                                           events[0], events[1])

    def delta_timed(self, proj, start_event, stop_event, stream=None):
        """delta() with the dispatch recording two raw hipEvent_t handles."""
        stream = stream or self.torch.cuda.current_stream(self.device)
        x = self.x[self.w.spec.proj_x[proj]]
        S.slora_lora_delta_timed(self.pool, self.seg, proj, x, self.y[proj], self.workspace,
                                 self.info["workspace_bytes"], stream, start_event, stop_event)

    def base_weight(self, proj=0):
        """The workload's dense base weight W of projection ``proj`` on the device."""
        if not hasattr(self, "_w_dev"):
            self._w_dev = {}
        if proj not in self._w_dev:
            self._w_dev[proj] = self.torch.from_numpy(self.w.base_weight(proj)).to(self.device)
        return self._w_dev[proj]

    def forward(self, proj=0, out=None, stream=None):
        """out = x W + s (x A) B (slora_lora_forward); returns out."""
        torch = self.torch
        stream = stream or torch.cuda.current_stream(self.device)
        if out is None:
            out = torch.empty((self.w.T, self.w.spec.h_out), dtype=self.tdtype, device=self.device)
        S.slora_lora_forward(self.pool, self.seg, proj, self.x[self.w.spec.proj_x[proj]],
                             self.base_weight(proj), out, self.workspace,
                             self.info["workspace_bytes"], stream)
        return out

    def forward_timed(self, proj, out, start_event, stop_event, stream=None):
        stream = stream or self.torch.cuda.current_stream(self.device)
        S.slora_lora_forward_timed(self.pool, self.seg, proj, self.x[self.w.spec.proj_x[proj]],
                                   self.base_weight(proj), out, self.workspace,
                                   self.info["workspace_bytes"], stream, start_event, stop_event)

    def shrink(self, proj=0, stream=None):
        stream = stream or self.torch.cuda.current_stream(self.device)
        S.slora_lora_shrink(self.pool, self.seg, proj, self.x[self.w.spec.proj_x[proj]],
                            self.workspace, self.info["workspace_bytes"], stream)

    def expand(self, proj=0, y=None, stream=None):
        stream = stream or self.torch.cuda.current_stream(self.device)
        S.slora_lora_expand(self.pool, self.seg, proj, self.y[proj] if y is None else y,
                            self.workspace, self.info["workspace_bytes"], stream)

    def algorithmic_bytes(self, proj=0):
        """(shrink, expand) bytes one projection must move: each distinct adapter's
        pages once, x once (shrink), y read and written (expand)."""
        spec, w = self.w.spec, self.w
        e = 2 if spec.dtype == "f16" else 4
        r_u = int(self.info["sum_rank"])
        routed = int(self.info["n_routed"])
        shrink = r_u * spec.h_in * e + routed * spec.h_in * e
        expand = r_u * spec.h_out * e + 2 * routed * spec.h_out * e
        return shrink, expand

    def algorithmic_flops(self, proj=0):
        spec = self.w.spec
        rt = int(self.info["sum_rank_tokens"])
        return 2 * rt * spec.h_in, 2 * rt * spec.h_out

    def reset_y(self):
        for y, y0 in zip(self.y, self.y0):
            y.copy_(y0)

    def close(self):
        if self.images or self.stages:
            self.torch.cuda.synchronize(self.device)
            self.images, self.stages = [], {}
        if getattr(self, "seg", None) is not None:
            S.slora_segments_destroy(self.seg)
            self.seg = None
        if getattr(self, "pool", None) is not None:
            S.slora_pool_destroy(self.pool)
            self.pool = None
