"""Device setup for a synthetic workload: what a serving engine's KV connector
does around the library.

Allocates the store arenas, the RoPE table and the paged cache with torch
(device memory only), puts every resident fact through store_put_fact,
builds the slot mapping with build_slot_mapping and copies it to the device,
and launches inject_topk.  All arithmetic of the path runs in libprkv.so.
"""

from __future__ import annotations

import math

import numpy as np
import torch

from . import prkv, workloads

GiB = 1 << 30


def cache_bytes(spec, num_blocks):
    return 2 * spec.num_layers * num_blocks * spec.block_size * spec.row_bytes


def fit_num_blocks(spec, reserve_bytes, device="cuda", margin=6 * GiB):
    """Largest block count <= spec.num_blocks whose K+V cache fits next to
    `reserve_bytes` of other allocations, rounded down to a multiple of 1024."""
    free, _ = torch.cuda.mem_get_info(device)
    per_block = cache_bytes(spec, 1)
    fit = (free - reserve_bytes - margin) // per_block
    if fit >= spec.num_blocks:
        return spec.num_blocks
    return int(fit // 1024 * 1024)


class DeviceWorkload:
    """A workload resident on one GPU: store, cache, mapping."""

    def __init__(self, w: workloads.Workload, device="cuda", gen_device=None, stream=None,
                 host_mapping=True, store_location="device", cache_from=None):
        self.w = w
        sp = w.spec
        self.device = torch.device(device)
        self.gen_device = gen_device or self.device
        self.stream = stream or torch.cuda.current_stream(self.device)
        self.desc = prkv.desc(sp.num_layers, sp.num_kv_heads, sp.head_dim, w.max_facts,
                              w.capacity_rows, sp.max_position, sp.rope_theta,
                              rope_style=sp.rope_style, key_layout=sp.key_layout,
                              llama3_scaling=sp.llama3_scaling, cache_layout=sp.cache_layout)
        arena_bytes, rope_bytes = prkv.store_required_bytes(self.desc)
        shape = (sp.num_layers, w.capacity_rows, sp.num_kv_heads, sp.head_dim)
        self.store_location = store_location
        if store_location == "device":
            self.k_arena = torch.empty(shape, dtype=torch.int16, device=self.device)
            self.v_arena = torch.empty(shape, dtype=torch.int16, device=self.device)
        elif store_location == "host":
            # pinned host memory mapped for the device: the inject kernel reads
            # the retrieved rows over PCIe directly (zero-copy)
            self.k_arena = torch.empty(shape, dtype=torch.int16, pin_memory=True)
            self.v_arena = torch.empty(shape, dtype=torch.int16, pin_memory=True)
        else:
            raise ValueError(store_location)
        self.rope = torch.empty(rope_bytes // 4, dtype=torch.float32, device=self.device)
        assert self.k_arena.numel() * 2 == arena_bytes
        self.store = prkv.store_create(self.desc, self.k_arena, self.v_arena, self.rope,
                                       stream=self.stream)
        self._put_all()
        self.hnd = sp.cache_layout == prkv.CACHE_HND
        if self.hnd:   # [L][block][H][bs][D]
            cshape = (sp.num_layers, w.num_blocks, sp.num_kv_heads, sp.block_size, sp.head_dim)
        else:          # [L][block][bs][H][D]
            cshape = (sp.num_layers, w.num_blocks, sp.block_size, sp.num_kv_heads, sp.head_dim)
        if cache_from is not None:
            # the paged cache of another workload of the same shape (e.g. the
            # same batch with its store in HBM and in host DRAM)
            assert tuple(cache_from.k_cache.shape) == cshape
            self.k_cache, self.v_cache = cache_from.k_cache, cache_from.v_cache
        else:
            self.k_cache = torch.empty(cshape, dtype=torch.int16, device=self.device)
            self.v_cache = torch.empty(cshape, dtype=torch.int16, device=self.device)
        self.reset_cache()
        self.status = torch.zeros(1, dtype=torch.int32, device=self.device)
        self.n_tokens = w.n_tokens
        if host_mapping:
            self.build_mapping()

    # -- store -------------------------------------------------------------
    def _put_all(self, batch=64):
        w = self.w
        pending = []
        with torch.cuda.stream(self.stream):
            for f in w.put_order:
                k, v = w.fact_kv(f, device=self.gen_device)
                if k.device != self.device:
                    k, v = k.to(self.device), v.to(self.device)
                prkv.store_put_fact(self.store, f, w.length_of(f), k, v, stream=self.stream)
                pending.append((k, v))
                if len(pending) >= batch:
                    self.stream.synchronize()
                    pending.clear()
        self.stream.synchronize()

    # -- cache -------------------------------------------------------------
    def reset_cache(self):
        with torch.cuda.stream(self.stream):
            self.k_cache.fill_(workloads.SENTINEL_BF16)
            self.v_cache.fill_(workloads.SENTINEL_BF16)

    def k_layers(self):
        return [self.k_cache[l] for l in range(self.w.spec.num_layers)]

    def v_layers(self):
        return [self.v_cache[l] for l in range(self.w.spec.num_layers)]

    # -- mapping -----------------------------------------------------------
    def build_mapping(self):
        w = self.w
        req_ptr, ids, start, bt, bt_len = w.csr()
        self.req_ptr, self.ids, self.start, self.bt, self.bt_len = req_ptr, ids, start, bt, bt_len
        n = w.n_tokens
        # two sets of pinned host buffers, used in turn by map_and_copy; each
        # set's event marks the end of the last copy out of it
        self.h_maps = [[torch.empty(max(n, 1), dtype=torch.int32, pin_memory=True)
                        for _ in range(3)] for _ in range(2)]
        self.h_events = [None, None]
        self.h_turn = 0
        src, pos, slot = prkv.build_slot_mapping(
            self.store, req_ptr, ids, start, bt, bt_len, w.spec.block_size, w.num_blocks,
            out=tuple(t.numpy() for t in self.h_maps[0]))
        self.n_tokens = len(src)
        with torch.cuda.stream(self.stream):
            self.d_map = [t.to(self.device, non_blocking=True) for t in self.h_maps[0]]
        self.stream.synchronize()
        return src, pos, slot

    def map_and_copy(self):
        """Host slot mapping into pinned buffers + async H2D of the three arrays.

        The host writes a buffer set only after the previous copy out of it
        has finished (its event), so a mapping that changes between calls can
        never be torn by a copy still queued behind earlier kernels; with two
        sets the host mapping of one call overlaps the copy and kernel of the
        previous one."""
        w = self.w
        self.h_turn ^= 1
        bufs, ev = self.h_maps[self.h_turn], self.h_events[self.h_turn]
        if ev is not None:
            ev.synchronize()
        prkv.build_slot_mapping(self.store, self.req_ptr, self.ids, self.start, self.bt,
                                self.bt_len, w.spec.block_size, w.num_blocks,
                                out=tuple(t.numpy() for t in bufs))
        with torch.cuda.stream(self.stream):
            for d, h in zip(self.d_map, bufs):
                d.copy_(h, non_blocking=True)
            ev = torch.cuda.Event()
            ev.record(self.stream)
        self.h_events[self.h_turn] = ev

    # -- device-resident batch (device-side slot mapping) --------------------
    def setup_device_batch(self, max_tokens=None, max_facts=None, flags=0):
        """Upload the batch description, the fact table and a workspace.
        flags: prkv.BATCH_CHECK_SLOTS to detect duplicate slots on the device."""
        w = self.w
        req_ptr, ids, start, bt, bt_len = w.csr()
        dev = self.device
        self.d_req_ptr = torch.from_numpy(req_ptr).to(dev)
        self.d_ids = torch.from_numpy(ids).to(dev)
        self.d_start = torch.from_numpy(start).to(dev)
        self.d_bt = torch.from_numpy(np.ascontiguousarray(bt)).to(dev)
        self.d_bt_len = torch.from_numpy(bt_len).to(dev)
        self.fact_table = torch.empty(2 * w.max_facts, dtype=torch.int32, device=dev)
        prkv.store_upload_fact_table(self.store, self.fact_table, stream=self.stream)
        self.max_facts = int(max_facts if max_facts is not None else len(ids))
        longest = max(w.length_of(f) for f in w.put_order)
        self.max_tokens = int(max_tokens if max_tokens is not None else len(ids) * longest)
        self.ws_bytes = prkv.inject_device_workspace_bytes(self.max_facts, self.max_tokens)
        self.workspace = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.ws_layout = prkv.workspace_layout(self.max_facts, self.max_tokens)
        self.batch = prkv.device_batch(len(req_ptr) - 1, bt.shape[1], self.max_facts,
                                       self.max_tokens, self.d_req_ptr, self.d_ids, self.d_start,
                                       self.d_bt, self.d_bt_len, flags=flags)
        self.stream.synchronize()

    def inject_device(self):
        prkv.inject_topk_device(self.store, self.fact_table, self.batch, self.k_layers(),
                                self.v_layers(), self.w.spec.block_size, self.w.num_blocks,
                                self.workspace, self.ws_bytes, d_status=self.status,
                                stream=self.stream)

    def inject_device_args(self):
        """Pre-marshalled arguments of inject_topk_device for timing loops."""
        import ctypes
        L = self.w.spec.num_layers
        kp = (ctypes.c_void_p * L)(*[t.data_ptr() for t in self.k_layers()])
        vp = (ctypes.c_void_p * L)(*[t.data_ptr() for t in self.v_layers()])
        return (self.store.handle, self.fact_table.data_ptr(), ctypes.byref(self.batch), kp, vp,
                self.w.spec.block_size, self.w.num_blocks, self.workspace.data_ptr(),
                self.ws_bytes, self.status.data_ptr(), self.stream.cuda_stream)

    def device_mapping(self):
        """(n_tokens, src_row, pos, slot) the device path wrote into its workspace."""
        ws = self.workspace.cpu().numpy()
        lay = self.ws_layout
        n = int(ws[lay["n_tokens"]:lay["n_tokens"] + 8].view(np.int64)[0])
        arr = {k: ws[lay[k]:lay[k] + 4 * n].view(np.int32) for k in ("src_row", "pos", "slot")}
        return n, arr["src_row"], arr["pos"], arr["slot"]

    # -- inject ------------------------------------------------------------
    def inject(self):
        prkv.inject_topk(self.store, self.n_tokens, self.d_map[0], self.d_map[1], self.d_map[2],
                         self.k_layers(), self.v_layers(), self.w.spec.block_size,
                         self.w.num_blocks, d_status=self.status, stream=self.stream)

    def inject_args(self):
        """Pre-marshalled arguments for tight timing loops."""
        import ctypes
        L = self.w.spec.num_layers
        kp = (ctypes.c_void_p * L)(*[t.data_ptr() for t in self.k_layers()])
        vp = (ctypes.c_void_p * L)(*[t.data_ptr() for t in self.v_layers()])
        return (self.store.handle, self.n_tokens, self.d_map[0].data_ptr(),
                self.d_map[1].data_ptr(), self.d_map[2].data_ptr(), kp, vp,
                self.w.spec.block_size, self.w.num_blocks, self.status.data_ptr(),
                self.stream.cuda_stream)

    # -- reading back ------------------------------------------------------
    def listed_blocks_host(self, blocks):
        """K and V cache contents of the given blocks, all layers, as uint16
        numpy [L][n][block_size][H][D] whatever the cache layout."""
        idx = torch.as_tensor(blocks, dtype=torch.long, device=self.device)
        out = []
        for cache in (self.k_cache, self.v_cache):
            sel = cache.index_select(1, idx)
            if self.hnd:
                sel = sel.permute(0, 1, 3, 2, 4).contiguous()
            out.append(sel.cpu().numpy().view(np.uint16))
        return tuple(out)

    def slot_rows(self, cache, slots):
        """Rows of the given slots (device int64 tensor), all layers and heads:
        a device tensor [L][n][H][D] whatever the cache layout."""
        bs = self.w.spec.block_size
        if not self.hnd:
            sp = self.w.spec
            return cache.view(sp.num_layers, -1, sp.num_kv_heads, sp.head_dim)[:, slots]
        # advanced indices around a slice: the result is [n][L][H][D]
        return cache[:, slots // bs, :, slots % bs].permute(1, 0, 2, 3)

    def slot_rows_layer(self, cache, layer, slots):
        """Rows of the given slots (device int64 tensor) in one layer: a
        device tensor [n][H][D] whatever the cache layout."""
        c = cache[layer]
        if not self.hnd:
            sp = self.w.spec
            return c.view(-1, sp.num_kv_heads, sp.head_dim)[slots]
        bs = self.w.spec.block_size
        return c[slots // bs, :, slots % bs]   # [block][H][bs][D] -> [n][H][D]

    def set_slot_row(self, cache, layer, slot, value):
        """Write one slot's [H][D] row of one layer."""
        bs = self.w.spec.block_size
        if self.hnd:
            cache[layer, slot // bs, :, slot % bs] = value
        else:
            cache[layer, slot // bs, slot % bs] = value

    def count_non_sentinel(self, chunk_elems=1 << 28):
        """Number of cache elements (K and V, all layers) != the sentinel."""
        total = 0
        for cache in (self.k_cache, self.v_cache):
            flat = cache.view(-1)
            for s in range(0, flat.numel(), chunk_elems):
                total += int((flat[s:s + chunk_elems] != workloads.SENTINEL_BF16).sum().item())
        return total


def chunk_facts(facts, lengths, chunks):
    """Cut a batch's flattened fact list (request order, then rank order)
    into at most `chunks` consecutive pieces of about equal token counts.
    Returns [(distinct facts of the piece in order, first token, end token)];
    the token ranges are those of the batch's slot mapping, which lists the
    tokens in the same order."""
    lens = np.asarray(lengths, np.int64)
    if len(lens) == 0:
        return []
    ends = np.cumsum(lens)
    total = int(ends[-1])
    chunks = max(1, min(int(chunks), len(lens)))
    cuts = [0] + [int(np.searchsorted(ends, total * c / chunks, side="left")) + 1
                  for c in range(1, chunks)] + [len(lens)]
    cuts = sorted(set(min(max(c, 0), len(lens)) for c in cuts))
    pieces = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        if b <= a:
            continue
        t0 = int(ends[a - 1]) if a > 0 else 0
        pieces.append((list(dict.fromkeys(facts[a:b])), t0, int(ends[b - 1])))
    return pieces


class StagedInjector:
    """Injection from a host-DRAM store through an HBM staging store: the
    batch's facts are copied host -> HBM (store_stage_facts) in chunks on a
    copy stream, and each chunk's tokens are injected on the workload's
    stream as soon as its facts have landed, so the copies of later chunks
    overlap the injection of earlier ones.  The staging store has the host
    store's descriptor and row layout (rows reserved in the same put order),
    so the host-built mapping serves both.

    host_dw: a DeviceWorkload with store_location="host" and a host mapping.
    k_arena, v_arena: HBM tensors with the host arenas' shape (they may be
    another workload's arenas for the same facts: the staged rows are the
    same rows with the same contents).
    chunks: how many pieces the batch's fact list is cut into (at fact
    boundaries, about equal token counts); 1 stages everything, then injects.
    """

    def __init__(self, host_dw, k_arena, v_arena, chunks=8, copy_stream=None):
        assert host_dw.store_location == "host" and k_arena.is_cuda
        assert tuple(k_arena.shape) == tuple(host_dw.k_arena.shape)
        w = host_dw.w
        self.dw = host_dw
        self.k_arena, self.v_arena = k_arena, v_arena
        self.store = prkv.store_create(host_dw.desc, k_arena, v_arena, host_dw.rope,
                                       stream=host_dw.stream)
        for f in w.put_order:      # the host store's rows, reserved (no data)
            prkv.store_put_fact(self.store, f, w.length_of(f))
        self.copy = copy_stream or torch.cuda.Stream(device=host_dw.device)
        flat = [f for ids in w.retrieved for f in ids]
        self.pieces = chunk_facts(flat, [w.length_of(f) for f in flat], chunks)
        assert sum(t1 - t0 for _, t0, t1 in self.pieces) == host_dw.n_tokens
        self.done = None   # event: the previous step's injections have read the staging rows

    def step(self):
        """Stage and inject the whole batch once (asynchronous)."""
        dw, w = self.dw, self.dw.w
        comp = dw.stream
        if self.done is not None:
            self.copy.wait_event(self.done)
        src, pos, slot = dw.d_map
        kl, vl = dw.k_layers(), dw.v_layers()
        for facts, t0, t1 in self.pieces:
            prkv.store_stage_facts(dw.store, self.store, facts, stream=self.copy)
            ev = torch.cuda.Event()
            ev.record(self.copy)
            comp.wait_event(ev)
            prkv.inject_topk(self.store, t1 - t0, src[t0:t1], pos[t0:t1], slot[t0:t1], kl, vl,
                             w.spec.block_size, w.num_blocks, d_status=dw.status, stream=comp)
        self.done = torch.cuda.Event()
        self.done.record(comp)
