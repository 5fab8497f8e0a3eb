"""Device-resident synthetic workloads for the tests, the smoke check and the
benchmark.

Glue only: inputs are drawn by ``synth`` (host numpy for normals, its device
fill for the quantised weights) and packed into the fixed-stride expert slab
by the library's own device packer.  Nothing here computes any part of the
MoE layer.
"""
from __future__ import annotations

import numpy as np
import torch

import int4_group_quantized_moe_amd as moe
import synth
from synth import device as synth_device


def desc_for(cfg, n_tokens: int | None = None, dense_q4: bool = False):
    return moe.make_desc(cfg.n_tokens if n_tokens is None else n_tokens, cfg.hidden,
                         cfg.n_experts, cfg.top_k, cfg.inter, cfg.shared_inter, bits=cfg.bits,
                         act=cfg.act, router_bias=bool(cfg.zipf_s), shared=True,
                         rms_eps=cfg.rms_eps, dense_q4=dense_q4)


def act_dtype(cfg):
    return torch.float32 if cfg.act == "f32" else torch.bfloat16


class Workload:
    """All layers of one configuration, resident in HBM.

    slab          uint8 [n_layers*E*stride] (one blob per slot)
    slot_tables   int32 [n_layers, E]
    shared        uint8 [n_layers, shared_stride] (blob + w_sg)
    router_w      fp32  [n_layers, E, H]
    router_bias   fp32  [n_layers, E] or None
    dense         uint8 [n_layers, dense bytes]: with dense_q4, the 4-bit router
                  rows and shared gate (moe_pack_dense); the layer calls then
                  take it as their router argument and the flag in `desc`
    """

    def __init__(self, cfg, n_layers: int | None = None, device="cuda", permute_seed=None,
                 batch: int = 32, layers: list | None = None, dense_q4: bool = False):
        self.cfg = cfg
        self.layer_ids = list(range(n_layers if n_layers is not None else cfg.layers)) \
            if layers is None else list(layers)
        L = len(self.layer_ids)
        E, H = cfg.n_experts, cfg.hidden
        self.dense_q4 = dense_q4
        self.desc = desc_for(cfg, dense_q4=dense_q4)
        self.stride = int(self.desc.expert_stride)
        self.layout = moe.moe_blob_layout(self.desc, cfg.inter)
        self.slayout = moe.moe_blob_layout(self.desc, cfg.shared_inter)
        self.shared_stride = int(self.slayout.shared_bytes)
        self.device = device
        stream = torch.cuda.current_stream().cuda_stream
        self.slab = torch.empty(L * E * self.stride, dtype=torch.uint8, device=device)
        self.shared = torch.zeros(L, self.shared_stride, dtype=torch.uint8, device=device)
        tables = []
        for i, l in enumerate(self.layer_ids):
            st = synth.slot_table(cfg, l, permute_seed).astype(np.int64) - l * E + i * E
            tables.append(st.astype(np.int32))
        self.slot_tables_np = np.stack(tables)
        self.slot_tables = torch.from_numpy(self.slot_tables_np).to(device)
        self.router_w = torch.empty(L, E, H, dtype=torch.float32, device=device)
        self.router_bias = (torch.empty(L, E, dtype=torch.float32, device=device)
                            if cfg.zipf_s else None)
        self.dense_bytes = int(moe.moe_dense_layout(self.desc).bytes)
        self.dense = (torch.empty(L, self.dense_bytes, dtype=torch.uint8, device=device)
                      if dense_q4 else None)
        I, Is = cfg.inter, cfg.shared_inter
        G = cfg.group
        B = min(batch, E)
        qg = torch.empty(B, I, H, dtype=torch.uint8, device=device)
        qu = torch.empty_like(qg)
        qd = torch.empty(B, H, I, dtype=torch.uint8, device=device)
        sbg = torch.empty(B, 2, I, H // G, dtype=torch.int16, device=device)
        sbu = torch.empty_like(sbg)
        sbd = torch.empty(B, 2, H, I // G, dtype=torch.int16, device=device)
        for i, l in enumerate(self.layer_ids):
            for e0 in range(0, E, B):
                n = min(B, E - e0)
                synth_device.fill_experts(cfg, l, e0, n, I, qg, qu, qd, sbg, sbu, sbd, stream)
                slots = [int(self.slot_tables_np[i, e]) for e in range(e0, e0 + n)]
                moe.moe_pack_experts_device(self.desc, I, n, qg, qu, qd, sbg, sbu, sbd, self.slab,
                                            slots)
            # shared expert: packed into its own blob, then w_sg appended
            sqg = torch.empty(1, Is, H, dtype=torch.uint8, device=device)
            squ = torch.empty_like(sqg)
            sqd = torch.empty(1, H, Is, dtype=torch.uint8, device=device)
            ssg = torch.empty(1, 2, Is, H // G, dtype=torch.int16, device=device)
            ssu = torch.empty_like(ssg)
            ssd = torch.empty(1, 2, H, Is // G, dtype=torch.int16, device=device)
            synth_device.fill_experts(cfg, l, synth.SHARED_EXPERT, 1, Is, sqg, squ, sqd, ssg, ssu,
                                      ssd, stream)
            moe.moe_pack_experts_device(self.desc, Is, 1, sqg, squ, sqd, ssg, ssu, ssd,
                                        self.shared[i], [0])
            wsg = torch.from_numpy(synth.shared_gate_weight(cfg, l)).to(device)
            off = int(self.slayout.shared_gate_offset)
            self.shared[i, off:off + 4 * H].copy_(wsg.view(torch.uint8))
            self.router_w[i].copy_(torch.from_numpy(synth.router_weight(cfg, l)))
            if dense_q4:
                a = synth.dense_q4_arrays(cfg, l)
                blob = np.zeros(self.dense_bytes, np.uint8)
                moe.moe_pack_dense(self.desc, np.ascontiguousarray(a["q"]),
                                   np.ascontiguousarray(np.stack([a["s"], a["b"]])), blob)
                self.dense[i].copy_(torch.from_numpy(blob))
            if self.router_bias is not None:
                self.router_bias[i].copy_(torch.from_numpy(synth.router_bias(cfg, l)))
        torch.cuda.synchronize()

    # per-layer views -------------------------------------------------------
    def layer_args(self, i: int):
        """(router_w, router_bias, slot_table, shared_blob) of layer index i
        (router_w: the dense blob with dense_q4)."""
        rb = self.router_bias[i] if self.router_bias is not None else None
        rw = self.dense[i] if self.dense_q4 else self.router_w[i]
        return rw, rb, self.slot_tables[i], self.shared[i]

    @property
    def router_all(self):
        """The router argument of a chain call over all layers."""
        return self.dense if self.dense_q4 else self.router_w

    def dense_rows(self, i: int) -> np.ndarray:
        """Layer index i's dense rows (router rows, then the shared gate) as the
        fp64 values they encode, through the oracle's dequantisation (tests)."""
        import oracle
        a = synth.dense_q4_arrays(self.cfg, self.layer_ids[i])
        return oracle.dequantize(a["q"], a["s"], a["b"], self.cfg.group)

    def workspace(self, desc=None):
        """Zero-filled workspace (the chain's exchange words must start at zero)."""
        n = moe.moe_workspace_bytes(desc or self.desc)
        return torch.zeros(max(n, 256), dtype=torch.uint8, device=self.device)


def act_tensor(cfg, x_np: np.ndarray, device="cuda"):
    """fp32 numpy values (exactly representable) -> device tensor of the act dtype."""
    return torch.from_numpy(np.ascontiguousarray(x_np, dtype=np.float32)).to(device).to(act_dtype(cfg))


def to_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)
