"""Torch-facing helper around the C ABI: PyTorch supplies device memory and streams only.

Every step of the decode path runs in the HIP engine kernel of libdec.so; this module only
allocates buffers, checks their shapes against the plan's layout contract and forwards
pointers.
"""
from __future__ import annotations

from typing import Dict, Optional

from . import binding as B

_TORCH_DTYPE = {"bf16": "bfloat16", "fp32": "float32", "i32": "int32", "fp8": "uint8", "fp4x2": "uint8",
                "e8m0": "uint8"}  # FP8 bytes, packed E2M1 pairs and E8M0 scales as uint8


class DecodeEngine:
    def __init__(self, cfg: dict, weights: Dict[str, "object"], kv_len: Optional[int] = None,
                 stream=None, watchdog_us: Optional[int] = None, max_len: Optional[int] = None,
                 static_workspace: bool = False):
        """A plan for kv_len (default: the config's), or, with max_len, a plan whose position
        is read per step from a device state (step_dynamic). A config with "verify": M plans a
        verification step of M tokens (x [M][hidden], out [M][vocab]). static_workspace: bind
        to the library's static per-device workspace (dec_plan_bind_scratch) instead of
        allocating one; the named intermediate buffers are then not readable through buffer()."""
        import torch
        if not torch.cuda.is_available():
            raise RuntimeError("DecodeEngine needs a GPU (gfx950); there is no CPU path")
        self.torch = torch
        self.cfg = cfg
        self.dynamic = max_len is not None
        self.kv_len = int(max_len) if self.dynamic else (cfg["kv_len"] if kv_len is None else int(kv_len))
        self.plan = B.Plan(cfg, self.kv_len, max_len=max_len)
        if watchdog_us is not None:
            self.plan.set_watchdog(watchdog_us)
        self.descs = self.plan.weight_descs()
        ptrs = []
        self._keep = []
        for d in self.descs:
            t = weights[d["name"]]
            want = getattr(torch, _TORCH_DTYPE[d["dtype"]])
            if t.dtype != want or tuple(t.shape) != tuple(d["shape"]) or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"weight {d['name']}: expected contiguous cuda {want} {d['shape']}, "
                                 f"got {t.dtype} {tuple(t.shape)} on {t.device}")
            ptrs.append(t.data_ptr())
            self._keep.append(t)
        self.sizes = self.plan.sizes()
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        if static_workspace:
            self.workspace = None
            self.plan.bind_scratch(ptrs, self.stream.cuda_stream)
        else:
            self.workspace = torch.empty(self.sizes["workspace_bytes"], dtype=torch.uint8, device="cuda")
            self.plan.bind(ptrs, self.workspace.data_ptr(), self.workspace.numel(), self.stream.cuda_stream)
        self.buffers = self.plan.buffers()
        self.n_tokens = self.plan.n_tokens
        out_n = cfg["vocab"] if cfg.get("vocab", 0) > 0 else cfg["hidden"]
        self.out = torch.empty(out_n, dtype=torch.float32, device="cuda")
        if self.n_tokens > 1:
            self.out = torch.empty(self.n_tokens, out_n, dtype=torch.float32, device="cuda")
        # {position, token, steps, 0}: read and advanced by every dynamic step
        self.state = torch.zeros(4, dtype=torch.int32, device="cuda") if self.dynamic else None

    def set_state(self, position: int, token: int = 0):
        """Set the dynamic plan's next position and token (on the engine's stream)."""
        torch = self.torch
        with torch.cuda.stream(self.stream):
            self.state.copy_(torch.tensor([int(position), int(token), 0, 0], dtype=torch.int32), non_blocking=False)

    def read_state(self):
        self.stream.synchronize()
        return [int(v) for v in self.state.cpu().tolist()]

    def step_dynamic(self, kv, x=None, out=None):
        """One step at the position in the device state (advanced by the step); without x the
        input is the embedding row of the state's token, and the step leaves its greedy choice
        there. No host synchronisation."""
        torch = self.torch
        out = self.out if out is None else out
        if x is not None:
            self._check_io(x, kv, out)
        else:
            if kv.dtype != torch.bfloat16 or kv.numel() * 2 != self.sizes["kv_bytes"] or not kv.is_contiguous() or not kv.is_cuda:
                raise ValueError(f"kv must be a contiguous cuda bf16 tensor of {self.sizes['kv_bytes']} bytes")
            if out.dtype != torch.float32 or out.numel() * 4 != self.sizes["out_bytes"] or not out.is_contiguous() or not out.is_cuda:
                raise ValueError("out must be contiguous cuda fp32 of length vocab (or hidden)")
        self.plan.step_dynamic(0 if x is None else x.data_ptr(), kv.data_ptr(), out.data_ptr(), self.state.data_ptr(),
                               self.stream.cuda_stream)
        return out

    def _check_io(self, x, kv, out):
        torch = self.torch
        if x.dtype != torch.bfloat16 or x.numel() * 2 != self.sizes["x_bytes"] or not x.is_contiguous() or not x.is_cuda:
            raise ValueError("x must be contiguous cuda bf16 [tokens per step][hidden]")
        if kv.dtype != torch.bfloat16 or kv.numel() * 2 != self.sizes["kv_bytes"] or not kv.is_contiguous() or not kv.is_cuda:
            raise ValueError(f"kv must be a contiguous cuda bf16 tensor of {self.sizes['kv_bytes']} bytes")
        if out.dtype != torch.float32 or out.numel() * 4 != self.sizes["out_bytes"] or not out.is_contiguous() or not out.is_cuda:
            raise ValueError("out must be contiguous cuda fp32 [tokens per step][vocab (or hidden)]")

    def step(self, x, kv, out=None):
        """One decode step: x bf16 [hidden], kv bf16 cache (written at slot kv_len); a
        verification plan: x [M][hidden], slots kv_len .. kv_len + M - 1, out [M][vocab]."""
        out = self.out if out is None else out
        self._check_io(x, kv, out)
        self.plan.step(x.data_ptr(), kv.data_ptr(), out.data_ptr(), self.stream.cuda_stream)
        return out

    @property
    def n_stages(self) -> int:
        return self.plan.n_stages()

    def step_stages(self, x, kv, out=None, stream=None):
        """The same step as one launch per stage (the launch-per-operator baseline), on
        `stream` (default: the engine's stream)."""
        out = self.out if out is None else out
        self._check_io(x, kv, out)
        h = (self.stream if stream is None else stream).cuda_stream
        for sg in range(self.plan.n_stages()):
            self.plan.step_stages(x.data_ptr(), kv.data_ptr(), out.data_ptr(), sg, sg + 1, h)
        return out

    def capture_stages(self, x, kv, out=None):
        """A torch CUDA (HIP) graph of one step's per-stage launches; replay() runs a step."""
        torch = self.torch
        out = self.out if out is None else out
        self._check_io(x, kv, out)
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(self.stream)
        with torch.cuda.graph(g, stream=side):
            self.step_stages(x, kv, out, stream=side)
        self.stream.wait_stream(side)
        return g

    def status(self):
        self.plan.status(self.stream.cuda_stream)

    def buffer(self, name: str):
        """A view of a named workspace buffer (per-layer intermediates of the last step)."""
        torch = self.torch
        if self.workspace is None:
            raise ValueError("an engine bound to the static workspace exposes no named buffers")
        b = self.buffers[name]
        nbytes = b["count"] * 4
        raw = self.workspace[b["offset"]:b["offset"] + nbytes]
        return raw.view(torch.int32 if b["dtype"] == "i32" else torch.float32)

    def task_log(self):
        """[n_log, 16] int64: execs, epoch, wg, xcd, t_start, t_ready, t_end, t_mid, t_staged,
        t_streamed, t_signal, t_aux[5] (times: the device's 100 MHz clock, low 32 bits; t_end,
        t_mid, t_staged, t_streamed and t_aux only in a build with the detailed log)."""
        return self.buffer("task_log").view(-1, 16).to(self.torch.int64) & 0xFFFFFFFF
