"""Expert-granularity offload of packed experts (Axolotl issue #3787,
"Expert-granularity CPU offload for quantized MoE", Proposed shape: every
layer's quantized expert tensors in pinned host memory, a single resident
expert layer on the device, layer N+1 prefetched on a side stream during
layer N's compute; Evidence: the frozen forward is bit-identical with
offload on or off).

Two device slots hold the layer in use and the one being filled.  Copies go
through ``moeq_qweight_copy_async`` on a side stream of default priority;
events order them against the compute stream both ways (a slot is refilled
only after the forward that read it has finished).  The forward itself is
``moeq_experts_forward`` on the slot, so its result is the resident one's
bit for bit.
"""

import torch

from . import QWeight, moeq_experts_forward, moeq_qweight_copy_async


class ExpertOffload:
    def __init__(self, layers, device):
        """``layers``: a list of ``(gate_up, down)`` :class:`QWeight` pairs
        (on any device); they are copied into pinned host memory here."""
        self.device = torch.device(device)
        self.host = []
        for gu, dn in layers:
            hg, hd = gu.like("cpu", pin_memory=True), dn.like("cpu", pin_memory=True)
            moeq_qweight_copy_async(gu, hg) if gu.qdata.is_cuda else _copy_host(gu, hg)
            moeq_qweight_copy_async(dn, hd) if dn.qdata.is_cuda else _copy_host(dn, hd)
            self.host.append((hg, hd))
        torch.cuda.synchronize(self.device)
        gu0, dn0 = self.host[0]
        self.slots = [(gu0.like(self.device), dn0.like(self.device)) for _ in range(2)]
        self.copy_stream = torch.cuda.Stream(self.device)
        self.ready = [torch.cuda.Event() for _ in range(2)]
        self.free = [torch.cuda.Event() for _ in range(2)]
        self.filled = [None, None]   # layer index held (or being filled) by each slot

    def __len__(self):
        return len(self.host)

    def layer_bytes(self, layer):
        gu, dn = self.host[layer]
        return gu.nbytes() + dn.nbytes()

    def prefetch(self, layer):
        """Start copying ``layer`` into its slot on the side stream (after the
        slot's previous reader has finished)."""
        slot = layer % 2
        if self.filled[slot] == layer:
            return
        self.copy_stream.wait_event(self.free[slot])
        hg, hd = self.host[layer]
        dg, dd = self.slots[slot]
        moeq_qweight_copy_async(hg, dg, stream=self.copy_stream)
        moeq_qweight_copy_async(hd, dd, stream=self.copy_stream)
        self.ready[slot].record(self.copy_stream)
        self.filled[slot] = layer

    def forward(self, layer, hidden, top_k_index, top_k_weights, out=None, workspace=None):
        """The experts forward of ``layer`` from its device slot; prefetches
        ``layer + 1`` first so the copy overlaps this layer's compute."""
        slot = layer % 2
        self.prefetch(layer)
        compute = torch.cuda.current_stream(self.device)
        compute.wait_event(self.ready[slot])
        if layer + 1 < len(self.host):
            self.prefetch(layer + 1)
        gu, dn = self.slots[slot]
        out = moeq_experts_forward(hidden, top_k_index, top_k_weights, gu, dn, out=out, workspace=workspace)
        self.free[slot].record(compute)
        return out


def _copy_host(src, dst):
    for d, t in zip(dst._tensors(), src._tensors()):
        d.copy_(t)
