"""Double-buffered streaming of packed prefill weights from host memory.

Disaggregated Quantization's on-demand prefill (ODP, the paragraph that
introduces it) keeps the prefill weights off the device, reads them one layer
block at a time into one of two device buffers, and overlaps the next block's
read with the current block's computation; long inputs hide the read, short
ones expose it.  Here a block's weights sit in pinned host memory (the
stand-in for the page's SSD) as packed NVFP4 blobs, one per linear layer, and
travel over PCIe on a copy stream while the compute stream runs quantize +
W4A4 GEMM of the previous block.  Every kernel is the library's; this module
only orders the copies and the launches with events.
"""

import torch

from . import qlin

_ALIGN = 256


class PrefillWeightStream:
    """Streams blocks of packed NVFP4 weight blobs host -> device.

    host_blocks: list of blocks; a block is a list of pinned uint8 CPU
    tensors (repacked blobs, one per linear layer, in execution order), and
    every block has the same layer count.  Two device buffers, each large
    enough for the biggest block, are allocated once; both streams keep the
    default priority.
    """

    def __init__(self, host_blocks, device=None):
        if not host_blocks or not host_blocks[0]:
            raise ValueError("no weight blobs")
        nl = len(host_blocks[0])
        for blk in host_blocks:
            if len(blk) != nl:
                raise ValueError("every block must have the same number of layers")
            for b in blk:
                if b.device.type != "cpu" or b.dtype != torch.uint8 or not b.is_pinned():
                    raise ValueError("host blobs must be pinned uint8 CPU tensors")
        self.host_blocks = host_blocks
        self.device = torch.device(device) if device is not None else torch.device("cuda")
        self.offsets = []
        cap = 0
        for blk in host_blocks:
            offs, o = [], 0
            for b in blk:
                offs.append(o)
                o += (b.numel() + _ALIGN - 1) // _ALIGN * _ALIGN
            self.offsets.append(offs)
            cap = max(cap, o)
        self.bufs = [torch.empty(cap, dtype=torch.uint8, device=self.device) for _ in range(2)]
        self.copy_stream = torch.cuda.Stream(device=self.device)
        self.ready = [torch.cuda.Event() for _ in range(2)]
        self.free = [torch.cuda.Event() for _ in range(2)]
        # free[b] has been recorded after the last GEMMs that read buffer b,
        # by this run() or an earlier one; a later copy into b must wait on it
        self.recorded = [False, False]

    def _blob(self, buf, blk, j):
        o = self.offsets[blk][j]
        return self.bufs[buf][o:o + self.host_blocks[blk][j].numel()]

    def _issue_copy(self, step, blk):
        b = step % 2
        with torch.cuda.stream(self.copy_stream):
            if self.recorded[b]:
                # buffer b holds the block of an earlier step (of this run or of
                # an earlier run) until the GEMMs that read it have run
                self.copy_stream.wait_event(self.free[b])
            for j, h in enumerate(self.host_blocks[blk]):
                self._blob(b, blk, j).copy_(h, non_blocking=True)
            self.ready[b].record(self.copy_stream)

    def run(self, order, shapes, xs, ys, codes, scales, tscales, workspaces):
        """Run the blocks listed in `order` (indices into host_blocks).

        For each block, layer j quantizes xs[j] and multiplies it by the
        block's streamed weights into ys[j]; shapes[j] = (n, k).  codes,
        scales, tscales and workspaces are the per-layer quantizer outputs and
        workspace (see qlin.quantize_nvfp4).  Work is enqueued on the current
        stream (compute) and the copy stream; nothing synchronises the host,
        and back-to-back calls are ordered on the device: a copy into a buffer
        waits for the GEMMs of any earlier call that read that buffer.
        """
        compute = torch.cuda.current_stream(self.device)
        self._issue_copy(0, order[0])
        for step, blk in enumerate(order):
            if step + 1 < len(order):
                self._issue_copy(step + 1, order[step + 1])
            b = step % 2
            for j, (n, k) in enumerate(shapes):
                qlin.quantize_nvfp4(xs[j], codes=codes[j], scales=scales[j],
                                    workspace=workspaces[j], ts_out=tscales[j])
                if j == 0:
                    compute.wait_event(self.ready[b])
                qlin.gemm_w4a4(codes[j], scales[j], tscales[j], self._blob(b, blk, j),
                               xs[j].shape[0], n, k, y=ys[j])
            self.free[b].record(compute)
            self.recorded[b] = True
        return ys
