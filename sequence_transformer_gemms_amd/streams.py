"""Streams on disjoint compute units, for a producer that feeds a chunk-gated
GEMM on the same GPU.

A chunk-gated GEMM keeps one persistent work-group per compute unit, and a
work-group whose chunk has not arrived spins on its ready flag.  When the
producer of the chunks (here: a side stream that copies them, standing in
for peers writing over xGMI) runs kernels on the same GPU, a producer
work-group can be dispatched to a CU held by such a waiting work-group and
never start.  Giving the two streams disjoint CU masks removes that
dependency; the library sizes its persistent grid from the mask of the
stream it is called on.

Both are blocking streams (the CU-mask creation call takes no flags), so
HIP's null stream orders itself against them: work enqueued on either waits
for the null stream's earlier work, and the null stream's work waits for
theirs.  A null stream that waits for a chunk-gated GEMM therefore holds
back a writer enqueued on the producer afterwards, and the GEMM waits for
that writer: issue the surrounding work on a non-blocking stream
(torch.cuda.Stream()), never on the null stream, while a gated GEMM waits.

The streams are created with hipExtStreamCreateWithCUMask and owned by the
returned MaskedStreams object, which destroys them (after synchronising
them) on close(), at the end of a `with` block, or at interpreter exit,
whichever comes first: the HIP runtime is never torn down with live streams
of ours.
"""
import atexit
import ctypes

__all__ = ["masked_streams", "MaskedStreams"]


def _runtime():
    return ctypes.CDLL("libamdhip64.so.7")  # the HIP runtime torch has loaded (already resident)


class MaskedStreams:
    """A (compute, producer) pair of torch streams on disjoint CU masks.
    Unpacks as `compute, producer = masked_streams(...)`."""

    def __init__(self, producer_cus: int, device: int):
        import torch
        self._hip = _runtime()
        self._handles = []
        self._device = device
        ncu = torch.cuda.get_device_properties(device).multi_processor_count
        if not 0 < producer_cus < ncu:
            raise ValueError(f"producer_cus must be in 1..{ncu - 1}")
        words = (ncu + 31) // 32
        prod, comp = [0] * words, [0] * words
        for i in range(ncu):
            (prod if i < producer_cus else comp)[i // 32] |= 1 << (i % 32)
        self.compute = self._make(comp, words)
        self.producer = self._make(prod, words)
        atexit.register(self.close)

    def _make(self, mask, words):
        import torch
        arr = (ctypes.c_uint32 * words)(*mask)
        handle = ctypes.c_void_p()
        with torch.cuda.device(self._device):
            rc = self._hip.hipExtStreamCreateWithCUMask(ctypes.byref(handle), ctypes.c_uint32(words), arr)
        if rc != 0:
            self.close()
            raise RuntimeError(f"hipExtStreamCreateWithCUMask failed with error {rc}")
        self._handles.append(handle.value)
        return torch.cuda.ExternalStream(handle.value, device=self._device)

    def close(self):
        """Synchronise and destroy the two streams (idempotent).  The torch
        stream objects must not be used afterwards."""
        while self._handles:
            h = ctypes.c_void_p(self._handles.pop())
            self._hip.hipStreamSynchronize(h)
            self._hip.hipStreamDestroy(h)
        atexit.unregister(self.close)

    def __iter__(self):
        return iter((self.compute, self.producer))

    def __getitem__(self, i):
        return (self.compute, self.producer)[i]

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
        return False


def masked_streams(producer_cus: int = 8, device: int = 0) -> MaskedStreams:
    """(compute, producer) streams: the producer may use CUs
    0 .. producer_cus-1 of the device's CU mask, the compute stream all the
    others."""
    return MaskedStreams(producer_cus, device)
