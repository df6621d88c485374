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
"""
import ctypes

__all__ = ["masked_streams"]

_hip = None


def _runtime():
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so.7")  # the HIP runtime torch has loaded
    return _hip


def masked_streams(producer_cus: int = 8, device: int = 0):
    """(compute, producer) torch streams: the producer may use CUs
    0 .. producer_cus-1 of the device's CU mask, the compute stream all the
    others."""
    import torch
    hip = _runtime()
    ncu = torch.cuda.get_device_properties(device).multi_processor_count
    if not 0 < producer_cus < ncu:
        raise ValueError(f"producer_cus must be in 1..{ncu - 1}")
    words = (ncu + 31) // 32
    prod, comp = [0] * words, [0] * words
    for i in range(ncu):
        (prod if i < producer_cus else comp)[i // 32] |= 1 << (i % 32)

    def make(mask):
        arr = (ctypes.c_uint32 * words)(*mask)
        handle = ctypes.c_void_p()
        with torch.cuda.device(device):
            rc = hip.hipExtStreamCreateWithCUMask(ctypes.byref(handle), ctypes.c_uint32(words), arr)
        if rc != 0:
            raise RuntimeError(f"hipExtStreamCreateWithCUMask failed with error {rc}")
        return torch.cuda.ExternalStream(handle.value, device=device)
    return make(comp), make(prod)

