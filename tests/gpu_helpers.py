"""Shared helpers for the GPU tests: moving seeded inputs to the device and
results back. No arithmetic of the method lives here."""
import numpy as np
import torch

import layer_streamed_nf4_amd as L


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU (gfx950); none is visible")
    L.lib()  # raises if the HIP library was not built


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def dev_bf16bits(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def ws_tensor(nbytes: int) -> torch.Tensor:
    return torch.empty(max(256, (nbytes + 255) // 256 * 256), dtype=torch.uint8, device="cuda")


def quantize_on_gpu(w: np.ndarray, dtype=L.DTYPE_F32, base: int = 0):
    """Quantise W on the device; returns (shard device tensor, desc, status)."""
    n, k = w.shape
    d = L.nf4s_tensor_layout(n, k, base)
    shard = torch.zeros(d.end, dtype=torch.uint8, device="cuda")
    ws = ws_tensor(L.nf4s_workspace_bytes(L.OP_QUANTIZE, 0, n, k))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    if dtype == L.DTYPE_F32:
        wd = dev_f32(w)
    else:
        wd = dev_bf16bits(w)
    L.nf4_quantize_shard(wd.data_ptr(), dtype, n, k, shard.data_ptr(), d, status.data_ptr(),
                         ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return shard, d, int(status.item())


def sections(shard: torch.Tensor, d):
    """Split a device shard into host numpy sections (packed, q8, nested, offset)."""
    h = shard.cpu().numpy()
    n = d.n_out * d.k_in
    nb = n // 64
    nn = (nb + 255) // 256
    packed = h[d.off_packed:d.off_packed + n // 2]
    q8 = h[d.off_q8:d.off_q8 + nb]
    nested = h[d.off_nested:d.off_nested + 4 * nn].view(np.float32)
    offset = h[d.off_offset:d.off_offset + 4].view(np.float32)[0]
    return packed, q8, nested, offset


def stream():
    return torch.cuda.current_stream().cuda_stream


def packed_rows_below(pk, M, K):
    """The bytes of a fragment-order buffer that hold rows < M."""
    Mp, Kp = -(-M // 256) * 256, -(-K // 64) * 64
    KB = Kp // 16
    idx = np.arange(Mp * Kp * 2 // 16)            # 16-byte chunks
    lane = idx % 64
    frag = idx // 64
    row = 32 * (frag // KB) + lane % 32
    keep = np.repeat(row < M, 16)
    return pk[keep]
