"""Pool layouts of the library boundary, as numpy views (test helpers).

K pool: [num_pages][Hkv][Dk/C][P][C] with C = 64 bytes of elements (64 FP8 codes or 32 bf16):
a token's row is cut into 64-byte chunks stored chunk by chunk inside the (page, head) block.
V pool: [num_pages][Hkv][Dv][P].  These helpers move between that physical order and the
logical [num_pages][Hkv][P][Dk] order the tests reason in.
"""
import numpy as np

FP8, BF16 = 0, 1


def k_chunk(kv_dt: int) -> int:
    return 64 if kv_dt == FP8 else 32


def k_shape(num_pages, Hkv, P, Dk, kv_dt):
    C = k_chunk(kv_dt)
    assert Dk % C == 0, "Dk must be a multiple of the 64-byte chunk"
    return (num_pages, Hkv, Dk // C, P, C)


def k_to_phys(k_logical: np.ndarray, kv_dt: int) -> np.ndarray:
    n, H, P, D = k_logical.shape
    C = k_chunk(kv_dt)
    return np.ascontiguousarray(k_logical.reshape(n, H, P, D // C, C).transpose(0, 1, 3, 2, 4))


def k_to_logical(k_phys: np.ndarray) -> np.ndarray:
    n, H, nc, P, C = k_phys.shape
    return np.ascontiguousarray(k_phys.transpose(0, 1, 3, 2, 4).reshape(n, H, P, nc * C))
