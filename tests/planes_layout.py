"""Unpack liblynx nibble planes into logical codes, from the layout that
include/lynx.h documents (test helper; index manipulation only, no method
arithmetic)."""
import numpy as np

PAGE, CHUNK, CHUNKS, D = 256, 32, 8, 128


def _nibbles(b: np.ndarray):
    b = b.astype(np.uint8)
    return b & 0x0F, b >> 4


def _signed4(n: np.ndarray) -> np.ndarray:
    n = n.astype(np.int16)
    return np.where(n >= 8, n - 16, n).astype(np.int8)


def value_token_order() -> np.ndarray:
    """Token (within a chunk) held by nibble k of word w, as [4][8]."""
    order = np.empty((4, 8), np.int64)
    for w in range(4):
        for k in range(8):
            order[w, k] = 4 * w + k if k < 4 else 16 + 4 * w + (k - 4)
    return order


def unpack_plane(plane: np.ndarray, P: int, H: int, role: int) -> np.ndarray:
    """uint8 plane bytes -> nibble values [P][256][H][128] (uint8, 0..15)."""
    plane = np.asarray(plane, np.uint8)
    if role == 0:
        b = plane.reshape(P, H, PAGE, D // 2)
        lo, hi = _nibbles(b)
        nib = np.empty((P, H, PAGE, D), np.uint8)
        nib[..., 0::2] = lo
        nib[..., 1::2] = hi
        return np.ascontiguousarray(nib.transpose(0, 2, 1, 3))
    b = plane.reshape(P, H, CHUNKS, D, 16)
    words = b.reshape(P, H, CHUNKS, D, 4, 4)             # 4 words x 4 bytes
    lo, hi = _nibbles(words)
    nib_w = np.empty((P, H, CHUNKS, D, 4, 8), np.uint8)  # nibble k of word w
    nib_w[..., 0::2] = lo
    nib_w[..., 1::2] = hi
    out = np.empty((P, H, CHUNKS, D, CHUNK), np.uint8)
    order = value_token_order()
    for w in range(4):
        for k in range(8):
            out[..., order[w, k]] = nib_w[..., w, k]
    # [P][H][c][D][t] -> [P][c][t][H][D]
    out = out.transpose(0, 2, 4, 1, 3).reshape(P, PAGE, H, D)
    return np.ascontiguousarray(out)


def unpack_codes(anchor: np.ndarray, residual: np.ndarray, P: int, H: int, role: int):
    """Return (anchor int8 -8..7, residual uint8 0..15, code int8), each [P][256][H][128]."""
    a = _signed4(unpack_plane(anchor, P, H, role))
    r = unpack_plane(residual, P, H, role)
    code = (a.astype(np.int16) * 16 + r.astype(np.int16)).astype(np.int8)
    return a, r, code
