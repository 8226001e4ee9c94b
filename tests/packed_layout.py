"""The packed ("matrix-core operand order") weight layout of qlin_pack_weights,
as a numpy reshape of the row-major codes: 32-row blocks cut into K slices of S
bytes (S = 32 for int8, 64 for E4M3), each slice stored as S/32 units of 1 KB in
which lane l's 16 bytes sit at 16 l:
    packed[((rb (K/S) + s) H + h) 1024 + 16 l + b] = w[32 rb + l % 32][S s + (S/2)(l / 32) + 16 h + b],
H = S / 32.  Test helper, shared by the CPU pin and the GPU parity tests."""
import numpy as np


def packed_reference(w: np.ndarray, S: int) -> np.ndarray:
    N, K = w.shape
    H = S // 32
    # axes of w: rb, r (= l % 32), s, half (= l / 32), h, b
    v = w.reshape(N // 32, 32, K // S, 2, H, 16)
    # packed order: rb, s, h, half, r, b   (l = 32 half + r)
    return np.ascontiguousarray(v.transpose(0, 2, 4, 3, 1, 5)).reshape(-1)
