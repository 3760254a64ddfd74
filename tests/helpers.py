"""Test-side helpers: golden-file parsing and bf16 bit-pattern conversions."""
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> numpy uint16 bit patterns."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def f32_to_bf16_bits(v) -> np.ndarray:
    """float32 values (exactly representable in bf16) -> bf16 bits, by truncation."""
    f = np.ascontiguousarray(v, dtype=np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _expand(field):
    out = []
    for item in field.split(","):
        if "*" in item:
            v, n = item.split("*")
            out += [int(v, 16)] * int(n)
        else:
            out.append(int(item, 16))
    return out


def hand_blocks():
    """Parse tests/golden/hand_blocks.txt -> list of dicts."""
    cases = []
    with open(os.path.join(GOLDEN, "hand_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            g = float.fromhex(parts[2]) if parts[2].startswith("0x") else float(parts[2])
            d = {"id": parts[0], "fmt": parts[1], "g": g, "scale": int(parts[3], 16)}
            for p in parts[4:]:
                k, v = p.split("=")
                d[k] = _expand(v)
            n = 32 if d["fmt"] == "mxfp8" else 16
            assert len(d["x"]) == n, d["id"]
            assert len(d["payload"]) == (n if d["fmt"] == "mxfp8" else n // 2), d["id"]
            cases.append(d)
    return cases


def swizzle_offsets():
    """Parse tests/golden/swizzle_offsets.txt -> (rows, cols, total, [(r, c, off)])."""
    pts = []
    meta = {}
    with open(os.path.join(GOLDEN, "swizzle_offsets.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if "=" in line:
                for kv in line.split():
                    k, v = kv.split("=")
                    meta[k] = int(v)
                continue
            r, c, off = (int(v) for v in line.split())
            pts.append((r, c, off))
    return meta, pts


def e4m3_table() -> np.ndarray:
    """All 256 E4M3 code values via torch's float8_e4m3fn decode (float64)."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def row_scaled_rows():
    """Parse tests/golden/row_scaled_rows.txt -> list of dicts (32-element rows)."""
    cases = []
    with open(os.path.join(GOLDEN, "row_scaled_rows.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            d = {"id": parts[0]}
            for p in parts[1:]:
                k, v = p.split("=")
                if k == "g":
                    d[k] = float.fromhex(v)
                elif k == "amax":
                    d[k] = int(v, 16)
                else:
                    d[k] = _expand(v)
            assert len(d["x"]) == 32 and len(d["payload"]) == 16 and len(d["scales"]) == 2, d["id"]
            cases.append(d)
    return cases
