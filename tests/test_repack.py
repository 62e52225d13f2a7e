"""The library's host-side expert repack (csrc/repack.h), built on its own
with g++ under the address and undefined-behaviour sanitizers (no GPU),
against a numpy statement of the record layouts documented in include/moe.h
and csrc/layout.h: for each weight format, the atom of row group g and K
chunk c holds lane l's part of row 16g + l % 16, K block 4c + l / 16; gate
and up row groups alternate; the down atoms follow; NVFP4 records end with
the three fp32 matrix scales.  Shapes include ragged chunk counts and one
large enough for the threaded path."""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MXFP4, BF16, NVFP4 = 0, 1, 2


@pytest.fixture(scope="module")
def repack(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("repack") / "repack_check")
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-pthread", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-o", exe,
                    os.path.join(ROOT, "tests", "repack_check.cpp")], check=True)
    return exe


def _atoms_fp4(q, N, K):
    """Code bytes of the atoms of a [N][K] 4-bit matrix: [N/16][K/128][1024]."""
    a = q.reshape(N // 16, 16, K // 128, 4, 16)          # g, row, c, block, byte
    return a.transpose(0, 2, 3, 1, 4).reshape(N // 16, K // 128, 1024)


def _scales(s, N, K, per):
    """Scale bytes of the atoms: lane l = 16 block + row, `per` bytes each."""
    a = s.reshape(N // 16, 16, K // 128, 4, per)
    return a.transpose(0, 2, 3, 1, 4).reshape(N // 16, K // 128, 64 * per)


def _atoms_bf16(w, N, K):
    """[N][K] bf16 patterns -> atoms: piece p of lane l at 1024 p + 16 l."""
    a = w.reshape(N // 16, 16, K // 128, 4, 4, 8)        # g, row, c, block, piece, value
    return a.transpose(0, 2, 4, 3, 1, 5).reshape(N // 16, K // 128, 4096 // 2).view(np.uint8)


def _record(fmt, H, I, m):
    def mat(q, s, N, K):
        if fmt == BF16:
            return _atoms_bf16(q.view(np.uint16).reshape(N, K), N, K)
        codes = _atoms_fp4(q, N, K)
        if fmt == NVFP4:
            return np.concatenate([codes, _scales(s[:-4], N, K, 2)], axis=2)
        return np.concatenate([codes, _scales(s, N, K, 1)], axis=2)
    g = mat(m["qg"], m.get("sg"), I, H)
    u = mat(m["qu"], m.get("su"), I, H)
    gu = np.stack([g, u], axis=1)                        # pair, gate/up, chunk, bytes
    d = mat(m["qd"], m.get("sd"), H, I)
    parts = [gu.ravel(), d.ravel()]
    if fmt == NVFP4:
        parts.append(np.concatenate([m["sg"][-4:], m["su"][-4:], m["sd"][-4:],
                                     np.zeros(4, np.uint8)]))
    return np.concatenate(parts)


@pytest.mark.parametrize("fmt", [MXFP4, BF16, NVFP4])
@pytest.mark.parametrize("H,I", [(128, 128), (384, 256), (256, 640), (4096, 2048)])
def test_repack_matches_the_documented_layout(repack, tmp_path, fmt, H, I):
    rng = np.random.default_rng(H * 7 + I + fmt)
    HI = H * I
    if fmt == BF16:
        m = {k: rng.integers(0, 256, HI * 2, dtype=np.uint8) for k in ("qg", "qu", "qd")}
    else:
        m = {k: rng.integers(0, 256, HI // 2, dtype=np.uint8) for k in ("qg", "qu", "qd")}
        ns = HI // 16 + 4 if fmt == NVFP4 else HI // 32
        m.update({k: rng.integers(0, 255, ns, dtype=np.uint8) for k in ("sg", "su", "sd")})
    for k, v in m.items():
        v.tofile(tmp_path / f"{k}.bin")
    r = subprocess.run([repack, str(fmt), str(H), str(I), str(tmp_path)], capture_output=True,
                       text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    rec = np.fromfile(tmp_path / "rec.bin", dtype=np.uint8)
    want = _record(fmt, H, I, m)
    assert rec.size == want.size
    bad = np.flatnonzero(rec != want)
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:5].tolist()}"
