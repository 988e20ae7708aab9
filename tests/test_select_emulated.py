"""The select core's own source (csrc/select_core.h) run on the CPU: every
GPU thread is a fiber, workgroup and wave barriers and the cross-workgroup
barrier are cooperative waits (tests/emu/). Checks the selection of one row
split over P workgroups at 16 and 32 keys per thread, on the window select
and the two-barrier radix select: exactly m keys, none left out above the
threshold, ties to the lower element. Needs g++ only."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "decode_attention_sparse_amd", "csrc")


@pytest.fixture(scope="module")
def emulator(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("select_emu")
    # select_core.h includes "sdkv_device.h": the emulation header takes its place
    shutil.copy(os.path.join(HERE, "emu", "emu_device.h"), d / "sdkv_device.h")
    shutil.copy(os.path.join(CSRC, "select_core.h"), d / "select_core.h")
    shutil.copy(os.path.join(HERE, "emu", "emu_fibers.h"), d / "emu_fibers.h")
    shutil.copy(os.path.join(HERE, "emu", "select_emu.cpp"), d / "select_emu.cpp")
    exe = d / "select_emu"
    subprocess.run(["g++", "-O2", "-std=c++17", "-o", str(exe), str(d / "select_emu.cpp")],
                   check=True, capture_output=True, text=True)
    return str(exe)


@pytest.mark.parametrize("spt,P,T,m,kind,window", [
    (16, 8, 131072, 13108, "normal", 1),     # the 128K layer row
    (16, 8, 131072, 13108, "ties", 1),       # window misses -> radix fallback
    (32, 8, 262144, 26215, "normal", 1),     # 32 keys per thread, window select
    (32, 9, 262144, 26215, "normal", 1),     # P = 9 (a Qwen-shaped row in one wave)
    (32, 4, 131072, 13108, "ties", 1),
    (32, 2, 65536, 6554, "plateau", 1),      # one value repeated on every 7th token
    (32, 8, 262144, 26215, "plateau", 1),    # threshold on the plateau: tie quota per workgroup
    (32, 8, 262144, 26215, "normal", 0),     # two-barrier radix select directly
    (8, 3, 20000, 2000, "normal", 1),        # ragged last chunk
])
@pytest.mark.parametrize("order", [0])
def test_select_core_emulated(emulator, spt, P, T, m, kind, window, order):
    _run_case(emulator, spt, P, T, m, kind, window, order)


# Fibers resumed in reversed and shuffled order between synchronisations: a
# selection that changed with the order would show two threads touching one
# location with no synchronisation between them.
@pytest.mark.parametrize("spt,P,T,m,kind,window,order", [
    (32, 8, 262144, 26215, "normal", 1, 1),
    (32, 8, 262144, 26215, "plateau", 1, 2),
    (32, 4, 131072, 13108, "ties", 1, 2),
    (16, 8, 131072, 13108, "normal", 0, 1),
])
def test_select_core_emulated_thread_order(emulator, spt, P, T, m, kind, window, order):
    _run_case(emulator, spt, P, T, m, kind, window, order)


def _run_case(emulator, spt, P, T, m, kind, window, order):
    r = subprocess.run([emulator, str(spt), str(P), str(T), str(m), str(spt * 100 + P), kind,
                        str(window), str(order)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    if window and kind != "ties":
        # the window holds the threshold: no workgroup falls back to the radix select
        assert "window fallbacks 0," in r.stdout, r.stdout
