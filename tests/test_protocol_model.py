"""The host-thread model of the signal and work-queue protocol
(tests/protocol/protocol_model.cpp), built with g++ and run on the CPU: with
threads standing in for workgroups, random delays and permuted arrival, it
checks claim-once queues, counted arrivals and their reset, epoch tagging,
the per-XCD phased queues with the MLP row-block dependencies, the MoE
producer queue (also after a launch that never ran) and the timeout path.
The same model under ThreadSanitizer, and built with planted mistakes, each
of which its checks must catch."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "protocol", "protocol_model.cpp")


def _build(tmp_path, name, *flags):
    exe = tmp_path / name
    subprocess.run(["g++", "-std=c++17", "-O2", "-pthread", *flags, SRC, "-o", str(exe)], check=True,
                   capture_output=True, text=True)
    return str(exe)


def _run(exe, iters, seed, timeout=240):
    return subprocess.run([exe, str(iters), str(seed)], capture_output=True, text=True, timeout=timeout)


def test_protocol_model(tmp_path):
    exe = _build(tmp_path, "model")
    for seed in (1, 2):
        r = _run(exe, 80, seed)
        assert r.returncode == 0, r.stdout[-2000:]
        for name in ("unit_decode", "epoch_tagging", "ag_queue_counted_arrival_epochs",
                     "ag_withheld_signal_timeout_and_recovery", "xcd_phased_queues_mlp_dependencies",
                     "moe_queue_reset_and_failed_launch", "rs_end_signal_joins_through_the_gemm"):
            assert f"ok {name}" in r.stdout, (name, r.stdout[-2000:])


def test_protocol_model_thread_sanitizer(tmp_path):
    try:
        exe = _build(tmp_path, "model_tsan", "-fsanitize=thread", "-g")
    except subprocess.CalledProcessError as e:  # pragma: no cover
        pytest.skip(f"ThreadSanitizer unavailable: {e.stderr[-300:]}")
    r = _run(exe, 20, 3)
    assert r.returncode == 0, (r.stdout[-1500:], r.stderr[-3000:])
    assert "WARNING: ThreadSanitizer" not in r.stderr, r.stderr[-3000:]


@pytest.mark.parametrize("mutation", [1, 2, 3, 4, 5])
def test_protocol_model_catches_planted_mistakes(tmp_path, mutation):
    exe = _build(tmp_path, f"model_m{mutation}", f"-DMUTATION={mutation}")
    r = _run(exe, 40, 4)
    assert r.returncode != 0 and "FAIL" in r.stdout, (mutation, r.stdout[-1500:])
