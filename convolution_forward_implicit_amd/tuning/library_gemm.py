"""Context measurement: the vendor GEMM (torch.matmul -> hipBLASLt) on the
plain GEMM each workload layer reduces to, with the operands already
materialised (A = the im2col matrix, M x C*Z*Y*X per group; B = the weights
as K_red x K).  This is the dense work the implicit kernels do without
building A; its throughput shows where the shapes themselves sit on this
GPU.  No epilogue (bias/GELU) is applied.

    python -m convolution_forward_implicit_amd.tuning.library_gemm

Needs a GPU.  Prints one line per shape: mean time per call over 50 calls
(after 10 untimed ones) and useful TFLOP/s.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# (name, groups, M, K_red, N) of the workload layers
SHAPES = [
    ("whisper_frontend_bf16_b32 layer 1", 1, 96000, 240, 384),
    ("whisper_frontend_bf16_b32 layer 2", 1, 48000, 1152, 384),
    ("grouped_conv2d_bf16", 4, 25088, 576, 64),
    ("grouped_conv3d_bf16_dil2", 8, 25088, 864, 32),
]


def main():
    import torch
    dev = torch.device("cuda:0")
    for name, G, M, Kr, N in SHAPES:
        A = torch.randn(G, M, Kr, device=dev).to(torch.bfloat16)
        B = torch.randn(G, Kr, N, device=dev).to(torch.bfloat16)
        C = torch.empty(G, M, N, device=dev, dtype=torch.bfloat16)
        if G == 1:
            f = lambda: torch.mm(A[0], B[0], out=C[0])
        else:
            f = lambda: torch.matmul(A, B, out=C)
        for _ in range(10):
            f()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(50):
            f()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / 50 * 1e3
        print("%-36s G=%d M=%d K_red=%d N=%d: %8.2f us  %7.1f TFLOP/s"
              % (name, G, M, Kr, N, us, 2.0 * G * M * Kr * N / us / 1e6), flush=True)


if __name__ == "__main__":
    main()
