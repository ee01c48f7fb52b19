// Accuracy probe for gfx950's matrix instructions: C = A · Bᵀ with f32 accumulation,
// A [m, k] and B [n, k] stored row-major, one 64-lane wave per 32 × 32 tile of C.
//
// It exists to measure how each instruction accumulates: the inputs are OCP FP8 E4M3FN
// codes (or their exact bf16 images), so every product is exact and the only error left
// is the instruction's own summation.  It is test infrastructure, not part of libidx.
//
//   mode 0: v_mfma_f32_32x32x16_fp8_fp8      (E4M3 × E4M3, 16 terms an instruction)
//   mode 1: v_mfma_f32_32x32x64_f8f6f4       (both operands E4M3, 64 terms an instruction,
//                                             the unscaled form of the block-scaled MFMA)
//   mode 2: v_mfma_f32_32x32x16_bf16         (bf16 × bf16, 16 terms an instruction)
//
// Operand layout used below (lane l of the wave, r = l % 32, h = l / 32): the A operand
// of lane l is row i0 + r of A and the B operand is row j0 + r of B, each over a run of
// k-indices picked by h.  Whatever order the hardware gives those k-indices inside an
// instruction, A and B name the same ones, so the tile is A · Bᵀ.  Output element q of
// lane l is C[i0 + 8(q/4) + 4h + q%4][j0 + r].
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

template <int MODE>
__global__ __launch_bounds__(64) void probe_kernel(const uint8_t* a, const uint8_t* b, float* c,
                                                   int n, int k) {
  const int lane = threadIdx.x;
  const int r = lane & 31, h = lane >> 5;
  const size_t i0 = (size_t)blockIdx.x * 32, j0 = (size_t)blockIdx.y * 32;
  v16f acc = {};
  if constexpr (MODE == 0) {
    const uint8_t* pa = a + (i0 + r) * k + h * 8;
    const uint8_t* pb = b + (j0 + r) * k + h * 8;
    for (int s = 0; s < k; s += 16)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(*(const long*)(pa + s), *(const long*)(pb + s),
                                                        acc, 0, 0, 0);
  } else if constexpr (MODE == 1) {
    const uint8_t* pa = a + (i0 + r) * k + h * 32;
    const uint8_t* pb = b + (j0 + r) * k + h * 32;
    for (int s = 0; s < k; s += 64)
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(*(const v8i*)(pa + s), *(const v8i*)(pb + s),
                                                             acc, 0, 0, 0, 0, 0, 0);
  } else {
    const uint16_t* pa = (const uint16_t*)a + (i0 + r) * k + h * 8;
    const uint16_t* pb = (const uint16_t*)b + (j0 + r) * k + h * 8;
    for (int s = 0; s < k; s += 16)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const v8bf*)(pa + s), *(const v8bf*)(pb + s),
                                                     acc, 0, 0, 0);
  }
#pragma unroll
  for (int q = 0; q < 16; q++) c[(i0 + 8 * (q / 4) + 4 * h + q % 4) * n + j0 + r] = acc[q];
}

// Issue rate of each instruction: every wave of a 2048 x 256-thread grid runs `iters`
// rounds of two independent 8-instruction chains, operands in registers.
template <int MODE>
__global__ __launch_bounds__(256) void rate_kernel(const uint32_t* in, float* out, int iters) {
  const int t = threadIdx.x;
  v16f acc0 = {}, acc1 = {};
  if constexpr (MODE == 3) {
    // v_mfma_f32_16x16x32_bf16: four independent chains (a shorter instruction)
    v8bf x[4], y[4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 8; j++) {
        x[i][j] = __builtin_bit_cast(__bf16, (uint16_t)(in[(t + 8 * i + j) & 255] & 0x3F80u));
        y[i][j] = __builtin_bit_cast(__bf16, (uint16_t)(in[(3 * t + i + j) & 255] & 0x3F80u));
      }
    v4f c[4] = {};
    for (int it = 0; it < iters; it++)
#pragma unroll
      for (int s = 0; s < 4; s++)
#pragma unroll
        for (int ch = 0; ch < 4; ch++)
          c[ch] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x[(s + ch) & 3], y[s], c[ch], 0, 0, 0);
#pragma unroll
    for (int ch = 0; ch < 4; ch++)
#pragma unroll
      for (int q = 0; q < 4; q++) acc0[4 * ch + q] = c[ch][q];
  } else if constexpr (MODE == 2) {
    v8bf x[8], y[8];
#pragma unroll
    for (int i = 0; i < 8; i++)
#pragma unroll
      for (int j = 0; j < 8; j++) {
        x[i][j] = __builtin_bit_cast(__bf16, (uint16_t)(in[(t + 8 * i + j) & 255] & 0x3F80u));
        y[i][j] = __builtin_bit_cast(__bf16, (uint16_t)(in[(3 * t + i + j) & 255] & 0x3F80u));
      }
    for (int it = 0; it < iters; it++)
#pragma unroll
      for (int s = 0; s < 8; s++) {
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[s], y[s], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[(s + 1) & 7], y[s], acc1, 0, 0, 0);
      }
  } else if constexpr (MODE == 1) {
    v8i x[2], y[2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
      for (int j = 0; j < 8; j++) {
        x[i][j] = (int)(in[(t + 8 * i + j) & 255] & 0x38383838u);
        y[i][j] = (int)(in[(3 * t + i + j) & 255] & 0x38383838u);
      }
    for (int it = 0; it < iters; it++)
#pragma unroll
      for (int s = 0; s < 8; s++) {
        acc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x[s & 1], y[s & 1], acc0, 0, 0, 0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x[(s + 1) & 1], y[s & 1], acc1, 0, 0, 0, 0, 0, 0);
      }
  } else {
    long x[8], y[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      x[i] = (long)(in[(t + i) & 255] & 0x38383838u) | ((long)(in[(t + i + 1) & 255] & 0x38383838u) << 32);
      y[i] = (long)(in[(3 * t + i) & 255] & 0x38383838u) | ((long)(in[(3 * t + i + 2) & 255] & 0x38383838u) << 32);
    }
    for (int it = 0; it < iters; it++)
#pragma unroll
      for (int s = 0; s < 8; s++) {
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(x[s], y[s], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(x[(s + 1) & 7], y[s], acc1, 0, 0, 0);
      }
  }
  float sum = 0.f;
#pragma unroll
  for (int q = 0; q < 16; q++) sum += acc0[q] + acc1[q];
  out[blockIdx.x * 256 + t] = sum;
}

// a, b, c: device pointers.  m and n multiples of 32, k a positive multiple of 64; a and b
// hold uint8 codes (modes 0 and 1) or bf16 bit patterns (mode 2), row stride k elements.
// Returns 0, 1 for a bad argument, or 2 when the launch fails.
extern "C" int mfma_probe(int mode, const void* a, const void* b, float* c, int m, int n, int k,
                          void* stream) {
  if (mode < 0 || mode > 2 || !a || !b || !c || m <= 0 || n <= 0 || k <= 0 || m % 32 || n % 32 ||
      k % 64 || n / 32 > 65535 || (long long)m * k > (1ll << 30) || (long long)n * k > (1ll << 30))
    return 1;
  const dim3 grid(m / 32, n / 32);
  hipStream_t s = (hipStream_t)stream;
  const uint8_t* pa = (const uint8_t*)a;
  const uint8_t* pb = (const uint8_t*)b;
  if (mode == 0) probe_kernel<0><<<grid, 64, 0, s>>>(pa, pb, c, n, k);
  else if (mode == 1) probe_kernel<1><<<grid, 64, 0, s>>>(pa, pb, c, n, k);
  else probe_kernel<2><<<grid, 64, 0, s>>>(pa, pb, c, n, k);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Dense rate of instruction `mode` (as mfma_probe, and 3: v_mfma_f32_16x16x32_bf16) in TFLOP/s: 2048 workgroups of 256 threads,
// each wave 16 instructions a round for `iters` rounds, timed over a second launch with HIP
// events.  in: device, 256 words; out: device, 2048 * 256 floats.  Returns 0, 1 (bad
// argument) or 2 (HIP failure).
extern "C" int mfma_rate(int mode, const uint32_t* in, float* out, int iters, double* tflops) {
  if (mode < 0 || mode > 3 || !in || !out || iters < 1 || !tflops) return 1;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 2;
  int rc = 0;
  for (int rep = 0; rep < 2 && rc == 0; rep++) {
    if (rep == 1 && hipEventRecord(e0, 0) != hipSuccess) rc = 2;
    if (mode == 0) rate_kernel<0><<<2048, 256>>>(in, out, iters);
    else if (mode == 1) rate_kernel<1><<<2048, 256>>>(in, out, iters);
    else if (mode == 2) rate_kernel<2><<<2048, 256>>>(in, out, iters);
    else rate_kernel<3><<<2048, 256>>>(in, out, iters);
    if (hipGetLastError() != hipSuccess) rc = 2;
  }
  float ms = 0.f;
  if (rc == 0 && (hipEventRecord(e1, 0) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                  hipEventElapsedTime(&ms, e0, e1) != hipSuccess))
    rc = 2;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (rc) return rc;
  const double per_instr = mode == 1 ? 131072.0 : (mode == 3 ? 16384.0 : 32768.0);   // flops of one instruction
  *tflops = 2048.0 * 4 * 16 * (double)iters * per_instr / (ms * 1e-3) / 1e12;
  return 0;
}
