// Visibility across XCDs within one launch: every workgroup stores a per-epoch pattern,
// waits for its stores to complete, and arrives on a device-scope counter; the last to
// arrive reads every word back and counts the ones that do not hold this epoch's value.
// Each XCD's L2 first caches other workgroups' words of the previous epoch, so a load
// that an L2 serves from its own copy reads a stale word.  Stores and loads carry either
// no cache-policy bits or sc1 (device scope).  Test infrastructure, not part of libidx.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {
constexpr int NT = 256, WORDS = 256;

template <int SAUX, int LAUX>
__global__ __launch_bounds__(NT) void probe(uint32_t* data, uint32_t* cnt, uint32_t* stale, uint32_t* checks,
                                            uint32_t* sink, int nwg, uint32_t epoch) {
  __shared__ uint32_t arrived;
  const int b = blockIdx.x, t = threadIdx.x;
  const int total = nwg * WORDS;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(data, (short)0, total * 4, 0x00020000);
  // another workgroup's words into this XCD's caches
  const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(r, (((b + 37) % nwg) * WORDS + t) * 4, 0, 0);
  if (w == 0xDEADBEEFu) sink[t] = w;
  __builtin_amdgcn_raw_buffer_store_b32(epoch * 1000003u + (uint32_t)(b * WORDS + t), r, (b * WORDS + t) * 4, 0, SAUX);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (t == 0) arrived = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (arrived != (uint32_t)nwg - 1u) return;
  uint32_t m = 0;
  for (int i = t; i < total; i += NT)
    m += __builtin_amdgcn_raw_buffer_load_b32(r, i * 4, 0, LAUX) != epoch * 1000003u + (uint32_t)i ? 1u : 0u;
  if (m) __hip_atomic_fetch_add(stale, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (t == 0) {
    __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(checks, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}
}  // namespace

// sc1_stores, sc1_loads: 0 or 1.  nwg workgroups (1..65535), epochs launches.  Writes the
// number of last-arriver checks and of stale words read.  Returns 0, 1 for a bad argument,
// 2 for a HIP failure.
extern "C" int xcd_coherence_probe(int sc1_stores, int sc1_loads, int nwg, int epochs, uint32_t* checks_out,
                                   uint32_t* stale_out) {
  if (sc1_stores < 0 || sc1_stores > 1 || sc1_loads < 0 || sc1_loads > 1 || nwg < 2 || nwg > 65535 || epochs < 1 ||
      !checks_out || !stale_out)
    return 1;
  uint32_t *data = nullptr, *ctr = nullptr;
  if (hipMalloc(&data, (size_t)nwg * WORDS * 4) != hipSuccess) return 2;
  if (hipMalloc(&ctr, (3 + NT) * 4) != hipSuccess) {
    (void)hipFree(data);
    return 2;
  }
  int rc = 0;
  if (hipMemset(data, 0, (size_t)nwg * WORDS * 4) != hipSuccess || hipMemset(ctr, 0, (3 + NT) * 4) != hipSuccess) rc = 2;
  uint32_t *cnt = ctr, *stale = ctr + 1, *checks = ctr + 2, *sink = ctr + 3;
  for (int e = 1; e <= epochs && rc == 0; e++) {
    const uint32_t ep = (uint32_t)e;
    switch (sc1_stores * 2 + sc1_loads) {
      case 0: probe<0, 0><<<nwg, NT>>>(data, cnt, stale, checks, sink, nwg, ep); break;
      case 1: probe<0, 16><<<nwg, NT>>>(data, cnt, stale, checks, sink, nwg, ep); break;
      case 2: probe<16, 0><<<nwg, NT>>>(data, cnt, stale, checks, sink, nwg, ep); break;
      default: probe<16, 16><<<nwg, NT>>>(data, cnt, stale, checks, sink, nwg, ep); break;
    }
    if (hipGetLastError() != hipSuccess) rc = 2;
  }
  uint32_t h[3] = {0, 0, 0};
  if (rc == 0 && (hipDeviceSynchronize() != hipSuccess || hipMemcpy(h, ctr, 12, hipMemcpyDeviceToHost) != hipSuccess)) rc = 2;
  *checks_out = h[2];
  *stale_out = h[1];
  (void)hipFree(data);
  (void)hipFree(ctr);
  return rc;
}
