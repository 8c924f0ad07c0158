// kvq_probe.hip — a plain streaming read of a device buffer: the attainable HBM read bandwidth
// the decode's roofline fraction is set against.  The forum post "3090 单卡跑 Qwen3.8-27B：NInfer
// 上机实测（180K 上下文 / C2 并发 / 4bit KV）" (二、测评) reasons about decode speed as bytes read
// per token against the card's bandwidth; this kernel measures that bandwidth on the device
// itself, with nothing else to do but read.
//
// A second probe reads the shader clock the kernels run at, from the GPU's own counters.
//
// Three load forms: 16-byte loads into registers, non-temporal (mode 0) or normal (mode 1), and
// the decode's own form, gfx950 direct-to-LDS 16-byte loads, non-temporal (mode 2).  Every byte
// is read once.  A per-lane xor of the loaded words goes to `sink` only if it equals a value
// no realistic data gives, so the loads cannot be dropped and almost nothing is written.
#include "kvq_attn_block.h"

namespace kvq {
namespace {

constexpr int kProbeThreads = 256;
constexpr uint32_t kSinkMagic = 0x9E3779B9u;

template <bool NT>
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                                     uint32_t* sink) {
  constexpr int U = 8;  // loads in flight per lane
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = NT ? __builtin_nontemporal_load(p + i + u * stride) : p[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = NT ? __builtin_nontemporal_load(p + i) : p[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == kSinkMagic) sink[0] = acc;
}

// Direct-to-LDS form: wave w of the grid reads 4 KB chunks w, w + waves, ... into a ring of
// eight 4 KB slots of its own LDS, keeping up to seven chunks in flight (the loaded bytes are
// not used).
__global__ __launch_bounds__(kProbeThreads) void stream_read_lds_kernel(const uint8_t* __restrict__ p,
                                                                         size_t n4k, uint32_t* sink) {
  constexpr int SLOTS = 8;
  __shared__ __attribute__((aligned(16))) uint8_t s_ring[kProbeThreads / kWave][SLOTS][4096];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const size_t waves = (size_t)gridDim.x * (kProbeThreads / kWave);
  const size_t wg = (size_t)blockIdx.x * (kProbeThreads / kWave) + w;
  const uint32_t ring0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)&s_ring[w][0][0]);
  int k = 0;
  for (size_t c = wg; c < n4k; c += waves, ++k) {
    // slot k % 8 was last filled 8 chunks ago: at most 7 chunks (28 loads) may still be out
    wait_vmcnt<4 * (SLOTS - 1)>();
    dma16<4>(p + c * 4096, 16u * lane, ring0 + (uint32_t)((k & (SLOTS - 1)) * 4096));
  }
  wait_vmcnt<0>();
  __syncthreads();
  if (threadIdx.x == 0 && s_ring[0][0][0] == 0xA5 && s_ring[0][0][1] == 0x5A && n4k == 0) sink[0] = kSinkMagic;
}

// Shader clock: each one-wave workgroup counts shader-clock cycles (s_memtime) across a spin
// of `ticks` ticks of the constant-rate counter (s_memrealtime); the spin ends when the
// constant-rate counter has moved that far, which it always does.  Lane 0 writes the cycles,
// the ticks and the XCD the wave ran on (hardware register XCC_ID).
__global__ __launch_bounds__(kWave) void clock_probe_kernel(unsigned long long* out, unsigned ticks) {
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  unsigned long long r1;
  do {
    r1 = __builtin_amdgcn_s_memrealtime();
  } while (r1 - r0 < ticks);
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  const unsigned xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20) & 0xFu;  // XCC_ID bits 3:0
  if (threadIdx.x == 0) {
    out[3 * blockIdx.x] = c1 - c0;
    out[3 * blockIdx.x + 1] = r1 - r0;
    out[3 * blockIdx.x + 2] = xcc;
  }
}

}  // namespace

hipError_t launch_clock_probe(unsigned long long* out, int workgroups, unsigned ticks, hipStream_t stream) {
  hipLaunchKernelGGL(clock_probe_kernel, dim3((unsigned)workgroups), dim3(kWave), 0, stream, out, ticks);
  return hipGetLastError();
}

hipError_t launch_stream_probe(const void* buf, size_t bytes, int mode, int workgroups, uint32_t* sink,
                               hipStream_t stream) {
  const dim3 grid((unsigned)workgroups), block(kProbeThreads);
  if (mode == 0)
    hipLaunchKernelGGL((stream_read_kernel<true>), grid, block, 0, stream, (const u32x4*)buf, bytes / 16, sink);
  else if (mode == 1)
    hipLaunchKernelGGL((stream_read_kernel<false>), grid, block, 0, stream, (const u32x4*)buf, bytes / 16, sink);
  else
    hipLaunchKernelGGL(stream_read_lds_kernel, grid, block, 0, stream, (const uint8_t*)buf, bytes / 4096, sink);
  return hipGetLastError();
}

}  // namespace kvq
